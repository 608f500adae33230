"""Buffers and call order of one SignMuon worker step on a flat parameter set.

This is host-side orchestration only: it owns the device buffers (through
torch) and calls the C ABI in the order of the "SignMuon: Otimização
Distribuída de Muon com Eficiência de Comunicação" summary, section 2,
"Fluxo Algorítmico (Distribuído)": local momentum and polar factor (step 1),
sign extraction packed to one bit per entry (steps 2-3), then the majority
vote and the update (step 4), optionally with the local re-orthogonalisation
of the vote (step 5).  All arithmetic runs in libmuon's kernels.
"""
from __future__ import annotations

from typing import Optional, Sequence, Tuple

import torch

from . import _abi

_TORCH_DTYPE = {"f32": torch.float32, "bf16": torch.bfloat16}


class SignMuonStep:
    """One worker's step over matrices ``shapes`` stored back to back in flat buffers.

    Parameters are the method's: ``beta``/``alpha`` of the momentum EMA,
    Newton-Schulz ``coeffs`` (a, b, c) and ``ns_steps``, the NS operand
    ``precision`` ("bf16" or "f32") and the step size ``eta``.

    The exchange needs only the packed signs of the polar directions.  Where
    the last Newton-Schulz product packs them itself (bf16 products on a wide
    matrix whose row length is a multiple of 64, every matrix starting on a
    64-bit word), the direction is not written unless ``keep_direction``;
    ``self.U`` then holds the directions of the other matrices only.  With
    ``keep_direction`` every direction is written to ``self.U``.
    """

    def __init__(self, shapes: Sequence[Tuple[int, int]], m_dtype: str = "bf16",
                 precision: str = "bf16", coeffs=(3.4445, -4.7750, 2.0315), ns_steps: int = 5,
                 beta: float = 0.95, alpha: Optional[float] = None, eta: float = 0.02,
                 device="cuda", keep_direction: bool = False):
        self.shapes = [tuple(int(x) for x in s) for s in shapes]
        self.device = torch.device(device)
        sizes = [r * c for r, c in self.shapes]
        offs = [0]
        for n in sizes:
            offs.append(offs[-1] + n)
        self.offsets_host = offs
        self.numel = offs[-1]
        # every matrix's signs start on a word boundary: ns_orthogonalize can
        # write them per matrix (from the last product's epilogue where it can)
        self.signs_per_matrix = all(o % 64 == 0 for o in offs[:-1])
        self.nwords = _abi.packed_words(self.numel)
        self.m_dtype = m_dtype
        self.precision = precision
        self.coeffs = tuple(float(x) for x in coeffs)
        self.ns_steps = int(ns_steps)
        self.beta = float(beta)
        self.alpha = float(1.0 - beta if alpha is None else alpha)
        self.eta = float(eta)
        self.keep_direction = bool(keep_direction)
        u_dtype = torch.float32 if precision == "f32" else torch.bfloat16
        self.offsets = torch.tensor(offs, dtype=torch.int64, device=self.device)
        self.sumsq = torch.zeros(len(self.shapes), dtype=torch.float32, device=self.device)
        self.U = torch.empty(self.numel, dtype=u_dtype, device=self.device)
        # workspace sized from the NS problems over a stand-in momentum buffer
        probe_M = torch.empty(self.numel, dtype=_TORCH_DTYPE[m_dtype], device=self.device)
        ns_bytes = _abi.ns_workspace_bytes(self._problems(probe_M), self.precision)
        mom_bytes = _abi.muon_momentum_workspace_bytes(self.numel, len(self.shapes))
        del probe_M
        self.ns_workspace = torch.empty(max(ns_bytes, 1), dtype=torch.uint8, device=self.device)
        self.mom_workspace = torch.empty(max(mom_bytes, 1), dtype=torch.uint8, device=self.device)
        self._prepared = {}   # marshalled orthogonalisation calls (see orthogonalize)

    def signs_fused(self, j: int) -> bool:
        """Whether matrix j's packed signs come from its last product (rule of
        ns_orthogonalize: bf16 products, which need a short side of at least 96)."""
        r, c = self.shapes[j]
        return (self.signs_per_matrix and self.precision == "bf16" and self.ns_steps > 0
                and r <= c and c % 64 == 0 and r >= _abi.ns_bf16_min_side())

    def _problems(self, M: torch.Tensor, bits_row: Optional[torch.Tensor] = None):
        probs = []
        for j, (r, c) in enumerate(self.shapes):
            lo, hi = self.offsets_host[j], self.offsets_host[j + 1]
            signs_only = bits_row is not None and self.signs_fused(j) and not self.keep_direction
            U = None if signs_only else self.U[lo:hi].view(r, c)
            prob = (M[lo:hi].view(r, c), U, self.sumsq[j:j + 1])
            if bits_row is not None:
                prob += (bits_row[lo // 64:(hi + 63) // 64],)
            probs.append(prob)
        return probs

    def new_bits(self, workers: int = 1) -> torch.Tensor:
        return torch.zeros((workers, self.nwords), dtype=torch.int64, device=self.device)

    # -- step pieces -------------------------------------------------------
    def momentum(self, M: torch.Tensor, G: torch.Tensor) -> None:
        _abi.muon_momentum(M, G, self.beta, self.alpha, self.offsets, self.sumsq, self.mom_workspace)

    def orthogonalize(self, M: torch.Tensor, bits_row: Optional[torch.Tensor] = None) -> None:
        """Polar directions into ``self.U`` (see ``keep_direction``); with ``bits_row``
        also their packed signs (requires ``signs_per_matrix``)."""
        # the marshalled call is kept per (momentum, sign words) buffer pair
        key = (M.data_ptr(), M.numel(), bits_row.data_ptr() if bits_row is not None else None,
               self.keep_direction)
        call = self._prepared.get(key)
        if call is None:
            a, b, c = self.coeffs
            call = _abi.PreparedNS(self._problems(M, bits_row), a, b, c, self.ns_steps, self.precision,
                                   self.ns_workspace)
            if len(self._prepared) >= 64:
                self._prepared.clear()
            self._prepared[key] = call
        call()

    def pack(self, bits_row: torch.Tensor) -> None:
        _abi.sign_pack(self.U, bits_row)

    def check(self) -> None:
        """Synchronise the current stream and raise if a split product of the last
        orthogonalisation gave up waiting for its other half (its output is invalid)."""
        _abi.ns_workspace_status(self.ns_workspace)

    def worker(self, M: torch.Tensor, G: torch.Tensor, bits_row: torch.Tensor) -> None:
        """Steps 1-3 for one worker: momentum, polar direction, packed signs."""
        self.momentum(M, G)
        if self.signs_per_matrix:
            self.orthogonalize(M, bits_row)
        else:
            self.orthogonalize(M)
            self.pack(bits_row)

    def vote_update(self, W: torch.Tensor, bits: torch.Tensor, vote_out: Optional[torch.Tensor] = None,
                    fused: bool = False, reorthogonalize: bool = False) -> None:
        """Step 4: majority vote over the rows of ``bits`` and ``W <- W - eta * vote``.

        With ``reorthogonalize`` the optional step 5 replaces the sign update:
        ``W <- W - eta * NS(vote)`` per matrix."""
        if fused and not reorthogonalize:
            _abi.vote_and_update(W, bits, self.eta)
            return
        if vote_out is None:
            vote_out = torch.empty(self.nwords, dtype=torch.int64, device=self.device)
        _abi.majority_vote(bits, vote_out)
        if reorthogonalize:
            self.reorthogonalized_update(W, vote_out)
        else:
            _abi.apply_update(W, vote_out, self.eta)

    def reorthogonalized_update(self, W: torch.Tensor, vote: torch.Tensor) -> None:
        """Step 5 of the summary's flow (optional): the vote as a +-1 matrix per
        weight matrix, orthogonalised locally, then ``W <- W - eta * NS(S_bar)``.
        The direction is left in ``self.U``."""
        if getattr(self, "_sbar", None) is None:
            self._sbar = torch.empty(self.numel, dtype=self.U.dtype, device=self.device)
            probs = self._sbar_problems()
            nbytes = _abi.ns_workspace_bytes(probs, self.precision)
            self._sbar_ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=self.device)
        _abi.unpack_signs(vote, self._sbar)
        a, b, c = self.coeffs
        _abi.ns_orthogonalize(self._sbar_problems(), a, b, c, self.ns_steps, self.precision,
                              self._sbar_ws)
        _abi.apply_update_dense(W, self.U, self.eta)

    def _sbar_problems(self):
        # the norm of a +-1 matrix is sqrt(rows * cols); the library forms it
        probs = []
        for j, (r, c) in enumerate(self.shapes):
            lo, hi = self.offsets_host[j], self.offsets_host[j + 1]
            probs.append((self._sbar[lo:hi].view(r, c), self.U[lo:hi].view(r, c), None))
        return probs
