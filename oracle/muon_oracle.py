"""Plain CPU oracle of the Muon step with SignMuon's sign / majority-vote tail.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this module.  The product path
(``matrix_aware_optimizer_amd``) never imports, calls or links it, and this
module imports nothing from the product path; the two share only the seeded
input generators in ``workloads``.

Everything is computed in float64 with numpy (``numpy.matmul`` is the only
library routine used for the matrix products), in the order the method states
it.  Bit-level stages (sign, packing, vote, update) are exact and also have
pure-Python loop versions for tiny inputs.

Sources (cited by page title and section):
* [SM]  "SignMuon: Otimização Distribuída de Muon com Eficiência de
  Comunicação" (gist.science technical summary), section 2 "Metodologia:
  Sign-Muon": "Mecanismo Central" items 1-3, "Fluxo Algorítmico
  (Distribuído)" steps 1-4, "Eficiência de Comunicação"; section 3
  "Geometria"; section 4 "nanoGPT" (Frobenius vs spectral scaling,
  iteration count); "Memória e Sobrecarga" (one momentum buffer).
* [MG]  "NVIDIA MegatronによるLLM学習高速化へ向けた新世代オプティマイザの高度化",
  paragraph 「分散モード」 (three matrix products per Newton-Schulz
  iteration) and 「SYRK と融合された all-reduce」 (the first two products
  are symmetric rank-k products writing the full matrix).

Readings where the pages are silent (each is listed with its reason in the
design notes):
* momentum is the EMA ``M <- beta*M + alpha*G`` (the pages name no formula);
* normalisation divides by the Frobenius norm, no epsilon; a zero matrix
  gives ``U = 0``;
* the iteration is ``X <- aX + (bA + cA^2)X`` with ``A = XX^T`` formed on the
  short side (``X^T X`` for tall matrices, an exact identity);
* ``sign(0) := +1``; the sign bit is ``!(u < 0)`` so ``-0.0`` and NaN give +1;
* bits are packed flat row-major, least significant bit first, 64 per word,
  zero padding;
* the vote is ``+1`` iff ``2 * count(+1) >= M`` (a tie gives +1);
* the update is computed in float32 and rounded to the storage type.
"""
from __future__ import annotations

from typing import List, Optional, Sequence, Tuple

import numpy as np

# ---------------------------------------------------------------------------
# Storage types.  The oracle decodes and rounds on its own (it does not use the
# helpers of the input module), so a mistake there cannot hide in both sides.
# ---------------------------------------------------------------------------


def decode(stored: np.ndarray, dtype: str) -> np.ndarray:
    """Exact float64 value of a stored array ("f32": float32, "bf16": uint16 bits)."""
    if dtype == "f32":
        return np.asarray(stored, dtype=np.float32).astype(np.float64)
    if dtype == "bf16":
        bits = np.asarray(stored, dtype=np.uint16).astype(np.uint32)
        return np.left_shift(bits, 16).view(np.float32).astype(np.float64)
    raise ValueError(f"unknown storage type {dtype!r}")


def _f32_to_bf16(x32: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bits, round to nearest with ties to even.

    Written from the definition: keep the upper 16 bits, add one unit of the
    last kept place when the dropped half is above one half, or exactly one
    half with an odd kept part.  NaN stays NaN (quiet bit set).
    """
    u = np.ascontiguousarray(x32, dtype=np.float32).view(np.uint32)
    hi = (u >> 16).astype(np.uint32)
    lo = (u & 0xFFFF).astype(np.uint32)
    round_up = (lo > 0x8000) | ((lo == 0x8000) & ((hi & 1) == 1))
    out = (hi + round_up.astype(np.uint32)).astype(np.uint16)
    nan = np.isnan(x32)
    if nan.any():
        out[nan] = (hi[nan] | 0x40).astype(np.uint16)
    return out


def round_to_storage(x64: np.ndarray, dtype: str) -> np.ndarray:
    """Round float64 to storage: to float32 (nearest-even), then to bfloat16 for "bf16"."""
    with np.errstate(over="ignore", invalid="ignore"):
        x32 = np.asarray(x64, dtype=np.float64).astype(np.float32)
    if dtype == "f32":
        return x32
    if dtype == "bf16":
        return _f32_to_bf16(x32)
    raise ValueError(f"unknown storage type {dtype!r}")


# ---------------------------------------------------------------------------
# a1: momentum.  [SM] Fluxo Algorítmico step 1: each worker updates its local
# momentum M_{t+1}; the formula is not printed, the reading is the EMA.
# ---------------------------------------------------------------------------


def momentum(M_stored: np.ndarray, m_dtype: str, G_stored: np.ndarray, g_dtype: str,
             beta: float, alpha: float) -> np.ndarray:
    """New stored momentum ``round(beta*M + alpha*G)`` (float64 arithmetic)."""
    M = decode(M_stored, m_dtype)
    G = decode(G_stored, g_dtype)
    with np.errstate(over="ignore", invalid="ignore"):
        return round_to_storage(beta * M + alpha * G, m_dtype)


def sumsq(M: np.ndarray) -> float:
    """Sum of squares of all entries (float64) -- the squared Frobenius norm."""
    M = np.asarray(M, dtype=np.float64).ravel()
    with np.errstate(over="ignore", invalid="ignore"):
        return float(np.dot(M, M))


def segment_sumsq(M: np.ndarray, offsets: Sequence[int]) -> np.ndarray:
    """Squared Frobenius norm of every matrix of a flat parameter set."""
    return np.array([sumsq(M[offsets[j]:offsets[j + 1]]) for j in range(len(offsets) - 1)])


# ---------------------------------------------------------------------------
# a2: normalisation.  [SM] section 3 "Geometria" (the direction has spectral
# norm at most 1 after normalisation) and section 4 nanoGPT (Frobenius or
# spectral scaling both work); the Frobenius norm is the reading taken.
# ---------------------------------------------------------------------------


def frobenius_normalize(M: np.ndarray) -> np.ndarray:
    """``X0 = M / ||M||_F``; the zero matrix maps to the zero matrix."""
    M = np.asarray(M, dtype=np.float64)
    s2 = sumsq(M)
    if s2 == 0.0:
        return np.zeros_like(M)
    with np.errstate(over="ignore", invalid="ignore", divide="ignore"):
        return M / np.sqrt(s2)


# ---------------------------------------------------------------------------
# a3-a5: one Newton-Schulz iteration in the three products of [MG] 「分散モード」:
# the Gram matrix, the polynomial in it, and the product with X.
# X is always in short-side orientation here (rows <= cols).
# ---------------------------------------------------------------------------


def gram(X: np.ndarray) -> np.ndarray:
    """a3: ``A = X X^T`` for a wide (or square) X -- symmetric, short side squared."""
    X = np.asarray(X, dtype=np.float64)
    assert X.shape[0] <= X.shape[1], "gram() expects short-side orientation"
    with np.errstate(over="ignore", invalid="ignore"):
        return np.matmul(X, X.T)


def poly(A: np.ndarray, b: float, c: float) -> np.ndarray:
    """a4: ``B = b A + c A A``."""
    A = np.asarray(A, dtype=np.float64)
    with np.errstate(over="ignore", invalid="ignore"):
        return b * A + c * np.matmul(A, A)


def apply_poly(B: np.ndarray, X: np.ndarray, a: float) -> np.ndarray:
    """a5: ``X' = a X + B X``."""
    with np.errstate(over="ignore", invalid="ignore"):
        return a * np.asarray(X, dtype=np.float64) + np.matmul(B, X)


def ns_iterate(X: np.ndarray, a: float, b: float, c: float, steps: int) -> np.ndarray:
    """``steps`` iterations ``X <- aX + b(XX^T)X + c(XX^T)^2 X`` on a short-side X."""
    X = np.asarray(X, dtype=np.float64)
    for _ in range(steps):
        A = gram(X)
        B = poly(A, b, c)
        X = apply_poly(B, X, a)
    return X


def newton_schulz(M: np.ndarray, a: float, b: float, c: float, steps: int) -> np.ndarray:
    """Polar direction ``U`` of one momentum matrix ([SM] Fluxo step 1).

    Normalises by the Frobenius norm, runs the iteration with the Gram matrix
    on the short side (transposing a tall matrix, then transposing back, which
    is exact in real arithmetic since (XX^T)^k X = X (X^T X)^k), and returns
    U in the input's orientation.
    """
    M = np.asarray(M, dtype=np.float64)
    assert M.ndim == 2
    if sumsq(M) == 0.0:
        return np.zeros_like(M)
    X0 = frobenius_normalize(M)
    tall = M.shape[0] > M.shape[1]
    X = X0.T if tall else X0
    U = ns_iterate(X, a, b, c, steps)
    return U.T.copy() if tall else U


# ---------------------------------------------------------------------------
# a6: sign and 1-bit packing.  [SM] Fluxo steps 2-3 (entrywise sign in
# {-1,+1}; the all-gather variant packs one bit per entry) and "Eficiência de
# Comunicação" (1 bit per parameter).
# ---------------------------------------------------------------------------


def sign_bits(U: np.ndarray) -> np.ndarray:
    """Boolean sign per entry: True means +1.  ``!(u < 0)``: 0, -0.0 and NaN give +1."""
    U = np.asarray(U)
    with np.errstate(invalid="ignore"):
        return ~(U < 0)


def pack_bits(bits: np.ndarray) -> np.ndarray:
    """Pack a flat boolean vector: entry i -> word i>>6, bit i&63; padding bits are 0."""
    bits = np.asarray(bits, dtype=bool).ravel()
    n = bits.size
    nwords = (n + 63) // 64
    padded = np.zeros(nwords * 64, dtype=bool)
    padded[:n] = bits
    as_bytes = np.packbits(padded, bitorder="little")
    return as_bytes.view("<u8").astype(np.uint64)


def unpack_bits(words: np.ndarray, n: int) -> np.ndarray:
    """Inverse of :func:`pack_bits` for the first ``n`` entries."""
    w = np.ascontiguousarray(words, dtype="<u8")
    return np.unpackbits(w.view(np.uint8), bitorder="little")[:n].astype(bool)


def pack_bits_loop(bits: Sequence[bool]) -> List[int]:
    """Pure-Python packing (tiny inputs): the same layout, one bit at a time."""
    bits = list(bits)
    words = [0] * ((len(bits) + 63) // 64)
    for i, b in enumerate(bits):
        if b:
            words[i >> 6] |= 1 << (i & 63)
    return words


def sign_pack(U: np.ndarray) -> np.ndarray:
    """a6: packed sign words of a flat (or flattened) direction."""
    return pack_bits(sign_bits(np.asarray(U).ravel()))


# ---------------------------------------------------------------------------
# a7: majority vote.  [SM] "Mecanismo Central" item 3: an integer sum of the
# workers' signs followed by a local threshold sign(sum S^(m)); with
# sign(0) := +1 this is "+1 iff 2*count(+1) >= M".
# ---------------------------------------------------------------------------


def majority_vote(words: np.ndarray, n: int) -> np.ndarray:
    """Vote over ``M`` packed buffers (shape [M, nwords]) for ``n`` entries."""
    words = np.atleast_2d(np.asarray(words, dtype=np.uint64))
    M = words.shape[0]
    signs = np.stack([np.where(unpack_bits(words[k], n), 1, -1) for k in range(M)])
    total = signs.astype(np.int64).sum(axis=0)       # integer SUM of +-1 signs
    return pack_bits(total >= 0)                     # sign(total) with sign(0) = +1


def majority_vote_loop(words: Sequence[Sequence[int]], n: int) -> List[int]:
    """Pure-Python vote (tiny inputs): count the +1 votes of every entry."""
    M = len(words)
    out_bits = []
    for i in range(n):
        count = sum((words[k][i >> 6] >> (i & 63)) & 1 for k in range(M))
        out_bits.append(2 * count >= M)
    return pack_bits_loop(out_bits)


# ---------------------------------------------------------------------------
# a8: update.  [SM] Fluxo step 4: W_{t+1} = W_t - eta_t * S_bar_t.
# ---------------------------------------------------------------------------


def apply_update(W_stored: np.ndarray, w_dtype: str, vote_words: np.ndarray,
                 eta: float) -> np.ndarray:
    """New stored weights: ``round_storage(float32(W) - float32(eta) * S_bar)``.

    ``eta * S_bar`` is exact in float32 (S_bar is +-1), and numpy's float32
    subtraction is one correctly rounded IEEE operation, so this is the exact
    difference rounded once to float32, then (bf16 storage) to bfloat16.
    """
    W32 = decode(W_stored, w_dtype).astype(np.float32)
    n = W32.size
    s = np.where(unpack_bits(vote_words, n), np.float32(1.0), np.float32(-1.0))
    step = np.float32(eta) * s.astype(np.float32)
    with np.errstate(over="ignore", invalid="ignore"):
        new32 = (W32.ravel() - step).astype(np.float32)
    if w_dtype == "f32":
        return new32.reshape(np.shape(W_stored))
    return _f32_to_bf16(new32).reshape(np.shape(W_stored))


# ---------------------------------------------------------------------------
# The int8 exchange format.  [SM] "Mecanismo Central" item 3 and Fluxo step 3
# (the all-reduce variant): every worker sends its signs as int8 values +-1,
# an integer SUM all-reduce adds them, and every worker thresholds the sum
# locally; "Eficiência de Comunicação" puts this at 8 bits per entry (4x
# less than fp32, against 32x for packed bits).  The sum over M <= 127
# workers fits int8.
# ---------------------------------------------------------------------------

INT8_MAX_VOTERS = 127


def sign_int8(U: np.ndarray) -> np.ndarray:
    """+1 / -1 per entry as int8, with the rule of :func:`sign_bits` (+1 iff !(u < 0))."""
    return np.where(sign_bits(np.asarray(U).ravel()), 1, -1).astype(np.int8)


def sum_int8(signs: np.ndarray) -> np.ndarray:
    """Integer SUM over the workers' int8 buffers (shape [M, n]), as the all-reduce gives it."""
    signs = np.atleast_2d(np.asarray(signs, dtype=np.int8))
    if signs.shape[0] > INT8_MAX_VOTERS:
        raise ValueError("the sum of more than 127 signs does not fit int8")
    return signs.astype(np.int64).sum(axis=0).astype(np.int8)


def threshold_pack(total: np.ndarray) -> np.ndarray:
    """Local threshold of the summed signs: +1 iff the sum is >= 0 (sign(0) := +1), packed."""
    return pack_bits(np.asarray(total, dtype=np.int64) >= 0)


# ---------------------------------------------------------------------------
# Local re-orthogonalisation of the vote.  [SM] Fluxo step 5 (optional): each
# worker may apply a local polar step to the aggregated sign matrix, at no
# communication cost.  Reading: per matrix, S_bar (+-1) goes through the same
# Newton-Schulz iteration as the momentum, and the update becomes
# W <- W - eta * NS(S_bar).  ||S_bar||_F = sqrt(rows * cols) exactly.
# ---------------------------------------------------------------------------


def unpack_signs(vote_words: np.ndarray, n: int) -> np.ndarray:
    """The vote as a float64 vector of +1 / -1 (bit 1 -> +1)."""
    return np.where(unpack_bits(vote_words, n), 1.0, -1.0)


def apply_update_dense(W_stored: np.ndarray, w_dtype: str, U_stored: np.ndarray, u_dtype: str,
                       eta: float) -> np.ndarray:
    """New stored weights ``round_storage(W - eta * U)``.

    W, eta and U are fp32 values, so eta * U is exact in float64; the float64
    difference is rounded once, then to float32 (and to bfloat16 for bf16
    storage)."""
    W = decode(W_stored, w_dtype).ravel()
    U = decode(U_stored, u_dtype).ravel()
    eta64 = float(np.float32(eta))
    with np.errstate(over="ignore", invalid="ignore"):
        return round_to_storage(W - eta64 * U, w_dtype).reshape(np.shape(W_stored))


def reorthogonalized_direction(vote_words: np.ndarray, shapes: Sequence[Tuple[int, int]],
                               a: float, b: float, c: float, steps: int) -> np.ndarray:
    """Flat float64 NS(S_bar) of every matrix of the set."""
    sizes = [r * cc for r, cc in shapes]
    n = int(np.sum(sizes))
    S = unpack_signs(vote_words, n)
    out = np.empty(n)
    off = 0
    for (r, cc), size in zip(shapes, sizes):
        out[off:off + size] = newton_schulz(S[off:off + size].reshape(r, cc), a, b, c, steps).ravel()
        off += size
    return out


# ---------------------------------------------------------------------------
# Dion ("대규모 AI 모델 학습을 10배 빠르게: Dion 옵티마이저를 사용한 분산 학습",
# algorithm steps).  Per weight matrix X (m x n) with momentum M, gradient G
# and the previous right factor Q (n x r):
#   B = M + G;  one power iteration warm-started from Q: P = orth(B Q),
#   R = B^T P;  error feedback M = B - (1 - mu) P R^T;
#   Q = ColumnNormalize(R);  X = X - eta P Q^T.
# orth is not spelled out on the page; the reading is the thin QR factor with
# a non-negative diagonal of R (Gram-Schmidt), where a column whose residual
# is at most DEPENDENT_TOL of its own norm counts as dependent on the earlier
# ones and becomes zero.  fp32 storage; arithmetic in float64.
# ---------------------------------------------------------------------------

DEPENDENT_TOL = 1e-4


def orthonormalize_columns(P: np.ndarray) -> np.ndarray:
    """Columns of P made orthonormal in order (modified Gram-Schmidt, done twice)."""
    Q = np.array(P, dtype=np.float64, copy=True)
    r = Q.shape[1]
    keep = np.ones(r, dtype=bool)
    for j in range(r):
        norm0 = np.linalg.norm(Q[:, j])
        for _ in range(2):                      # a second pass restores orthogonality
            for i in range(j):
                if keep[i]:
                    Q[:, j] -= np.dot(Q[:, i], Q[:, j]) * Q[:, i]
        nrm = np.linalg.norm(Q[:, j])
        if nrm <= DEPENDENT_TOL * norm0 or nrm == 0.0:
            keep[j] = False
            Q[:, j] = 0.0
        else:
            Q[:, j] /= nrm
    return Q


def column_normalize(R: np.ndarray) -> np.ndarray:
    """Each column divided by its Euclidean norm; a zero column stays zero."""
    R = np.asarray(R, dtype=np.float64)
    n = np.linalg.norm(R, axis=0)
    return np.where(n > 0, R / np.where(n > 0, n, 1.0), 0.0)


def dion_step(M: np.ndarray, G: np.ndarray, X: np.ndarray, Q: np.ndarray, mu: float,
              eta: float) -> dict:
    """One Dion step on one matrix (fp32 inputs); returns the new stored M, Q, X and P (float64)."""
    B = round_to_storage(decode(M, "f32") + decode(G, "f32"), "f32").astype(np.float64)
    P = orthonormalize_columns(B @ np.asarray(Q, np.float64))
    R = B.T @ P
    M_new = B - (1.0 - mu) * (P @ R.T)
    Q_new = column_normalize(R)
    X_new = decode(X, "f32") - eta * (P @ Q_new.T)
    return {"B": B, "P": P, "M": round_to_storage(M_new, "f32"), "Q": round_to_storage(Q_new, "f32"),
            "X": round_to_storage(X_new, "f32")}


# ---------------------------------------------------------------------------
# The whole step for one worker and for M simulated workers.
# ---------------------------------------------------------------------------


def worker_direction(M_stored: np.ndarray, m_dtype: str, shapes: Sequence[Tuple[int, int]],
                     offsets: Sequence[int], a: float, b: float, c: float,
                     steps: int) -> np.ndarray:
    """Flat float64 polar direction U of a worker's whole (stored) momentum set."""
    Mf = decode(M_stored, m_dtype)
    U = np.empty_like(Mf)
    for j, (r, cc) in enumerate(shapes):
        U[offsets[j]:offsets[j + 1]] = newton_schulz(
            Mf[offsets[j]:offsets[j + 1]].reshape(r, cc), a, b, c, steps).ravel()
    return U


def signmuon_step(W_stored: Optional[np.ndarray], w_dtype: Optional[str],
                  M_stored: Sequence[np.ndarray], m_dtype: str,
                  G_stored: Sequence[np.ndarray], g_dtype: str,
                  shapes: Sequence[Tuple[int, int]], beta: float, alpha: float,
                  eta: float, a: float, b: float, c: float, steps: int) -> dict:
    """One synchronous SignMuon step over ``len(G_stored)`` workers ([SM] Fluxo 1-4).

    Returns the new stored momenta, the float64 directions, every worker's
    packed signs, the packed vote and the new stored weights (None if no W).
    """
    offsets = np.concatenate([[0], np.cumsum([r * c_ for r, c_ in shapes])]).astype(np.int64)
    n = int(offsets[-1])
    new_M, dirs, packed = [], [], []
    for Mk, Gk in zip(M_stored, G_stored):
        Mn = momentum(Mk, m_dtype, Gk, g_dtype, beta, alpha)
        U = worker_direction(Mn, m_dtype, shapes, offsets, a, b, c, steps)
        new_M.append(Mn)
        dirs.append(U)
        packed.append(sign_pack(U))
    packed = np.stack(packed)
    vote = majority_vote(packed, n)
    W_new = None if W_stored is None else apply_update(W_stored, w_dtype, vote, eta)
    return {"M": new_M, "U": dirs, "packed": packed, "vote": vote, "W": W_new}


__all__ = [
    "decode", "round_to_storage", "momentum", "sumsq", "segment_sumsq",
    "frobenius_normalize", "gram", "poly", "apply_poly", "ns_iterate", "newton_schulz",
    "sign_bits", "pack_bits", "unpack_bits", "pack_bits_loop", "sign_pack",
    "majority_vote", "majority_vote_loop", "apply_update", "worker_direction",
    "signmuon_step", "INT8_MAX_VOTERS", "sign_int8", "sum_int8", "threshold_pack",
    "unpack_signs", "apply_update_dense", "reorthogonalized_direction",
    "DEPENDENT_TOL", "orthonormalize_columns", "column_normalize", "dion_step",
]
