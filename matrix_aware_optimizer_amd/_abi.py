"""ctypes binding of libmuon's C ABI (argument marshalling only).

Every function here has the name of the C entry point it calls, converts
torch tensors to (device pointer, dtype code, size) and the current HIP
stream, and raises :class:`MuonError` on a non-zero status.  No arithmetic
of the method happens in Python, and there is no fallback: if libmuon.so is
missing the first call raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence, Tuple, Union

import torch  # imported first so libmuon binds to the HIP runtime torch loaded

_PKG_DIR = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG_DIR, "libmuon.so")

MUON_F32, MUON_BF16 = 0, 1
MUON_NS_PAD = 256
MUON_MAX_VOTERS = 1023
MUON_MAX_NUMEL = 1 << 38   # largest element count of the elementwise calls

_c_void_p, _c_int, _c_i64, _c_size, _c_float = (ctypes.c_void_p, ctypes.c_int, ctypes.c_int64,
                                                 ctypes.c_size_t, ctypes.c_float)


class MuonError(RuntimeError):
    """A libmuon call returned a non-zero status."""

    def __init__(self, name: str, status: int, text: str):
        super().__init__(f"{name} failed with status {status}: {text}")
        self.status = status


class NSProblem(ctypes.Structure):
    """Mirror of ``struct muon_ns_problem``."""

    _fields_ = [("M", _c_void_p), ("U", _c_void_p), ("sumsq", _c_void_p),
                ("rows", _c_i64), ("cols", _c_i64), ("m_dtype", ctypes.c_int32),
                ("u_dtype", ctypes.c_int32), ("bits", _c_void_p)]


# (name, restype, argtypes) of every exported symbol declared in include/muon.h
SIGNATURES = {
    "muon_status_string": (ctypes.c_char_p, [_c_int]),
    "muon_version": (_c_int, []),
    "muon_time_next_launch": (_c_int, [_c_void_p, _c_void_p]),
    "muon_momentum_workspace_bytes": (_c_size, [_c_i64, _c_int]),
    "muon_momentum": (_c_int, [_c_void_p, _c_int, _c_void_p, _c_int, _c_i64, _c_void_p, _c_int,
                               _c_float, _c_float, _c_void_p, _c_void_p, _c_size, _c_void_p]),
    "muon_momentum_noalloc": (_c_int, [_c_void_p, _c_int, _c_void_p, _c_int, _c_i64, _c_void_p, _c_int,
                                       _c_float, _c_float, _c_void_p, _c_void_p]),
    "ns_workspace_bytes": (_c_size, [ctypes.POINTER(NSProblem), _c_int, _c_int]),
    "ns_orthogonalize": (_c_int, [ctypes.POINTER(NSProblem), _c_int, _c_float, _c_float, _c_float,
                                  _c_int, _c_int, _c_void_p, _c_size, _c_void_p]),
    "ns_normalize": (_c_int, [_c_void_p, _c_int, _c_i64, _c_i64, _c_i64, _c_void_p, _c_void_p,
                              _c_int, _c_void_p]),
    "ns_stage_workspace_bytes": (_c_size, [_c_i64, _c_i64, _c_i64, _c_int]),
    "ns_gram": (_c_int, [_c_void_p, _c_void_p, _c_i64, _c_i64, _c_i64, _c_int, _c_void_p,
                         _c_void_p, _c_size, _c_void_p]),
    "ns_poly": (_c_int, [_c_void_p, _c_void_p, _c_i64, _c_i64, _c_float, _c_float, _c_int,
                         _c_void_p, _c_size, _c_void_p]),
    "ns_apply": (_c_int, [_c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_i64, _c_i64, _c_i64,
                          _c_float, _c_float, _c_int, _c_void_p, _c_void_p, _c_size, _c_void_p]),
    "ns_apply_signs": (_c_int, [_c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_i64, _c_i64,
                                _c_i64, _c_float, _c_float, _c_int, _c_void_p, _c_void_p, _c_size,
                                _c_void_p]),
    "ns_workspace_status": (_c_int, [_c_void_p, _c_size, _c_void_p]),
    "ns_residual_iterations": (_c_int, [_c_i64, _c_i64, _c_float, _c_float, _c_float, _c_int, _c_int]),
    "ns_bf16_min_side": (_c_int, []),
    "muon_set_split_wait_limit": (_c_int, [_c_int]),
    "muon_get_split_wait_limit": (_c_int, []),
    "sign_pack": (_c_int, [_c_void_p, _c_int, _c_i64, _c_void_p, _c_void_p]),
    "majority_vote": (_c_int, [_c_void_p, _c_int, _c_i64, _c_void_p, _c_void_p]),
    "apply_update": (_c_int, [_c_void_p, _c_int, _c_i64, _c_void_p, _c_float, _c_void_p]),
    "vote_and_update": (_c_int, [_c_void_p, _c_int, _c_i64, _c_void_p, _c_int, _c_float,
                                 _c_void_p]),
    "sign_int8": (_c_int, [_c_void_p, _c_int, _c_i64, _c_void_p, _c_void_p]),
    "sum_int8": (_c_int, [_c_void_p, _c_int, _c_i64, _c_void_p, _c_void_p]),
    "threshold_pack": (_c_int, [_c_void_p, _c_i64, _c_void_p, _c_void_p]),
    "unpack_signs": (_c_int, [_c_void_p, _c_i64, _c_void_p, _c_int, _c_void_p]),
    "apply_update_dense": (_c_int, [_c_void_p, _c_int, _c_i64, _c_void_p, _c_int, _c_float, _c_void_p]),
    "dion_workspace_bytes": (_c_size, [ctypes.c_void_p, _c_int, _c_int]),
    "dion_step": (_c_int, [ctypes.c_void_p, _c_int, _c_int, _c_float, _c_float, _c_void_p, _c_size,
                           _c_void_p]),
}

_LIB: Optional[ctypes.CDLL] = None


def lib() -> ctypes.CDLL:
    """Load libmuon.so (once).  Raises if it has not been built."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with `python -m matrix_aware_optimizer_amd.build` "
                "(there is no fallback implementation)")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _LIB = handle
    return _LIB


def status_string(status: int) -> str:
    return lib().muon_status_string(status).decode()


def _check(name: str, status: int) -> None:
    if status != 0:
        raise MuonError(name, status, status_string(status))


def dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return MUON_F32
    if t.dtype == torch.bfloat16:
        return MUON_BF16
    raise TypeError(f"unsupported dtype {t.dtype} (float32 or bfloat16)")


def precision_code(p: Union[str, int]) -> int:
    if isinstance(p, int):
        return p
    return {"f32": MUON_F32, "fp32": MUON_F32, "float32": MUON_F32,
            "bf16": MUON_BF16, "bfloat16": MUON_BF16}[p]


def _dev(t: Optional[torch.Tensor], name: str) -> Optional[int]:
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.data_ptr()


def _stream(stream) -> int:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


def _workspace(nbytes: int, like: torch.Tensor, workspace: Optional[torch.Tensor]) -> torch.Tensor:
    if workspace is not None:
        return workspace
    return torch.empty(max(nbytes, 1), dtype=torch.uint8, device=like.device)


# ---------------------------------------------------------------------------
# a1
# ---------------------------------------------------------------------------

def muon_momentum_workspace_bytes(numel: int, nseg: int) -> int:
    return int(lib().muon_momentum_workspace_bytes(numel, nseg))


def muon_momentum(M: torch.Tensor, G: torch.Tensor, beta: float, alpha: float,
                  seg_offsets: Optional[torch.Tensor] = None,
                  sumsq_out: Optional[torch.Tensor] = None,
                  workspace: Optional[torch.Tensor] = None, stream=None) -> None:
    """``M <- beta*M + alpha*G`` in place; optional per-matrix sum of squares."""
    if M.numel() != G.numel():
        raise ValueError("M and G must have the same number of entries")
    nseg, ws_ptr, ws_bytes = 0, None, 0
    if sumsq_out is not None:
        if seg_offsets is None:
            raise ValueError("seg_offsets is required with sumsq_out")
        nseg = seg_offsets.numel() - 1
        need = muon_momentum_workspace_bytes(M.numel(), nseg)
        workspace = _workspace(need, M, workspace)
        ws_ptr, ws_bytes = _dev(workspace, "workspace"), workspace.numel() * workspace.element_size()
    _check("muon_momentum", lib().muon_momentum(
        _dev(M, "M"), dtype_code(M), _dev(G, "G"), dtype_code(G), M.numel(),
        _dev(seg_offsets, "seg_offsets") if sumsq_out is not None else None, nseg,
        float(beta), float(alpha), _dev(sumsq_out, "sumsq_out"), ws_ptr, ws_bytes, _stream(stream)))


def muon_momentum_noalloc(M: torch.Tensor, G: torch.Tensor, beta: float, alpha: float,
                          seg_offsets: Optional[torch.Tensor] = None,
                          sumsq_out: Optional[torch.Tensor] = None, stream=None) -> None:
    """muon_momentum without a workspace: the library's fixed per-device scratch holds
    the partial sums (nothing is allocated here or in the library).  Calls that overlap
    on one device race."""
    if M.numel() != G.numel():
        raise ValueError("M and G must have the same number of entries")
    nseg = 0
    if sumsq_out is not None:
        if seg_offsets is None:
            raise ValueError("seg_offsets is required with sumsq_out")
        nseg = seg_offsets.numel() - 1
    _check("muon_momentum_noalloc", lib().muon_momentum_noalloc(
        _dev(M, "M"), dtype_code(M), _dev(G, "G"), dtype_code(G), M.numel(),
        _dev(seg_offsets, "seg_offsets") if sumsq_out is not None else None, nseg,
        float(beta), float(alpha), _dev(sumsq_out, "sumsq_out"), _stream(stream)))


# ---------------------------------------------------------------------------
# a2-a5
# ---------------------------------------------------------------------------

# (M, U, sumsq) or (M, U, sumsq, bits); U may be None when bits are given and
# the signs are fused (bf16, wide, cols % 64 == 0, steps > 0)
ProblemLike = Tuple[torch.Tensor, ...]


def _problems(problems: Sequence[ProblemLike]):
    arr = (NSProblem * len(problems))()
    for i, prob in enumerate(problems):
        M, U, sumsq = prob[:3]
        bits = prob[3] if len(prob) > 3 else None
        if M.dim() != 2 or (U is not None and U.shape != M.shape):
            raise ValueError("each problem needs a 2-D M and a U of the same shape")
        if bits is not None and (bits.element_size() != 8 or bits.numel() < packed_words(M.numel())):
            raise ValueError("bits must hold ceil(rows * cols / 64) 64-bit words")
        arr[i].M = _dev(M, "M")
        arr[i].U = _dev(U, "U")
        arr[i].sumsq = _dev(sumsq, "sumsq") if sumsq is not None else None
        arr[i].bits = _dev(bits, "bits")
        arr[i].rows, arr[i].cols = M.shape
        arr[i].m_dtype = dtype_code(M)
        arr[i].u_dtype = dtype_code(U) if U is not None else dtype_code(M)
    return arr


def ns_workspace_bytes(problems: Sequence[ProblemLike], precision="bf16") -> int:
    arr = _problems(problems)
    return int(lib().ns_workspace_bytes(arr, len(problems), precision_code(precision)))


def ns_orthogonalize(problems: Sequence[ProblemLike], a: float, b: float, c: float, steps: int,
                     precision="bf16", workspace: Optional[torch.Tensor] = None,
                     stream=None) -> None:
    """Polar directions of every (M, U, sumsq-or-None) problem, written into U."""
    if len(problems) == 0:
        return
    arr = _problems(problems)
    prec = precision_code(precision)
    need = int(lib().ns_workspace_bytes(arr, len(problems), prec))
    workspace = _workspace(need, problems[0][0], workspace)
    _check("ns_orthogonalize", lib().ns_orthogonalize(
        arr, len(problems), float(a), float(b), float(c), int(steps), prec,
        _dev(workspace, "workspace"), workspace.numel() * workspace.element_size(),
        _stream(stream)))


class PreparedNS:
    """One ns_orthogonalize call whose problem array is marshalled once.

    For a caller that orthogonalises the same device buffers every step (a
    parameter set's momentum, directions and sign words): building the ctypes
    array of a layer set costs the host hundreds of microseconds, long enough
    to leave the GPU idle between the momentum and the first product.  Calling
    the object only enqueues the work, on ``stream`` (default: the current one)."""

    def __init__(self, problems: Sequence[ProblemLike], a: float, b: float, c: float, steps: int,
                 precision="bf16", workspace: Optional[torch.Tensor] = None):
        if len(problems) == 0:
            raise ValueError("no problems")
        self._problems = list(problems)     # keeps the tensors alive
        self._arr = _problems(self._problems)
        self._n = len(self._problems)
        prec = precision_code(precision)
        self._args = (float(a), float(b), float(c), int(steps), prec)
        need = int(lib().ns_workspace_bytes(self._arr, self._n, prec))
        self.workspace = _workspace(need, self._problems[0][0], workspace)
        self._ws = (_dev(self.workspace, "workspace"), self.workspace.numel() * self.workspace.element_size())
        if self._ws[1] < need:
            raise ValueError(f"workspace holds {self._ws[1]} bytes, the call needs {need}")

    def __call__(self, stream=None) -> None:
        _check("ns_orthogonalize", lib().ns_orthogonalize(self._arr, self._n, *self._args, *self._ws,
                                                          _stream(stream)))


def _batch3(t: torch.Tensor) -> Tuple[int, int, int]:
    if t.dim() == 2:
        return 1, t.shape[0], t.shape[1]
    if t.dim() == 3:
        return t.shape[0], t.shape[1], t.shape[2]
    raise ValueError("expected a 2-D or 3-D tensor")


def ns_normalize(M: torch.Tensor, sumsq: torch.Tensor, X0: torch.Tensor, precision="bf16",
                 stream=None) -> None:
    batch, rows, cols = _batch3(M)
    _check("ns_normalize", lib().ns_normalize(
        _dev(M, "M"), dtype_code(M), rows, cols, batch, _dev(sumsq, "sumsq"), _dev(X0, "X0"),
        precision_code(precision), _stream(stream)))


def ns_stage_workspace_bytes(s: int, l: int, batch: int = 1, precision="bf16") -> int:
    return int(lib().ns_stage_workspace_bytes(s, l, batch, precision_code(precision)))


def new_stage_workspace(s: int, l: int, batch: int = 1, precision="bf16", device=None) -> torch.Tensor:
    """Zeroed workspace for the stage calls on [batch][s][l] (its counters start at zero).
    At least the 1024-byte counter block, so that ns_workspace_status can read its
    error word also when nothing splits."""
    n = ns_stage_workspace_bytes(s, l, batch, precision)
    return torch.zeros(max(n, 1024), dtype=torch.uint8, device=device or "cuda")


def _stage_ws(workspace, split: bool, s: int, l: int, batch: int, precision, like: torch.Tensor):
    """(pointer, bytes) of the stage workspace: the caller's, a fresh zeroed one, or none."""
    if not split:
        return None, 0
    if workspace is None:
        workspace = new_stage_workspace(s, l, batch, precision, like.device)
    return _dev(workspace, "workspace"), workspace.numel() * workspace.element_size()


def ns_gram(X: torch.Tensor, A: torch.Tensor, precision="bf16", stream=None,
            sumsq: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
            split: bool = True) -> None:
    """A = X X^T, or M M^T / sumsq with the raw momentum as X.  With split
    (the default) the work is split as ns_orthogonalize splits it, in
    `workspace` (from new_stage_workspace) or a fresh one."""
    batch, s, l = _batch3(X)
    ws, nbytes = _stage_ws(workspace, split, s, l, batch, precision, X)
    _check("ns_gram", lib().ns_gram(_dev(X, "X"), _dev(A, "A"), s, l, batch,
                                    precision_code(precision), _dev(sumsq, "sumsq"), ws, nbytes,
                                    _stream(stream)))


def ns_poly(A: torch.Tensor, B: torch.Tensor, b: float, c: float, precision="bf16",
            stream=None, workspace: Optional[torch.Tensor] = None, split: bool = True) -> None:
    """B = b A + c A A."""
    batch, s, _ = _batch3(A)
    ws, nbytes = _stage_ws(workspace, split, s, s, batch, precision, A)
    _check("ns_poly", lib().ns_poly(_dev(A, "A"), _dev(B, "B"), s, batch, float(b), float(c),
                                    precision_code(precision), ws, nbytes, _stream(stream)))


def ns_apply(B: torch.Tensor, X: torch.Tensor, Xout: torch.Tensor, a: float, alpha: float = 1.0,
             precision="bf16", stream=None, sumsq: Optional[torch.Tensor] = None,
             workspace: Optional[torch.Tensor] = None, split: bool = True,
             X_lo: Optional[torch.Tensor] = None, Xout_lo: Optional[torch.Tensor] = None) -> None:
    """Xout = a X + alpha B X, or (a M + alpha B M) / sqrt(sumsq) with the raw momentum as X.
    With ``X_lo`` the addend is a (X + X_lo); ``Xout_lo`` receives the bf16 rounding
    residual of Xout (bf16 only; the two may be one tensor)."""
    batch, s, l = _batch3(X)
    ws, nbytes = _stage_ws(workspace, split, s, l, batch, precision, X)
    _check("ns_apply", lib().ns_apply(_dev(B, "B"), _dev(X, "X"), _dev(X_lo, "X_lo"), _dev(Xout, "Xout"),
                                      _dev(Xout_lo, "Xout_lo"), s, l, batch, float(a), float(alpha),
                                      precision_code(precision), _dev(sumsq, "sumsq"), ws, nbytes,
                                      _stream(stream)))


def ns_apply_signs(B: torch.Tensor, X: torch.Tensor, Xout: Optional[torch.Tensor], bits: torch.Tensor,
                   a: float, alpha: float = 1.0, precision="bf16", stream=None,
                   sumsq: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                   split: bool = True, X_lo: Optional[torch.Tensor] = None) -> None:
    """ns_apply that also packs the signs of Xout into ``bits`` ([batch][s*l/64] words);
    with Xout None only the signs are written."""
    batch, s, l = _batch3(X)
    if bits.element_size() != 8 or bits.numel() < batch * (s * l // 64):
        raise ValueError("bits must hold batch * s * l / 64 64-bit words")
    ws, nbytes = _stage_ws(workspace, split, s, l, batch, precision, X)
    _check("ns_apply_signs", lib().ns_apply_signs(
        _dev(B, "B"), _dev(X, "X"), _dev(X_lo, "X_lo"), _dev(Xout, "Xout"), _dev(bits, "bits"), s, l,
        batch, float(a), float(alpha), precision_code(precision), _dev(sumsq, "sumsq"), ws, nbytes,
        _stream(stream)))


def ns_workspace_status(workspace: torch.Tensor, stream=None) -> None:
    """Synchronise ``stream`` and raise MuonError (MUON_ESPLIT) if a split product that
    used ``workspace`` gave up waiting for its other half (its tile was not written)."""
    _check("ns_workspace_status", lib().ns_workspace_status(
        _dev(workspace, "workspace"), workspace.numel() * workspace.element_size(), _stream(stream)))


def ns_residual_iterations(rows: int, cols: int, a: float, b: float, c: float, steps: int,
                           precision="bf16") -> int:
    """How many leading iterations of ns_orthogonalize keep the bf16 residual of their output."""
    k = int(lib().ns_residual_iterations(rows, cols, float(a), float(b), float(c), int(steps),
                                         precision_code(precision)))
    if k < 0:
        _check("ns_residual_iterations", k)
    return k


def ns_bf16_min_side() -> int:
    """The shortest short side that ns_orthogonalize runs on bf16 products (smaller
    problems asked for bf16 run on the fp32 products)."""
    return int(lib().ns_bf16_min_side())


def set_split_wait_limit(polls: int) -> int:
    """Set the polls a split product's second half waits for the first (process-wide);
    returns the previous limit."""
    prev = int(lib().muon_get_split_wait_limit())
    _check("muon_set_split_wait_limit", lib().muon_set_split_wait_limit(int(polls)))
    return prev


# ---------------------------------------------------------------------------
# a6-a8
# ---------------------------------------------------------------------------

def packed_words(numel: int) -> int:
    return (numel + 63) // 64


def sign_pack(U: torch.Tensor, bits: torch.Tensor, stream=None) -> None:
    """Pack the signs of U (flat) into ``bits`` (int64/uint64, ceil(numel/64) words)."""
    if bits.numel() < packed_words(U.numel()) or bits.element_size() != 8:
        raise ValueError("bits must hold ceil(numel/64) 64-bit words")
    _check("sign_pack", lib().sign_pack(_dev(U, "U"), dtype_code(U), U.numel(), _dev(bits, "bits"),
                                        _stream(stream)))


def majority_vote(bits: torch.Tensor, out: torch.Tensor, stream=None) -> None:
    """Vote over the rows of ``bits`` ([M, nwords] 64-bit words) into ``out`` ([nwords])."""
    if bits.dim() != 2 or bits.element_size() != 8 or out.numel() < bits.shape[1]:
        raise ValueError("bits must be [M, nwords] 64-bit words and out hold nwords")
    _check("majority_vote", lib().majority_vote(_dev(bits, "bits"), bits.shape[0], bits.shape[1],
                                                _dev(out, "out"), _stream(stream)))


def apply_update(W: torch.Tensor, vote_bits: torch.Tensor, eta: float, stream=None) -> None:
    if vote_bits.numel() < packed_words(W.numel()) or vote_bits.element_size() != 8:
        raise ValueError("vote_bits must hold ceil(numel/64) 64-bit words")
    _check("apply_update", lib().apply_update(_dev(W, "W"), dtype_code(W), W.numel(),
                                              _dev(vote_bits, "vote_bits"), float(eta),
                                              _stream(stream)))


def vote_and_update(W: torch.Tensor, bits: torch.Tensor, eta: float, stream=None) -> None:
    if bits.dim() != 2 or bits.element_size() != 8 or bits.shape[1] != packed_words(W.numel()):
        raise ValueError("bits must be [M, ceil(numel/64)] 64-bit words")
    _check("vote_and_update", lib().vote_and_update(_dev(W, "W"), dtype_code(W), W.numel(),
                                                    _dev(bits, "bits"), bits.shape[0], float(eta),
                                                    _stream(stream)))


def muon_version() -> int:
    return int(lib().muon_version())


def time_next_launch(start: Optional[torch.cuda.Event], stop: Optional[torch.cuda.Event]) -> None:
    """Make the next kernel this thread launches through the library record ``start`` and
    ``stop`` (torch timing events) at its own start and end.  Each event must have been
    recorded once already (torch creates the underlying HIP event on its first record)."""
    handles = []
    for ev in (start, stop):
        if ev is None:
            handles.append(None)
            continue
        h = ev.cuda_event
        if not h:
            raise ValueError("record the event once before passing it (the HIP event is created lazily)")
        handles.append(h)
    _check("muon_time_next_launch", lib().muon_time_next_launch(handles[0], handles[1]))


# ---------------------------------------------------------------------------
# int8 exchange format
# ---------------------------------------------------------------------------

MUON_INT8_MAX_VOTERS = 127


def _int8(t: torch.Tensor, name: str) -> int:
    if t.dtype != torch.int8:
        raise TypeError(f"{name} must be an int8 tensor")
    return _dev(t, name)


def sign_int8(U: torch.Tensor, S: torch.Tensor, stream=None) -> None:
    """S[i] = +1 if !(U[i] < 0) else -1 (int8)."""
    if S.numel() < U.numel():
        raise ValueError("S needs one int8 per entry of U")
    _check("sign_int8", lib().sign_int8(_dev(U, "U"), dtype_code(U), U.numel(), _int8(S, "S"),
                                        _stream(stream)))


def sum_int8(S: torch.Tensor, out: torch.Tensor, stream=None) -> None:
    """out = sum over the rows of S ([M, n] int8), as the SUM all-reduce delivers it."""
    if S.dim() != 2 or out.numel() < S.shape[1]:
        raise ValueError("S must be [M, n] and out hold n entries")
    _check("sum_int8", lib().sum_int8(_int8(S, "S"), S.shape[0], S.shape[1], _int8(out, "out"),
                                      _stream(stream)))


def threshold_pack(total: torch.Tensor, bits: torch.Tensor, stream=None) -> None:
    """Packed vote bits: bit i = 1 iff total[i] >= 0."""
    if bits.numel() < packed_words(total.numel()):
        raise ValueError("bits too small")
    _check("threshold_pack", lib().threshold_pack(_int8(total, "sum"), total.numel(),
                                                  _dev(bits, "bits"), _stream(stream)))


# ---------------------------------------------------------------------------
# local re-orthogonalisation of the vote
# ---------------------------------------------------------------------------

def unpack_signs(vote_bits: torch.Tensor, out: torch.Tensor, stream=None) -> None:
    """out[i] = +1 if vote bit i is set, else -1 (bf16 or fp32)."""
    if vote_bits.numel() < packed_words(out.numel()):
        raise ValueError("vote_bits too small")
    _check("unpack_signs", lib().unpack_signs(_dev(vote_bits, "vote_bits"), out.numel(), _dev(out, "out"),
                                              dtype_code(out), _stream(stream)))


def apply_update_dense(W: torch.Tensor, U: torch.Tensor, eta: float, stream=None) -> None:
    """W <- W - eta * U (one rounding in fp64, then to W's type)."""
    if U.numel() != W.numel():
        raise ValueError("W and U differ in size")
    _check("apply_update_dense", lib().apply_update_dense(_dev(W, "W"), dtype_code(W), W.numel(),
                                                          _dev(U, "U"), dtype_code(U), float(eta),
                                                          _stream(stream)))


# ---------------------------------------------------------------------------
# Dion
# ---------------------------------------------------------------------------

MUON_DION_MAX_RANK = 192


class DionProblem(ctypes.Structure):
    _fields_ = [("M", _c_void_p), ("G", _c_void_p), ("X", _c_void_p), ("Q", _c_void_p),
                ("rows", _c_i64), ("cols", _c_i64)]


def _dion_problems(problems):
    arr = (DionProblem * len(problems))()
    for i, (M, G, X, Q) in enumerate(problems):
        for name, t in (("M", M), ("G", G), ("X", X), ("Q", Q)):
            if t.dtype != torch.float32:
                raise TypeError(f"Dion tensors are fp32 ({name})")
        if M.dim() != 2 or G.shape != M.shape or X.shape != M.shape or Q.dim() != 2 or Q.shape[0] != M.shape[1]:
            raise ValueError("Dion problem shapes: M, G, X m x n and Q n x rank")
        arr[i].M, arr[i].G, arr[i].X, arr[i].Q = (_dev(M, "M"), _dev(G, "G"), _dev(X, "X"), _dev(Q, "Q"))
        arr[i].rows, arr[i].cols = M.shape
    return arr


def dion_workspace_bytes(problems, rank: int) -> int:
    arr = _dion_problems(problems)
    return int(lib().dion_workspace_bytes(ctypes.cast(arr, ctypes.c_void_p), len(problems), int(rank)))


def dion_step(problems, rank: int, mu: float, eta: float, workspace: Optional[torch.Tensor] = None,
              stream=None) -> None:
    """One Dion step on every (M, G, X, Q) problem (fp32 tensors; M, X, Q updated in place)."""
    if not problems:
        return
    arr = _dion_problems(problems)
    nbytes = int(lib().dion_workspace_bytes(ctypes.cast(arr, ctypes.c_void_p), len(problems), int(rank)))
    ws = _workspace(nbytes, problems[0][0], workspace)
    _check("dion_step", lib().dion_step(ctypes.cast(arr, ctypes.c_void_p), len(problems), int(rank),
                                        float(mu), float(eta), _dev(ws, "workspace"),
                                        ws.numel() * ws.element_size(), _stream(stream)))
