"""Host-side checks of libmuon (no GPU): exports, argument validation, workspace sizing.

Every call here fails validation (or is a pure size query) before the
library touches the HIP runtime, so nothing is launched.
"""
import ctypes
import os
import re

import numpy as np
import pytest

import matrix_aware_optimizer_amd as mao
from matrix_aware_optimizer_amd import _abi

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "muon.h")

OK, EINVAL, EDTYPE, EALIGN, EWORKSPACE = 0, -1, -2, -3, -4
A1, A2, A3 = ctypes.c_void_p(0x10000), ctypes.c_void_p(0x20000), ctypes.c_void_p(0x30000)
MISALIGNED = ctypes.c_void_p(0x10008)


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s+(\w+)\s*\(", text, flags=re.M)))


@pytest.fixture(scope="module")
def L():
    return mao.lib()


def test_every_declared_symbol_is_exported_and_bound(L):
    names = declared_functions()
    assert len(names) >= 14
    for name in names:
        assert hasattr(L, name), f"{name} declared in muon.h but not exported"
    assert sorted(_abi.SIGNATURES) == names


def test_status_strings(L):
    for code in [0, -1, -2, -3, -4, -5, -6, -7]:
        assert mao.status_string(code)
    assert mao.status_string(-99) == "unknown status"
    assert mao.muon_version() >= 100


def test_momentum_validation(L):
    f = L.muon_momentum
    assert f(None, 1, A2, 1, 100, None, 0, 0.9, 0.1, None, None, 0, None) == EINVAL
    assert f(A1, 1, A2, 1, -1, None, 0, 0.9, 0.1, None, None, 0, None) == EINVAL
    assert f(A1, 5, A2, 1, 100, None, 0, 0.9, 0.1, None, None, 0, None) == EDTYPE
    assert f(MISALIGNED, 1, A2, 1, 100, None, 0, 0.9, 0.1, None, None, 0, None) == EALIGN
    # norms requested: offsets and workspace are required and sized
    assert f(A1, 1, A2, 1, 100, None, 1, 0.9, 0.1, A3, None, 0, None) == EINVAL
    need = L.muon_momentum_workspace_bytes(100, 1)
    assert need >= 16
    assert f(A1, 1, A2, 1, 100, A3, 1, 0.9, 0.1, A3, A3, need - 1, None) == EWORKSPACE
    assert f(A1, 1, A2, 1, 0, None, 0, 0.9, 0.1, None, None, 0, None) == OK   # empty: no launch


def test_momentum_workspace_formula(L):
    # one double per 4096-entry chunk and per segment, plus one, rounded to 256 bytes
    for numel, nseg in [(1, 1), (4096, 1), (4097, 2), (58720256, 1), (84934656, 48)]:
        chunks = -(-numel // 4096)
        expect = -(-(chunks + nseg + 1) * 8 // 256) * 256
        assert L.muon_momentum_workspace_bytes(numel, nseg) == expect


def test_pack_vote_update_validation(L):
    assert L.sign_pack(A1, 1, -5, A2, None) == EINVAL
    assert L.sign_pack(A1, 9, 64, A2, None) == EDTYPE
    assert L.sign_pack(A1, 1, 64, MISALIGNED, None) == EALIGN
    assert L.sign_pack(None, 1, 64, A2, None) == EINVAL
    assert L.sign_pack(None, 1, 0, None, None) == OK
    assert L.majority_vote(A1, 0, 10, A2, None) == EINVAL
    assert L.majority_vote(A1, 1024, 10, A2, None) == EINVAL
    assert L.majority_vote(MISALIGNED, 3, 10, A2, None) == EALIGN
    assert L.apply_update(A1, 3, 10, A2, 0.1, None) == EDTYPE
    assert L.apply_update(A1, 1, 10, None, 0.1, None) == EINVAL
    assert L.vote_and_update(A1, 1, 10, A2, 0, 0.1, None) == EINVAL
    assert L.vote_and_update(A1, 1, 10, MISALIGNED, 3, 0.1, None) == EALIGN


def test_stage_validation(L):
    assert L.ns_gram(A1, A2, 250, 512, 1, 1, None, None, 0, None) == EINVAL      # s not padded
    assert L.ns_gram(A1, A2, 512, 256, 1, 1, None, None, 0, None) == EINVAL      # s > l
    assert L.ns_gram(A1, A2, 256, 512, 1, 7, None, None, 0, None) == EDTYPE
    assert L.ns_gram(A1, A2, 256, 512, 1, 0, A3, None, 0, None) == EDTYPE        # folded scaling: bf16 only
    assert L.ns_poly(A1, MISALIGNED, 256, 1, 1.0, 1.0, 1, None, 0, None) == EALIGN
    assert L.ns_apply(A1, A2, None, None, None, 256, 256, 1, 1.0, 1.0, 1, None, None, 0, None) == EINVAL
    assert L.ns_apply(A1, A2, None, A3, None, 256, 256, 1, 1.0, 1.0, 0, A3, None, 0, None) == EDTYPE
    # bf16 residuals: bf16 only, 16-byte aligned
    assert L.ns_apply(A1, A2, A1, A3, None, 256, 256, 1, 1.0, 1.0, 0, None, None, 0, None) == EDTYPE
    assert L.ns_apply(A1, A2, None, A3, A1, 256, 256, 1, 1.0, 1.0, 0, None, None, 0, None) == EDTYPE
    assert L.ns_apply(A1, A2, MISALIGNED, A3, None, 256, 256, 1, 1.0, 1.0, 1, None, None, 0, None) == EALIGN
    assert L.ns_apply(A1, A2, None, A3, MISALIGNED, 256, 256, 1, 1.0, 1.0, 1, None, None, 0, None) == EALIGN
    assert L.ns_normalize(A1, 1, 0, 5, 1, A2, A3, 1, None) == EINVAL
    assert L.ns_gram(A1, A2, 256, 256, 0, 1, None, None, 0, None) == OK           # empty batch: no launch
    # a stage workspace, when given, must be large enough and aligned
    need = L.ns_stage_workspace_bytes(4096, 14336, 1, 1)
    assert L.ns_gram(A1, A2, 4096, 14336, 1, 1, None, A3, need - 1, None) == EWORKSPACE
    assert L.ns_apply(A1, A2, None, A3, None, 4096, 14336, 1, 1.0, 1.0, 1, None, A1, need - 1, None) == EWORKSPACE
    assert L.ns_gram(A1, A2, 4096, 14336, 1, 1, None, MISALIGNED, need, None) == EALIGN


def test_stage_workspace_bytes(L):
    """Split scratch: 1024 bytes of arrival counters and the error word, then one fp32 256 x 256 partial
    tile per split tile.  Only symmetric products with a contraction of at least
    8192 whose n_p^2 units (n_p = s / 256) fit one round of 256 CUs split: the Gram
    of 4096 x 14336 splits its 120 off-diagonal tiles; fp32 never splits."""
    tile = 256 * 256 * 4
    assert L.ns_stage_workspace_bytes(4096, 14336, 1, 1) == 1024 + 120 * tile
    assert L.ns_stage_workspace_bytes(4096, 14336, 1, 0) == 0
    assert L.ns_stage_workspace_bytes(4096, 4096, 1, 1) == 0                 # contraction too short
    assert L.ns_stage_workspace_bytes(7168, 18432, 1, 1) == 0                # 28^2 units > 256
    assert L.ns_stage_workspace_bytes(1024, 8192, 3, 1) == 1024 + 18 * tile  # 16 x 3 units
    assert L.ns_stage_workspace_bytes(1024, 8192, 17, 1) == 0                # 16 x 17 units > 256
    assert L.ns_stage_workspace_bytes(256, 8192, 5, 1) == 0                  # diagonal units only
    assert L.ns_stage_workspace_bytes(768, 2304, 12, 1) == 0
    assert L.ns_stage_workspace_bytes(250, 512, 1, 1) == 0                   # invalid shape


def _problems(specs):
    arr = (_abi.NSProblem * len(specs))()
    for i, spec in enumerate(specs):
        M, U, s, r, c, md, ud = spec[:7]
        arr[i].M, arr[i].U, arr[i].sumsq = M, U, s
        arr[i].rows, arr[i].cols, arr[i].m_dtype, arr[i].u_dtype = r, c, md, ud
        arr[i].bits = spec[7] if len(spec) > 7 else None
    return arr


def _ns_bytes(count, s, l, es=2, sumsq=True, part=0, split=0):
    """Run buffers (two X, the bf16 residual of X, A, B, sums, norm partials) after
    the split scratch: 1024 bytes of counters and error word (always there), then
    one fp32 256 x 256 partial tile per split tile."""
    def up(x):
        return -(-x // 256) * 256
    scratch = 1024 + split * 256 * 256 * 4
    residual = up(count * s * l * es) if es == 2 else 0
    return (scratch + 2 * up(count * s * l * es) + residual + 2 * up(count * s * s * es)
            + (0 if sumsq else up(4 * count)) + up(part))


def test_ns_workspace_single_and_padding(L):
    arr = _problems([(0x10000, 0x20000, 0x30000, 4096, 14336, 1, 1)])
    # split tiles: the Gram's 120 off-diagonal tiles
    assert L.ns_workspace_bytes(arr, 1, 1) == _ns_bytes(1, 4096, 14336, split=120)
    arr = _problems([(0x10000, 0x20000, 0x30000, 300, 70, 1, 1)])    # tall, ragged
    # a short side below 96 runs on the fp32 products, also when bf16 is asked for
    assert L.ns_bf16_min_side() == 96
    assert L.ns_workspace_bytes(arr, 1, 1) == _ns_bytes(1, 256, 512, es=4)
    assert L.ns_workspace_bytes(arr, 1, 0) == _ns_bytes(1, 256, 512, es=4)
    arr = _problems([(0x10000, 0x20000, 0x30000, 300, 96, 1, 1)])    # tall, ragged, bf16 products
    assert L.ns_workspace_bytes(arr, 1, 1) == _ns_bytes(1, 256, 512)
    assert L.ns_workspace_bytes(arr, 0, 1) == 0
    assert L.ns_workspace_bytes(arr, 1, 9) == 0


def test_ns_grouping_batches_evenly_spaced_problems(L):
    # 12 layers x {768x2304, 768x768, 768x3072, 3072x768} laid out flat, given in layer order
    shapes = [(768, 2304), (768, 768), (768, 3072), (3072, 768)] * 12
    off, specs = 0, []
    for j, (r, c) in enumerate(shapes):
        specs.append((0x100000 + 2 * off, 0x40000000 + 2 * off, 0x80000 + 4 * j, r, c, 1, 1))
        off += r * c
    arr = _problems(specs)
    # four runs (the wide and the tall 768 x 3072 ones are separate runs) on two lanes,
    # largest first onto the lane with less work: lane 0 gets 768x3072 and 768x2304,
    # lane 1 3072x768 and 768x768.  Each lane has its own counters and run buffers,
    # lane 0's sized for every run (the largest: 12 matrices of 768x3072)
    assert L.ns_workspace_bytes(arr, 48, 1) == 2 * _ns_bytes(12, 768, 3072)
    # irregular spacing defeats batching: every problem is its own run
    specs2 = [(M + (j * j % 7) * 4096 * 0, U, s, r, c, md, ud) for j, (M, U, s, r, c, md, ud) in enumerate(specs)]
    specs2[1] = (specs2[1][0], specs2[1][1] + 16, specs2[1][2], *specs2[1][3:])
    arr2 = _problems(specs2)
    assert L.ns_workspace_bytes(arr2, 48, 1) == 2 * _ns_bytes(12, 768, 3072)   # five runs, lane 1 gets 3072x768
    # without norms the run also holds its sums and partial sums
    specs3 = [(M, U, None, r, c, md, ud) for (M, U, s, r, c, md, ud) in specs[:1]]
    part = L.muon_momentum_workspace_bytes(768 * 2304, 1)
    assert L.ns_workspace_bytes(_problems(specs3), 1, 1) == _ns_bytes(1, 768, 2304, sumsq=False, part=part)


def test_ns_orthogonalize_validation(L):
    arr = _problems([(0x10000, 0x20000, 0x30000, 512, 1024, 1, 1)])
    need = L.ns_workspace_bytes(arr, 1, 1)
    f = L.ns_orthogonalize
    assert f(arr, 1, 1.0, 1.0, 1.0, 5, 1, A3, need - 1, None) == EWORKSPACE
    assert f(arr, 1, 1.0, 1.0, 1.0, 5, 1, None, need, None) == EWORKSPACE
    assert f(arr, 1, 1.0, 1.0, 1.0, -1, 1, A3, need, None) == EINVAL
    assert f(arr, 1, 1.0, 1.0, 1.0, 5, 4, A3, need, None) == EDTYPE
    bad = _problems([(0x10008, 0x20000, 0x30000, 512, 1024, 1, 1)])
    assert f(bad, 1, 1.0, 1.0, 1.0, 5, 1, A3, need, None) == EALIGN
    bad = _problems([(0x10000, 0x20000, 0x30000, 0, 1024, 1, 1)])
    assert f(bad, 1, 1.0, 1.0, 1.0, 5, 1, A3, need, None) == EINVAL
    bad = _problems([(0x10000, 0x20000, 0x30000, 8, 8, 1, 3)])
    assert f(bad, 1, 1.0, 1.0, 1.0, 5, 1, A3, need, None) == EDTYPE
    assert f(arr, 0, 1.0, 1.0, 1.0, 5, 1, None, 0, None) == OK


def test_ns_orthogonalize_sign_bits_validation(L):
    """U may be NULL only where the signs come from the last product's epilogue:
    bf16 products (bf16 precision and a short side of at least 96), steps > 0,
    rows <= cols and cols % 64 == 0."""
    f = L.ns_orthogonalize
    ok = _problems([(0x10000, None, 0x30000, 512, 1024, 1, 1, 0x40000)])
    need = L.ns_workspace_bytes(ok, 1, 1)
    assert need == _ns_bytes(1, 512, 1024)                     # the signs need no workspace
    assert f(ok, 1, 1.0, 1.0, 1.0, 5, 1, A3, need - 1, None) == EWORKSPACE   # passes validation
    assert f(ok, 1, 1.0, 1.0, 1.0, 5, 0, A3, need, None) == EINVAL           # f32: not fused, U needed
    assert f(ok, 1, 1.0, 1.0, 1.0, 0, 1, A3, need, None) == EINVAL           # steps == 0: U needed
    tall = _problems([(0x10000, None, 0x30000, 1024, 512, 1, 1, 0x40000)])
    assert f(tall, 1, 1.0, 1.0, 1.0, 5, 1, A3, need, None) == EINVAL
    ragged = _problems([(0x10000, None, 0x30000, 512, 1000, 1, 1, 0x40000)])
    assert f(ragged, 1, 1.0, 1.0, 1.0, 5, 1, A3, need, None) == EINVAL
    small = _problems([(0x10000, None, 0x30000, 95, 1024, 1, 1, 0x40000)])    # fp32 products
    assert f(small, 1, 1.0, 1.0, 1.0, 5, 1, A3, need, None) == EINVAL
    smallest_bf16 = _problems([(0x10000, None, 0x30000, 96, 1024, 1, 1, 0x40000)])
    assert f(smallest_bf16, 1, 1.0, 1.0, 1.0, 5, 1, A3, 16, None) == EWORKSPACE
    neither = _problems([(0x10000, None, 0x30000, 512, 1024, 1, 1)])
    assert L.ns_workspace_bytes(neither, 1, 1) == 0
    assert f(neither, 1, 1.0, 1.0, 1.0, 5, 1, A3, need, None) == EINVAL
    misaligned = _problems([(0x10000, 0x20000, 0x30000, 512, 1024, 1, 1, 0x40004)])
    assert f(misaligned, 1, 1.0, 1.0, 1.0, 5, 1, A3, need, None) == EALIGN


def test_ns_grouping_with_sign_bits(L):
    """Problems with evenly spaced bits (and U, or no U) still form one run;
    bits that break the spacing split it."""
    specs = []
    for j in range(12):
        off = j * 768 * 3072
        specs.append((0x100000 + 2 * off, None, 0x80000 + 4 * j, 768, 3072, 1, 1, 0x8000000 + off // 8))
    assert L.ns_workspace_bytes(_problems(specs), 12, 1) == _ns_bytes(12, 768, 3072)
    with_u = [(M, 0x40000000 + 2 * j * 768 * 3072, *rest) for j, (M, _, *rest) in enumerate(specs)]
    assert L.ns_workspace_bytes(_problems(with_u), 12, 1) == _ns_bytes(12, 768, 3072)
    broken = list(specs)
    broken[6] = (*broken[6][:7], broken[6][7] + 8)
    # runs of 6, 2 (the shifted words and the next) and 4 problems on two lanes: 6 on lane 0,
    # 4 and 2 on lane 1
    assert L.ns_workspace_bytes(_problems(broken), 12, 1) == _ns_bytes(6, 768, 3072) + _ns_bytes(4, 768, 3072)


def test_ns_apply_signs_validation(L):
    f = L.ns_apply_signs
    assert f(A1, A2, None, None, A3, 256, 512, 1, 1.0, 1.0, 0, None, None, 0, None) == EDTYPE   # bf16 only
    assert f(A1, A2, None, None, None, 256, 512, 1, 1.0, 1.0, 1, None, None, 0, None) == EINVAL
    assert f(None, A2, None, None, A3, 256, 512, 1, 1.0, 1.0, 1, None, None, 0, None) == EINVAL
    assert f(A1, A2, None, None, ctypes.c_void_p(0x30004), 256, 512, 1, 1.0, 1.0, 1, None, None, 0, None) == EALIGN
    assert f(A1, A2, None, MISALIGNED, A3, 256, 512, 1, 1.0, 1.0, 1, None, None, 0, None) == EALIGN
    assert f(A1, A2, None, None, A3, 250, 512, 1, 1.0, 1.0, 1, None, None, 0, None) == EINVAL
    assert f(A1, A2, None, None, A3, 256, 512, 0, 1.0, 1.0, 1, None, None, 0, None) == OK      # empty batch
    assert f(A1, A2, MISALIGNED, None, A3, 256, 512, 1, 1.0, 1.0, 1, None, None, 0, None) == EALIGN
    need = L.ns_stage_workspace_bytes(4096, 14336, 1, 1)
    assert f(A1, A2, None, None, A3, 4096, 14336, 1, 1.0, 1.0, 1, None, A1, need - 1, None) == EWORKSPACE


def test_split_status_and_wait_limit_validation(L):
    """ns_workspace_status needs a workspace holding the 1 KB counter block; the
    split wait limit is a non-negative poll count, readable back."""
    assert L.ns_workspace_status(None, 4096, None) == EINVAL
    assert L.ns_workspace_status(A1, 1023, None) == EINVAL
    assert L.ns_workspace_status(MISALIGNED, 4096, None) == EALIGN
    prev = L.muon_get_split_wait_limit()
    assert prev == 1 << 22
    assert L.muon_set_split_wait_limit(-1) == EINVAL
    assert L.muon_get_split_wait_limit() == prev
    assert L.muon_set_split_wait_limit(7) == OK
    assert L.muon_get_split_wait_limit() == 7
    assert mao.set_split_wait_limit(prev) == 7
    assert L.muon_get_split_wait_limit() == prev


def test_binding_rejects_host_tensors():
    import torch
    t = torch.zeros(64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        mao.sign_pack(t, torch.zeros(1, dtype=torch.int64))
    with pytest.raises(TypeError):
        _abi.dtype_code(torch.zeros(2, dtype=torch.float16))


def test_element_count_limit(L):
    """Counts above MUON_MAX_NUMEL (2^38) are rejected before anything launches,
    so no launch grid can exceed its 32-bit limit; the limit itself passes
    validation (the calls below then fail only on their null pointers)."""
    text = open(HEADER).read()
    assert re.search(r"#define MUON_MAX_NUMEL \(INT64_C\(1\) << 38\)", text)
    big = mao.MUON_MAX_NUMEL + 1
    assert mao.MUON_MAX_NUMEL == 1 << 38
    assert L.muon_momentum_workspace_bytes(big, 1) == 0
    assert L.muon_momentum_workspace_bytes(mao.MUON_MAX_NUMEL, 1) > 0
    assert L.muon_momentum(A1, 1, A2, 1, big, None, 0, 0.9, 0.1, None, None, 0, None) == EINVAL
    assert L.sign_pack(A1, 1, big, A2, None) == EINVAL
    assert L.majority_vote(A1, 3, big // 64 + 1, A2, None) == EINVAL
    assert L.majority_vote(None, 3, mao.MUON_MAX_NUMEL // 64, A2, None) == EINVAL   # null, not size
    assert L.apply_update(A1, 1, big, A2, 0.1, None) == EINVAL
    assert L.vote_and_update(A1, 1, big, A2, 3, 0.1, None) == EINVAL
    assert L.sign_int8(A1, 1, big, A2, None) == EINVAL
    assert L.sum_int8(A1, 3, big, A2, None) == EINVAL
    assert L.threshold_pack(A1, big, A2, None) == EINVAL
    assert L.unpack_signs(A1, big, A2, 1, None) == EINVAL
    assert L.apply_update_dense(A1, 1, big, A2, 1, 0.1, None) == EINVAL
    # at the limit the size check passes and the misaligned pointer is what fails
    assert L.sign_pack(MISALIGNED, 1, mao.MUON_MAX_NUMEL, A2, None) == EALIGN
    assert L.apply_update_dense(A1, 1, mao.MUON_MAX_NUMEL, MISALIGNED, 1, 0.1, None) == EALIGN


def test_int8_exchange_validation(L):
    assert L.sign_int8(A1, 1, -1, A2, None) == EINVAL
    assert L.sign_int8(A1, 5, 16, A2, None) == EDTYPE
    assert L.sign_int8(MISALIGNED, 1, 16, A2, None) == EALIGN
    assert L.sign_int8(None, 1, 0, None, None) == OK
    assert L.sum_int8(A1, 0, 16, A2, None) == EINVAL
    assert L.sum_int8(A1, 128, 16, A2, None) == EINVAL          # the int8 sum of 128 signs can overflow
    assert L.sum_int8(A1, 3, 16, MISALIGNED, None) == EALIGN
    assert L.threshold_pack(A1, -1, A2, None) == EINVAL
    assert L.threshold_pack(A1, 10, None, None) == EINVAL
    assert L.threshold_pack(MISALIGNED, 10, A2, None) == EALIGN
    assert mao.MUON_INT8_MAX_VOTERS == 127


def test_reorthogonalisation_validation(L):
    assert L.unpack_signs(A1, -1, A2, 1, None) == EINVAL
    assert L.unpack_signs(A1, 10, A2, 4, None) == EDTYPE
    assert L.unpack_signs(MISALIGNED, 10, A2, 1, None) == EALIGN
    assert L.unpack_signs(None, 0, None, 1, None) == OK
    assert L.apply_update_dense(A1, 1, -3, A2, 1, 0.1, None) == EINVAL
    assert L.apply_update_dense(A1, 1, 10, A2, 7, 0.1, None) == EDTYPE
    assert L.apply_update_dense(A1, 1, 10, MISALIGNED, 1, 0.1, None) == EALIGN
    assert L.apply_update_dense(A1, 1, 10, None, 1, 0.1, None) == EINVAL


def test_dion_validation(L):
    from matrix_aware_optimizer_amd._abi import DionProblem
    arr = (DionProblem * 1)()
    arr[0].M, arr[0].G, arr[0].X, arr[0].Q = 0x10000, 0x20000, 0x30000, 0x40000
    arr[0].rows, arr[0].cols = 768, 3072
    p = ctypes.cast(arr, ctypes.c_void_p)
    need = L.dion_workspace_bytes(p, 1, 192)
    # P twice (m x r) and R (n x r) per run, the Grams and their inverse factors
    # (r x r per matrix), one split-k partial buffer, and the 16 KB page of zeros
    # the DMA-staged products read past the contraction: ranges per product =
    # ceil(512 / output tiles of 64 x 64), at most K / 256 and 16, at least 1
    up = lambda x: -(-x // 256) * 256

    def part(M, N, K, b=1):
        blocks = -(-N // 64) * -(-M // 64) * b
        sp = max(1, min(-(-512 // blocks), max(1, K // 256), 16))
        return sp * b * M * N * 4 if sp > 1 else 0

    m, n, r = 768, 3072, 192
    parts = max(part(m, r, n), part(r, r, m), part(m, r, r), part(n, r, m), part(m, n, r))
    assert parts == 12 * m * r * 4                     # B Q: 36 tiles, 12 k ranges of 256
    assert need == 2 * up(m * r * 4) + up(n * r * 4) + 2 * up(r * r * 4) + up(parts) + 16384
    assert L.dion_workspace_bytes(p, 1, 193) == 0                       # above the LDS limit
    # launch-grid limits: a side above 65535 tiles of 64, more than 4095 problems
    arr[0].rows = 65535 * 64 + 1
    assert L.dion_workspace_bytes(p, 1, 8) == 0
    assert L.dion_step(p, 1, 8, 0.9, 0.1, A3, need, None) == EINVAL
    arr[0].rows = 768
    many = (DionProblem * 4096)()
    for k in range(4096):
        many[k].M, many[k].G, many[k].X, many[k].Q = 0x10000, 0x20000, 0x30000, 0x40000
        many[k].rows, many[k].cols = 64, 64
    pm = ctypes.cast(many, ctypes.c_void_p)
    assert L.dion_workspace_bytes(pm, 4095, 8) > 0
    assert L.dion_workspace_bytes(pm, 4096, 8) == 0
    assert L.dion_step(p, 1, 0, 0.9, 0.1, A3, need, None) == EINVAL
    assert L.dion_step(p, 1, 193, 0.9, 0.1, A3, need, None) == EINVAL
    assert L.dion_step(p, 1, 192, 0.9, 0.1, A3, need - 1, None) == EWORKSPACE
    arr[0].X = 0x30008
    assert L.dion_step(p, 1, 192, 0.9, 0.1, A3, need, None) == EALIGN
    arr[0].X = 0x30000
    arr[0].rows = 0
    assert L.dion_step(p, 1, 192, 0.9, 0.1, A3, need, None) == EINVAL
    assert L.dion_step(p, 0, 192, 0.9, 0.1, None, 0, None) == OK
    assert mao.MUON_DION_MAX_RANK == 192

    # two shapes: the larger run on the caller's stream, the other on the
    # library's second stream, which gets a split-k buffer of its own (the
    # first lane's is sized for both runs)
    two = (DionProblem * 2)()
    for k, (rows, cols) in enumerate([(768, 3072), (256, 512)]):
        two[k].M, two[k].G, two[k].X, two[k].Q = 0x100000 * (k + 1), 0x200000 * (k + 1), 0x300000 * (k + 1), 0x400000 * (k + 1)
        two[k].rows, two[k].cols = rows, cols
    parts_of = lambda M_, N_: max(part(M_, r, N_), part(r, r, M_), part(M_, r, r), part(N_, r, M_), part(M_, N_, r))
    p2 = ctypes.cast(two, ctypes.c_void_p)
    runs = [(768, 3072), (256, 512)]
    bufs = sum(2 * up(mm * r * 4) + up(nn * r * 4) for mm, nn in runs)
    expect = bufs + 2 * up(2 * r * r * 4) + up(max(parts_of(*x) for x in runs)) + up(parts_of(256, 512)) + 16384
    assert parts_of(256, 512) > 0
    assert L.dion_workspace_bytes(p2, 2, 192) == expect


def test_residual_iterations_rule(L):
    """The leading iterations that keep their bf16 residual: the larger of (1) how
    long the typical normalised singular value of a well-conditioned matrix,
    1/sqrt(short side), iterated through p(x) = a x + b x^3 + c x^5, stays below
    the first x with p'(x) <= a / 2 (0.365 for the quintic, 0.708 for the cubic),
    and (2) steps - 2; at most steps - 1.  Short sides under 96 run on fp32
    products, which keep no residual."""
    q, cu = (3.4445, -4.775, 2.0315), (1.5, -0.5, 0.0)
    f = mao.ns_residual_iterations
    assert [f(s, 4 * s, *q, 5) for s in (1, 3, 37, 86, 87, 95, 96, 256, 768, 1020, 1021, 4096, 7168)] == \
        [0, 0, 0, 0, 0, 0, 3, 3, 3, 3, 3, 3, 3]
    assert f(14336, 4096, *q, 5) == 3                    # the short side decides
    assert f(95, 4096, *q, 5) == 0 and f(4096, 95, *q, 5) == 0
    assert f(256, 512, *cu, 5) == 4 and f(256, 512, *cu, 3) == 2 and f(256, 512, *q, 1) == 0
    assert f(256, 512, *q, 2) == 1                       # the typical value: p(1/16) = 0.21 < 0.365
    assert f(4096, 8192, *q, 3) == 2                     # capped at steps - 1
    assert f(96, 1000, *cu, 5) == 4
    assert f(4096, 4096, *q, 5, "f32") == 0               # fp32 products keep no residual
    assert f(4096, 4096, 0.0, 1.0, 1.0, 5) == 0           # no a X term
    assert L.ns_residual_iterations(0, 5, 1.0, 1.0, 1.0, 5, 1) == EINVAL
    assert L.ns_residual_iterations(5, 5, 1.0, 1.0, 1.0, -1, 1) == EINVAL
    assert L.ns_residual_iterations(5, 5, 1.0, 1.0, 1.0, 5, 3) == EDTYPE


def test_noalloc_momentum_validation(L):
    """The allocation-free momentum rejects, before launching anything, what its fixed
    4 MiB scratch cannot hold (workspace_bytes(numel, nseg) > 4 MiB) and the same bad
    arguments as muon_momentum."""
    f = L.muon_momentum_noalloc
    ESCRATCH = -7
    assert mao.status_string(ESCRATCH) != "unknown status"
    cap = 1 << 22
    big = (cap // 8) * 4096                       # nchunks alone fills the array
    assert L.muon_momentum_workspace_bytes(big, 1) > cap
    assert f(A1, 1, A2, 1, big, A3, 1, 0.9, 0.1, A3, None) == ESCRATCH
    fits = ((cap // 8) - 1 - 48) * 4096            # the largest set of 48 matrices that fits
    assert L.muon_momentum_workspace_bytes(fits, 48) == cap
    assert L.muon_momentum_workspace_bytes(fits + 1, 48) > cap
    assert f(A1, 1, A2, 1, fits + 1, A3, 48, 0.9, 0.1, A3, None) == ESCRATCH
    assert f(None, 1, A2, 1, 100, None, 0, 0.9, 0.1, None, None) == EINVAL
    assert f(A1, 5, A2, 1, 100, None, 0, 0.9, 0.1, None, None) == EDTYPE
    assert f(MISALIGNED, 1, A2, 1, 100, None, 0, 0.9, 0.1, None, None) == EALIGN
    assert f(A1, 1, A2, 1, 100, None, 1, 0.9, 0.1, A3, None) == EINVAL        # sums need offsets
    assert f(A1, 1, A2, 1, 100, MISALIGNED, 1, 0.9, 0.1, A3, None) == EALIGN
    assert f(A1, 1, A2, 1, (1 << 38) + 1, None, 0, 0.9, 0.1, None, None) == EINVAL
    assert f(A1, 1, A2, 1, 0, None, 0, 0.9, 0.1, None, None) == OK            # empty: no launch
