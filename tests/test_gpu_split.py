"""GPU parity of the work units that fill the CUs: split symmetric products and
the B X product's last round as column strips.

A symmetric product with a contraction of at least 8192 whose n_p^2 units
(n_p = s / 256) fit one round of the CUs runs each off-diagonal 256 x 256
tile as two halves of the contraction, whose fp32 partials meet through the
workspace, and each diagonal tile as one unit that computes only its lower
half.  Each case is checked against the fp64 oracle at the stage tolerance
(one bf16 rounding of the output), against the same call without splitting
(the halves change only where the fp32 sum is split), for exact symmetry off
the 32 x 32 diagonal blocks, for zero padding, and for the arrival counters
being left at zero.
"""
import numpy as np
import pytest
import torch

import matrix_aware_optimizer_amd as mao
import oracle.muon_oracle as O
from helpers import from_dev, rel_fro, to_dev
from workloads import QUINTIC, random_matrix, store

pytestmark = pytest.mark.gpu

TOL_STAGE = 2.0 ** -8
# split and unsplit sums differ by fp32 reassociation before one bf16 rounding
TOL_SPLIT_VS_WHOLE = 2.0 ** -9


def _counters_clear(ws):
    return not ws[:1024].cpu().numpy().any()


def _X(batch, s, l, seed, sv=None, lv=None):
    sv, lv = sv or s, lv or l
    X = np.zeros((batch, s, l))
    X[:, :sv, :lv] = random_matrix((batch, sv, lv), [320, seed]) / np.sqrt(sv * lv)
    return store(X, "bf16")


def _off_diagonal_block_symmetry(A, s):
    """A equals A^T exactly outside the 32 x 32 blocks on the diagonal (those are
    computed whole; every other block is stored once and mirrored)."""
    mask = np.ones((s, s), bool)
    for k in range(0, s, 32):
        mask[k:k + 32, k:k + 32] = False
    return np.array_equal(A[mask], A.T[mask])


@pytest.mark.parametrize("batch,s,l,sv,lv", [(1, 512, 8192, 512, 8000), (3, 1024, 8192, 1000, 8192),
                                              (1, 4096, 8192, 4096, 8192), (12, 768, 8192, 768, 8192),
                                              (2, 256, 8192, 200, 8192), (1, 4096, 14336, 4096, 14336)])
def test_gram_split_units(batch, s, l, sv, lv):
    Xs = _X(batch, s, l, 1, sv, lv)
    Xd = to_dev(Xs, "bf16").view(batch, s, l)
    ws = mao.new_stage_workspace(s, l, batch)
    A = torch.empty((batch, s, s), dtype=torch.bfloat16, device="cuda")
    A0 = torch.empty_like(A)
    mao.ns_gram(Xd, A, workspace=ws)
    mao.ns_gram(Xd, A0, split=False)
    torch.cuda.synchronize()
    assert _counters_clear(ws)
    raw = from_dev(A).reshape(batch, s, s)
    got = O.decode(raw, "bf16")
    whole = O.decode(from_dev(A0), "bf16").reshape(batch, s, s)
    X = O.decode(Xs, "bf16")
    for b in sorted({0, batch - 1}):
        ref = O.gram(X[b])
        assert rel_fro(got[b], ref) <= TOL_STAGE
        assert rel_fro(got[b], whole[b]) <= TOL_SPLIT_VS_WHOLE
        assert _off_diagonal_block_symmetry(raw[b], s)
        assert not got[b][sv:, :].any() and not got[b][:, sv:].any()      # padding stays zero


def test_gram_split_with_folded_scaling():
    """The first iteration's Gram reads the raw momentum and scales by 1/sum(M^2) in
    both epilogues (the K halves' and the diagonal units')."""
    s, l = 1024, 8192
    M = store(random_matrix((1, s, l), [323, 0]), "bf16")
    Md = to_dev(M, "bf16").view(1, s, l)
    Mf = O.decode(M, "bf16")
    sums = torch.tensor([O.sumsq(Mf[0])], dtype=torch.float32, device="cuda")
    A = torch.empty((1, s, s), dtype=torch.bfloat16, device="cuda")
    mao.ns_gram(Md, A, sumsq=sums)
    got = O.decode(from_dev(A), "bf16").reshape(s, s)
    assert rel_fro(got, O.gram(O.frobenius_normalize(Mf[0]))) <= TOL_STAGE


def test_gram_split_zero_matrix():
    s, l = 512, 8192
    Md = torch.zeros((1, s, l), dtype=torch.bfloat16, device="cuda")
    A = torch.full((1, s, s), 3.0, dtype=torch.bfloat16, device="cuda")
    mao.ns_gram(Md, A, sumsq=torch.zeros(1, dtype=torch.float32, device="cuda"))
    assert not from_dev(A).any()


def test_split_calls_are_repeatable_on_one_workspace():
    """Three Gram calls on one workspace (each leaves the counters at zero) give
    identical bits."""
    s, l = 4096, 8192
    Xd = to_dev(_X(1, s, l, 4), "bf16").view(1, s, l)
    ws = mao.new_stage_workspace(s, l, 1)
    outs = []
    for _ in range(3):
        A = torch.empty((1, s, s), dtype=torch.bfloat16, device="cuda")
        mao.ns_gram(Xd, A, workspace=ws)
        outs.append(from_dev(A))
    torch.cuda.synchronize()
    assert _counters_clear(ws)
    for o in outs[1:]:
        assert np.array_equal(outs[0], o)


@pytest.mark.parametrize("shape", [(1024, 8192), (8192, 1024)])
def test_ns_with_split_gram_matches_oracle(shape):
    """Whole iteration whose Grams split (4^2 units): wide (scaling folded into the first
    iteration) and tall (normalised and transposed first, U transposed back)."""
    M = store(random_matrix(shape, [322, shape[0]]), "bf16")
    Md = to_dev(M, "bf16").view(*shape)
    U = torch.empty(shape, dtype=torch.bfloat16, device="cuda")
    sums = torch.tensor([O.sumsq(O.decode(M, "bf16"))], dtype=torch.float32, device="cuda")
    mao.ns_orthogonalize([(Md, U, sums)], *QUINTIC, 5, "bf16")
    ref = O.newton_schulz(O.decode(M, "bf16"), *QUINTIC, 5)
    assert rel_fro(O.decode(from_dev(U), "bf16"), ref) <= 2e-2


@pytest.mark.parametrize("s,l", [(4096, 14336), (4096, 5120)])
def test_apply_last_round_as_column_strips(s, l):
    """B X on 256 x 256 tiles whose last round would leave half of the 256 CUs idle
    runs that round's column strips as 128 x 256 tiles: 4096 x 14336 has 896 tiles,
    the last 128 (2048 columns) become 256; 4096 x 5120 has 320, the last 64 become
    128.  Both launches write one output; checked against the fp64 product."""
    Xs = _X(1, s, l, 3)
    R = random_matrix((1, s, s), [321, 0]) / np.sqrt(s)
    Bs = store(R + np.transpose(R, (0, 2, 1)), "bf16")
    Xd = to_dev(Xs, "bf16").view(1, s, l)
    out = torch.empty_like(Xd)
    mao.ns_apply(to_dev(Bs, "bf16").view(1, s, s), Xd, out, QUINTIC[0], 1.0)
    got = O.decode(from_dev(out), "bf16").reshape(s, l)
    ref = O.apply_poly(O.decode(Bs, "bf16")[0], O.decode(Xs, "bf16")[0], QUINTIC[0])
    assert rel_fro(got, ref) <= TOL_STAGE
    # the strips of the second launch are checked on their own
    assert rel_fro(got[:, -1024:], ref[:, -1024:]) <= TOL_STAGE


@pytest.mark.parametrize("shape", [(4096, 5120), (5120, 4096)])
def test_ns_final_iteration_through_column_strips(shape):
    """One iteration on 4096 x 5120 (wide, scaling folded in) and 5120 x 4096 (tall:
    the final epilogue writes U transposed): the last 1024 working columns are
    produced by the 128 x 256-tile launch, whose U rows or columns sit at an offset."""
    M = store(random_matrix(shape, [324, shape[0]]), "bf16")
    Md = to_dev(M, "bf16").view(*shape)
    U = torch.empty(shape, dtype=torch.bfloat16, device="cuda")
    mao.ns_orthogonalize([(Md, U, None)], *QUINTIC, 1, "bf16")
    got = O.decode(from_dev(U), "bf16")
    ref = O.newton_schulz(O.decode(M, "bf16"), *QUINTIC, 1)
    # the Newton-Schulz gate (a misplaced strip would give an error of order one)
    assert rel_fro(got, ref) <= 2e-2
    tail = (slice(None), slice(-1024, None)) if shape[0] < shape[1] else (slice(-1024, None), slice(None))
    assert rel_fro(got[tail], ref[tail]) <= 2e-2


@pytest.mark.parametrize("batch,s,sv", [(1, 4096, 4096), (3, 1024, 1000), (12, 768, 768), (1, 512, 512),
                                        (2, 2048, 2048), (1, 256, 256)])
def test_poly_column_halves_and_diagonal_units(batch, s, sv):
    """B = b A + c A^2 as n_p^2 units per matrix when they fit one round of the CUs:
    the two 256 x 128 column halves of every off-diagonal 256 x 256 tile (stored
    and mirrored) and the lower half of every diagonal tile.  4096: 240 + 16 units
    for 256 CUs; 1024 x 3 and 2048 x 2 batched.  768 x 12 and 512 (side below
    1024 and a short contraction) run 128 x 128 tiles instead, and 256 one tile;
    all are checked the same way: against the fp64 product at the stage
    tolerance, for exact symmetry off the 32 x 32 diagonal blocks, and for zero
    padding."""
    R = np.zeros((batch, s, s))
    R[:, :sv, :sv] = random_matrix((batch, sv, sv), [325, s]) / np.sqrt(sv)
    As = store(R + np.transpose(R, (0, 2, 1)), "bf16")
    Ad = to_dev(As, "bf16").view(batch, s, s)
    B = torch.full((batch, s, s), 7.0, dtype=torch.bfloat16, device="cuda")
    b, c = QUINTIC[1], QUINTIC[2]
    mao.ns_poly(Ad, B, b, c)
    raw = from_dev(B).reshape(batch, s, s)
    got = O.decode(raw, "bf16")
    A = O.decode(As, "bf16")
    for k in sorted({0, batch - 1}):
        ref = O.poly(A[k], b, c)
        assert rel_fro(got[k], ref) <= TOL_STAGE
        assert _off_diagonal_block_symmetry(raw[k], s)
        assert not got[k][sv:, :].any() and not got[k][:, sv:].any()


def test_split_wait_that_runs_out_is_reported():
    """A second K half that gives up waiting (forced from the host: a wait limit of 0
    polls, so every kernel still exits normally) leaves its tile unwritten and sets
    the workspace's error word, which ns_workspace_status reports; a fresh workspace
    and the default limit give the normal result and status again.  ns_orthogonalize
    clears the word at the start of each call."""
    batch, s, l = 1, 1024, 8192
    Xd = to_dev(_X(batch, s, l, 9), "bf16").view(batch, s, l)
    good = torch.empty((batch, s, s), dtype=torch.bfloat16, device="cuda")
    mao.ns_gram(Xd, good, split=False)
    sentinel = torch.full_like(good, 7.0)
    ws = mao.new_stage_workspace(s, l, batch)
    prev = mao.set_split_wait_limit(0)
    try:
        mao.ns_gram(Xd, sentinel, workspace=ws)
    finally:
        mao.set_split_wait_limit(prev)
    with pytest.raises(mao.MuonError) as err:
        mao.ns_workspace_status(ws)
    assert err.value.status == -6
    got = from_dev(sentinel).reshape(s, s)
    assert (got == from_dev(torch.full((1,), 7.0, dtype=torch.bfloat16))[0]).any()   # tiles left unwritten
    ws2 = mao.new_stage_workspace(s, l, batch)
    A = torch.empty_like(good)
    mao.ns_gram(Xd, A, workspace=ws2)
    mao.ns_workspace_status(ws2)
    assert _counters_clear(ws2)
    assert rel_fro(O.decode(from_dev(A), "bf16"), O.decode(from_dev(good), "bf16")) <= TOL_SPLIT_VS_WHOLE

    # the whole iteration at a splitting shape: the status of each call
    rows, cols = 1024, 8192
    M = to_dev(store(random_matrix((rows, cols), [321, 0]), "bf16"), "bf16").view(rows, cols)
    U = torch.empty_like(M)
    probs = [(M, U, None)]
    wsn = torch.empty(mao.ns_workspace_bytes(probs), dtype=torch.uint8, device="cuda")
    prev = mao.set_split_wait_limit(0)
    try:
        mao.ns_orthogonalize(probs, *QUINTIC, 5, "bf16", workspace=wsn)
    finally:
        mao.set_split_wait_limit(prev)
    with pytest.raises(mao.MuonError):
        mao.ns_workspace_status(wsn)
    mao.ns_orthogonalize(probs, *QUINTIC, 5, "bf16", workspace=wsn)
    mao.ns_workspace_status(wsn)
    ref = O.newton_schulz(O.decode(from_dev(M), "bf16").reshape(rows, cols), *QUINTIC, 5)
    assert rel_fro(O.decode(from_dev(U), "bf16").reshape(rows, cols), ref) <= 2e-2
