"""Pins of the CPU oracle against facts fixed by the pages and by mathematics.

Nothing here compares the oracle with itself: every check is a closed form,
an invariant, a textbook routine (SVD polar factor), brute force over all
bit patterns, or a value worked by hand (tests/golden).  The planted-mistake
tests at the end break one oracle function at a time and show that some pin
then fails.
"""
import json
import math
import os
import struct

import numpy as np
import pytest

import oracle.muon_oracle as O
from workloads import CUBIC, QUINTIC, random_matrix, store

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _orthonormal(n, k, seed):
    q, _ = np.linalg.qr(random_matrix((n, k), [77, seed]))
    return q


def scalar_map(x, coeffs, steps):
    a, b, c = coeffs
    for _ in range(steps):
        x = a * x + b * x ** 3 + c * x ** 5
    return x


# ---------------------------------------------------------------------------
# P-1: closed form.  NS is an odd matrix polynomial X q(X^T X), so with
# X = Q1 diag(s) Q2^T the output is Q1 diag(phi(s / ||s||_2)) Q2^T where phi is
# the steps-fold scalar map x -> a x + b x^3 + c x^5.
# ---------------------------------------------------------------------------

def check_closed_form(shape, coeffs, steps, sigma_seed=0, rank=None):
    r, c = shape
    k = min(r, c) if rank is None else rank
    Q1, Q2 = _orthonormal(r, k, 1 + sigma_seed), _orthonormal(c, k, 2 + sigma_seed)
    sig = np.logspace(-3, 0, k)[::-1] * (1.0 + 0.1 * np.arange(k))
    M = (Q1 * sig) @ Q2.T
    U = O.newton_schulz(M, *coeffs, steps)
    phi = scalar_map(sig / np.linalg.norm(sig), coeffs, steps)
    expect = (Q1 * phi) @ Q2.T
    err = np.linalg.norm(U - expect) / max(np.linalg.norm(expect), 1e-300)
    assert err < 1e-11, f"closed form mismatch {err:.3e} for {shape} {coeffs} steps={steps}"


@pytest.mark.parametrize("shape", [(5, 9), (9, 5), (8, 8), (1, 7), (7, 1), (16, 40)])
@pytest.mark.parametrize("coeffs", [CUBIC, QUINTIC, (2.0, -1.5, 0.5)])
@pytest.mark.parametrize("steps", [0, 1, 5])
def test_closed_form(shape, coeffs, steps):
    check_closed_form(shape, coeffs, steps)


def test_closed_form_rank_deficient():
    check_closed_form((10, 14), QUINTIC, 5, rank=4)
    check_closed_form((14, 10), CUBIC, 3, rank=2)


# ---------------------------------------------------------------------------
# P-2: polar factor.  Cubic (1.5, -0.5, 0) converges to U V^T of the SVD.
# ---------------------------------------------------------------------------

def check_polar(shape, seed):
    M = random_matrix(shape, [91, seed])
    U = O.newton_schulz(M, *CUBIC, 60)
    u, s, vt = np.linalg.svd(M, full_matrices=False)
    polar = u @ vt
    assert np.linalg.norm(U - polar) / np.linalg.norm(polar) < 1e-11
    k = min(shape)
    gram = U.T @ U if shape[0] >= shape[1] else U @ U.T
    assert np.allclose(gram, np.eye(k), atol=1e-11)
    H = U.T @ M                      # symmetric positive semidefinite factor
    assert np.allclose(H, H.T, atol=1e-10)
    assert np.linalg.eigvalsh((H + H.T) / 2).min() > -1e-10


@pytest.mark.parametrize("shape", [(2, 2), (3, 5), (5, 3), (8, 8), (16, 24), (24, 16)])
def test_polar_limit(shape):
    for seed in range(3):
        check_polar(shape, seed)


# ---------------------------------------------------------------------------
# P-3: invariants.
# ---------------------------------------------------------------------------

def test_normalised_spectral_norm_at_most_one():
    for seed in range(5):
        M = random_matrix((12, 30), [5, seed], "student_t3")
        X0 = O.frobenius_normalize(M)
        assert np.linalg.norm(X0, 2) <= 1.0 + 1e-12
        assert abs(np.linalg.norm(X0) - 1.0) < 1e-12


def test_quintic_singular_value_band():
    # max of the 5-fold quintic map on [0, 1] (dense grid): bounds every singular value
    grid = np.linspace(0.0, 1.0, 200001)
    bound = scalar_map(grid, QUINTIC, 5).max()
    assert 1.20 < bound < 1.21
    for seed in range(3):
        M = random_matrix((20, 48), [6, seed])
        s = np.linalg.svd(O.newton_schulz(M, *QUINTIC, 5), compute_uv=False)
        assert s.max() <= bound + 1e-9 and s.min() >= 0.0


def test_cubic_is_contractive_and_monotone():
    M = random_matrix((10, 26), [8, 0])
    s_in = np.linalg.svd(O.frobenius_normalize(M), compute_uv=False)
    s_out = np.linalg.svd(O.newton_schulz(M, *CUBIC, 5), compute_uv=False)
    assert s_out.max() <= 1.0 + 1e-12
    assert np.all(np.diff(s_out) <= 1e-12)          # same order as the inputs
    assert np.all(s_out >= s_in - 1e-12)            # the cubic map never shrinks x in [0, 1]


def test_equivariances():
    M = random_matrix((9, 21), [10, 0])
    U = O.newton_schulz(M, *QUINTIC, 5)
    assert np.allclose(O.newton_schulz(3.7 * M, *QUINTIC, 5), U, atol=1e-12)
    assert np.allclose(O.newton_schulz(-M, *QUINTIC, 5), -U, atol=1e-12)
    assert np.allclose(O.newton_schulz(M.T, *QUINTIC, 5), U.T, atol=1e-12)
    Q1, Q2 = _orthonormal(9, 9, 30), _orthonormal(21, 21, 31)
    assert np.allclose(O.newton_schulz(Q1 @ M @ Q2, *QUINTIC, 5), Q1 @ U @ Q2, atol=1e-11)


def test_stage_products_are_symmetric():
    X = random_matrix((7, 19), [11, 0])
    A = O.gram(X)
    B = O.poly(A, QUINTIC[1], QUINTIC[2])
    assert np.array_equal(A, A.T) or np.allclose(A, A.T, atol=1e-14)
    assert np.allclose(B, B.T, atol=1e-13)
    # U^T X symmetric for the NS output (odd polynomial of X)
    U = O.ns_iterate(O.frobenius_normalize(X), *QUINTIC, 3)
    H = U.T @ X
    assert np.allclose(H, H.T, atol=1e-12)


# ---------------------------------------------------------------------------
# P-4: hand-worked iterations.
# ---------------------------------------------------------------------------

def test_hand_worked_ns():
    d = json.load(open(os.path.join(GOLDEN, "ns_hand.json")))
    for case in d["cases"]:
        M = np.array(case["M_exact"], dtype=np.float64)
        U = O.newton_schulz(M, *case["coeffs"], case["steps"])
        assert np.allclose(U, np.array(case["U"]), rtol=0, atol=1e-12), case["name"]


# ---------------------------------------------------------------------------
# P-5: vote by brute force over every bit pattern.
# ---------------------------------------------------------------------------

def _enumerated_buffers(M):
    n = 1 << M
    j = np.arange(n)
    bufs = np.stack([O.pack_bits(((j >> k) & 1).astype(bool)) for k in range(M)])
    expect = np.array([2 * bin(x).count("1") >= M for x in range(n)])
    return bufs, n, expect


@pytest.mark.parametrize("M", list(range(1, 12)) + [15])
def test_vote_all_patterns(M):
    bufs, n, expect = _enumerated_buffers(M)
    got = O.unpack_bits(O.majority_vote(bufs, n), n)
    assert np.array_equal(got, expect)


# ---------------------------------------------------------------------------
# int8 exchange: the SUM of +-1 signs followed by sign(sum) is the majority
# vote ([SM] "Mecanismo Central" item 3), so for every pattern of M signs
# it must give the same bit as the 1-bit vote; the sum itself is fixed by
# counting: 2 * count(+1) - M, so |sum| <= M and sum = M (mod 2).
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("M", list(range(1, 12)) + [15])
def test_int8_vote_all_patterns(M):
    bufs, n, expect = _enumerated_buffers(M)
    signs = np.stack([np.where(O.unpack_bits(bufs[k], n), 1, -1).astype(np.int8) for k in range(M)])
    total = O.sum_int8(signs)
    plus = np.array([bin(j).count("1") for j in range(n)])
    assert np.array_equal(total.astype(np.int64), 2 * plus - M)
    assert np.array_equal(O.unpack_bits(O.threshold_pack(total), n), expect)


def test_int8_vote_golden_and_limits():
    # hand-worked: three workers, four entries
    U = [np.array([0.5, -1.0, 0.0, -0.0]), np.array([-2.0, -3.0, 1.0, np.nan]),
         np.array([1.0, 4.0, -1.0, -5.0])]
    signs = np.stack([O.sign_int8(u) for u in U])
    assert signs.tolist() == [[1, -1, 1, 1], [-1, -1, 1, 1], [1, 1, -1, -1]]
    assert O.sum_int8(signs).tolist() == [1, -1, 1, 1]
    assert O.unpack_bits(O.threshold_pack(O.sum_int8(signs)), 4).tolist() == [True, False, True, True]
    # 127 workers fit int8; 128 do not
    assert O.sum_int8(np.ones((127, 3), np.int8)).tolist() == [127, 127, 127]
    assert O.sum_int8(-np.ones((127, 1), np.int8)).tolist() == [-127]
    with pytest.raises(ValueError):
        O.sum_int8(np.ones((128, 1), np.int8))
    # an even tie (sum 0) votes +1
    assert O.unpack_bits(O.threshold_pack(np.array([0, -2, 2], np.int8)), 3).tolist() == [True, False, True]


def test_vote_loop_matches_and_textbook_majority():
    rng = np.random.default_rng(3)
    n = 200
    bits = rng.integers(0, 2, size=(3, n)).astype(bool)
    bufs = np.stack([O.pack_bits(b) for b in bits])
    out = O.majority_vote(bufs, n)
    a, b, c = bits
    assert np.array_equal(O.unpack_bits(out, n), (a & b) | (a & c) | (b & c))
    loop = O.majority_vote_loop([[int(w) for w in buf] for buf in bufs], n)
    assert [int(w) for w in out] == loop


def test_vote_properties():
    rng = np.random.default_rng(4)
    n, M = 333, 7
    bits = rng.integers(0, 2, size=(M, n)).astype(bool)
    bufs = np.stack([O.pack_bits(b) for b in bits])
    out = O.majority_vote(bufs, n)
    assert np.array_equal(O.majority_vote(bufs[:1], n), bufs[0])                # M = 1
    assert np.array_equal(O.majority_vote(np.stack([bufs[2]] * 5), n), bufs[2])  # identical
    assert np.array_equal(O.majority_vote(bufs[rng.permutation(M)], n), out)     # order-free
    neg = np.stack([O.pack_bits(~b) for b in bits])                               # odd M
    assert np.array_equal(O.unpack_bits(O.majority_vote(neg, n), n), ~O.unpack_bits(out, n))
    # int8 SUM of +-1 signs, then sign with sign(0) = +1
    s8 = np.where(bits, 1, -1).astype(np.int8).sum(axis=0, dtype=np.int8)
    assert np.array_equal(O.unpack_bits(out, n), s8 >= 0)


def test_vote_golden():
    d = json.load(open(os.path.join(GOLDEN, "bits_hand.json")))["vote"]
    bufs = np.array([int(x, 16) for x in d["buffers"]], dtype=np.uint64)[:, None]
    assert int(O.majority_vote(bufs, d["n"])[0]) == int(d["out_m3"], 16)
    assert int(O.majority_vote(bufs[:2], d["n"])[0]) == int(d["out_m2"], 16)


# ---------------------------------------------------------------------------
# P-6: sign and packing.
# ---------------------------------------------------------------------------

def test_pack_golden_and_sizes():
    d = json.load(open(os.path.join(GOLDEN, "bits_hand.json")))["pack"]
    U = [1.5, -2.0, 0.0, -0.0, float("nan"), -1e-30, 3.0, -0.5]
    U += [1.0 if i % 2 == 0 else -1.0 for i in range(8, 64)]
    U += [-3.0, 2.0, -1.0, -1.0, -1.0, -1.0]
    words = O.sign_pack(np.array(U))
    assert [int(w) for w in words] == [int(x, 16) for x in d["words"]]
    # bf16 storage of the same values packs identically
    from workloads import store
    Ub = O.decode(store(np.array(U), "bf16"), "bf16")
    assert [int(w) for w in O.sign_pack(Ub)] == [int(x, 16) for x in d["words"]]
    for n in [1, 63, 64, 65, 4096 * 14336 // 1024]:
        assert O.pack_bits(np.ones(n, bool)).nbytes == 8 * ((n + 63) // 64)


def test_pack_roundtrip_loop_and_counts():
    rng = np.random.default_rng(5)
    for n in [1, 5, 64, 65, 130, 1000]:
        U = rng.standard_normal(n)
        U[rng.integers(0, n, size=max(1, n // 10))] = 0.0
        bits = O.sign_bits(U)
        words = O.pack_bits(bits)
        assert np.array_equal(O.unpack_bits(words, n), U >= 0)
        assert [int(w) for w in words] == O.pack_bits_loop(list(bits))
        assert sum(bin(int(w)).count("1") for w in words) == int((U >= 0).sum())
        pad = O.unpack_bits(words, len(words) * 64)[n:]
        assert not pad.any()


# ---------------------------------------------------------------------------
# P-7 / P-8 / P-9: update, momentum, norm.
# ---------------------------------------------------------------------------

def test_update_golden():
    d = json.load(open(os.path.join(GOLDEN, "bits_hand.json")))
    f = d["update_f32"]
    W = np.array(f["W"], dtype=np.float32)
    out = O.apply_update(W, "f32", np.array([int(f["vote"], 16)], dtype=np.uint64), f["eta"])
    assert out.tolist() == f["W_new"]
    b = d["update_bf16"]
    Wb = np.array([int(x, 16) for x in b["W_bits"]], dtype=np.uint16)
    out = O.apply_update(Wb, "bf16", np.array([int(b["vote"], 16)], dtype=np.uint64), b["eta"])
    assert [int(x) for x in out] == [int(x, 16) for x in b["W_new_bits"]]


def test_update_properties():
    rng = np.random.default_rng(6)
    n = 500
    W = rng.standard_normal(n).astype(np.float32)
    vote = O.pack_bits(rng.integers(0, 2, n).astype(bool))
    assert np.array_equal(O.apply_update(W, "f32", vote, 0.0), W)
    eta = 0.02
    new = O.apply_update(W, "f32", vote, eta).astype(np.float64)
    s = np.where(O.unpack_bits(vote, n), 1.0, -1.0)
    step = W.astype(np.float64) - new
    assert np.allclose(step, eta * s, rtol=0, atol=np.spacing(np.abs(W)).max() + 1e-9)


def test_momentum_golden_and_special_cases():
    d = json.load(open(os.path.join(GOLDEN, "bits_hand.json")))["momentum"]
    f = d["f32"]
    out = O.momentum(np.array(f["M"], np.float32), "f32", np.array(f["G"], np.float32), "f32",
                     f["beta"], f["alpha"])
    assert out.tolist() == f["M_new"]
    b = d["bf16"]
    Mb = np.array([int(x, 16) for x in b["M_bits"]], np.uint16)
    Gb = np.array([int(x, 16) for x in b["G_bits"]], np.uint16)
    out = O.momentum(Mb, "bf16", Gb, "bf16", b["beta"], b["alpha"])
    assert [int(x) for x in out] == [int(x, 16) for x in b["M_new_bits"]]
    rng = np.random.default_rng(7)
    M = rng.standard_normal(100).astype(np.float32)
    G = rng.standard_normal(100).astype(np.float32)
    alpha = float(np.float32(0.05))
    assert np.array_equal(O.momentum(M, "f32", G, "f32", 0.0, alpha),
                          (np.float32(alpha) * G).astype(np.float32))
    assert np.array_equal(O.momentum(M, "f32", G, "f32", 1.0, 0.0), M)


def test_norm_golden():
    d = json.load(open(os.path.join(GOLDEN, "bits_hand.json")))["norm"]
    M1 = np.array(d["M1"])
    assert O.sumsq(M1) == d["sumsq1"]
    assert np.allclose(O.frobenius_normalize(M1), np.array(d["X0_1"]), atol=1e-15)
    M2 = np.full(d["M2_shape"], d["M2_value"])
    assert O.sumsq(M2) == d["sumsq2"]
    assert math.isclose(math.sqrt(O.sumsq(M2)), 1.5 * math.sqrt(6.0), rel_tol=1e-15)


def test_special_values_follow_sign_rule():
    # NaN anywhere makes the norm NaN, every U entry NaN, every sign +1
    M = random_matrix((4, 6), [12, 0])
    M[1, 2] = np.nan
    U = O.newton_schulz(M, *QUINTIC, 2)
    assert np.isnan(U).all()
    assert O.sign_bits(U).all()
    assert O.sign_bits(np.zeros((3, 3))).all()


# ---------------------------------------------------------------------------
# The whole step, brute force.  For a rank-1 matrix (one row or one column)
# X X^T is the scalar ||X||^2, so after Frobenius scaling every iteration maps
# the single singular value s to a s + b s^3 + c s^5: U = phi(1) * M / ||M||_F
# exactly.  On a flat set of such matrices the whole SignMuon step (momentum,
# per-matrix polar direction, signs, packing, vote, update) can then be worked
# out one entry at a time in plain Python floats.
# ---------------------------------------------------------------------------

def _f32(x):
    """Round a Python float to the nearest binary32 value (ties to even)."""
    return struct.unpack("<f", struct.pack("<f", x))[0]


def _brute_force_step(W, M0, Gs, shapes, beta, alpha, eta, coeffs, steps):
    phi1 = scalar_map(1.0, coeffs, steps)
    sizes = [r * c for r, c in shapes]
    n, workers = sum(sizes), len(Gs)
    dirs, signs = [], []
    for G in Gs:
        m = [_f32(beta * M0[i] + alpha * G[i]) for i in range(n)]
        U, start = [], 0
        for size in sizes:
            seg = m[start:start + size]
            norm = math.sqrt(sum(v * v for v in seg))
            U += [0.0 if norm == 0 else phi1 * v / norm for v in seg]
            start += size
        dirs.append(U)
        signs.append([not (u < 0) for u in U])
    vote = [2 * sum(signs[k][i] for k in range(workers)) >= workers for i in range(n)]
    W_new = [_f32(W[i] - _f32(eta) * (1.0 if vote[i] else -1.0)) for i in range(n)]
    return dirs, signs, vote, W_new


@pytest.mark.parametrize("coeffs,steps", [(CUBIC, 5), (QUINTIC, 5), ((2.0, -1.5, 0.5), 3)])
def test_whole_step_on_rank_one_matrices(coeffs, steps):
    shapes = [(1, 8), (8, 1), (1, 5), (3, 1), (1, 64), (2, 1)]
    n = sum(r * c for r, c in shapes)
    workers = 5
    rng = np.random.default_rng(31)
    W = rng.standard_normal(n).astype(np.float32)
    M0 = rng.standard_normal(n).astype(np.float32)
    Gs = [rng.standard_normal(n).astype(np.float32) for _ in range(workers)]
    # one matrix whose momentum is exactly zero for worker 1 (U = 0, all signs +1)
    M0[8:16] = 0.0
    Gs[1][8:16] = 0.0
    beta, alpha, eta = float(np.float32(0.95)), float(np.float32(0.05)), float(np.float32(0.02))
    out = O.signmuon_step(W, "f32", [M0] * workers, "f32", Gs, "f32", shapes, beta, alpha, eta,
                          *coeffs, steps)
    dirs, signs, vote, W_new = _brute_force_step(W.tolist(), M0.tolist(), [G.tolist() for G in Gs],
                                                 shapes, beta, alpha, eta, coeffs, steps)
    for k in range(workers):
        assert np.allclose(out["U"][k], dirs[k], rtol=1e-12, atol=1e-15)
        assert O.unpack_bits(out["packed"][k], n).tolist() == signs[k]
    assert (np.asarray(out["U"][1][8:16]) == 0).all()
    assert O.unpack_bits(out["vote"], n).tolist() == vote
    assert out["W"].tolist() == W_new


def test_segment_sums_of_squares():
    # constant segments: c^2 * size exactly (every value and sum is a small dyadic number)
    values, sizes = [0.5, -3.0, 0.0, 1.25], [6, 1, 9, 16]
    M = np.concatenate([np.full(sz, v) for v, sz in zip(values, sizes)])
    offsets = np.concatenate([[0], np.cumsum(sizes)])
    assert O.segment_sumsq(M, offsets).tolist() == [v * v * sz for v, sz in zip(values, sizes)]


# ---------------------------------------------------------------------------
# Local re-orthogonalisation of the vote ([SM] Fluxo step 5).  A rank-1 vote
# matrix S = u v^T (u, v vectors of +-1) has the single singular value
# ||S||_F = sqrt(rows * cols), so NS(S) = phi(1) * S / sqrt(rows * cols)
# exactly; the dense update is W - eta * U with one rounding.
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("coeffs,steps", [(QUINTIC, 5), (CUBIC, 3)])
def test_reorthogonalized_direction_on_rank_one_votes(coeffs, steps):
    shapes = [(4, 6), (5, 3), (1, 7)]
    rng = np.random.default_rng(41)
    mats = []
    for r, c in shapes:
        u, v = rng.choice([-1.0, 1.0], r), rng.choice([-1.0, 1.0], c)
        mats.append(np.outer(u, v))
    flat = np.concatenate([m.ravel() for m in mats])
    words = O.pack_bits(flat > 0)
    assert np.array_equal(O.unpack_signs(words, flat.size), flat)
    got = O.reorthogonalized_direction(words, shapes, *coeffs, steps)
    phi1 = scalar_map(1.0, coeffs, steps)
    want = np.concatenate([phi1 * m.ravel() / math.sqrt(m.size) for m in mats])
    assert np.allclose(got, want, rtol=1e-12, atol=1e-15)


def test_apply_update_dense_values():
    W = np.array([1.0, -2.0, 0.5, 3.0], np.float32)
    U = np.array([0.25, -0.5, 0.0, 1.0], np.float32)
    eta = float(np.float32(0.02))
    got = O.apply_update_dense(W, "f32", U, "f32", eta)
    # each difference worked out in float64 then rounded to float32 once
    want = np.array([1.0 - eta * 0.25, -2.0 + eta * 0.5, 0.5, 3.0 - eta], np.float64).astype(np.float32)
    assert got.tolist() == want.tolist()
    assert np.array_equal(O.apply_update_dense(W, "f32", U, "f32", 0.0), W)
    # bf16 storage: 1.0 - 0.02 * 0.25 = 0.995 rounds to the bf16 value 0.99609375
    Wb = store(np.array([1.0]), "bf16")
    Ub = store(np.array([0.25]), "bf16")
    assert O.decode(O.apply_update_dense(Wb, "bf16", Ub, "bf16", eta), "bf16").tolist() == [0.99609375]


# ---------------------------------------------------------------------------
# Dion.  (i) The orthonormalisation is the thin QR factor with a non-negative
# R diagonal: against numpy's QR (a textbook routine) with its signs fixed.
# (ii) Closed form: for B = U diag(s) V^T of rank r and a warm start Q = V,
# the power iteration gives P = U, R = V diag(s), so the error feedback leaves
# M = mu * B, the new Q is V and the update direction is U V^T.
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("shape", [(6, 3), (40, 8), (9, 9)])
def test_dion_orthonormalisation_is_qr(shape):
    P = random_matrix(shape, [60, shape[0]])
    q, r = np.linalg.qr(P)
    q = q * np.sign(np.diag(r))                  # R with a non-negative diagonal
    assert np.allclose(O.orthonormalize_columns(P), q, atol=1e-12)
    # a column that repeats an earlier one comes out zero
    P2 = np.concatenate([P[:, :2], P[:, :1]], axis=1)
    Q2 = O.orthonormalize_columns(P2)
    assert np.allclose(Q2[:, :2], q[:, :2], atol=1e-12)
    assert not Q2[:, 2].any()
    # a zero column stays zero and does not disturb the others
    P3 = P.copy()
    P3[:, 1] = 0.0
    Q3 = O.orthonormalize_columns(P3)
    assert not Q3[:, 1].any() and np.allclose(np.abs(Q3[:, 0]), np.abs(q[:, 0]), atol=1e-12)


def test_dion_column_normalize():
    R = np.array([[3.0, 0.0, 1.0], [4.0, 0.0, -1.0]])
    assert np.allclose(O.column_normalize(R), [[0.6, 0.0, 1 / np.sqrt(2)], [0.8, 0.0, -1 / np.sqrt(2)]])


@pytest.mark.parametrize("m,n,r", [(12, 20, 3), (30, 10, 4)])
def test_dion_step_closed_form_on_rank_r(m, n, r):
    U = np.linalg.qr(random_matrix((m, r), [61, m]))[0]
    V = np.linalg.qr(random_matrix((n, r), [62, n]))[0]
    sv = np.array([4.0, 2.0, 1.0, 0.5][:r])
    B = (U * sv) @ V.T
    # stored fp32 inputs: G = 0 and M = B exactly representable (scaled to a dyadic grid)
    B = np.round(B * 2 ** 20) / 2 ** 20
    M = B.astype(np.float32)
    Bf = M.astype(np.float64)
    # recompute the exact factors of the stored (rounded) B
    u, s_, vt = np.linalg.svd(Bf, full_matrices=False)
    U, sv, V = u[:, :r], s_[:r], vt[:r].T
    X = random_matrix((m, n), [63, 0]).astype(np.float32)
    mu, eta = 0.9, 0.1
    out = O.dion_step(M, np.zeros_like(M), X, V.astype(np.float32), mu, eta)
    # the warm start is V rounded to fp32: compare at that precision
    assert np.allclose(np.abs(out["P"].T @ U), np.eye(r), atol=1e-5)
    assert np.allclose(out["M"], mu * Bf, rtol=1e-5, atol=1e-6 * np.abs(Bf).max())
    signs = np.sign(np.diag(out["P"].T @ U))
    assert np.allclose(out["Q"] * signs, V, atol=1e-5)
    dX = out["X"].astype(np.float64) - X.astype(np.float64)
    assert np.allclose(dX, -eta * U @ V.T, atol=1e-5)


# ---------------------------------------------------------------------------
# Planted mistakes: each breaks one oracle function; some pin must fail.
# ---------------------------------------------------------------------------

def _pins_ns():
    for shape in [(8, 8), (5, 9), (9, 5)]:
        check_closed_form(shape, QUINTIC, 2)
        check_closed_form(shape, (2.0, -1.5, 0.5), 1)
    test_hand_worked_ns()


def _pins_bits():
    test_pack_golden_and_sizes()
    test_pack_roundtrip_loop_and_counts()
    for M in [2, 3, 4, 5]:
        test_vote_all_patterns(M)
    test_vote_golden()
    test_update_golden()
    test_momentum_golden_and_special_cases()


def _pins_step():
    test_whole_step_on_rank_one_matrices(QUINTIC, 5)
    test_segment_sums_of_squares()


def _pins_int8():
    for M in [2, 3, 4, 5]:
        test_int8_vote_all_patterns(M)
    test_int8_vote_golden_and_limits()


def _pins_reorth():
    test_reorthogonalized_direction_on_rank_one_votes(QUINTIC, 5)
    test_apply_update_dense_values()


def _pins_dion():
    for shape in [(6, 3), (40, 8)]:
        test_dion_orthonormalisation_is_qr(shape)
    test_dion_column_normalize()
    test_dion_step_closed_form_on_rank_r(12, 20, 3)


MUTANTS = {
    "dion feedback with mu": ("dion_step", lambda M, G, X, Q, mu, eta: _real_dion(M, G, X, Q, 1.0 - mu, eta),
                              _pins_dion),
    "dion normalises rows": ("column_normalize", lambda R: (np.asarray(R, float).T / np.maximum(
        np.linalg.norm(np.asarray(R, float), axis=1), 1e-300)).T, _pins_dion),
    "dion orth without renormalising": ("orthonormalize_columns", lambda P: np.asarray(P, float), _pins_dion),
    "dense update adds": ("apply_update_dense", lambda W, wd, U, ud, eta: O.round_to_storage(
        O.decode(W, wd).ravel() + float(np.float32(eta)) * O.decode(U, ud).ravel(), wd), _pins_reorth),
    "unpack signs inverted": ("unpack_signs", lambda w, n: np.where(O.unpack_bits(w, n), -1.0, 1.0),
                              _pins_reorth),
    "int8 sign(0) := -1": ("sign_int8", lambda U: np.where(np.asarray(U).ravel() > 0, 1, -1).astype(np.int8),
                           _pins_int8),
    "int8 threshold strict": ("threshold_pack", lambda t: O.pack_bits(np.asarray(t, np.int64) > 0), _pins_int8),
    "direction ignores matrix boundaries": ("worker_direction", lambda M, md, shapes, offs, a, b, c, steps:
        O.newton_schulz(O.decode(M, md).reshape(1, -1), a, b, c, steps).ravel(), _pins_step),
    "segment sums shifted by one entry": ("segment_sumsq", lambda M, offs: np.array(
        [O.sumsq(np.asarray(M)[lo + 1:hi + 1]) for lo, hi in zip(offs[:-1], offs[1:])]), _pins_step),
    "poly drops the c term": ("poly", lambda A, b, c: b * A, _pins_ns),
    "poly flips the sign of b": ("poly", lambda A, b, c: -b * A + c * A @ A, _pins_ns),
    "apply drops aX": ("apply_poly", lambda B, X, a: B @ X, _pins_ns),
    "apply multiplies on the right": ("apply_poly", lambda B, X, a: a * X + X @ B, _pins_ns),
    "gram on the long side": ("gram", lambda X: np.asarray(X).T @ np.asarray(X), _pins_ns),
    "gram without transpose": ("gram", lambda X: np.asarray(X)[:, :X.shape[0]] @ np.asarray(X)[:, :X.shape[0]], _pins_ns),
    "normalise by max entry": ("frobenius_normalize", lambda M: M / np.abs(M).max(), _pins_ns),
    "normalise by squared norm": ("frobenius_normalize", lambda M: M / O.sumsq(M), _pins_ns),
    "sign(0) := -1": ("sign_bits", lambda U: np.asarray(U) > 0, _pins_bits),
    "pack MSB first": ("pack_bits", lambda b: np.packbits(
        np.concatenate([np.asarray(b, bool).ravel(), np.zeros((-len(np.asarray(b).ravel())) % 64, bool)]),
        bitorder="big").view("<u8").astype(np.uint64), _pins_bits),
    "vote strict majority": ("majority_vote", lambda w, n: O.pack_bits(
        2 * np.stack([O.unpack_bits(x, n) for x in np.atleast_2d(w)]).sum(0) > np.atleast_2d(w).shape[0]),
        _pins_bits),
    "update adds the step": ("apply_update", lambda W, dt, v, eta: _wrong_update(W, dt, v, eta), _pins_bits),
    "momentum heavy-ball": ("momentum", lambda M, md, G, gd, beta, alpha: O.round_to_storage(
        beta * O.decode(M, md) + O.decode(G, gd), md), _pins_bits),
}

_REAL_APPLY_UPDATE = O.apply_update
_REAL_DION = O.dion_step


def _real_dion(M, G, X, Q, mu, eta):
    return _REAL_DION(M, G, X, Q, mu, eta)


def _wrong_update(W, dt, v, eta):
    return _REAL_APPLY_UPDATE(W, dt, v, -eta)


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(name, monkeypatch):
    attr, broken, pins = MUTANTS[name]
    monkeypatch.setattr(O, attr, broken)
    with pytest.raises((AssertionError, ValueError)):
        pins()
