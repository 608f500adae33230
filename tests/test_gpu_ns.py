"""GPU parity of the Newton-Schulz stages (a2-a5) and of the whole iteration.

Stage tolerances follow from one rounding of the output to the working type
(bf16: unit roundoff 2^-8 bounds the relative Frobenius error, fp32 2^-23
plus fp32 accumulation); the whole iteration is gated at 2e-2 (bf16) and
1e-4 (fp32) relative Frobenius error against the fp64 oracle fed the same
stored momentum.
"""
import numpy as np
import pytest
import torch

import matrix_aware_optimizer_amd as mao
import oracle.muon_oracle as O
from helpers import from_dev, rel_fro, to_dev
from workloads import CUBIC, QUINTIC, random_matrix, store

pytestmark = pytest.mark.gpu

TOL_STAGE = {"bf16": 2.0 ** -8, "f32": 2e-6}
TOL_NS = {"bf16": 2e-2, "f32": 1e-4}
TORCH = {"bf16": torch.bfloat16, "f32": torch.float32}


def padded(x, s, l):
    out = np.zeros((x.shape[0], s, l))
    out[:, :x.shape[1], :x.shape[2]] = x
    return out


def _stage_X(batch, s, l, sv, lv, prec, seed):
    X = np.zeros((batch, s, l))
    X[:, :sv, :lv] = random_matrix((batch, sv, lv), [300, seed]) / np.sqrt(sv * lv)
    Xs = store(X, prec)
    return Xs, O.decode(Xs, prec)


@pytest.mark.parametrize("prec", ["bf16", "f32"])
@pytest.mark.parametrize("batch,s,l,sv,lv", [(1, 256, 256, 256, 256), (2, 256, 768, 200, 700),
                                              (1, 512, 1024, 512, 1000), (3, 768, 768, 768, 768)])
def test_gram(prec, batch, s, l, sv, lv):
    Xs, X = _stage_X(batch, s, l, sv, lv, prec, 1)
    A = torch.empty((batch, s, s), dtype=TORCH[prec], device="cuda")
    mao.ns_gram(to_dev(Xs, prec).view(batch, s, l), A, prec)
    got = O.decode(from_dev(A), prec).reshape(batch, s, s)
    for b in range(batch):
        ref = O.gram(X[b])
        assert rel_fro(got[b], ref) <= TOL_STAGE[prec]
        assert rel_fro(got[b], got[b].T) <= TOL_STAGE[prec]                 # symmetric
        assert not got[b][sv:, :].any() and not got[b][:, sv:].any()     # padding stays zero


@pytest.mark.parametrize("prec", ["bf16", "f32"])
@pytest.mark.parametrize("coeffs", [QUINTIC, (2.0, -1.5, 0.5)])
@pytest.mark.parametrize("batch,s,sv", [(1, 256, 256), (2, 512, 300), (1, 1024, 1024)])
def test_poly(prec, coeffs, batch, s, sv):
    Xs, X = _stage_X(batch, s, s, sv, sv, prec, 2)
    A = torch.empty((batch, s, s), dtype=TORCH[prec], device="cuda")
    mao.ns_gram(to_dev(Xs, prec).view(batch, s, s), A, prec)
    B = torch.empty_like(A)
    mao.ns_poly(A, B, coeffs[1], coeffs[2], prec)
    Ain = O.decode(from_dev(A), prec).reshape(batch, s, s)
    got = O.decode(from_dev(B), prec).reshape(batch, s, s)
    for b in range(batch):
        ref = O.poly(Ain[b], coeffs[1], coeffs[2])
        assert rel_fro(got[b], ref) <= TOL_STAGE[prec]
        assert not got[b][sv:, :].any() and not got[b][:, sv:].any()


@pytest.mark.parametrize("prec", ["bf16", "f32"])
@pytest.mark.parametrize("a,alpha", [(QUINTIC[0], 1.0), (1.5, -0.5), (0.0, 1.0)])
@pytest.mark.parametrize("batch,s,l,sv,lv", [(1, 256, 256, 256, 256), (2, 256, 768, 200, 700),
                                              (1, 512, 1536, 512, 1536), (1, 2048, 2560, 2000, 2500)])
def test_apply(prec, a, alpha, batch, s, l, sv, lv):
    Xs, X = _stage_X(batch, s, l, sv, lv, prec, 3)
    Bm = np.zeros((batch, s, s))
    R = random_matrix((batch, sv, sv), [301, 0]) / np.sqrt(sv)
    Bm[:, :sv, :sv] = R + np.transpose(R, (0, 2, 1))
    Bs = store(Bm, prec)
    Xd = to_dev(Xs, prec).view(batch, s, l)
    out = torch.empty_like(Xd)
    mao.ns_apply(to_dev(Bs, prec).view(batch, s, s), Xd, out, a, alpha, prec)
    got = O.decode(from_dev(out), prec).reshape(batch, s, l)
    Bd = O.decode(Bs, prec)
    for b in range(batch):
        ref = O.apply_poly(alpha * Bd[b], X[b], a)
        assert rel_fro(got[b], ref) <= TOL_STAGE[prec]
        assert not got[b][sv:, :].any() and not got[b][:, lv:].any()


@pytest.mark.parametrize("prec", ["bf16", "f32"])
@pytest.mark.parametrize("m_dtype", ["bf16", "f32"])
@pytest.mark.parametrize("rows,cols,batch", [(300, 70, 2), (70, 300, 1), (256, 256, 1), (5, 3, 4),
                                            (200, 520, 2), (3072, 768, 1), (768, 3072, 1)])
def test_normalize(prec, m_dtype, rows, cols, batch):
    M = store(random_matrix((batch, rows, cols), [302, rows]), m_dtype)
    Mf = O.decode(M, m_dtype).reshape(batch, rows, cols)
    sums = torch.tensor([O.sumsq(Mf[b]) for b in range(batch)], dtype=torch.float32, device="cuda")
    s, l = min(rows, cols), max(rows, cols)
    sp, lp = -(-s // 256) * 256, -(-l // 256) * 256
    X0 = torch.full((batch, sp, lp), 7.0, dtype=TORCH[prec], device="cuda")
    mao.ns_normalize(to_dev(M, m_dtype).view(batch, rows, cols), sums, X0, prec)
    got = O.decode(from_dev(X0), prec).reshape(batch, sp, lp)
    for b in range(batch):
        ref = O.frobenius_normalize(Mf[b])
        ref = ref.T if rows > cols else ref
        assert np.allclose(got[b][:s, :l], ref, rtol=TOL_STAGE[prec], atol=1e-30)
        assert not got[b][s:, :].any() and not got[b][:, l:].any()


def _ns_gpu(M_list, m_dtype, u_dtype, coeffs, steps, prec, with_sums=True):
    """Run ns_orthogonalize over matrices stored back to back in one flat buffer."""
    flat = np.concatenate([m.ravel() for m in M_list])
    Md = to_dev(flat, m_dtype)
    U = torch.zeros(flat.size, dtype=TORCH[u_dtype], device="cuda")
    sums = torch.tensor([O.sumsq(O.decode(m, m_dtype)) for m in M_list], dtype=torch.float32,
                        device="cuda")
    probs, off = [], 0
    for j, m in enumerate(M_list):
        n = m.size
        probs.append((Md[off:off + n].view(*m.shape), U[off:off + n].view(*m.shape),
                      sums[j:j + 1] if with_sums else None))
        off += n
    mao.ns_orthogonalize(probs, *coeffs, steps, prec)
    out, off = [], 0
    Uh = O.decode(from_dev(U), u_dtype)
    for m in M_list:
        out.append(Uh[off:off + m.size].reshape(m.shape))
        off += m.size
    return out


@pytest.mark.parametrize("shape", [(256, 256), (37, 300), (300, 37), (512, 1536), (1536, 512),
                                   (768, 768), (1, 1), (3, 1000)])
@pytest.mark.parametrize("prec,coeffs", [("f32", CUBIC), ("bf16", QUINTIC), ("f32", QUINTIC),
                                         ("bf16", CUBIC)])
@pytest.mark.parametrize("steps", [0, 1, 5])
def test_ns_matches_oracle(shape, prec, coeffs, steps):
    """bf16 wide shapes with sides that are multiples of 256 take the path that folds the
    Frobenius scaling into the first iteration; the others normalise first."""
    m_dtype = prec
    M = store(random_matrix(shape, [303, shape[0], shape[1]]), m_dtype)
    (U,) = _ns_gpu([M], m_dtype, prec, coeffs, steps, prec)
    ref = O.newton_schulz(O.decode(M, m_dtype), *coeffs, steps)
    assert rel_fro(U, ref) <= TOL_NS[prec], rel_fro(U, ref)


def test_ns_computes_its_own_norm_and_handles_zero():
    Ms = [store(random_matrix((200, 520), [304, 0]), "bf16"),
          store(np.zeros((64, 64)), "bf16"),
          store(random_matrix((520, 200), [304, 1]) * 1e-3, "bf16"),
          store(np.zeros((256, 512)), "bf16"),                          # folded scaling path
          store(random_matrix((256, 768), [304, 2]) * 1e-3, "bf16")]
    got = _ns_gpu(Ms, "bf16", "bf16", QUINTIC, 5, "bf16", with_sums=False)
    assert not got[1].any() and not got[3].any()
    for j in (0, 2, 4):
        ref = O.newton_schulz(O.decode(Ms[j], "bf16"), *QUINTIC, 5)
        assert rel_fro(got[j], ref) <= TOL_NS["bf16"]


@pytest.mark.parametrize("shape", [(100, 300), (256, 512)])
def test_ns_nan_momentum_gives_nan_direction(shape):
    """A NaN makes the norm NaN and, on both the normalising and the folded path, every
    entry of U NaN (so every sign +1), as the oracle's arithmetic gives."""
    M = random_matrix(shape, [313, 0])
    M[3, 7] = np.nan
    (U,) = _ns_gpu([store(M, "bf16")], "bf16", "bf16", QUINTIC, 5, "bf16")
    assert np.isnan(U).all()
    assert np.isnan(O.newton_schulz(O.decode(store(M, "bf16"), "bf16"), *QUINTIC, 5)).all()


@pytest.mark.parametrize("batch,s,l", [(1, 256, 768), (3, 512, 1024)])
def test_stages_with_folded_scaling(batch, s, l):
    """ns_gram / ns_apply given the raw momentum and its sums of squares equal the
    stages on X0 = M / ||M||_F (against the oracle), including a zero matrix."""
    M = random_matrix((batch, s, l), [314, s]) * 0.3
    M[-1] = 0.0
    Ms = store(M, "bf16")
    Mf = O.decode(Ms, "bf16").reshape(batch, s, l)
    sums = torch.tensor([O.sumsq(Mf[b]) for b in range(batch)], dtype=torch.float32, device="cuda")
    Md = to_dev(Ms, "bf16").view(batch, s, l)
    A = torch.empty((batch, s, s), dtype=torch.bfloat16, device="cuda")
    mao.ns_gram(Md, A, "bf16", sumsq=sums)
    R = random_matrix((batch, s, s), [315, 0]) / np.sqrt(s)
    Bs = store(R + np.transpose(R, (0, 2, 1)), "bf16")
    out = torch.empty_like(Md)
    mao.ns_apply(to_dev(Bs, "bf16").view(batch, s, s), Md, out, 1.5, 0.7, "bf16", sumsq=sums)
    gotA = O.decode(from_dev(A), "bf16").reshape(batch, s, s)
    gotX = O.decode(from_dev(out), "bf16").reshape(batch, s, l)
    Bd = O.decode(Bs, "bf16").reshape(batch, s, s)
    for b in range(batch):
        X0 = O.frobenius_normalize(Mf[b])
        if b == batch - 1:
            assert not gotA[b].any() and not gotX[b].any()
            continue
        assert rel_fro(gotA[b], O.gram(X0)) <= TOL_STAGE["bf16"]
        assert rel_fro(gotX[b], O.apply_poly(0.7 * Bd[b], X0, 1.5)) <= TOL_STAGE["bf16"]


def test_ns_batched_interleaved_shapes():
    # layer-ordered problems of two shapes: grouped into two batched runs internally
    shapes = [(256, 768), (768, 256), (256, 256)] * 4
    Ms = [store(random_matrix(s, [305, j]), "bf16") for j, s in enumerate(shapes)]
    got = _ns_gpu(Ms, "bf16", "bf16", QUINTIC, 5, "bf16")
    for M, U in zip(Ms, got):
        ref = O.newton_schulz(O.decode(M, "bf16"), *QUINTIC, 5)
        assert rel_fro(U, ref) <= TOL_NS["bf16"]


def test_ns_many_runs_in_one_call():
    """Six shapes (one tall, one with rows that are not a multiple of the padding), two
    matrices each in layer order: six batched runs of two in one call, one after the
    other through the same workspace.  Every direction against the oracle."""
    shapes = [(256, 256), (256, 512), (200, 768), (256, 1024), (256, 1280), (768, 256)] * 2
    Ms = [store(random_matrix(s, [322, j]), "bf16") for j, s in enumerate(shapes)]
    got = _ns_gpu(Ms, "bf16", "bf16", QUINTIC, 5, "bf16")
    for M, U in zip(Ms, got):
        ref = O.newton_schulz(O.decode(M, "bf16"), *QUINTIC, 5)
        assert rel_fro(U, ref) <= TOL_NS["bf16"]


def test_ns_mixed_dtypes_fp32_momentum_bf16_ops():
    M = store(random_matrix((300, 900), [306, 0], "student_t3"), "f32")
    (U,) = _ns_gpu([M], "f32", "bf16", QUINTIC, 5, "bf16")
    ref = O.newton_schulz(O.decode(M, "f32"), *QUINTIC, 5)
    assert rel_fro(U, ref) <= TOL_NS["bf16"]


@pytest.mark.parametrize("prec,coeffs,steps,lo", [("f32", CUBIC, 30, -2.0), ("f32", QUINTIC, 5, -2.0),
                                                  ("bf16", QUINTIC, 5, -1.0), ("bf16", QUINTIC, 5, -2.0),
                                                  ("bf16", CUBIC, 5, -2.0)])
def test_ns_closed_form_spectrum(prec, coeffs, steps, lo):
    """Singular values spread over one and two decades.  In bf16 the outputs of the
    first three iterations keep their rounding residual (the small directions grow
    about 3.4x per iteration together with any noise picked up while small); without
    it two decades measured 2.03e-2 to 2.55e-2."""
    # known spectrum: U = Q1 phi(sigma/||sigma||) Q2^T (closed form of the iteration)
    r, c = 256, 512
    Q1, _ = np.linalg.qr(random_matrix((r, r), [307, 0]))
    Q2, _ = np.linalg.qr(random_matrix((c, r), [307, 1]))
    sig = np.logspace(lo, 0, r)
    M = store((Q1 * sig) @ Q2.T, prec)
    (U,) = _ns_gpu([M], prec, prec, coeffs, steps, prec)
    x = sig / np.linalg.norm(sig)
    for _ in range(steps):
        x = coeffs[0] * x + coeffs[1] * x ** 3 + coeffs[2] * x ** 5
    expect = (Q1 * x) @ Q2.T
    # the stored M is a rounded copy of the exact one: in bf16 that rounding moves
    # small singular values by more than the gate, so only fp32 meets the exact form
    if prec == "f32":
        assert rel_fro(U, expect) <= TOL_NS[prec]
    assert rel_fro(U, O.newton_schulz(O.decode(M, prec), *coeffs, steps)) <= TOL_NS[prec]


@pytest.mark.parametrize("steps", [1, 2, 3, 4])
@pytest.mark.parametrize("shape", [(1024, 2048), (2048, 1024), (768, 2304), (1000, 1000)])
def test_ns_few_steps_with_residuals(steps, shape):
    """Fewer steps than five (residual iterations: 0, 1, 2, 2 for 1, 2, 3, 4 steps),
    wide, tall with its final transposed write, and ragged: step counts where the
    last product reads a residual (2, 3) or not (1, 4)."""
    r, c = shape
    Q1, _ = np.linalg.qr(random_matrix((r, min(r, c)), [316, r]))
    Q2, _ = np.linalg.qr(random_matrix((c, min(r, c)), [316, c]))
    M = store((Q1 * np.logspace(-2, 0, min(r, c))) @ Q2.T, "bf16")
    (U,) = _ns_gpu([M], "bf16", "bf16", QUINTIC, steps, "bf16")
    assert rel_fro(U, O.newton_schulz(O.decode(M, "bf16"), *QUINTIC, steps)) <= TOL_NS["bf16"]


def _spectrum_matrix(r, c, sig, seed):
    Q1, _ = np.linalg.qr(random_matrix((r, r), [seed, 0]))
    Q2, _ = np.linalg.qr(random_matrix((c, r), [seed, 1]))
    return (Q1 * sig) @ Q2.T


HARD_SPECTRA = {
    "three_decades": lambda s: np.logspace(-3, 0, s),
    "rank_s_over_8_plus_1e-3": lambda s: np.r_[np.ones(s // 8), 1e-3 * np.ones(s - s // 8)],
    "rank_s_over_8_plus_1e-2": lambda s: np.r_[np.ones(s // 8), 1e-2 * np.ones(s - s // 8)],
    "two_levels_30x_apart": lambda s: np.r_[np.ones(s // 2), 0.03 * np.ones(s - s // 2)],
}


@pytest.mark.parametrize("kind", sorted(HARD_SPECTRA))
@pytest.mark.parametrize("shape", [(768, 2304), (1024, 4096)])
def test_ns_bf16_hard_spectra(kind, shape):
    """Ill-conditioned momenta against the bf16 gate through ns_orthogonalize: three
    residual iterations (quintic, five steps) measured 5.5e-3 to 9.9e-3 on these,
    where two reached 2.2e-2 and one 8.6e-2."""
    r, c = shape
    M = store(_spectrum_matrix(r, c, HARD_SPECTRA[kind](r), 330 + r), "bf16")
    (U,) = _ns_gpu([M], "bf16", "bf16", QUINTIC, 5, "bf16")
    assert rel_fro(U, O.newton_schulz(O.decode(M, "bf16"), *QUINTIC, 5)) <= TOL_NS["bf16"]


def test_ns_bf16_hard_spectrum_llama_mlp_shape():
    """A rank-512 momentum plus noise 1e-3 times smaller at 4096 x 14336 (two residual
    iterations measured 2.75e-2 here, three 7.7e-3)."""
    r, c = 4096, 14336
    M = store(_spectrum_matrix(r, c, HARD_SPECTRA["rank_s_over_8_plus_1e-3"](r), 331), "bf16")
    (U,) = _ns_gpu([M], "bf16", "bf16", QUINTIC, 5, "bf16")
    assert rel_fro(U, O.newton_schulz(O.decode(M, "bf16"), *QUINTIC, 5)) <= TOL_NS["bf16"]


@pytest.mark.parametrize("seed", range(4))
@pytest.mark.parametrize("shape", [(16, 128), (37, 300), (300, 37), (95, 760)])
def test_ns_small_bf16_problems_run_on_fp32_products(shape, seed):
    """Short sides below ns_bf16_min_side() (96) run on the fp32 products when bf16 is
    asked for: bf16 products measured 1.8e-2 to 2.4e-2 on such Gaussian momenta.  With
    an fp32 direction the result meets the fp32 bar against the oracle."""
    assert mao.ns_bf16_min_side() == 96
    M = store(random_matrix(shape, [332, seed]), "bf16")
    (U,) = _ns_gpu([M], "bf16", "f32", QUINTIC, 5, "bf16")
    assert rel_fro(U, O.newton_schulz(O.decode(M, "bf16"), *QUINTIC, 5)) <= TOL_NS["f32"]


@pytest.mark.parametrize("seed", range(3))
@pytest.mark.parametrize("shape", [(96, 768), (128, 1024)])
def test_ns_smallest_bf16_products(shape, seed):
    """The smallest short sides on bf16 products, Gaussian momenta (measured at most
    1.4e-2 in emulation of the kernels' rounding)."""
    M = store(random_matrix(shape, [333, seed]), "bf16")
    (U,) = _ns_gpu([M], "bf16", "bf16", QUINTIC, 5, "bf16")
    assert rel_fro(U, O.newton_schulz(O.decode(M, "bf16"), *QUINTIC, 5)) <= TOL_NS["bf16"]


@pytest.mark.parametrize("in_place", [False, True])
@pytest.mark.parametrize("batch,s,l", [(1, 4096, 14336), (2, 768, 2304), (1, 1024, 4096)])
def test_apply_residuals(in_place, batch, s, l):
    """ns_apply with the addend's residual X_lo and the output's residual: Xout + Xout_lo
    equals a (X + X_lo) + B X to fp32 accumulation (the residual keeps about 16
    significant bits), Xout_lo is within half a bf16 unit of Xout, and zero residuals
    reproduce the plain product.  4096 x 14336 takes the one-launch whole-tile and
    column-strip path; in place, X_lo and Xout_lo are one buffer."""
    Xs = store(random_matrix((batch, s, l), [317, s]) / np.sqrt(s * l), "bf16")
    Ls = store(random_matrix((batch, s, l), [318, s]) / np.sqrt(s * l) * 2.0 ** -9, "bf16")
    R = random_matrix((batch, s, s), [319, s]) / np.sqrt(s)
    Bs = store(R + np.transpose(R, (0, 2, 1)), "bf16")
    Xd, Ld = to_dev(Xs, "bf16").view(batch, s, l), to_dev(Ls, "bf16").view(batch, s, l)
    Bd = to_dev(Bs, "bf16").view(batch, s, s)
    a = QUINTIC[0]
    out = torch.empty_like(Xd)
    lo_out = Ld if in_place else torch.empty_like(Xd)
    mao.ns_apply(Bd, Xd, out, a, 1.0, X_lo=Ld, Xout_lo=lo_out)
    hi = O.decode(from_dev(out), "bf16").reshape(batch, s, l)
    lo = O.decode(from_dev(lo_out), "bf16").reshape(batch, s, l)
    X = O.decode(Xs, "bf16").reshape(batch, s, l)
    Lx = O.decode(Ls, "bf16").reshape(batch, s, l)
    B = O.decode(Bs, "bf16").reshape(batch, s, s)
    for b in (0, batch - 1):
        ref = O.apply_poly(B[b], X[b], a) + a * Lx[b]
        # bf16 alone would be about 1e-3 off; the pair is off by the residual's own
        # rounding and the fp32 accumulation
        assert rel_fro(hi[b] + lo[b], ref) <= 3e-5
        assert np.all(np.abs(lo[b]) <= 2.0 ** -8 * np.abs(hi[b]))
    # zero residuals: the plain product's values
    zeros = torch.zeros_like(Xd)
    plain = torch.empty_like(Xd)
    mao.ns_apply(Bd, Xd, plain, a, 1.0)
    with_zero = torch.empty_like(Xd)
    mao.ns_apply(Bd, Xd, with_zero, a, 1.0, X_lo=zeros, Xout_lo=zeros)
    assert np.array_equal(O.decode(from_dev(plain), "bf16"), O.decode(from_dev(with_zero), "bf16"))


@pytest.mark.parametrize("kind,batch,s,l", [("gram", 16, 2048, 2048), ("poly", 16, 2048, 2048),
                                             ("apply", 16, 1024, 2048), ("apply", 3, 2048, 2304),
                                             ("gram", 1, 4096, 4096), ("apply", 1, 4096, 14336),
                                             ("gram", 1, 4096, 14336), ("poly", 1, 4096, 4096)])
def test_stages_at_large_tile_sizes(kind, batch, s, l):
    """Stage shapes that take the 256 x 256-tile kernels (symmetric products, or B X with
    a contraction of 2048 or more) next to ones that take the 128 x 128 tiles."""
    prec = "bf16"
    Xs = store(random_matrix((batch, s, l), [308, s]) / np.sqrt(l), prec)
    Xd = to_dev(Xs, prec).view(batch, s, l)
    check = [0, batch - 1]
    if kind == "gram":
        A = torch.empty((batch, s, s), dtype=torch.bfloat16, device="cuda")
        mao.ns_gram(Xd, A, prec)
        got = O.decode(from_dev(A), prec).reshape(batch, s, s)
        X = O.decode(Xs, prec)
        for b in check:
            assert rel_fro(got[b], O.gram(X[b])) <= TOL_STAGE[prec]
    elif kind == "poly":
        A = torch.empty((batch, s, s), dtype=torch.bfloat16, device="cuda")
        mao.ns_gram(Xd, A, prec)
        B = torch.empty_like(A)
        mao.ns_poly(A, B, QUINTIC[1], QUINTIC[2], prec)
        Ain = O.decode(from_dev(A), prec).reshape(batch, s, s)
        got = O.decode(from_dev(B), prec).reshape(batch, s, s)
        for b in check:
            assert rel_fro(got[b], O.poly(Ain[b], QUINTIC[1], QUINTIC[2])) <= TOL_STAGE[prec]
    else:
        R = random_matrix((batch, s, s), [309, 0]) / np.sqrt(s)
        Bs = store(R + np.transpose(R, (0, 2, 1)), prec)
        out = torch.empty_like(Xd)
        mao.ns_apply(to_dev(Bs, prec).view(batch, s, s), Xd, out, QUINTIC[0], 1.0, prec)
        got = O.decode(from_dev(out), prec).reshape(batch, s, l)
        X, Bd = O.decode(Xs, prec), O.decode(Bs, prec)
        for b in check:
            assert rel_fro(got[b], O.apply_poly(Bd[b], X[b], QUINTIC[0])) <= TOL_STAGE[prec]


def test_stage_sequence_equals_ns_orthogonalize():
    """The stage calls bench.py times (gram / poly / apply five times, the first on the
    raw momentum with the scaling folded in) compute exactly what ns_orthogonalize
    computes: on a pad-free wide matrix the final X equals U bit for bit."""
    prec, rows, cols = "bf16", 4096, 14336
    M = store(random_matrix((rows, cols), [312, 0]), prec)
    Md = to_dev(M, prec).view(rows, cols)
    sums = torch.tensor([O.sumsq(O.decode(M, prec))], dtype=torch.float32, device="cuda")
    U = torch.empty((rows, cols), dtype=torch.bfloat16, device="cuda")
    a, b, c = QUINTIC
    mao.ns_orthogonalize([(Md, U, sums)], a, b, c, 5, prec)
    X = [torch.empty((1, rows, cols), dtype=torch.bfloat16, device="cuda") for _ in range(2)]
    A = torch.empty((1, rows, rows), dtype=torch.bfloat16, device="cuda")
    B = torch.empty_like(A)
    # a bf16 wide pad-free momentum: the first iteration reads M and folds the scaling;
    # the outputs of the first three iterations keep their residual, read by the next
    M3 = Md.view(1, rows, cols)
    Xlo = torch.empty_like(X[0])
    k = mao.ns_residual_iterations(rows, cols, a, b, c, 5, prec)
    assert k == 3
    for it in range(5):
        Xc, ss = (M3, sums) if it == 0 else (X[it % 2], None)
        mao.ns_gram(Xc, A, prec, sumsq=ss)
        mao.ns_poly(A, B, b, c, prec)
        mao.ns_apply(B, Xc, X[(it + 1) % 2], a, 1.0, prec, sumsq=ss,
                     X_lo=Xlo if 1 <= it <= k else None, Xout_lo=Xlo if it < k and it < 4 else None)
    assert np.array_equal(from_dev(X[1]).reshape(rows, cols), from_dev(U))
