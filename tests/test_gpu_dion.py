"""GPU parity of the Dion step (dion_step) against the fp64 oracle.

Everything runs in fp32 on the GPU, so the bar is the fp32 one: 1e-4 relative
Frobenius error on the error-feedback term B - M_new, the new right factor Q
and the weight update X_new - X.  B = M + G itself is bit-exact.
"""
import numpy as np
import pytest
import torch

import matrix_aware_optimizer_amd as mao
import oracle.muon_oracle as O
from helpers import rel_fro
from workloads import DION_WORKLOADS, gen_dion, random_matrix

pytestmark = pytest.mark.gpu
TOL = 1e-4


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()


def check_against_oracle(M0, G, X0, Q0, out, mu, eta):
    """out: the GPU's (M, Q, X) after one step."""
    ref = O.dion_step(M0, G, X0, Q0, mu, eta)
    B = ref["B"]
    Mg, Qg, Xg = (o.astype(np.float64) for o in out)
    assert rel_fro(B - Mg, B - ref["M"].astype(np.float64)) <= TOL, "error feedback"
    assert rel_fro(Qg, ref["Q"].astype(np.float64)) <= TOL, "right factor"
    dX = ref["X"].astype(np.float64) - X0.astype(np.float64)
    assert rel_fro(Xg - X0.astype(np.float64), dX) <= TOL, "update"
    return ref


def run_single(M0, G, X0, Q0, rank, mu, eta):
    M, X, Q = dev(M0), dev(X0), dev(Q0)
    mao.dion_step([(M, dev(G), X, Q)], rank, mu, eta)
    torch.cuda.synchronize()
    return M.cpu().numpy(), Q.cpu().numpy(), X.cpu().numpy()


@pytest.mark.parametrize("m,n,r", [(100, 70, 1), (100, 70, 5), (64, 64, 64), (300, 130, 48), (130, 300, 48),
                                   (768, 768, 192), (96, 1000, 17),
                                   (200, 324, 96), (140, 260, 128),   # B = M + G in B Q: ragged rows, k tail
                                   (70, 260, 128), (200, 60, 96),    # rank above a side: P of rank min(m, n)
                                   (300, 260, 80), (200, 516, 160),  # fused update on 16-deep stages, 5 and 10 of them
                                   (37, 91, 6),      # m n odd: element-wise B = M + G; rows of Q not 16-byte multiples
                                   (8, 5000, 4)])    # n >> m: the column-norm chunks number exactly m
def test_dion_single_matrix(m, n, r):
    M0 = (random_matrix((m, n), [600, m]) * 0.02).astype(np.float32)
    G = (random_matrix((m, n), [601, n]) * 0.02).astype(np.float32)
    X0 = (random_matrix((m, n), [602, r]) * 0.02).astype(np.float32)
    Q0 = random_matrix((n, r), [603, r]).astype(np.float32)
    out = run_single(M0, G, X0, Q0, r, 0.95, 0.02)
    check_against_oracle(M0, G, X0, Q0, out, 0.95, 0.02)
    # the new right factor has unit columns, min(m, n, r) of them (the rest zero:
    # B Q has rank at most min(m, n))
    nrm = np.linalg.norm(out[1].astype(np.float64), axis=0)
    unit = np.isclose(nrm, 1.0, atol=1e-5)
    assert np.all(unit | (nrm == 0.0)) and unit.sum() == min(m, n, r)


def test_dion_closed_form_rank_r():
    """B = U diag(s) V^T of rank r and Q = V: M_new = mu B, Q_new = V, update -eta U V^T."""
    m, n, r = 200, 150, 8
    U = np.linalg.qr(random_matrix((m, r), [604, 0]))[0]
    V = np.linalg.qr(random_matrix((n, r), [605, 0]))[0]
    B = ((U * np.linspace(2.0, 0.5, r)) @ V.T).astype(np.float32)
    u, s, vt = np.linalg.svd(B.astype(np.float64), full_matrices=False)
    U, V = u[:, :r], vt[:r].T
    X0 = np.zeros((m, n), np.float32)
    Mg, Qg, Xg = run_single(B, np.zeros_like(B), X0, V.astype(np.float32), r, 0.9, 0.1)
    assert rel_fro(Mg, 0.9 * B.astype(np.float64)) <= 1e-5
    signs = np.sign(np.diag(Qg.astype(np.float64).T @ V))
    assert np.allclose(Qg * signs, V, atol=1e-5)
    assert rel_fro(Xg, -0.1 * (U * signs) @ (V * signs).T) <= 1e-5


def test_dion_zero_inputs():
    m, n, r = 96, 80, 12
    Z = np.zeros((m, n), np.float32)
    X0 = random_matrix((m, n), [606, 0]).astype(np.float32)
    Mg, Qg, Xg = run_single(Z, Z, X0, random_matrix((n, r), [607, 0]).astype(np.float32), r, 0.95, 0.02)
    assert not Mg.any() and not Qg.any() and np.array_equal(Xg, X0)


def test_dion_two_steps_warm_start():
    m, n, r = 256, 384, 32
    M = (random_matrix((m, n), [608, 0]) * 0.02).astype(np.float32)
    X = (random_matrix((m, n), [609, 0]) * 0.02).astype(np.float32)
    Q = random_matrix((n, r), [610, 0]).astype(np.float32)
    for t in range(2):
        G = (random_matrix((m, n), [611, t]) * 0.02).astype(np.float32)
        out = run_single(M, G, X, Q, r, 0.95, 0.02)
        check_against_oracle(M, G, X, Q, out, 0.95, 0.02)
        M, Q, X = out          # the GPU's state carries into the next step


@pytest.mark.timeout(600)
@pytest.mark.parametrize("rank", [192, 48])
def test_dion_layer_set(rank):
    """The d = 768 layer set (48 matrices of 4 shapes) in one batched call; sampled
    matrices against the oracle."""
    wl = DION_WORKLOADS[rank]
    inp = gen_dion(wl)
    offs, qoffs = wl.offsets, wl.q_offsets
    M = torch.zeros(wl.numel, dtype=torch.float32, device="cuda")
    G, X, Q = dev(inp["G"]), dev(inp["W0"]), dev(inp["Q0"])
    probs = []
    for j, (r_, c_) in enumerate(wl.shapes):
        probs.append((M[offs[j]:offs[j + 1]].view(r_, c_), G[offs[j]:offs[j + 1]].view(r_, c_),
                      X[offs[j]:offs[j + 1]].view(r_, c_), Q[qoffs[j]:qoffs[j + 1]].view(c_, rank)))
    mao.dion_step(probs, rank, wl.mu, wl.eta)
    torch.cuda.synchronize()
    Mh, Xh, Qh = M.cpu().numpy(), X.cpu().numpy(), Q.cpu().numpy()
    for j in [0, 1, 2, 3, 25, 46, 47]:
        r_, c_ = wl.shapes[j]
        sl, ql = slice(offs[j], offs[j + 1]), slice(qoffs[j], qoffs[j + 1])
        check_against_oracle(np.zeros((r_, c_), np.float32), inp["G"][sl].reshape(r_, c_),
                             inp["W0"][sl].reshape(r_, c_), inp["Q0"][ql].reshape(c_, rank),
                             (Mh[sl].reshape(r_, c_), Qh[ql].reshape(c_, rank), Xh[sl].reshape(r_, c_)),
                             wl.mu, wl.eta)


@pytest.mark.timeout(600)
@pytest.mark.parametrize("rank", [96, 48])
def test_dion_lanes_match_one_call_per_shape(rank):
    """The layer set's four shapes share two streams in one call; every run's
    products, factorisations and column norms are the same kernels on the same
    data as in a call that holds that run alone (one stream), so the two agree
    bit for bit.  Two steps, so the second starts from the first's state."""
    wl = DION_WORKLOADS[48]
    inp = gen_dion(wl)
    offs = wl.offsets
    qn = [c_ * rank for _, c_ in wl.shapes]
    qoffs = np.concatenate([[0], np.cumsum(qn)])
    Q0 = random_matrix((int(qoffs[-1]),), [612, rank]).astype(np.float32)

    def state():
        return (torch.zeros(wl.numel, dtype=torch.float32, device="cuda"), dev(inp["W0"]), dev(Q0))

    def probs_of(M, G, X, Q, js):
        out = []
        for j in js:
            r_, c_ = wl.shapes[j]
            out.append((M[offs[j]:offs[j + 1]].view(r_, c_), G[offs[j]:offs[j + 1]].view(r_, c_),
                        X[offs[j]:offs[j + 1]].view(r_, c_), Q[qoffs[j]:qoffs[j + 1]].view(c_, rank)))
        return out

    G = dev(inp["G"])
    one, per = state(), state()
    shapes = sorted(set(wl.shapes))
    for _ in range(2):
        mao.dion_step(probs_of(*one[:1], G, *one[1:], range(len(wl.shapes))), rank, wl.mu, wl.eta)
        for sh in shapes:
            js = [j for j, s in enumerate(wl.shapes) if s == sh]
            mao.dion_step(probs_of(*per[:1], G, *per[1:], js), rank, wl.mu, wl.eta)
    torch.cuda.synchronize()
    for name, a, b in zip(("M", "X", "Q"), one, per):
        assert torch.equal(a, b), f"{name} differs between one call and one call per shape"


@pytest.mark.parametrize("rank", [16, 44])
def test_dion_more_runs_than_streams(rank):
    """Six shapes (six runs) in one call share four streams, so some streams
    take two runs and factor both runs' matrices in one launch; the result
    equals one call per shape bit for bit, and sampled matrices match the
    oracle."""
    shapes = [(64, 128), (64, 128), (96, 64), (96, 64), (96, 64), (128, 256), (48, 72), (48, 72), (200, 100),
              (256, 96)]
    sizes = [r_ * c_ for r_, c_ in shapes]
    offs = np.concatenate([[0], np.cumsum(sizes)])
    qoffs = np.concatenate([[0], np.cumsum([c_ * rank for _, c_ in shapes])])
    G = (random_matrix((int(offs[-1]),), [613, rank]) * 0.02).astype(np.float32)
    X0 = (random_matrix((int(offs[-1]),), [614, rank]) * 0.02).astype(np.float32)
    Q0 = random_matrix((int(qoffs[-1]),), [615, rank]).astype(np.float32)

    def state():
        return torch.zeros(int(offs[-1]), dtype=torch.float32, device="cuda"), dev(X0), dev(Q0)

    def probs_of(M, Gd, X, Q, js):
        return [(M[offs[j]:offs[j + 1]].view(*shapes[j]), Gd[offs[j]:offs[j + 1]].view(*shapes[j]),
                 X[offs[j]:offs[j + 1]].view(*shapes[j]), Q[qoffs[j]:qoffs[j + 1]].view(shapes[j][1], rank))
                for j in js]

    Gd = dev(G)
    one, per = state(), state()
    mao.dion_step(probs_of(one[0], Gd, one[1], one[2], range(len(shapes))), rank, 0.95, 0.02)
    for sh in sorted(set(shapes)):
        js = [j for j, s in enumerate(shapes) if s == sh]
        mao.dion_step(probs_of(per[0], Gd, per[1], per[2], js), rank, 0.95, 0.02)
    torch.cuda.synchronize()
    for name, a, b in zip(("M", "X", "Q"), one, per):
        assert torch.equal(a, b), f"{name} differs between one call and one call per shape"
    Mh, Xh, Qh = (t.cpu().numpy() for t in one)
    for j in (0, 4, 5, 7, 9):
        r_, c_ = shapes[j]
        sl, ql = slice(offs[j], offs[j + 1]), slice(qoffs[j], qoffs[j + 1])
        check_against_oracle(np.zeros((r_, c_), np.float32), G[sl].reshape(r_, c_), X0[sl].reshape(r_, c_),
                             Q0[ql].reshape(c_, rank),
                             (Mh[sl].reshape(r_, c_), Qh[ql].reshape(c_, rank), Xh[sl].reshape(r_, c_)), 0.95, 0.02)
