"""GPU parity of the HBM-bound stages against the CPU oracle.

a1 momentum: stored values bit-exact (exact products, one fp64 rounding,
then storage rounding on both sides), per-matrix sums of squares within
1e-5 relative;
a6 sign/pack, a7 vote and a8 update: bit-exact.  All through the C ABI.
"""
import numpy as np
import pytest
import torch

import matrix_aware_optimizer_amd as mao
import oracle.muon_oracle as O
from helpers import bits_to_dev, from_dev, to_dev, ulp_distance
from workloads import random_matrix, store

pytestmark = pytest.mark.gpu


def _momentum_case(numel, offsets, m_dtype, g_dtype, beta, alpha, seed):
    M = store(random_matrix((numel,), [200, seed]), m_dtype)
    G = store(random_matrix((numel,), [201, seed]) * 3.0, g_dtype)
    Md, Gd = to_dev(M, m_dtype), to_dev(G, g_dtype)
    offs = torch.tensor(offsets, dtype=torch.int64, device="cuda")
    sums = torch.full((len(offsets) - 1,), -1.0, dtype=torch.float32, device="cuda")
    mao.muon_momentum(Md, Gd, beta, alpha, offs, sums)
    got = from_dev(Md)
    ref = O.momentum(M, m_dtype, G, g_dtype, beta, alpha)
    assert ulp_distance(got, ref, m_dtype).max(initial=0) == 0
    ref_s = O.segment_sumsq(O.decode(got, m_dtype), offsets)
    s = from_dev(sums).astype(np.float64)
    assert np.all(np.abs(s - ref_s) <= 1e-5 * np.maximum(ref_s, 1e-30)), (s, ref_s)
    return Md, Gd, offs


@pytest.mark.parametrize("m_dtype,g_dtype", [("bf16", "bf16"), ("f32", "f32"), ("f32", "bf16"),
                                             ("bf16", "f32")])
@pytest.mark.parametrize("offsets", [[0, 1], [0, 7], [0, 4096], [0, 4097], [0, 8192], [0, 8193], [0, 100003],
                                     [0, 0, 5, 5, 8200, 8201, 30000, 30000],
                                     [0] + list(np.cumsum([768 * 2304, 768 * 768, 13, 3072 * 768]))])
def test_momentum(m_dtype, g_dtype, offsets):
    beta, alpha = float(np.float32(0.95)), float(np.float32(0.05))
    _momentum_case(int(offsets[-1]), [int(x) for x in offsets], m_dtype, g_dtype, beta, alpha, 1)


def test_momentum_special_cases_and_determinism():
    n = 50000
    for m_dtype in ["bf16", "f32"]:
        M = store(random_matrix((n,), [202, 0]), m_dtype)
        G = store(random_matrix((n,), [203, 0]), m_dtype)
        offs = torch.tensor([0, 12345, n], dtype=torch.int64, device="cuda")
        # beta = 1, alpha = 0 is the identity (bitwise)
        Md = to_dev(M, m_dtype)
        mao.muon_momentum(Md, to_dev(G, m_dtype), 1.0, 0.0)
        assert np.array_equal(from_dev(Md), M)
        # beta = 0 gives alpha * G, matching the oracle bitwise
        Md = to_dev(M, m_dtype)
        mao.muon_momentum(Md, to_dev(G, m_dtype), 0.0, 0.25)
        assert np.array_equal(from_dev(Md), O.momentum(M, m_dtype, G, m_dtype, 0.0, 0.25))
        # two identical runs give bit-identical sums
        outs = []
        for _ in range(2):
            Md = to_dev(M, m_dtype)
            s = torch.zeros(2, dtype=torch.float32, device="cuda")
            mao.muon_momentum(Md, to_dev(G, m_dtype), 0.9, 0.1, offs, s)
            outs.append(from_dev(s).tobytes())
        assert outs[0] == outs[1]


def test_momentum_golden(golden_dir):
    import json
    import os
    d = json.load(open(os.path.join(golden_dir, "bits_hand.json")))["momentum"]
    f = d["f32"]
    Md = to_dev(np.array(f["M"], np.float32), "f32")
    mao.muon_momentum(Md, to_dev(np.array(f["G"], np.float32), "f32"), f["beta"], f["alpha"])
    assert from_dev(Md).tolist() == f["M_new"]
    b = d["bf16"]
    Md = to_dev(np.array([int(x, 16) for x in b["M_bits"]], np.uint16), "bf16")
    Gd = to_dev(np.array([int(x, 16) for x in b["G_bits"]], np.uint16), "bf16")
    mao.muon_momentum(Md, Gd, b["beta"], b["alpha"])
    assert [int(x) for x in from_dev(Md)] == [int(x, 16) for x in b["M_new_bits"]]


# ---------------------------------------------------------------------------
# a6
# ---------------------------------------------------------------------------

def _special_vector(n, seed):
    x = random_matrix((n,), [210, seed])
    rng = np.random.default_rng(seed)
    k = max(1, n // 20)
    x[rng.integers(0, n, k)] = 0.0
    x[rng.integers(0, n, k)] = -0.0
    x[rng.integers(0, n, k)] = np.nan
    x[rng.integers(0, n, k)] = -1e-38
    return x


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("n", [1, 8, 63, 64, 65, 511, 512, 513, 1000, 123457, 4096 * 1024 + 3])
def test_sign_pack(dtype, n):
    U = store(_special_vector(n, n), dtype)
    nw = (n + 63) // 64
    bits = torch.full((nw + 1,), -1, dtype=torch.int64, device="cuda")   # sentinel after the end
    mao.sign_pack(to_dev(U, dtype), bits)
    got = from_dev(bits)
    ref = O.sign_pack(O.decode(U, dtype))
    assert np.array_equal(got[:nw], ref)
    assert got[nw] == np.uint64(0xFFFFFFFFFFFFFFFF)


def test_sign_pack_golden(golden_dir):
    import json
    import os
    d = json.load(open(os.path.join(golden_dir, "bits_hand.json")))["pack"]
    U = [1.5, -2.0, 0.0, -0.0, float("nan"), -1e-30, 3.0, -0.5]
    U += [1.0 if i % 2 == 0 else -1.0 for i in range(8, 64)]
    U += [-3.0, 2.0, -1.0, -1.0, -1.0, -1.0]
    for dtype in ["f32", "bf16"]:
        bits = torch.zeros(2, dtype=torch.int64, device="cuda")
        mao.sign_pack(to_dev(store(np.array(U), dtype), dtype), bits)
        assert [int(w) for w in from_dev(bits)] == [int(x, 16) for x in d["words"]]


# ---------------------------------------------------------------------------
# a7
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("M", [1, 2, 3, 4, 7, 8, 15, 16, 31, 100, 1023])
@pytest.mark.parametrize("nwords", [1, 2, 3, 255, 256, 257, 10000, 10001])
def test_majority_vote(M, nwords):
    rng = np.random.default_rng(M * 7919 + nwords)
    words = rng.integers(0, 2 ** 63, size=(M, nwords), dtype=np.int64).view(np.uint64)
    words ^= rng.integers(0, 2, size=(M, nwords), dtype=np.int64).astype(np.uint64) << np.uint64(63)
    out = torch.zeros(nwords, dtype=torch.int64, device="cuda")
    mao.majority_vote(bits_to_dev(words), out)
    assert np.array_equal(from_dev(out), O.majority_vote(words, nwords * 64))


@pytest.mark.parametrize("M", list(range(1, 12)))
def test_majority_vote_all_patterns(M):
    n = 1 << M
    j = np.arange(max(n, 64))
    bufs = np.stack([O.pack_bits(((j >> k) & 1).astype(bool) & (j < n)) for k in range(M)])
    out = torch.zeros(bufs.shape[1], dtype=torch.int64, device="cuda")
    mao.majority_vote(bits_to_dev(bufs), out)
    got = O.unpack_bits(from_dev(out), n)
    assert np.array_equal(got, np.array([2 * bin(x).count("1") >= M for x in range(n)]))


# ---------------------------------------------------------------------------
# a8 and the fused a7 + a8
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("n", [1, 9, 64, 1000, 65537, 1 << 20])
@pytest.mark.parametrize("eta", [0.02, 0.0, 3.0])
def test_apply_update(dtype, n, eta):
    W = store(random_matrix((n,), [220, n]), dtype)
    vote = O.pack_bits(np.random.default_rng(n).integers(0, 2, n).astype(bool))
    Wd = to_dev(W, dtype)
    mao.apply_update(Wd, bits_to_dev(vote), eta)
    assert np.array_equal(from_dev(Wd), O.apply_update(W, dtype, vote, eta))


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("M", [1, 3, 7, 15, 16])
@pytest.mark.parametrize("n", [5, 4097, 300001])
def test_vote_and_update(dtype, M, n):
    rng = np.random.default_rng(M + n)
    W = store(random_matrix((n,), [221, n]), dtype)
    bufs = np.stack([O.pack_bits(rng.integers(0, 2, n).astype(bool)) for _ in range(M)])
    Wd = to_dev(W, dtype)
    mao.vote_and_update(Wd, bits_to_dev(bufs), 0.02)
    vote = O.majority_vote(bufs, n)
    assert np.array_equal(from_dev(Wd), O.apply_update(W, dtype, vote, 0.02))


def test_update_golden(golden_dir):
    import json
    import os
    d = json.load(open(os.path.join(golden_dir, "bits_hand.json")))
    f = d["update_f32"]
    Wd = to_dev(np.array(f["W"], np.float32), "f32")
    mao.apply_update(Wd, bits_to_dev(np.array([int(f["vote"], 16)], np.uint64)), f["eta"])
    assert from_dev(Wd).tolist() == f["W_new"]
    b = d["update_bf16"]
    Wd = to_dev(np.array([int(x, 16) for x in b["W_bits"]], np.uint16), "bf16")
    mao.apply_update(Wd, bits_to_dev(np.array([int(b["vote"], 16)], np.uint64)), b["eta"])
    assert [int(x) for x in from_dev(Wd)] == [int(x, 16) for x in b["W_new_bits"]]
