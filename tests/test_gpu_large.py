"""Element counts past 2^31: the elementwise kernels index in 64 bits.

N = 2^31 + 4133 entries, so the flat index crosses 2^31 and the last 64-bit
word is ragged (37 entries).  Inputs are drawn on the device from seeded
generators.  Three windows are copied back and given to the oracle: the first
64 words, the 64 words around entry 2^31, and the last 64 words (with the
padding bits).  Each call also runs whole, so an indexing error anywhere
would show at least at the 2^31 boundary or in the tail.
"""
import numpy as np
import pytest
import torch

import matrix_aware_optimizer_amd as mao
import oracle.muon_oracle as O
from helpers import from_dev

pytestmark = pytest.mark.gpu

N = 2 ** 31 + 4133
NW = (N + 63) // 64
WINDOWS = [(0, 64), (2 ** 31 // 64 - 32, 2 ** 31 // 64 + 32), (NW - 64, NW)]


def _bf16_normal(n, seed):
    g = torch.Generator(device="cuda").manual_seed(seed)
    out = torch.empty(n, dtype=torch.bfloat16, device="cuda")
    chunk = 1 << 28                                   # bounds the fp32 temporary
    for i in range(0, n, chunk):
        m = min(chunk, n - i)
        out[i:i + m] = torch.randn(m, generator=g, device="cuda").to(torch.bfloat16)
    return out


def _random_words(rows, nw, seed):
    g = torch.Generator(device="cuda").manual_seed(seed)
    b = torch.randint(0, 256, (rows * nw * 8,), dtype=torch.uint8, device="cuda", generator=g)
    return b.view(torch.int64).view(rows, nw)


def _entries(t, w0, w1):
    """The entries covered by words [w0, w1) of a flat length-N tensor."""
    return t[w0 * 64:min(w1 * 64, N)]


def test_sign_pack_past_2_31():
    U = _bf16_normal(N, 1)
    bits = torch.full((NW,), -1, dtype=torch.int64, device="cuda")   # stale bits show
    mao.sign_pack(U, bits)
    for w0, w1 in WINDOWS:
        want = O.sign_pack(O.decode(from_dev(_entries(U, w0, w1)), "bf16"))
        assert np.array_equal(from_dev(bits[w0:w1]), want), (w0, w1)


def test_vote_and_update_past_2_31():
    M, eta = 3, 0.02
    W = _bf16_normal(N, 2)
    before = {w: from_dev(_entries(W, *w)).copy() for w in WINDOWS}
    bits = _random_words(M, NW, 3)
    mao.vote_and_update(W, bits, eta)
    for w0, w1 in WINDOWS:
        n = min(w1 * 64, N) - w0 * 64
        vote = O.majority_vote(from_dev(bits[:, w0:w1]), n)
        want = O.apply_update(before[(w0, w1)], "bf16", vote, eta)
        assert np.array_equal(from_dev(_entries(W, w0, w1)), want), (w0, w1)


def test_int8_sum_and_threshold_past_2_31():
    M = 3
    S = (_random_words(M, (N + 7) // 8, 4).view(torch.uint8)[:, :N] & 2).to(torch.int8) - 1   # +-1
    S = S.contiguous()
    total = torch.empty(N, dtype=torch.int8, device="cuda")
    mao.sum_int8(S, total)
    bits = torch.full((NW,), -1, dtype=torch.int64, device="cuda")
    mao.threshold_pack(total, bits)
    for w0, w1 in WINDOWS:
        sl = slice(w0 * 64, min(w1 * 64, N))
        want_sum = O.sum_int8(S[:, sl].cpu().numpy())
        assert np.array_equal(total[sl].cpu().numpy(), want_sum), (w0, w1)
        assert np.array_equal(from_dev(bits[w0:w1]), O.threshold_pack(want_sum)), (w0, w1)


def test_momentum_past_2_31():
    """a1 on N bf16 entries in two segments that meet 320 entries before 2^31.
    The state is compared with the oracle on the windows. Each segment's
    sum of squares is compared with an fp64 reduction of the stored state:
    a property that holds at any size, because the oracle's one-by-one sum
    over 2^31 entries is too slow to run here (relative 1e-5, as at small
    sizes)."""
    beta, alpha = float(np.float32(0.95)), float(np.float32(0.05))   # the fp32 values the call receives
    M = _bf16_normal(N, 5)
    G = _bf16_normal(N, 6)
    before = {w: (from_dev(_entries(M, *w)).copy(), from_dev(_entries(G, *w)).copy()) for w in WINDOWS}
    cut = 2 ** 31 - 320
    offs = torch.tensor([0, cut, N], dtype=torch.int64, device="cuda")
    sums = torch.zeros(2, dtype=torch.float32, device="cuda")
    mao.muon_momentum(M, G, beta, alpha, offs, sums)
    for w in WINDOWS:
        want = O.momentum(before[w][0], "bf16", before[w][1], "bf16", beta, alpha)
        assert np.array_equal(from_dev(_entries(M, *w)), want), w
    ref = [0.0, 0.0]
    chunk = 1 << 28
    for i in range(0, N, chunk):
        j = min(i + chunk, N)
        for k, (lo, hi) in enumerate([(0, cut), (cut, N)]):
            a, b = max(i, lo), min(j, hi)
            if a < b:
                ref[k] += float((M[a:b].double() ** 2).sum())
    got = sums.cpu().numpy().astype(np.float64)
    assert np.all(np.abs(got - np.array(ref)) <= 1e-5 * np.array(ref)), (got, ref)
