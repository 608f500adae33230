"""GPU check of muon_momentum_noalloc, the allocation-free variant of muon_momentum.

Through the C ABI, the new entry point must give bit-identical momentum and
per-matrix sums of squares to muon_momentum with its own workspace, on the
same inputs, on two calls in a row where the second is smaller (the fixed
scratch keeps the first call's partials, which the second must not pick up).
"""
import numpy as np
import pytest
import torch

import matrix_aware_optimizer_amd as mao
from helpers import from_dev, to_dev
from workloads import WORKLOADS, random_matrix, store

pytestmark = pytest.mark.gpu


def _case(sizes, m_dtype, g_dtype, seed):
    n = int(sum(sizes))
    M = store(random_matrix((n,), [340, seed]), m_dtype)
    G = store(random_matrix((n,), [341, seed]) * 0.1, g_dtype)
    offs = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int64)
    return M, G, offs


def _both(M, G, offs, m_dtype, g_dtype, beta=0.95, alpha=0.05):
    dev = torch.device("cuda", 0)
    offs_d = torch.from_numpy(offs).to(dev)
    nseg = offs.size - 1
    outs = []
    for noalloc in (False, True):
        Md, Gd = to_dev(M, m_dtype), to_dev(G, g_dtype)
        sums = torch.full((nseg,), -1.0, dtype=torch.float32, device=dev)
        if noalloc:
            mao.muon_momentum_noalloc(Md, Gd, beta, alpha, offs_d, sums)
        else:
            mao.muon_momentum(Md, Gd, beta, alpha, offs_d, sums)
        torch.cuda.synchronize()
        outs.append((from_dev(Md), sums.cpu().numpy()))
    return outs


def test_noalloc_momentum_matches_workspace_entry_point_twice():
    # first call: the GPT-2-small layer set (48 matrices, 84.9 M bf16 entries)
    wl = WORKLOADS[2]
    sizes1 = [r * c for r, c in wl.shapes]
    M, G, offs = _case(sizes1, "bf16", "bf16", 1)
    (m_ref, s_ref), (m_new, s_new) = _both(M, G, offs, "bf16", "bf16")
    assert np.array_equal(m_new, m_ref)
    assert np.array_equal(s_new.view(np.uint32), s_ref.view(np.uint32))
    assert (s_new > 0).all()
    # second call, smaller: three ragged matrices, fp32 momentum and bf16 gradient
    sizes2 = [5003, 70001, 1234567]
    M, G, offs = _case(sizes2, "f32", "bf16", 2)
    (m_ref, s_ref), (m_new, s_new) = _both(M, G, offs, "f32", "bf16")
    assert np.array_equal(m_new.view(np.uint32), m_ref.view(np.uint32))
    assert np.array_equal(s_new.view(np.uint32), s_ref.view(np.uint32))
    assert s_new.size == 3 and (s_new > 0).all()


def test_noalloc_momentum_without_sums_and_limit():
    """Without sums the scratch is not used; too large a set is refused (nothing launched)."""
    n = 1 << 20
    M, G, _ = _case([n], "bf16", "f32", 3)
    Md, Gd = to_dev(M, "bf16"), to_dev(G, "f32")
    Mr = Md.clone()
    mao.muon_momentum_noalloc(Md, Gd, 0.9, 0.1)
    mao.muon_momentum(Mr, Gd, 0.9, 0.1)
    torch.cuda.synchronize()
    assert np.array_equal(from_dev(Md), from_dev(Mr))
    offs = torch.tensor([0, n], dtype=torch.int64, device="cuda")
    sums = torch.zeros(1, dtype=torch.float32, device="cuda")
    L = mao.lib()
    too_many = ((1 << 22) // 8) * 4096        # one matrix whose partials alone fill 4 MiB
    status = L.muon_momentum_noalloc(Md.data_ptr(), 1, Gd.data_ptr(), 0, too_many, offs.data_ptr(), 1,
                                     0.9, 0.1, sums.data_ptr(), None)
    assert status == -7
