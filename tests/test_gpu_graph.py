"""A whole worker step (momentum, Newton-Schulz with packed signs, vote and update)
captured into a HIP graph and replayed: every replay equals the same step run
eagerly, with eager work and synchronisations between the replays.

The entry points clear what must start at zero with fill kernels (no
hipMemsetAsync in a captured stream), and the orthogonalisation of several
matrix shapes forks onto the library's second stream and joins back with
events, which the capture follows.
"""
import numpy as np
import pytest
import torch

import matrix_aware_optimizer_amd as mao
from helpers import from_dev, to_dev
from workloads import QUINTIC, random_matrix, store

pytestmark = pytest.mark.gpu

SHAPES = [(768, 2304), (768, 768), (1024, 2048), (3072, 768)]


def _inputs(seed):
    n = sum(r * c for r, c in SHAPES)
    G = to_dev(store(random_matrix((n,), [350, seed, 0]), "bf16"), "bf16")
    W = to_dev(store(random_matrix((n,), [350, seed, 1]), "bf16"), "bf16")
    return G, W


def test_worker_step_replayed_from_a_graph_matches_eager():
    step = mao.SignMuonStep(SHAPES, m_dtype="bf16", precision="bf16", coeffs=QUINTIC, ns_steps=5,
                            beta=0.95, eta=0.02)
    G, W0 = _inputs(0)
    others = step.new_bits(3)
    for k in range(1, 3):                       # two other workers' signs, made eagerly
        Gk, _ = _inputs(k)
        Mk = torch.zeros_like(Gk)
        step.worker(Mk, Gk, others[k])
    torch.cuda.synchronize()

    def run(M, W, bits):
        step.worker(M, G, bits[0])
        step.vote_update(W, bits, fused=True)

    # eager reference: two steps from zero momentum
    M_ref, W_ref, bits_ref = torch.zeros_like(G), W0.clone(), others.clone()
    expect = []
    for _ in range(2):
        run(M_ref, W_ref, bits_ref)
        expect.append((from_dev(M_ref).copy(), from_dev(W_ref).copy(), from_dev(bits_ref).copy()))
    torch.cuda.synchronize()

    # the same buffers captured once (warm-up first, so the library's one-time
    # set-up, second stream and events exist before the capture)
    M, W, bits = torch.zeros_like(G), W0.clone(), others.clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run(torch.zeros_like(G), W0.clone(), others.clone())
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run(M, W, bits)
    for replay in range(3):
        M.zero_()
        W.copy_(W0)
        bits.copy_(others)
        torch.cuda.synchronize()
        for j in range(2):
            graph.replay()
            torch.cuda.synchronize()
            got = (from_dev(M), from_dev(W), from_dev(bits))
            for name, a, b in zip(("momentum", "weights", "signs"), got, expect[j]):
                assert np.array_equal(a, b), f"{name} differs at replay {replay}, step {j}"
        # eager work between replays
        step.momentum(torch.zeros_like(G), G)
        torch.cuda.synchronize()
