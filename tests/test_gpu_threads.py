"""Host threads that call the library at the same time, each on its own stream
with its own buffers, get exactly the results of one-at-a-time calls.

The library keeps no per-call state; what it sets once per device (kernel LDS
limits, the CU count) is held in atomics, and ctypes releases the interpreter
lock during each call, so the threads' calls overlap on the host and their
kernels overlap on the device.
"""
import threading

import numpy as np
import pytest
import torch

import matrix_aware_optimizer_amd as mao
from helpers import to_dev
from workloads import QUINTIC, random_matrix, store

pytestmark = pytest.mark.gpu

# small tiles; a split Gram with 256 x 256 apply tiles; a batched pair; a tall one;
# three shapes (runs on the library's two lanes, whose second stream the threads share)
SHAPES = [[(768, 2304)], [(2048, 8192)], [(512, 1536), (512, 1536)], [(2048, 512)],
          [(768, 2304), (768, 768), (1024, 2048)]]


def _case(k, shapes):
    probs = []
    for j, (r, c) in enumerate(shapes):
        M = to_dev(store(random_matrix((r, c), [340, k, j]), "bf16"), "bf16").view(r, c)
        U = torch.empty(r, c, dtype=torch.bfloat16, device="cuda")
        bits = torch.zeros((r * c + 63) // 64, dtype=torch.int64, device="cuda")
        probs.append((M, U, None, bits))
    return probs


def _outputs(probs):
    return [(U.clone(), bits.clone()) for _, U, _, bits in probs]


def test_concurrent_host_threads_match_serial():
    cases = [_case(k, shapes) for k, shapes in enumerate(SHAPES)]
    want = []
    for probs in cases:
        mao.ns_orthogonalize(probs, *QUINTIC, 5, "bf16")
        want.append(_outputs(probs))
    torch.cuda.synchronize()
    for probs in cases:                       # stale outputs would show
        for _, U, _, bits in probs:
            U.fill_(7.0)
            bits.fill_(-1)
    torch.cuda.synchronize()

    streams = [torch.cuda.Stream() for _ in cases]
    errors = []
    start = threading.Barrier(len(cases))

    def work(k):
        try:
            start.wait()
            with torch.cuda.stream(streams[k]):
                for _ in range(3):
                    mao.ns_orthogonalize(cases[k], *QUINTIC, 5, "bf16")
            streams[k].synchronize()
        except Exception as e:                # reported below, in the test's thread
            errors.append((k, e))

    threads = [threading.Thread(target=work, args=(k,)) for k in range(len(cases))]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=60)
    assert not any(t.is_alive() for t in threads)
    assert not errors, errors
    for k, probs in enumerate(cases):
        for j, ((U, bits), (U0, bits0)) in enumerate(zip(_outputs(probs), want[k])):
            assert torch.equal(U.view(torch.int16), U0.view(torch.int16)), f"case {k} matrix {j}: U"
            assert torch.equal(bits, bits0), f"case {k} matrix {j}: signs"
