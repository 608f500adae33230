"""GPU parity of the local re-orthogonalisation of the vote (the optional step 5).

* unpack_signs and apply_update_dense: bit-exact against the oracle;
* the whole update: NS(S_bar) of every matrix within the Newton-Schulz
  tolerance of the fp64 oracle, and the new weights bit-exact against the
  oracle's dense update fed the GPU's direction.
"""
import numpy as np
import pytest
import torch

import matrix_aware_optimizer_amd as mao
import oracle.muon_oracle as O
from helpers import bits_to_dev, from_dev, rel_fro, to_dev
from workloads import QUINTIC, random_matrix, store

pytestmark = pytest.mark.gpu

TORCH = {"bf16": torch.bfloat16, "f32": torch.float32}
TOL_NS = {"bf16": 2e-2, "f32": 1e-4}


def _vote(n, seed):
    return O.pack_bits(np.random.default_rng([500, seed]).random(n) < 0.5)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("n", [1, 7, 8, 9, 64, 1000, 123457])
def test_unpack_signs(dtype, n):
    words = _vote(n, n)
    out = torch.zeros(n, dtype=TORCH[dtype], device="cuda")
    mao.unpack_signs(bits_to_dev(words), out)
    assert np.array_equal(O.decode(from_dev(out), dtype), O.unpack_signs(words, n))


@pytest.mark.parametrize("w_dtype,u_dtype", [("bf16", "bf16"), ("f32", "f32"), ("bf16", "f32"), ("f32", "bf16")])
@pytest.mark.parametrize("n", [5, 8, 1000, 65537])
@pytest.mark.parametrize("eta", [0.02, 0.0, 3.0])
def test_apply_update_dense(w_dtype, u_dtype, n, eta):
    eta = float(np.float32(eta))
    W = store(random_matrix((n,), [501, n]), w_dtype)
    U = store(random_matrix((n,), [502, n]) * 0.05, u_dtype)
    Wd = to_dev(W, w_dtype)
    mao.apply_update_dense(Wd, to_dev(U, u_dtype), eta)
    assert np.array_equal(from_dev(Wd), O.apply_update_dense(W, w_dtype, U, u_dtype, eta))


@pytest.mark.parametrize("prec,shapes", [
    ("bf16", [(256, 512), (300, 70), (64, 64)]),
    ("f32", [(256, 256), (37, 120)]),
    ("bf16", [(4096, 14336)]),
])
def test_reorthogonalized_update(prec, shapes):
    step = mao.SignMuonStep(shapes, m_dtype=prec, precision=prec, coeffs=QUINTIC, ns_steps=5, eta=0.02)
    n = step.numel
    words = _vote(n, 7)
    W0 = store(random_matrix((n,), [503, 0]), prec)
    W = to_dev(W0, prec)
    step.reorthogonalized_update(W, bits_to_dev(words))
    torch.cuda.synchronize()
    U = from_dev(step.U)
    # the direction, matrix by matrix, against the fp64 oracle
    ref = O.reorthogonalized_direction(words, shapes, *QUINTIC, 5)
    Ud = O.decode(U, prec)
    for j, (r, c) in enumerate(shapes):
        lo, hi = step.offsets_host[j], step.offsets_host[j + 1]
        err = rel_fro(Ud[lo:hi], ref[lo:hi])
        assert err <= TOL_NS[prec], f"NS(S_bar) error {err:.3e} on matrix {j}"
    # the update, bit for bit, given the GPU's direction
    assert np.array_equal(from_dev(W), O.apply_update_dense(W0, prec, U, prec, step.eta))
