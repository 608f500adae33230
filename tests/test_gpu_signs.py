"""GPU parity of the packed signs written by the last Newton-Schulz product.

The final B X product can pack the signs of the values it stores (one ballot
per column offset in its epilogue), so the 1-bit exchange buffer is written
without re-reading the direction.  The signs must be bit-identical to
sign_pack over the stored direction (the same bf16 or fp32 encodings), and
the direction itself must not change; where the fusion does not apply (tall
matrices, fp32 products, no iteration, rows that do not fill whole 64-bit
words) ns_orthogonalize packs the stored direction instead.  The oracle ties
both to the method: its sign packing of the decoded GPU direction is the
expected bit pattern.
"""
import numpy as np
import pytest
import torch

import matrix_aware_optimizer_amd as mao
import oracle.muon_oracle as O
from helpers import from_dev, rel_fro, to_dev
from workloads import QUINTIC, random_matrix, store

pytestmark = pytest.mark.gpu


def _words(n):
    return torch.full((n,), -1, dtype=torch.int64, device="cuda")   # all ones: stale bits show


def _stage_inputs(batch, s, l, seed):
    X = store(random_matrix((batch, s, l), [330, seed]) / np.sqrt(s * l), "bf16")
    R = random_matrix((batch, s, s), [331, seed]) / np.sqrt(s)
    B = store(R + np.transpose(R, (0, 2, 1)), "bf16")
    return to_dev(B, "bf16").view(batch, s, s), to_dev(X, "bf16").view(batch, s, l)


@pytest.mark.parametrize("batch,s,l", [(1, 4096, 14336), (1, 4096, 5120), (1, 1024, 4096),
                                       (3, 768, 2304), (1, 256, 512)])
def test_apply_signs_match_sign_pack_of_output(batch, s, l):
    """4096 x 14336 and 4096 x 5120 run their last round as 128 x 256 column strips
    (the words of the second launch sit at a column offset); 1024 x 4096 and the
    smaller ones run 128 x 128 tiles; 768 x 2304 is batched."""
    B, X = _stage_inputs(batch, s, l, s + l)
    a = QUINTIC[0]
    ref = torch.empty_like(X)
    mao.ns_apply(B, X, ref, a, 1.0)
    out = torch.empty_like(X)
    bits = _words(batch * s * l // 64)
    mao.ns_apply_signs(B, X, out, bits, a, 1.0)
    only = _words(batch * s * l // 64)
    mao.ns_apply_signs(B, X, None, only, a, 1.0)
    refh = from_dev(ref)
    assert np.array_equal(from_dev(out), refh)                   # the direction is unchanged
    want = np.concatenate([O.sign_pack(O.decode(refh.reshape(batch, -1)[b], "bf16")) for b in range(batch)])
    assert np.array_equal(from_dev(bits), want)
    assert np.array_equal(from_dev(only), want)                  # signs only: same words


def test_apply_signs_with_folded_scaling():
    """First iteration read from the raw momentum (scaled by 1/sqrt(sumsq) in the epilogue)."""
    s, l = 1024, 8192
    M = store(random_matrix((1, s, l), [332, 0]), "bf16")
    Md = to_dev(M, "bf16").view(1, s, l)
    sums = torch.tensor([O.sumsq(O.decode(M, "bf16")[0])], dtype=torch.float32, device="cuda")
    R = random_matrix((1, s, s), [333, 0]) / np.sqrt(s)
    B = to_dev(store(R + np.transpose(R, (0, 2, 1)), "bf16"), "bf16").view(1, s, s)
    ref = torch.empty_like(Md)
    mao.ns_apply(B, Md, ref, QUINTIC[0], 1.0, sumsq=sums)
    bits = _words(s * l // 64)
    mao.ns_apply_signs(B, Md, None, bits, QUINTIC[0], 1.0, sumsq=sums)
    assert np.array_equal(from_dev(bits), O.sign_pack(O.decode(from_dev(ref), "bf16")))


def _ns_case(shapes, u_dtype="bf16", precision="bf16", steps=5, keep_u=True, seed=0):
    """Problems laid out flat (M, U and bits back to back), as an optimizer holds them."""
    sizes = [r * c for r, c in shapes]
    offs = np.concatenate([[0], np.cumsum(sizes)]).astype(int)
    assert all(o % 64 == 0 for o in offs[:-1])
    Mh = store(random_matrix((offs[-1],), [334, seed]), "bf16")
    Md = to_dev(Mh, "bf16")
    tdt = torch.bfloat16 if u_dtype == "bf16" else torch.float32
    U = torch.empty(offs[-1], dtype=tdt, device="cuda")
    bits = _words((offs[-1] + 63) // 64)
    probs = []
    for j, (r, c) in enumerate(shapes):
        lo, hi = offs[j], offs[j + 1]
        probs.append((Md[lo:hi].view(r, c), U[lo:hi].view(r, c) if keep_u else None, None,
                      bits[lo // 64:(hi + 63) // 64]))
    mao.ns_orthogonalize(probs, *QUINTIC, steps, precision)
    return Mh, offs, U, bits


@pytest.mark.parametrize("shapes,u_dtype,precision,steps", [
    ([(1024, 4096)], "bf16", "bf16", 5),                       # fused
    ([(1024, 4096)], "f32", "bf16", 5),                        # fused, fp32 direction
    ([(1000, 4096)], "bf16", "bf16", 5),                       # fused, padded rows
    ([(512, 4032)], "bf16", "bf16", 5),                        # fused, padded columns
    ([(768, 2304)] * 3 + [(768, 768)], "bf16", "bf16", 5),     # batched run + a square one
    ([(4096, 1024)], "bf16", "bf16", 5),                       # tall: packed from U
    ([(512, 1000)], "bf16", "bf16", 5),                        # rows not whole words: packed from U
    ([(64, 1024)], "bf16", "bf16", 5),                         # short side below 96: fp32 products
    ([(512, 1024)], "f32", "f32", 3),                          # fp32 products: packed from U
    ([(512, 1024), (1024, 512)], "bf16", "bf16", 0),           # no iteration: packed from U
])
def test_ns_orthogonalize_signs_match_packed_direction(shapes, u_dtype, precision, steps):
    Mh, offs, U, bits = _ns_case(shapes, u_dtype, precision, steps)
    Uh = O.decode(from_dev(U), u_dtype)
    got = from_dev(bits)
    for j in range(len(shapes)):
        lo, hi = offs[j], offs[j + 1]
        assert np.array_equal(got[lo // 64:(hi + 63) // 64], O.sign_pack(Uh[lo:hi])), f"matrix {j}"


def test_ns_orthogonalize_signs_only():
    """U omitted (fused case): the same words as with U written."""
    shapes = [(768, 2304)] * 2
    _, _, _, with_u = _ns_case(shapes, seed=5)
    _, _, _, only = _ns_case(shapes, keep_u=False, seed=5)
    assert np.array_equal(from_dev(with_u), from_dev(only))


def test_prepared_call_matches_direct_calls():
    """PreparedNS (the problem array marshalled once) gives the same words as
    ns_orthogonalize, on two calls in a row and after the momentum changes in place
    (the norms are computed by the call itself here).  SignMuonStep keeps one such
    call per buffer pair; its second step is checked in the workload tests."""
    shapes = [(768, 2304)] * 2 + [(768, 768), (3072, 768)]
    Mh, offs, U, direct = _ns_case(shapes, seed=9)
    _, _, _, direct2 = _ns_case(shapes, seed=10)
    M1 = to_dev(Mh, "bf16")
    U2 = torch.zeros_like(M1)
    bits = torch.zeros(direct.numel(), dtype=torch.int64, device="cuda")
    probs = [(M1[offs[j]:offs[j + 1]].view(*shp), U2[offs[j]:offs[j + 1]].view(*shp), None,
              bits[offs[j] // 64:(offs[j + 1] + 63) // 64]) for j, shp in enumerate(shapes)]
    call = mao.PreparedNS(probs, *QUINTIC, 5, "bf16")
    for _ in range(2):
        bits.zero_()
        call()
        assert np.array_equal(from_dev(bits), from_dev(direct))
    Mh2, _, _, _ = _ns_case(shapes, seed=10)
    M1.copy_(to_dev(Mh2, "bf16"))
    call()
    assert np.array_equal(from_dev(bits), from_dev(direct2))


@pytest.mark.parametrize("steps", [5, 0])
def test_runs_on_two_lanes_match_one_call_per_run(steps):
    """A call with runs of several shapes (spread over the library's two streams)
    writes exactly what separate calls, one run each, write: directions and words.
    Among them a short side under 96 (fp32 products) and a tall run."""
    shapes = ([(768, 2304)] * 3 + [(768, 768)] * 2 + [(1024, 2048)] * 2 + [(3072, 768)] * 2
              + [(64, 1024)] * 2)
    Mh, offs, U, bits = _ns_case(shapes, steps=steps, seed=11)
    Md = to_dev(Mh, "bf16")
    U2 = torch.empty_like(U)
    bits2 = torch.zeros_like(bits)
    groups = {}
    for j, (r, c) in enumerate(shapes):
        lo, hi = offs[j], offs[j + 1]
        groups.setdefault((r, c), []).append((Md[lo:hi].view(r, c), U2[lo:hi].view(r, c), None,
                                              bits2[lo // 64:(hi + 63) // 64]))
    for probs in groups.values():
        mao.ns_orthogonalize(probs, *QUINTIC, steps, "bf16")
    assert np.array_equal(from_dev(U), from_dev(U2))
    assert np.array_equal(from_dev(bits), from_dev(bits2))


def test_ns_signs_agree_with_oracle_direction():
    """Against the fp64 oracle's direction: signs agree wherever the oracle's entry is
    clear of the bf16 iteration's error (|U| above a quarter of its RMS, more than ten
    times the 2e-2 relative error the iteration is held to)."""
    r, c = 512, 2048
    Mh, offs, U, bits = _ns_case([(r, c)], seed=7)
    ref = O.newton_schulz(O.decode(Mh, "bf16").reshape(r, c), *QUINTIC, 5).ravel()
    got = np.unpackbits(from_dev(bits).view(np.uint8), bitorder="little")[:r * c].astype(bool)
    clear = np.abs(ref) > 0.25 * np.sqrt(np.mean(ref ** 2))
    assert clear.mean() > 0.5
    assert np.array_equal(got[clear], O.sign_bits(ref)[clear])
    assert rel_fro(O.decode(from_dev(U), "bf16"), ref) <= 2e-2


def test_apply_signs_non_finite_and_no_addend():
    """Signs of stored non-finite values follow sign_pack's rule (NaN gives 1, -inf
    gives 0), and a = 0 (no addend read) packs the same way."""
    batch, s, l = 1, 1024, 4096
    B, X = _stage_inputs(batch, s, l, 77)
    Xh = from_dev(X).reshape(s, l).copy()
    Xh[5, :] = 0x7FC0            # NaN row: NaN wherever B[:, 5] is non-zero
    Xh[9, 100:200] = 0xFF80      # -inf entries
    Xh[17, 300:400] = 0x7F80     # +inf entries
    Xd = to_dev(Xh, "bf16").view(1, s, l)
    for a in (QUINTIC[0], 0.0):
        ref = torch.empty_like(Xd)
        mao.ns_apply(B, Xd, ref, a, 1.0)
        bits = _words(s * l // 64)
        mao.ns_apply_signs(B, Xd, None, bits, a, 1.0)
        want = O.sign_pack(O.decode(from_dev(ref), "bf16"))
        assert np.array_equal(from_dev(bits), want), f"a = {a}"


def test_ns_orthogonalize_signs_cubic():
    """c = 0 (cubic coefficients): the last product is a X + b A X, packed in place."""
    from workloads import CUBIC
    shapes = [(1024, 2048)]
    sizes = [r * c for r, c in shapes]
    Mh = store(random_matrix((sizes[0],), [335, 0]), "bf16")
    Md = to_dev(Mh, "bf16")
    U = torch.empty(sizes[0], dtype=torch.bfloat16, device="cuda")
    bits = _words(sizes[0] // 64)
    mao.ns_orthogonalize([(Md.view(*shapes[0]), U.view(*shapes[0]), None, bits)], *CUBIC, 5, "bf16")
    assert np.array_equal(from_dev(bits), O.sign_pack(O.decode(from_dev(U), "bf16")))
