"""Pins of the oracle's rotate-quant prologue.

* R4: the float32 path equals an exact-rational evaluation that rounds to binary32 with an
  independently written round-to-nearest-even function, op by op (tiny shapes).
* R1: theta == 0 reduces the prologue to plain per-group e4m3 quantisation of x*cs, checked
  with torch's float8_e4m3fn conversion.
* R2: orthogonality (norm preservation, exact inverse) of the fp64 rotation.
* R3: the inference identity y = rot(x*cs) W^T == x (cs * rot^-1(W))^T.
* I1-I3: scale, saturation and row-sum invariants on every output group.
* record building: hand-checked cos/sin rounding and permutation validation.
"""
import math
from fractions import Fraction

import numpy as np
import pytest
import torch

import synth
from oracle import awq, e4m3, prologue, records

WL = synth.WORKLOADS["tiny"]


def rnd32(x: Fraction) -> Fraction:
    """Round an exact rational to the nearest binary32 value (ties to even); no overflow."""
    if x == 0:
        return Fraction(0)
    s = -1 if x < 0 else 1
    a = abs(x)
    e = math.floor(math.log2(a.numerator) - math.log2(a.denominator))
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    e = max(e, -126)
    ulp = Fraction(2) ** (e - 23)
    n = a / ulp
    f = n.numerator // n.denominator
    rem = n - f
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and f % 2 == 1):
        f += 1
    return s * f * ulp


def F(v) -> Fraction:
    return Fraction(float(v))


def test_rnd32_agrees_with_float32_on_samples():
    r = np.random.default_rng(0)
    a = r.standard_normal(300).astype(np.float32)
    b = r.standard_normal(300).astype(np.float32)
    for x, y in zip(a, b):
        assert rnd32(F(x) * F(y)) == F(np.float32(x) * np.float32(y))


def _tiny_inputs(seed=0, K=256, M=3):
    r = np.random.default_rng(seed)
    x = r.standard_normal((M, K)).astype(np.float16)
    pairs = np.stack([np.concatenate([r.permutation(128) for _ in range(K // 128)]) for _ in range(8)]).astype(np.int16)
    theta = r.uniform(-np.pi, np.pi, (8, K // 2)).astype(np.float16)
    cs = np.exp(r.normal(0, 0.3, K)).astype(np.float16)
    return x, pairs, theta, cs


def test_R4_bruteforce_rational():
    x, pairs, theta, cs = _tiny_inputs(K=256, M=2)
    rec = records.build(pairs, theta)
    v32 = prologue.rotate_f32(x, rec, cs)
    A, ASG, RS = prologue.quantize_groups(v32)
    M, K = x.shape
    for m in range(M):
        v = [rnd32(F(x[m, k]) * F(cs[k])) for k in range(K)]
        for r in range(8):
            for p in range(K // 2):
                base = (p // 64) * 128
                i, j = base + int(pairs[r, 2 * p]), base + int(pairs[r, 2 * p + 1])
                c, s = F(rec["cos"][r, p]), F(rec["sin"][r, p])
                a, b = v[i], v[j]
                v[i] = rnd32(rnd32(c * a) + rnd32(s * b))
                v[j] = rnd32(rnd32(c * b) - rnd32(s * a))
        assert [F(t) for t in v32[m]] == v
        c448 = rnd32(Fraction(1, 448))
        for g in range(K // 128):
            vg = v[g * 128:(g + 1) * 128]
            amax = max(abs(t) for t in vg)
            asg = rnd32(amax * c448)
            inv = rnd32(1 / asg)
            codes = []
            for t in vg:
                q = rnd32(t * inv)
                code = _bruteforce_code(q)
                codes.append(code)
            assert F(ASG[m, g]) == asg
            assert A[m, g * 128:(g + 1) * 128].tolist() == codes
            exact = sum(Fraction(float(e4m3.DECODE[c])) for c in codes)
            assert F(RS[m, g]) == rnd32(exact)


def _bruteforce_code(q: Fraction) -> int:
    neg = q < 0
    a = min(abs(q), Fraction(448))
    best = None
    for c in range(0x7F):
        d = abs(Fraction(float(e4m3.DECODE[c])) - a)
        if best is None or d < best[0] or (d == best[0] and c % 2 == 0):
            best = (d, c)
    c = best[1]
    return c | 0x80 if neg else c


def test_R1_theta_zero_is_plain_quantisation():
    x, pairs, theta, cs = _tiny_inputs(seed=4, K=256, M=5)
    theta[:] = 0
    rec = records.build(pairs, theta)
    assert np.all(rec["cos"] == 1) and np.all(rec["sin"] == 0)
    v = prologue.rotate_f32(x, rec, cs)
    assert np.array_equal(v, x.astype(np.float32) * cs.astype(np.float32))
    A, ASG, RS = prologue.quantize_groups(v)
    # independent: torch fp8 cast of v / asg (q never exceeds 448 in magnitude here)
    vt = torch.from_numpy(v).reshape(5, 2, 128)
    amax = vt.abs().amax(-1)
    asg = amax * torch.tensor(1.0, dtype=torch.float32).div(448.0)
    q = vt * (1.0 / asg)[..., None]
    codes = q.to(torch.float8_e4m3fn)
    negzero = (q == 0) & torch.signbit(q)
    cu = codes.view(torch.uint8).clone()
    cu[negzero] = 0
    assert np.array_equal(A.reshape(5, 2, 128), cu.numpy())
    assert np.array_equal(ASG, asg.numpy())
    rs = codes.to(torch.float64).sum(-1).to(torch.float32)
    assert np.array_equal(RS, rs.numpy())


def test_R2_orthogonality():
    x, pairs, theta, cs = _tiny_inputs(seed=2, K=512, M=4)
    v = x.astype(np.float64)
    y = records.rotate_f64(v, pairs, theta)
    assert np.allclose(np.linalg.norm(y, axis=1), np.linalg.norm(v, axis=1), rtol=1e-14)
    # per 128-group norms are preserved too (rotations are local to a group)
    assert np.allclose(np.linalg.norm(y.reshape(4, 4, 128), axis=2),
                       np.linalg.norm(v.reshape(4, 4, 128), axis=2), rtol=1e-14)
    back = records.rotate_f64(y, pairs, theta, inverse=True)
    assert np.allclose(back, v, atol=1e-13)
    # with f16 records the norm drifts by no more than the f16 cos/sin error allows
    y16 = records.rotate_f64(v, pairs, theta, exact_angles=False)
    drift = np.abs(np.linalg.norm(y16, axis=1) / np.linalg.norm(v, axis=1) - 1)
    assert drift.max() < 8 * 2.0 ** -10


def test_R2_single_pair_closed_form():
    """One layer acting on a basis vector: (a, b) = (1, 0) -> (c, -s)."""
    K = 128
    pairs = np.tile(np.arange(128, dtype=np.int16), (8, 1))
    theta = np.zeros((8, 64), dtype=np.float16)
    theta[0, 0] = np.float16(0.5)
    v = np.zeros((1, K))
    v[0, 0] = 1.0
    y = records.rotate_f64(v, pairs, theta)
    t = float(np.float16(0.5))
    assert np.isclose(y[0, 0], math.cos(t), rtol=0, atol=1e-15)
    assert np.isclose(y[0, 1], -math.sin(t), rtol=0, atol=1e-15)
    assert np.all(y[0, 2:] == 0)


def test_R3_inference_identity():
    K, N, M = 256, 24, 3
    x, pairs, theta, cs = _tiny_inputs(seed=8, K=K, M=M)
    r = np.random.default_rng(11)
    c = r.integers(0, 16, (K, N), dtype=np.uint8)
    zp = r.integers(2, 15, (K // 128, N), dtype=np.uint8)
    sc = r.uniform(0.002, 0.02, (K // 128, N)).astype(np.float16)
    Wt = awq.dequant(synth.awq_pack(c), synth.awq_pack(zp), sc)     # [K, N]
    xs = x.astype(np.float64) * cs.astype(np.float64)
    y1 = records.rotate_f64(xs, pairs, theta) @ Wt
    Weff = cs.astype(np.float64)[None, :] * records.rotate_f64(Wt.T, pairs, theta, inverse=True)   # [N, K]
    y2 = x.astype(np.float64) @ Weff.T
    assert np.linalg.norm(y1 - y2) / np.linalg.norm(y1) < 1e-13


def test_invariants_on_workload_tiny():
    x = synth.activations(WL)
    pl, tl, cl = synth.rotations(WL)
    A, ASG, RS = prologue.rotate_quant(x, pl, tl, cl)
    rec = records.build(pl[0], tl[0])
    v = prologue.rotate_f32(x, rec, cl[0]).reshape(WL.M, WL.G, 128)
    # I1
    assert np.array_equal(ASG[0], (np.abs(v).max(-1) * prologue.C448).astype(np.float32))
    # I2: every non-zero group holds a code of magnitude 448
    mags = np.abs(e4m3.decode(A[0].reshape(WL.M, WL.G, 128)))
    assert np.all(mags.max(-1)[ASG[0] > 0] == 448.0)
    # I3
    assert np.array_equal(RS[0], e4m3.decode(A[0].reshape(WL.M, WL.G, 128)).sum(-1).astype(np.float32))


def test_zero_group():
    x = np.zeros((2, 256), dtype=np.float16)
    x[1, 200] = 1.0
    pairs, theta = _tiny_inputs(K=256)[1:3]
    rec = records.build(pairs, theta)
    A, ASG, RS = prologue.quantize_groups(prologue.rotate_f32(x, rec, np.ones(256, np.float16)))
    assert np.all(A[0] == 0) and np.all(ASG[0] == 0) and np.all(RS[0] == 0)
    assert np.all(A[1, :128] == 0) and ASG[1, 0] == 0 and ASG[1, 1] > 0


def test_records_cos_sin_rounding():
    pairs = np.tile(np.arange(128, dtype=np.int16), (8, 1))
    theta = np.full((8, 64), np.float16(1.0), dtype=np.float16)
    theta[0, 1] = np.float16(-np.pi)
    rec = records.build(pairs, theta)
    # cos(1) = 0.5403023058681398 -> nearest f16 is 0.54052734375 (0x3853)
    assert rec["cos16"][1, 0] == 0x3853
    # sin(1) = 0.8414709848078965 -> f16 0.84130859375 (0x3abb)
    assert rec["sin16"][1, 0] == 0x3ABB
    assert rec["i"][0, 3] == 6 and rec["j"][0, 3] == 7


def test_records_reject_non_permutation():
    pairs = np.tile(np.arange(128, dtype=np.int16), (8, 1))
    pairs[3, 5] = 6
    with pytest.raises(ValueError):
        records.build(pairs, np.zeros((8, 64), np.float16))
