"""Pins of the oracle's rotate-quant prologue.

* R4: the float32 path equals an exact-rational evaluation that rounds to binary32 with an
  independently written round-to-nearest-even function, op by op (tiny shapes).
* R1: theta == 0 reduces the prologue to plain per-group e4m3 quantisation of x*cs, checked
  with torch's float8_e4m3fn conversion.
* R2: orthogonality (norm preservation, exact inverse) of the fp64 rotation.
* R3: the inference identity y = rot(x*cs) W^T == x (cs * rot^-1(W))^T.
* R5: the float32 rotation every parity test uses tracks the fp64 rotation with the same f16
  records (the one R2/R3 pin) within a derived binary32 bound, and keeps each group's norm inside
  the interval the f16 coefficients allow.
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


@pytest.mark.parametrize("name", ["tiny", "qkv"])
def test_R5_f32_rotation_tracks_f64(name):
    """rotate_f32 (binary32, one rounding per written operation) against rotate_f64 with the same
    f16 cos/sin (exact_angles=False), per partition, token and 128-group.

    Bound: a layer maps a pair (a, b) to (c a + s b, c b - s a); with one rounding per product and
    per sum each output is off by at most 2u(|c a| + |s b|) <= 2u (1 + 2^-10) ||(a, b)||, so one
    layer adds at most 2.85u ||v_g|| to the group's error vector (u = 2^-24), and the later layers
    scale it by at most (1 + 2^-10) each: ||v32 - v64||_g <= 8 * 2.85 * 1.008 u ||v||_g < 24u ||v||_g.
    A sign or index slip in either function moves some group by O(||v||_g).

    Norms: one exact layer multiplies ||(a, b)||^2 by c^2 + s^2 of its f16 record, so
    ||R v||_g / ||v||_g lies between the products over the layers of sqrt(min) and sqrt(max) of
    c^2 + s^2 over the group's 64 pairs; the binary32 path stays within 24u of that interval."""
    wl = synth.WORKLOADS[name]
    x = synth.activations(wl)
    pl, tl, cl = synth.rotations(wl)
    u = 2.0 ** -24
    for pairs, theta, cs in zip(pl, tl, cl):
        rec = records.build(pairs, theta)
        v32 = prologue.rotate_f32(x, rec, cs).astype(np.float64)
        v = x.astype(np.float64) * cs.astype(np.float64)              # x * cs, exact
        v64 = records.rotate_f64(v, pairs, theta, exact_angles=False, rec=rec)
        M, K = v.shape
        G = K // 128
        n_in = np.linalg.norm(v.reshape(M, G, 128), axis=2)
        err = np.linalg.norm((v32 - v64).reshape(M, G, 128), axis=2)
        assert np.all(err <= 24 * u * n_in), (err / np.maximum(n_in, 1e-300)).max() / u
        kappa = (rec["cos"].astype(np.float64) ** 2 + rec["sin"].astype(np.float64) ** 2).reshape(8, G, 64)
        lo = np.sqrt(kappa.min(axis=2)).prod(axis=0)                   # [G]
        hi = np.sqrt(kappa.max(axis=2)).prod(axis=0)
        ratio = np.linalg.norm(v32.reshape(M, G, 128), axis=2) / n_in
        assert np.all(ratio >= lo[None, :] - 24 * u) and np.all(ratio <= hi[None, :] + 24 * u)
        # the interval is narrow: f16 cos/sin keep c^2 + s^2 within a few 2^-11 of 1
        assert np.all(hi - lo < 8 * 2.0 ** -10)


def test_R5_planted_sign_slip_is_caught():
    """A second-update sign slip (c b + s a) keeps the f32 and f64 paths far apart and breaks the
    norm interval: the bounds above are not vacuous."""
    x, pairs, theta, cs = _tiny_inputs(seed=3, K=256, M=4)
    rec = records.build(pairs, theta)
    v = x.astype(np.float64) * cs.astype(np.float64)
    v64 = records.rotate_f64(v, pairs, theta, exact_angles=False, rec=rec)
    w = (x.astype(np.float32) * cs.astype(np.float32)).astype(np.float32)
    base = (np.arange(128) // 64) * 128
    for r in range(8):
        I, J = rec["i"][r] + base, rec["j"][r] + base
        a, b = w[:, I].copy(), w[:, J].copy()
        w[:, I] = rec["cos"][r] * a + rec["sin"][r] * b
        w[:, J] = rec["cos"][r] * b + rec["sin"][r] * a               # the slip
    err = np.linalg.norm((w - v64).reshape(4, 2, 128), axis=2)
    n_in = np.linalg.norm(v.reshape(4, 2, 128), axis=2)
    assert np.all(err > 1e3 * 24 * 2.0 ** -24 * n_in)
    ratio = np.linalg.norm(w.astype(np.float64).reshape(4, 2, 128), axis=2) / n_in
    assert np.abs(ratio - 1).max() > 1e-2


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
