"""Pins of the int8 per-group oracle (oracle/int8.py), each against something other than itself.

* I8-1: exact-rational evaluation of the steps (scale by division, reciprocal, product) with an
  independently written binary32 rounding and a rational round-half-even, on tiny rows.
* I8-2: invariants: every non-zero group holds a code +-127 (its amax element: q = 127 (1 +- a
  few ulps) rounds to 127) and none beyond; rs is the integer sum of the codes; zero groups give
  zero codes, scale and row-sum.
* I8-3: the theta = 0, unit channel-scale case is plain symmetric per-group int8 quantisation of
  x: the codes are within one step of x / (amax / 127) rounded, and reproduce x to half a step.
* G-I8-1: exact-rational evaluation of the GEMM definition on a tiny shape; G-I8-2: the same
  product with torch's exact int64 matmul per group.
"""
from fractions import Fraction
import math

import numpy as np
import torch

import synth
from oracle import awq, gemm, int8

from test_oracle_prologue import F, rnd32


def rne_int(x: Fraction) -> int:
    f = math.floor(x)
    r = x - f
    if r > Fraction(1, 2) or (r == Fraction(1, 2) and f % 2 == 1):
        f += 1
    return int(f)


def test_I8_1_exact_rational_steps():
    r = np.random.default_rng(11)
    for trial in range(5):
        v = (r.standard_normal((2, 256)) * np.exp(r.normal(0, 2))).astype(np.float32)
        q, asg, rs = int8.quantize_groups_i8(v)
        for m in range(2):
            for g in range(2):
                seg = v[m, 128 * g:128 * g + 128]
                amax = max(abs(F(t)) for t in seg)
                a = rnd32(amax / 127)
                assert F(asg[m, g]) == a
                inv = rnd32(1 / a)
                want = [max(-127, min(127, rne_int(rnd32(F(t) * inv)))) for t in seg]
                assert q[m, 128 * g:128 * g + 128].tolist() == want
                assert rs[m, g] == sum(want)


def test_I8_2_invariants_and_zero_group():
    wl = synth.WORKLOADS["qkv"]
    x = synth.activations(wl).copy()
    x[2, 256:384] = 0
    pl, tl, cl = synth.rotations(wl)
    A, ASG, RS = int8.rotate_quant_i8(x, pl, tl, cl)
    G = wl.G
    Ag = A.reshape(wl.P, wl.M, G, 128).astype(np.int64)
    mx = np.abs(Ag).max(axis=3)
    zero = ASG == 0
    assert np.all(mx[~zero] == 127) and np.all(mx <= 127)
    assert np.all(Ag[zero] == 0) and np.all(RS[zero] == 0)
    assert np.array_equal(RS, Ag.sum(axis=3).astype(np.float32))
    assert zero[:, 2, 2].all()


def test_I8_3_theta_zero_is_plain_int8_quantisation():
    r = np.random.default_rng(12)
    M, K = 5, 384
    x = r.standard_normal((M, K)).astype(np.float16)
    pairs = [np.tile(np.arange(128, dtype=np.int16), (8, K // 128))]
    theta = [np.zeros((8, K // 2), np.float16)]
    ones = [np.ones(K, np.float16)]
    A, ASG, _ = int8.rotate_quant_i8(x, pairs, theta, ones)
    xf = x.astype(np.float64).reshape(M, K // 128, 128)
    step = np.abs(xf).max(axis=2) / 127.0
    q = A[0].reshape(M, K // 128, 128).astype(np.float64)
    assert np.allclose(ASG[0], step, rtol=2 ** -23)
    assert np.all(np.abs(q - xf / step[:, :, None]) <= 0.5 + 1e-6)


def test_GI8_1_exact_rational():
    wl = synth.WORKLOADS["tiny"]
    x = synth.activations(wl)
    pl, tl, cl = synth.rotations(wl)
    w = synth.weights(wl)
    A, ASG, _ = int8.rotate_quant_i8(x, pl, tl, cl)
    y = int8.gemm_ref_i8(A, ASG, w.qweight, w.qzeros, w.scales, *wl.bounds)
    c, zp = awq.unpack(w.qweight), awq.unpack(w.qzeros)
    for m in range(wl.M):
        for n in (0, 9, 63, wl.N - 1):
            exact = Fraction(0)
            for g in range(wl.G):
                dot = sum(int(A[0, m, k]) * (int(c[k, n]) - int(zp[g, n])) for k in range(128 * g, 128 * g + 128))
                exact += F(ASG[0, m, g]) * F(w.scales[g, n]) * dot
            assert abs(Fraction(float(y[m, n])) - exact) <= abs(exact) * Fraction(1, 2 ** 50) + Fraction(1, 2 ** 80)


def test_GI8_2_integer_matmul():
    wl = synth.WORKLOADS["qkv"]
    x = synth.activations(wl)
    pl, tl, cl = synth.rotations(wl)
    w = synth.weights(wl)
    A, ASG, _ = int8.rotate_quant_i8(x, pl, tl, cl)
    y = int8.gemm_ref_i8(A, ASG, w.qweight, w.qzeros, w.scales, *wl.bounds)
    c = torch.from_numpy(awq.unpack(w.qweight).astype(np.int64))
    zp = torch.from_numpy(awq.unpack(w.qzeros).astype(np.int64))
    part = gemm.partition_of_columns(wl.N, *wl.bounds)
    ref = np.zeros_like(y)
    for g in range(wl.G):
        wg = c[128 * g:128 * g + 128] - zp[g][None, :]                      # [128, N]
        for p in range(wl.P):
            cols = np.flatnonzero(part == p)
            qg = torch.from_numpy(A[p, :, 128 * g:128 * g + 128].astype(np.int64))
            d = (qg @ wg[:, cols]).numpy().astype(np.float64)
            ref[:, cols] += ASG[p, :, g][:, None].astype(np.float64) * w.scales[g, cols].astype(np.float64)[None, :] * d
    assert gemm.rel_frobenius(y, ref) < 1e-13
