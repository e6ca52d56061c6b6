"""Pins of the oracle's same-codes GEMM.

* G1: exact-rational brute force of the per-group definition on the tiny workload.
* G2: "dequantise both operands, then one fp64 matmul" (a different factorisation).
* G4: zero activations give exactly zero; a single group with unit scales is an exact
  integer matmul.
* partition select: columns read the partition their boundary range names.
"""
from fractions import Fraction

import numpy as np

import synth
from oracle import awq, e4m3, gemm, prologue

WL = synth.WORKLOADS["tiny"]


def _tiny():
    x = synth.activations(WL)
    pl, tl, cl = synth.rotations(WL)
    A, ASG, RS = prologue.rotate_quant(x, pl, tl, cl)
    w = synth.weights(WL)
    return A, ASG, w


def test_G1_exact_rational():
    A, ASG, w = _tiny()
    y = gemm.gemm_ref(A, ASG, w.qweight, w.qzeros, w.scales, *WL.bounds)
    c, zp, sc = w.codes, w.zp, w.scales
    D = [[Fraction(float(e4m3.DECODE[v])) for v in row] for row in A[0]]
    for m in range(WL.M):
        for n in range(0, WL.N, 9):
            tot = Fraction(0)
            for g in range(WL.G):
                dot = sum(D[m][k] * (int(c[k, n]) - int(zp[g, n])) for k in range(g * 128, (g + 1) * 128))
                tot += Fraction(float(ASG[0, m, g])) * Fraction(float(sc[g, n])) * dot
            assert abs(Fraction(y[m, n]) - tot) <= abs(tot) * Fraction(1, 2 ** 50) + Fraction(1, 2 ** 200)


def test_G2_dequantise_both_sides():
    A, ASG, w = _tiny()
    y = gemm.gemm_ref(A, ASG, w.qweight, w.qzeros, w.scales, *WL.bounds)
    Aq = e4m3.decode(A[0]) * np.repeat(ASG[0].astype(np.float64), 128, axis=1)
    y2 = Aq @ awq.dequant(w.qweight, w.qzeros, w.scales)
    assert np.linalg.norm(y - y2) / np.linalg.norm(y2) < 1e-14


def test_G4_zero_and_integer_exact():
    A, ASG, w = _tiny()
    y0 = gemm.gemm_ref(np.zeros_like(A), ASG, w.qweight, w.qzeros, w.scales, *WL.bounds)
    assert np.all(y0 == 0)
    r = np.random.default_rng(2)
    M, K, N = 5, 128, 16
    ints = r.integers(-16, 17, (1, M, K))
    lut = {int(v): c for c, v in enumerate(e4m3.DECODE[:0x80]) if np.isfinite(v) and v == int(v)}
    lut.update({-v: c | 0x80 for v, c in list(lut.items()) if v > 0})
    Ac = np.vectorize(lambda v: lut[int(v)])(ints).astype(np.uint8)
    codes = r.integers(0, 16, (K, N), dtype=np.uint8)
    zp = r.integers(0, 16, (1, N), dtype=np.uint8)
    y = gemm.gemm_ref(Ac, np.ones((1, M, 1), np.float32), synth.awq_pack(codes), synth.awq_pack(zp),
                      np.ones((1, N), np.float16), synth.NO_BOUNDARY, synth.NO_BOUNDARY)
    exact = ints[0].astype(np.int64) @ (codes.astype(np.int64) - zp.astype(np.int64))
    assert np.array_equal(y, exact.astype(np.float64))


def test_partition_select():
    N = 8192
    p = gemm.partition_of_columns(N, 6144, 7168)
    assert p[0] == 0 and p[6143] == 0 and p[6144] == 1 and p[7167] == 1 and p[7168] == 2 and p[-1] == 2
    assert np.all(gemm.partition_of_columns(N, synth.NO_BOUNDARY, synth.NO_BOUNDARY) == 0)


def test_partitions_read_their_own_activations():
    """With three partitions, each column range equals a one-partition GEMM on its own A."""
    r = np.random.default_rng(4)
    P, M, K, N = 3, 2, 256, 48
    A = r.integers(0, 0x7F, (P, M, K), dtype=np.uint8)
    ASG = r.uniform(0.1, 1, (P, M, K // 128)).astype(np.float32)
    codes = r.integers(0, 16, (K, N), dtype=np.uint8)
    zp = r.integers(2, 15, (K // 128, N), dtype=np.uint8)
    sc = r.uniform(0.002, 0.02, (K // 128, N)).astype(np.float16)
    qw, qz = synth.awq_pack(codes), synth.awq_pack(zp)
    y = gemm.gemm_ref(A, ASG, qw, qz, sc, 16, 32)
    for p, (n0, n1) in enumerate([(0, 16), (16, 32), (32, 48)]):
        yp = gemm.gemm_ref(A[p:p + 1], ASG[p:p + 1], qw, qz, sc, synth.NO_BOUNDARY, synth.NO_BOUNDARY)
        assert np.array_equal(y[:, n0:n1], yp[:, n0:n1])


def test_rows_subset():
    A, ASG, w = _tiny()
    y = gemm.gemm_ref(A, ASG, w.qweight, w.qzeros, w.scales, *WL.bounds)
    ys = gemm.gemm_ref(A, ASG, w.qweight, w.qzeros, w.scales, *WL.bounds, rows=np.array([3, 1]))
    assert np.array_equal(ys, y[[3, 1]])
