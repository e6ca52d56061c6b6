"""Pins of the int5 bit-plane oracle (oracle/int5.py), each against something other than itself.

* I5-1: the fifth-bit plane read bit by bit in plain Python (and closed-form words) equals
  ``unpack_hi``; the generator's codes are recovered from the packed planes.
* I5-2: with every fifth bit zero the int5 reference equals the pinned int4 reference on the same
  low words, bit for bit (the definitions coincide for codes below 16).
* I5-3: exact-rational evaluation of the definition on a tiny shape, using the generator's code
  and zero-point arrays (not the oracle's unpack).
* I5-4: every c - 16 for c in 0..31 is exact in e4m3, also scaled by 2^-9 (the page's reason why
  5 bits carry over and 6 would not; 17 is the first integer e4m3 cannot hold).
* I5-5: closed form: one group, unit scales, every activation 1 and every weight code 31 with zero
  point 0 gives y = 128 * 31 * sc.
"""
from fractions import Fraction

import numpy as np

import synth
from oracle import e4m3, gemm, int5, prologue

from test_oracle_prologue import F


def test_I5_1_bit_plane_layout():
    r = np.random.default_rng(51)
    words = r.integers(-2**31, 2**31, (3, 4), dtype=np.int64).astype(np.int32)
    bits = int5.unpack_hi(words)
    for row in range(3):
        for w in range(4):
            v = int(words[row, w]) & 0xFFFFFFFF
            for j in range(32):
                assert bits[row, 32 * w + j] == (v >> j) & 1
    one = int5.unpack_hi(np.array([[1, -2**31]], dtype=np.int32))
    assert one[0, 0] == 1 and one[0, 1:32].sum() == 0 and one[0, 63] == 1 and one[0, 32:63].sum() == 0
    wl = synth.Workload("i5", 150, 2, 256, 64)
    w = synth.weights5(wl)
    assert np.array_equal(int5.codes5(w.qweight, w.qweight_hi), w.codes)
    assert np.array_equal(int5.codes5(w.qzeros, w.qzeros_hi), w.zp)
    assert w.codes.max() == 31 and w.codes.min() == 0


def test_I5_2_zero_fifth_bits_reduce_to_int4():
    wl = synth.WORKLOADS["qkv"]
    x = synth.activations(wl)
    pl, tl, cl = synth.rotations(wl)
    A, S, _ = prologue.rotate_quant(x, pl, tl, cl)
    w4 = synth.weights(wl)
    zero_k = np.zeros((wl.K, wl.N // 32), dtype=np.int32)
    zero_g = np.zeros((wl.G, wl.N // 32), dtype=np.int32)
    y5 = int5.gemm_ref5(A, S, w4.qweight, zero_k, w4.qzeros, zero_g, w4.scales, *wl.bounds)
    y4 = gemm.gemm_ref(A, S, w4.qweight, w4.qzeros, w4.scales, *wl.bounds)
    assert np.array_equal(y5, y4)


def test_I5_3_exact_rational():
    wl = synth.Workload("i5tiny", 151, 3, 256, 64)
    x = synth.activations(wl)
    pl, tl, cl = synth.rotations(wl)
    A, S, _ = prologue.rotate_quant(x, pl, tl, cl)
    w = synth.weights5(wl)
    y = int5.gemm_ref5(A, S, w.qweight, w.qweight_hi, w.qzeros, w.qzeros_hi, w.scales, *wl.bounds)
    D = e4m3.decode(A[0])
    for m in range(wl.M):
        for n in (0, 17, 31, 32, wl.N - 1):
            exact = Fraction(0)
            for g in range(wl.G):
                dot = sum(Fraction(float(D[m, k])) * (int(w.codes[k, n]) - int(w.zp[g, n]))
                          for k in range(128 * g, 128 * g + 128))
                exact += F(S[0, m, g]) * F(w.scales[g, n]) * dot
            assert abs(Fraction(float(y[m, n])) - exact) <= abs(exact) * Fraction(1, 2 ** 50) + Fraction(1, 2 ** 80)


def test_I5_4_signed_codes_exact_in_e4m3():
    v = np.arange(-16, 16, dtype=np.float64)
    for scale in (1.0, 2.0 ** -9):
        q = (v * scale).astype(np.float32)
        assert np.array_equal(e4m3.decode(e4m3.encode(q)), v * scale)
    # the first integer e4m3 cannot represent
    assert e4m3.decode(e4m3.encode(np.array([17.0], dtype=np.float32)))[0] != 17.0


def test_I5_5_closed_form():
    K, N = 128, 64
    one = e4m3.encode(np.array([1.0], dtype=np.float32))[0]
    A = np.full((1, 1, K), one, dtype=np.uint8)
    S = np.ones((1, 1, 1), dtype=np.float32)
    codes = np.full((K, N), 31, dtype=np.uint8)
    zp = np.zeros((1, N), dtype=np.uint8)
    sc = synth.rng(152).uniform(0.001, 0.01, (1, N)).astype(np.float16)
    y = int5.gemm_ref5(A, S, synth.awq_pack(codes & 15), synth.bitplane_pack(codes >> 4),
                       synth.awq_pack(zp & 15), synth.bitplane_pack(zp >> 4), sc, synth.NO_BOUNDARY, synth.NO_BOUNDARY)
    assert np.array_equal(y[0], 128 * 31 * sc[0].astype(np.float64))
