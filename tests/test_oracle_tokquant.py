"""Pins of the per-token oracle (oracle/tokquant.py), each against something other than itself.

* T1: the token scale equals the largest group scale the per-group oracle computes on the same
  input, bit for bit (the page states that taking the maximum before or after the division by
  448 gives the same scale).
* T2: when every group of a token has the same amax, per-token and per-group quantisation must
  coincide: same codes, same row-sums, and the token scale equals every group scale.
* T3: exact-rational evaluation of the steps (amax, scale, reciprocal, product) with an
  independently written binary32 rounding, then the pinned encoder, on tiny rows.
* T4: invariants: each non-zero row holds a code of magnitude 448 and none above; a zero row
  gives zero codes, scale and row-sums.
* G-T1: the per-token GEMM equals the pinned per-group GEMM with the token scale broadcast to
  every group; G-T2: an exact-rational evaluation of the definition on a tiny shape.
"""
from fractions import Fraction

import numpy as np

import synth
from oracle import e4m3, gemm, prologue, tokquant

from test_oracle_prologue import F, rnd32

WL = synth.WORKLOADS["tiny"]


def _inputs(wl, seed_shift=0):
    x = synth.activations(wl)
    pl, tl, cl = synth.rotations(wl)
    return x, pl, tl, cl


def test_T1_token_scale_is_max_group_scale():
    for name in ("tiny", "qkv"):
        wl = synth.WORKLOADS[name]
        x, pl, tl, cl = _inputs(wl)
        _, ASG, _ = prologue.rotate_quant(x, pl, tl, cl)
        _, AS, _ = tokquant.rotate_quant_tok(x, pl, tl, cl)
        assert np.array_equal(AS.view(np.uint32), ASG.max(axis=2).view(np.uint32)), name


def test_T2_equal_group_amax_reduces_to_per_group():
    r = np.random.default_rng(3)
    M, K = 6, 512
    x = (r.uniform(-1, 1, (M, K)) * 2.0).astype(np.float16)
    # every 128-group of a row holds the same largest magnitude, at a random position and sign
    for m in range(M):
        a = np.float16(3.0 + m)
        for g in range(K // 128):
            x[m, 128 * g + r.integers(128)] = a if r.integers(2) else -a
    zero_theta = [np.zeros((8, K // 2), np.float16)]
    pairs = [np.tile(np.arange(128, dtype=np.int16), (8, K // 128))]
    ones = [np.ones(K, np.float16)]
    A1, ASG, RS1 = prologue.rotate_quant(x, pairs, zero_theta, ones)
    A2, AS, RS2 = tokquant.rotate_quant_tok(x, pairs, zero_theta, ones)
    assert np.array_equal(A1, A2)
    assert np.array_equal(RS1.view(np.uint32), RS2.view(np.uint32))
    assert np.array_equal(np.broadcast_to(AS[:, :, None], ASG.shape).view(np.uint32), ASG.view(np.uint32))


def test_T3_exact_rational_steps():
    r = np.random.default_rng(5)
    K = 256
    for trial in range(4):
        v = (r.standard_normal((2, K)) * np.exp(r.normal(0, 2))).astype(np.float32)
        codes, As, rs = tokquant.quantize_tokens(v)
        c448 = rnd32(Fraction(1, 448))
        for m in range(2):
            amax = max(abs(F(t)) for t in v[m])
            as_m = rnd32(amax * c448)
            assert F(As[m]) == as_m
            inv = rnd32(1 / as_m)
            q = np.array([float(rnd32(F(t) * inv)) for t in v[m]], dtype=np.float32)
            want = e4m3.encode(q)
            assert np.array_equal(codes[m], want)
            for g in range(K // 128):
                exact = sum(Fraction(float(d)) for d in e4m3.decode(want[128 * g:128 * g + 128]))
                assert F(rs[m, g]) == rnd32(exact)


def test_T4_invariants_and_zero_row():
    wl = synth.WORKLOADS["qkv"]
    x, pl, tl, cl = _inputs(wl)
    x = x.copy()
    x[1] = 0
    A, AS, RS = tokquant.rotate_quant_tok(x, pl, tl, cl)
    D = np.abs(e4m3.decode(A))
    for p in range(A.shape[0]):
        for m in range(A.shape[1]):
            if m == 1:
                assert not A[p, m].any() and AS[p, m] == 0 and not RS[p, m].any()
                assert not np.signbit(AS[p, m])
                continue
            assert D[p, m].max() == 448.0
    G = A.shape[2] // 128
    dec = e4m3.decode(A).reshape(A.shape[0], A.shape[1], G, 128).sum(axis=3)
    assert np.array_equal(RS, dec.astype(np.float32))


def test_GT1_reduces_to_per_group_gemm():
    for name in ("tiny", "qkv"):
        wl = synth.WORKLOADS[name]
        x, pl, tl, cl = _inputs(wl)
        w = synth.weights(wl)
        A, AS, _ = tokquant.rotate_quant_tok(x, pl, tl, cl)
        G = A.shape[2] // 128
        ASG = np.repeat(AS[:, :, None], G, axis=2)
        y_tok = tokquant.gemm_ref_tok(A, AS, w.qweight, w.qzeros, w.scales, *wl.bounds)
        y_grp = gemm.gemm_ref(A, ASG, w.qweight, w.qzeros, w.scales, *wl.bounds)
        assert gemm.rel_frobenius(y_tok, y_grp) < 1e-13, name


def test_GT2_exact_rational():
    wl = WL
    x, pl, tl, cl = _inputs(wl)
    w = synth.weights(wl)
    A, AS, _ = tokquant.rotate_quant_tok(x, pl, tl, cl)
    from oracle import awq
    c = awq.unpack(w.qweight)
    zp = awq.unpack(w.qzeros)
    sc = w.scales
    D = e4m3.decode(A[0])
    y = tokquant.gemm_ref_tok(A, AS, w.qweight, w.qzeros, w.scales, *wl.bounds)
    for m in range(wl.M):
        for n in (0, 5, 77, wl.N - 1):
            tot = Fraction(0)
            for g in range(wl.K // 128):
                dot = sum(Fraction(float(D[m, k])) * (int(c[k, n]) - int(zp[g, n])) for k in range(128 * g, 128 * g + 128))
                tot += F(sc[g, n]) * dot
            exact = F(AS[0, m]) * tot
            assert abs(Fraction(float(y[m, n])) - exact) <= abs(exact) * Fraction(1, 2 ** 50) + Fraction(1, 2 ** 80)
