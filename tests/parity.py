"""GEMM parity gates shared by the GPU tests (test logic only; the references come from oracle/).

Every GEMM variant is gated three ways against the oracle's fp64 reference on the same activation
codes:

1. Frobenius: ``||y - y_ref||_F / ||y_ref||_F <= 2e-3`` overall and per partition range (the
   reading of the page's "rel" in its "Gates passed" section; bf16 output rounding alone gives
   ~1.66e-3 on random data).
2. Element-wise: for every output element

       |y - y_ref| <= 2^-8 |y_ref| + (1 + 2^-8) (g1 Y_raw + g2 Z_raw + g3 Z_q) + 2^-133

   where the three magnitudes are the absolute sizes of what the kernels actually add up:

   * ``Y_raw[m, n] = sum_g s[m, g] sc[g, n] sum_k |D(a_mk)| |w_kn|``: the group products on the
     matrix core with the raw weight operand ``w`` (the 4-bit code c, or c - 16 for int5), folded
     with the group factor in binary32;
   * ``Z_raw[m, n] = sum_g s[m, g] |rs[m, g]| sc[g, n] z[g, n]``: the zero-point term, z = zp for
     int4 (the factor 8 sc + zsc) and |zp - 16| for int5;
   * ``Z_q[m, n] = sum_g s[m, g] |rs[m, g]| sc[g, n] |zp - o|``: the part of that term that passes
     through the f16 rounding of ``zsc = fl16(sc (zp - o))`` stored in the page's SZ format
     (o = 8, or 16 for int5), which the oracle does not round.

   with u = 2^-24 and G groups:

   * ``g1 = (2*128 + G + 16) u``: a 128-term binary32 sum inside the matrix core in any order
     (error <= 127 u sum|p|, doubled for a truncating adder), then per group the factor product,
     the fused multiply-add of the fold and the partial-sum merges;
   * ``g2 = 2^-14 + (3G + 16) u``: the prefill kernel's bf16-split zero-point product
     (a1 z1 + a1 z2 + a2 z1 misses at most 3.02 * 2^-16 of a z) accumulated over 3G terms, and
     the decode kernel's in-loop binary32 form (a few roundings per group);
   * ``g3 = 2^-11``: half an ulp of f16 relative to ``sc (zp - o)`` (a normal f16 here).

   ``2^-8 |y_ref|`` is the bf16 round-to-nearest step (half an ulp of an 8-bit significand), and
   ``(1 + 2^-8)`` carries the binary32 error through that rounding.
3. Rows past M untouched (checked by the callers with sentinels).

The per-element diagnostic ``max |y - y_ref| / ||y_ref[m, :]||_inf`` is printed with every check.
"""
import numpy as np

from oracle import awq, e4m3, int5 as oint5

TOL = 2e-3
U = 2.0 ** -24
GROUP = 128


def gammas(G):
    return (2 * 128 + G + 16) * U, 2.0 ** -14 + (3 * G + 16) * U, 2.0 ** -11


def _partitions(N, pb1, pb2):
    n = np.arange(N)
    return (n >= pb1).astype(np.int64) + (n >= pb2).astype(np.int64)


def magnitudes(D, s, wraw, zfac, zq, sc, pb1, pb2, chunk=2048):
    """D float64 [P, R, K] decoded activation codes; s float64 [P, R, G] activation scale of each
    group (the token scale repeated for the per-token path); wraw float64 [K, N] raw weight operand;
    zfac, zq float64 [G, N]; sc float64 [G, N]. Returns (Y_raw, Z_raw, Z_q) float64 [R, N]."""
    P, R, K = D.shape
    G = K // GROUP
    N = sc.shape[1]
    part = _partitions(N, pb1, pb2)
    Dabs = np.abs(D)
    rs = np.abs(D.reshape(P, R, G, GROUP).sum(-1))          # |exact row-sum| per group
    Y = np.zeros((R, N))
    Z = np.zeros((R, N))
    Zq = np.zeros((R, N))
    for n0 in range(0, N, chunk):
        n1 = min(N, n0 + chunk)
        pc = part[n0:n1]
        for p in np.unique(pc):
            cols = n0 + np.flatnonzero(pc == p)
            wa = np.abs(wraw[:, cols])
            acc = np.zeros((R, len(cols)))
            for g in range(G):
                ks = slice(g * GROUP, (g + 1) * GROUP)
                acc += (s[p][:, g][:, None] * sc[g, cols][None, :]) * (Dabs[p][:, ks] @ wa[ks])
            Y[:, cols] = acc
            ar = s[p] * rs[p]                                 # [R, G]
            Z[:, cols] = ar @ (sc[:, cols] * zfac[:, cols])
            Zq[:, cols] = ar @ (sc[:, cols] * zq[:, cols])
    return Y, Z, Zq


def magnitudes_int4(A, S, w, pb1, pb2, rows=None, act="e4m3", tok=False):
    """Magnitudes for pq_gemm / pq_gemm_tok (e4m3 codes) and pq_gemm_i8 (act="int8") on the int4
    weights ``w`` (synth.Weights); S is ASG [P, M, G], or AS [P, M] with tok=True."""
    A = np.asarray(A)
    rows = np.arange(A.shape[1]) if rows is None else rows
    A = A[:, rows]
    D = A.astype(np.int8).astype(np.float64) if act == "int8" else e4m3.decode(A)
    G = A.shape[2] // GROUP
    S = np.asarray(S, dtype=np.float32)
    s = np.repeat(S[:, rows, None], G, axis=2) if tok else S[:, rows]
    c = awq.unpack(np.asarray(w.qweight)).astype(np.float64)
    zp = awq.unpack(np.asarray(w.qzeros)).astype(np.float64)
    sc = np.asarray(w.scales, dtype=np.float16).astype(np.float64)
    return magnitudes(D, s.astype(np.float64), c, zp, np.abs(zp - 8), sc, pb1, pb2)


def magnitudes_int5(A, S, w5, pb1, pb2, rows=None):
    """Magnitudes for pq_gemm5 on the int5 weights ``w5`` (synth.Weights5)."""
    A = np.asarray(A)
    rows = np.arange(A.shape[1]) if rows is None else rows
    A = A[:, rows]
    c = oint5.codes5(w5.qweight, w5.qweight_hi).astype(np.float64)
    zp = oint5.codes5(w5.qzeros, w5.qzeros_hi).astype(np.float64)
    sc = np.asarray(w5.scales, dtype=np.float16).astype(np.float64)
    S = np.asarray(S, dtype=np.float32)[:, rows].astype(np.float64)
    return magnitudes(e4m3.decode(A), S, c - 16, np.abs(zp - 16), np.abs(zp - 16), sc, pb1, pb2)


def rel_frobenius(y, y_ref):
    den = np.linalg.norm(y_ref)
    return float(np.linalg.norm(y - y_ref) / den) if den > 0 else float(np.linalg.norm(y))


def check(tag, y, y_ref, mags, bounds, G):
    """All three gates on y (float64 [R, N], the GPU's bf16 output) against y_ref; raises
    AssertionError naming the first violated gate."""
    y = np.asarray(y, dtype=np.float64)
    y_ref = np.asarray(y_ref, dtype=np.float64)
    R, N = y_ref.shape
    assert y.shape == y_ref.shape
    assert np.all(np.isfinite(y)), f"{tag}: non-finite output"
    pb1, pb2 = bounds
    edges = [0] + [b for b in (pb1, pb2) if b < N] + [N]
    parts = [rel_frobenius(y[:, a:b], y_ref[:, a:b]) for a, b in zip(edges[:-1], edges[1:])]
    rel = rel_frobenius(y, y_ref)
    g1, g2, g3 = gammas(G)
    Y, Z, Zq = mags
    err = np.abs(y - y_ref)
    bound = 2.0 ** -8 * np.abs(y_ref) + (1 + 2.0 ** -8) * (g1 * Y + g2 * Z + g3 * Zq) + 2.0 ** -133
    ratio = err / bound
    rowinf = np.abs(y_ref).max(axis=1, keepdims=True)
    o6 = float((err / np.where(rowinf > 0, rowinf, 1.0)).max()) if err.size else 0.0
    worst = np.unravel_index(int(np.argmax(ratio)), ratio.shape) if ratio.size else (0, 0)
    print(f"[{tag}] rows={R} rel={rel:.3e} per-partition={[f'{p:.3e}' for p in parts]} "
          f"max|err|/||y_ref[m,:]||_inf={o6:.3e} max err/bound={ratio.max() if ratio.size else 0:.3f} "
          f"at (m={worst[0]}, n={worst[1]})", flush=True)
    assert rel <= TOL and max(parts) <= TOL, f"{tag}: Frobenius gate rel={rel:.3e} parts={parts}"
    bad = int(np.count_nonzero(err > bound))
    assert bad == 0, f"{tag}: {bad} elements outside the element-wise bound (worst ratio {ratio.max():.3f})"
    return rel
