"""Per-group int8 activation mode (prologue and GEMM) — oracle, test infrastructure only.

Source: "ParoQuant (PARO) W4A8 on gfx1201 — engineering log":
* section "2026-09-11: I8 mode -- int8 activations on the iu8 WMMA (W5A8-int8) ...": every
  activation producer has an int8 variant with scale amax/127, round and clamp to +-127 and
  integer row-sums; the weight codes multiply the int8 codes in integer arithmetic (int32
  products per group) and the fold algebra and SZ layout are those of the e4m3 path;
* section "2026-09-11 (late): SAME-STACK reference -- ... int8 per-group wins" and "2026-09-11
  (evening): per-group int8 on the A-tiled band": the per-group granularity (one scale per
  token and 128-group), as in the e4m3 path.

Definition, for each partition p, token m, group g (v = the rotated float32 row of the e4m3
oracle, ``prologue.rotate_f32``):

1. ``amax = max_{k in g} |v_k|``;  ``asg = fl32(amax / 127)``
2. ``amax == 0``: all codes 0, asg = +0, rs = +0
3. else ``inv = fl32(1/asg)``;  ``q_k = clamp(rne(fl32(v_k * inv)), -127, 127)`` (int8)
4. ``rs = sum_{k in g} q_k`` (an integer, |rs| <= 127*128, exact in float32)

GEMM, for column n in partition p(n):

    y[m, n] = sum_g asg_p[m, g] * sc[g, n] * sum_{k in g} q_p[m, k] * (c[k, n] - zp[g, n])

Readings taken: the scale is a true division by 127 (the page writes amax/127; the e4m3 path
spells out a multiply by fl32(1/448)); codes go through a reciprocal multiply like the e4m3
path; "round" is round-half-even, the IEEE default.
"""
import numpy as np

from . import awq
from . import records as _records
from .gemm import partition_of_columns
from .prologue import GROUP, rotate_f32


def quantize_groups_i8(v):
    """Steps 1-4 on rotated float32 v [M, K] -> (codes int8 [M, K], asg f32 [M, G], rs f32 [M, G])."""
    M, K = v.shape
    G = K // GROUP
    vg = v.reshape(M, G, GROUP)
    amax = np.abs(vg).max(axis=2)
    asg = (amax / np.float32(127.0)).astype(np.float32)      # f32 division, one rounding
    zero = amax == 0
    with np.errstate(divide="ignore", invalid="ignore"):
        inv = np.float32(1.0) / asg
        q = vg * inv[:, :, None]                             # f32 multiply
    q = np.rint(np.where(zero[:, :, None], np.float32(0.0), q))   # round half to even
    q = np.clip(q, -127, 127).astype(np.int8)
    rs = q.astype(np.int64).sum(axis=2).astype(np.float32)
    asg = np.where(zero, np.float32(0.0), asg).astype(np.float32)
    return q.reshape(M, K), asg, rs


def rotate_quant_i8(x, pairs_list, theta_list, cs_list):
    """P partitions -> A int8 [P, M, K], ASG f32 [P, M, G], RS f32 [P, M, G]."""
    outs = []
    for pairs, theta, cs in zip(pairs_list, theta_list, cs_list):
        rec = _records.build(pairs, theta)
        outs.append(quantize_groups_i8(rotate_f32(x, rec, cs)))
    return tuple(np.stack([o[i] for o in outs]) for i in range(3))


def gemm_ref_i8(A, ASG, qweight, qzeros, scales, pb1, pb2, rows=None, chunk=2048):
    """A int8 [P, M, K], ASG f32 [P, M, G], AWQ tensors -> y float64 [len(rows), N]. The per-group
    integer sums are exact in fp64 (|q (c - zp)| <= 127 * 15, 128 terms)."""
    A = np.asarray(A)
    P, M, K = A.shape
    G = K // GROUP
    if rows is None:
        rows = np.arange(M)
    Q = A[:, rows, :].astype(np.float64)
    asg = np.asarray(ASG, dtype=np.float32)[:, rows, :].astype(np.float64)
    N = np.asarray(scales).shape[1]
    part = partition_of_columns(N, pb1, pb2)
    y = np.zeros((len(rows), N), dtype=np.float64)
    for n0 in range(0, N, chunk):
        n1 = min(N, n0 + chunk)
        c = awq.unpack(np.asarray(qweight)[:, n0 // 8:n1 // 8]).astype(np.float64)
        zp = awq.unpack(np.asarray(qzeros)[:, n0 // 8:n1 // 8]).astype(np.float64)
        sc = np.asarray(scales, dtype=np.float16)[:, n0:n1].astype(np.float64)
        pc = part[n0:n1]
        for p in np.unique(pc):
            cols = np.flatnonzero(pc == p)
            acc = np.zeros((len(rows), len(cols)), dtype=np.float64)
            for g in range(G):
                ks = slice(g * GROUP, (g + 1) * GROUP)
                w = c[ks][:, cols] - zp[g, cols][None, :]
                acc += (asg[p][:, g][:, None] * sc[g, cols][None, :]) * (Q[p][:, ks] @ w)
            y[:, n0 + cols] = acc
    return y
