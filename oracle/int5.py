"""int5 bit-plane weights (W5A8) GEMM — oracle, test infrastructure only.

Source: "ParoQuant (PARO) W4A8 on gfx1201 — engineering log", section "2026-09-10: int5 W5A8
ParoQuant -- round-to-nearest checkpoint, kernel and first served numbers":
* weights are uniform asymmetric 5-bit codes c in 0..31 per 128-group, with a zero point in
  0..31 and an f16 scale; a weight dequantises as sc * (c - zp), as in the int4 format;
* the "int5-bitplane" checkpoint keeps the low four bits of the codes and of the zero points in
  the int4 (AWQ) words ``qweight [K, N/8]`` / ``qzeros [G, N/8]`` and the fifth bits in the planes
  ``qweight_hi [K, N/32]`` / ``qzeros_hi [G, N/32]`` (int32);
* the activations, their per-group scales and the GEMM algebra are those of the int4 path (the
  kernel feeds c - 16, which is exact in e4m3 for every code).

Definition computed here, for column n in partition p(n):

    y[m, n] = sum_g asg_p[m, g] * sc[g, n] * sum_{k in g} D(A_p[m, k]) * (c[k, n] - zp[g, n])

with c = low4 + 16 * bit5 (and likewise zp). The inner sum is exact in fp64 (|c - zp| <= 31).

Readings (the page gives the planes' shapes only): bit j of plane word [r, w] is the fifth bit
of column 32w + j; ``qzeros_hi`` has one row per group. Against a real checkpoint this layout is
parity unpinned (none is available here).
"""
import numpy as np

from . import awq, e4m3
from .gemm import GROUP, partition_of_columns


def unpack_hi(plane) -> np.ndarray:
    """int32 [R, N/32] -> uint8 bits [R, N] (0/1): bit j of word w is column 32w + j."""
    w = np.asarray(plane).astype(np.int64) & 0xFFFFFFFF
    R, N32 = w.shape
    out = np.empty((R, N32 * 32), dtype=np.uint8)
    for j in range(32):
        out[:, j::32] = ((w >> j) & 1).astype(np.uint8)
    return out


def codes5(low_words, hi_plane) -> np.ndarray:
    """AWQ low-nibble words [R, N/8] + fifth-bit plane [R, N/32] -> uint8 codes [R, N] in 0..31."""
    return (awq.unpack(low_words) + 16 * unpack_hi(hi_plane)).astype(np.uint8)


def dequant5(qweight, qweight_hi, qzeros, qzeros_hi, scales) -> np.ndarray:
    """Exact fp64 W^T [K, N]: sc[g(k), n] * (c[k, n] - zp[g(k), n])."""
    c = codes5(qweight, qweight_hi).astype(np.float64)
    zp = codes5(qzeros, qzeros_hi).astype(np.float64)
    sc = np.asarray(scales, dtype=np.float16).astype(np.float64)
    g = np.arange(c.shape[0]) // GROUP
    return sc[g, :] * (c - zp[g, :])


def gemm_ref5(A, ASG, qweight, qweight_hi, qzeros, qzeros_hi, scales, pb1, pb2, rows=None, chunk=2048):
    """A u8 [P, M, K] (e4m3 codes), ASG f32 [P, M, G], int5 bit-plane tensors -> y float64
    [len(rows), N]."""
    A = np.asarray(A)
    P, M, K = A.shape
    G = K // GROUP
    if rows is None:
        rows = np.arange(M)
    Dv = e4m3.decode(A[:, rows, :])
    asg = np.asarray(ASG, dtype=np.float32)[:, rows, :].astype(np.float64)
    N = np.asarray(scales).shape[1]
    part = partition_of_columns(N, pb1, pb2)
    y = np.zeros((len(rows), N), dtype=np.float64)
    chunk = max(32, chunk // 32 * 32)
    for n0 in range(0, N, chunk):
        n1 = min(N, n0 + chunk)
        c = codes5(np.asarray(qweight)[:, n0 // 8:n1 // 8], np.asarray(qweight_hi)[:, n0 // 32:n1 // 32]).astype(np.float64)
        zp = codes5(np.asarray(qzeros)[:, n0 // 8:n1 // 8], np.asarray(qzeros_hi)[:, n0 // 32:n1 // 32]).astype(np.float64)
        sc = np.asarray(scales, dtype=np.float16)[:, n0:n1].astype(np.float64)
        pc = part[n0:n1]
        for p in np.unique(pc):
            cols = np.flatnonzero(pc == p)
            acc = np.zeros((len(rows), len(cols)), dtype=np.float64)
            for g in range(G):
                ks = slice(g * GROUP, (g + 1) * GROUP)
                w = c[ks][:, cols] - zp[g, cols][None, :]
                acc += (asg[p][:, g][:, None] * sc[g, cols][None, :]) * (Dv[p][:, ks] @ w)
            y[:, n0 + cols] = acc
    return y
