"""Per-token activation-scale path (prologue and GEMM) — oracle, test infrastructure only.

Source: "ParoQuant (PARO) W4A8 on gfx1201 — engineering log":
* section "Numbers", the per-token prefill bullet: the token scale is the largest of the token's
  group scales, the codes are encoded with it, the row-sums are plain code sums, and the GEMM
  applies the token scale in its epilogue while folding the column scales per group;
* section "2026-09-08: MXFP4-PARO prod decode -- the launch-count regression and its three
  fixes", item 1: the fused prologue keeps the rotated row on chip between the token amax and
  the encode, and taking the maximum before or after the division by 448 gives the same scale;
* section "2026-09-09 (late): int4 PARO gets the MXFP4-PARO lessons ...": the fused prologue
  also emits the plain per-group code row-sums, with no bf16 round trip of the rotated row.

Definition, for each partition p and token m (v = the rotated float32 row of the per-group
oracle, ``prologue.rotate_f32``):

1. ``amax = max_k |v_k|`` over the whole row; ``As = fl32(amax * fl32(1/448))``
2. ``amax == 0``: all codes 0x00, As = +0, every rs = +0
3. else ``inv = fl32(1/As)``; ``code_k = E(fl32(v_k * inv))``
4. ``rs[g] = fl32(sum_{k in g} D(code_k))`` (exact sum, rounded once)

GEMM, for column n in partition p(n):

    y[m, n] = As_p[m] * sum_g sc[g, n] * sum_{k in g} D(A_p[m, k]) * (c[k, n] - zp[g, n])

Reading taken: the codes are encoded from the float32 rotated values (the page's first build
went through a bf16 scratch row; its final fused prologue has none).
"""
import numpy as np

from . import awq, e4m3
from . import records as _records
from .gemm import partition_of_columns
from .prologue import C448, GROUP, rotate_f32


def quantize_tokens(v):
    """Steps 1-4 on rotated float32 v [M, K] -> (codes u8 [M, K], As f32 [M], rs f32 [M, G])."""
    M, K = v.shape
    G = K // GROUP
    amax = np.abs(v).max(axis=1)                        # exact
    As = (amax * C448).astype(np.float32)               # one f32 rounding
    zero = amax == 0
    with np.errstate(divide="ignore", invalid="ignore"):
        inv = np.float32(1.0) / As                      # correctly rounded f32 reciprocal
        q = v * inv[:, None]                            # f32 multiply
    codes = e4m3.encode(q)
    codes[zero] = 0
    rs = e4m3.decode(codes.reshape(M, G, GROUP)).sum(axis=2).astype(np.float32)
    As = np.where(zero, np.float32(0.0), As).astype(np.float32)
    rs[zero] = 0
    return codes, As, rs


def rotate_quant_tok(x, pairs_list, theta_list, cs_list):
    """Full per-token prologue for P partitions -> A u8 [P, M, K], AS f32 [P, M], RS f32 [P, M, G]."""
    outs = []
    for pairs, theta, cs in zip(pairs_list, theta_list, cs_list):
        rec = _records.build(pairs, theta)
        outs.append(quantize_tokens(rotate_f32(x, rec, cs)))
    return tuple(np.stack([o[i] for o in outs]) for i in range(3))


def gemm_ref_tok(A, AS, qweight, qzeros, scales, pb1, pb2, rows=None, chunk=2048):
    """A u8 [P, M, K], AS f32 [P, M], AWQ tensors -> y float64 [len(rows), N]. The per-group
    inner sums are exact in fp64, as in the per-group reference."""
    A = np.asarray(A)
    P, M, K = A.shape
    G = K // GROUP
    if rows is None:
        rows = np.arange(M)
    Dv = e4m3.decode(A[:, rows, :])                     # [P, R, K] float64
    As = np.asarray(AS, dtype=np.float32)[:, rows].astype(np.float64)
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
                acc += sc[g, cols][None, :] * (Dv[p][:, ks] @ w)
            y[:, n0 + cols] = As[p][:, None] * acc
    return y
