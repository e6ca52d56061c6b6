"""Same-codes reference GEMM in fp64 — oracle, test infrastructure only.

Source: "ParoQuant (PARO) W4A8 on gfx1201 — engineering log":
* section "Format": W[n, k] = sc[g, n] * (c[k, n] - zp[g, n]) with AWQ-packed codes;
* section "Design" items 1-2 and 4: per 128-group the activation codes carry one scale
  ``asg[m, g]``; a merged linear holds P activation partitions and column n reads the
  partition whose column range contains it;
* section "Gates passed": the GEMM is gated against a same-codes fp64 reference.

Definition computed here, for column n in partition p(n):

    y[m, n] = sum_g asg_p[m, g] * sc[g, n] * sum_{k in g} D(A_p[m, k]) * (c[k, n] - zp[g, n])

The inner sum is exact in fp64 (|D| * 2^9 <= 448 * 512, |c - zp| <= 15, 128 terms: far
below 2^53 units of 2^-9), so its value does not depend on summation order. The outer sum
over groups is an ordinary fp64 sum. The zero point enters exactly (not through any f16
rounding of ``sc * (zp - 8)``). Columns are processed in chunks to bound host memory.
"""
import numpy as np

from . import awq, e4m3

GROUP = 128


def partition_of_columns(N, pb1, pb2):
    """p(n) = [n >= pb1] + [n >= pb2] (boundaries past N mean 'no boundary')."""
    n = np.arange(N)
    return (n >= pb1).astype(np.int64) + (n >= pb2).astype(np.int64)


def gemm_ref(A, ASG, qweight, qzeros, scales, pb1, pb2, rows=None, chunk=2048):
    """A u8 [P, M, K], ASG f32 [P, M, G], AWQ tensors -> y float64 [len(rows), N].

    ``rows`` (optional index array) restricts the output to a sample of token rows.
    """
    A = np.asarray(A)
    P, M, K = A.shape
    G = K // GROUP
    if rows is None:
        rows = np.arange(M)
    Dv = e4m3.decode(A[:, rows, :])                     # [P, R, K] float64
    asg = np.asarray(ASG, dtype=np.float32)[:, rows, :].astype(np.float64)
    N = np.asarray(scales).shape[1]
    part = partition_of_columns(N, pb1, pb2)
    y = np.zeros((len(rows), N), dtype=np.float64)
    for n0 in range(0, N, chunk):
        n1 = min(N, n0 + chunk)
        c = awq.unpack(np.asarray(qweight)[:, n0 // 8:n1 // 8]).astype(np.float64)   # [K, nc]
        zp = awq.unpack(np.asarray(qzeros)[:, n0 // 8:n1 // 8]).astype(np.float64)   # [G, nc]
        sc = np.asarray(scales, dtype=np.float16)[:, n0:n1].astype(np.float64)        # [G, nc]
        pc = part[n0:n1]
        for p in np.unique(pc):
            cols = np.flatnonzero(pc == p)
            acc = np.zeros((len(rows), len(cols)), dtype=np.float64)
            for g in range(G):
                ks = slice(g * GROUP, (g + 1) * GROUP)
                w = c[ks][:, cols] - zp[g, cols][None, :]          # integer-valued
                dot = Dv[p][:, ks] @ w                              # exact per group
                acc += (asg[p][:, g][:, None] * sc[g, cols][None, :]) * dot
            y[:, n0 + cols] = acc
    return y


def rel_frobenius(y, y_ref):
    """||y - y_ref||_F / ||y_ref||_F."""
    y = np.asarray(y, dtype=np.float64)
    y_ref = np.asarray(y_ref, dtype=np.float64)
    den = np.linalg.norm(y_ref)
    return float(np.linalg.norm(y - y_ref) / den) if den > 0 else float(np.linalg.norm(y))
