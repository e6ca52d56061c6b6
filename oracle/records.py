"""Givens pair records — oracle, test infrastructure only.

Source: "ParoQuant (PARO) W4A8 on gfx1201 — engineering log", section "Format" (``pairs
[8, K]`` i16 holds Givens pair indices local to each 128-channel group, a permutation of
0..127 per group and layer; ``theta [8, K/2]`` f16 holds one angle per pair) and section
"Design" item 3 (each rotation record carries the two channel indices and f16 cos/sin).

Readings taken where the page is silent:
* pair ``p`` of layer ``r`` is ``(pairs[r, 2p], pairs[r, 2p+1])``, local to group ``p // 64``,
  with angle ``theta[r, p]`` (consecutive entries form the 64 pairs of a group);
* ``cos``/``sin`` are computed in fp64 from the f16 angle and rounded once to f16 (RNE).
"""
import numpy as np

GROUP = 128
LAYERS = 8


def build(pairs, theta):
    """pairs int16 [8, K], theta f16 [8, K/2] -> dict of arrays, each [8, K/2]:

    ``i``, ``j`` (int, local channel 0..127), ``cos16``/``sin16`` (uint16 f16 bit patterns),
    ``cos``/``sin`` (float32 values of those f16 numbers).
    Raises ValueError if a 128-slice of a layer is not a permutation of 0..127.
    """
    pairs = np.asarray(pairs, dtype=np.int64)
    theta = np.asarray(theta, dtype=np.float16)
    L, K = pairs.shape
    if L != LAYERS or K % GROUP or theta.shape != (LAYERS, K // 2):
        raise ValueError("bad pairs/theta shape")
    for r in range(L):
        for g in range(K // GROUP):
            sl = pairs[r, g * GROUP:(g + 1) * GROUP]
            if not np.array_equal(np.sort(sl), np.arange(GROUP)):
                raise ValueError(f"layer {r} group {g}: pairs are not a permutation of 0..127")
    i = pairs[:, 0::2]
    j = pairs[:, 1::2]
    th = theta.astype(np.float64)
    c16 = np.cos(th).astype(np.float16)   # one rounding, fp64 -> f16 RNE
    s16 = np.sin(th).astype(np.float16)
    return {
        "i": i, "j": j,
        "cos16": c16.view(np.uint16), "sin16": s16.view(np.uint16),
        "cos": c16.astype(np.float32), "sin": s16.astype(np.float32),
    }


def rotate_f64(v, pairs, theta, inverse=False, exact_angles=True, rec=None):
    """fp64 rotation of rows of ``v`` [M, K] (a diagnostic / pin helper).

    Forward: layers 0..7, each pair (i, j) maps (a, b) -> (c*a + s*b, c*b - s*a).
    Inverse: layers 7..0 with the angle negated. ``exact_angles`` uses fp64 cos/sin of the
    f16 angle; otherwise the f16-rounded record values.
    """
    v = np.array(v, dtype=np.float64, copy=True)
    pairs = np.asarray(pairs, dtype=np.int64)
    K = v.shape[1]
    base = (np.arange(K // 2) // 64) * GROUP
    I = pairs[:, 0::2] + base
    J = pairs[:, 1::2] + base
    if exact_angles:
        th = np.asarray(theta, dtype=np.float16).astype(np.float64)
        C, S = np.cos(th), np.sin(th)
    else:
        rec = rec if rec is not None else build(pairs, theta)
        C, S = rec["cos"].astype(np.float64), rec["sin"].astype(np.float64)
    layers = range(LAYERS - 1, -1, -1) if inverse else range(LAYERS)
    for r in layers:
        c, s = C[r], (-S[r] if inverse else S[r])
        a, b = v[:, I[r]], v[:, J[r]]
        v[:, I[r]] = c * a + s * b
        v[:, J[r]] = c * b - s * a
    return v
