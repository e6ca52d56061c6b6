"""Rotate-quant prologue — oracle, test infrastructure only.

Source: "ParoQuant (PARO) W4A8 on gfx1201 — engineering log":
* section "Format", inference identity: activations are multiplied by the (pre-inverted)
  channel scales and rotated forward, layers 0..7, inside each 128-channel group;
* section "Design" items 2-3: one e4m3 scale per (token, 128-group); the prologue fuses
  channel scale, rotation, amax, e4m3 encode (RNE, saturating) and code-domain row-sums;
* section "Gates passed": the scale is ``amax * (1/448.f)``.

Every step is emulated in IEEE binary32 with numpy float32 arrays (one rounding per written
operation, no fused multiply-add), in this order, for each partition p, token m, group g:

1. ``v = f32(x) * f32(cs)``                        (exact: 11 x 11 significand bits)
2. for layer r = 0..7, every pair (i, j, c, s) of the layer in g:
   ``a, b = v_i, v_j;  v_i = (c*a) + (s*b);  v_j = (c*b) - (s*a)``
3. ``amax = max |v|``;  ``asg = amax * fl32(1/448)``
4. ``amax == 0``: all codes 0x00, asg = +0, rs = +0
5. else ``inv = fl32(1/asg)``; ``q = v * inv``; ``code = E(q)``
6. ``rs = fl32(sum D(code))``, the sum taken exactly (every D value is a multiple of 2^-9
   and |sum| * 2^9 < 2^25, so the fp64 sum is exact) and rounded once.

Readings taken where the page is silent (the Givens sign convention, the no-contraction
fp32 form, encoding through a reciprocal multiply, the all-zero group) are listed in the
module docstrings and the design notes.
"""
import numpy as np

from . import e4m3
from . import records as _records

GROUP = 128
C448 = np.float32(1.0) / np.float32(448.0)   # fl32(1/448) == 0x3B124925


def rotate_f32(x, rec, cs):
    """Steps 1-2 for one partition: x f16 [M, K], rec from records.build, cs f16 [K]
    -> rotated float32 [M, K]."""
    v = np.asarray(x, dtype=np.float16).astype(np.float32) * \
        np.asarray(cs, dtype=np.float16).reshape(-1).astype(np.float32)
    K = v.shape[1]
    base = (np.arange(K // 2) // 64) * GROUP
    for r in range(rec["i"].shape[0]):
        I = rec["i"][r] + base
        J = rec["j"][r] + base
        c = rec["cos"][r]
        s = rec["sin"][r]
        a = v[:, I].copy()
        b = v[:, J].copy()
        v[:, I] = (c * a) + (s * b)
        v[:, J] = (c * b) - (s * a)
    return v


def quantize_groups(v):
    """Steps 3-6 on rotated float32 v [M, K] -> (codes u8 [M, K], asg f32 [M, G], rs f32 [M, G])."""
    M, K = v.shape
    G = K // GROUP
    vg = v.reshape(M, G, GROUP)
    amax = np.abs(vg).max(axis=2)                       # exact
    asg = (amax * C448).astype(np.float32)              # one f32 rounding
    zero = amax == 0
    with np.errstate(divide="ignore", invalid="ignore"):
        inv = np.float32(1.0) / asg                     # correctly rounded f32 reciprocal
        q = vg * inv[:, :, None]                        # f32 multiply
    codes = e4m3.encode(q)
    codes[zero] = 0
    rs = e4m3.decode(codes).sum(axis=2).astype(np.float32)   # exact fp64 sum, rounded once
    asg = np.where(zero, np.float32(0.0), asg).astype(np.float32)
    rs = np.where(zero, np.float32(0.0), rs).astype(np.float32)
    return codes.reshape(M, K), asg, rs


def rotate_quant(x, pairs_list, theta_list, cs_list):
    """Full prologue for P partitions (lists of per-partition pairs/theta/cs).

    Returns A u8 [P, M, K], ASG f32 [P, M, G], RS f32 [P, M, G].
    """
    outs = []
    for pairs, theta, cs in zip(pairs_list, theta_list, cs_list):
        rec = _records.build(pairs, theta)
        outs.append(quantize_groups(rotate_f32(x, rec, cs)))
    A = np.stack([o[0] for o in outs])
    ASG = np.stack([o[1] for o in outs])
    RS = np.stack([o[2] for o in outs])
    return A, ASG, RS
