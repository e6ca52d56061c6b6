"""Fused residual add + RMSNorm + rotate + quant producer — oracle, test infrastructure only.

Source: "ParoQuant (PARO) W4A8 on gfx1201 — engineering log", section "2026-09-02/03: rotation
stream (fused add + RMSNorm + rotate + quant producers)": for every norm-fed linear one kernel does
the residual add, the (Gemma) RMSNorm, the channel scale, the rotation and the per-group quant and
returns the normalised row, the new residual and the prologue tuple (A, ASG, RS). Its gates: the
residual exact, the normalised row within a few parts per million of a CPU reference (the norm's
reduction order is not fixed), and the codes those of the unfused chain.

Definition, per token row (x, r, w f16 [K], eps > 0):

1. ``h = fl16(fl32(x) + fl32(r))``: the new residual stream, stored in the activation format;
2. ``ms = (sum_k h_k^2) / K`` and ``rstd = 1 / sqrt(ms + eps)``, in fp64;
3. ``hs = fl16(h * rstd * w')`` with ``w' = 1 + w`` (the Gemma form) or ``w' = w`` (plain), the
   products in fp64 and one rounding;
4. ``(A, ASG, RS)`` = the per-group prologue (``prologue.rotate_quant``) applied to ``hs``.

Readings (the page names the steps and says only that the norm follows the serving stack's order,
which it does not spell out): the add is one binary32 addition rounded once to f16, and the norm
reads that stored residual; the norm itself is the exact expression above rounded once to f16, so
an implementation in binary32 with any reduction order lands within one f16 step of it; the
quantisation is the pinned per-group prologue on the f16 normalised row, as in the unfused chain.
"""
import numpy as np

from . import prologue


def add_rms(x, r, w, eps, gemma=True):
    """Steps 1-3: f16 [M, K] x, r, f16 [K] w -> (h f16 [M, K], hs f16 [M, K])."""
    h = (np.asarray(x, dtype=np.float16).astype(np.float32) +
         np.asarray(r, dtype=np.float16).astype(np.float32)).astype(np.float16)
    hd = h.astype(np.float64)
    ms = np.mean(hd * hd, axis=1)
    rstd = 1.0 / np.sqrt(ms + float(eps))
    wd = np.asarray(w, dtype=np.float16).astype(np.float64)
    wp = 1.0 + wd if gemma else wd
    hs = (hd * rstd[:, None] * wp[None, :]).astype(np.float16)
    return h, hs


def add_rms_rotate_quant(x, r, w, eps, pairs_list, theta_list, cs_list, gemma=True):
    """Steps 1-4 -> (h, hs, A u8 [P, M, K], ASG f32 [P, M, G], RS f32 [P, M, G])."""
    h, hs = add_rms(x, r, w, eps, gemma)
    A, ASG, RS = prologue.rotate_quant(hs, pairs_list, theta_list, cs_list)
    return h, hs, A, ASG, RS
