"""AWQ uint4 unpack and the dequantised weight — oracle, test infrastructure only.

Source: "ParoQuant (PARO) W4A8 on gfx1201 — engineering log", section "Format":
``qweight [K, N/8]`` and ``qzeros [K/128, N/8]`` are int32 words of eight 4-bit codes in
nibble order 0,2,4,6,1,3,5,7; zero points are stored as-is (not offset by one);
``scales [K/128, N]`` are f16. A weight dequantises as ``sc * (c - zp)`` in its 128-group.

Reading of the nibble order (the page lists it without a direction): nibble ``i`` (bits
4i..4i+3) of word ``j`` holds column ``8*j + ORDER[i]``.
"""
import numpy as np

GROUP = 128
ORDER = (0, 2, 4, 6, 1, 3, 5, 7)


def unpack(words) -> np.ndarray:
    """int32 [R, N/8] -> uint8 codes [R, N] (each 0..15)."""
    w = np.asarray(words).astype(np.int64) & 0xFFFFFFFF
    R, N8 = w.shape
    out = np.empty((R, N8 * 8), dtype=np.uint8)
    for i in range(8):
        out[:, ORDER[i]::8] = ((w >> (4 * i)) & 0xF).astype(np.uint8)
    return out


def dequant(qweight, qzeros, scales) -> np.ndarray:
    """Exact fp64 W^T, shape [K, N]: W[k, n] = sc[g(k), n] * (c[k, n] - zp[g(k), n])."""
    c = unpack(qweight).astype(np.float64)
    zp = unpack(qzeros).astype(np.float64)
    sc = np.asarray(scales, dtype=np.float16).astype(np.float64)
    K = c.shape[0]
    g = np.arange(K) // GROUP
    return sc[g, :] * (c - zp[g, :])
