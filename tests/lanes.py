"""Test helpers for the library's rotation records (pq_build_records): field decoding, the LDS
bank rules the prologue relies on, and a float32 simulation of the prologue's register / LDS
dataflow driven by the records alone (no GPU).

Record word (per layer r, group g, lane l): bits 0-6 channel u (the lane's first operand), bit 7
"v arrives negated" (t = -1), bits 8-14 channel v (second operand), bit 15 "keep v's output",
bits 16-23 the hand-off row read in layers 1..7 (v's value), bits 24-31 the hand-off row written
in layers 0..6 (the output not kept); then f16 f1, f16 f2 = (c, t*s), or (-s, t*c) when v's output
is kept. A lane reads w = t*v and computes keep = f1*u + f2*w and hand = f1*w - f2*u; layer 7
writes t*hand as v's output.
"""
import numpy as np

LAYERS = 8


def lds_row(ch):
    return ch + (ch >> 3)


def decode(lib):
    """lib uint8 [8, K/2, 8] -> dict of [8, K/2] arrays."""
    w = lib[..., :4].copy().view(np.uint32)[..., 0].astype(np.int64)
    f1 = lib[..., 4:6].copy().view(np.uint16)[..., 0]
    f2 = lib[..., 6:8].copy().view(np.uint16)[..., 0]
    return dict(u=w & 0x7F, v=(w >> 8) & 0x7F, keep_v=(w >> 15) & 1, rslot=(w >> 16) & 0xFF,
                wslot=(w >> 24) & 0xFF, f1=f1, f2=f2, neg_v=(w >> 7) & 1)


def canonical(d, r, sl):
    """The rotations that layer r's records in slice sl apply, as (i, j, cos16, sin16) with i < j
    (a pair listed as (j, i) with sin negated is the same rotation)."""
    out = []
    for u, v, kv, t, f1, f2 in zip(d["u"][r, sl], d["v"][r, sl], d["keep_v"][r, sl], d["neg_v"][r, sl],
                                   d["f1"][r, sl], d["f2"][r, sl]):
        f2 = int(f2) ^ (0x8000 if t else 0)                                 # undo v's sign
        c, s = (f2, int(f1) ^ 0x8000) if kv else (int(f1), f2)              # kept v: (f1, f2) = (-s, c)
        out.append((int(u), int(v), c, s) if u < v else (int(v), int(u), c, s ^ 0x8000))
    return sorted(out)


def check_lanes(lib):
    """The LDS bank rules of gfx950 for 16-byte accesses (16-lane blocks of a read need rows
    distinct mod 16, 8-lane blocks of a write rows distinct mod 8), for every access of the layer
    chain: layer 0 reads of the image rows, the hand-off reads of layers 1..7 and writes of layers
    0..6. Also layer 0's operands arrive as they are, layer 7 keeps nothing and the slots are
    rows < 64."""
    d = decode(lib)
    assert not d["neg_v"][0].any()
    assert not d["keep_v"][LAYERS - 1].any()
    assert d["rslot"].max() < 64 and d["wslot"].max() < 64
    n = lib.shape[1] // 64
    for g in range(n):
        sl = slice(64 * g, 64 * g + 64)
        reads = [lds_row(d["u"][0, sl]), lds_row(d["v"][0, sl])] + [d["rslot"][r, sl] for r in range(1, LAYERS)]
        writes = [d["wslot"][r, sl] for r in range(LAYERS - 1)]
        for k, rows in enumerate(reads):
            for blk in range(4):
                assert len(set(rows[16 * blk:16 * blk + 16] % 16)) == 16, ("read", g, k, blk)
        for k, rows in enumerate(writes):
            assert len(set(rows)) == 64, ("slots", g, k)
            for hb in range(8):
                assert len(set(rows[8 * hb:8 * hb + 8] % 8)) == 8, ("write", g, k, hb)


def simulate(lib, xv):
    """The prologue's rotation as its kernels run it, from the records alone: xv float32 [T, K]
    (activations times channel scales) -> rotated float32 [T, K]. Per group: the image holds
    channel ch at row lds_row(ch); in each layer every lane first reads (layer 0 both channels
    from the image, later layers v from its hand-off row, u from its register), then every lane
    writes (layers 0..6 the output not kept to its hand-off row, layer 7 both outputs to the
    image rows of u and v). Every product and sum rounds to float32. Handed-off values travel
    with the sign the records give them; only the last layer's outputs are the rotation's."""
    d = decode(lib)
    f1 = d["f1"].view(np.float16).astype(np.float32)
    f2 = d["f2"].view(np.float16).astype(np.float32)
    T, K = xv.shape
    out = np.empty_like(xv)
    ch = np.arange(128)
    for g in range(K // 128):
        sl = slice(64 * g, 64 * g + 64)
        mem = np.full((144, T), np.nan, np.float32)
        mem[lds_row(ch)] = xv[:, 128 * g + ch].T
        reg = None
        for r in range(LAYERS):
            u, v = d["u"][r, sl], d["v"][r, sl]
            a = mem[lds_row(u)] if r == 0 else reg
            b = mem[lds_row(v)] if r == 0 else mem[d["rslot"][r, sl]]
            F1, F2 = f1[r, sl][:, None], f2[r, sl][:, None]
            sign = np.where(d["neg_v"][r, sl][:, None] == 1, np.float32(-1), np.float32(1))
            Gm, Dm = (F1, F2) if r < LAYERS - 1 else (sign * F1, sign * F2)
            keep = (F1 * a) + (F2 * b)
            other = (Gm * b) - (Dm * a)
            if r < LAYERS - 1:
                reg = keep
                mem[d["wslot"][r, sl]] = other
            else:
                mem[lds_row(u)] = keep
                mem[lds_row(v)] = other
        out[:, 128 * g + ch] = mem[lds_row(ch)].T
    return out
