"""Seeded synthetic inputs for the PARO W4A8 linear path (shared by tests, smoke and bench).

This module draws random tensors of the shapes, value distributions and structure of the
workloads below and stores them in the checkpoint format (AWQ-packed int32 words). It holds
none of the method's arithmetic: no rotation, no quantisation, no GEMM.

Seeding: tensor ``t`` of workload ``w`` (partition ``p`` where tensors are per partition) is
drawn from ``numpy.random.default_rng([w, t])`` / ``default_rng([w, t, p])``, so a draw does
not depend on the order in which tensors are requested. Values are drawn in fp64 and cast
once (RNE) to their storage type.

Workloads (per the checkpoint format of "ParoQuant (PARO) W4A8 on gfx1201 — engineering
log", section "Format"; shapes are one tensor-parallel rank's share of a 27B model's
projections):

=====  =========================================================================
tiny     M=4, K=256 (2 groups), N=128, 1 partition
decode   M in {1, 8}, K=5120, N=17408 (gate_up), 1 partition
qkv      M=4, K=5120, N=8192 split 6144 | 1024 | 1024, 3 distinct partitions
prefill  M=2048, K=5120, N=17408; 1% outlier channels x20; 10% of groups x1e-3
full     M=8192, K=5120, N=17408 and down-proj M=8192, K=17408, N=5120 (as prefill)
=====  =========================================================================
"""
from dataclasses import dataclass, field
from typing import List, Optional, Tuple

import numpy as np

GROUP = 128
LAYERS = 8
NO_BOUNDARY = 2 ** 31 - 1
AWQ_ORDER = (0, 2, 4, 6, 1, 3, 5, 7)

# tensor ids for the seed tuple
T_X, T_PAIRS, T_THETA, T_CS, T_CODES, T_ZP, T_SCALES, T_OUTCH, T_SMALLG, T_SUBN, T_RES, T_NORMW = range(12)


@dataclass(frozen=True)
class Workload:
    name: str
    wid: int                  # seed id
    M: int
    K: int
    N: int
    splits: Tuple[int, ...] = ()   # partition column widths (empty -> 1 partition)
    outliers: bool = False         # 1% channels x20 and 10% of groups x1e-3

    @property
    def P(self) -> int:
        return max(1, len(self.splits))

    @property
    def G(self) -> int:
        return self.K // GROUP

    @property
    def bounds(self) -> Tuple[int, int]:
        """(pb1, pb2) as column indices; NO_BOUNDARY where unused."""
        if self.P == 1:
            return NO_BOUNDARY, NO_BOUNDARY
        cuts = np.cumsum(self.splits)[:-1].tolist()
        cuts += [NO_BOUNDARY] * (2 - len(cuts))
        return int(cuts[0]), int(cuts[1])


WORKLOADS = {
    "tiny": Workload("tiny", 0, 4, 256, 128),
    "decode_m1": Workload("decode_m1", 1, 1, 5120, 17408),
    "decode_m8": Workload("decode_m8", 1, 8, 5120, 17408),
    "qkv": Workload("qkv", 2, 4, 5120, 8192, splits=(6144, 1024, 1024)),
    "prefill": Workload("prefill", 3, 2048, 5120, 17408, outliers=True),
    "full_gate_up": Workload("full_gate_up", 4, 8192, 5120, 17408, outliers=True),
    "full_down": Workload("full_down", 5, 8192, 17408, 5120, outliers=True),
}


def rng(*key) -> np.random.Generator:
    return np.random.default_rng(list(key))


def awq_pack(codes: np.ndarray) -> np.ndarray:
    """uint8 codes [R, N] (0..15) -> int32 words [R, N/8]: nibble i of word j holds column
    8j + AWQ_ORDER[i] (the checkpoint's nibble order)."""
    codes = np.asarray(codes, dtype=np.uint32)
    R, N = codes.shape
    assert N % 8 == 0
    w = np.zeros((R, N // 8), dtype=np.uint32)
    for i in range(8):
        w |= (codes[:, AWQ_ORDER[i]::8] & 0xF) << np.uint32(4 * i)
    return w.view(np.int32)


def activations(wl: Workload, M: Optional[int] = None) -> np.ndarray:
    """x f16 [M, K] ~ N(0, 1); with ``outliers``: round(1% K) seeded channels x20 and 10% of
    the 128-groups (seeded) x1e-3, applied before the f16 cast (some values become f16
    subnormals)."""
    M = wl.M if M is None else M
    x = rng(wl.wid, T_X).standard_normal((M, wl.K))
    if wl.outliers:
        n_out = int(round(0.01 * wl.K))
        ch = rng(wl.wid, T_OUTCH).choice(wl.K, size=n_out, replace=False)
        x[:, ch] *= 20.0
        n_small = int(round(0.10 * wl.G))
        gs = rng(wl.wid, T_SMALLG).choice(wl.G, size=n_small, replace=False)
        for g in gs:
            x[:, g * GROUP:(g + 1) * GROUP] *= 1e-3
    return x.astype(np.float16)


def activations_one_signed(wl: Workload, M: Optional[int] = None) -> np.ndarray:
    """x f16 [M, K] = |N(0, 1)| with round(1% K) seeded outlier channels x20: every value >= 0,
    as post-activation inputs of a down projection are. With identity rotations
    (``rotations_identity``) the e4m3 codes stay one-signed, the case where the code-domain
    zero-point correction cancels hardest against the raw-code products."""
    M = wl.M if M is None else M
    x = np.abs(rng(wl.wid, T_X, 1).standard_normal((M, wl.K)))
    n_out = int(round(0.01 * wl.K))
    ch = rng(wl.wid, T_OUTCH, 1).choice(wl.K, size=n_out, replace=False)
    x[:, ch] *= 20.0
    return x.astype(np.float16)


def rotations_identity(wl: Workload):
    """Per partition: seeded pairs as in ``rotations`` with every angle 0 (cos 1, sin 0: no
    rotation) and channel scales as in ``rotations``."""
    pairs_l, theta_l, cs_l = rotations(wl)
    return pairs_l, [np.zeros_like(t) for t in theta_l], cs_l


def residual(wl: Workload, M: Optional[int] = None) -> np.ndarray:
    """The residual stream beside ``activations``: f16 [M, K] ~ N(0, 2^2)."""
    M = wl.M if M is None else M
    return (rng(wl.wid, T_RES).standard_normal((M, wl.K)) * 2.0).astype(np.float16)


def norm_weight(wl: Workload) -> np.ndarray:
    """RMSNorm weights f16 [K] ~ N(0, 0.1^2) (the Gemma form scales by 1 + w)."""
    return (rng(wl.wid, T_NORMW).standard_normal(wl.K) * 0.1).astype(np.float16)


def rotations(wl: Workload):
    """Per partition: pairs int16 [8, K] (each 128-slice of a layer a seeded permutation of
    0..127), theta f16 [8, K/2] ~ U(-pi, pi), channel_scales f16 [K] ~ lognormal(0, 0.3).
    Returns three lists of length P."""
    pairs_l, theta_l, cs_l = [], [], []
    for p in range(wl.P):
        r = rng(wl.wid, T_PAIRS, p)
        pairs = np.empty((LAYERS, wl.K), dtype=np.int16)
        for layer in range(LAYERS):
            for g in range(wl.G):
                pairs[layer, g * GROUP:(g + 1) * GROUP] = r.permutation(GROUP)
        theta = rng(wl.wid, T_THETA, p).uniform(-np.pi, np.pi, (LAYERS, wl.K // 2)).astype(np.float16)
        cs = np.exp(rng(wl.wid, T_CS, p).normal(0.0, 0.3, wl.K)).astype(np.float16)
        pairs_l.append(pairs)
        theta_l.append(theta)
        cs_l.append(cs)
    return pairs_l, theta_l, cs_l


@dataclass
class Weights:
    codes: np.ndarray     # uint8 [K, N] 0..15
    zp: np.ndarray        # uint8 [G, N] 2..14
    scales: np.ndarray    # f16 [G, N] ~ U(0.002, 0.02)
    qweight: np.ndarray   # int32 [K, N/8]
    qzeros: np.ndarray    # int32 [G, N/8]


def weights(wl: Workload) -> Weights:
    codes = rng(wl.wid, T_CODES).integers(0, 16, (wl.K, wl.N), dtype=np.uint8)
    zp = rng(wl.wid, T_ZP).integers(2, 15, (wl.G, wl.N), dtype=np.uint8)
    scales = rng(wl.wid, T_SCALES).uniform(0.002, 0.02, (wl.G, wl.N)).astype(np.float16)
    return Weights(codes, zp, scales, awq_pack(codes), awq_pack(zp))


def bitplane_pack(bits: np.ndarray) -> np.ndarray:
    """uint8 bits [R, N] (0/1) -> int32 words [R, N/32]: bit j of word w holds column 32w + j
    (the int5 checkpoint's fifth-bit plane)."""
    bits = np.asarray(bits, dtype=np.uint32) & 1
    R, N = bits.shape
    assert N % 32 == 0
    w = np.zeros((R, N // 32), dtype=np.uint32)
    for j in range(32):
        w |= bits[:, j::32] << np.uint32(j)
    return w.view(np.int32)


@dataclass
class Weights5:
    codes: np.ndarray      # uint8 [K, N] 0..31
    zp: np.ndarray         # uint8 [G, N] 4..28
    scales: np.ndarray     # f16 [G, N] ~ U(0.001, 0.01)
    qweight: np.ndarray    # int32 [K, N/8]   low four bits, AWQ order
    qweight_hi: np.ndarray  # int32 [K, N/32] fifth bits
    qzeros: np.ndarray     # int32 [G, N/8]
    qzeros_hi: np.ndarray  # int32 [G, N/32]


def weights5(wl: Workload) -> Weights5:
    """int5 bit-plane weights: codes ~ U{0..31}, zero points ~ U{4..28}, scales ~ U(0.001, 0.01)
    (half the int4 range, so the dequantised weights span about the same values); the low four
    bits packed as the int4 checkpoint, the fifth bits as [R, N/32] planes."""
    codes = rng(wl.wid, T_CODES, 5).integers(0, 32, (wl.K, wl.N), dtype=np.uint8)
    zp = rng(wl.wid, T_ZP, 5).integers(4, 29, (wl.G, wl.N), dtype=np.uint8)
    scales = rng(wl.wid, T_SCALES, 5).uniform(0.001, 0.01, (wl.G, wl.N)).astype(np.float16)
    return Weights5(codes, zp, scales, awq_pack(codes & 15), bitplane_pack(codes >> 4),
                    awq_pack(zp & 15), bitplane_pack(zp >> 4))


def subnormal_heavy_codes(wl: Workload, M: Optional[int] = None):
    """GEMM-only activations with many e4m3 subnormal codes: random codes (finite, not NaN)
    with, in 10% of the (row, group) blocks, half of the codes drawn from 0x01-0x07 /
    0x81-0x87; per-(row, group) scales ~ U(1e-3, 1e-1). Returns (A u8 [P, M, K],
    ASG f32 [P, M, G]); row-sums are left to the caller."""
    M = wl.M if M is None else M
    r = rng(wl.wid, T_SUBN)
    P, K, G = wl.P, wl.K, wl.G
    A = r.integers(0, 0x7F, (P, M, K), dtype=np.uint8)             # 0x00..0x7E magnitudes
    A |= (r.integers(0, 2, (P, M, K), dtype=np.uint8) << 7)          # random sign
    blocks = r.random((P, M, G)) < 0.10
    sub = r.integers(1, 8, (P, M, K), dtype=np.uint8) | (r.integers(0, 2, (P, M, K), dtype=np.uint8) << 7)
    half = r.random((P, M, K)) < 0.5
    sel = np.repeat(blocks, GROUP, axis=2) & half
    A = np.where(sel, sub, A).astype(np.uint8)
    ASG = r.uniform(1e-3, 1e-1, (P, M, G)).astype(np.float32)
    return A, ASG
