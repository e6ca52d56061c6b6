"""GPU parity of the W4A8 group GEMM against the oracle's same-codes fp64 reference.

Gates (tests/parity.py): ||y - y_ref||_F / ||y_ref||_F <= 2e-3 overall and per partition, every
element within the derived bound, rows past M never written (sentinel-checked), at every
workload's full shape. Workloads up to 2048 rows compare all rows on oracle-made activation codes;
the 8192-row workloads run prologue + GEMM on the GPU and compare 64 sampled rows end to end.
One-signed activations (identity rotation, |N(0,1)| with outliers) stress the code-domain
zero-point correction at decode and prefill sizes.
"""
import numpy as np
import pytest
import torch

import rotated_w4a8_group_amd as pq
import synth
from oracle import e4m3 as oe4m3
from oracle import gemm as ogemm
from oracle import prologue as opro

import parity
from gpu_util import SENT_BF16, bf16_to_f64, packed_weights, prologue_gpu, to_dev

pytestmark = pytest.mark.gpu

EXTRA_ROWS = 3


def _run_gemm(A, S, R, wpk, sz, N, pb1, pb2):
    P, M, K = A.shape
    ybuf = torch.empty((M + EXTRA_ROWS, N), dtype=torch.bfloat16, device="cuda")
    ybuf.view(torch.int16).fill_(SENT_BF16)
    pq.gemm(A, S, R, wpk, sz, N, pb1, pb2, out=ybuf[:M])
    torch.cuda.synchronize()
    assert torch.all(ybuf[M:].view(torch.int16) == SENT_BF16), "rows past M were written"
    return ybuf[:M]


def _check(name, y, A, S, w, wl, rows=None):
    """Reference and magnitudes for the rows of A/S (all, or `rows`), then every gate."""
    y_ref = ogemm.gemm_ref(A, S, w.qweight, w.qzeros, w.scales, *wl.bounds, rows=rows)
    mags = parity.magnitudes_int4(A, S, w, *wl.bounds, rows=rows)
    parity.check(f"gemm {name}", y, y_ref, mags, wl.bounds, wl.G)


@pytest.mark.parametrize("name", ["tiny", "decode_m1", "decode_m8", "qkv", "prefill"])
def test_gemm_parity(name):
    """All rows, every column (2048 x 17408 at the gate_up prefill workload)."""
    wl = synth.WORKLOADS[name]
    print(f"[gemm {name}] M={wl.M} K={wl.K} N={wl.N} P={wl.P}", flush=True)
    x = synth.activations(wl)
    pl, tl, cl = synth.rotations(wl)
    A, S, R = opro.rotate_quant(x, pl, tl, cl)
    w = synth.weights(wl)
    wpk, sz = packed_weights(w)
    y = _run_gemm(to_dev(A), to_dev(S), to_dev(R), wpk, sz, wl.N, *wl.bounds)
    _check(name, bf16_to_f64(y), A, S, w, wl)


@pytest.mark.parametrize("M", [1, 8, 2048])
def test_gemm_one_signed_activations(M):
    """Identity rotations on |N(0,1)| activations with 1% outlier channels x20: every code is
    non-negative, so the zero-point term (8 sc + zsc) * rs is as large as the raw-code products it
    cancels against (decode kernel's in-loop form at M <= 16, the prefill kernel's bf16-split
    epilogue above)."""
    wl = synth.Workload("onesigned", 95, M, 5120, 17408)
    print(f"[gemm one-signed] M={M} K={wl.K} N={wl.N}", flush=True)
    x = synth.activations_one_signed(wl)
    pl, tl, cl = synth.rotations_identity(wl)
    A, S, R = opro.rotate_quant(x, pl, tl, cl)
    assert np.all(A < 0x80)
    w = synth.weights(wl)
    wpk, sz = packed_weights(w)
    y = _run_gemm(to_dev(A), to_dev(S), to_dev(R), wpk, sz, wl.N, *wl.bounds)
    _check(f"one-signed M={M}", bf16_to_f64(y), A, S, w, wl)


@pytest.mark.parametrize("name", ["full_gate_up", "full_down"])
def test_end_to_end_full_shapes(name):
    """Prologue + GEMM on the GPU at 8192 rows; sampled rows recomputed by the oracle from x."""
    wl = synth.WORKLOADS[name]
    print(f"[e2e {name}] M={wl.M} K={wl.K} N={wl.N}", flush=True)
    x = synth.activations(wl)
    pl, tl, cl = synth.rotations(wl)
    A, S, R = prologue_gpu(wl, x, pl, tl, cl, guard=False)
    w = synth.weights(wl)
    wpk, sz = packed_weights(w)
    y = _run_gemm(A, S, R, wpk, sz, wl.N, *wl.bounds)
    rows = np.sort(np.concatenate([[0, wl.M - 1], np.random.default_rng(6).choice(np.arange(1, wl.M - 1), 62, replace=False)]))
    Ar, Sr, _ = opro.rotate_quant(x[rows], pl, tl, cl)
    _check(name, bf16_to_f64(y)[rows], Ar, Sr, w, wl)


@pytest.mark.parametrize("M,K,N,splits", [
    (17, 256, 144, ()), (130, 384, 272, (128, 144)), (1, 128, 16, ()), (16, 640, 96, ()),
    (33, 256, 384, (128, 128, 128)), (300, 1024, 2048, ()),
    # whole 256x256 tiles only, with 9, 1 and 3 groups (odd and short group counts)
    (512, 1152, 512, ()), (256, 128, 256, ()), (256, 384, 512, ()),
    # row tiles in two whole bands of 4 and a last band of 1 (a whole round, then pieces), and in
    # one whole band and a last band of 2 with three partitions (pieces only)
    (2300, 256, 8192, ()), (1300, 512, 4096, (1024, 1024, 2048)),
])
def test_gemm_ragged_shapes(M, K, N, splits):
    wl = synth.Workload("ragged", 50 + M, M, K, N, splits=splits)
    x = synth.activations(wl)
    pl, tl, cl = synth.rotations(wl)
    A, S, R = opro.rotate_quant(x, pl, tl, cl)
    w = synth.weights(wl)
    wpk, sz = packed_weights(w)
    y = _run_gemm(to_dev(A), to_dev(S), to_dev(R), wpk, sz, N, *wl.bounds)
    _check(f"ragged M={M} K={K} N={N}", bf16_to_f64(y), A, S, w, wl)


@pytest.mark.parametrize("M", [4, 300])
def test_gemm_subnormal_heavy_codes(M):
    """10% of (row, group) blocks hold half e4m3 subnormal codes; row-sums from the oracle."""
    wl = synth.Workload("subn", 60, M, 1024, 512, splits=(256, 128, 128))
    A, S = synth.subnormal_heavy_codes(wl)
    R = oe4m3.decode(A.reshape(wl.P, M, wl.G, 128)).sum(-1).astype(np.float32)
    w = synth.weights(wl)
    wpk, sz = packed_weights(w)
    y = _run_gemm(to_dev(A), to_dev(S), to_dev(R), wpk, sz, wl.N, *wl.bounds)
    _check(f"subnormal M={M}", bf16_to_f64(y), A, S, w, wl)


@pytest.mark.parametrize("M", [4, 200])
def test_identical_partitions_equal_single(M):
    """G3: three partitions carrying the same activations give bitwise the P = 1 result."""
    wl = synth.Workload("g3", 70, M, 512, 768)
    x = synth.activations(wl)
    pl, tl, cl = synth.rotations(wl)
    A, S, R = opro.rotate_quant(x, pl, tl, cl)
    w = synth.weights(wl)
    wpk, sz = packed_weights(w)
    y1 = _run_gemm(to_dev(A), to_dev(S), to_dev(R), wpk, sz, 768, pq.NO_BOUNDARY, pq.NO_BOUNDARY)
    A3, S3, R3 = (np.concatenate([t] * 3) for t in (A, S, R))
    y3 = _run_gemm(to_dev(A3), to_dev(S3), to_dev(R3), wpk, sz, 768, 256, 512)
    assert torch.equal(y1.view(torch.int16), y3.view(torch.int16))


def test_zero_activations_give_zero():
    wl = synth.Workload("zero", 71, 20, 256, 128)
    A = np.zeros((1, 20, 256), np.uint8)
    S = np.zeros((1, 20, 2), np.float32)
    w = synth.weights(wl)
    wpk, sz = packed_weights(w)
    y = _run_gemm(to_dev(A), to_dev(S), to_dev(S), wpk, sz, 128, pq.NO_BOUNDARY, pq.NO_BOUNDARY)
    assert torch.all(y.float() == 0)


def test_packed_sz_definition():
    """SZ = {sc, fl16(sc * (zp - 8))} for every (group, column)."""
    wl = synth.Workload("sz", 72, 1, 512, 256)
    w = synth.weights(wl)
    _, sz = packed_weights(w)
    sz = sz.cpu().numpy()
    assert np.array_equal(sz[..., 0].view(np.uint16), w.scales.view(np.uint16))
    want = (w.scales.astype(np.float32) * (w.zp.astype(np.float32) - 8)).astype(np.float16)
    assert np.array_equal(sz[..., 1].view(np.uint16), want.view(np.uint16))


def test_device_bf16_rounding_exhaustive():
    """The bf16 rounding of the GEMM outputs and zero-point operands (pq_bf16_round: pairs through
    the epilogues' packed convert, an odd last element through the single one) on all 2^32 fp32
    bit patterns: round to nearest even as torch's float32 -> bfloat16 conversion does it for every
    non-NaN input, and a NaN kept quiet with its sign and top payload bits ((u >> 16) | 0x40)."""
    chunk = 1 << 28
    bad = 0
    for c in range(1 << 4):
        lo = -(1 << 31) + c * chunk
        bits = torch.arange(lo, lo + chunk + (1 if c == 0 else 0), dtype=torch.int32, device="cuda")  # odd length once
        got = pq.bf16_round(bits.view(torch.float32)).to(torch.int32) & 0xFFFF
        want = bits.view(torch.float32).to(torch.bfloat16).view(torch.int16).to(torch.int32) & 0xFFFF
        nan = (bits & 0x7FFFFFFF) > 0x7F800000
        want = torch.where(nan, ((bits >> 16) & 0xFFFF) | 0x40, want)
        bad += int((got != want).sum())
        del bits, got, want, nan
    print(f"[bf16] mismatches over 2^32 inputs: {bad}", flush=True)
    assert bad == 0
