"""GPU parity of the int5 bit-plane weight GEMM (pq_pack_weights5 + pq_gemm5) against
oracle/int5.py.

Gates (tests/parity.py): Frobenius 2e-3 overall and per partition and the element-wise bound
against the fp64 reference on the same activation codes, rows past M never written
(sentinel-checked), at the decode shapes (M = 1, 8), the merged-QKV shape (three partitions), the
gate_up prefill shape (all 2048 rows), one-signed activations and ragged shapes. The packed SZ
words are checked against their definition.
"""
import numpy as np
import pytest
import torch

import rotated_w4a8_group_amd as pq
import synth
from oracle import gemm as ogemm
from oracle import int5 as oint5
from oracle import prologue as opro

import parity
from gpu_util import SENT_BF16, bf16_to_f64, prologue_gpu, to_dev

pytestmark = pytest.mark.gpu

EXTRA_ROWS = 3


def _pack5(w):
    return pq.pack_weights5(to_dev(w.qweight), to_dev(w.qweight_hi), to_dev(w.qzeros), to_dev(w.qzeros_hi),
                            to_dev(w.scales))


def _run(A, S, R, wpk, sz, N, pb1, pb2):
    P, M, K = A.shape
    ybuf = torch.empty((M + EXTRA_ROWS, N), dtype=torch.bfloat16, device="cuda")
    ybuf.view(torch.int16).fill_(SENT_BF16)
    pq.gemm5(A, S, R, wpk, sz, N, pb1, pb2, out=ybuf[:M])
    torch.cuda.synchronize()
    assert torch.all(ybuf[M:].view(torch.int16) == SENT_BF16), "rows past M were written"
    return ybuf[:M]


def _check(name, y, A, S, w, wl):
    y_ref = oint5.gemm_ref5(A, S, w.qweight, w.qweight_hi, w.qzeros, w.qzeros_hi, w.scales, *wl.bounds)
    mags = parity.magnitudes_int5(A, S, w, *wl.bounds)
    parity.check(f"gemm5 {name}", y, y_ref, mags, wl.bounds, wl.G)


@pytest.mark.parametrize("name", ["tiny", "decode_m1", "decode_m8", "qkv", "prefill"])
def test_gemm5_parity(name):
    wl = synth.WORKLOADS[name]
    print(f"[gemm5 {name}] M={wl.M} K={wl.K} N={wl.N} P={wl.P}", flush=True)
    x = synth.activations(wl)
    pl, tl, cl = synth.rotations(wl)
    A, S, R = opro.rotate_quant(x, pl, tl, cl)
    w = synth.weights5(wl)
    wpk, sz = _pack5(w)
    y = _run(to_dev(A), to_dev(S), to_dev(R), wpk, sz, wl.N, *wl.bounds)
    _check(name, bf16_to_f64(y), A, S, w, wl)


@pytest.mark.parametrize("M", [8, 300])
def test_gemm5_one_signed_activations(M):
    """Identity rotations on |N(0,1)| activations with outliers: one-signed codes (decode and
    prefill kernels)."""
    wl = synth.Workload("onesigned5", 175, M, 1024, 2048)
    x = synth.activations_one_signed(wl)
    pl, tl, cl = synth.rotations_identity(wl)
    A, S, R = opro.rotate_quant(x, pl, tl, cl)
    w = synth.weights5(wl)
    wpk, sz = _pack5(w)
    y = _run(to_dev(A), to_dev(S), to_dev(R), wpk, sz, wl.N, *wl.bounds)
    _check(f"one-signed M={M}", bf16_to_f64(y), A, S, w, wl)


@pytest.mark.parametrize("M,K,N,splits", [
    (17, 256, 160, ()), (130, 384, 288, (128, 160)), (1, 128, 32, ()), (16, 640, 96, ()),
    (33, 256, 384, (128, 128, 128)), (300, 1024, 2048, ()), (5, 384, 16 * 515 * 2, ()),
    # whole 256x256 tiles on the two-stage ring, with 9, 1 and 3 groups
    (512, 1152, 512, ()), (256, 128, 256, ()), (256, 384, 512, ()),
])
def test_gemm5_ragged_shapes(M, K, N, splits):
    wl = synth.Workload("ragged5", 160 + M, M, K, N, splits=splits)
    x = synth.activations(wl)
    pl, tl, cl = synth.rotations(wl)
    A, S, R = opro.rotate_quant(x, pl, tl, cl)
    w = synth.weights5(wl)
    wpk, sz = _pack5(w)
    y = _run(to_dev(A), to_dev(S), to_dev(R), wpk, sz, N, *wl.bounds)
    _check(f"ragged M={M} K={K} N={N}", bf16_to_f64(y), A, S, w, wl)


def test_packed_sz5_definition():
    """SZ = {sc, fl16(sc * (zp - 16))} for every (group, column), zp the full 5-bit zero point."""
    wl = synth.Workload("sz5", 170, 1, 512, 256)
    w = synth.weights5(wl)
    _, sz = _pack5(w)
    sz = sz.cpu().numpy()
    assert np.array_equal(sz[..., 0].view(np.uint16), w.scales.view(np.uint16))
    want = (w.scales.astype(np.float32) * (w.zp.astype(np.float32) - 16)).astype(np.float16)
    assert np.array_equal(sz[..., 1].view(np.uint16), want.view(np.uint16))
