"""GPU parity of the per-group int8 activation mode against oracle/int8.py.

Prologue: int8 codes, group scales and row-sums bitwise equal to the oracle, guards untouched, on
every workload (sampled rows at 8192) and on ragged / zero / saturating / strided inputs. GEMM:
the gates of tests/parity.py (Frobenius 2e-3 overall and per partition, element-wise bound), all
rows up to 2048, one-signed activations, rows past M never written.
"""
import numpy as np
import pytest
import torch

import rotated_w4a8_group_amd as pq
import synth
from oracle import gemm as ogemm
from oracle import int8 as oi8

import parity
from gpu_util import SENT_BF16, SENT_F32, SENT_U8, bf16_to_f64, guarded, packed_weights, records_for, to_dev

pytestmark = pytest.mark.gpu

EXTRA_ROWS = 3
SAMPLE_ROWS = 192


def _prologue_i8(wl, x, pl, tl, cl):
    rec = to_dev(records_for(pl, tl))
    cs = to_dev(np.stack(cl))
    P, M, K, G = wl.P, x.shape[0], wl.K, wl.K // 128
    A, Ab, nA = guarded((P, M, K), torch.uint8, SENT_U8)
    S, Sb, nS = guarded((P, M, G), torch.float32, None)
    R, Rb, nR = guarded((P, M, G), torch.float32, None)
    pq.rotate_quant_i8(to_dev(x), rec, cs, out=(A.view(torch.int8), S, R))
    torch.cuda.synchronize()
    sent = int(SENT_F32.view(np.int32))
    assert torch.all(Ab[nA:] == SENT_U8)
    assert torch.all(Sb[nS:].view(torch.int32) == sent) and torch.all(Rb[nR:].view(torch.int32) == sent)
    return A.view(torch.int8), S, R


def _compare(name, A, S, R, x, pl, tl, cl, rows):
    A_ref, S_ref, R_ref = oi8.rotate_quant_i8(x[rows], pl, tl, cl)
    A_g, S_g, R_g = A[:, rows].cpu().numpy(), S[:, rows].cpu().numpy(), R[:, rows].cpu().numpy()
    bad = (np.count_nonzero(A_g != A_ref), np.count_nonzero(S_g.view(np.uint32) != S_ref.view(np.uint32)),
           np.count_nonzero(R_g.view(np.uint32) != R_ref.view(np.uint32)))
    print(f"[i8 prologue {name}] rows={len(rows)} mismatches codes/asg/rs={bad}", flush=True)
    assert bad == (0, 0, 0)


@pytest.mark.parametrize("name", ["tiny", "decode_m1", "decode_m8", "qkv", "prefill", "full_gate_up", "full_down"])
def test_prologue_i8_bit_exact(name):
    wl = synth.WORKLOADS[name]
    print(f"[i8 prologue {name}] M={wl.M} K={wl.K} P={wl.P}", flush=True)
    x = synth.activations(wl)
    pl, tl, cl = synth.rotations(wl)
    A, S, R = _prologue_i8(wl, x, pl, tl, cl)
    if wl.M <= 2048:
        rows = np.arange(wl.M)
    else:
        r = np.random.default_rng(29)
        rows = np.sort(np.concatenate([[0, wl.M - 1], r.choice(np.arange(1, wl.M - 1), SAMPLE_ROWS - 2, replace=False)]))
    _compare(name, A, S, R, x, pl, tl, cl, rows)


def test_prologue_i8_edge_cases():
    wl = synth.Workload("i8edge", 82, 37, 384, 128, splits=(64, 32, 32))
    x = synth.activations(wl)
    x[3] = 0
    x[5, :128] = 0
    x[7] = np.float16(6.0e4)
    x[8, ::2] = np.float16(-6.0e-8)
    x[9] = np.float16(2.0 ** -24)
    pl, tl, cl = synth.rotations(wl)
    A, S, R = _prologue_i8(wl, x, pl, tl, cl)
    _compare("edge", A, S, R, x, pl, tl, cl, np.arange(wl.M))
    rec, cs = to_dev(records_for(pl, tl)), to_dev(np.stack(cl))
    for pad, start in ((64, 0), (2, 0), (6, 2)):
        wide = np.zeros((wl.M, wl.K + pad), dtype=np.float16)
        wide[:, start:start + wl.K] = x
        A2, S2, R2 = pq.rotate_quant_i8(to_dev(wide)[:, start:start + wl.K], rec, cs)
        assert torch.equal(A2, A) and torch.equal(S2.view(torch.int32), S.view(torch.int32))
        assert torch.equal(R2.view(torch.int32), R.view(torch.int32))


def _run_gemm_i8(A, S, R, wpk, sz, N, pb1, pb2):
    P, M, K = A.shape
    ybuf = torch.empty((M + EXTRA_ROWS, N), dtype=torch.bfloat16, device="cuda")
    ybuf.view(torch.int16).fill_(SENT_BF16)
    pq.gemm_i8(A, S, R, wpk, sz, N, pb1, pb2, out=ybuf[:M])
    torch.cuda.synchronize()
    assert torch.all(ybuf[M:].view(torch.int16) == SENT_BF16), "rows past M were written"
    return ybuf[:M]


def _check(name, y, A, S, w, wl):
    y_ref = oi8.gemm_ref_i8(A, S, w.qweight, w.qzeros, w.scales, *wl.bounds)
    mags = parity.magnitudes_int4(A, S, w, *wl.bounds, act="int8")
    parity.check(f"i8 gemm {name}", y, y_ref, mags, wl.bounds, wl.G)


@pytest.mark.parametrize("name", ["tiny", "decode_m1", "decode_m8", "qkv", "prefill"])
def test_gemm_i8_parity(name):
    wl = synth.WORKLOADS[name]
    print(f"[i8 gemm {name}] M={wl.M} K={wl.K} N={wl.N} P={wl.P}", flush=True)
    x = synth.activations(wl)
    pl, tl, cl = synth.rotations(wl)
    A, S, R = oi8.rotate_quant_i8(x, pl, tl, cl)
    w = synth.weights(wl)
    wpk, sz = packed_weights(w)
    y = _run_gemm_i8(to_dev(A), to_dev(S), to_dev(R), wpk, sz, wl.N, *wl.bounds)
    _check(name, bf16_to_f64(y), A, S, w, wl)


@pytest.mark.parametrize("M", [8, 300])
def test_gemm_i8_one_signed_activations(M):
    """Identity rotations on |N(0,1)| activations with outliers: one-signed int8 codes."""
    wl = synth.Workload("onesigned8", 115, M, 1024, 2048)
    x = synth.activations_one_signed(wl)
    pl, tl, cl = synth.rotations_identity(wl)
    A, S, R = oi8.rotate_quant_i8(x, pl, tl, cl)
    assert np.all(A >= 0)
    w = synth.weights(wl)
    wpk, sz = packed_weights(w)
    y = _run_gemm_i8(to_dev(A), to_dev(S), to_dev(R), wpk, sz, wl.N, *wl.bounds)
    _check(f"one-signed M={M}", bf16_to_f64(y), A, S, w, wl)


@pytest.mark.parametrize("name", ["full_gate_up", "full_down"])
def test_i8_end_to_end_full_shapes(name):
    wl = synth.WORKLOADS[name]
    print(f"[i8 e2e {name}] M={wl.M} K={wl.K} N={wl.N}", flush=True)
    x = synth.activations(wl)
    pl, tl, cl = synth.rotations(wl)
    A, S, R = pq.rotate_quant_i8(to_dev(x), to_dev(records_for(pl, tl)), to_dev(np.stack(cl)))
    w = synth.weights(wl)
    wpk, sz = packed_weights(w)
    y = _run_gemm_i8(A, S, R, wpk, sz, wl.N, *wl.bounds)
    rows = np.sort(np.concatenate([[0, wl.M - 1], np.random.default_rng(28).choice(np.arange(1, wl.M - 1), 62, replace=False)]))
    Ar, Sr, _ = oi8.rotate_quant_i8(x[rows], pl, tl, cl)
    _check(name, bf16_to_f64(y)[rows], Ar, Sr, w, wl)


@pytest.mark.parametrize("M,K,N,splits", [
    (17, 256, 144, ()), (130, 384, 272, (128, 144)), (1, 128, 16, ()), (33, 256, 384, (128, 128, 128)),
    (300, 1024, 2048, ()), (512, 1152, 512, ()),
])
def test_gemm_i8_ragged_shapes(M, K, N, splits):
    wl = synth.Workload("i8ragged", 110 + M, M, K, N, splits=splits)
    x = synth.activations(wl)
    pl, tl, cl = synth.rotations(wl)
    A, S, R = oi8.rotate_quant_i8(x, pl, tl, cl)
    w = synth.weights(wl)
    wpk, sz = packed_weights(w)
    y = _run_gemm_i8(to_dev(A), to_dev(S), to_dev(R), wpk, sz, N, *wl.bounds)
    _check(f"ragged M={M} K={K} N={N}", bf16_to_f64(y), A, S, w, wl)
