"""GPU parity of the per-token activation-scale path against oracle/tokquant.py.

Prologue: codes, token scales and row-sums bitwise equal to the oracle (scales and row-sums as
uint32 bit patterns), guard regions past the outputs untouched, on every workload (sampled rows
for the 8192-row ones), plus ragged, zero, saturating, strided and 4-byte-aligned inputs. GEMM:
the gates of tests/parity.py (Frobenius 2e-3 overall and per partition, element-wise bound)
against the fp64 reference, all rows up to 2048, one-signed activations, rows past M never
written.
"""
import numpy as np
import pytest
import torch

import rotated_w4a8_group_amd as pq
import synth
from oracle import gemm as ogemm
from oracle import tokquant as otok

import parity
from gpu_util import SENT_BF16, SENT_F32, SENT_U8, bf16_to_f64, guarded, packed_weights, records_for, to_dev

pytestmark = pytest.mark.gpu

EXTRA_ROWS = 3
SAMPLE_ROWS = 192


def _prologue_tok(wl, x, pl, tl, cl):
    rec = to_dev(records_for(pl, tl))
    cs = to_dev(np.stack(cl))
    P, M, K, G = wl.P, x.shape[0], wl.K, wl.K // 128
    A, Ab, nA = guarded((P, M, K), torch.uint8, SENT_U8)
    S, Sb, nS = guarded((P, M), torch.float32, None)
    R, Rb, nR = guarded((P, M, G), torch.float32, None)
    pq.rotate_quant_tok(to_dev(x), rec, cs, out=(A, S, R))
    torch.cuda.synchronize()
    sent = int(SENT_F32.view(np.int32))
    assert torch.all(Ab[nA:] == SENT_U8)
    assert torch.all(Sb[nS:].view(torch.int32) == sent) and torch.all(Rb[nR:].view(torch.int32) == sent)
    return A, S, R


def _compare(name, A, S, R, x, pl, tl, cl, rows):
    A_ref, S_ref, R_ref = otok.rotate_quant_tok(x[rows], pl, tl, cl)
    A_g, S_g, R_g = A[:, rows].cpu().numpy(), S[:, rows].cpu().numpy(), R[:, rows].cpu().numpy()
    bad = (np.count_nonzero(A_g != A_ref), np.count_nonzero(S_g.view(np.uint32) != S_ref.view(np.uint32)),
           np.count_nonzero(R_g.view(np.uint32) != R_ref.view(np.uint32)))
    print(f"[tok prologue {name}] rows={len(rows)} mismatches codes/as/rs={bad}", flush=True)
    assert bad == (0, 0, 0)


@pytest.mark.parametrize("name", ["tiny", "decode_m1", "decode_m8", "qkv", "prefill", "full_gate_up", "full_down"])
def test_prologue_tok_bit_exact(name):
    wl = synth.WORKLOADS[name]
    print(f"[tok prologue {name}] M={wl.M} K={wl.K} P={wl.P}", flush=True)
    x = synth.activations(wl)
    pl, tl, cl = synth.rotations(wl)
    A, S, R = _prologue_tok(wl, x, pl, tl, cl)
    if wl.M <= 2048:
        rows = np.arange(wl.M)
    else:
        r = np.random.default_rng(19)
        rows = np.sort(np.concatenate([[0, wl.M - 1], r.choice(np.arange(1, wl.M - 1), SAMPLE_ROWS - 2, replace=False)]))
    _compare(name, A, S, R, x, pl, tl, cl, rows)


def test_prologue_tok_edge_cases():
    """Ragged token count (37, not a multiple of the 4-token quad), zero rows, one zero group,
    saturating magnitudes, f16 subnormals, three partitions; a strided x and 4-byte-aligned rows
    must give the same bytes."""
    wl = synth.Workload("tokedge", 80, 37, 640, 128, splits=(64, 32, 32))
    x = synth.activations(wl)
    x[3] = 0
    x[36] = 0
    x[5, :128] = 0
    x[7] = np.float16(6.0e4)
    x[8, ::2] = np.float16(-6.0e-8)
    x[9] = np.float16(2.0 ** -24)
    pl, tl, cl = synth.rotations(wl)
    A, S, R = _prologue_tok(wl, x, pl, tl, cl)
    _compare("edge", A, S, R, x, pl, tl, cl, np.arange(wl.M))
    rec, cs = to_dev(records_for(pl, tl)), to_dev(np.stack(cl))
    for pad, start in ((64, 0), (2, 0), (6, 2)):
        wide = np.zeros((wl.M, wl.K + pad), dtype=np.float16)
        wide[:, start:start + wl.K] = x
        A2, S2, R2 = pq.rotate_quant_tok(to_dev(wide)[:, start:start + wl.K], rec, cs)
        assert torch.equal(A2, A) and torch.equal(S2.view(torch.int32), S.view(torch.int32))
        assert torch.equal(R2.view(torch.int32), R.view(torch.int32))
    # one token, one group
    wl1 = synth.Workload("tok1", 81, 1, 128, 16)
    x1 = synth.activations(wl1)
    pl1, tl1, cl1 = synth.rotations(wl1)
    A1, S1, R1 = _prologue_tok(wl1, x1, pl1, tl1, cl1)
    _compare("one", A1, S1, R1, x1, pl1, tl1, cl1, np.arange(1))


def test_prologue_tok_longest_row():
    """K = 18432, the longest row the per-token kernel takes: 144 groups, exactly 9 parked in
    every one of the 16 waves (no wave has a group slot left over), ragged token count, two
    partitions; bit-exact on every row."""
    wl = synth.Workload("tokmax", 83, 6, 18432, 128, splits=(64, 64))
    print(f"[tok prologue longest row] M={wl.M} K={wl.K} P={wl.P}", flush=True)
    x = synth.activations(wl)
    pl, tl, cl = synth.rotations(wl)
    A, S, R = _prologue_tok(wl, x, pl, tl, cl)
    _compare("longest row", A, S, R, x, pl, tl, cl, np.arange(wl.M))


def test_prologue_tok_rejects_long_rows():
    x = torch.zeros((4, 18560), dtype=torch.float16, device="cuda")
    rec = torch.zeros((1, 8, 18560 // 2, 8), dtype=torch.uint8, device="cuda")
    cs = torch.zeros((1, 18560), dtype=torch.float16, device="cuda")
    with pytest.raises(pq.PQError) as e:
        pq.rotate_quant_tok(x, rec, cs)
    assert e.value.code == -2


def _run_gemm_tok(A, S, R, wpk, sz, N, pb1, pb2):
    P, M, K = A.shape
    ybuf = torch.empty((M + EXTRA_ROWS, N), dtype=torch.bfloat16, device="cuda")
    ybuf.view(torch.int16).fill_(SENT_BF16)
    pq.gemm_tok(A, S, R, wpk, sz, N, pb1, pb2, out=ybuf[:M])
    torch.cuda.synchronize()
    assert torch.all(ybuf[M:].view(torch.int16) == SENT_BF16), "rows past M were written"
    return ybuf[:M]


def _check(name, y, A, S, w, wl):
    y_ref = otok.gemm_ref_tok(A, S, w.qweight, w.qzeros, w.scales, *wl.bounds)
    mags = parity.magnitudes_int4(A, S, w, *wl.bounds, tok=True)
    parity.check(f"tok gemm {name}", y, y_ref, mags, wl.bounds, wl.G)


@pytest.mark.parametrize("name", ["tiny", "decode_m1", "decode_m8", "qkv", "prefill"])
def test_gemm_tok_parity(name):
    wl = synth.WORKLOADS[name]
    print(f"[tok gemm {name}] M={wl.M} K={wl.K} N={wl.N} P={wl.P}", flush=True)
    x = synth.activations(wl)
    pl, tl, cl = synth.rotations(wl)
    A, S, R = otok.rotate_quant_tok(x, pl, tl, cl)
    w = synth.weights(wl)
    wpk, sz = packed_weights(w)
    y = _run_gemm_tok(to_dev(A), to_dev(S), to_dev(R), wpk, sz, wl.N, *wl.bounds)
    _check(name, bf16_to_f64(y), A, S, w, wl)


@pytest.mark.parametrize("M", [8, 300])
def test_gemm_tok_one_signed_activations(M):
    """Identity rotations on |N(0,1)| activations with outliers: one-signed codes."""
    wl = synth.Workload("onesignedtok", 105, M, 1024, 2048)
    x = synth.activations_one_signed(wl)
    pl, tl, cl = synth.rotations_identity(wl)
    A, S, R = otok.rotate_quant_tok(x, pl, tl, cl)
    assert np.all(A < 0x80)
    w = synth.weights(wl)
    wpk, sz = packed_weights(w)
    y = _run_gemm_tok(to_dev(A), to_dev(S), to_dev(R), wpk, sz, wl.N, *wl.bounds)
    _check(f"one-signed M={M}", bf16_to_f64(y), A, S, w, wl)


@pytest.mark.parametrize("name", ["full_gate_up", "full_down"])
def test_tok_end_to_end_full_shapes(name):
    wl = synth.WORKLOADS[name]
    print(f"[tok e2e {name}] M={wl.M} K={wl.K} N={wl.N}", flush=True)
    x = synth.activations(wl)
    pl, tl, cl = synth.rotations(wl)
    A, S, R = pq.rotate_quant_tok(to_dev(x), to_dev(records_for(pl, tl)), to_dev(np.stack(cl)))
    w = synth.weights(wl)
    wpk, sz = packed_weights(w)
    y = _run_gemm_tok(A, S, R, wpk, sz, wl.N, *wl.bounds)
    rows = np.sort(np.concatenate([[0, wl.M - 1], np.random.default_rng(9).choice(np.arange(1, wl.M - 1), 62, replace=False)]))
    Ar, Sr, _ = otok.rotate_quant_tok(x[rows], pl, tl, cl)
    _check(name, bf16_to_f64(y)[rows], Ar, Sr, w, wl)


@pytest.mark.parametrize("M,K,N,splits", [
    (17, 256, 144, ()), (130, 384, 272, (128, 144)), (1, 128, 16, ()), (33, 256, 384, (128, 128, 128)),
    (300, 1024, 2048, ()), (512, 1152, 512, ()),
])
def test_gemm_tok_ragged_shapes(M, K, N, splits):
    wl = synth.Workload("tokragged", 90 + M, M, K, N, splits=splits)
    x = synth.activations(wl)
    pl, tl, cl = synth.rotations(wl)
    A, S, R = otok.rotate_quant_tok(x, pl, tl, cl)
    w = synth.weights(wl)
    wpk, sz = packed_weights(w)
    y = _run_gemm_tok(to_dev(A), to_dev(S), to_dev(R), wpk, sz, N, *wl.bounds)
    _check(f"ragged M={M} K={K} N={N}", bf16_to_f64(y), A, S, w, wl)
