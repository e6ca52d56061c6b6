"""GPU parity of the fused residual add + RMSNorm + rotate + quant producer
(pq_add_rms_rotate_quant) against oracle/producer.py.

Gates (the page's: residual exact, normalised row within ppm of a CPU reference): the new
residual bit-exact; the normalised row within one f16 step of the oracle's everywhere, with at
most 1e-3 of its elements off by that step; the codes, group scales and row-sums bit-exact against
the pinned oracle prologue applied to the kernel's own normalised row; rows past M never written.
"""
import numpy as np
import pytest
import torch

import rotated_w4a8_group_amd as pq
import synth
from oracle import producer as oprod
from oracle import prologue as opro

from gpu_util import SENT_F32, SENT_U8, guarded, records_for, to_dev

pytestmark = pytest.mark.gpu

EPS = 1e-6
SENT16 = 0x7C01   # an f16 NaN pattern the kernel never writes


def _f16_steps(a, b):
    """Elementwise distance in f16 steps between two finite f16 arrays (same sign bit order)."""
    ia = a.view(np.int16).astype(np.int32)
    ib = b.view(np.int16).astype(np.int32)
    ia = np.where(ia < 0, -(ia & 0x7FFF), ia)
    ib = np.where(ib < 0, -(ib & 0x7FFF), ib)
    return np.abs(ia - ib)


def _run(wl, x, r, w, pl, tl, cl, gemma=True, inplace=False):
    P, M, K, G = wl.P, x.shape[0], wl.K, wl.K // 128
    rec = to_dev(records_for(pl, tl))
    cs = to_dev(np.stack(cl))
    xd, rd, wd = to_dev(x), to_dev(r), to_dev(w)
    A, Ab, nA = guarded((P, M, K), torch.uint8, SENT_U8)
    S, Sb, nS = guarded((P, M, G), torch.float32, None)
    R, Rb, nR = guarded((P, M, G), torch.float32, None)
    hbuf = torch.empty((M + 3, K), dtype=torch.float16, device="cuda")
    hbuf.view(torch.int16).fill_(SENT16)
    if inplace:
        ro = rd
    else:
        obuf = torch.empty((M + 3, K), dtype=torch.float16, device="cuda")
        obuf.view(torch.int16).fill_(SENT16)
        ro = obuf[:M]
    pq.add_rms_rotate_quant(xd, rd, wd, EPS, rec, cs, gemma=gemma, residual_out=ro, out=(hbuf[:M], A, S, R))
    torch.cuda.synchronize()
    sent = int(SENT_F32.view(np.int32))
    assert torch.all(Ab[nA:] == SENT_U8)
    assert torch.all(Sb[nS:].view(torch.int32) == sent) and torch.all(Rb[nR:].view(torch.int32) == sent)
    assert torch.all(hbuf[M:].view(torch.int16) == SENT16), "normalised rows past M were written"
    if not inplace:
        assert torch.all(obuf[M:].view(torch.int16) == SENT16), "residual rows past M were written"
    return ro.cpu().numpy(), hbuf[:M].cpu().numpy(), A.cpu().numpy(), S.cpu().numpy(), R.cpu().numpy()


def _check(name, wl, x, r, w, pl, tl, cl, out, gemma=True, rows=None):
    ro, hs, A, S, R = out
    if rows is None:
        rows = np.arange(x.shape[0])
    h_ref, hs_ref = oprod.add_rms(x[rows], r[rows], w, EPS, gemma)
    assert np.array_equal(ro[rows].view(np.uint16), h_ref.view(np.uint16)), "residual not exact"
    steps = _f16_steps(hs[rows], hs_ref)
    frac = np.count_nonzero(steps) / steps.size
    A_ref, S_ref, R_ref = opro.rotate_quant(hs[rows], pl, tl, cl)
    bad = (np.count_nonzero(A[:, rows] != A_ref), np.count_nonzero(S[:, rows].view(np.uint32) != S_ref.view(np.uint32)),
           np.count_nonzero(R[:, rows].view(np.uint32) != R_ref.view(np.uint32)))
    print(f"[producer {name}] rows={len(rows)} hs max steps={steps.max()} frac off={frac:.2e} "
          f"code/scale/rowsum mismatches={bad}", flush=True)
    assert steps.max() <= 1 and frac <= 1e-3
    assert bad == (0, 0, 0)


@pytest.mark.parametrize("name", ["tiny", "decode_m1", "decode_m8", "qkv", "prefill"])
def test_producer_parity(name):
    wl = synth.WORKLOADS[name]
    print(f"[producer {name}] M={wl.M} K={wl.K} P={wl.P}", flush=True)
    x, r, w = synth.activations(wl), synth.residual(wl), synth.norm_weight(wl)
    pl, tl, cl = synth.rotations(wl)
    out = _run(wl, x, r, w, pl, tl, cl)
    rows = None if wl.M <= 64 else np.sort(np.random.default_rng(31).choice(wl.M, 256, replace=False))
    _check(name, wl, x, r, w, pl, tl, cl, out, rows=rows)


@pytest.mark.parametrize("M,K,splits", [(37, 640, (64, 32, 32)), (8, 17408, ()), (1, 128, ()), (5, 2176, (64, 64)),
                                         (6, 18432, ()), (70, 18432, ())])
def test_producer_shapes(M, K, splits):
    wl = synth.Workload("prod", 190 + M, M, K, 128, splits=splits)
    x, r, w = synth.activations(wl), synth.residual(wl), synth.norm_weight(wl)
    pl, tl, cl = synth.rotations(wl)
    _check(f"M={M} K={K}", wl, x, r, w, pl, tl, cl, _run(wl, x, r, w, pl, tl, cl))


def test_producer_plain_inplace_and_cancelled_rows():
    wl = synth.Workload("prod2", 199, 9, 768, 128, splits=(64, 64))
    x, r, w = synth.activations(wl), synth.residual(wl), synth.norm_weight(wl)
    r[2] = (-x[2].astype(np.float32)).astype(np.float16)   # cancelled row: zero residual, zero codes
    pl, tl, cl = synth.rotations(wl)
    _check("plain", wl, x, r, w, pl, tl, cl, _run(wl, x, r, w, pl, tl, cl, gemma=False), gemma=False)
    out = _run(wl, x, r, w, pl, tl, cl, inplace=True)
    _check("in-place", wl, x, r, w, pl, tl, cl, out)
    assert not out[1][2].any() and not out[2][:, 2].any() and not out[3][:, 2].any()


@pytest.mark.parametrize("M,K", [(1, 5120), (8, 5120), (37, 5120), (8, 17408)])
def test_producer_inplace_residual(M, K):
    """res_out == res at the token counts that use several workgroups per token quad when the
    residual goes elsewhere (M <= 64): the in-place call must equal the oracle (and so the
    out-of-place call) bit for bit."""
    wl = synth.Workload("prodinplace", 210 + M + K // 128, M, K, 128)
    print(f"[producer in-place] M={M} K={K}", flush=True)
    x, r, w = synth.activations(wl), synth.residual(wl), synth.norm_weight(wl)
    pl, tl, cl = synth.rotations(wl)
    out_sep = _run(wl, x, r, w, pl, tl, cl)
    out_inp = _run(wl, x, r, w, pl, tl, cl, inplace=True)
    _check(f"in-place M={M} K={K}", wl, x, r, w, pl, tl, cl, out_inp)
    for a, b in zip(out_sep, out_inp):
        assert np.array_equal(a.view(np.uint8), b.view(np.uint8))


def test_producer_rejects_partial_residual_overlap():
    """res_out shifted by one row inside res: rejected before any launch, outputs untouched."""
    M, K = 8, 256
    res = torch.zeros((M + 1, K), dtype=torch.float16, device="cuda")
    x = torch.zeros((M, K), dtype=torch.float16, device="cuda")
    w = torch.zeros(K, dtype=torch.float16, device="cuda")
    rec = torch.zeros((1, 8, K // 2, 8), dtype=torch.uint8, device="cuda")
    cs = torch.zeros((1, K), dtype=torch.float16, device="cuda")
    with pytest.raises(pq.PQError) as e:
        pq.add_rms_rotate_quant(x, res[:M], w, EPS, rec, cs, residual_out=res[1:M + 1])
    assert e.value.code == -2
