"""GPU tests of the prologue/GEMM pair that shares the GEMM's workspace
(pq_rotate_quant_for_gemm + pq_gemm_prepared).

The pair must give exactly the two-call path's results: the prologue's codes, group scales and
row-sums bit for bit equal to pq_rotate_quant's, and the GEMM output bit for bit equal to
pq_gemm's on the same codes (the prologue writes the prefill operands with the arithmetic of
pq_gemm's own pass). The workspace starts filled with 0xFF bytes (bf16 and f32 NaN patterns), so
an operand slot the prologue fails to write (a padding k' past 3G, a partition, a row) turns the
output into NaN. Each case also passes the oracle gates (tests/parity.py) on sampled rows, rows
past M stay untouched, and the decode band (M <= 16) runs without a workspace.
"""
import numpy as np
import pytest
import torch

import rotated_w4a8_group_amd as pq
import synth
from oracle import gemm as ogemm

import parity
from gpu_util import SENT_BF16, bf16_to_f64, packed_weights, records_for, to_dev

pytestmark = pytest.mark.gpu

EXTRA_ROWS = 3


def _pair_vs_two_calls(wl, sample_rows):
    M, K, N = wl.M, wl.K, wl.N
    print(f"[prepared {wl.name}] M={M} K={K} N={N} P={wl.P} bounds={wl.bounds}", flush=True)
    x = to_dev(synth.activations(wl))
    pl, tl, cl = synth.rotations(wl)
    rec, cs = to_dev(records_for(pl, tl)), to_dev(np.stack(cl))
    w = synth.weights(wl)
    wpk, sz = packed_weights(w)

    need = pq.gemm_workspace_bytes(M, N, K)
    ws = torch.full((max(need, 1),), 0xFF, dtype=torch.uint8, device="cuda") if need else None
    A1, S1, R1 = pq.rotate_quant_for_gemm(x, rec, cs, ws)
    y1buf = torch.empty((M + EXTRA_ROWS, N), dtype=torch.bfloat16, device="cuda")
    y1buf.view(torch.int16).fill_(SENT_BF16)
    pq.gemm_prepared(A1, S1, R1, wpk, sz, N, *wl.bounds, out=y1buf[:M], workspace=ws)

    A0, S0, R0 = pq.rotate_quant(x, rec, cs)
    y0 = pq.gemm(A0, S0, R0, wpk, sz, N, *wl.bounds)
    torch.cuda.synchronize()

    assert torch.equal(A1, A0), "codes differ from pq_rotate_quant"
    assert torch.equal(S1.view(torch.int32), S0.view(torch.int32)), "group scales differ"
    assert torch.equal(R1.view(torch.int32), R0.view(torch.int32)), "row-sums differ"
    assert torch.all(y1buf[M:].view(torch.int16) == SENT_BF16), "rows past M were written"
    y1 = y1buf[:M]
    assert not torch.isnan(y1.float()).any(), "NaN: an operand slot was left unwritten"
    diff = (y1.view(torch.int16) != y0.view(torch.int16)).sum().item()
    assert diff == 0, f"{diff} outputs differ from pq_gemm"

    rows = np.unique(np.linspace(0, M - 1, sample_rows).astype(np.int64))
    A, S = A1.cpu().numpy(), S1.cpu().numpy()
    y_ref = ogemm.gemm_ref(A, S, w.qweight, w.qzeros, w.scales, *wl.bounds, rows=rows)
    mags = parity.magnitudes_int4(A, S, w, *wl.bounds, rows=rows)
    parity.check(f"prepared {wl.name}", bf16_to_f64(y1[torch.from_numpy(rows).cuda()]), y_ref, mags,
                 wl.bounds, wl.G)


def test_prepared_headline_workload():
    """The gate_up prefill workload (M=2048, K=5120, N=17408): every output bit-equal."""
    _pair_vs_two_calls(synth.WORKLOADS["prefill"], 256)


@pytest.mark.parametrize("M,K,N,splits", [
    (37, 5120, 8192, (6144, 1024, 1024)),      # merged QKV, three partitions, ragged rows
    (300, 1024, 2048, (1024, 512, 512)),       # 256-column boundaries, P = 3
    (300, 1024, 1920, (768, 640, 512)),        # boundaries off the 256 line: 128x128 tiles
    (300, 17408, 1024, ()),                    # G = 136: 3G = 408, eight padding k'
    (33, 256, 384, ()),                        # G = 2: 26 padding k', two row tiles
    (17, 5120, 2048, (1024, 1024)),            # the smallest prefill M, P = 2
])
def test_prepared_shapes(M, K, N, splits):
    wl = synth.Workload("prepared", 300 + M % 97 + K % 89 + N % 83, M, K, N, splits=splits)
    _pair_vs_two_calls(wl, min(M, 64))


@pytest.mark.parametrize("M", [1, 8, 16])
def test_prepared_decode_band_needs_no_workspace(M):
    wl = synth.Workload("prepared_dec", 340 + M, M, 5120, 4096)
    _pair_vs_two_calls(wl, M)
