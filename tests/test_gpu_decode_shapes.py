"""GPU checks of the decode kernel (M <= 16) at shapes whose column tiles do not divide evenly
over the workgroups (runs of different lengths), three partitions with uneven widths, one group per
tile, M = 16, and the down projection's shape (few tiles, long K).

Gates: the oracle's fp64 reference through tests/parity.py (Frobenius 2e-3 and the element-wise
bound, as every GEMM test); the same call repeated and replayed from a captured graph gives the
same bits.
"""
import numpy as np
import pytest
import torch

import rotated_w4a8_group_amd as pq
import synth
from oracle import gemm as ogemm
from oracle import prologue as opro

import parity
from gpu_util import bf16_to_f64, packed_weights, to_dev

pytestmark = pytest.mark.gpu

# (M, K, N, partition widths); N/16 tiles against 512 resident workgroups on 256 CUs
SHAPES = [
    (1, 256, 16 * 513, ()),                        # one workgroup with an extra tile
    (3, 384, 16 * 700, (3840, 2560, 4800)),        # three partitions, uneven runs in each
    (16, 128, 16 * 1100, ()),                      # one group per tile, M = 16
    (8, 1280, 16 * 515, ()),
    (1, 5120, 17408, ()),                          # gate_up decode: runs of 2 and 3 tiles
    (1, 17408, 5120, ()),                          # down decode: one tile per workgroup, long K
]


def _case(M, K, N, splits):
    wl = synth.Workload("decsplit", 120 + M + K // 128, M, K, N, splits=splits)
    x = synth.activations(wl)
    pl, tl, cl = synth.rotations(wl)
    A, S, R = opro.rotate_quant(x, pl, tl, cl)
    w = synth.weights(wl)
    return wl, A, S, R, w


@pytest.mark.parametrize("M,K,N,splits", SHAPES)
def test_decode_shape_parity_and_determinism(M, K, N, splits):
    print(f"[decode shape] M={M} K={K} N={N} splits={splits}", flush=True)
    wl, A, S, R, w = _case(M, K, N, splits)
    wpk, sz = packed_weights(w)
    Ad, Sd, Rd = to_dev(A), to_dev(S), to_dev(R)
    y1 = pq.gemm(Ad, Sd, Rd, wpk, sz, N, *wl.bounds)
    y2 = pq.gemm(Ad, Sd, Rd, wpk, sz, N, *wl.bounds)
    torch.cuda.synchronize()
    assert torch.equal(y1.view(torch.int16), y2.view(torch.int16))
    y_ref = ogemm.gemm_ref(A, S, w.qweight, w.qzeros, w.scales, *wl.bounds)
    mags = parity.magnitudes_int4(A, S, w, *wl.bounds)
    parity.check(f"decode shape M={M} K={K} N={N}", bf16_to_f64(y1), y_ref, mags, wl.bounds, wl.G)


def test_decode_graph_replay():
    """A captured decode launch replays to the eager result."""
    M, K, N, splits = SHAPES[3]
    wl, A, S, R, w = _case(M, K, N, splits)
    wpk, sz = packed_weights(w)
    Ad, Sd, Rd = to_dev(A), to_dev(S), to_dev(R)
    y_eager = pq.gemm(Ad, Sd, Rd, wpk, sz, N, *wl.bounds).clone()
    out = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        pq.gemm(Ad, Sd, Rd, wpk, sz, N, *wl.bounds, out=out)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        pq.gemm(Ad, Sd, Rd, wpk, sz, N, *wl.bounds, out=out)
    for r in range(3):
        out.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), y_eager.view(torch.int16)), f"replay {r}"
        # eager work between replays
        pq.gemm(Ad, Sd, Rd, wpk, sz, N, *wl.bounds)
        torch.cuda.synchronize()
