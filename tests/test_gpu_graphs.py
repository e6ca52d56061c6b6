"""HIP-graph capture of every prefill path.

A captured step (prologue + GEMM, or the fused producer + GEMM) must replay to the eager result
bit for bit. Each case replays three times, zeroing the outputs before each replay and running
the same entry points eagerly between replays. Shape M=300, K=1024, N=2048 covers whole 256x256
tiles, last-round pieces and the zero-point pre-pass with its workspace.
"""
import numpy as np
import pytest
import torch

import rotated_w4a8_group_amd as pq
import synth

from gpu_util import packed_weights, records_for, to_dev

pytestmark = pytest.mark.gpu

M, K, N = 300, 1024, 2048
G = K // 128


def _inputs(seed):
    wl = synth.Workload("graph", seed, M, K, N)
    pl, tl, cl = synth.rotations(wl)
    return wl, to_dev(synth.activations(wl)), to_dev(records_for(pl, tl)), to_dev(np.stack(cl))


def _replays(name, step, outs):
    step()
    torch.cuda.synchronize()
    ref = [o.clone() for o in outs]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for r in range(3):
        for o in outs:
            o.zero_()
        g.replay()
        torch.cuda.synchronize()
        for i, (o, e) in enumerate(zip(outs, ref)):
            assert torch.equal(o.view(torch.uint8), e.view(torch.uint8)), f"{name}: replay {r}, output {i}"
        step()
        torch.cuda.synchronize()
    print(f"[graph {name}] 3 replays bit-equal to the eager step", flush=True)


def _bufs():
    A = torch.empty((1, M, K), dtype=torch.uint8, device="cuda")
    S = torch.empty((1, M, G), dtype=torch.float32, device="cuda")
    R = torch.empty((1, M, G), dtype=torch.float32, device="cuda")
    y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(max(1, pq.gemm_workspace_bytes(M, N, K)), dtype=torch.uint8, device="cuda")
    return A, S, R, y, ws


def test_graph_per_group():
    wl, x, rec, cs = _inputs(401)
    wpk, sz = packed_weights(synth.weights(wl))
    A, S, R, y, ws = _bufs()

    def step():
        pq.rotate_quant(x, rec, cs, out=(A, S, R))
        pq.gemm(A, S, R, wpk, sz, N, out=y, workspace=ws)
    _replays("per-group", step, [A, S, R, y])


def test_graph_shared_workspace_pair():
    """The prologue writes the GEMM's operands into the workspace, the GEMM reads them there."""
    wl, x, rec, cs = _inputs(406)
    wpk, sz = packed_weights(synth.weights(wl))
    A, S, R, y, ws = _bufs()

    def step():
        pq.rotate_quant_for_gemm(x, rec, cs, ws, out=(A, S, R))
        pq.gemm_prepared(A, S, R, wpk, sz, N, out=y, workspace=ws)
    _replays("shared workspace", step, [A, S, R, y])


def test_graph_per_token():
    wl, x, rec, cs = _inputs(402)
    wpk, sz = packed_weights(synth.weights(wl))
    A, _, R, y, _ = _bufs()
    AS = torch.empty((1, M), dtype=torch.float32, device="cuda")
    ws = torch.empty(max(1, pq.gemm_tok_workspace_bytes(M, N, K)), dtype=torch.uint8, device="cuda")

    def step():
        pq.rotate_quant_tok(x, rec, cs, out=(A, AS, R))
        pq.gemm_tok(A, AS, R, wpk, sz, N, out=y, workspace=ws)
    _replays("per-token", step, [A, AS, R, y])


def test_graph_int8():
    wl, x, rec, cs = _inputs(403)
    wpk, sz = packed_weights(synth.weights(wl))
    A, S, R, y, ws = _bufs()
    A8 = A.view(torch.int8)

    def step():
        pq.rotate_quant_i8(x, rec, cs, out=(A8, S, R))
        pq.gemm_i8(A8, S, R, wpk, sz, N, out=y, workspace=ws)
    _replays("int8", step, [A, S, R, y])


def test_graph_int5():
    wl, x, rec, cs = _inputs(404)
    w = synth.weights5(wl)
    wpk, sz = pq.pack_weights5(to_dev(w.qweight), to_dev(w.qweight_hi), to_dev(w.qzeros), to_dev(w.qzeros_hi),
                               to_dev(w.scales))
    A, S, R, y, ws = _bufs()

    def step():
        pq.rotate_quant(x, rec, cs, out=(A, S, R))
        pq.gemm5(A, S, R, wpk, sz, N, out=y, workspace=ws)
    _replays("int5", step, [A, S, R, y])


def test_graph_fused_producer():
    wl, x, rec, cs = _inputs(405)
    wpk, sz = packed_weights(synth.weights(wl))
    res = to_dev(synth.residual(wl))
    nw = to_dev(synth.norm_weight(wl))
    A, S, R, y, ws = _bufs()
    ro = torch.empty((M, K), dtype=torch.float16, device="cuda")
    hs = torch.empty((M, K), dtype=torch.float16, device="cuda")

    def step():
        pq.add_rms_rotate_quant(x, res, nw, 1e-6, rec, cs, residual_out=ro, out=(hs, A, S, R))
        pq.gemm(A, S, R, wpk, sz, N, out=y, workspace=ws)
    _replays("fused producer", step, [ro, hs, A, S, R, y])
