"""pq_gemm_noalloc (no workspace, the library's per-device scratch) against pq_gemm (caller
workspace) through the C ABI: the same kernels, so the outputs must be equal bit for bit, on calls
in a row whose sizes shrink (the scratch keeps the previous call's contents), at the prefill,
merged-QKV and decode sizes; one small case also goes through the oracle gates. Rows past M stay
untouched."""
import numpy as np
import pytest
import torch

import rotated_w4a8_group_amd as pq
import synth
from oracle import gemm as ogemm
from oracle import prologue as opro

import parity
from gpu_util import SENT_BF16, bf16_to_f64, packed_weights, to_dev

pytestmark = pytest.mark.gpu


def _inputs(wl):
    x = synth.activations(wl)
    pl, tl, cl = synth.rotations(wl)
    A, S, R = opro.rotate_quant(x, pl, tl, cl)
    w = synth.weights(wl)
    return A, S, R, w


def _both(A, S, R, wpk, sz, N, bounds):
    P, M, K = A.shape
    Ad, Sd, Rd = to_dev(A), to_dev(S), to_dev(R)
    y_ws = pq.gemm(Ad, Sd, Rd, wpk, sz, N, *bounds)
    ybuf = torch.empty((M + 3, N), dtype=torch.bfloat16, device="cuda")
    ybuf.view(torch.int16).fill_(SENT_BF16)
    pq.gemm_noalloc(Ad, Sd, Rd, wpk, sz, N, *bounds, out=ybuf[:M])
    torch.cuda.synchronize()
    assert torch.all(ybuf[M:].view(torch.int16) == SENT_BF16), "rows past M were written"
    return y_ws, ybuf[:M]


def test_noalloc_equals_workspace_path_on_shrinking_calls():
    """gate_up M=2048 (2.5 MB of scratch), then merged QKV M=256 with three partitions, then a
    ragged M=300 with fewer groups, then decode M=8 (no scratch): each equal to pq_gemm."""
    cases = [synth.Workload("na_big", 230, 2048, 5120, 17408),
             synth.Workload("na_qkv", 231, 256, 5120, 8192, splits=(6144, 1024, 1024)),
             synth.Workload("na_small", 232, 300, 1024, 2048),
             synth.Workload("na_dec", 233, 8, 1024, 2048)]
    for wl in cases:
        print(f"[noalloc] M={wl.M} K={wl.K} N={wl.N} P={wl.P}", flush=True)
        A, S, R, w = _inputs(wl)
        wpk, sz = packed_weights(w)
        y_ws, y_na = _both(A, S, R, wpk, sz, wl.N, wl.bounds)
        assert torch.equal(y_ws.view(torch.int16), y_na.view(torch.int16)), wl.name
        if wl.M <= 300 and wl.N <= 2048:
            y_ref = ogemm.gemm_ref(A, S, w.qweight, w.qzeros, w.scales, *wl.bounds)
            parity.check(f"noalloc {wl.name}", bf16_to_f64(y_na), y_ref,
                         parity.magnitudes_int4(A, S, w, *wl.bounds), wl.bounds, wl.G)


def test_noalloc_twice_then_smaller():
    """Two calls in a row on the same inputs, then a smaller one: every result equals pq_gemm."""
    wl = synth.Workload("na_rep", 234, 1024, 2048, 4096)
    A, S, R, w = _inputs(wl)
    wpk, sz = packed_weights(w)
    y1, z1 = _both(A, S, R, wpk, sz, wl.N, wl.bounds)
    y2, z2 = _both(A, S, R, wpk, sz, wl.N, wl.bounds)
    assert torch.equal(z1.view(torch.int16), y1.view(torch.int16))
    assert torch.equal(z2.view(torch.int16), y1.view(torch.int16))
    m = 40
    y3, z3 = _both(A[:, :m].copy(), S[:, :m].copy(), R[:, :m].copy(), wpk, sz, wl.N, wl.bounds)
    assert torch.equal(z3.view(torch.int16), y3.view(torch.int16))
    assert torch.equal(z3.view(torch.int16), y1[:m].view(torch.int16))


def test_noalloc_rejects_calls_beyond_its_scratch():
    """M = 8192 at K = 17408 with two partitions needs about 22 MB: refused before any launch."""
    P, M, K, N = 2, 8192, 17408, 256
    G = K // 128
    A = torch.zeros((P, M, K), dtype=torch.uint8, device="cuda")
    S = torch.zeros((P, M, G), dtype=torch.float32, device="cuda")
    wpk = torch.zeros(pq.lib().pq_packed_weight_bytes(K, N), dtype=torch.uint8, device="cuda")
    sz = torch.zeros((G, N, 2), dtype=torch.float16, device="cuda")
    y = torch.full((M, N), 7.0, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(pq.PQError) as e:
        pq.gemm_noalloc(A, S, S, wpk, sz, N, 128, pq.NO_BOUNDARY, out=y)
    assert e.value.code == -2 and "scratch" in str(e.value)
    torch.cuda.synchronize()
    assert torch.all(y == 7.0)
