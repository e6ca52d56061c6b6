"""Token-count sweep at the real projection shapes: every GEMM and prologue instantiation the
library dispatches on M, at the gate_up shape (K=5120, N=17408, one partition) and the merged QKV
shape (K=5120, N=8192 = 6144 | 1024 | 1024, three distinct rotations).

M = 1..16 runs the decode kernel (runs of column tiles per workgroup, 1 or 4 live rows per lane);
M = 17..255 runs the prefill kernel with one 256-row tile (ragged rows inside it) plus the split
last round; 256 is one whole row tile. The page gates each instantiation over many token counts at
every shape ("Gates passed"); this sweep does the same for the switch points of this library.

Gates: the prologue bit-exact against the oracle (codes, scales, row-sums), the GEMM against the
oracle's fp64 reference through tests/parity.py (Frobenius and element-wise), rows past M
untouched.
"""
import numpy as np
import pytest
import torch

import rotated_w4a8_group_amd as pq
import synth
from oracle import gemm as ogemm
from oracle import prologue as opro

import parity
from gpu_util import SENT_BF16, bf16_to_f64, packed_weights, prologue_gpu, to_dev

pytestmark = pytest.mark.gpu

MS = [1, 2, 3, 5, 7, 9, 12, 16, 17, 32, 64, 127, 255, 256]
MMAX = max(MS)
SHAPES = {
    "gate_up": synth.Workload("sweep_gate_up", 130, MMAX, 5120, 17408),
    "qkv": synth.Workload("sweep_qkv", 131, MMAX, 5120, 8192, splits=(6144, 1024, 1024)),
}
_CACHE = {}


def _data(shape):
    """Oracle prologue, packed weights, reference and magnitudes for MMAX rows (each M takes the
    first M rows: rows are independent in both the prologue and the GEMM)."""
    if shape not in _CACHE:
        wl = SHAPES[shape]
        x = synth.activations(wl)
        pl, tl, cl = synth.rotations(wl)
        A, S, R = opro.rotate_quant(x, pl, tl, cl)
        w = synth.weights(wl)
        y_ref = ogemm.gemm_ref(A, S, w.qweight, w.qzeros, w.scales, *wl.bounds)
        mags = parity.magnitudes_int4(A, S, w, *wl.bounds)
        _CACHE[shape] = (wl, x, (pl, tl, cl), (A, S, R), packed_weights(w), y_ref, mags)
    return _CACHE[shape]


@pytest.mark.parametrize("M", MS)
@pytest.mark.parametrize("shape", list(SHAPES))
def test_sweep(shape, M):
    wl, x, (pl, tl, cl), (A, S, R), (wpk, sz), y_ref, mags = _data(shape)
    print(f"[sweep {shape}] M={M} K={wl.K} N={wl.N} P={wl.P}", flush=True)
    # prologue on the GPU for the first M rows, bit-exact against the oracle's codes
    wlm = synth.Workload(wl.name, wl.wid, M, wl.K, wl.N, splits=wl.splits)
    Ag, Sg, Rg = prologue_gpu(wlm, x[:M], pl, tl, cl)
    assert np.array_equal(Ag.cpu().numpy(), A[:, :M])
    assert np.array_equal(Sg.cpu().numpy().view(np.uint32), S[:, :M].view(np.uint32))
    assert np.array_equal(Rg.cpu().numpy().view(np.uint32), R[:, :M].view(np.uint32))
    # the GEMM on those codes
    ybuf = torch.empty((M + 3, wl.N), dtype=torch.bfloat16, device="cuda")
    ybuf.view(torch.int16).fill_(SENT_BF16)
    pq.gemm(Ag, Sg, Rg, wpk, sz, wl.N, *wl.bounds, out=ybuf[:M])
    torch.cuda.synchronize()
    assert torch.all(ybuf[M:].view(torch.int16) == SENT_BF16), "rows past M were written"
    parity.check(f"sweep {shape} M={M}", bf16_to_f64(ybuf[:M]), y_ref[:M],
                 tuple(t[:M] for t in mags), wl.bounds, wl.G)
