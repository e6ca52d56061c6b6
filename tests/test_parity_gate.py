"""CPU checks of the GEMM parity gate in tests/parity.py (no GPU).

The gate must admit every result that differs from the fp64 reference only by the roundings the
kernels are allowed (binary32 group products and folds, the f16 zero-point factor of the SZ format,
the bf16-split zero-point product, the bf16 output), and must reject a result with one wrong
16x16 output block, even where the Frobenius gate alone would pass it. The kernels' arithmetic is
emulated here in float32 from its description (raw weight codes on the matrix core, the factor
512 sc, the zero point as 8 sc + fl16(sc (zp - 8)) times the row-sum); the mistakes are planted
in that emulation's output.
"""
import numpy as np
import pytest
import torch

import synth
from oracle import awq, e4m3, gemm as ogemm, prologue as opro

import parity


def _bf16(y32):
    return torch.from_numpy(np.ascontiguousarray(y32, dtype=np.float32)).to(torch.bfloat16).double().numpy()


def _emulate(A, S, w, split_zero):
    """float32 emulation of the int4 e4m3 GEMM as the kernels compute it (P = 1)."""
    D = e4m3.decode(A[0])                                  # [M, K] fp64 (exact)
    c = awq.unpack(w.qweight).astype(np.float64)
    zp = awq.unpack(w.qzeros).astype(np.float32)
    sc = w.scales.astype(np.float32)
    M, K = D.shape
    G = K // 128
    asg = S[0].astype(np.float32)
    rs = D.reshape(M, G, 128).sum(-1).astype(np.float32)
    zsc = (sc * (zp - np.float32(8))).astype(np.float16).astype(np.float32)
    zf = (sc * np.float32(8) + zsc).astype(np.float32)    # exact in binary32
    acc = np.zeros((M, c.shape[1]), np.float32)
    for g in range(G):
        ks = slice(128 * g, 128 * g + 128)
        T = ((D[:, ks] @ c[ks]) * 2.0 ** -9).astype(np.float32)       # one rounding
        f = (asg[:, g][:, None] * (sc[g] * np.float32(512))[None, :]).astype(np.float32)
        acc = (acc + (f * T).astype(np.float32)).astype(np.float32)
    ar = (asg * rs).astype(np.float32)
    if split_zero:
        # bf16 pieces a1 + a2 and z1 + z2, product a1 z1 + a1 z2 + a2 z1 (fp64 sum, one rounding)
        def pieces(v):
            v1 = torch.from_numpy(v).to(torch.bfloat16).float().numpy()
            v2 = torch.from_numpy((v - v1).astype(np.float32)).to(torch.bfloat16).float().numpy()
            return v1.astype(np.float64), v2.astype(np.float64)
        a1, a2 = pieces(ar)
        z1, z2 = pieces(zf)
        Zt = (a1 @ z1 + a1 @ z2 + a2 @ z1).astype(np.float32)
    else:
        Zt = (ar.astype(np.float64) @ zf.astype(np.float64)).astype(np.float32)
    return _bf16((acc - Zt).astype(np.float32))


def _case(one_signed, M=40, K=512, N=256, wid=900):
    wl = synth.Workload("gate", wid, M, K, N)
    if one_signed:
        x = synth.activations_one_signed(wl)
        pl, tl, cl = synth.rotations_identity(wl)
    else:
        x = synth.activations(wl)
        pl, tl, cl = synth.rotations(wl)
    A, S, _ = opro.rotate_quant(x, pl, tl, cl)
    w = synth.weights(wl)
    y_ref = ogemm.gemm_ref(A, S, w.qweight, w.qzeros, w.scales, *wl.bounds)
    mags = parity.magnitudes_int4(A, S, w, *wl.bounds)
    return wl, A, S, w, y_ref, mags


@pytest.mark.parametrize("one_signed", [False, True])
@pytest.mark.parametrize("split_zero", [False, True])
def test_gate_admits_kernel_arithmetic(one_signed, split_zero):
    wl, A, S, w, y_ref, mags = _case(one_signed)
    if one_signed:
        assert np.all(e4m3.decode(A) >= 0)                 # one-signed codes reach the GEMM
    y = _emulate(A, S, w, split_zero)
    parity.check("gate emulation", y, y_ref, mags, wl.bounds, wl.G)


@pytest.mark.parametrize("one_signed", [False, True])
def test_gate_rejects_one_wrong_block(one_signed):
    """One 16x16 block with 2% of one group's contribution missing (a dropped term in a few of its
    products would look like this): small enough to pass the Frobenius gate on mixed-sign data,
    caught by the element-wise one."""
    wl, A, S, w, y_ref, mags = _case(one_signed, M=64, N=512)
    y = _emulate(A, S, w, True)
    D = e4m3.decode(A[0])
    W = awq.dequant(w.qweight, w.qzeros, w.scales)          # [K, N] fp64
    g, r0, c0 = 2, 16, 32
    ks = slice(128 * g, 128 * g + 128)
    term = (S[0][r0:r0 + 16, g].astype(np.float64)[:, None]) * (D[r0:r0 + 16, ks] @ W[ks, c0:c0 + 16])
    bad = y.copy()
    bad[r0:r0 + 16, c0:c0 + 16] = _bf16(y[r0:r0 + 16, c0:c0 + 16] - 0.02 * term)
    assert ogemm.rel_frobenius(bad, y_ref) < 2e-3 or one_signed   # the aggregate gate can miss it
    with pytest.raises(AssertionError, match="element-wise"):
        parity.check("gate planted block", bad, y_ref, mags, wl.bounds, wl.G)


def test_gate_rejects_zero_point_factor_error():
    """A 1% error on every group's zero-point factor (far above its f16 rounding) shifts the
    one-signed outputs, where the row-sums are largest, out of the bound."""
    wl, A, S, w, y_ref, mags = _case(True)
    y = _emulate(A, S, w, False)
    D = e4m3.decode(A[0])
    zp = awq.unpack(w.qzeros).astype(np.float64)
    sc = w.scales.astype(np.float64)
    rs = D.reshape(wl.M, wl.G, 128).sum(-1)
    shift = (S[0].astype(np.float64) * rs) @ (0.01 * sc * zp)
    with pytest.raises(AssertionError):
        parity.check("gate planted zero point", _bf16((y + shift).astype(np.float32)), y_ref, mags, wl.bounds, wl.G)
