"""GPU parity of the rotate-quant prologue against the oracle: codes, group scales and
row-sums must be bitwise equal (compared as integer bit patterns), on every workload, with
guard regions checked for stray writes. Also the exhaustive checks of the device encoder
and reciprocal the prologue uses."""
import numpy as np
import pytest
import torch

import rotated_w4a8_group_amd as pq
import synth
from oracle import e4m3 as oe4m3
from oracle import prologue as opro

from gpu_util import prologue_gpu, to_dev

pytestmark = pytest.mark.gpu

SAMPLE_ROWS = 192


def _compare(name, A, S, R, x, pl, tl, cl, rows):
    A_ref, S_ref, R_ref = opro.rotate_quant(x[rows], pl, tl, cl)
    A_g = A[:, rows].cpu().numpy()
    S_g = S[:, rows].cpu().numpy()
    R_g = R[:, rows].cpu().numpy()
    bad_a = np.count_nonzero(A_g != A_ref)
    bad_s = np.count_nonzero(S_g.view(np.uint32) != S_ref.view(np.uint32))
    bad_r = np.count_nonzero(R_g.view(np.uint32) != R_ref.view(np.uint32))
    print(f"[prologue {name}] rows={len(rows)} code mismatches={bad_a} asg={bad_s} rs={bad_r}", flush=True)
    assert bad_a == 0 and bad_s == 0 and bad_r == 0


@pytest.mark.parametrize("name", ["tiny", "decode_m1", "decode_m8", "qkv", "prefill", "full_gate_up", "full_down"])
def test_prologue_bit_exact(name):
    wl = synth.WORKLOADS[name]
    print(f"[prologue {name}] M={wl.M} K={wl.K} P={wl.P}", flush=True)
    x = synth.activations(wl)
    pl, tl, cl = synth.rotations(wl)
    A, S, R = prologue_gpu(wl, x, pl, tl, cl)
    if wl.M <= 2048:
        rows = np.arange(wl.M)
    else:
        r = np.random.default_rng(17)
        rows = np.sort(np.concatenate([[0, wl.M - 1], r.choice(np.arange(1, wl.M - 1), SAMPLE_ROWS - 2, replace=False)]))
    _compare(name, A, S, R, x, pl, tl, cl, rows)


def test_prologue_edge_cases():
    """Ragged token count, a single group, zero rows, saturating magnitudes, f16 subnormals,
    a strided x (ldx > K), three partitions."""
    wl = synth.Workload("edge", 40, 37, 384, 128, splits=(64, 32, 32))
    x = synth.activations(wl)
    x[3] = 0
    x[5, :128] = 0
    x[7] = np.float16(6.0e4)
    x[8, ::2] = np.float16(-6.0e-8)
    x[9] = np.float16(2.0 ** -24)
    pl, tl, cl = synth.rotations(wl)
    A, S, R = prologue_gpu(wl, x, pl, tl, cl)
    _compare("edge", A, S, R, x, pl, tl, cl, np.arange(wl.M))
    # strided activations: x is a column slice of a wider tensor
    wide = np.zeros((wl.M, wl.K + 64), dtype=np.float16)
    wide[:, :wl.K] = x
    from gpu_util import records_for
    xs = to_dev(wide)[:, :wl.K]
    A2, S2, R2 = pq.rotate_quant(xs, to_dev(records_for(pl, tl)), to_dev(np.stack(cl)))
    assert torch.equal(A2, A) and torch.equal(S2.view(torch.int32), S.view(torch.int32))
    assert torch.equal(R2.view(torch.int32), R.view(torch.int32))
    # x rows that are only 4-byte aligned: ldx = K + 2, and a view starting 2 columns in
    for pad, start in ((2, 0), (6, 2)):
        wide = np.zeros((wl.M, wl.K + pad), dtype=np.float16)
        wide[:, start:start + wl.K] = x
        xs = to_dev(wide)[:, start:start + wl.K]
        A3, S3, R3 = pq.rotate_quant(xs, to_dev(records_for(pl, tl)), to_dev(np.stack(cl)))
        assert torch.equal(A3, A) and torch.equal(S3.view(torch.int32), S.view(torch.int32))
        assert torch.equal(R3.view(torch.int32), R.view(torch.int32))
    # K = 128, one token
    wl1 = synth.Workload("edge1", 41, 1, 128, 16)
    x1 = synth.activations(wl1)
    pl1, tl1, cl1 = synth.rotations(wl1)
    A1, S1, R1 = prologue_gpu(wl1, x1, pl1, tl1, cl1)
    _compare("edge1", A1, S1, R1, x1, pl1, tl1, cl1, np.arange(1))


def _encode_boundaries():
    """For k = 1..126 the smallest positive fp32 bit pattern whose oracle code is >= k
    (the oracle's encoder is monotone in |q|)."""
    lo = np.zeros(126, dtype=np.int64)
    hi = np.full(126, 0x7F800000, dtype=np.int64)       # +inf encodes to 0x7E >= k
    ks = np.arange(1, 127)
    while np.any(hi - lo > 1):
        mid = (lo + hi) // 2
        c = oe4m3.encode(mid.astype(np.uint32).view(np.float32)).astype(np.int64)
        ge = c >= ks
        hi = np.where(ge, mid, hi)
        lo = np.where(ge, lo, mid)
    return hi


def test_device_encoder_exhaustive():
    """E4: the device encoder equals the oracle's E on all 2^32 fp32 bit patterns."""
    bnd = torch.tensor(_encode_boundaries(), dtype=torch.int32, device="cuda")
    chunk = 1 << 28
    bad = 0
    for c in range(1 << 4):
        lo = -(1 << 31) + c * chunk
        bits = torch.arange(lo, lo + chunk, dtype=torch.int32, device="cuda")
        codes = pq.e4m3_encode(bits.view(torch.float32)).to(torch.int32)
        mag = bits & 0x7FFFFFFF
        want = torch.bucketize(mag, bnd, out_int32=True, right=True)
        nan = mag > 0x7F800000
        neg = (bits < 0) & (mag != 0) & ~nan
        want = torch.where(neg, want | 0x80, want)
        want = torch.where(nan, torch.zeros_like(want), want)
        bad += int((codes != want).sum())
        del bits, codes, mag, want
    print(f"[encoder] mismatches over 2^32 inputs: {bad}", flush=True)
    assert bad == 0


def test_device_recip_correctly_rounded():
    """E5: 1/x on device is the correctly rounded fp32 reciprocal for every x in
    [2^-126, 2^126) (positive normals whose reciprocal is normal; group scales live far inside
    this range). With y the device result, correct rounding means 1/x lies within half the
    spacing on its side of y: x*y - 1 <= x*ulp_below(y)/2 when y > 1/x, 1 - x*y <= x*ulp(y)/2
    otherwise, evaluated exactly in fp64 (x*y has at most 48 significant bits)."""
    lo_b, hi_b = 0x00800000, 0x7E800000
    chunk = 1 << 27
    bad = 0
    for start in range(lo_b, hi_b, chunk):
        end = min(hi_b, start + chunk)
        bits = torch.arange(start, end, dtype=torch.int32, device="cuda")
        x = bits.view(torch.float32)
        y = pq.recip_f32(x)
        xd, yd = x.double(), y.double()
        d = xd * yd - 1.0
        f, e = torch.frexp(yd)
        ulp = torch.ldexp(torch.ones_like(yd), (e - 24).to(torch.int64))
        below = torch.where(f == 0.5, ulp * 0.5, ulp)
        bad += int(((d > 0) & (d > xd * below * 0.5)).sum()) + int(((d <= 0) & (-d > xd * ulp * 0.5)).sum())
        del bits, x, y, xd, yd, d, f, e, ulp, below
    print(f"[recip] incorrectly rounded: {bad}", flush=True)
    assert bad == 0
