"""Pins of the fused add + RMSNorm producer oracle (oracle/producer.py).

* P1: the new residual equals torch's own float32 add rounded to f16, bit for bit.
* P2: the plain norm equals torch.nn.functional.rms_norm evaluated in float64 and rounded to f16
  (an independent implementation of the same expression).
* P3: the Gemma form with w = 0 equals the plain form with unit weights; the Gemma form with w
  equals the plain form with weight 1 + w where 1 + w is exact in f16.
* P4: closed forms: a constant row normalises to sign(c) * w' (eps far below c^2); a row whose
  residual cancels the input is all zero and quantises to zero codes, scales and row-sums.
"""
import numpy as np
import torch

import synth
from oracle import producer, prologue


def _rows(M, K, seed):
    r = np.random.default_rng(seed)
    x = (r.standard_normal((M, K)) * 3).astype(np.float16)
    res = (r.standard_normal((M, K)) * 5).astype(np.float16)
    w = (r.standard_normal(K) * 0.2).astype(np.float16)
    return x, res, w


def test_P1_residual_is_f32_add_rounded_once():
    x, r, w = _rows(6, 640, 1)
    h, _ = producer.add_rms(x, r, w, 1e-6)
    want = (torch.from_numpy(x).float() + torch.from_numpy(r).float()).half().numpy()
    assert np.array_equal(h.view(np.uint16), want.view(np.uint16))


def test_P2_plain_norm_matches_torch_rms_norm():
    x, r, w = _rows(8, 1024, 2)
    h, hs = producer.add_rms(x, r, w, 1e-5, gemma=False)
    ref = torch.nn.functional.rms_norm(torch.from_numpy(h).double(), (1024,),
                                       weight=torch.from_numpy(w).double(), eps=1e-5)
    assert np.array_equal(hs.view(np.uint16), ref.half().numpy().view(np.uint16))


def test_P3_gemma_form():
    x, r, w = _rows(4, 512, 3)
    _, g0 = producer.add_rms(x, r, np.zeros(512, np.float16), 1e-6, gemma=True)
    _, p1 = producer.add_rms(x, r, np.ones(512, np.float16), 1e-6, gemma=False)
    assert np.array_equal(g0.view(np.uint16), p1.view(np.uint16))
    # weights whose 1 + w is exact in f16 (multiples of 2^-10 in [-1, 1))
    wq = (np.random.default_rng(4).integers(-1024, 1024, 512) / 1024.0).astype(np.float16)
    _, g = producer.add_rms(x, r, wq, 1e-6, gemma=True)
    _, p = producer.add_rms(x, r, (1.0 + wq.astype(np.float64)).astype(np.float16), 1e-6, gemma=False)
    assert np.array_equal(g.view(np.uint16), p.view(np.uint16))


def test_P4_closed_forms():
    K = 256
    x = np.full((2, K), 2.0, np.float16)
    x[1] = -3.0
    r = np.zeros((2, K), np.float16)
    w = np.zeros(K, np.float16)
    _, hs = producer.add_rms(x, r, w, 1e-9, gemma=True)
    assert np.all(hs[0] == 1.0) and np.all(hs[1] == -1.0)
    # residual cancels the input: zero row, zero codes
    wl = synth.Workload("prodzero", 180, 3, K, 64)
    xs = synth.activations(wl)
    pl, tl, cl = synth.rotations(wl)
    rr = (-xs.astype(np.float32)).astype(np.float16)
    rr[1] = 0
    h, hs, A, ASG, RS = producer.add_rms_rotate_quant(xs, rr, w, 1e-6, pl, tl, cl)
    assert not h[0].any() and not hs[0].any() and not h[2].any()
    assert not A[:, 0].any() and not ASG[:, 0].any() and not RS[:, 0].any()
    # the live row is the plain prologue of its normalised values
    A1, S1, R1 = prologue.rotate_quant(hs[1:2], pl, tl, cl)
    assert np.array_equal(A[:, 1:2], A1) and np.array_equal(ASG[:, 1:2], S1) and np.array_equal(RS[:, 1:2], R1)
