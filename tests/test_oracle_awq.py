"""Pins of the oracle's AWQ unpack and dequant: hand-written words (tests/golden), the inverse
of the generator's packer, and a byte-level decomposition written independently."""
import os

import numpy as np

import synth
from oracle import awq

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "awq_nibbles.txt")


def test_golden_words():
    words, cols = [], []
    for line in open(GOLDEN):
        line = line.split("#")[0].strip()
        if not line:
            continue
        p = line.split()
        words.append(int(p[0], 16))
        cols.append([int(v) for v in p[1:]])
    w = np.array(words, dtype=np.uint32).view(np.int32).reshape(-1, 1)
    got = awq.unpack(w)
    assert got.tolist() == cols


def test_unpack_inverts_generator_pack():
    c = np.random.default_rng(3).integers(0, 16, (37, 64), dtype=np.uint8)
    assert np.array_equal(awq.unpack(synth.awq_pack(c)), c)


def test_unpack_bytewise():
    """Column 8j+ORDER[i] is nibble i; nibble i lives in byte i//2, high half if i is odd."""
    w = np.random.default_rng(5).integers(0, 2 ** 32, (9, 4), dtype=np.uint64).astype(np.uint32)
    b = w.view(np.uint8).reshape(9, 4, 4)    # little-endian bytes of each word
    got = awq.unpack(w.view(np.int32))
    order = [0, 2, 4, 6, 1, 3, 5, 7]
    for i in range(8):
        nib = (b[:, :, i // 2] >> (4 * (i % 2))) & 0xF
        assert np.array_equal(got[:, order[i]::8], nib)


def test_dequant_definition():
    r = np.random.default_rng(9)
    K, N = 256, 16
    c = r.integers(0, 16, (K, N), dtype=np.uint8)
    zp = r.integers(2, 15, (K // 128, N), dtype=np.uint8)
    sc = r.uniform(0.002, 0.02, (K // 128, N)).astype(np.float16)
    W = awq.dequant(synth.awq_pack(c), synth.awq_pack(zp), sc)
    for k in (0, 127, 128, 255):
        for n in (0, 7, 15):
            g = k // 128
            assert W[k, n] == float(sc[g, n]) * (int(c[k, n]) - int(zp[g, n]))
