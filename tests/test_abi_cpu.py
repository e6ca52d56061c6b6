"""CPU-side tests of the C-ABI library: it loads, exports every symbol include/pq.h declares,
its host-only record builder agrees with the oracle, and every validation path returns the
documented error before anything is launched (no GPU is touched here)."""
import ctypes
import os
import re

import numpy as np
import pytest

import rotated_w4a8_group_amd as pq
import synth
from oracle import prologue as oprologue
from oracle import records as orec

import lanes

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "pq.h")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(pq_[a-z0-9_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    L = pq.lib()
    names = _declared()
    assert len(names) >= 10
    for n in names:
        assert hasattr(L, n), n
    assert set(names) == set(pq.SIGNATURES), "binding signatures out of step with include/pq.h"


def test_abi_version():
    m = re.search(r"#define PQ_ABI_VERSION (\d+)", open(HEADER).read())
    assert pq.lib().pq_abi_version() == int(m.group(1))


def _ref_rotations(ref, r, sl):
    return sorted((int(i), int(j), int(c), int(s)) if i < j else (int(j), int(i), int(c), int(s) ^ 0x8000)
                  for i, j, c, s in zip(ref["i"][r, sl], ref["j"][r, sl], ref["cos16"][r, sl], ref["sin16"][r, sl]))


@pytest.mark.parametrize("wl_name", ["tiny", "qkv"])
def test_records_match_oracle_up_to_lane_order(wl_name):
    """Each (layer, group) of records applies exactly the oracle's 64 rotations, in some lane
    order and orientation."""
    wl = synth.WORKLOADS[wl_name]
    pl, tl, _ = synth.rotations(wl)
    for pairs, theta in zip(pl, tl):
        if wl.K > 1024:
            pairs, theta = pairs[:, :1024], theta[:, :512]
        lib = pq.build_records(pairs, theta)          # [8, K/2, 8]
        ref = orec.build(pairs, theta)
        d = lanes.decode(lib)
        for r in range(8):
            for g in range(pairs.shape[1] // 128):
                sl = slice(64 * g, 64 * g + 64)
                assert lanes.canonical(d, r, sl) == _ref_rotations(ref, r, sl), (r, g)


def test_records_lane_order_is_bank_conflict_free():
    wl = synth.WORKLOADS["qkv"]
    pl, tl, _ = synth.rotations(wl)
    lanes.check_lanes(pq.build_records(pl[1][:, :2048], tl[1][:, :1024]))


@pytest.mark.parametrize("seed", range(4))
def test_records_lane_order_any_pairing(seed):
    """Any pairing of each group's channels orders conflict-free, including adversarial ones
    (every pair inside one 8-channel block, pairs with equal rows mod 16, identity pairing)."""
    rng = np.random.default_rng(seed)
    K = 128 * 8
    pairs = np.empty((8, K), np.int16)
    for r in range(8):
        for g in range(K // 128):
            kind = (r + g + seed) % 4
            if kind == 0:
                perm = rng.permutation(128)
            elif kind == 1:
                perm = np.arange(128)                      # (0,1), (2,3), ...: same 8-block
            elif kind == 2:
                # pair ch with the channel whose row is 16 higher: equal rows mod 16
                order = sorted(range(128), key=lambda ch: (lanes.lds_row(ch) % 16, ch))
                perm = np.array(order)
            else:
                perm = np.concatenate([np.arange(0, 128, 2), np.arange(1, 128, 2)])
                perm = perm.reshape(2, 64).T.reshape(-1)  # (0,1),(2,3) interleaved differently
                perm = rng.permutation(perm.reshape(64, 2)).reshape(-1)
            pairs[r, 128 * g:128 * g + 128] = perm
    theta = rng.standard_normal((8, K // 2)).astype(np.float16)
    lib = pq.build_records(pairs, theta)
    lanes.check_lanes(lib)
    # and the records still hold exactly the given rotations, and compute them
    ref = orec.build(pairs, theta)
    d = lanes.decode(lib)
    for r in range(8):
        for g in range(K // 128):
            sl = slice(64 * g, 64 * g + 64)
            assert lanes.canonical(d, r, sl) == _ref_rotations(ref, r, sl), (r, g)
    cs = np.ones(K, np.float16)
    x = rng.standard_normal((5, K)).astype(np.float16)
    want = oprologue.rotate_f32(x, ref, cs)
    got = lanes.simulate(lib, x.astype(np.float32))
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))


def test_records_reject_bad_pairs():
    pairs = np.tile(np.arange(128, dtype=np.int16), (8, 2))
    theta = np.zeros((8, 128), np.float16)
    pairs[5, 130] = pairs[5, 131]
    with pytest.raises(pq.PQError) as e:
        pq.build_records(pairs, theta)
    assert e.value.code == -5
    with pytest.raises(pq.PQError) as e:
        pq.lib().pq_build_records(None, None, 256, None) and None
        pq._check("pq_build_records", pq.lib().pq_build_records(None, None, 256, None))
    assert e.value.code == -1


FAKE = ctypes.c_void_p(0x100000)   # aligned, never dereferenced: validation fails first or M == 0


def _gemm(**kw):
    a = dict(a=FAKE, asg=FAKE, rs=FAKE, M=4, K=256, P=1, wpk=FAKE, sz=FAKE, N=128,
             pb1=pq.NO_BOUNDARY, pb2=pq.NO_BOUNDARY, y=FAKE, ldy=128, ws=FAKE, ws_bytes=1 << 24, s=None)
    a.update(kw)
    return pq.lib().pq_gemm(a["a"], a["asg"], a["rs"], a["M"], a["K"], a["P"], a["wpk"], a["sz"],
                            a["N"], a["pb1"], a["pb2"], a["y"], a["ldy"], a["ws"], a["ws_bytes"], a["s"])


@pytest.mark.parametrize("kw,code", [
    (dict(K=100), -2), (dict(K=0), -2), (dict(N=120), -2), (dict(M=-1), -2), (dict(ldy=64), -2),
    (dict(ldy=129), -2), (dict(P=0), -4), (dict(P=4), -4), (dict(P=2), -4),
    (dict(P=2, pb1=64), -4), (dict(P=2, pb1=0), -4), (dict(P=3, pb1=256, pb2=128, N=512, ldy=512), -4),
    (dict(P=1, pb1=128, N=256, ldy=256), -4),
    (dict(P=2, pb1=pq.NO_BOUNDARY, pb2=128, N=256, ldy=256), -4),
    (dict(a=None), -1), (dict(y=None), -1), (dict(a=ctypes.c_void_p(0x100004)), -3),
    (dict(y=ctypes.c_void_p(0x100002)), -3),
])
def test_gemm_validation(kw, code):
    assert _gemm(**kw) == code
    assert pq.lib().pq_last_error().decode()


def test_gemm_m0_is_noop_and_partition_ok():
    assert _gemm(M=0, a=None, y=None) == 0
    assert _gemm(M=0, P=3, N=8192, pb1=6144, pb2=7168, ldy=8192) == 0
    assert _gemm(M=0, P=2, N=256, pb1=128, ldy=256) == 0
    assert pq.gemm_workspace_bytes(8, 17408, 5120) == 0
    # zero-point operand (3 partitions x 128 row tiles x 4 chunks x 1 KiB) + transposed scales
    assert pq.gemm_workspace_bytes(2048, 17408, 5120) == 3 * 128 * 4 * 1024 + 3 * 40 * 2048 * 4
    assert _gemm(M=32, ws=None, ws_bytes=1 << 20) == -1


def test_gemm_rejects_rows_beyond_32_bit_offsets():
    # the prefill kernel addresses a partition's activations with 32-bit offsets: M * K must stay
    # below 2^31 (300000 x 8192 = 2.46e9); the call fails before any launch
    assert _gemm(M=300000, K=8192, N=128, ws_bytes=1 << 40) == -2
    assert "too large" in pq.lib().pq_last_error().decode()


def test_gemm_noalloc_validation_and_scratch_limit():
    lib = pq.lib()
    S = lib.pq_gemm_noalloc_max_scratch_bytes()
    assert S == 16 << 20

    def call(M, K, P, N=256, pb1=pq.NO_BOUNDARY, pb2=pq.NO_BOUNDARY, **kw):
        a = dict(a=FAKE, y=FAKE)
        a.update(kw)
        return lib.pq_gemm_noalloc(a["a"], FAKE, FAKE, M, K, P, FAKE, FAKE, N, pb1, pb2, a["y"], N, None)
    # beyond the scratch: rejected before anything else is touched (no device needed)
    assert call(8192, 17408, 2, pb1=128) == -2 and "scratch" in lib.pq_last_error().decode()
    assert call(16384, 17408, 1) == -2
    # the same validation as pq_gemm
    assert call(4, 100, 1) == -2 and call(4, 256, 2) == -4 and call(4, 256, 1, a=None) == -1
    assert call(4, 256, 1, a=ctypes.c_void_p(0x100004)) == -3
    assert call(0, 256, 1, a=None, y=None) == 0


def test_gemm5_and_pack5_validation():
    lib = pq.lib()
    # int5 needs N % 32 == 0 (the fifth-bit planes hold 32 columns per word)
    assert lib.pq_gemm5(FAKE, FAKE, FAKE, 4, 256, 1, FAKE, FAKE, 48, pq.NO_BOUNDARY, pq.NO_BOUNDARY,
                        FAKE, 48, FAKE, 1 << 24, None) == -2
    assert lib.pq_gemm5(None, FAKE, FAKE, 4, 256, 1, FAKE, FAKE, 64, pq.NO_BOUNDARY, pq.NO_BOUNDARY,
                        FAKE, 64, FAKE, 1 << 24, None) == -1
    assert lib.pq_gemm5(FAKE, FAKE, FAKE, 0, 256, 1, FAKE, FAKE, 64, pq.NO_BOUNDARY, pq.NO_BOUNDARY,
                        FAKE, 64, FAKE, 1 << 24, None) == 0
    assert lib.pq_pack_weights5(FAKE, FAKE, FAKE, FAKE, FAKE, 256, 48, FAKE, FAKE, None) == -2
    assert lib.pq_pack_weights5(FAKE, FAKE, FAKE, FAKE, FAKE, 100, 64, FAKE, FAKE, None) == -2
    assert lib.pq_pack_weights5(FAKE, None, FAKE, FAKE, FAKE, 256, 64, FAKE, FAKE, None) == -1
    # nibble image + fifth-bit planes (K N / 8) + zero-point operand
    assert lib.pq_packed_weight5_bytes(5120, 17408) == 5120 * 17408 // 2 + 5120 * 17408 // 8 + 1088 * 4 * 1024 + 40 * 17408 * 4
    assert lib.pq_packed_weight5_bytes(256, 48) == 0


def test_add_rms_rotate_quant_validation():
    f = pq.lib().pq_add_rms_rotate_quant
    ok = dict(x=FAKE, ldx=256, r=FAKE, ldr=256, w=FAKE, eps=1e-6, gemma=1, M=4, K=256, P=1, rec=FAKE, cs=FAKE,
              ro=FAKE, ldo=256, hs=FAKE, A=FAKE, S=FAKE, R=FAKE)

    def call(**kw):
        a = dict(ok, **kw)
        return f(a["x"], a["ldx"], a["r"], a["ldr"], a["w"], a["eps"], a["gemma"], a["M"], a["K"], a["P"], a["rec"],
                 a["cs"], a["ro"], a["ldo"], a["hs"], a["A"], a["S"], a["R"], None)
    assert call(M=0) == 0
    assert call(K=100) == -2 and call(K=18560, ldx=18560, ldr=18560, ldo=18560) == -2
    assert call(ldx=260) == -2 and call(ldo=128) == -2
    assert call(eps=0.0) == -2 and call(eps=float("inf")) == -2
    assert call(P=4) == -4
    assert call(r=None) == -1 and call(hs=None) == -1
    assert call(x=ctypes.c_void_p(0x100008)) == -3
    # the new residual overlapping the old one other than as the same rows: rejected before launch
    assert call(ro=ctypes.c_void_p(0x100000 + 512)) == -2                  # one row further on
    assert call(ro=ctypes.c_void_p(0x100000 + 16)) == -2                   # inside the first row
    assert call(ldo=264) == -2                                             # same start, other stride
    assert call(r=ctypes.c_void_p(0x100000 + 3 * 512)) == -2               # res starts in res_out's rows
    assert "overlaps" in pq.lib().pq_last_error().decode()


def _rq(**kw):
    a = dict(x=FAKE, ldx=256, M=4, K=256, P=1, rec=FAKE, cs=FAKE, A=FAKE, asg=FAKE, rs=FAKE, s=None)
    a.update(kw)
    return pq.lib().pq_rotate_quant(a["x"], a["ldx"], a["M"], a["K"], a["P"], a["rec"], a["cs"],
                                    a["A"], a["asg"], a["rs"], a["s"])


@pytest.mark.parametrize("kw,code", [
    (dict(K=200), -2), (dict(M=-2), -2), (dict(ldx=255), -2), (dict(ldx=128), -2), (dict(P=4), -4),
    (dict(P=0), -4), (dict(x=None), -1), (dict(rs=None), -1), (dict(A=ctypes.c_void_p(0x100008)), -3),
    (dict(x=ctypes.c_void_p(0x100002)), -3), (dict(rec=ctypes.c_void_p(0x100004)), -3),
])
def test_rotate_quant_validation(kw, code):
    assert _rq(**kw) == code


def test_rotate_quant_m0_noop():
    assert _rq(M=0, x=None, A=None) == 0


def test_pack_validation():
    L = pq.lib()
    assert L.pq_pack_weights(FAKE, FAKE, FAKE, 100, 128, FAKE, FAKE, None) == -2
    assert L.pq_pack_weights(FAKE, FAKE, FAKE, 256, 8, FAKE, FAKE, None) == -2
    assert L.pq_pack_weights(None, FAKE, FAKE, 256, 128, FAKE, FAKE, None) == -1
    assert L.pq_pack_weights(FAKE, FAKE, FAKE, 256, 128, ctypes.c_void_p(0x100008), FAKE, None) == -3
    # codes (K*N/2) + the zero-point epilogue operand: N/16 tiles x ceil(3G/32) chunks x 1 KiB
    # + the fp32 column factors of the prefill fold (G x N x 4 bytes)
    assert L.pq_packed_weight_bytes(5120, 17408) == 5120 * 17408 // 2 + (17408 // 16) * 4 * 1024 + 40 * 17408 * 4
    assert L.pq_packed_weight_bytes(17408, 5120) == 17408 * 5120 // 2 + (5120 // 16) * 13 * 1024 + 136 * 5120 * 4
    assert L.pq_packed_weight_bytes(100, 16) == 0


def _gemm_variant(name, **kw):
    a = dict(a=FAKE, asg=FAKE, rs=FAKE, M=4, K=256, P=1, wpk=FAKE, sz=FAKE, N=128,
             pb1=pq.NO_BOUNDARY, pb2=pq.NO_BOUNDARY, y=FAKE, ldy=128, ws=FAKE, ws_bytes=1 << 24, s=None)
    a.update(kw)
    return getattr(pq.lib(), name)(a["a"], a["asg"], a["rs"], a["M"], a["K"], a["P"], a["wpk"], a["sz"],
                                   a["N"], a["pb1"], a["pb2"], a["y"], a["ldy"], a["ws"], a["ws_bytes"], a["s"])


@pytest.mark.parametrize("name", ["pq_gemm_tok", "pq_gemm_i8"])
def test_gemm_variant_validation(name):
    assert _gemm_variant(name, M=0, a=None, y=None) == 0
    assert _gemm_variant(name, K=100) == -2 and _gemm_variant(name, N=120) == -2
    assert _gemm_variant(name, ldy=64) == -2 and _gemm_variant(name, M=-1) == -2
    assert _gemm_variant(name, P=2) == -4 and _gemm_variant(name, P=4) == -4
    assert _gemm_variant(name, a=None) == -1 and _gemm_variant(name, rs=None) == -1
    assert _gemm_variant(name, y=ctypes.c_void_p(0x100002)) == -3
    assert _gemm_variant(name, M=32, ws=None, ws_bytes=1 << 20) == -1
    assert pq.lib().pq_last_error().decode().startswith(name)


def test_gemm_tok_workspace_sizes():
    L = pq.lib()
    # decode (M <= 16): the token scale repeated for every group, 3 partitions, 256-byte multiple
    assert L.pq_gemm_tok_workspace_bytes(8, 17408, 5120) == (3 * 8 * 40 * 4 + 255) // 256 * 256
    # prefill: the zero-point activation operand only (no transposed group scales)
    assert L.pq_gemm_tok_workspace_bytes(2048, 17408, 5120) == 3 * 128 * 4 * 1024
    assert L.pq_gemm_tok_workspace_bytes(0, 17408, 5120) == 0
    assert L.pq_gemm_tok_workspace_bytes(8, 17408, 100) == 0


def _rq_variant(name, **kw):
    a = dict(x=FAKE, ldx=256, M=4, K=256, P=1, rec=FAKE, cs=FAKE, A=FAKE, asg=FAKE, rs=FAKE, s=None)
    a.update(kw)
    return getattr(pq.lib(), name)(a["x"], a["ldx"], a["M"], a["K"], a["P"], a["rec"], a["cs"],
                                   a["A"], a["asg"], a["rs"], a["s"])


@pytest.mark.parametrize("name", ["pq_rotate_quant_tok", "pq_rotate_quant_i8"])
def test_prologue_variant_validation(name):
    assert _rq_variant(name, M=0, x=None, A=None) == 0
    assert _rq_variant(name, K=200) == -2 and _rq_variant(name, M=-2) == -2
    assert _rq_variant(name, ldx=128) == -2
    assert _rq_variant(name, P=0) == -4 and _rq_variant(name, P=4) == -4
    assert _rq_variant(name, x=None) == -1 and _rq_variant(name, rs=None) == -1
    assert _rq_variant(name, x=ctypes.c_void_p(0x100002)) == -3
    assert pq.lib().pq_last_error().decode().startswith(name)


def test_prologue_tok_row_limit():
    # the per-token kernel keeps a whole row on chip: at most 16 waves x 9 groups x 128 channels
    assert _rq_variant("pq_rotate_quant_tok", K=18432, ldx=18432, M=0) == 0
    assert _rq_variant("pq_rotate_quant_tok", K=18560, ldx=18560) == -2
    assert _rq_variant("pq_rotate_quant_tok", ldx=257) == -2   # odd row stride


def test_hooks_validation():
    L = pq.lib()
    assert L.pq_e4m3_encode(FAKE, FAKE, -1, None) == -2
    assert L.pq_e4m3_encode(None, None, 0, None) == 0
    assert L.pq_recip_f32(None, FAKE, 5, None) == -1
    assert L.pq_bf16_round(FAKE, FAKE, -1, None) == -2
    assert L.pq_bf16_round(None, None, 0, None) == 0
    assert L.pq_bf16_round(FAKE, None, 3, None) == -1


def _proj(seed, K=256, ncols=128):
    rng = np.random.default_rng(seed)
    pairs = np.concatenate([rng.permutation(128) for _ in range(8 * K // 128)]).reshape(8, K).astype(np.int16)
    theta = rng.uniform(-np.pi, np.pi, (8, K // 2)).astype(np.float16)
    cs = np.exp(rng.normal(0, 0.3, K)).astype(np.float16)
    return [ncols, pairs, theta, cs]


def test_plan_partitions_pages_examples():
    """The pages' two examples ("Design" item 4): an attention QKV with three distinct rotations
    stays at P = 3; in_proj_qkvz, whose q, k and v share one rotation and z has its own, loads as
    4 projections and plans to P = 2 with the boundary after v."""
    q, k, v = _proj(1, ncols=256), _proj(2, ncols=128), _proj(3, ncols=128)
    assert pq.plan_partitions([q, k, v]) == (3, 256, 384, [0, 1, 2])
    shared = _proj(4, ncols=128)
    z = _proj(5, ncols=256)
    qkv_same = [[n] + shared[1:] for n in (256, 128, 128)]
    assert pq.plan_partitions(qkv_same + [z]) == (2, 512, pq.NO_BOUNDARY, [0, 3])
    assert pq.plan_partitions([shared]) == (1, pq.NO_BOUNDARY, pq.NO_BOUNDARY, [0])


def test_plan_partitions_merges_only_adjacent_and_exact():
    a, b = _proj(6), _proj(7)
    # A B A: three runs (identical but not adjacent rotations are not merged)
    assert pq.plan_partitions([a, b, a])[0] == 3
    # one f16 ulp in one channel scale breaks the identity
    a2 = [a[0], a[1], a[2], a[3].copy()]
    a2[3].view(np.uint16)[17] += 1
    assert pq.plan_partitions([a, a2])[0] == 2
    with pytest.raises(pq.PQError) as e:       # four runs
        pq.plan_partitions([a, b, a, b])
    assert e.value.code == -4
    with pytest.raises(pq.PQError) as e:       # a run boundary off the 128-column grid
        pq.plan_partitions([[144] + a[1:], b])
    assert e.value.code == -4
    with pytest.raises(pq.PQError) as e:       # columns not a multiple of 16
        pq.plan_partitions([[100] + a[1:]])
    assert e.value.code == -2


@pytest.mark.parametrize("wl_name", ["tiny", "qkv", "decode_m1"])
def test_records_chain_computes_the_oracle_rotation(wl_name):
    """Driving the prologue's register / LDS dataflow with the records alone (first layer from
    the image, later layers from a register and a hand-off row, last layer back to the image)
    gives the oracle's float32 rotation bit for bit, on every partition of the workload."""
    wl = synth.WORKLOADS[wl_name]
    pl, tl, cl = synth.rotations(wl)
    x = synth.activations(wl, M=6)
    K = min(wl.K, 2048)
    for pairs, theta, cs in zip(pl, tl, cl):
        pairs, theta, cs = pairs[:, :K], theta[:, :K // 2], cs[:K]
        lib = pq.build_records(pairs, theta)
        lanes.check_lanes(lib)
        xv = x[:, :K].astype(np.float32) * cs.astype(np.float32)
        want = oprologue.rotate_f32(x[:, :K], orec.build(pairs, theta), cs)
        got = lanes.simulate(lib, xv)
        assert np.array_equal(got.view(np.uint32), want.view(np.uint32))


@pytest.mark.parametrize("layer,shift", [(3, 16), (3, 24), (0, 24), (7, 16)])
def test_records_chain_simulation_catches_a_wrong_slot(layer, shift):
    """The simulation is sensitive to the routing: one hand-off row swapped between two lanes of
    a layer changes the result (a middle layer's read and write rows, layer 0's write row and
    layer 7's read row)."""
    wl = synth.WORKLOADS["tiny"]
    pl, tl, cl = synth.rotations(wl)
    lib = pq.build_records(pl[0], tl[0]).copy()
    x = synth.activations(wl).astype(np.float32)
    good = lanes.simulate(lib, x)
    w = lib[layer, :, :4].copy().view(np.uint32)[:, 0]
    mask = np.uint32(0xFF << shift)
    r0, r1 = w[5] & mask, w[9] & mask
    assert r0 != r1
    w[5] = (w[5] & ~mask) | r1
    w[9] = (w[9] & ~mask) | r0
    lib[layer, :, :4] = w.view(np.uint8).reshape(-1, 4)
    assert not np.array_equal(lanes.simulate(lib, x).view(np.uint32), good.view(np.uint32))


@pytest.mark.parametrize("layer,field", [(7, "neg_v"), (3, "f2"), (0, "f1")])
def test_records_chain_simulation_catches_a_wrong_sign(layer, field):
    """The signs folded into the records matter: the last layer's "v arrives negated" bit, or one
    coefficient's sign in a middle layer (where the hand-off sign is folded into f2) or in the
    first, flipped for one lane, changes the result; and such a flip in a middle layer is also
    seen by the decoding of the records' rotations."""
    wl = synth.WORKLOADS["tiny"]
    pl, tl, cl = synth.rotations(wl)
    lib = pq.build_records(pl[0], tl[0]).copy()
    x = synth.activations(wl).astype(np.float32)
    good = lanes.simulate(lib, x)
    lane = 5
    if field == "neg_v":
        lib[layer, lane, 0] ^= 0x80
    else:
        lib[layer, lane, 5 if field == "f1" else 7] ^= 0x80       # the f16's sign bit
    assert not np.array_equal(lanes.simulate(lib, x).view(np.uint32), good.view(np.uint32))
    if field != "neg_v":
        ref = orec.build(pl[0][:, :128], tl[0][:, :64])
        assert lanes.canonical(lanes.decode(lib), layer, slice(0, 64)) != _ref_rotations(ref, layer, slice(0, 64))


def _rq_ws(**kw):
    a = dict(x=FAKE, ldx=256, M=32, K=256, P=1, rec=FAKE, cs=FAKE, A=FAKE, asg=FAKE, rs=FAKE, ws=FAKE,
             ws_bytes=1 << 24, s=None)
    a.update(kw)
    return pq.lib().pq_rotate_quant_for_gemm(a["x"], a["ldx"], a["M"], a["K"], a["P"], a["rec"], a["cs"],
                                             a["A"], a["asg"], a["rs"], a["ws"], a["ws_bytes"], a["s"])


def test_rotate_quant_for_gemm_validation():
    L = pq.lib()
    assert _rq_ws(M=0, x=None, A=None, ws=None, ws_bytes=0) == 0
    # the prologue's own checks, at a prefill M and in the decode band
    for M in (4, 32):
        assert _rq_ws(M=M, K=200) == -2 and _rq_ws(M=M, ldx=128) == -2 and _rq_ws(M=M, P=4) == -4
        assert _rq_ws(M=M, x=None) == -1 and _rq_ws(M=M, x=ctypes.c_void_p(0x100002)) == -3
    # the workspace: required above the decode band, sized as pq_gemm's, 16-byte aligned
    need = L.pq_gemm_workspace_bytes(32, 0, 256)
    assert need > 0
    assert _rq_ws(ws=None) == -1
    assert _rq_ws(ws_bytes=need - 1) == -6
    assert _rq_ws(ws=ctypes.c_void_p(0x100008)) == -3
    assert pq.lib().pq_last_error().decode().startswith("pq_rotate_quant_for_gemm")
    # M * K past the prefill GEMM's 32-bit offsets fails before any launch
    assert _rq_ws(M=300000, K=8192, ldx=8192, ws_bytes=1 << 40) == -2
    assert "too large" in L.pq_last_error().decode()


def test_gemm_prepared_validation():
    name = "pq_gemm_prepared"
    assert _gemm_variant(name, M=0, a=None, y=None) == 0
    assert _gemm_variant(name, K=100) == -2 and _gemm_variant(name, N=120) == -2
    assert _gemm_variant(name, P=2) == -4 and _gemm_variant(name, a=None) == -1
    assert _gemm_variant(name, M=32, ws=None, ws_bytes=1 << 20) == -1
    assert _gemm_variant(name, M=32, ws_bytes=pq.gemm_workspace_bytes(32, 128, 256) - 1) == -6
    assert _gemm_variant(name, M=300000, K=8192, ws_bytes=1 << 40) == -2
    assert pq.lib().pq_last_error().decode().startswith(name)
