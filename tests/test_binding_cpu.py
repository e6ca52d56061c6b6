"""CPU tests of the Python binding's argument checks: the C ABI sees no buffer lengths, so every
wrapper checks each tensor's dtype and shape against (P, M, K, N) before calling the library. Each
case below gets one tensor wrong and must raise ValueError (TypeError for a wrong dtype) without
reaching the library; with every shape right the CPU tensors are then refused as not on the GPU,
which shows the shape checks ran first. No GPU is used."""
import pytest
import torch

import rotated_w4a8_group_amd as pq

P, M, K, N = 2, 6, 256, 128
G = K // 128
u8, i8, i32, f16, f32, bf16 = torch.uint8, torch.int8, torch.int32, torch.float16, torch.float32, torch.bfloat16


def t(shape, dtype):
    return torch.zeros(shape, dtype=dtype)


def gemm_args(**kw):
    a = dict(A=t((P, M, K), u8), S=t((P, M, G), f32), R=t((P, M, G), f32),
             wpk=t(pq.lib().pq_packed_weight_bytes(K, N), u8), sz=t((G, N, 2), f16), N=N,
             pb1=64 * 2, pb2=pq.NO_BOUNDARY, out=None, workspace=None)
    a.update(kw)
    return a


def call_gemm(fn=pq.gemm, **kw):
    a = gemm_args(**kw)
    return fn(a["A"], a["S"], a["R"], a["wpk"], a["sz"], a["N"], a["pb1"], a["pb2"], out=a["out"],
              workspace=a["workspace"])


@pytest.mark.parametrize("kw", [
    dict(S=t((P, M, G + 1), f32)), dict(S=t((1, M, G), f32)), dict(R=t((P, M - 1, G), f32)),
    dict(wpk=t(pq.lib().pq_packed_weight_bytes(K, N) - 1, u8)), dict(sz=t((G, N, 1), f16)),
    dict(sz=t((G, 2 * N, 2), f16)), dict(N=120), dict(A=t((M, K), u8)), dict(A=t((P, M, 200), u8)),
    dict(out=t((M - 1, N), bf16)), dict(out=t((M, N - 2), bf16)), dict(out=t((M, 2 * N), bf16)[:, ::2]),
    dict(workspace=t(1, u8), A=t((P, 64, K), u8), S=t((P, 64, G), f32), R=t((P, 64, G), f32)),
])
def test_gemm_shape_mismatch_raises(kw):
    with pytest.raises(ValueError):
        call_gemm(**kw)


@pytest.mark.parametrize("kw", [dict(A=t((P, M, K), i8)), dict(S=t((P, M, G), f16)), dict(sz=t((G, N, 2), bf16))])
def test_gemm_dtype_mismatch_raises(kw):
    with pytest.raises(TypeError):
        call_gemm(**kw)


def test_gemm_all_shapes_right_refuses_cpu_tensors():
    with pytest.raises(TypeError, match="CUDA"):
        call_gemm()
    with pytest.raises(TypeError, match="CUDA"):
        call_gemm(out=t((M, N + 8), bf16))


def test_gemm_variants_check_their_own_shapes():
    with pytest.raises(ValueError):      # the token path takes AS [P, M]
        call_gemm(pq.gemm_tok, S=t((P, M, G), f32))
    with pytest.raises(TypeError, match="CUDA"):
        call_gemm(pq.gemm_tok, S=t((P, M), f32))
    with pytest.raises(TypeError):       # int8 codes
        call_gemm(pq.gemm_i8)
    with pytest.raises(TypeError, match="CUDA"):
        call_gemm(pq.gemm_i8, A=t((P, M, K), i8))
    n5 = pq.lib().pq_packed_weight5_bytes(K, N)
    with pytest.raises(ValueError):      # the int4 image is too short for int5 weights
        call_gemm(pq.gemm5)
    with pytest.raises(TypeError, match="CUDA"):
        call_gemm(pq.gemm5, wpk=t(n5, u8))
    with pytest.raises(ValueError):      # int5 needs N % 32
        call_gemm(pq.gemm5, N=112, sz=t((G, 112, 2), f16), wpk=t(n5, u8))


def rq_args(**kw):
    a = dict(x=t((M, K), f16), rec=t((P, 8, K // 2, 8), u8), cs=t((P, K), f16), out=None)
    a.update(kw)
    return a


@pytest.mark.parametrize("fn", [pq.rotate_quant, pq.rotate_quant_i8, pq.rotate_quant_tok])
@pytest.mark.parametrize("kw", [
    dict(rec=t((P, 8, K // 2 - 1, 8), u8)), dict(rec=t((P + 1, 8, K // 2, 8), u8)), dict(rec=t((8, K // 2, 8), u8)),
    dict(cs=t((P, K + 128), f16)), dict(cs=t((4, K), f16)), dict(x=t((M, 200), f16)), dict(x=t((M, K, 1), f16)),
    dict(x=t((M, 2 * K), f16)[:, ::2]),
])
def test_prologue_shape_mismatch_raises(fn, kw):
    a = rq_args(**kw)
    with pytest.raises(ValueError):
        fn(a["x"], a["rec"], a["cs"], out=a["out"])


@pytest.mark.parametrize("fn,a_dtype,tok", [(pq.rotate_quant, u8, False), (pq.rotate_quant_i8, i8, False),
                                            (pq.rotate_quant_tok, u8, True)])
def test_prologue_output_shapes_checked(fn, a_dtype, tok):
    a = rq_args()
    s_shape = (P, M) if tok else (P, M, G)
    good = (t((P, M, K), a_dtype), t(s_shape, f32), t((P, M, G), f32))
    for i, bad in enumerate((t((P, M, K - 1), a_dtype), t((P, M + 1) if tok else (P, M, G + 1), f32), t((P, M, 1), f32))):
        out = list(good)
        out[i] = bad
        with pytest.raises(ValueError):
            fn(a["x"], a["rec"], a["cs"], out=tuple(out))
    with pytest.raises(TypeError, match="CUDA"):
        fn(a["x"], a["rec"], a["cs"], out=good)


def test_producer_shapes_checked():
    x, r, w = t((M, K), f16), t((M, K), f16), t(K, f16)
    rec, cs = t((P, 8, K // 2, 8), u8), t((P, K), f16)
    with pytest.raises(ValueError):
        pq.add_rms_rotate_quant(x, t((M + 1, K), f16), w, 1e-6, rec, cs)
    with pytest.raises(ValueError):
        pq.add_rms_rotate_quant(x, r, t(K - 8, f16), 1e-6, rec, cs)
    with pytest.raises(ValueError):
        pq.add_rms_rotate_quant(x, r, w, 1e-6, rec, cs, residual_out=t((M, K - 128), f16))
    with pytest.raises(ValueError):
        pq.add_rms_rotate_quant(x, r, w, 1e-6, rec, cs,
                                out=(t((M, K), f16), t((P, M, K), u8), t((P, M, G), f32), t((P, M, 1), f32)))
    with pytest.raises(ValueError):
        pq.add_rms_rotate_quant(x, r, w, 1e-6, t((P, 8, 4, 8), u8), cs)
    with pytest.raises(TypeError, match="CUDA"):
        pq.add_rms_rotate_quant(x, r, w, 1e-6, rec, cs)


def test_pack_shapes_checked():
    qw, qz, sc = t((K, N // 8), i32), t((G, N // 8), i32), t((G, N), f16)
    with pytest.raises(ValueError):
        pq.pack_weights(qw, t((G + 1, N // 8), i32), sc)
    with pytest.raises(ValueError):
        pq.pack_weights(qw, qz, t((G, N - 8), f16))
    with pytest.raises(ValueError):
        pq.pack_weights(t((K + 8, N // 8), i32), qz, sc)
    with pytest.raises(TypeError, match="CUDA"):
        pq.pack_weights(qw, qz, sc)
    qwh, qzh = t((K, N // 32), i32), t((G, N // 32), i32)
    with pytest.raises(ValueError):
        pq.pack_weights5(qw, t((K, N // 16), i32), qz, qzh, sc)
    with pytest.raises(ValueError):
        pq.pack_weights5(qw, qwh, qz, t((G + 1, N // 32), i32), sc)
    with pytest.raises(TypeError, match="CUDA"):
        pq.pack_weights5(qw, qwh, qz, qzh, sc)


def test_prepared_pair_checks_the_workspace():
    """rotate_quant_for_gemm / gemm_prepared: the workspace is required above the decode band
    (M > 16) and checked against gemm_workspace_bytes; the other arguments as rotate_quant / gemm."""
    Mp = 64
    x, rec, cs = t((Mp, K), f16), t((P, 8, K // 2, 8), u8), t((P, K), f16)
    need = pq.gemm_workspace_bytes(Mp, N, K)
    assert need > 0
    with pytest.raises(ValueError):
        pq.rotate_quant_for_gemm(x, rec, cs, None)
    with pytest.raises(ValueError):
        pq.rotate_quant_for_gemm(x, rec, cs, t(need - 1, u8))
    with pytest.raises(ValueError):
        pq.rotate_quant_for_gemm(t((Mp, 200), f16), rec, cs, t(need, u8))
    with pytest.raises(TypeError, match="CUDA"):
        pq.rotate_quant_for_gemm(x, rec, cs, t(need, u8))
    with pytest.raises(TypeError, match="CUDA"):     # decode band: no workspace needed
        pq.rotate_quant_for_gemm(t((M, K), f16), rec, cs, None)
    big = dict(A=t((P, Mp, K), u8), S=t((P, Mp, G), f32), R=t((P, Mp, G), f32))
    with pytest.raises(ValueError):                  # a fresh workspace would hold no operands
        call_gemm(pq.gemm_prepared, **big)
    with pytest.raises(ValueError):
        call_gemm(pq.gemm_prepared, workspace=t(need - 1, u8), **big)
    with pytest.raises(ValueError):
        call_gemm(pq.gemm_prepared, sz=t((G, N, 1), f16), workspace=t(need, u8), **big)
    with pytest.raises(TypeError, match="CUDA"):
        call_gemm(pq.gemm_prepared, workspace=t(need, u8), **big)
