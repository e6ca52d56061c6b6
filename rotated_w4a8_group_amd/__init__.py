"""PARO W4A8 linear hot path on AMD Instinct MI355X (gfx950).

Thin Python binding over the C ABI in ``include/pq.h`` (``libpq.so`` in this directory).
It only marshals arguments: every step of the path runs in the library's HIP kernels.
PyTorch supplies device memory and the current HIP stream. There is no fallback: if the
library is missing or fails to load, every call raises.

Calls (same names as the C entry points, without the ``pq_`` prefix):

* ``build_records(pairs, theta)``            host; numpy int16 [8, K], f16 [8, K/2]
* ``pack_weights(qweight, qzeros, scales)``  device; AWQ tensors -> (wpk, sz)
* ``rotate_quant(x, rec, cs)``               device; -> (A, ASG, RS)
* ``gemm(A, ASG, RS, wpk, sz, N, pb1, pb2)`` device; -> y bf16
* ``e4m3_encode(q)``, ``recip_f32(x)``       device verification hooks
"""
import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libpq.so")

GROUP = 128
LAYERS = 8
NO_BOUNDARY = 0x7FFFFFFF

PQ_OK = 0
ERRORS = {
    -1: "PQ_ERR_NULL", -2: "PQ_ERR_SHAPE", -3: "PQ_ERR_ALIGN", -4: "PQ_ERR_PARTITION",
    -5: "PQ_ERR_RECORDS", -6: "PQ_ERR_WORKSPACE", -7: "PQ_ERR_DEVICE",
}

# name -> (restype, argtypes); keep in step with include/pq.h
_P = ctypes.c_void_p
_I = ctypes.c_int
_I64 = ctypes.c_int64
_SZ = ctypes.c_size_t
SIGNATURES = {
    "pq_abi_version": (_I, []),
    "pq_last_error": (ctypes.c_char_p, []),
    "pq_build_records": (_I, [_P, _P, _I, _P]),
    "pq_plan_partitions": (_I, [_I, _P, _P, _P, _P, _I, _P, _P, _P]),
    "pq_packed_weight_bytes": (_SZ, [_I, _I]),
    "pq_pack_weights": (_I, [_P, _P, _P, _I, _I, _P, _P, _P]),
    "pq_rotate_quant": (_I, [_P, _I64, _I, _I, _I, _P, _P, _P, _P, _P, _P]),
    "pq_gemm_workspace_bytes": (_SZ, [_I, _I, _I]),
    "pq_gemm": (_I, [_P, _P, _P, _I, _I, _I, _P, _P, _I, _I, _I, _P, _I64, _P, _SZ, _P]),
    "pq_rotate_quant_for_gemm": (_I, [_P, _I64, _I, _I, _I, _P, _P, _P, _P, _P, _P, _SZ, _P]),
    "pq_gemm_prepared": (_I, [_P, _P, _P, _I, _I, _I, _P, _P, _I, _I, _I, _P, _I64, _P, _SZ, _P]),
    "pq_gemm_noalloc_max_scratch_bytes": (_SZ, []),
    "pq_gemm_noalloc": (_I, [_P, _P, _P, _I, _I, _I, _P, _P, _I, _I, _I, _P, _I64, _P]),
    "pq_rotate_quant_tok": (_I, [_P, _I64, _I, _I, _I, _P, _P, _P, _P, _P, _P]),
    "pq_gemm_tok_workspace_bytes": (_SZ, [_I, _I, _I]),
    "pq_gemm_tok": (_I, [_P, _P, _P, _I, _I, _I, _P, _P, _I, _I, _I, _P, _I64, _P, _SZ, _P]),
    "pq_rotate_quant_i8": (_I, [_P, _I64, _I, _I, _I, _P, _P, _P, _P, _P, _P]),
    "pq_gemm_i8": (_I, [_P, _P, _P, _I, _I, _I, _P, _P, _I, _I, _I, _P, _I64, _P, _SZ, _P]),
    "pq_packed_weight5_bytes": (_SZ, [_I, _I]),
    "pq_pack_weights5": (_I, [_P, _P, _P, _P, _P, _I, _I, _P, _P, _P]),
    "pq_gemm5": (_I, [_P, _P, _P, _I, _I, _I, _P, _P, _I, _I, _I, _P, _I64, _P, _SZ, _P]),
    "pq_add_rms_rotate_quant": (_I, [_P, _I64, _P, _I64, _P, ctypes.c_float, _I, _I, _I, _I, _P, _P, _P, _I64,
                                     _P, _P, _P, _P, _P]),
    "pq_e4m3_encode": (_I, [_P, _P, _I64, _P]),
    "pq_recip_f32": (_I, [_P, _P, _I64, _P]),
    "pq_bf16_round": (_I, [_P, _P, _I64, _P]),
}


class PQError(RuntimeError):
    def __init__(self, fn, code, msg):
        super().__init__(f"{fn}: {ERRORS.get(code, code)}: {msg}")
        self.code = code


_lib = None


def lib():
    """The loaded C library (loaded once). Raises if it is not built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: run `python -m rotated_w4a8_group_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def _check(fn, code):
    if code != PQ_OK:
        raise PQError(fn, code, lib().pq_last_error().decode())


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _stream(stream=None):
    import torch
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _nbytes(t):
    """Size in bytes of an optional workspace tensor (0 for None); the library checks it."""
    if t is None:
        return 0
    if not t.is_cuda or not t.is_contiguous():
        raise TypeError("workspace: expected a contiguous CUDA tensor")
    return t.numel() * t.element_size()


def _need(t, dtype, name):
    import torch
    if not isinstance(t, torch.Tensor) or t.dtype != dtype or not t.is_cuda or not t.is_contiguous():
        raise TypeError(f"{name}: expected a contiguous CUDA tensor of {dtype}")


def _validate(specs, rows=()):
    """Checks every argument the C ABI cannot see before anything is called.

    specs: (tensor, name, dtype, shape) for contiguous tensors, where shape is a tuple or an int
    (a minimum number of elements). rows: (tensor, name, dtype, (M, K)) for row-strided 2-D
    tensors (unit column stride). Dtypes and shapes of all of them are checked first (TypeError /
    ValueError), then that each is a CUDA tensor on the first one's device (TypeError), so a
    shape mismatch is reported the same way whatever the devices."""
    import torch
    for t, name, dtype, shape in list(specs) + list(rows):
        if not isinstance(t, torch.Tensor) or t.dtype != dtype:
            raise TypeError(f"{name}: expected a tensor of {dtype}")
    for t, name, dtype, shape in specs:
        if isinstance(shape, tuple):
            if tuple(t.shape) != tuple(int(d) for d in shape):
                raise ValueError(f"{name}: shape {tuple(t.shape)}, expected {tuple(shape)}")
        elif t.numel() < shape:
            raise ValueError(f"{name}: {t.numel()} elements, at least {shape} needed")
    for t, name, dtype, shape in rows:
        if t.dim() != 2 or tuple(t.shape) != tuple(shape) or t.stride(1) != 1:
            raise ValueError(f"{name}: expected a [{shape[0]}, {shape[1]}] tensor with unit column stride, "
                             f"got shape {tuple(t.shape)} strides {t.stride()}")
    devs = set()
    for t, name, dtype, shape in list(specs) + list(rows):
        if not t.is_cuda:
            raise TypeError(f"{name}: expected a CUDA tensor")
        devs.add(t.device)
    if len(devs) > 1:
        raise TypeError(f"tensors on several devices: {sorted(str(d) for d in devs)}")
    for t, name, dtype, shape in specs:
        if not t.is_contiguous():
            raise TypeError(f"{name}: expected a contiguous tensor")


def _partitions(cs, K):
    """P from the channel-scale tensor: [P, K] or [K] (one partition)."""
    if cs.dim() == 2:
        return cs.shape[0]
    if cs.dim() == 1:
        return 1
    raise ValueError(f"cs: expected [P, K] or [K], got shape {tuple(cs.shape)}")


def _prologue_specs(x, rec, cs, K):
    """The inputs every prologue shares: x [M, K] rows, records [P][8][K/2] (8 bytes each),
    channel scales [P, K]; returns (P, specs, rows)."""
    import torch
    if not isinstance(x, torch.Tensor) or x.dim() != 2:
        raise ValueError("x: expected a [M, K] tensor")
    if K <= 0 or K % GROUP:
        raise ValueError(f"x: K={K} must be a positive multiple of {GROUP}")
    P = _partitions(cs, K)
    if not 1 <= P <= 3:
        raise ValueError(f"cs: {P} partitions, expected 1..3")
    rec_shape = (P, LAYERS, K // 2, 8) if rec.dim() == 4 else (LAYERS, K // 2, 8)
    if rec.dim() == 3 and P != 1:
        raise ValueError("rec: a [8, K/2, 8] record set serves one partition only")
    cs_shape = (P, K) if cs.dim() == 2 else (K,)
    return P, [(rec, "rec", torch.uint8, rec_shape), (cs, "cs", torch.float16, cs_shape)]


# ------------------------------------------------------------------------------------------
def build_records(pairs, theta):
    """pairs int16 [8, K], theta f16 [8, K/2] (numpy, host) -> uint8 [8, K/2, 8] records."""
    pairs = np.ascontiguousarray(pairs, dtype=np.int16)
    theta = np.ascontiguousarray(theta, dtype=np.float16)
    K = pairs.shape[1]
    out = np.zeros((LAYERS, K // 2, 8), dtype=np.uint8)
    _check("pq_build_records", lib().pq_build_records(
        pairs.ctypes.data_as(_P), theta.view(np.uint16).ctypes.data_as(_P), K, out.ctypes.data_as(_P)))
    return out


def plan_partitions(projections):
    """projections: list of (ncols, pairs int16 [8, K], theta f16 [8, K/2], cs f16 [K]) in column
    order (numpy, host). Adjacent projections with identical rotation data merge into one
    partition. Returns (P, pb1, pb2, reps): reps[q] is the projection whose rotation partition q
    uses."""
    J = len(projections)
    arrs = [(np.ascontiguousarray(p, dtype=np.int16), np.ascontiguousarray(t, dtype=np.float16).view(np.uint16),
             np.ascontiguousarray(c, dtype=np.float16).view(np.uint16)) for _, p, t, c in projections]
    K = arrs[0][0].shape[1] if J else 0
    for p, t, c in arrs:
        if p.shape != (LAYERS, K) or t.shape != (LAYERS, K // 2) or c.shape != (K,):
            raise ValueError("plan_partitions: every projection needs pairs [8, K], theta [8, K/2], cs [K]")
    ncols = np.array([n for n, *_ in projections], dtype=np.int32)
    ptrs = [(ctypes.c_void_p * J)(*[a[i].ctypes.data for a in arrs]) for i in range(3)]
    P = ctypes.c_int()
    pb = (ctypes.c_int * 2)()
    rep = (ctypes.c_int * 3)()
    _check("pq_plan_partitions", lib().pq_plan_partitions(
        J, ncols.ctypes.data_as(_P), ptrs[0], ptrs[1], ptrs[2], K, ctypes.byref(P), pb, rep))
    return P.value, pb[0], pb[1], [r for r in rep[:P.value]]


def pack_weights(qweight, qzeros, scales, stream=None):
    """AWQ qweight int32 [K, N/8], qzeros int32 [K/128, N/8], scales f16 [K/128, N] (CUDA)
    -> (wpk uint8 [K*N/2], sz f16 [K/128, N, 2])."""
    import torch
    if not isinstance(qweight, torch.Tensor) or qweight.dim() != 2:
        raise ValueError("qweight: expected an int32 [K, N/8] tensor")
    K, N = qweight.shape[0], qweight.shape[1] * 8
    if K % GROUP or N % 16 or K == 0:
        raise ValueError(f"qweight: K={K} must be a multiple of {GROUP} and N={N} of 16")
    _validate([(qweight, "qweight", torch.int32, (K, N // 8)), (qzeros, "qzeros", torch.int32, (K // GROUP, N // 8)),
               (scales, "scales", torch.float16, (K // GROUP, N))])
    wpk = torch.empty(lib().pq_packed_weight_bytes(K, N), dtype=torch.uint8, device=qweight.device)
    sz = torch.empty((K // GROUP, N, 2), dtype=torch.float16, device=qweight.device)
    _check("pq_pack_weights", lib().pq_pack_weights(
        _ptr(qweight), _ptr(qzeros), _ptr(scales), K, N, _ptr(wpk), _ptr(sz), _stream(stream)))
    return wpk, sz


def pack_weights5(qweight, qweight_hi, qzeros, qzeros_hi, scales, stream=None):
    """int5 bit-plane weights: qweight int32 [K, N/8], qweight_hi int32 [K, N/32], qzeros int32
    [K/128, N/8], qzeros_hi int32 [K/128, N/32], scales f16 [K/128, N] (CUDA)
    -> (wpk5 uint8 [pq_packed_weight5_bytes], sz f16 [K/128, N, 2])."""
    import torch
    if not isinstance(qweight, torch.Tensor) or qweight.dim() != 2:
        raise ValueError("qweight: expected an int32 [K, N/8] tensor")
    K, N = qweight.shape[0], qweight.shape[1] * 8
    if K % GROUP or N % 32 or K == 0:
        raise ValueError(f"qweight: K={K} must be a multiple of {GROUP} and N={N} of 32")
    _validate([(qweight, "qweight", torch.int32, (K, N // 8)), (qweight_hi, "qweight_hi", torch.int32, (K, N // 32)),
               (qzeros, "qzeros", torch.int32, (K // GROUP, N // 8)),
               (qzeros_hi, "qzeros_hi", torch.int32, (K // GROUP, N // 32)),
               (scales, "scales", torch.float16, (K // GROUP, N))])
    wpk = torch.empty(max(1, lib().pq_packed_weight5_bytes(K, N)), dtype=torch.uint8, device=qweight.device)
    sz = torch.empty((K // GROUP, N, 2), dtype=torch.float16, device=qweight.device)
    _check("pq_pack_weights5", lib().pq_pack_weights5(
        _ptr(qweight), _ptr(qweight_hi), _ptr(qzeros), _ptr(qzeros_hi), _ptr(scales), K, N,
        _ptr(wpk), _ptr(sz), _stream(stream)))
    return wpk, sz


def _rotate_quant_common(fn, x, rec, cs, out, stream, a_dtype, tok=False, workspace=False):
    """Checks x [M, K], the records and channel scales, and caller-given outputs (codes [P, M, K],
    scales [P, M, G] or [P, M] with tok, row-sums [P, M, G]); allocates missing outputs.
    workspace (pq_rotate_quant_for_gemm): the GEMM workspace tensor the call also fills, checked
    against gemm_workspace_bytes(M, N, K)."""
    import torch
    if not isinstance(x, torch.Tensor) or x.dim() != 2:
        raise ValueError("x: expected a [M, K] tensor")
    M, K = x.shape
    P, specs = _prologue_specs(x, rec, cs, K)
    G = K // GROUP
    s_shape = (P, M) if tok else (P, M, G)
    if out is not None:
        A, S, R = out
        specs += [(A, "A", a_dtype, (P, M, K)), (S, "AS" if tok else "ASG", torch.float32, s_shape),
                  (R, "RS", torch.float32, (P, M, G))]
    if workspace is not False:
        ws_bytes = gemm_workspace_bytes(M, 0, K)
        if workspace is None:
            if ws_bytes:
                raise ValueError(f"workspace: {ws_bytes} bytes needed at M={M}, K={K}")
        else:
            specs.append((workspace, "workspace", torch.uint8, ws_bytes))
    _validate(specs, rows=[(x, "x", torch.float16, (M, K))])
    ws_args = () if workspace is False else (_ptr(workspace), _nbytes(workspace))
    if out is None:
        A = torch.empty((P, M, K), dtype=a_dtype, device=x.device)
        S = torch.empty(s_shape, dtype=torch.float32, device=x.device)
        R = torch.empty((P, M, G), dtype=torch.float32, device=x.device)
    _check(fn, getattr(lib(), fn)(
        _ptr(x), x.stride(0), M, K, P, _ptr(rec), _ptr(cs), _ptr(A), _ptr(S), _ptr(R), *ws_args, _stream(stream)))
    return A, S, R


def rotate_quant(x, rec, cs, out=None, stream=None):
    """x f16 [M, K] (row stride may exceed K), rec uint8 [P, 8, K/2, 8] (or [8, K/2, 8]),
    cs f16 [P, K] (or [K]) -> (A u8 [P, M, K], ASG f32 [P, M, G], RS f32 [P, M, G])."""
    import torch
    return _rotate_quant_common("pq_rotate_quant", x, rec, cs, out, stream, torch.uint8)


def rotate_quant_for_gemm(x, rec, cs, workspace, out=None, stream=None):
    """pq_rotate_quant_for_gemm: ``rotate_quant`` that also writes, when M > 16, the prefill GEMM's
    activation-side operands into ``workspace`` (uint8, gemm_workspace_bytes(M, N, K) bytes; None
    allowed at M <= 16) for a following ``gemm_prepared`` on the returned (A, ASG, RS)."""
    import torch
    return _rotate_quant_common("pq_rotate_quant_for_gemm", x, rec, cs, out, stream, torch.uint8,
                                workspace=workspace)


def gemm_workspace_bytes(M, N, K):
    return int(lib().pq_gemm_workspace_bytes(M, N, K))


def _gemm_common(fn, A, S, RS, wpk, sz, N, pb1, pb2, out, workspace, stream, *, a_dtype, tok=False, w5=False,
                 prepared=False):
    """Checks every tensor against (P, M, K, N), allocates what is missing, calls `fn`."""
    import torch
    if not isinstance(A, torch.Tensor) or A.dim() != 3:
        raise ValueError("A: expected a [P, M, K] tensor")
    P, M, K = A.shape
    if K == 0 or K % GROUP:
        raise ValueError(f"A: K={K} must be a positive multiple of {GROUP}")
    G = K // GROUP
    L = lib()
    need = L.pq_packed_weight5_bytes(K, N) if w5 else L.pq_packed_weight_bytes(K, N)
    if need == 0:
        raise ValueError(f"N={N}: not a shape the library packs (N % {32 if w5 else 16} == 0 needed)")
    specs = [(A, "A", a_dtype, (P, M, K)), (S, "AS" if tok else "ASG", torch.float32, (P, M) if tok else (P, M, G)),
             (RS, "RS", torch.float32, (P, M, G)), (wpk, "wpk5" if w5 else "wpk", torch.uint8, int(need)),
             (sz, "sz", torch.float16, (G, N, 2))]
    ws_bytes = int(L.pq_gemm_tok_workspace_bytes(M, N, K) if tok else L.pq_gemm_workspace_bytes(M, N, K))
    if workspace is not None:
        specs.append((workspace, "workspace", torch.uint8, ws_bytes))
    elif prepared and ws_bytes:
        raise ValueError("workspace: gemm_prepared reads the workspace rotate_quant_for_gemm filled")
    if out is None:
        _validate(specs)
        out = torch.empty((M, N), dtype=torch.bfloat16, device=A.device)
    else:
        if not isinstance(out, torch.Tensor) or out.dim() != 2 or out.shape[0] != M or out.shape[1] < N:
            raise ValueError(f"out: expected a bf16 [{M}, >= {N}] tensor")
        _validate(specs, rows=[(out, "out", torch.bfloat16, (M, out.shape[1]))])
    if workspace is None and ws_bytes:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=A.device)
    _check(fn, getattr(L, fn)(
        _ptr(A), _ptr(S), _ptr(RS), M, K, P, _ptr(wpk), _ptr(sz), N, pb1, pb2,
        _ptr(out), out.stride(0), _ptr(workspace), _nbytes(workspace), _stream(stream)))
    return out


def gemm(A, ASG, RS, wpk, sz, N, pb1=NO_BOUNDARY, pb2=NO_BOUNDARY, out=None, workspace=None, stream=None):
    """A u8 [P, M, K], ASG/RS f32 [P, M, G], packed weights (wpk from pack_weights, sz [G, N, 2])
    -> y bf16 [M, N] (or into ``out``, a bf16 [M, ldy >= N] view with unit column stride)."""
    import torch
    return _gemm_common("pq_gemm", A, ASG, RS, wpk, sz, N, pb1, pb2, out, workspace, stream, a_dtype=torch.uint8)


def gemm_prepared(A, ASG, RS, wpk, sz, N, pb1=NO_BOUNDARY, pb2=NO_BOUNDARY, out=None, workspace=None, stream=None):
    """pq_gemm_prepared: ``gemm`` on the workspace that ``rotate_quant_for_gemm`` filled for this same
    (A, ASG, RS) (required when M > 16; nothing may write it in between)."""
    import torch
    return _gemm_common("pq_gemm_prepared", A, ASG, RS, wpk, sz, N, pb1, pb2, out, workspace, stream,
                        a_dtype=torch.uint8, prepared=True)


def gemm_noalloc(A, ASG, RS, wpk, sz, N, pb1=NO_BOUNDARY, pb2=NO_BOUNDARY, out=None, stream=None):
    """pq_gemm_noalloc: the result of ``gemm`` with the library's own per-device scratch in place of
    a workspace (no device allocation in the call; ``out``, a bf16 [M, ldy >= N] tensor, is
    required). Calls that overlap on one device race on that scratch."""
    import torch
    if out is None:
        raise ValueError("out: gemm_noalloc writes into a caller-given bf16 [M, N] tensor")
    if not isinstance(A, torch.Tensor) or A.dim() != 3:
        raise ValueError("A: expected a [P, M, K] tensor")
    P, M, K = A.shape
    if K == 0 or K % GROUP:
        raise ValueError(f"A: K={K} must be a positive multiple of {GROUP}")
    G = K // GROUP
    need = lib().pq_packed_weight_bytes(K, N)
    if need == 0:
        raise ValueError(f"N={N}: not a shape the library packs (N % 16 == 0 needed)")
    if not isinstance(out, torch.Tensor) or out.dim() != 2 or out.shape[0] != M or out.shape[1] < N:
        raise ValueError(f"out: expected a bf16 [{M}, >= {N}] tensor")
    _validate([(A, "A", torch.uint8, (P, M, K)), (ASG, "ASG", torch.float32, (P, M, G)),
               (RS, "RS", torch.float32, (P, M, G)), (wpk, "wpk", torch.uint8, int(need)),
               (sz, "sz", torch.float16, (G, N, 2))], rows=[(out, "out", torch.bfloat16, (M, out.shape[1]))])
    _check("pq_gemm_noalloc", lib().pq_gemm_noalloc(
        _ptr(A), _ptr(ASG), _ptr(RS), M, K, P, _ptr(wpk), _ptr(sz), N, pb1, pb2, _ptr(out), out.stride(0),
        _stream(stream)))
    return out


def gemm5(A, ASG, RS, wpk5, sz, N, pb1=NO_BOUNDARY, pb2=NO_BOUNDARY, out=None, workspace=None, stream=None):
    """int5 bit-plane weights (from pack_weights5) with the e4m3 prologue's A/ASG/RS -> y bf16 [M, N]."""
    import torch
    return _gemm_common("pq_gemm5", A, ASG, RS, wpk5, sz, N, pb1, pb2, out, workspace, stream,
                        a_dtype=torch.uint8, w5=True)


def add_rms_rotate_quant(x, residual, weight, eps, rec, cs, gemma=True, residual_out=None, out=None, stream=None):
    """Fused producer: x, residual f16 [M, K] (row strides multiples of 8), weight f16 [K], rec
    [P, 8, K/2, 8], cs f16 [P, K] -> (residual_out f16 [M, K] (``residual`` itself may be passed to
    update it in place), hs f16 [M, K], A u8 [P, M, K], ASG f32 [P, M, G], RS f32 [P, M, G])."""
    import torch
    if not isinstance(x, torch.Tensor) or x.dim() != 2:
        raise ValueError("x: expected a [M, K] tensor")
    M, K = x.shape
    P, specs = _prologue_specs(x, rec, cs, K)
    G = K // GROUP
    specs.append((weight, "weight", torch.float16, (K,)))
    rows = [(x, "x", torch.float16, (M, K)), (residual, "residual", torch.float16, (M, K))]
    if residual_out is not None:
        rows.append((residual_out, "residual_out", torch.float16, (M, K)))
    if out is not None:
        hs, A, S, R = out
        specs += [(hs, "hs", torch.float16, (M, K)), (A, "A", torch.uint8, (P, M, K)),
                  (S, "ASG", torch.float32, (P, M, G)), (R, "RS", torch.float32, (P, M, G))]
    _validate(specs, rows=rows)
    if residual_out is None:
        residual_out = torch.empty((M, K), dtype=torch.float16, device=x.device)
    if out is None:
        hs = torch.empty((M, K), dtype=torch.float16, device=x.device)
        A = torch.empty((P, M, K), dtype=torch.uint8, device=x.device)
        S = torch.empty((P, M, G), dtype=torch.float32, device=x.device)
        R = torch.empty((P, M, G), dtype=torch.float32, device=x.device)
    _check("pq_add_rms_rotate_quant", lib().pq_add_rms_rotate_quant(
        _ptr(x), x.stride(0), _ptr(residual), residual.stride(0), _ptr(weight), float(eps), 1 if gemma else 0,
        M, K, P, _ptr(rec), _ptr(cs), _ptr(residual_out), residual_out.stride(0), _ptr(hs), _ptr(A), _ptr(S),
        _ptr(R), _stream(stream)))
    return residual_out, hs, A, S, R


def rotate_quant_i8(x, rec, cs, out=None, stream=None):
    """Per-group int8 mode: x f16 [M, K], rec [P, 8, K/2, 8], cs f16 [P, K] -> (A int8 [P, M, K],
    ASG f32 [P, M, G], RS f32 [P, M, G])."""
    import torch
    return _rotate_quant_common("pq_rotate_quant_i8", x, rec, cs, out, stream, torch.int8)


def gemm_i8(A, ASG, RS, wpk, sz, N, pb1=NO_BOUNDARY, pb2=NO_BOUNDARY, out=None, workspace=None, stream=None):
    """Per-group int8 GEMM: A int8 [P, M, K], ASG/RS f32 [P, M, G], packed weights -> y bf16."""
    import torch
    return _gemm_common("pq_gemm_i8", A, ASG, RS, wpk, sz, N, pb1, pb2, out, workspace, stream, a_dtype=torch.int8)


def rotate_quant_tok(x, rec, cs, out=None, stream=None):
    """Per-token path: x f16 [M, K], rec [P, 8, K/2, 8], cs f16 [P, K] -> (A u8 [P, M, K],
    AS f32 [P, M], RS f32 [P, M, G])."""
    import torch
    return _rotate_quant_common("pq_rotate_quant_tok", x, rec, cs, out, stream, torch.uint8, tok=True)


def gemm_tok_workspace_bytes(M, N, K):
    return int(lib().pq_gemm_tok_workspace_bytes(M, N, K))


def gemm_tok(A, AS, RS, wpk, sz, N, pb1=NO_BOUNDARY, pb2=NO_BOUNDARY, out=None, workspace=None, stream=None):
    """Per-token GEMM: A u8 [P, M, K], AS f32 [P, M], RS f32 [P, M, G], packed weights -> y bf16."""
    import torch
    return _gemm_common("pq_gemm_tok", A, AS, RS, wpk, sz, N, pb1, pb2, out, workspace, stream,
                        a_dtype=torch.uint8, tok=True)


def e4m3_encode(q, stream=None):
    """float32 CUDA tensor -> uint8 codes with the prologue's device encoder."""
    import torch
    _need(q, torch.float32, "q")
    out = torch.empty(q.shape, dtype=torch.uint8, device=q.device)
    _check("pq_e4m3_encode", lib().pq_e4m3_encode(_ptr(q), _ptr(out), q.numel(), _stream(stream)))
    return out


def recip_f32(x, stream=None):
    """float32 CUDA tensor -> 1/x with the prologue's device reciprocal."""
    import torch
    _need(x, torch.float32, "x")
    out = torch.empty_like(x)
    _check("pq_recip_f32", lib().pq_recip_f32(_ptr(x), _ptr(out), x.numel(), _stream(stream)))
    return out


def bf16_round(x, stream=None):
    """float32 CUDA tensor -> int16 tensor of bf16 bit patterns with the GEMM's device rounding."""
    import torch
    _need(x, torch.float32, "x")
    out = torch.empty(x.shape, dtype=torch.int16, device=x.device)
    _check("pq_bf16_round", lib().pq_bf16_round(_ptr(x), _ptr(out), x.numel(), _stream(stream)))
    return out
