// W4A8 group GEMM for gfx950: weight packing, the decode kernel (M <= 16) and the prefill
// kernel, all on the fp8 matrix cores (v_mfma_f32_16x16x128_f8f6f4).
//
// Method ("ParoQuant (PARO) W4A8 on gfx1201 — engineering log", section "Design" items 1, 2
// and 4): per 128-group g the weight value is sc * (c - zp) with (c - zp) = (c - 8) - d,
// d = zp - 8, so
//     y[m,n] = sum_g asg[m,g] * ( sc * sum_k D(a_k) (c_k - 8) - fl16(sc*d) * rs[m,g] ),
// with rs the code-domain row-sum the prologue emits and SZ = {sc, fl16(sc*d)} interleaved.
//
// gfx950 operand choice (this library's, not the page's): the matrix core takes the raw
// 4-bit code c as an OCP e4m3 byte. Codes 0x00..0x0F are exactly c * 2^-9 (subnormals, then
// the first normal binade), and the MFMA handles e4m3 subnormals exactly, so unpacking a
// nibble is a mask — no lookup table. The MFMA then returns T = 2^-9 * sum_k D(a_k) c_k and
//     sc * sum_k D(a_k)(c_k - 8) - zsc * rs = (512 sc) * T - (8 sc + zsc) * rs,
// both factors exact in fp32 (512 sc is a power-of-two scaling, 8 sc + zsc needs < 24 bits).
//
// Packed weight layout (pq_pack_weights): for each 16-column tile t and group g, 1 KiB at
// ((t * G + g) * 1024): lane l (column 16t + l%16, k = 128g + 32*(l/16) + 0..31) owns 16 bytes
// = 4 words; byte b of word q holds code(k0 + 8q + b) in its low nibble and code(k0 + 8q + 4 + b)
// in its high nibble. (w & 0x0F0F0F0F) and ((w >> 4) & 0x0F0F0F0F) are then the lane's B
// operand registers 2q and 2q+1, matching the A operand's 32 consecutive k bytes.
#include "pq_device.h"
#include "pq_internal.h"

namespace pq {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ v4f mfma_fp8(const v8i& a, const v8i& b) {
  const v4f zero = {0.f, 0.f, 0.f, 0.f};
  // format 0 = OCP e4m3 for both operands; scale operands 0 select the unscaled instruction
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, zero, 0, 0, 0, 0, 0, 0);
}

__device__ __forceinline__ v8i unpack_codes(const u32x4& w) {
  v8i b;
  b[0] = static_cast<int>(w.x & 0x0F0F0F0Fu);
  b[1] = static_cast<int>((w.x >> 4) & 0x0F0F0F0Fu);
  b[2] = static_cast<int>(w.y & 0x0F0F0F0Fu);
  b[3] = static_cast<int>((w.y >> 4) & 0x0F0F0F0Fu);
  b[4] = static_cast<int>(w.z & 0x0F0F0F0Fu);
  b[5] = static_cast<int>((w.z >> 4) & 0x0F0F0F0Fu);
  b[6] = static_cast<int>(w.w & 0x0F0F0F0Fu);
  b[7] = static_cast<int>((w.w >> 4) & 0x0F0F0F0Fu);
  return b;
}

// {512*sc, 8*sc + zsc} from one SZ word (sc in the low half).
__device__ __forceinline__ float2 sz_factors(uint32_t w) {
  const float sc = f16_to_f32(w), zsc = f16_to_f32(w >> 16);
  return make_float2(sc * 512.0f, __builtin_fmaf(sc, 8.0f, zsc));
}

// column n -> nibble position inside its AWQ word (inverse of the order 0,2,4,6,1,3,5,7)
__device__ __forceinline__ int awq_shift(int n) {
  const int c = n & 7;
  return 4 * ((c >> 1) + ((c & 1) << 2));
}

// ---------------------------------------------------------------------------------------
// packing
__global__ void pack_weights_kernel(const int32_t* __restrict__ qweight, int K, int N,
                                    uint32_t* __restrict__ wpk) {
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  const int64_t total = static_cast<int64_t>(K) * N / 8;
  if (idx >= total) return;
  const int G = K >> 7;
  const int q = static_cast<int>(idx & 3);
  const int l = static_cast<int>((idx >> 2) & 63);
  const int64_t rest = idx >> 8;
  const int g = static_cast<int>(rest % G);
  const int t = static_cast<int>(rest / G);
  const int n = 16 * t + (l & 15);
  const int k0 = 128 * g + 32 * (l >> 4) + 8 * q;
  const int shift = awq_shift(n);
  const int64_t N8 = N / 8;
  uint32_t w = 0;
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    const uint32_t lo = (static_cast<uint32_t>(qweight[(k0 + b) * N8 + n / 8]) >> shift) & 0xFu;
    const uint32_t hi = (static_cast<uint32_t>(qweight[(k0 + 4 + b) * N8 + n / 8]) >> shift) & 0xFu;
    w |= (lo | (hi << 4)) << (8 * b);
  }
  wpk[idx] = w;
}

__global__ void pack_sz_kernel(const int32_t* __restrict__ qzeros, const uint16_t* __restrict__ scales,
                               int G, int N, uint32_t* __restrict__ sz) {
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (idx >= static_cast<int64_t>(G) * N) return;
  const int g = static_cast<int>(idx / N), n = static_cast<int>(idx % N);
  const uint32_t zp = (static_cast<uint32_t>(qzeros[static_cast<int64_t>(g) * (N / 8) + n / 8]) >> awq_shift(n)) & 0xFu;
  const uint16_t sc = scales[idx];
  // sc * (zp - 8) is exact in fp32 (11 x 4 significand bits); one rounding to f16
  const _Float16 zsc = static_cast<_Float16>(f16_to_f32(sc) * static_cast<float>(static_cast<int>(zp) - 8));
  sz[idx] = static_cast<uint32_t>(sc) | (static_cast<uint32_t>(__builtin_bit_cast(uint16_t, zsc)) << 16);
}

// ---------------------------------------------------------------------------------------
// decode: M <= 16. One workgroup per 16*NT columns; its WV waves split the groups and their
// partial sums meet in LDS. Each wave streams NT x 1 KiB of packed weights per group.
template <int NT, int WV>
__global__ __launch_bounds__(64 * WV) void gemm_decode_kernel(
    const uint8_t* __restrict__ A, const float* __restrict__ ASG, const float* __restrict__ RS,
    int M, int K, const u32x4* __restrict__ wpk, const uint32_t* __restrict__ sz, int N,
    int pb1, int pb2, uint16_t* __restrict__ y, int64_t ldy) {
  const int G = K >> 7;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int col = lane & 15, kq = lane >> 4;
  const int n0 = blockIdx.x * (16 * NT);
  const int p = (n0 >= pb1) + (n0 >= pb2);
  const int g0 = (G * wave) / WV, g1 = (G * (wave + 1)) / WV;

  const bool arow = col < M;  // A operand row = lane % 16
  const uint8_t* Ap = A + (static_cast<size_t>(p) * M + (arow ? col : 0)) * K + 32 * kq;
  const float* asgp = ASG + static_cast<size_t>(p) * M * G;
  const float* rsp = RS + static_cast<size_t>(p) * M * G;
  const u32x4* wp = wpk + static_cast<size_t>(n0 / 16) * G * 64 + lane;

  v4f acc[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) acc[t] = v4f{0.f, 0.f, 0.f, 0.f};

  for (int g = g0; g < g1; ++g) {
    u32x4 bw[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) bw[t] = __builtin_nontemporal_load(wp + (static_cast<size_t>(t) * G + g) * 64);
    v8i a = {0, 0, 0, 0, 0, 0, 0, 0};
    if (arow) {
      const uint4 a0 = *reinterpret_cast<const uint4*>(Ap + 128 * g);
      const uint4 a1 = *reinterpret_cast<const uint4*>(Ap + 128 * g + 16);
      a = v8i{(int)a0.x, (int)a0.y, (int)a0.z, (int)a0.w, (int)a1.x, (int)a1.y, (int)a1.z, (int)a1.w};
    }
    float as[4], rs[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = 4 * kq + i;
      as[i] = (m < M) ? asgp[static_cast<size_t>(m) * G + g] : 0.f;
      rs[i] = (m < M) ? rsp[static_cast<size_t>(m) * G + g] : 0.f;
    }
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const float2 f = sz_factors(sz[static_cast<size_t>(g) * N + n0 + 16 * t + col]);
      const v4f T = mfma_fp8(a, unpack_codes(bw[t]));
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[t][i] += as[i] * (f.x * T[i] - f.y * rs[i]);
    }
  }

  __shared__ float sred[WV][16][16 * NT];
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int i = 0; i < 4; ++i) sred[wave][4 * kq + i][16 * t + col] = acc[t][i];
  __syncthreads();
  const int outs = M * 16 * NT;
  for (int idx = threadIdx.x; idx < outs; idx += 64 * WV) {
    const int m = idx / (16 * NT), c = idx % (16 * NT);
    float s = 0.f;
#pragma unroll
    for (int w = 0; w < WV; ++w) s += sred[w][m][c];
    y[static_cast<size_t>(m) * ldy + n0 + c] = static_cast<uint16_t>(f32_to_bf16(s));
  }
}

// ---------------------------------------------------------------------------------------
// prefill: 128x128 output tile per 256-thread workgroup, 2x2 waves of 64x64, one 128-group
// per k-step, operands staged in LDS in fragment order (double buffered).
constexpr int kPBM = 128, kPBN = 128;

__global__ __launch_bounds__(256) void gemm_prefill_kernel(
    const uint8_t* __restrict__ A, const float* __restrict__ ASG, const float* __restrict__ RS,
    int M, int K, const u32x4* __restrict__ wpk, const uint32_t* __restrict__ sz, int N,
    int pb1, int pb2, uint16_t* __restrict__ y, int64_t ldy) {
  const int G = K >> 7;
  const int tiles_n = (N + kPBN - 1) / kPBN;
  const int tm = blockIdx.x / tiles_n, tn = blockIdx.x % tiles_n;
  const int m0 = tm * kPBM, n0 = tn * kPBN;
  const int p = (n0 >= pb1) + (n0 >= pb2);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int col = lane & 15, kq = lane >> 4;

  __shared__ __attribute__((aligned(16))) uint8_t sA[2][kPBM / 16][64 * 32];  // 2 x 16 KiB
  __shared__ __attribute__((aligned(16))) u32x4 sB[2][kPBN / 16][64];         // 2 x 8 KiB
  __shared__ __attribute__((aligned(16))) float sAsg[2][kPBM];
  __shared__ __attribute__((aligned(16))) float sRs[2][kPBM];
  __shared__ __attribute__((aligned(16))) uint32_t sSz[2][kPBN];

  const uint8_t* Ab = A + static_cast<size_t>(p) * M * K;
  const float* asgp = ASG + static_cast<size_t>(p) * M * G;
  const float* rsp = RS + static_cast<size_t>(p) * M * G;

  // global -> register staging for one group
  uint4 ra[4];
  u32x4 rb[2];
  float rscal;
  uint32_t rsz;
  auto load_group = [&](int g) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int c = tid + 256 * j;          // 16-byte chunk 0..1023 of the 128x128 A tile
      const int r = c >> 3, part = c & 7;
      const int m = m0 + r;
      ra[j] = (m < M) ? *reinterpret_cast<const uint4*>(Ab + static_cast<size_t>(m) * K + 128 * g + 16 * part)
                      : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int c = tid + 256 * j;          // 16-byte chunk 0..511 of the 8 fragments
      const int f = c >> 6, l = c & 63;
      const int n = n0 + 16 * f;
      rb[j] = (n < N) ? wpk[(static_cast<size_t>(n / 16) * G + g) * 64 + l] : u32x4{0u, 0u, 0u, 0u};
    }
    {
      const int r = tid & 127, m = m0 + r;
      const float* src = (tid < 128) ? asgp : rsp;
      rscal = (m < M) ? src[static_cast<size_t>(m) * G + g] : 0.f;
      const int n = n0 + (tid & 127);
      rsz = (tid < 128 && n < N) ? sz[static_cast<size_t>(g) * N + n] : 0u;
    }
  };
  auto store_group = [&](int buf) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int c = tid + 256 * j;
      const int r = c >> 3, part = c & 7;
      const int mf = r >> 4, fl = (r & 15) + 16 * (part >> 1);
      *reinterpret_cast<uint4*>(&sA[buf][mf][fl * 32 + 16 * (part & 1)]) = ra[j];
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int c = tid + 256 * j;
      sB[buf][c >> 6][c & 63] = rb[j];
    }
    if (tid < 128) { sAsg[buf][tid] = rscal; sSz[buf][tid] = rsz; }
    else sRs[buf][tid - 128] = rscal;
  };

  v4f acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

  load_group(0);
  store_group(0);
  __syncthreads();
  for (int g = 0; g < G; ++g) {
    const int buf = g & 1;
    if (g + 1 < G) load_group(g + 1);
    // B fragments and their scale factors
    v8i bf[4];
    float2 fz[4];
#pragma unroll
    for (int nf = 0; nf < 4; ++nf) {
      bf[nf] = unpack_codes(sB[buf][wn * 4 + nf][lane]);
      fz[nf] = sz_factors(sSz[buf][wn * 64 + 16 * nf + col]);
    }
#pragma unroll
    for (int mf = 0; mf < 4; ++mf) {
      const uint4* ap = reinterpret_cast<const uint4*>(&sA[buf][wm * 4 + mf][lane * 32]);
      const uint4 a0 = ap[0], a1 = ap[1];
      const v8i a = v8i{(int)a0.x, (int)a0.y, (int)a0.z, (int)a0.w, (int)a1.x, (int)a1.y, (int)a1.z, (int)a1.w};
      const float4 as = *reinterpret_cast<const float4*>(&sAsg[buf][wm * 64 + 16 * mf + 4 * kq]);
      const float4 rs = *reinterpret_cast<const float4*>(&sRs[buf][wm * 64 + 16 * mf + 4 * kq]);
#pragma unroll
      for (int nf = 0; nf < 4; ++nf) {
        const v4f T = mfma_fp8(a, bf[nf]);
        acc[mf][nf][0] += as.x * (fz[nf].x * T[0] - fz[nf].y * rs.x);
        acc[mf][nf][1] += as.y * (fz[nf].x * T[1] - fz[nf].y * rs.y);
        acc[mf][nf][2] += as.z * (fz[nf].x * T[2] - fz[nf].y * rs.z);
        acc[mf][nf][3] += as.w * (fz[nf].x * T[3] - fz[nf].y * rs.w);
      }
    }
    if (g + 1 < G) store_group(buf ^ 1);
    __syncthreads();
  }

#pragma unroll
  for (int mf = 0; mf < 4; ++mf)
#pragma unroll
    for (int nf = 0; nf < 4; ++nf) {
      const int n = n0 + wn * 64 + 16 * nf + col;
      if (n >= N) continue;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int m = m0 + wm * 64 + 16 * mf + 4 * kq + i;
        if (m < M) y[static_cast<size_t>(m) * ldy + n] = static_cast<uint16_t>(f32_to_bf16(acc[mf][nf][i]));
      }
    }
}

static int launch_status(const char* what) {
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return set_error(PQ_ERR_DEVICE, "%s: launch failed: %s", what, hipGetErrorString(e));
  return PQ_OK;
}

}  // namespace pq

extern "C" {

size_t pq_packed_weight_bytes(int K, int N) {
  if (K <= 0 || N <= 0) return 0;
  return static_cast<size_t>(K) * static_cast<size_t>(N) / 2;
}

int pq_pack_weights(const int32_t* qweight_d, const int32_t* qzeros_d, const uint16_t* scales_d,
                    int K, int N, void* wpk_d, uint16_t* sz_d, pq_stream_t stream) {
  using namespace pq;
  clear_error();
  if (K <= 0 || K % PQ_GROUP || K > (1 << 24)) return set_error(PQ_ERR_SHAPE, "pq_pack_weights: K=%d must be a positive multiple of 128", K);
  if (N <= 0 || N % 16 || N > (1 << 24)) return set_error(PQ_ERR_SHAPE, "pq_pack_weights: N=%d must be a positive multiple of 16", N);
  if (!qweight_d || !qzeros_d || !scales_d || !wpk_d || !sz_d) return set_error(PQ_ERR_NULL, "pq_pack_weights: NULL pointer");
  if (!aligned(qweight_d, 4) || !aligned(qzeros_d, 4) || !aligned(scales_d, 2) || !aligned(wpk_d, 16) || !aligned(sz_d, 4))
    return set_error(PQ_ERR_ALIGN, "pq_pack_weights: misaligned pointer");
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const int64_t words = static_cast<int64_t>(K) * N / 8;
  hipLaunchKernelGGL(pack_weights_kernel, dim3(static_cast<unsigned>((words + 255) / 256)), dim3(256), 0, s,
                     qweight_d, K, N, static_cast<uint32_t*>(wpk_d));
  const int64_t gn = static_cast<int64_t>(K / PQ_GROUP) * N;
  hipLaunchKernelGGL(pack_sz_kernel, dim3(static_cast<unsigned>((gn + 255) / 256)), dim3(256), 0, s,
                     qzeros_d, scales_d, K / PQ_GROUP, N, reinterpret_cast<uint32_t*>(sz_d));
  return launch_status("pq_pack_weights");
}

size_t pq_gemm_workspace_bytes(int M, int N, int K) {
  (void)M; (void)N; (void)K;
  return 0;
}

int pq_gemm(const uint8_t* a_d, const float* asg_d, const float* rs_d, int M, int K, int P,
            const void* wpk_d, const uint16_t* sz_d, int N, int pb1, int pb2, uint16_t* y_d,
            int64_t ldy, void* ws_d, size_t ws_bytes, pq_stream_t stream) {
  using namespace pq;
  clear_error();
  (void)ws_d;
  if (M < 0) return set_error(PQ_ERR_SHAPE, "pq_gemm: M=%d < 0", M);
  if (K <= 0 || K % PQ_GROUP || K > (1 << 24)) return set_error(PQ_ERR_SHAPE, "pq_gemm: K=%d must be a positive multiple of 128", K);
  if (N <= 0 || N % 16 || N > (1 << 24)) return set_error(PQ_ERR_SHAPE, "pq_gemm: N=%d must be a positive multiple of 16", N);
  if (ldy < N || (ldy & 1)) return set_error(PQ_ERR_SHAPE, "pq_gemm: ldy=%lld must be even and >= N=%d", static_cast<long long>(ldy), N);
  const int perr = check_partitions(P, pb1, pb2, N);
  if (perr != PQ_OK) return perr;
  if (ws_bytes < pq_gemm_workspace_bytes(M, N, K)) return set_error(PQ_ERR_WORKSPACE, "pq_gemm: workspace too small");
  if (M == 0) return PQ_OK;
  if (!a_d || !asg_d || !rs_d || !wpk_d || !sz_d || !y_d) return set_error(PQ_ERR_NULL, "pq_gemm: NULL pointer");
  if (!aligned(a_d, 16) || !aligned(asg_d, 4) || !aligned(rs_d, 4) || !aligned(wpk_d, 16) || !aligned(sz_d, 4) || !aligned(y_d, 4))
    return set_error(PQ_ERR_ALIGN, "pq_gemm: misaligned pointer");
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const u32x4* wpk = static_cast<const u32x4*>(wpk_d);
  const uint32_t* sz = reinterpret_cast<const uint32_t*>(sz_d);
  if (M <= 16) {
    if (N % 64 == 0) {
      hipLaunchKernelGGL((gemm_decode_kernel<4, 8>), dim3(N / 64), dim3(512), 0, s,
                         a_d, asg_d, rs_d, M, K, wpk, sz, N, pb1, pb2, y_d, ldy);
    } else {
      hipLaunchKernelGGL((gemm_decode_kernel<1, 8>), dim3(N / 16), dim3(512), 0, s,
                         a_d, asg_d, rs_d, M, K, wpk, sz, N, pb1, pb2, y_d, ldy);
    }
    return launch_status("pq_gemm(decode)");
  }
  const int64_t tiles = static_cast<int64_t>((M + kPBM - 1) / kPBM) * ((N + kPBN - 1) / kPBN);
  if (tiles > 0x7FFFFFFF) return set_error(PQ_ERR_SHAPE, "pq_gemm: problem too large");
  hipLaunchKernelGGL(gemm_prefill_kernel, dim3(static_cast<unsigned>(tiles)), dim3(256), 0, s,
                     a_d, asg_d, rs_d, M, K, wpk, sz, N, pb1, pb2, y_d, ldy);
  return launch_status("pq_gemm(prefill)");
}

}  // extern "C"
