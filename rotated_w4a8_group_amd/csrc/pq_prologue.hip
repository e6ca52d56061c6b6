// Rotate-quant prologue for gfx950, and the verification hooks for its arithmetic.
//
// Computes what "ParoQuant (PARO) W4A8 on gfx1201 — engineering log" describes in section
// "Format" (activations times pre-inverted channel scales, rotated forward through layers
// 0..7 inside each 128-channel group) and section "Design" items 2-3 (one e4m3 scale per
// (token, group), fused amax + OCP e4m3 encode + code-domain row-sums), with the scale of
// section "Gates passed" (amax * (1/448.f)).
//
// This translation unit is compiled with -ffp-contract=off: every multiply and add in the
// rotation rounds separately in binary32, which is the arithmetic the results are defined by.
//
// Launch shape: one 256-thread workgroup (4 waves) per (partition, group, token chunk). The
// workgroup stages the 512 records of its (partition, group) in LDS once; each wave then keeps
// its lane's 8 records in registers and processes TOK tokens at a time. A token-group lives
// in the wave as 2 channels per lane; the layers update a 512-byte LDS copy of it in place.
// Record lane order (pq_build_records) makes every one of those reads and writes free of bank
// conflicts. amax and the row-sum are wave reductions.
#include "pq_device.h"
#include "pq_internal.h"

#pragma clang fp contract(off)

namespace pq {

constexpr int kProWaves = 4;
constexpr int kProTok = 4;  // tokens a wave rotates concurrently

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = __builtin_fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

__device__ __forceinline__ int wave_sum(int v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

__device__ __forceinline__ float recip_rn(float a) { return 1.0f / a; }

__global__ __launch_bounds__(256) void rotate_quant_kernel(
    const uint16_t* __restrict__ x, int64_t ldx, int M, int K, int P,
    const uint2* __restrict__ rec, const uint16_t* __restrict__ cs, uint8_t* __restrict__ A,
    float* __restrict__ ASG, float* __restrict__ RS, int tok_per_block) {
  const int G = K >> 7;
  int bid = blockIdx.x;
  const int p = bid % P;
  bid /= P;
  const int g = bid % G;
  const int chunk = bid / G;

  __shared__ uint2 srec[PQ_LAYERS * 64];
  __shared__ float sbuf[kProWaves][kProTok][128];

  const int half = K >> 1;
  for (int t = threadIdx.x; t < PQ_LAYERS * 64; t += blockDim.x) {
    const int r = t >> 6, l = t & 63;
    srec[t] = rec[(static_cast<size_t>(p) * PQ_LAYERS + r) * half + g * 64 + l];
  }
  __syncthreads();

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  float cr[PQ_LAYERS], sr[PQ_LAYERS];
  uint32_t ti[PQ_LAYERS], hi[PQ_LAYERS];
#pragma unroll
  for (int r = 0; r < PQ_LAYERS; ++r) {
    const uint2 q = srec[r * 64 + lane];
    ti[r] = q.x & 0x7Fu;           // channel indices are 0..127
    hi[r] = (q.x >> 8) & 0x7Fu;
    cr[r] = f16_to_f32(q.y);
    sr[r] = f16_to_f32(q.y >> 16);
  }
  const uint32_t csw = *reinterpret_cast<const uint32_t*>(cs + static_cast<size_t>(p) * K + g * 128 + 2 * lane);
  const float cs0 = f16_to_f32(csw), cs1 = f16_to_f32(csw >> 16);

  float* buf = &sbuf[wave][0][0];
  const int m_begin = chunk * tok_per_block;
  const int m_end = min(M, m_begin + tok_per_block);
  const size_t out_base = static_cast<size_t>(p) * M;

  for (int mb = m_begin + wave * kProTok; mb < m_end; mb += kProWaves * kProTok) {
    uint32_t xw[kProTok];
#pragma unroll
    for (int t = 0; t < kProTok; ++t) {
      const int m = mb + t;
      xw[t] = (m < m_end) ? *reinterpret_cast<const uint32_t*>(x + static_cast<size_t>(m) * ldx + g * 128 + 2 * lane) : 0u;
    }
#pragma unroll
    for (int t = 0; t < kProTok; ++t) {
      float2 v;
      v.x = f16_to_f32(xw[t]) * cs0;       // exact: 11 x 11 significand bits
      v.y = f16_to_f32(xw[t] >> 16) * cs1;
      *reinterpret_cast<float2*>(buf + t * 128 + 2 * lane) = v;
    }
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int r = 0; r < PQ_LAYERS; ++r) {
      float a[kProTok], b[kProTok];
#pragma unroll
      for (int t = 0; t < kProTok; ++t) {
        a[t] = buf[t * 128 + ti[r]];
        b[t] = buf[t * 128 + hi[r]];
      }
#pragma unroll
      for (int t = 0; t < kProTok; ++t) {
        const float ca = cr[r] * a[t], sb = sr[r] * b[t];
        const float cb = cr[r] * b[t], sa = sr[r] * a[t];
        buf[t * 128 + ti[r]] = ca + sb;
        buf[t * 128 + hi[r]] = cb - sa;
      }
      __builtin_amdgcn_wave_barrier();
    }
#pragma unroll
    for (int t = 0; t < kProTok; ++t) {
      const int m = mb + t;
      const float2 v = *reinterpret_cast<const float2*>(buf + t * 128 + 2 * lane);
      const float amax = wave_max(__builtin_fmaxf(__builtin_fabsf(v.x), __builtin_fabsf(v.y)));
      const float asg = amax * 0x1.24924ap-9f;   // fl32(1/448) = 0x3B124925
      const float inv = recip_rn(asg);             // 1/0 = inf -> 0*inf = NaN -> code 0
      const uint32_t codes = e4m3_encode2(v.x * inv, v.y * inv);
      const int units = wave_sum(e4m3_units(codes & 0xFFu) + e4m3_units(codes >> 8));
      if (m < m_end) {
        *reinterpret_cast<uint16_t*>(A + (out_base + m) * K + g * 128 + 2 * lane) = static_cast<uint16_t>(codes);
        if (lane == 0) {
          ASG[(out_base + m) * G + g] = asg;
          RS[(out_base + m) * G + g] = static_cast<float>(units) * 0x1p-9f;
        }
      }
    }
    __builtin_amdgcn_wave_barrier();
  }
}

__global__ void e4m3_encode_kernel(const float* __restrict__ q, uint8_t* __restrict__ out, int64_t n) {
  const int64_t i = (static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x) * 2;
  if (i + 1 < n) {
    const uint32_t c = e4m3_encode2(q[i], q[i + 1]);
    *reinterpret_cast<uint16_t*>(out + i) = static_cast<uint16_t>(c);  // i is even: aligned
  } else if (i < n) {
    out[i] = static_cast<uint8_t>(e4m3_encode2(q[i], 0.0f));
  }
}

__global__ void recip_kernel(const float* __restrict__ x, float* __restrict__ y, int64_t n) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i < n) y[i] = recip_rn(x[i]);
}

static int launch_status(const char* what) {
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return set_error(PQ_ERR_DEVICE, "%s: launch failed: %s", what, hipGetErrorString(e));
  return PQ_OK;
}

}  // namespace pq

extern "C" {

int pq_rotate_quant(const uint16_t* x_d, int64_t ldx, int M, int K, int P, const void* rec_d,
                    const uint16_t* cs_d, uint8_t* a_d, float* asg_d, float* rs_d,
                    pq_stream_t stream) {
  using namespace pq;
  clear_error();
  if (M < 0) return set_error(PQ_ERR_SHAPE, "pq_rotate_quant: M=%d < 0", M);
  if (K <= 0 || K % PQ_GROUP || K > (1 << 24)) return set_error(PQ_ERR_SHAPE, "pq_rotate_quant: K=%d must be a positive multiple of 128", K);
  if (P < 1 || P > PQ_MAX_PARTITIONS) return set_error(PQ_ERR_PARTITION, "pq_rotate_quant: P=%d must be in 1..3", P);
  if (ldx < K || (ldx & 1)) return set_error(PQ_ERR_SHAPE, "pq_rotate_quant: ldx=%lld must be even and >= K=%d", static_cast<long long>(ldx), K);
  if (M == 0) return PQ_OK;
  if (!x_d || !rec_d || !cs_d || !a_d || !asg_d || !rs_d) return set_error(PQ_ERR_NULL, "pq_rotate_quant: NULL pointer");
  if (!aligned(x_d, 4) || !aligned(rec_d, 8) || !aligned(cs_d, 4) || !aligned(a_d, 16) || !aligned(asg_d, 4) || !aligned(rs_d, 4))
    return set_error(PQ_ERR_ALIGN, "pq_rotate_quant: misaligned pointer");
  const int G = K / PQ_GROUP;
  // tokens per workgroup: aim for >= ~2048 workgroups, 16..256 tokens each
  const int64_t want = (static_cast<int64_t>(M) * G * P + 2047) / 2048;
  int tok = static_cast<int>(std::min<int64_t>(256, std::max<int64_t>(16, (want + 15) / 16 * 16)));
  const int64_t chunks = (M + tok - 1) / tok;
  const int64_t blocks = chunks * G * P;
  if (blocks > 0x7FFFFFFF) return set_error(PQ_ERR_SHAPE, "pq_rotate_quant: problem too large");
  hipLaunchKernelGGL(rotate_quant_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0,
                     reinterpret_cast<hipStream_t>(stream), x_d, ldx, M, K, P,
                     static_cast<const uint2*>(rec_d), cs_d, a_d, asg_d, rs_d, tok);
  return launch_status("pq_rotate_quant");
}

int pq_e4m3_encode(const float* q_d, uint8_t* codes_d, int64_t n, pq_stream_t stream) {
  using namespace pq;
  clear_error();
  if (n < 0) return set_error(PQ_ERR_SHAPE, "pq_e4m3_encode: n < 0");
  if (n == 0) return PQ_OK;
  if (!q_d || !codes_d) return set_error(PQ_ERR_NULL, "pq_e4m3_encode: NULL pointer");
  if (!aligned(q_d, 4) || !aligned(codes_d, 2)) return set_error(PQ_ERR_ALIGN, "pq_e4m3_encode: misaligned pointer");
  const int64_t threads = (n + 1) / 2;
  const int64_t blocks = (threads + 255) / 256;
  if (blocks > 0x7FFFFFFF) return set_error(PQ_ERR_SHAPE, "pq_e4m3_encode: n too large");
  hipLaunchKernelGGL(e4m3_encode_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0,
                     reinterpret_cast<hipStream_t>(stream), q_d, codes_d, n);
  return launch_status("pq_e4m3_encode");
}

int pq_recip_f32(const float* x_d, float* y_d, int64_t n, pq_stream_t stream) {
  using namespace pq;
  clear_error();
  if (n < 0) return set_error(PQ_ERR_SHAPE, "pq_recip_f32: n < 0");
  if (n == 0) return PQ_OK;
  if (!x_d || !y_d) return set_error(PQ_ERR_NULL, "pq_recip_f32: NULL pointer");
  if (!aligned(x_d, 4) || !aligned(y_d, 4)) return set_error(PQ_ERR_ALIGN, "pq_recip_f32: misaligned pointer");
  const int64_t blocks = (n + 255) / 256;
  if (blocks > 0x7FFFFFFF) return set_error(PQ_ERR_SHAPE, "pq_recip_f32: n too large");
  hipLaunchKernelGGL(recip_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0,
                     reinterpret_cast<hipStream_t>(stream), x_d, y_d, n);
  return launch_status("pq_recip_f32");
}

}  // extern "C"
