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
// Packed weight layout (pq_pack_weights), tile-major so that one column tile's whole K extent
// is one contiguous run: for 16-column tile t and group g, 1 KiB at ((t * G + g) * 1024): lane l (column 16t + l%16, k = 128g + 32*(l/16) + 0..31) owns 16 bytes
// = 4 words; byte b of word q holds code(k0 + 8q + b) in its low nibble and code(k0 + 8q + 4 + b)
// in its high nibble. (w & 0x0F0F0F0F) and ((w >> 4) & 0x0F0F0F0F) are then the lane's B
// operand registers 2q and 2q+1, matching the A operand's 32 consecutive k bytes.
#include <algorithm>

#include "pq_device.h"
#include "pq_internal.h"

namespace pq {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

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
  const int q = static_cast<int>(idx & 3);
  const int l = static_cast<int>((idx >> 2) & 63);
  const int64_t rest = idx >> 8;
  const int G = K >> 7;
  const int t = static_cast<int>(rest / G);
  const int g = static_cast<int>(rest % G);
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
// zero-point epilogue operand (load time). The prefill kernel moves the zero-point term
//   Z[m, n] = sum_g (asg * rs)[m, g] * (8 sc + zsc)[g, n]
// out of its group loop ("zero-point epilogue" of the page) and computes it once per tile as
// a bf16 matrix-core product with split operands: ar = a1 + a2 and zz = z1 + z2 (each piece the
// bf16 rounding of what is left), Z ~= a1 z1 + a1 z2 + a2 z1 (relative error ~2^-16).
// K' = 3G is laid out as [a1 | a1 | a2] x [z1 ; z2 ; z1], padded with zeros to whole chunks of 32.
// Layout per 16-column tile t and chunk c: 1 KiB, lane l (column 16t + l%16) holds the 8 bf16
// at k' = 32c + 8(l/16) + 0..7 — the bf16 16x16x32 B operand.
__host__ __device__ constexpr int zpe_chunks(int G) { return (3 * G + 31) / 32; }

__device__ __forceinline__ float bf16_to_f32(uint32_t h) { return __builtin_bit_cast(float, (h & 0xFFFFu) << 16); }

__global__ void pack_zpe_kernel(const uint32_t* __restrict__ sz, int G, int N, u32x4* __restrict__ zpe) {
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  const int KC = zpe_chunks(G);
  if (idx >= static_cast<int64_t>(N / 16) * KC * 64) return;
  const int l = static_cast<int>(idx & 63);
  const int c = static_cast<int>((idx >> 6) % KC);
  const int t = static_cast<int>((idx >> 6) / KC);
  const int n = 16 * t + (l & 15);
  uint32_t h[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int kp = 32 * c + 8 * (l >> 4) + e;
    uint32_t v = 0;
    if (kp < 3 * G) {
      const int piece = kp / G, g = kp % G;
      const float2 f = sz_factors(sz[static_cast<size_t>(g) * N + n]);
      const uint32_t z1 = f32_to_bf16(f.y);
      v = (piece == 1) ? f32_to_bf16(f.y - bf16_to_f32(z1)) : z1;
    }
    h[e] = v;
  }
  zpe[idx] = u32x4{h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16), h[6] | (h[7] << 16)};
}

// Activation side of the zero-point epilogue, built per GEMM call into the workspace:
// for partition p, 16-row tile mt and chunk c, 1 KiB where lane l (row 16mt + l%16) holds the
// 8 bf16 at k' = 32c + 8(l/16) + 0..7 of -[a1 | a1 | a2], ar = asg * rs = a1 + a2 (bf16 pieces).
__global__ void zpe_act_kernel(const float* __restrict__ ASG, const float* __restrict__ RS, int M, int G,
                               int P, u32x4* __restrict__ zpa) {
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  const int KC = zpe_chunks(G), MT = (M + 15) / 16;
  if (idx >= static_cast<int64_t>(P) * MT * KC * 64) return;
  const int l = static_cast<int>(idx & 63);
  int64_t rest = idx >> 6;
  const int c = static_cast<int>(rest % KC);
  rest /= KC;
  const int mt = static_cast<int>(rest % MT);
  const int p = static_cast<int>(rest / MT);
  const int row = 16 * mt + (l & 15);
  uint32_t h[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int kp = 32 * c + 8 * (l >> 4) + e;
    uint32_t v = 0;
    if (kp < 3 * G && row < M) {
      const int piece = kp / G, g = kp % G;
      const size_t o = (static_cast<size_t>(p) * M + row) * G + g;
      const float ar = ASG[o] * RS[o];
      const uint32_t a1 = f32_to_bf16(ar);
      v = ((piece == 2) ? f32_to_bf16(ar - bf16_to_f32(a1)) : a1) ^ 0x8000u;   // negated
    }
    h[e] = v;
  }
  zpa[idx] = u32x4{h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16), h[6] | (h[7] << 16)};
}

size_t zpe_act_bytes(int M, int G, int P) {
  return static_cast<size_t>(P) * ((M + 15) / 16) * zpe_chunks(G) * 1024;
}

// ---------------------------------------------------------------------------------------
// Direct global -> LDS loads (64 lanes x 4 or 16 bytes to M0 + lane * size; inactive lanes write
// nothing)
// Issued as inline asm so the compiler does not see the LDS write: it would otherwise wait for
// every outstanding request before each LDS read. Completion is tracked explicitly with
// s_waitcnt vmcnt before the workgroup barrier (vmcnt completes in order, so the compiler's
// own waits on its loads stay correct).
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>(p));
}
__device__ __forceinline__ void lds_dma16(const void* g, uint32_t lds) {
  asm volatile("global_load_lds_dwordx4 %0, off" ::"v"(g), "{m0}"(lds) : "memory");
}
__device__ __forceinline__ void lds_dma4(const void* g, uint32_t lds) {
  asm volatile("global_load_lds_dword %0, off" ::"v"(g), "{m0}"(lds) : "memory");
}

__device__ __forceinline__ void lds_dma16_on(const void* g, uint32_t lds, bool on) {
  if (on) lds_dma16(g, lds);
}
__device__ __forceinline__ void lds_dma4_on(const void* g, uint32_t lds, bool on) {
  if (on) lds_dma4(g, lds);
}
// scalar base + per-lane 32-bit offset: the per-group address arithmetic stays on the SALU
__device__ __forceinline__ void lds_dma16_s(const void* sbase, uint32_t voff, uint32_t lds) {
  asm volatile("global_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(sbase), "{m0}"(lds) : "memory");
}
__device__ __forceinline__ void lds_dma4_s(const void* sbase, uint32_t voff, uint32_t lds) {
  asm volatile("global_load_lds_dword %0, %1" ::"v"(voff), "s"(sbase), "{m0}"(lds) : "memory");
}
template <int N>
__device__ __forceinline__ void wait_vm() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// ---------------------------------------------------------------------------------------
// decode: M <= 16, a stream of the packed weights. A CU's memory pipeline delivers a bounded
// rate, so the kernel time is set by the CU with the most bytes: the column tiles (16 columns
// each) are dealt out so that every CU streams the same amount. The grid is a multiple of the
// CU count; each workgroup takes a contiguous run of 1..kDecMaxNT tiles inside one partition,
// runs differing by at most one tile (DecodeMap). The 4 waves of a workgroup split the groups;
// their partial sums meet in LDS at the end.
// Each wave streams its groups through a private LDS ring of D slots with direct LDS loads: a
// slot holds one group's NT weight tiles, the activation fragment, the SZ words and the rows'
// asg/rs values. Group g+D-1 is requested before group g is computed and an explicit vmcnt wait
// covers exactly group g, so D-1 groups stay in flight. The loads are invisible to the
// compiler, which therefore never inserts waits of its own on them (register rings lose their
// depth to such waits when the allocator copies an in-flight register). Two workgroups share a
// CU so that two waves per SIMD hide each other's LDS and matrix-core latencies.
constexpr int kDecWaves = 4;
constexpr int kDecMaxNT = 6;
constexpr int kDecRingBytes = 20480;   // per wave
constexpr int kDecLds = kDecWaves * kDecRingBytes;
constexpr int kDecPerCU = 2;           // workgroups resident per CU (LDS-bound)
struct DecodeMap {
  int wg0[4];   // first workgroup of partition q; wg0[3] = grid size
  int t0[3];    // first tile of partition q
  int nt[3];    // tiles of partition q
};

template <int NT>
struct DecodeSlot {
  static constexpr int kSzLoads = (NT + 3) / 4;                 // 64 SZ words per load
  static constexpr int kOffA = NT * 1024;                       // [2 halves][64 lanes][16 B]
  static constexpr int kOffSz = (NT + 2) * 1024;                // [16 NT] words
  static constexpr int kOffSc = kOffSz + kSzLoads * 256;        // [16] asg, [16] rs
  static constexpr int kBytes = kOffSc + 128;
  static constexpr int kDepth = kDecRingBytes / kBytes > 16 ? 16 : kDecRingBytes / kBytes;
  static constexpr int kLoads = NT + 2 + kSzLoads + 2;          // loads per group
  static_assert(kDepth >= 2 && (kDepth - 1) * kLoads <= 63, "decode ring does not fit vmcnt");
};

// MR = activation rows held per lane that can be live (1 when M == 1, else 4)
template <int NT, int MR>
__device__ __forceinline__ void decode_body(
    const uint8_t* __restrict__ A, const float* __restrict__ asgp, const float* __restrict__ rsp,
    int M, int K, const u32x4* __restrict__ wpk, const uint32_t* __restrict__ sz, int N, int p,
    int tfirst, uint16_t* __restrict__ y, int64_t ldy, uint8_t* smem) {
  using S = DecodeSlot<NT>;
  constexpr int D = S::kDepth;
  const int G = K >> 7;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform: scalar loop bounds
  const int col = lane & 15, kq = lane >> 4;
  const int n0 = 16 * tfirst;
  const int g0 = (G * wave) / kDecWaves, g1 = (G * (wave + 1)) / kDecWaves;

  // Sources: a scalar base per group plus a fixed per-lane offset. A operand row = lane % 16:
  // lanes with row >= M load nothing and their products land in output rows that are never
  // stored; the same holds for scale rows >= M.
  const uint8_t* wbase = reinterpret_cast<const uint8_t*>(wpk) + static_cast<size_t>(tfirst) * G * 1024;
  const uint32_t woff = 16 * lane;
  const bool a_on = col < M;
  const uint8_t* abase = A + static_cast<size_t>(p) * M * K;
  const uint32_t aoff = static_cast<uint32_t>((a_on ? col : 0) * K + 32 * kq);
  const uint8_t* zbase = reinterpret_cast<const uint8_t*>(sz + n0);
  const uint32_t zoff = 4 * lane;
  const int srow = lane & 15;
  const bool as_on = lane < 16 && srow < M, rs_on = lane >= 16 && lane < 32 && srow < M;
  const uint32_t soff = static_cast<uint32_t>(4 * (srow < M ? srow : 0) * G);

  uint8_t* ringp = smem + wave * kDecRingBytes;
  const uint32_t ring = lds_addr(ringp);
  auto issue = [&](int g, int slot) {
    const uint32_t sb = ring + slot * S::kBytes;
    const uint8_t* wg = wbase + static_cast<size_t>(g) * 1024;
#pragma unroll
    for (int t = 0; t < NT; ++t) lds_dma16_s(wg + static_cast<size_t>(t) * G * 1024, woff, sb + t * 1024);
    if (a_on) {
      lds_dma16_s(abase + 128 * g, aoff, sb + S::kOffA);
      lds_dma16_s(abase + 128 * g + 16, aoff, sb + S::kOffA + 1024);
    }
    const uint8_t* zg = zbase + static_cast<size_t>(g) * N * 4;
#pragma unroll
    for (int j = 0; j < S::kSzLoads; ++j)
      if (lane + 64 * j < 16 * NT) lds_dma4_s(zg + 256 * j, zoff, sb + S::kOffSz + j * 256);
    if (as_on) lds_dma4_s(asgp + g, soff, sb + S::kOffSc);
    if (rs_on) lds_dma4_s(rsp + g, soff, sb + S::kOffSc);
  };
  // Each load above has a live lane in every wave (lane 0 for weights, A, SZ and asg; lane 16
  // for rs), so each one is issued and counted by vmcnt.
  const int ng = g1 - g0;
  for (int i = 0; i < D - 1 && i < ng; ++i) issue(g0 + i, i);

  v4f acc[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) acc[t] = v4f{0.f, 0.f, 0.f, 0.f};
  int slot = 0;
  for (int g = g0; g < g1; ++g) {
    if (g + D - 1 < g1) {
      issue(g + D - 1, slot == 0 ? D - 1 : slot - 1);
      wait_vm<(D - 1) * S::kLoads>();   // group g has landed; D-1 groups remain in flight
    } else {
      wait_vm<0>();
    }
    const uint8_t* sp = ringp + slot * S::kBytes;
    const u32x4 a0 = *reinterpret_cast<const u32x4*>(sp + S::kOffA + 16 * lane);
    const u32x4 a1 = *reinterpret_cast<const u32x4*>(sp + S::kOffA + 1024 + 16 * lane);
    const v8i av = v8i{(int)a0.x, (int)a0.y, (int)a0.z, (int)a0.w, (int)a1.x, (int)a1.y, (int)a1.z, (int)a1.w};
    const v4f as = *reinterpret_cast<const v4f*>(sp + S::kOffSc + 16 * kq);
    const v4f rs = *reinterpret_cast<const v4f*>(sp + S::kOffSc + 64 + 16 * kq);
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const u32x4 bw = *reinterpret_cast<const u32x4*>(sp + t * 1024 + 16 * lane);
      const float2 f = sz_factors(*reinterpret_cast<const uint32_t*>(sp + S::kOffSz + 4 * (16 * t + col)));
      const v4f T = mfma_fp8(av, unpack_codes(bw));
#pragma unroll
      for (int i = 0; i < MR; ++i) acc[t][i] += as[i] * (f.x * T[i] - f.y * rs[i]);
    }
    slot = slot + 1 == D ? 0 : slot + 1;
  }

  __syncthreads();   // every ring has drained: the reduction reuses that LDS
  float* sred = reinterpret_cast<float*>(smem);   // [waves][16][16 NT]
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int i = 0; i < 4; ++i) sred[(wave * 16 + 4 * kq + i) * 16 * NT + 16 * t + col] = acc[t][i];
  __syncthreads();
  const int outs = M * 16 * NT;
  for (int idx = tid; idx < outs; idx += 64 * kDecWaves) {
    const int m = idx / (16 * NT), c = idx % (16 * NT);
    float s = 0.f;
#pragma unroll
    for (int w = 0; w < kDecWaves; ++w) s += sred[(w * 16 + m) * 16 * NT + c];
    y[static_cast<size_t>(m) * ldy + n0 + c] = static_cast<uint16_t>(f32_to_bf16(s));
  }
}

__global__ __launch_bounds__(64 * kDecWaves, kDecPerCU) void gemm_decode_kernel(
    const uint8_t* __restrict__ A, const float* __restrict__ ASG, const float* __restrict__ RS,
    int M, int K, const u32x4* __restrict__ wpk, const uint32_t* __restrict__ sz, int N,
    DecodeMap map, uint16_t* __restrict__ y, int64_t ldy) {
  __shared__ __attribute__((aligned(1024))) uint8_t smem[kDecLds];
  const int b = blockIdx.x;
  const int q = (b >= map.wg0[1]) + (b >= map.wg0[2]);          // partition
  const int nwq = map.wg0[q + 1] - map.wg0[q], bq = b - map.wg0[q];
  const int base = map.nt[q] / nwq, extra = map.nt[q] % nwq;
  const int cnt = base + (bq < extra);
  const int tfirst = map.t0[q] + bq * base + (bq < extra ? bq : extra);
  const size_t MG = static_cast<size_t>(M) * (K >> 7);
  const float* asgp = ASG + q * MG;
  const float* rsp = RS + q * MG;
#define PQ_DECODE_CASE(n)                                                                      \
  case n:                                                                                      \
    if (M == 1) decode_body<n, 1>(A, asgp, rsp, M, K, wpk, sz, N, q, tfirst, y, ldy, smem);   \
    else decode_body<n, 4>(A, asgp, rsp, M, K, wpk, sz, N, q, tfirst, y, ldy, smem);          \
    break;
  switch (cnt) {
    PQ_DECODE_CASE(1) PQ_DECODE_CASE(2) PQ_DECODE_CASE(3)
    PQ_DECODE_CASE(4) PQ_DECODE_CASE(5) PQ_DECODE_CASE(6)
    default: break;
  }
#undef PQ_DECODE_CASE
}

// Deals the N/16 column tiles out to workgroups: a grid that is a multiple of the resident
// workgroup slots (kDecPerCU per CU), each workgroup taking at most kDecMaxNT tiles per round,
// split over the partitions in proportion to their tiles; returns the largest run of tiles any
// workgroup gets.
int decode_map(int N, int pb1, int pb2, int cus, DecodeMap* map) {
  const int NTT = N / 16;
  const int tb[4] = {0, pb1 < N ? pb1 / 16 : NTT, pb2 < N ? pb2 / 16 : NTT, NTT};
  const int64_t slots = static_cast<int64_t>(kDecPerCU) * cus;
  const int64_t rounds = (NTT + kDecMaxNT * slots - 1) / (kDecMaxNT * slots);
  const int64_t W = std::min<int64_t>(NTT, rounds * slots);
  int maxrun = 0, wg = 0;
  for (int q = 0; q < 3; ++q) {
    const int nt = tb[q + 1] - tb[q];
    map->wg0[q] = wg;
    map->t0[q] = tb[q];
    map->nt[q] = nt;
    if (nt <= 0) continue;
    int64_t w = (W * nt + NTT / 2) / NTT;
    w = std::max<int64_t>(w, (nt + kDecMaxNT - 1) / kDecMaxNT);
    w = std::min<int64_t>(std::max<int64_t>(w, 1), nt);
    wg += static_cast<int>(w);
    maxrun = std::max(maxrun, static_cast<int>((nt + w - 1) / w));
  }
  map->wg0[3] = wg;
  return maxrun;
}

// ---------------------------------------------------------------------------------------
// prefill: one 512-thread workgroup per CU-sized 256x256 output tile, 8 waves as 2 (rows) x 4
// (columns) of 128x64, one 128-group per k-step. Operands move global -> LDS by direct LDS DMA
// through a 3-stage ring (2 groups ahead); LDS images are in fragment order so every lane reads
// 16 contiguous bytes. Per group and wave: 32 products T = MFMA(A_g, codes_g), each folded as
// acc += (asg * 512 sc) * T (2 VALU per output), issued one row-fragment ahead of its fold so
// the matrix core and the VALU overlap. After the loop the zero-point term is subtracted as a
// bf16 matrix-core product (pack_zpe_kernel / zpe_act_kernel operands) and bf16 results are
// stored for rows < M, columns < N. Tiles are numbered so that the ones an XCD runs at the
// same time share their activation rows and weight columns in that XCD's L2.
constexpr int kTM = 256, kTN = 256, kStages = 3;
constexpr int kOffA = 0;          // [16 mf][2 half][64 lanes][16 B] = 32 KiB
constexpr int kOffB = 32768;      // [16 nf][64 lanes][16 B]          = 16 KiB
constexpr int kOffAsg = 49152;    // [256] f32
constexpr int kOffSz = 50176;     // [256] u32
constexpr int kStageBytes = 51200;

// Direct global -> LDS DMA: lane l's 16 (or 4) bytes land at LDS address m0 + 16 l (4 l).
// Workgroups are dispatched to the 8 XCDs round-robin; give each XCD a contiguous range of
// tile numbers, and number tiles rows-fastest so that a range covers few column tiles.
__device__ __forceinline__ int xcd_tile(int bid, int ntiles) {
  const int q = ntiles / 8;
  return bid < 8 * q ? (bid % 8) * q + bid / 8 : bid;
}

__global__ __launch_bounds__(512, 1) void gemm_prefill_kernel(
    const uint8_t* __restrict__ A, const float* __restrict__ ASG,
    int M, int K, const u32x4* __restrict__ wpk, const u32x4* __restrict__ zpe,
    const u32x4* __restrict__ zpa, const uint32_t* __restrict__ sz, int N, int pb1, int pb2,
    uint16_t* __restrict__ y, int64_t ldy) {
  __shared__ __attribute__((aligned(1024))) uint8_t smem[kStages * kStageBytes];
  const int G = K >> 7;
  const int tiles_m = (M + kTM - 1) / kTM, tiles_n = (N + kTN - 1) / kTN;
  const int t = xcd_tile(blockIdx.x, tiles_m * tiles_n);
  const int m0 = (t % tiles_m) * kTM, n0 = (t / tiles_m) * kTN;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 2, wn = wave & 3;
  const int col = lane & 15, kq = lane >> 4;
  const int last_tile = N / 16 - 1;

  // the tile's partition (the launcher guarantees boundaries are multiples of 256 here)
  const int p = (n0 >= pb1) + (n0 >= pb2);

  // Per-lane DMA sources for group 0. A rows past M and column tiles past N are clamped to
  // valid memory; their results are never stored.
  const uint8_t* srcA[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int j = wave * 4 + i, mf = j >> 1, h = j & 1;
    const int row = min(m0 + 16 * mf + (lane & 15), M - 1);
    srcA[i] = A + (static_cast<size_t>(p) * M + row) * K + 32 * (lane >> 4) + 16 * h;
  }
  const uint8_t* srcB[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int nf = wave * 2 + i;
    const int tt = min(n0 / 16 + nf, last_tile);
    srcB[i] = reinterpret_cast<const uint8_t*>(wpk + static_cast<size_t>(tt) * G * 64 + lane);
  }
  const void* srcS;
  if (wave < 4) srcS = ASG + (static_cast<size_t>(p) * M + min(m0 + 64 * wave + lane, M - 1)) * G;
  else srcS = sz + min(n0 + 64 * (wave - 4) + lane, N - 1);

  const uint32_t lds0 = lds_addr(smem);
  auto issue = [&](int stage, int g) {
    const uint32_t st = lds0 + stage * kStageBytes;
#pragma unroll
    for (int i = 0; i < 4; ++i) lds_dma16(srcA[i] + 128 * g, st + kOffA + (wave * 4 + i) * 1024);
#pragma unroll
    for (int i = 0; i < 2; ++i) lds_dma16(srcB[i] + static_cast<size_t>(g) * 1024, st + kOffB + (wave * 2 + i) * 1024);
    if (wave < 4) lds_dma4(static_cast<const float*>(srcS) + g, st + kOffAsg + wave * 256);
    else lds_dma4(static_cast<const uint32_t*>(srcS) + static_cast<size_t>(g) * N, st + kOffSz + (wave - 4) * 256);
  };

  v4f acc[8][4];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

  issue(0, 0);
  if (G > 1) issue(1, 1);
  for (int g = 0; g < G; ++g) {
    // This wave's DMA for group g has landed once at most the 7 requests of group g+1 are
    // outstanding; the barrier then makes every wave's group-g data visible and guarantees no
    // wave still reads stage (g+2)%3. (__syncthreads would also drain the group g+1 requests.)
    if (g + 1 < G) asm volatile("s_waitcnt vmcnt(7) lgkmcnt(0)\n\ts_barrier" ::: "memory");
    else asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
    if (g + 2 < G) issue((g + 2) % kStages, g + 2);
    const uint8_t* st = smem + (g % kStages) * kStageBytes;

    v8i bf[4];
    float s9[4];
#pragma unroll
    for (int nf = 0; nf < 4; ++nf) {
      bf[nf] = unpack_codes(*reinterpret_cast<const u32x4*>(st + kOffB + (wn * 4 + nf) * 1024 + lane * 16));
      s9[nf] = f16_to_f32(*reinterpret_cast<const uint32_t*>(st + kOffSz + (wn * 64 + 16 * nf + col) * 4)) * 512.0f;
    }
    // products for row fragment mf are issued before the fold of mf-1
    v4f Tb[2][4];
    float4 asb[2];
#pragma unroll
    for (int mf = 0; mf <= 8; ++mf) {
      if (mf < 8) {
        const uint8_t* ap = st + kOffA + ((wm * 8 + mf) * 2) * 1024 + lane * 16;
        const u32x4 a0 = *reinterpret_cast<const u32x4*>(ap);
        const u32x4 a1 = *reinterpret_cast<const u32x4*>(ap + 1024);
        const v8i a = v8i{(int)a0.x, (int)a0.y, (int)a0.z, (int)a0.w, (int)a1.x, (int)a1.y, (int)a1.z, (int)a1.w};
        asb[mf & 1] = *reinterpret_cast<const float4*>(st + kOffAsg + (wm * 128 + 16 * mf + 4 * kq) * 4);
#pragma unroll
        for (int nf = 0; nf < 4; ++nf) Tb[mf & 1][nf] = mfma_fp8(a, bf[nf]);
      }
      if (mf > 0) {
        const int pm = mf - 1;
        const float4 as = asb[pm & 1];
#pragma unroll
        for (int nf = 0; nf < 4; ++nf) {
          acc[pm][nf][0] = __builtin_fmaf(as.x * s9[nf], Tb[pm & 1][nf][0], acc[pm][nf][0]);
          acc[pm][nf][1] = __builtin_fmaf(as.y * s9[nf], Tb[pm & 1][nf][1], acc[pm][nf][1]);
          acc[pm][nf][2] = __builtin_fmaf(as.z * s9[nf], Tb[pm & 1][nf][2], acc[pm][nf][2]);
          acc[pm][nf][3] = __builtin_fmaf(as.w * s9[nf], Tb[pm & 1][nf][3], acc[pm][nf][3]);
        }
      }
    }
  }

  // ---- zero-point epilogue: acc += (-[a1|a1|a2]) x [z1;z2;z1] over KC chunks of 32 k'
  {
    const int KC = zpe_chunks(G), MT = (M + 15) / 16;
    const u32x4* zab = zpa + static_cast<size_t>(p) * MT * KC * 64 + lane;
    for (int c = 0; c < KC; ++c) {
      u32x4 zb[4], za[8];
#pragma unroll
      for (int nf = 0; nf < 4; ++nf) {
        const int tt = min(n0 / 16 + wn * 4 + nf, last_tile);
        zb[nf] = zpe[(static_cast<size_t>(tt) * KC + c) * 64 + lane];
      }
#pragma unroll
      for (int mf = 0; mf < 8; ++mf) {
        const int mt = min((m0 + wm * 128) / 16 + mf, MT - 1);
        za[mf] = zab[(static_cast<size_t>(mt) * KC + c) * 64];
      }
#pragma unroll
      for (int mf = 0; mf < 8; ++mf)
#pragma unroll
        for (int nf = 0; nf < 4; ++nf)
          acc[mf][nf] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, za[mf]),
                                                                 __builtin_bit_cast(bf16x8, zb[nf]), acc[mf][nf], 0, 0, 0);
    }
  }

#pragma unroll
  for (int nf = 0; nf < 4; ++nf) {
    const int n = n0 + wn * 64 + 16 * nf + col;
    if (n >= N) continue;
#pragma unroll
    for (int mf = 0; mf < 8; ++mf)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int m = m0 + wm * 128 + 16 * mf + 4 * kq + i;
        if (m < M) y[static_cast<size_t>(m) * ldy + n] = static_cast<uint16_t>(f32_to_bf16(acc[mf][nf][i]));
      }
  }
}

// ---------------------------------------------------------------------------------------
// prefill, 128-wide tiles (used when a partition boundary is not a multiple of 256):
// 128x128 output tile per 256-thread workgroup, 2x2 waves of 64x64, one 128-group per
// k-step. Operands move global -> LDS by direct LDS DMA (no register staging) through a
// 3-stage ring; the LDS images are in fragment order so every lane reads 16 contiguous bytes.
// Per group: T = MFMA(A_g, codes_g) for 16 fragments, then acc += (asg * 512 sc) * T
// (2 VALU per output). After the loop the zero-point term is subtracted as one bf16
// matrix-core product (see pack_zpe_kernel), then bf16 results are stored for rows < M.
constexpr int kBM = 128, kBN = 128, kStages128 = 3;
constexpr int kOffA128 = 0;                    // [8 mf][2 half][64 lanes][16 B]
constexpr int kOffB128 = 16384;                // [8 nf][64 lanes][16 B]
constexpr int kOffAsg128 = 24576;              // [128] f32
constexpr int kOffSz128 = 25088;               // [128] u32
constexpr int kStageBytes128 = 25600;

__global__ __launch_bounds__(256, 2) void gemm_prefill128_kernel(
    const uint8_t* __restrict__ A, const float* __restrict__ ASG,
    int M, int K, const u32x4* __restrict__ wpk, const u32x4* __restrict__ zpe,
    const u32x4* __restrict__ zpa, const uint32_t* __restrict__ sz, int N, int pb1, int pb2,
    uint16_t* __restrict__ y, int64_t ldy) {
  __shared__ __attribute__((aligned(1024))) uint8_t smem[kStages128 * kStageBytes128];
  const int G = K >> 7;
  const int tiles_n = (N + kBN - 1) / kBN;
  const int tm = blockIdx.x / tiles_n, tn = blockIdx.x % tiles_n;
  const int m0 = tm * kBM, n0 = tn * kBN;
  const int p = (n0 >= pb1) + (n0 >= pb2);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform: LDS DMA bases stay scalar
  const int wm = wave >> 1, wn = wave & 1;
  const int col = lane & 15, kq = lane >> 4;

  const uint8_t* Ab = A + static_cast<size_t>(p) * M * K;
  const float* asgp = ASG + static_cast<size_t>(p) * M * G;
    const int last_tile = N / 16 - 1;

  // Per-lane DMA sources (group 0); rows past M and column tiles past N are clamped to valid
  // memory — their results are never stored.
  const uint8_t* srcA[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int j = wave * 4 + i, mf = j >> 1, h = j & 1;
    const int row = min(m0 + 16 * mf + (lane & 15), M - 1);
    srcA[i] = Ab + static_cast<size_t>(row) * K + 32 * (lane >> 4) + 16 * h;
  }
  const uint8_t* srcB[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int nf = wave * 2 + i;
    const int t = min(n0 / 16 + nf, last_tile);
    srcB[i] = reinterpret_cast<const uint8_t*>(wpk + static_cast<size_t>(t) * G * 64 + lane);
  }
  const void* srcS;
  if (wave < 2) srcS = asgp + static_cast<size_t>(min(m0 + 64 * wave + lane, M - 1)) * G;
  else srcS = sz + min(n0 + 64 * (wave - 2) + lane, N - 1);

  const uint32_t lds0 = lds_addr(smem);
  auto issue = [&](int stage, int g) {
    const uint32_t st = lds0 + stage * kStageBytes128;
#pragma unroll
    for (int i = 0; i < 4; ++i) lds_dma16(srcA[i] + 128 * g, st + kOffA128 + (wave * 4 + i) * 1024);
#pragma unroll
    for (int i = 0; i < 2; ++i) lds_dma16(srcB[i] + static_cast<size_t>(g) * 1024, st + kOffB128 + (wave * 2 + i) * 1024);
    if (wave < 2) lds_dma4(static_cast<const float*>(srcS) + g, st + kOffAsg128 + wave * 256);
    else lds_dma4(static_cast<const uint32_t*>(srcS) + static_cast<size_t>(g) * N, st + kOffSz128 + (wave - 2) * 256);
  };

  v4f acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

  issue(0, 0);
  if (G > 1) issue(1, 1);
  for (int g = 0; g < G; ++g) {
    // This wave's DMA for group g has landed once at most the 7 requests of group g+1 are
    // outstanding; the barrier then makes every wave's group-g data visible and guarantees no
    // wave still reads stage (g+2)%3. (__syncthreads would also drain the group g+1 requests.)
    if (g + 1 < G) asm volatile("s_waitcnt vmcnt(7) lgkmcnt(0)\n\ts_barrier" ::: "memory");
    else asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
    if (g + 2 < G) issue((g + 2) % kStages128, g + 2);
    const uint8_t* st = smem + (g % kStages128) * kStageBytes128;

    v8i bf[4];
    float s9[4];
#pragma unroll
    for (int nf = 0; nf < 4; ++nf) {
      bf[nf] = unpack_codes(*reinterpret_cast<const u32x4*>(st + kOffB128 + (wn * 4 + nf) * 1024 + lane * 16));
      s9[nf] = f16_to_f32(*reinterpret_cast<const uint32_t*>(st + kOffSz128 + (wn * 64 + 16 * nf + col) * 4)) * 512.0f;
    }
    // all 16 products of the group first (distinct result registers), then the folds: the
    // matrix core works through the queue while the VALU folds finished results
    v4f T[4][4];
    float4 as[4];
#pragma unroll
    for (int mf = 0; mf < 4; ++mf) {
      const u32x4 a0 = *reinterpret_cast<const u32x4*>(st + kOffA128 + ((wm * 4 + mf) * 2 + 0) * 1024 + lane * 16);
      const u32x4 a1 = *reinterpret_cast<const u32x4*>(st + kOffA128 + ((wm * 4 + mf) * 2 + 1) * 1024 + lane * 16);
      const v8i a = v8i{(int)a0.x, (int)a0.y, (int)a0.z, (int)a0.w, (int)a1.x, (int)a1.y, (int)a1.z, (int)a1.w};
      as[mf] = *reinterpret_cast<const float4*>(st + kOffAsg128 + (wm * 64 + 16 * mf + 4 * kq) * 4);
#pragma unroll
      for (int nf = 0; nf < 4; ++nf) T[mf][nf] = mfma_fp8(a, bf[nf]);
    }
#pragma unroll
    for (int mf = 0; mf < 4; ++mf)
#pragma unroll
      for (int nf = 0; nf < 4; ++nf) {
        acc[mf][nf][0] = __builtin_fmaf(as[mf].x * s9[nf], T[mf][nf][0], acc[mf][nf][0]);
        acc[mf][nf][1] = __builtin_fmaf(as[mf].y * s9[nf], T[mf][nf][1], acc[mf][nf][1]);
        acc[mf][nf][2] = __builtin_fmaf(as[mf].z * s9[nf], T[mf][nf][2], acc[mf][nf][2]);
        acc[mf][nf][3] = __builtin_fmaf(as[mf].w * s9[nf], T[mf][nf][3], acc[mf][nf][3]);
      }
  }

  // ---- zero-point epilogue: acc += (-[a1|a1|a2]) x [z1;z2;z1] over KC chunks of 32 k'
  {
    const int KC = zpe_chunks(G), MT = (M + 15) / 16;
    const u32x4* zab = zpa + static_cast<size_t>(p) * MT * KC * 64 + lane;
    for (int c = 0; c < KC; ++c) {
      bf16x8 zb[4], za[4];
#pragma unroll
      for (int nf = 0; nf < 4; ++nf) {
        const int t = min(n0 / 16 + wn * 4 + nf, last_tile);
        zb[nf] = __builtin_bit_cast(bf16x8, zpe[(static_cast<size_t>(t) * KC + c) * 64 + lane]);
      }
#pragma unroll
      for (int mf = 0; mf < 4; ++mf) {
        const int mt = min((m0 + wm * 64) / 16 + mf, MT - 1);
        za[mf] = __builtin_bit_cast(bf16x8, zab[(static_cast<size_t>(mt) * KC + c) * 64]);
      }
#pragma unroll
      for (int mf = 0; mf < 4; ++mf)
#pragma unroll
        for (int nf = 0; nf < 4; ++nf)
          acc[mf][nf] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(za[mf], zb[nf], acc[mf][nf], 0, 0, 0);
    }
  }

#pragma unroll
  for (int nf = 0; nf < 4; ++nf) {
    const int n = n0 + wn * 64 + 16 * nf + col;
    if (n >= N) continue;
#pragma unroll
    for (int mf = 0; mf < 4; ++mf)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int m = m0 + wm * 64 + 16 * mf + 4 * kq + i;
        if (m < M) y[static_cast<size_t>(m) * ldy + n] = static_cast<uint16_t>(f32_to_bf16(acc[mf][nf][i]));
      }
  }
}

// Compute units of the current device (cached per device).
static int cu_count() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cached[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cached[dev] = n;
  }
  return cached[dev];
}

static int launch_status(const char* what) {
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return set_error(PQ_ERR_DEVICE, "%s: launch failed: %s", what, hipGetErrorString(e));
  return PQ_OK;
}

}  // namespace pq

extern "C" {

size_t pq_packed_weight_bytes(int K, int N) {
  if (K <= 0 || N <= 0 || K % PQ_GROUP || N % 16) return 0;
  const size_t codes = static_cast<size_t>(K) * static_cast<size_t>(N) / 2;
  const size_t zpe = static_cast<size_t>(N / 16) * pq::zpe_chunks(K / PQ_GROUP) * 1024;
  return codes + zpe;
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
  const int G = K / PQ_GROUP;
  const int64_t words = static_cast<int64_t>(K) * N / 8;
  hipLaunchKernelGGL(pack_weights_kernel, dim3(static_cast<unsigned>((words + 255) / 256)), dim3(256), 0, s,
                     qweight_d, K, N, static_cast<uint32_t*>(wpk_d));
  const int64_t gn = static_cast<int64_t>(G) * N;
  hipLaunchKernelGGL(pack_sz_kernel, dim3(static_cast<unsigned>((gn + 255) / 256)), dim3(256), 0, s,
                     qzeros_d, scales_d, G, N, reinterpret_cast<uint32_t*>(sz_d));
  const int64_t zl = static_cast<int64_t>(N / 16) * zpe_chunks(G) * 64;
  u32x4* zpe = reinterpret_cast<u32x4*>(static_cast<uint8_t*>(wpk_d) + static_cast<size_t>(K) * N / 2);
  hipLaunchKernelGGL(pack_zpe_kernel, dim3(static_cast<unsigned>((zl + 255) / 256)), dim3(256), 0, s,
                     reinterpret_cast<const uint32_t*>(sz_d), G, N, zpe);
  return launch_status("pq_pack_weights");
}

size_t pq_gemm_workspace_bytes(int M, int N, int K) {
  (void)N;
  if (M <= 16 || K <= 0 || K % PQ_GROUP) return 0;     // the decode kernel needs none
  return pq::zpe_act_bytes(M, K / PQ_GROUP, PQ_MAX_PARTITIONS);
}

int pq_gemm(const uint8_t* a_d, const float* asg_d, const float* rs_d, int M, int K, int P,
            const void* wpk_d, const uint16_t* sz_d, int N, int pb1, int pb2, uint16_t* y_d,
            int64_t ldy, void* ws_d, size_t ws_bytes, pq_stream_t stream) {
  using namespace pq;
  clear_error();
  if (M < 0) return set_error(PQ_ERR_SHAPE, "pq_gemm: M=%d < 0", M);
  if (K <= 0 || K % PQ_GROUP || K > (1 << 24)) return set_error(PQ_ERR_SHAPE, "pq_gemm: K=%d must be a positive multiple of 128", K);
  if (N <= 0 || N % 16 || N > (1 << 24)) return set_error(PQ_ERR_SHAPE, "pq_gemm: N=%d must be a positive multiple of 16", N);
  if (ldy < N || (ldy & 1)) return set_error(PQ_ERR_SHAPE, "pq_gemm: ldy=%lld must be even and >= N=%d", static_cast<long long>(ldy), N);
  const int perr = check_partitions(P, pb1, pb2, N);
  if (perr != PQ_OK) return perr;
  if (ws_bytes < pq_gemm_workspace_bytes(M, N, K)) return set_error(PQ_ERR_WORKSPACE, "pq_gemm: workspace too small");
  if (M == 0) return PQ_OK;
  if (!a_d || !asg_d || !rs_d || !wpk_d || !sz_d || !y_d) return set_error(PQ_ERR_NULL, "pq_gemm: NULL pointer");
  if (pq_gemm_workspace_bytes(M, N, K) && !ws_d) return set_error(PQ_ERR_NULL, "pq_gemm: NULL workspace");
  if (!aligned(a_d, 16) || !aligned(asg_d, 4) || !aligned(rs_d, 4) || !aligned(wpk_d, 16) || !aligned(sz_d, 4) ||
      !aligned(y_d, 4) || !aligned(ws_d, 16))
    return set_error(PQ_ERR_ALIGN, "pq_gemm: misaligned pointer");
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const int G = K / PQ_GROUP;
  const u32x4* wpk = static_cast<const u32x4*>(wpk_d);
  const uint32_t* sz = reinterpret_cast<const uint32_t*>(sz_d);
  if (M <= 16) {
    DecodeMap map;
    decode_map(N, pb1, pb2, cu_count(), &map);
    hipLaunchKernelGGL(gemm_decode_kernel, dim3(map.wg0[3]), dim3(64 * kDecWaves), 0, s,
                       a_d, asg_d, rs_d, M, K, wpk, sz, N, map, y_d, ldy);
    return launch_status("pq_gemm(decode)");
  }
  // 256x256 tiles (one workgroup per CU) move half the bytes per output of 128x128 tiles (two
  // per CU); take them unless a partition boundary is not on a 256-column line or they fill the
  // CUs' last round of tiles worse.
  const int64_t t256 = static_cast<int64_t>((M + kTM - 1) / kTM) * ((N + kTN - 1) / kTN);
  const int64_t t128 = static_cast<int64_t>((M + kBM - 1) / kBM) * ((N + kBN - 1) / kBN);
  const int cus = cu_count();
  auto fill = [](int64_t tiles, int64_t slots) {
    return static_cast<double>(tiles) / (static_cast<double>((tiles + slots - 1) / slots) * slots);
  };
  const bool aligned256 = (pb1 >= N || pb1 % kTN == 0) && (pb2 >= N || pb2 % kTN == 0);
  const bool wide = aligned256 && fill(t256, cus) >= fill(t128, 2 * cus) - 1e-9;
  const int64_t tiles = wide ? t256 : t128;
  if (tiles > 0x7FFFFFFF) return set_error(PQ_ERR_SHAPE, "pq_gemm: problem too large");
  const u32x4* zpe = reinterpret_cast<const u32x4*>(static_cast<const uint8_t*>(wpk_d) + static_cast<size_t>(K) * N / 2);
  u32x4* zpa = static_cast<u32x4*>(ws_d);
  const int64_t zt = static_cast<int64_t>(P) * ((M + 15) / 16) * zpe_chunks(G) * 64;
  hipLaunchKernelGGL(zpe_act_kernel, dim3(static_cast<unsigned>((zt + 255) / 256)), dim3(256), 0, s,
                     asg_d, rs_d, M, G, P, zpa);
  if (wide)
    hipLaunchKernelGGL(gemm_prefill_kernel, dim3(static_cast<unsigned>(tiles)), dim3(512), 0, s,
                       a_d, asg_d, M, K, wpk, zpe, zpa, sz, N, pb1, pb2, y_d, ldy);
  else
    hipLaunchKernelGGL(gemm_prefill128_kernel, dim3(static_cast<unsigned>(tiles)), dim3(256), 0, s,
                       a_d, asg_d, M, K, wpk, zpe, zpa, sz, N, pb1, pb2, y_d, ldy);
  return launch_status("pq_gemm(prefill)");
}

}  // extern "C"
