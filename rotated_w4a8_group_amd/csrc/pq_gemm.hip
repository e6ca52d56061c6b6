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
// Packed weight image (pq_pack_weights): the codes below, then the zero-point epilogue operand,
// then the prefill fold's fp32 column factors 512 sc [G][N].
// Packed code layout, tile-major so that one column tile's whole K extent
// is one contiguous run: for 16-column tile t and group g, 1 KiB at ((t * G + g) * 1024): lane l (column 16t + l%16, k = 128g + 32*(l/16) + 0..31) owns 16 bytes
// = 4 words; byte b of word q holds code(k0 + 8q + b) in its low nibble and code(k0 + 8q + 4 + b)
// in its high nibble. (w & 0x0F0F0F0F) and ((w >> 4) & 0x0F0F0F0F) are then the lane's B
// operand registers 2q and 2q+1, matching the A operand's 32 consecutive k bytes.
#include <algorithm>
#include <mutex>

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

typedef int v4i __attribute__((ext_vector_type(4)));

// Integer-code product of one 128-group: two 16x16x64 int8 matrix-core steps over the same
// 32-byte fragments as the fp8 step (each step pairs the same byte positions of A and B, so the
// two halves together cover every k of the group once); exact in int32, returned as float.
__device__ __forceinline__ v4f mfma_i8(const v8i& a, const v8i& b) {
  v4i c = {0, 0, 0, 0};
  c = __builtin_amdgcn_mfma_i32_16x16x64_i8(v4i{a[0], a[1], a[2], a[3]}, v4i{b[0], b[1], b[2], b[3]}, c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_i32_16x16x64_i8(v4i{a[4], a[5], a[6], a[7]}, v4i{b[4], b[5], b[6], b[7]}, c, 0, 0, 0);
  return v4f{static_cast<float>(c[0]), static_cast<float>(c[1]), static_cast<float>(c[2]), static_cast<float>(c[3])};
}

// The group product for either activation code domain: e4m3 codes times the raw weight codes as
// e4m3 values c * 2^-9, or int8 codes times the raw codes as integers.
template <bool kI8>
__device__ __forceinline__ v4f group_product(const v8i& a, const v8i& b) {
  if constexpr (kI8) return mfma_i8(a, b);
  else return mfma_fp8(a, b);
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

// int5 weights: the codes' fifth bits ride in a plane beside the nibble image, and the matrix
// core takes c - 16 as the e4m3 value (c - 16) * 2^-9, exact for every code. With the fifth bit
// set that is the low nibble's own byte (as in the int4 path); without it the value is negative
// with magnitude 16 - l, whose e4m3 byte is 0x80 | (16 - l) = 0x90 - l (16 * 2^-9 = 2^-5 is the
// byte 0x10). Bit 8b + j of a lane's plane word belongs to byte b of operand dword j; v_perm
// takes each byte from the nibble value (selector 4 + b) or its negative (selector b).
template <int J>
__device__ __forceinline__ int w5_dword(uint32_t L, uint32_t H) {
  const uint32_t hb = (J >= 2 ? (H >> (J - 2)) : (H << (2 - J))) & 0x04040404u;
  return static_cast<int>(__builtin_amdgcn_perm(L, 0x90909090u - L, 0x03020100u | hb));
}

__device__ __forceinline__ v8i unpack_codes5(const u32x4& w, uint32_t H) {
  v8i b;
  b[0] = w5_dword<0>(w.x & 0x0F0F0F0Fu, H);
  b[1] = w5_dword<1>((w.x >> 4) & 0x0F0F0F0Fu, H);
  b[2] = w5_dword<2>(w.y & 0x0F0F0F0Fu, H);
  b[3] = w5_dword<3>((w.y >> 4) & 0x0F0F0F0Fu, H);
  b[4] = w5_dword<4>(w.z & 0x0F0F0F0Fu, H);
  b[5] = w5_dword<5>((w.z >> 4) & 0x0F0F0F0Fu, H);
  b[6] = w5_dword<6>(w.w & 0x0F0F0F0Fu, H);
  b[7] = w5_dword<7>((w.w >> 4) & 0x0F0F0F0Fu, H);
  return b;
}

// The weight operand of one fragment: int4 nibbles, or nibbles plus the fifth-bit word.
template <bool kW5>
__device__ __forceinline__ v8i weight_operand(const u32x4& w, uint32_t H) {
  if constexpr (kW5) return unpack_codes5(w, H);
  else return unpack_codes(w);
}

// {512*sc, zero-point factor} from one SZ word (sc in the low half, zsc in the high half). The
// product is fed the raw int4 code c (factor 8*sc + zsc = sc * zp, zsc = sc * (zp - 8)) or the
// signed int5 code c - 16 (factor zsc = sc * (zp - 16)).
template <bool kW5 = false>
__device__ __forceinline__ float2 sz_factors(uint32_t w) {
  const float sc = f16_to_f32(w), zsc = f16_to_f32(w >> 16);
  if constexpr (kW5) return make_float2(sc * 512.0f, zsc);
  else return make_float2(sc * 512.0f, __builtin_fmaf(sc, 8.0f, zsc));
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

// int5 fifth-bit plane image: per (16-column tile t, group g) 64 lanes x 4 B; bit 8b + j of lane
// l's word is the fifth bit of the code at k = 128g + 32(l/16) + 4j + b, column 16t + l%16 (the
// k of byte b of dword j of the lane's weight operand). One thread per word.
__global__ void pack_hi_kernel(const int32_t* __restrict__ qweight_hi, int K, int N, uint32_t* __restrict__ hi) {
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  const int G = K >> 7;
  if (idx >= static_cast<int64_t>(N / 16) * G * 64) return;
  const int l = static_cast<int>(idx & 63);
  const int64_t rest = idx >> 6;
  const int t = static_cast<int>(rest / G), g = static_cast<int>(rest % G);
  const int n = 16 * t + (l & 15);
  const int k0 = 128 * g + 32 * (l >> 4);
  const int64_t N32 = N / 32;
  uint32_t word = 0;
#pragma unroll
  for (int j = 0; j < 8; ++j)
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const uint32_t bit = (static_cast<uint32_t>(qweight_hi[static_cast<int64_t>(k0 + 4 * j + b) * N32 + n / 32]) >> (n & 31)) & 1u;
      word |= bit << (8 * b + j);
    }
  hi[idx] = word;
}

// SZ words of int5 weights: {sc, fl16(sc * (zp - 16))}, zp = low nibble + 16 * fifth bit; the
// product sc * (zp - 16) is exact in fp32 (11 x 5 significand bits), rounded once to f16.
__global__ void pack_sz5_kernel(const int32_t* __restrict__ qzeros, const int32_t* __restrict__ qzeros_hi,
                                const uint16_t* __restrict__ scales, int G, int N, uint32_t* __restrict__ sz) {
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (idx >= static_cast<int64_t>(G) * N) return;
  const int g = static_cast<int>(idx / N), n = static_cast<int>(idx % N);
  const uint32_t lo = (static_cast<uint32_t>(qzeros[static_cast<int64_t>(g) * (N / 8) + n / 8]) >> awq_shift(n)) & 0xFu;
  const uint32_t h5 = (static_cast<uint32_t>(qzeros_hi[static_cast<int64_t>(g) * (N / 32) + n / 32]) >> (n & 31)) & 1u;
  const int zp = static_cast<int>(lo + 16 * h5);
  const uint16_t sc = scales[idx];
  const _Float16 zsc = static_cast<_Float16>(f16_to_f32(sc) * static_cast<float>(zp - 16));
  sz[idx] = static_cast<uint32_t>(sc) | (static_cast<uint32_t>(__builtin_bit_cast(uint16_t, zsc)) << 16);
}

// Column factors of the prefill kernel's fold, fp32 [G][N]: 512 sc from the SZ words (exact: a
// power-of-two scaling of an f16 value), so the group loop reads them with no conversion.
__global__ void pack_s9_kernel(const uint32_t* __restrict__ sz, int64_t gn, float* __restrict__ s9) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i < gn) s9[i] = f16_to_f32(sz[i]) * 512.0f;
}

// ---------------------------------------------------------------------------------------
// zero-point epilogue operand (load time). The prefill kernel moves the zero-point term
//   Z[m, n] = sum_g (asg * rs)[m, g] * (8 sc + zsc)[g, n]
// out of its group loop ("zero-point epilogue" of the page) and computes it once per tile as
// a bf16 matrix-core product with split operands: ar = a1 + a2 and zz = z1 + z2 (each piece the
// bf16 rounding of what is left), Z ~= a1 z1 + a1 z2 + a2 z1 (relative error ~2^-16).
// K' = 3G is laid out as [a1 | a1 | a2] x [z1 ; z2 ; z1], padded with zeros to whole chunks of 32.
// Layout per 16-column tile t and chunk c (zpe_chunks): 1 KiB, lane l (column 16t + l%16) holds
// the 8 bf16 at k' = 32c + 8(l/16) + 0..7 — the bf16 16x16x32 B operand.

template <bool kW5>
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
      const float2 f = sz_factors<kW5>(sz[static_cast<size_t>(g) * N + n]);
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
// kTok: per-token scales, the operand is the plain row-sum (the row scale comes in the epilogue)
// and no transposed copy is written.
template <bool kTok>
__global__ void zpe_act_kernel(const float* __restrict__ ASG, const float* __restrict__ RS, int M, int G,
                               int P, u32x4* __restrict__ zpa, float* __restrict__ asgt) {
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
  // every load first (clamped to valid memory), then the arithmetic, then the stores: a store
  // between loads would make each load wait for the previous store
  const size_t rbase = (static_cast<size_t>(p) * M + min(row, M - 1)) * G;
  float av[8], rv[8];
  int piece[8], gg[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int kp = 32 * c + 8 * (l >> 4) + e;
    piece[e] = (kp < 3 * G && row < M) ? kp / G : -1;
    gg[e] = kp < 3 * G ? kp % G : 0;
    av[e] = kTok ? 1.0f : ASG[rbase + gg[e]];
    rv[e] = RS[rbase + gg[e]];
  }
  uint32_t h[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    // ar = fl32(asg rs) and a2 = bf16(ar - a1) round separately, as where the prologue writes
    // these operands: the multiply must not fuse into the subtraction
#pragma clang fp contract(off)
    uint32_t v = 0;
    if (piece[e] >= 0) {
      const float ar = kTok ? rv[e] : av[e] * rv[e];
      const uint32_t a1 = f32_to_bf16(ar);
      v = ((piece[e] == 2) ? f32_to_bf16(ar - bf16_to_f32(a1)) : a1) ^ 0x8000u;   // negated
    }
    h[e] = v;
  }
  if (!kTok) {
#pragma unroll
    for (int e = 0; e < 8; ++e)
      if (piece[e] == 0) asgt[(static_cast<size_t>(p) * G + gg[e]) * M + row] = av[e];   // [P][G][M] copy
  }
  zpa[idx] = u32x4{h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16), h[6] | (h[7] << 16)};
}

// Per-token scales broadcast to every group, [P][M][G], for the decode kernel.
__global__ void tok_expand_kernel(const float* __restrict__ AS, int PM, int G, float* __restrict__ asg) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i < static_cast<int64_t>(PM) * G) asg[i] = AS[i / G];
}

size_t zpe_act_bytes(int M, int G, int P) {
  return static_cast<size_t>(P) * ((M + 15) / 16) * zpe_chunks(G) * 1024;
}

// The group scales transposed to [P][G][M] (f32), so that a tile's scales of one group are
// contiguous for the direct loads.
size_t asgt_bytes(int M, int G, int P) {
  return (static_cast<size_t>(P) * G * M * 4 + 255) / 256 * 256;
}

// ---------------------------------------------------------------------------------------
// Direct global -> LDS loads (64 lanes x 4 or 16 bytes to M0 + lane * size; inactive lanes write
// nothing)
// Issued as inline asm so the compiler does not see the LDS write: it would otherwise wait for
// every outstanding request before each LDS read. Completion is tracked explicitly with
// s_waitcnt vmcnt before the workgroup barrier (vmcnt completes in order, so the compiler's
// own waits on its loads stay correct).
// The compiler's hazard checks do not look inside inline asm, so each helper carries the wait
// states its operands may need: a vector memory instruction that reads an SGPR written by a VALU
// instruction (the compiler reloads spilled SGPRs with v_readlane) needs 5, and one that reads M0
// right after an SALU write of M0 needs 1.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>(p));
}
__device__ __forceinline__ void lds_dma16(const void* g, uint32_t lds) {
  asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(g), "{m0}"(lds) : "memory");
}
__device__ __forceinline__ void lds_dma4(const void* g, uint32_t lds) {
  asm volatile("s_nop 0\n\tglobal_load_lds_dword %0, off" ::"v"(g), "{m0}"(lds) : "memory");
}

__device__ __forceinline__ void lds_dma16_on(const void* g, uint32_t lds, bool on) {
  if (on) lds_dma16(g, lds);
}
__device__ __forceinline__ void lds_dma4_on(const void* g, uint32_t lds, bool on) {
  if (on) lds_dma4(g, lds);
}
// scalar base + per-lane 32-bit offset: the per-group address arithmetic stays on the SALU
__device__ __forceinline__ void lds_dma16_s(const void* sbase, uint32_t voff, uint32_t lds) {
  asm volatile("s_nop 4\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(sbase), "{m0}"(lds) : "memory");
}
__device__ __forceinline__ void lds_dma4_s(const void* sbase, uint32_t voff, uint32_t lds) {
  asm volatile("s_nop 4\n\tglobal_load_lds_dword %0, %1" ::"v"(voff), "s"(sbase), "{m0}"(lds) : "memory");
}
template <int N>
__device__ __forceinline__ void wait_vm() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// ---------------------------------------------------------------------------------------
// decode: M <= 16, a stream of the packed weights. A CU's memory pipeline delivers a bounded
// rate, so the kernel time is set by the CU with the most bytes. The columns are therefore dealt
// out in quarters of a tile (4 columns): one 8-wave workgroup per CU (its ring fills the LDS), each
// taking a contiguous column range of the same number of quarters (gate_up N = 17408 on 256 CUs:
// exactly 68 columns each; ranges differ by at most one quarter in general), inside one
// partition. A range starts and ends anywhere on a 4-column line, so the tiles at its two ends are
// loaded with the lanes of the other columns masked off (each lane owns one column of a tile
// block) and their products for those columns are dropped. Consecutive ranges go to the same
// XCD (workgroups are dispatched to the XCDs round-robin), so a cache line shared by two
// neighbouring ranges is fetched once into that XCD's L2.
// The 8 waves of a workgroup split the groups; each streams its groups through a private LDS ring
// of D slots with direct LDS loads: a slot holds one group's tile blocks, the activation rows, the
// SZ words and the rows' asg/rs values. Group g+D-1 is requested before group g is computed and an
// explicit vmcnt wait covers exactly group g, so D-1 groups stay in flight. The loads are
// invisible to the compiler, which therefore never inserts waits of its own on them (register
// rings lose their depth to such waits when the allocator copies an in-flight register). The
// waves' partial sums meet in LDS at the end.
constexpr int kDecWaves = 8;
constexpr int kDecMaxNT = 6;                       // tile blocks one range touches
constexpr int kDecMaxQ = 4 * (kDecMaxNT - 1);      // quarters per range at most (80 columns)
constexpr int kDecRingBytes = 20480;               // per wave
constexpr int kDecLds = kDecWaves * kDecRingBytes; // 160 KiB: one workgroup per CU
struct DecodeMap {
  int wg0[4];   // first range of partition q; wg0[3] = number of ranges (the grid)
  int c0[3];    // first column of partition q
  int nq[3];    // quarters (4 columns) of partition q
  int xcd;      // 1: range r = (b % 8) * (grid / 8) + b / 8 for workgroup b
};

// MA = activation rows held in a slot (8 when M <= 8, else 16)
template <int NT, int MA, bool kW5>
struct DecodeSlot {
  static constexpr int kSzWords = 16 * NT;
  static constexpr int kSzLoads = (kSzWords + 63) / 64;         // 64 SZ words per load
  static constexpr int kOffA = NT * 1024;                       // [MA rows][128 B]
  static constexpr int kOffSz = kOffA + MA * 128;               // [16 NT] words
  static constexpr int kOffSc = kOffSz + (kSzWords * 4 + 15) / 16 * 16;   // [16] asg, [16] rs
  static constexpr int kOffH = kOffSc + 128;                    // int5: [NT][64 lanes] fifth-bit words
  static constexpr int kBytes = kOffH + (kW5 ? NT * 256 : 0);
  static constexpr int kDepth = kDecRingBytes / kBytes > 16 ? 16 : kDecRingBytes / kBytes;
  static constexpr int kLoads = NT + MA / 8 + kSzLoads + 2 + (kW5 ? NT : 0);   // loads per group
  static_assert(kDepth >= 2 && (kDepth - 1) * kLoads <= 63, "decode ring does not fit vmcnt");
};

// MR = activation rows held per lane that can be live (1 when M == 1, else 4)
template <int NT, int MR, int MA, bool kI8, bool kW5>
__device__ __forceinline__ void decode_body(
    const uint8_t* __restrict__ A, const float* __restrict__ asgp, const float* __restrict__ rsp,
    int M, int K, const u32x4* __restrict__ wpk, const uint32_t* __restrict__ hi,
    const uint32_t* __restrict__ sz, int N, int p, int c0, int c1, uint16_t* __restrict__ y, int64_t ldy,
    uint8_t* smem) {
  using S = DecodeSlot<NT, MA, kW5>;
  constexpr int D = S::kDepth;
  const int G = K >> 7;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform: scalar loop bounds
  const int col = lane & 15, kq = lane >> 4;
  const int tfirst = c0 >> 4, n0 = 16 * tfirst;
  const int g0 = (G * wave) / kDecWaves, g1 = (G * (wave + 1)) / kDecWaves;

  // Sources: a scalar base per group plus a fixed per-lane offset. Weight tile t: every lane owns
  // column n0 + 16t + lane % 16; lanes whose column is outside [c0, c1) load nothing (each tile
  // keeps at least 4 columns, so every load has live lanes in every wave and is counted by
  // vmcnt). Activation rows: lane l loads 16 bytes of row l / 8 (rows past M repeat row M - 1).
  const uint8_t* wbase = reinterpret_cast<const uint8_t*>(wpk) + static_cast<size_t>(tfirst) * G * 1024;
  const uint32_t woff = 16 * lane;
  bool won[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const int n = n0 + 16 * t + col;
    won[t] = n >= c0 && n < c1;
  }
  const uint8_t* hbase = reinterpret_cast<const uint8_t*>(hi) + static_cast<size_t>(tfirst) * G * 256;
  const uint8_t* abase = A + static_cast<size_t>(p) * M * K;
  const int ar0 = min(lane >> 3, M - 1), ar1 = min((lane >> 3) + 8, M - 1);
  const uint32_t aoff0 = static_cast<uint32_t>(ar0 * K + 16 * (lane & 7));
  const uint32_t aoff1 = static_cast<uint32_t>(ar1 * K + 16 * (lane & 7));
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
    for (int t = 0; t < NT; ++t)
      if (won[t]) lds_dma16_s(wg + static_cast<size_t>(t) * G * 1024, woff, sb + t * 1024);
    if constexpr (kW5) {
#pragma unroll
      for (int t = 0; t < NT; ++t)
        if (won[t]) lds_dma4_s(hbase + (static_cast<size_t>(t) * G + g) * 256, 4 * lane, sb + S::kOffH + t * 256);
    }
    lds_dma16_s(abase + 128 * g, aoff0, sb + S::kOffA);
    if constexpr (MA == 16) lds_dma16_s(abase + 128 * g, aoff1, sb + S::kOffA + 1024);
    const uint8_t* zg = zbase + static_cast<size_t>(g) * N * 4;
#pragma unroll
    for (int j = 0; j < S::kSzLoads; ++j)
      if (lane + 64 * j < S::kSzWords) lds_dma4_s(zg + 256 * j, zoff, sb + S::kOffSz + j * 256);
    if (as_on) lds_dma4_s(asgp + g, soff, sb + S::kOffSc);
    if (rs_on) lds_dma4_s(rsp + g, soff, sb + S::kOffSc);
  };
  const int ng = g1 - g0;
  for (int i = 0; i < D - 1 && i < ng; ++i) issue(g0 + i, i);

  v4f acc[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) acc[t] = v4f{0.f, 0.f, 0.f, 0.f};
  // MFMA A operand: lane l takes row l % 16 (folded onto the MA rows held), k 32 (l / 16) .. + 31
  const int arow = (lane & 15) & (MA - 1);
  int slot = 0;
  for (int g = g0; g < g1; ++g) {
    if (g + D - 1 < g1) {
      issue(g + D - 1, slot == 0 ? D - 1 : slot - 1);
      wait_vm<(D - 1) * S::kLoads>();   // group g has landed; D-1 groups remain in flight
    } else {
      wait_vm<0>();
    }
    const uint8_t* sp = ringp + slot * S::kBytes;
    const u32x4 a0 = *reinterpret_cast<const u32x4*>(sp + S::kOffA + arow * 128 + 32 * kq);
    const u32x4 a1 = *reinterpret_cast<const u32x4*>(sp + S::kOffA + arow * 128 + 32 * kq + 16);
    const v8i av = v8i{(int)a0.x, (int)a0.y, (int)a0.z, (int)a0.w, (int)a1.x, (int)a1.y, (int)a1.z, (int)a1.w};
    const v4f as = *reinterpret_cast<const v4f*>(sp + S::kOffSc + 16 * kq);
    const v4f rs = *reinterpret_cast<const v4f*>(sp + S::kOffSc + 64 + 16 * kq);
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const u32x4 bw = *reinterpret_cast<const u32x4*>(sp + t * 1024 + 16 * lane);
      float2 f = sz_factors<kW5>(*reinterpret_cast<const uint32_t*>(sp + S::kOffSz + 4 * (16 * t + col)));
      if constexpr (kI8) f.x *= 0x1p-9f;   // integer products carry no 2^-9
      const uint32_t hw = kW5 ? *reinterpret_cast<const uint32_t*>(sp + S::kOffH + t * 256 + 4 * lane) : 0u;
      const v4f T = group_product<kI8>(av, weight_operand<kW5>(bw, hw));
#pragma unroll
      for (int i = 0; i < MR; ++i) acc[t][i] += as[i] * (f.x * T[i] - f.y * rs[i]);
    }
    slot = slot + 1 == D ? 0 : slot + 1;
  }

  __syncthreads();   // every ring has drained: the reduction reuses that LDS
  float* sred = reinterpret_cast<float*>(smem);   // [waves][16 rows][16 NT]
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int i = 0; i < MR; ++i) sred[(wave * 16 + 4 * kq + i) * 16 * NT + 16 * t + col] = acc[t][i];
  __syncthreads();
  // bf16 pairs of columns (c0, c1 and ldy even: 4-byte stores)
  const int half = (c1 - c0) >> 1, pairs = M * half;
  for (int idx = tid; idx < pairs; idx += 64 * kDecWaves) {
    const int m = idx / half, c = c0 - n0 + 2 * (idx % half);
    float s0 = 0.f, s1 = 0.f;
#pragma unroll
    for (int w = 0; w < kDecWaves; ++w) {
      s0 += sred[(w * 16 + m) * 16 * NT + c];
      s1 += sred[(w * 16 + m) * 16 * NT + c + 1];
    }
    *reinterpret_cast<uint32_t*>(y + static_cast<size_t>(m) * ldy + n0 + c) = bf16x2_rn(s0, s1);
  }
}

template <bool kI8, bool kW5>
__global__ __launch_bounds__(64 * kDecWaves, 1) void gemm_decode_kernel(
    const uint8_t* __restrict__ A, const float* __restrict__ ASG, const float* __restrict__ RS,
    int M, int K, const u32x4* __restrict__ wpk, const uint32_t* __restrict__ hi,
    const uint32_t* __restrict__ sz, int N, DecodeMap map, uint16_t* __restrict__ y, int64_t ldy) {
  __shared__ __attribute__((aligned(1024))) uint8_t smem[kDecLds];
  const int b = blockIdx.x, W = map.wg0[3];
  const int r = map.xcd ? (b % 8) * (W / 8) + b / 8 : b;
  const int q = (r >= map.wg0[1]) + (r >= map.wg0[2]);          // partition
  const int nwq = map.wg0[q + 1] - map.wg0[q], rq = r - map.wg0[q];
  const int base = map.nq[q] / nwq, extra = map.nq[q] % nwq;
  const int cnt = base + (rq < extra);
  const int c0 = map.c0[q] + 4 * (rq * base + (rq < extra ? rq : extra));
  const int c1 = c0 + 4 * cnt;
  const int nt = ((c1 - 1) >> 4) - (c0 >> 4) + 1;
  const size_t MG = static_cast<size_t>(M) * (K >> 7);
  const float* asgp = ASG + q * MG;
  const float* rsp = RS + q * MG;
#define PQ_DECODE_CASE(n)                                                                                           \
  case n:                                                                                                           \
    if (M == 1) decode_body<n, 1, 8, kI8, kW5>(A, asgp, rsp, M, K, wpk, hi, sz, N, q, c0, c1, y, ldy, smem);         \
    else if (M <= 8) decode_body<n, 4, 8, kI8, kW5>(A, asgp, rsp, M, K, wpk, hi, sz, N, q, c0, c1, y, ldy, smem);    \
    else decode_body<n, 4, 16, kI8, kW5>(A, asgp, rsp, M, K, wpk, hi, sz, N, q, c0, c1, y, ldy, smem);               \
    break;
  switch (nt) {
    PQ_DECODE_CASE(1) PQ_DECODE_CASE(2) PQ_DECODE_CASE(3)
    PQ_DECODE_CASE(4) PQ_DECODE_CASE(5) PQ_DECODE_CASE(6)
    default: break;
  }
#undef PQ_DECODE_CASE
}

// Deals the N/4 column quarters out to ranges: about one range per CU (at most kDecMaxQ quarters
// each, more ranges in rounds when N is that large), split over the partitions in proportion to
// their quarters, each partition's quarters split evenly over its ranges.
void decode_map(int N, int pb1, int pb2, int cus, DecodeMap* map) {
  const int cb[4] = {0, pb1 < N ? pb1 : N, pb2 < N ? pb2 : N, N};
  const int64_t Q = N / 4;
  const int64_t tq = std::max<int64_t>(1, std::min<int64_t>(kDecMaxQ, (Q + cus - 1) / cus));
  int wg = 0;
  for (int q = 0; q < 3; ++q) {
    const int nq = (cb[q + 1] - cb[q]) / 4;
    map->wg0[q] = wg;
    map->c0[q] = cb[q];
    map->nq[q] = nq;
    if (nq > 0) wg += static_cast<int>((nq + tq - 1) / tq);
  }
  map->wg0[3] = wg;
  map->xcd = (wg % 8) == 0;
}

// ---------------------------------------------------------------------------------------
// prefill (M > 16). One 512-thread workgroup (8 waves) per output tile of TM x TN; the waves
// form a WM x WN grid of (TM/WM) x (TN/WN) blocks; one 128-group per k-step. Operands move
// global -> LDS by direct LDS loads through a ring of S stages (S - 1 groups ahead: 3 stages, or 2
// for int5 256x256 tiles whose stage does not fit three times in LDS). The activation slab
// arrives as whole 128-byte rows (8 rows per load, fully used cache lines) with the 16-byte chunk
// index XOR-swizzled by (row%8) ^ ((row/8)%2): each 16-lane quarter of a fragment read then
// covers the 64 LDS banks once (measured on gfx950: (row/2)%8 and row%8 read ~40% slower); the
// weight image is already in fragment order (each lane reads 16 contiguous bytes). Per group and
// wave the products T = MFMA(codes_g, A_g) are folded as acc += (asg * 512 sc) * T (2 VALU per output),
// each row fragment's products issued before the previous fragment's fold. The zero-point term is
// subtracted as a bf16 matrix-core product (pack_zpe_kernel / zpe_act_kernel operands) in KC more
// k-steps of the same ring, their loads issued while the last groups compute; the bf16 tile is then
// staged in LDS and written as whole rows.
//
// Tiles (PrefillMap): whole rounds of 256x256 tiles, one workgroup per CU, numbered in bands of
// 4 row tiles (tile_rc) so that the tiles an XCD runs at once share their activation and weight
// codes in its L2; the tiles of the last, partial round are cut into 2, 4 or 8 pieces (128x256,
// 128x128, 64x128) so that round costs a fraction of a full one instead of a full round at low
// occupancy. Partition boundaries that are not multiples of 256 switch the whole launch to
// 128x128 tiles (pieces 64x128).
constexpr int kPfStages = 3;
constexpr int kPfWaves = 8;
constexpr int kPfLds = kPfStages * 51200;   // the 256x256 ring (the largest)

template <int TM, int TN, int WM, int WN, bool kTok = false, bool kW5 = false, int S = kPfStages>
struct PfTile {
  static constexpr int MF = TM / WM / 16, NF = TN / WN / 16;   // fragments per wave
  static constexpr int kOffA = 0;                              // [TM rows][8 chunks][16 B], chunks swizzled
  static constexpr int kOffB = TM * 128;                       // [TN/16 tiles][64 lanes][16 B]
  static constexpr int kOffAsg = kOffB + TN * 64;              // [TM] f32
  static constexpr int kOffS9 = kOffAsg + TM * 4;              // [TN] f32 column factors 512 sc
  static constexpr int kOffH = kOffS9 + TN * 4;                // int5: [TN/16 tiles][64 lanes] u32
  static constexpr int kStage = (kOffH + (kW5 ? TN * 16 : 0) + 255) / 256 * 256;
  static constexpr int nA = TM / 8, nB = TN / 16, nAs = kTok ? 0 : TM / 64, nS9 = TN / 64;
  static constexpr int nH = kW5 ? TN / 16 : 0;
  static constexpr int nD = nA + nB + nAs + nS9 + nH;          // direct loads per group
  static constexpr int kPerWave = (nD + 3) / 4;                 // loads per wave of the issuing half
  static constexpr int kOutStride = TN + 8;                    // bf16 per staged output row
  static_assert(WM * WN == kPfWaves && MF >= 1 && NF >= 1 && TM % 64 == 0 && TN % 64 == 0, "tile");
  static_assert(S >= 2 && S * kStage <= kPfLds && TM * kOutStride * 2 <= kPfLds, "LDS");
  static_assert(kPerWave <= 31, "vmcnt");
};

template <int N>
__device__ __forceinline__ void wait_vm_lgkm_barrier() {
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(N) : "memory");
}

// Writes an LDS-staged bf16 tile [TM rows][STRIDE] to y (rows < M, columns < N): 16-byte stores
// of 8 columns when y and ldy allow it (vec16), else 4-byte stores of 2 columns. Uses all threads
// of the workgroup.
template <int TM, int TN, int STRIDE>
__device__ __forceinline__ void store_tile_rows(const uint16_t* ot, uint16_t* __restrict__ y, int64_t ldy,
                                                int m0, int n0, int M, int N, bool vec16) {
  const int nthr = blockDim.x;
  if (vec16) {
    constexpr int CH = TN / 8;
    for (int c = threadIdx.x; c < TM * CH; c += nthr) {
      const int r = c / CH, ch = c % CH;
      const int m = m0 + r, n = n0 + 8 * ch;
      if (m < M && n < N)
        *reinterpret_cast<u32x4*>(y + static_cast<size_t>(m) * ldy + n) =
            *reinterpret_cast<const u32x4*>(ot + r * STRIDE + 8 * ch);
    }
  } else {
    constexpr int CH = TN / 2;
    for (int c = threadIdx.x; c < TM * CH; c += nthr) {
      const int r = c / CH, ch = c % CH;
      const int m = m0 + r, n = n0 + 2 * ch;
      if (m < M && n < N)
        *reinterpret_cast<uint32_t*>(y + static_cast<size_t>(m) * ldy + n) =
            *reinterpret_cast<const uint32_t*>(ot + r * STRIDE + 2 * ch);
    }
  }
}

// Workgroups are dispatched to the 8 XCDs round-robin; give each XCD a contiguous range of
// tile numbers.
__device__ __forceinline__ int xcd_tile(int bid, int ntiles) {
  const int q = ntiles / 8;
  return bid < 8 * q ? (bid % 8) * q + bid / 8 : bid;
}

// Tile number -> (row tile, column tile), in bands of kPfBand row tiles: within a band the
// columns in order, within a column the band's rows (a last, shorter band takes the remaining
// rows). An XCD's contiguous range of numbers then covers a few row tiles by many columns, so
// the tiles it runs at once share both operands in its L2: 32 tiles as 4 rows x 8 columns need
// 128 KiB of activation codes and 128 KiB of weight codes per group step (256x256 tiles),
// where a column of 32 row tiles needs 1 MiB of activation codes.
constexpr int kPfBand = 4;
__device__ __forceinline__ void tile_rc(int t, int tiles_m, int tiles_n, int& row, int& col) {
  const int bands = tiles_m / kPfBand, band_tiles = kPfBand * tiles_n;
  const int band = t / band_tiles;
  if (band < bands) {
    const int rem = t - band * band_tiles;
    col = rem / kPfBand;
    row = band * kPfBand + rem % kPfBand;
  } else {
    const int last = tiles_m - bands * kPfBand, rem = t - bands * band_tiles;
    col = rem / last;
    row = bands * kPfBand + rem % last;
  }
}

template <int TM, int TN, int WM, int WN, bool kTok, bool kI8, bool kW5, int S = kPfStages>
__device__ __forceinline__ void prefill_tile(
    const uint8_t* __restrict__ A, const float* __restrict__ ASGT, int M, int K,
    const u32x4* __restrict__ wpk, const uint32_t* __restrict__ hi, const u32x4* __restrict__ zpe,
    const u32x4* __restrict__ zpa, const float* __restrict__ s9img, int N, int p, int m0, int n0,
    uint16_t* __restrict__ y, int64_t ldy, bool vec16, uint8_t* smem) {
  using TL = PfTile<TM, TN, WM, WN, kTok, kW5, S>;
  static_assert(S == 2 || S == 3, "the wait counts below cover rings of 2 and 3 stages");
  constexpr int D = S - 1;   // groups loaded ahead
  constexpr int MF = TL::MF, NF = TL::NF, PW = TL::kPerWave;
  const int G = K >> 7;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform: load table stays scalar
  const int wm = wave / WN, wn = wave % WN;
  const int kq = lane >> 4;
  const int last_tile = N / 16 - 1;
  const float* asgp = ASGT + static_cast<size_t>(p) * G * M;   // [G][M] for this partition

  // The direct loads of a group are issued by one half of the workgroup, waves 0-3 for even
  // groups and waves 4-7 for odd ones (one wave per SIMD each), so that on every SIMD one wave
  // computes while its partner is held up issuing loads. This wave's share: entry
  // d = (wave % 4) + 4 i of the tile's list (A half-fragments, weight tiles, asg rows, SZ
  // columns), taken modulo the list length so every wave of a half issues PW loads (a repeated
  // entry writes the same bytes again). Each entry is a scalar
  // base (advanced per group on the scalar unit) plus a fixed 32-bit lane offset. Rows past M
  // and column tiles past N are clamped to valid memory; their results are never stored.
  const uint8_t* sbase[PW];
  uint32_t voff[PW];
  size_t step[PW];
  uint32_t dst[PW];
  bool wide[PW];
  const uint8_t* Ap = A + static_cast<size_t>(p) * M * K;
#pragma unroll
  for (int i = 0; i < PW; ++i) {
    const int d = ((wave & 3) + 4 * i) % TL::nD;
    if (d < TL::nA) {
      const int r = 8 * d + (lane >> 3);                 // tile row; lane%8 = chunk slot
      const int row = min(m0 + r, M - 1);
      sbase[i] = Ap;
      voff[i] = static_cast<uint32_t>(row * K + 16 * ((lane & 7) ^ (r & 7) ^ ((r >> 3) & 1)));
      step[i] = 128; dst[i] = TL::kOffA + d * 1024; wide[i] = true;
    } else if (d < TL::nA + TL::nB) {
      const int j = d - TL::nA;
      const int tt = min(n0 / 16 + j, last_tile);
      sbase[i] = reinterpret_cast<const uint8_t*>(wpk) + static_cast<size_t>(tt) * G * 1024;
      voff[i] = 16 * lane;
      step[i] = 1024; dst[i] = TL::kOffB + j * 1024; wide[i] = true;
    } else if (d < TL::nA + TL::nB + TL::nAs) {
      const int j = d - TL::nA - TL::nB;
      sbase[i] = reinterpret_cast<const uint8_t*>(asgp);
      voff[i] = static_cast<uint32_t>(min(m0 + 64 * j + lane, M - 1) * 4);
      step[i] = static_cast<size_t>(M) * 4; dst[i] = TL::kOffAsg + j * 256; wide[i] = false;
    } else if (d < TL::nA + TL::nB + TL::nAs + TL::nS9) {
      const int j = d - TL::nA - TL::nB - TL::nAs;
      sbase[i] = reinterpret_cast<const uint8_t*>(s9img);
      voff[i] = static_cast<uint32_t>(min(n0 + 64 * j + lane, N - 1) * 4);
      step[i] = static_cast<size_t>(N) * 4; dst[i] = TL::kOffS9 + j * 256; wide[i] = false;
    } else {
      const int j = d - TL::nA - TL::nB - TL::nAs - TL::nS9;   // int5 fifth-bit words of tile j
      const int tt = min(n0 / 16 + j, last_tile);
      sbase[i] = reinterpret_cast<const uint8_t*>(hi) + static_cast<size_t>(tt) * G * 256;
      voff[i] = 4 * lane;
      step[i] = 256; dst[i] = TL::kOffH + j * 256; wide[i] = false;
    }
  }
  const uint32_t lds0 = lds_addr(smem);
  auto issue = [&](int stage, int g) {
    const uint32_t st = lds0 + stage * TL::kStage;
#pragma unroll
    for (int i = 0; i < PW; ++i) {
      if (wide[i]) lds_dma16_s(sbase[i] + g * step[i], voff[i], st + dst[i]);
      else lds_dma4_s(sbase[i] + g * step[i], voff[i], st + dst[i]);
    }
  };
  // Zero-point epilogue operands (pack_zpe_kernel / zpe_act_kernel): for chunk c of KC, the tile's
  // TM/16 activation-side and TN/16 weight-side fragments, 1 KiB each, go to a stage at
  // f * 1024 (f = fragment) like one more group; this half's share: fragments (wave % 4) + 4 i.
  // The source of each is computed on the scalar unit when it is issued.
  constexpr int NZ = TM / 16 + TN / 16, PWZ = (NZ + 3) / 4;
  static_assert(PWZ <= PW && NZ * 1024 <= TL::kStage, "zero-point chunks ride the group ring");
  const int KC = zpe_chunks(G), MT = (M + 15) / 16;
  auto zissue = [&](int stage, int c) {
    const uint32_t st = lds0 + stage * TL::kStage;
#pragma unroll
    for (int i = 0; i < PWZ; ++i) {
      const int f = (wave & 3) + 4 * i;
      if (f < NZ) {
        const uint8_t* src = (f < TM / 16)
            ? reinterpret_cast<const uint8_t*>(zpa) + ((static_cast<size_t>(p) * MT + min(m0 / 16 + f, MT - 1)) * KC + c) * 1024
            : reinterpret_cast<const uint8_t*>(zpe) + (static_cast<size_t>(min(n0 / 16 + f - TM / 16, last_tile)) * KC + c) * 1024;
        lds_dma16_s(src, 16 * lane, st + f * 1024);
      }
    }
  };
  // k-steps 0 .. G-1 are the groups, G .. G+KC-1 the zero-point chunks
  const int GT = G + KC;
  auto issue_step = [&](int stage, int j) {
    if (j < G) issue(stage, j);
    else zissue(stage, j - G);
  };

  v4f acc[MF][NF];
#pragma unroll
  for (int i = 0; i < MF; ++i)
#pragma unroll
    for (int j = 0; j < NF; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

  // Group j's loads go into stage j % S and are issued during group j - D (D = S - 1 groups
  // ahead; the first D groups before the loop) by half (j - D) % 2.
  const int half = wave >> 2;
  for (int j = 0; j < D && j < GT; ++j)
    if (((j - D) & 1) == half) issue_step(j % S, j);
  // Step g was loaded by half (g - D) % 2, whose only outstanding loads are step g's: it waits
  // for all of them. With D = 2 the other half's outstanding loads (at most PW, step g+1) need
  // not land; with D = 1 it has none. The barrier then makes step g visible to every wave and
  // guarantees that no wave still reads stage (g + D) % S, the one step g - 1 used.
  // (__syncthreads would also drain the step g+1 loads.) A zero-point chunk step has at most
  // PWZ <= PW loads per wave, so the same waits hold.
  auto step_begin = [&](int g) {
    if (((g - D) & 1) == half) wait_vm_lgkm_barrier<0>();
    else wait_vm_lgkm_barrier<D >= 2 ? PW : 0>();
    if (g + D < GT && (g & 1) == half) issue_step((g + D) % S, g + D);
  };
  for (int g = 0; g < G; ++g) {
    step_begin(g);
    const uint8_t* st = smem + (g % S) * TL::kStage;

    // Products are taken as (weights) x (activations)^T, so a lane's 4 results are one output row
    // (the fragment row lane % 16) and 4 consecutive columns (4 (lane / 16) .. + 3): the row scale
    // is one value per lane, the column factors a float4.
    u32x4 braw[NF];
    uint32_t hw[NF];
    v8i bf[NF];
    float4 s9[NF];
#pragma unroll
    for (int nf = 0; nf < NF; ++nf) {
      hw[nf] = kW5 ? *reinterpret_cast<const uint32_t*>(st + TL::kOffH + (wn * NF + nf) * 256 + lane * 4) : 0u;
      braw[nf] = *reinterpret_cast<const u32x4*>(st + TL::kOffB + (wn * NF + nf) * 1024 + lane * 16);
      s9[nf] = *reinterpret_cast<const float4*>(st + TL::kOffS9 + (wn * NF * 16 + 16 * nf + 4 * kq) * 4);
    }
    // fragment lane l: row l%16 of the 16-row block, k chunks 2(l/16) and 2(l/16)+1, swizzled
    const int arow = lane & 15, ac0 = 2 * (lane >> 4), asw = (arow & 7) ^ (arow >> 3);
    const int aoff0 = arow * 128 + 16 * (ac0 ^ asw), aoff1 = arow * 128 + 16 * ((ac0 + 1) ^ asw);
    auto load_a = [&](int mf, v8i& a, float& as) {
      const uint8_t* ap = st + TL::kOffA + (wm * MF + mf) * 2048;
      const u32x4 a0 = *reinterpret_cast<const u32x4*>(ap + aoff0);
      const u32x4 a1 = *reinterpret_cast<const u32x4*>(ap + aoff1);
      a = v8i{(int)a0.x, (int)a0.y, (int)a0.z, (int)a0.w, (int)a1.x, (int)a1.y, (int)a1.z, (int)a1.w};
      if constexpr (!kTok) as = *reinterpret_cast<const float*>(st + TL::kOffAsg + (wm * MF * 16 + 16 * mf + arow) * 4);
    };
    // Row fragment mf's products are interleaved one for one with the folds of fragment mf-1
    // (acc += f T, f = asg * 512 sc: 8 VALU per product), so the matrix core and the vector ALU
    // work side by side; fragment mf+1's operands are read from LDS while mf computes, and the
    // weight codes are unpacked beside fragment 0's products.
    v4f Tb[2][NF];
    v8i a[2];
    float asb[2] = {0.f, 0.f};
    load_a(0, a[0], asb[0]);
#pragma unroll
    for (int mf = 0; mf <= MF; ++mf) {
      // fragment mf-1's row scale is taken before the prefetch reuses its slot
      const int pm = mf - 1;
      float as = 0.f;
      if constexpr (!kTok) as = kI8 ? asb[pm & 1] * 0x1p-9f : asb[pm & 1];   // integer products carry no 2^-9
      if (mf + 1 < MF) load_a(mf + 1, a[(mf + 1) & 1], asb[(mf + 1) & 1]);
#pragma unroll
      for (int nf = 0; nf < NF; ++nf) {
        if (mf == 0) bf[nf] = weight_operand<kW5>(braw[nf], hw[nf]);
        if (mf < MF) Tb[mf & 1][nf] = group_product<kI8>(bf[nf], a[mf & 1]);
        if (mf > 0) {
          const v4f& T = Tb[pm & 1][nf];
          if constexpr (kTok) {
            // per-token scales: the row scale is applied once in the epilogue
            acc[pm][nf][0] = __builtin_fmaf(s9[nf].x, T[0], acc[pm][nf][0]);
            acc[pm][nf][1] = __builtin_fmaf(s9[nf].y, T[1], acc[pm][nf][1]);
            acc[pm][nf][2] = __builtin_fmaf(s9[nf].z, T[2], acc[pm][nf][2]);
            acc[pm][nf][3] = __builtin_fmaf(s9[nf].w, T[3], acc[pm][nf][3]);
          } else {
            // the four factors first, in registers of their own (the empty asm keeps the compiler
            // from pairing each multiply with its dependent FMA through one temporary)
            const float f0 = as * s9[nf].x, f1 = as * s9[nf].y, f2 = as * s9[nf].z, f3 = as * s9[nf].w;
            asm volatile("" ::"v"(f0), "v"(f1), "v"(f2), "v"(f3));
            acc[pm][nf][0] = __builtin_fmaf(f0, T[0], acc[pm][nf][0]);
            acc[pm][nf][1] = __builtin_fmaf(f1, T[1], acc[pm][nf][1]);
            acc[pm][nf][2] = __builtin_fmaf(f2, T[2], acc[pm][nf][2]);
            acc[pm][nf][3] = __builtin_fmaf(f3, T[3], acc[pm][nf][3]);
          }
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  }
  // zero-point chunk c = g - G: acc += (-[a1|a1|a2]) x [z1;z2;z1] over its 32 k' (bf16 pieces of
  // asg*rs and of the zero-point factor, relative error ~2^-16), weights as the first operand
  for (int g = G; g < GT; ++g) {
    step_begin(g);
    const uint8_t* st = smem + (g % S) * TL::kStage;
    u32x4 zb[NF];
#pragma unroll
    for (int nf = 0; nf < NF; ++nf)
      zb[nf] = *reinterpret_cast<const u32x4*>(st + (TM / 16 + wn * NF + nf) * 1024 + lane * 16);
#pragma unroll
    for (int mf = 0; mf < MF; ++mf) {
      const u32x4 za = *reinterpret_cast<const u32x4*>(st + (wm * MF + mf) * 1024 + lane * 16);
#pragma unroll
      for (int nf = 0; nf < NF; ++nf)
        acc[mf][nf] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, zb[nf]),
                                                               __builtin_bit_cast(bf16x8, za), acc[mf][nf], 0, 0, 0);
    }
  }

  // ---- bf16 tile through LDS (the ring is idle now), then whole rows with wide stores
  __syncthreads();   // every wave has finished reading the ring
  // (per-token path: each row's token scale is applied here; ASGT holds AS [P][M] in that mode and
  // the lane's row is lane % 16 of the fragment)
  uint16_t* ot = reinterpret_cast<uint16_t*>(smem);
#pragma unroll
  for (int mf = 0; mf < MF; ++mf) {
    float a = 1.0f;
    if constexpr (kTok) a = ASGT[static_cast<size_t>(p) * M + min(m0 + wm * MF * 16 + 16 * mf + (lane & 15), M - 1)];
#pragma unroll
    for (int nf = 0; nf < NF; ++nf) {
      v4f v = acc[mf][nf];
      if constexpr (kTok) v *= a;
      *reinterpret_cast<uint2*>(ot + (wm * MF * 16 + 16 * mf + (lane & 15)) * TL::kOutStride + wn * NF * 16 + 16 * nf + 4 * kq) =
          make_uint2(bf16x2_rn(v[0], v[1]), bf16x2_rn(v[2], v[3]));
    }
  }
  __syncthreads();
  store_tile_rows<TM, TN, TL::kOutStride>(ot, y, ldy, m0, n0, M, N, vec16);
}

// Tile shapes of the prefill grid: 256x256 (pieces 128x256, 128x128, 64x128), or 128x128 (pieces
// 64x128) when a partition boundary is not on a 256-column line. int5 whole 256x256 tiles run a
// ring of two stages: the fifth-bit planes make a stage 54 KiB, and three do not fit in LDS.
enum PfShape : int { kPfWide = 0, kPfNarrow = 1 };
struct PrefillMap {
  int tiles_m;   // whole tiles per tile column
  int tiles_n;   // whole tiles per tile row
  int ntiles;    // whole tiles
  int full;      // workgroups that run whole tiles (whole rounds); the rest run pieces
  int split;     // pieces per remaining tile: 1, 2, 4 or 8 (wide) / 1 or 2 (narrow)
  int shape;     // PfShape
};

template <bool kTok, bool kI8, bool kW5>
__global__ __launch_bounds__(512, 1) void gemm_prefill_kernel(
    const uint8_t* __restrict__ A, const float* __restrict__ ASGT, int M, int K,
    const u32x4* __restrict__ wpk, const uint32_t* __restrict__ hi, const u32x4* __restrict__ zpe,
    const u32x4* __restrict__ zpa, const float* __restrict__ s9img, int N, int pb1, int pb2,
    uint16_t* __restrict__ y, int64_t ldy, PrefillMap map, bool vec16) {
  __shared__ __attribute__((aligned(1024))) uint8_t smem[kPfLds];
  const int b = blockIdx.x;
  const int bm = map.shape == kPfWide ? 256 : 128, bn = map.shape == kPfNarrow ? 128 : 256;
  const bool piece = b >= map.full;
  const int big = piece ? map.full + (b - map.full) / map.split : b;
  const int r = piece ? (b - map.full) % map.split : 0;
  const int t = xcd_tile(big, map.ntiles);
  int trow, tcol;
  tile_rc(t, map.tiles_m, map.tiles_n, trow, tcol);
  int m0 = trow * bm, n0 = tcol * bn;
  const int split = piece ? map.split : 1;
  // piece r of a whole tile: split 2 -> 2 row halves; 4 -> 2 x 2 quarters; 8 -> 4 row x 2 column
  if (split == 2) m0 += (bm / 2) * r;
  else if (split == 4) { m0 += 128 * (r & 1); n0 += 128 * (r >> 1); }
  else if (split == 8) { m0 += 64 * (r & 3); n0 += 128 * (r >> 2); }
  if (m0 >= M || n0 >= N) return;   // a piece wholly past the matrix
  const int p = (n0 >= pb1) + (n0 >= pb2);
  if constexpr (kW5) {
    if (map.shape == kPfWide) {
      // the fifth-bit planes make a 256x256 stage 54 KiB: a ring of two (one group loaded ahead)
      if (split == 1) prefill_tile<256, 256, 2, 4, kTok, kI8, true, 2>(A, ASGT, M, K, wpk, hi, zpe, zpa, s9img, N, p, m0, n0, y, ldy, vec16, smem);
      else if (split == 2) prefill_tile<128, 256, 2, 4, kTok, kI8, true>(A, ASGT, M, K, wpk, hi, zpe, zpa, s9img, N, p, m0, n0, y, ldy, vec16, smem);
      else if (split == 4) prefill_tile<128, 128, 2, 4, kTok, kI8, true>(A, ASGT, M, K, wpk, hi, zpe, zpa, s9img, N, p, m0, n0, y, ldy, vec16, smem);
      else prefill_tile<64, 128, 2, 4, kTok, kI8, true>(A, ASGT, M, K, wpk, hi, zpe, zpa, s9img, N, p, m0, n0, y, ldy, vec16, smem);
      return;
    }
    if (split == 1) prefill_tile<128, 128, 2, 4, kTok, kI8, true>(A, ASGT, M, K, wpk, hi, zpe, zpa, s9img, N, p, m0, n0, y, ldy, vec16, smem);
    else prefill_tile<64, 128, 2, 4, kTok, kI8, true>(A, ASGT, M, K, wpk, hi, zpe, zpa, s9img, N, p, m0, n0, y, ldy, vec16, smem);
  } else if (map.shape == kPfWide) {
    if (split == 1) prefill_tile<256, 256, 2, 4, kTok, kI8, false>(A, ASGT, M, K, wpk, hi, zpe, zpa, s9img, N, p, m0, n0, y, ldy, vec16, smem);
    else if (split == 2) prefill_tile<128, 256, 2, 4, kTok, kI8, false>(A, ASGT, M, K, wpk, hi, zpe, zpa, s9img, N, p, m0, n0, y, ldy, vec16, smem);
    else if (split == 4) prefill_tile<128, 128, 2, 4, kTok, kI8, false>(A, ASGT, M, K, wpk, hi, zpe, zpa, s9img, N, p, m0, n0, y, ldy, vec16, smem);
    else prefill_tile<64, 128, 2, 4, kTok, kI8, false>(A, ASGT, M, K, wpk, hi, zpe, zpa, s9img, N, p, m0, n0, y, ldy, vec16, smem);
  } else {
    if (split == 1) prefill_tile<128, 128, 2, 4, kTok, kI8, false>(A, ASGT, M, K, wpk, hi, zpe, zpa, s9img, N, p, m0, n0, y, ldy, vec16, smem);
    else prefill_tile<64, 128, 2, 4, kTok, kI8, false>(A, ASGT, M, K, wpk, hi, zpe, zpa, s9img, N, p, m0, n0, y, ldy, vec16, smem);
  }
}

// Whole rounds of tiles (one workgroup per CU), then the remaining tiles in pieces.
PrefillMap prefill_map(int M, int N, int shape, int cus) {
  PrefillMap m{};
  const int bm = shape == kPfWide ? 256 : 128, bn = shape == kPfNarrow ? 128 : 256;
  m.shape = shape;
  m.tiles_m = (M + bm - 1) / bm;
  m.tiles_n = (N + bn - 1) / bn;
  const int64_t nt = static_cast<int64_t>(m.tiles_m) * m.tiles_n;
  m.ntiles = static_cast<int>(nt);
  const int64_t full = (nt / cus) * cus, rem = nt - full;
  m.full = static_cast<int>(full);
  m.split = 1;
  if (rem > 0) {
    static const int cands[2][3] = {{8, 4, 2}, {2, 0, 0}};
    for (int i = 0; i < 3 && cands[shape][i]; ++i)
      if (rem * cands[shape][i] <= cus) { m.split = cands[shape][i]; break; }
  }
  return m;
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
  return codes + zpe + static_cast<size_t>(K / PQ_GROUP) * N * 4;
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
  auto zk = pack_zpe_kernel<false>;
  hipLaunchKernelGGL(zk, dim3(static_cast<unsigned>((zl + 255) / 256)), dim3(256), 0, s,
                     reinterpret_cast<const uint32_t*>(sz_d), G, N, zpe);
  float* s9 = reinterpret_cast<float*>(reinterpret_cast<uint8_t*>(zpe) + static_cast<size_t>(N / 16) * zpe_chunks(G) * 1024);
  hipLaunchKernelGGL(pack_s9_kernel, dim3(static_cast<unsigned>((gn + 255) / 256)), dim3(256), 0, s,
                     reinterpret_cast<const uint32_t*>(sz_d), gn, s9);
  return launch_status("pq_pack_weights");
}

size_t pq_packed_weight5_bytes(int K, int N) {
  if (K <= 0 || N <= 0 || K % PQ_GROUP || N % 32) return 0;
  const size_t kn = static_cast<size_t>(K) * static_cast<size_t>(N);
  const size_t zpe = static_cast<size_t>(N / 16) * pq::zpe_chunks(K / PQ_GROUP) * 1024;
  return kn / 2 + kn / 8 + zpe + static_cast<size_t>(K / PQ_GROUP) * N * 4;
}

int pq_pack_weights5(const int32_t* qweight_d, const int32_t* qweight_hi_d, const int32_t* qzeros_d,
                     const int32_t* qzeros_hi_d, const uint16_t* scales_d, int K, int N, void* wpk_d,
                     uint16_t* sz_d, pq_stream_t stream) {
  using namespace pq;
  clear_error();
  if (K <= 0 || K % PQ_GROUP || K > (1 << 24)) return set_error(PQ_ERR_SHAPE, "pq_pack_weights5: K=%d must be a positive multiple of 128", K);
  if (N <= 0 || N % 32 || N > (1 << 24)) return set_error(PQ_ERR_SHAPE, "pq_pack_weights5: N=%d must be a positive multiple of 32", N);
  if (!qweight_d || !qweight_hi_d || !qzeros_d || !qzeros_hi_d || !scales_d || !wpk_d || !sz_d)
    return set_error(PQ_ERR_NULL, "pq_pack_weights5: NULL pointer");
  if (!aligned(qweight_d, 4) || !aligned(qweight_hi_d, 4) || !aligned(qzeros_d, 4) || !aligned(qzeros_hi_d, 4) ||
      !aligned(scales_d, 2) || !aligned(wpk_d, 16) || !aligned(sz_d, 4))
    return set_error(PQ_ERR_ALIGN, "pq_pack_weights5: misaligned pointer");
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const int G = K / PQ_GROUP;
  const int64_t words = static_cast<int64_t>(K) * N / 8;
  uint8_t* wb = static_cast<uint8_t*>(wpk_d);
  hipLaunchKernelGGL(pack_weights_kernel, dim3(static_cast<unsigned>((words + 255) / 256)), dim3(256), 0, s,
                     qweight_d, K, N, reinterpret_cast<uint32_t*>(wb));
  const int64_t hw = static_cast<int64_t>(N / 16) * G * 64;
  hipLaunchKernelGGL(pack_hi_kernel, dim3(static_cast<unsigned>((hw + 255) / 256)), dim3(256), 0, s,
                     qweight_hi_d, K, N, reinterpret_cast<uint32_t*>(wb + static_cast<size_t>(K) * N / 2));
  const int64_t gn = static_cast<int64_t>(G) * N;
  hipLaunchKernelGGL(pack_sz5_kernel, dim3(static_cast<unsigned>((gn + 255) / 256)), dim3(256), 0, s,
                     qzeros_d, qzeros_hi_d, scales_d, G, N, reinterpret_cast<uint32_t*>(sz_d));
  const int64_t zl = static_cast<int64_t>(N / 16) * zpe_chunks(G) * 64;
  u32x4* zpe = reinterpret_cast<u32x4*>(wb + static_cast<size_t>(K) * N / 2 + static_cast<size_t>(K) * N / 8);
  auto zk = pack_zpe_kernel<true>;
  hipLaunchKernelGGL(zk, dim3(static_cast<unsigned>((zl + 255) / 256)), dim3(256), 0, s,
                     reinterpret_cast<const uint32_t*>(sz_d), G, N, zpe);
  float* s9 = reinterpret_cast<float*>(reinterpret_cast<uint8_t*>(zpe) + static_cast<size_t>(N / 16) * zpe_chunks(G) * 1024);
  hipLaunchKernelGGL(pack_s9_kernel, dim3(static_cast<unsigned>((gn + 255) / 256)), dim3(256), 0, s,
                     reinterpret_cast<const uint32_t*>(sz_d), gn, s9);
  return launch_status("pq_pack_weights5");
}

size_t pq_gemm_workspace_bytes(int M, int N, int K) {
  (void)N;
  if (M <= 16 || K <= 0 || K % PQ_GROUP) return 0;     // the decode kernel needs none
  return pq::zpe_act_bytes(M, K / PQ_GROUP, PQ_MAX_PARTITIONS) + pq::asgt_bytes(M, K / PQ_GROUP, PQ_MAX_PARTITIONS);
}

size_t pq_gemm_tok_workspace_bytes(int M, int N, int K) {
  (void)N;
  if (M <= 0 || K <= 0 || K % PQ_GROUP) return 0;
  const int G = K / PQ_GROUP;
  if (M <= 16) return (static_cast<size_t>(PQ_MAX_PARTITIONS) * M * G * 4 + 255) / 256 * 256;   // scales per group
  return pq::zpe_act_bytes(M, G, PQ_MAX_PARTITIONS);
}

}  // extern "C"

namespace pq {

// The GEMM behind pq_gemm (kTok = false: a_scale = ASG [P, M, G]), pq_gemm_tok (kTok = true:
// a_scale = AS [P, M]), pq_gemm_i8 (kI8) and pq_gemm5 (kW5: int5 packed weights); validation is
// the caller's.
// ws_parts: the partition count the workspace layout is sized for (the transposed scales follow
// the zero-point operand of that many partitions).
// prepared: the workspace already holds those operands (pq_rotate_quant_for_gemm wrote them).
template <bool kTok, bool kI8, bool kW5 = false>
static int gemm_launch(const char* what, const uint8_t* a_d, const float* a_scale, const float* rs_d, int M, int K,
                       int P, const void* wpk_d, const uint16_t* sz_d, int N, int pb1, int pb2, uint16_t* y_d,
                       int64_t ldy, void* ws_d, hipStream_t s, int ws_parts = PQ_MAX_PARTITIONS,
                       bool prepared = false) {
  const int G = K / PQ_GROUP;
  const u32x4* wpk = static_cast<const u32x4*>(wpk_d);
  const uint32_t* sz = reinterpret_cast<const uint32_t*>(sz_d);
  // packed image: codes (K N / 2 bytes), [int5: fifth-bit planes (K N / 8)], zero-point operand
  const uint8_t* wb = static_cast<const uint8_t*>(wpk_d);
  const uint32_t* hi = kW5 ? reinterpret_cast<const uint32_t*>(wb + static_cast<size_t>(K) * N / 2) : nullptr;
  const u32x4* zpe = reinterpret_cast<const u32x4*>(wb + static_cast<size_t>(K) * N / 2 + (kW5 ? static_cast<size_t>(K) * N / 8 : 0));
  const float* s9img = reinterpret_cast<const float*>(reinterpret_cast<const uint8_t*>(zpe) +
                                                      static_cast<size_t>(N / 16) * zpe_chunks(G) * 1024);
  if (M <= 16) {
    const float* asg = a_scale;
    if (kTok) {
      // the decode kernel folds per group: give every group the token's scale
      float* ex = static_cast<float*>(ws_d);
      const int64_t n = static_cast<int64_t>(P) * M * G;
      hipLaunchKernelGGL(tok_expand_kernel, dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256), 0, s,
                         a_scale, P * M, G, ex);
      asg = ex;
    }
    DecodeMap map;
    decode_map(N, pb1, pb2, cu_count(), &map);
    auto dec = gemm_decode_kernel<kI8, kW5>;
    hipLaunchKernelGGL(dec, dim3(map.wg0[3]), dim3(64 * kDecWaves), 0, s,
                       a_d, asg, rs_d, M, K, wpk, hi, sz, N, map, y_d, ldy);
    return launch_status(what);
  }
  // 256x256 tiles (one workgroup per CU) unless a partition boundary is not on
  // a 256-column line
  const bool on256 = (pb1 >= N || pb1 % 256 == 0) && (pb2 >= N || pb2 % 256 == 0);
  const int shape = !on256 ? kPfNarrow : kPfWide;
  const int64_t tiles = static_cast<int64_t>((M + 127) / 128) * ((N + 127) / 128);
  if (tiles * 8 > 0x7FFFFFFF) return set_error(PQ_ERR_SHAPE, "%s: problem too large", what);
  // the prefill kernel addresses a partition's activations with 32-bit lane offsets
  if (static_cast<int64_t>(M) * K > 0x7FFFFFFF || static_cast<int64_t>(M) * (K / PQ_GROUP) * 4 > 0x7FFFFFFF)
    return set_error(PQ_ERR_SHAPE, "%s: M * K too large for one call (split the rows)", what);
  const PrefillMap map = prefill_map(M, N, shape, cu_count());
  const int64_t grid = static_cast<int64_t>(map.full) + static_cast<int64_t>(map.ntiles - map.full) * map.split;
  u32x4* zpa = static_cast<u32x4*>(ws_d);
  float* asgt = kTok ? nullptr
                     : reinterpret_cast<float*>(static_cast<uint8_t*>(ws_d) + zpe_act_bytes(M, G, ws_parts));
  if (!prepared) {
    const int64_t zt = static_cast<int64_t>(P) * ((M + 15) / 16) * zpe_chunks(G) * 64;
    hipLaunchKernelGGL(zpe_act_kernel<kTok>, dim3(static_cast<unsigned>((zt + 255) / 256)), dim3(256), 0, s,
                       a_scale, rs_d, M, G, P, zpa, asgt);
  }
  // 16-byte output stores need a 16-byte aligned y and a row pitch of 8 elements
  const bool vec16 = aligned(y_d, 16) && ldy % 8 == 0;
  auto prefill = gemm_prefill_kernel<kTok, kI8, kW5>;
  hipLaunchKernelGGL(prefill, dim3(static_cast<unsigned>(grid)), dim3(64 * kPfWaves), 0, s,
                     a_d, kTok ? a_scale : asgt, M, K, wpk, hi, zpe, zpa, s9img, N, pb1, pb2, y_d, ldy, map, vec16);
  return launch_status(what);
}

// Shared validation of pq_gemm / pq_gemm_tok; returns PQ_OK to go on, 1 for the M == 0 no-op.
static int gemm_check(const char* what, const uint8_t* a_d, const float* scale_d, const float* rs_d, int M, int K,
                      int P, const void* wpk_d, const uint16_t* sz_d, int N, int pb1, int pb2, uint16_t* y_d,
                      int64_t ldy, void* ws_d, size_t ws_bytes, size_t ws_need) {
  if (M < 0) return set_error(PQ_ERR_SHAPE, "%s: M=%d < 0", what, M);
  if (K <= 0 || K % PQ_GROUP || K > (1 << 24)) return set_error(PQ_ERR_SHAPE, "%s: K=%d must be a positive multiple of 128", what, K);
  if (N <= 0 || N % 16 || N > (1 << 24)) return set_error(PQ_ERR_SHAPE, "%s: N=%d must be a positive multiple of 16", what, N);
  if (ldy < N || (ldy & 1)) return set_error(PQ_ERR_SHAPE, "%s: ldy=%lld must be even and >= N=%d", what, static_cast<long long>(ldy), N);
  const int perr = check_partitions(P, pb1, pb2, N);
  if (perr != PQ_OK) return perr;
  if (ws_bytes < ws_need) return set_error(PQ_ERR_WORKSPACE, "%s: workspace too small", what);
  if (M == 0) return 1;
  if (!a_d || !scale_d || !rs_d || !wpk_d || !sz_d || !y_d) return set_error(PQ_ERR_NULL, "%s: NULL pointer", what);
  if (ws_need && !ws_d) return set_error(PQ_ERR_NULL, "%s: NULL workspace", what);
  if (!aligned(a_d, 16) || !aligned(scale_d, 4) || !aligned(rs_d, 4) || !aligned(wpk_d, 16) || !aligned(sz_d, 4) ||
      !aligned(y_d, 4) || !aligned(ws_d, 16))
    return set_error(PQ_ERR_ALIGN, "%s: misaligned pointer", what);
  return PQ_OK;
}

}  // namespace pq

extern "C" {

int pq_gemm(const uint8_t* a_d, const float* asg_d, const float* rs_d, int M, int K, int P,
            const void* wpk_d, const uint16_t* sz_d, int N, int pb1, int pb2, uint16_t* y_d,
            int64_t ldy, void* ws_d, size_t ws_bytes, pq_stream_t stream) {
  using namespace pq;
  clear_error();
  const int rc = gemm_check("pq_gemm", a_d, asg_d, rs_d, M, K, P, wpk_d, sz_d, N, pb1, pb2, y_d, ldy, ws_d, ws_bytes,
                            pq_gemm_workspace_bytes(M, N, K));
  if (rc != PQ_OK) return rc == 1 ? PQ_OK : rc;
  return gemm_launch<false, false>("pq_gemm", a_d, asg_d, rs_d, M, K, P, wpk_d, sz_d, N, pb1, pb2, y_d, ldy, ws_d,
                            reinterpret_cast<hipStream_t>(stream));
}

int pq_gemm_prepared(const uint8_t* a_d, const float* asg_d, const float* rs_d, int M, int K, int P,
                     const void* wpk_d, const uint16_t* sz_d, int N, int pb1, int pb2, uint16_t* y_d,
                     int64_t ldy, void* ws_d, size_t ws_bytes, pq_stream_t stream) {
  using namespace pq;
  clear_error();
  const int rc = gemm_check("pq_gemm_prepared", a_d, asg_d, rs_d, M, K, P, wpk_d, sz_d, N, pb1, pb2, y_d, ldy, ws_d,
                            ws_bytes, pq_gemm_workspace_bytes(M, N, K));
  if (rc != PQ_OK) return rc == 1 ? PQ_OK : rc;
  return gemm_launch<false, false>("pq_gemm_prepared", a_d, asg_d, rs_d, M, K, P, wpk_d, sz_d, N, pb1, pb2, y_d, ldy,
                                   ws_d, reinterpret_cast<hipStream_t>(stream), PQ_MAX_PARTITIONS, true);
}

int pq_gemm_tok(const uint8_t* a_d, const float* as_d, const float* rs_d, int M, int K, int P,
                const void* wpk_d, const uint16_t* sz_d, int N, int pb1, int pb2, uint16_t* y_d,
                int64_t ldy, void* ws_d, size_t ws_bytes, pq_stream_t stream) {
  using namespace pq;
  clear_error();
  const int rc = gemm_check("pq_gemm_tok", a_d, as_d, rs_d, M, K, P, wpk_d, sz_d, N, pb1, pb2, y_d, ldy, ws_d,
                            ws_bytes, pq_gemm_tok_workspace_bytes(M, N, K));
  if (rc != PQ_OK) return rc == 1 ? PQ_OK : rc;
  return gemm_launch<true, false>("pq_gemm_tok", a_d, as_d, rs_d, M, K, P, wpk_d, sz_d, N, pb1, pb2, y_d, ldy, ws_d,
                           reinterpret_cast<hipStream_t>(stream));
}

int pq_gemm5(const uint8_t* a_d, const float* asg_d, const float* rs_d, int M, int K, int P,
             const void* wpk5_d, const uint16_t* sz_d, int N, int pb1, int pb2, uint16_t* y_d,
             int64_t ldy, void* ws_d, size_t ws_bytes, pq_stream_t stream) {
  using namespace pq;
  clear_error();
  if (N % 32) return set_error(PQ_ERR_SHAPE, "pq_gemm5: N=%d must be a multiple of 32", N);
  const int rc = gemm_check("pq_gemm5", a_d, asg_d, rs_d, M, K, P, wpk5_d, sz_d, N, pb1, pb2, y_d, ldy, ws_d, ws_bytes,
                            pq_gemm_workspace_bytes(M, N, K));
  if (rc != PQ_OK) return rc == 1 ? PQ_OK : rc;
  return gemm_launch<false, false, true>("pq_gemm5", a_d, asg_d, rs_d, M, K, P, wpk5_d, sz_d, N, pb1, pb2, y_d, ldy,
                                         ws_d, reinterpret_cast<hipStream_t>(stream));
}

int pq_gemm_i8(const int8_t* a_d, const float* asg_d, const float* rs_d, int M, int K, int P,
               const void* wpk_d, const uint16_t* sz_d, int N, int pb1, int pb2, uint16_t* y_d,
               int64_t ldy, void* ws_d, size_t ws_bytes, pq_stream_t stream) {
  using namespace pq;
  clear_error();
  const uint8_t* a8 = reinterpret_cast<const uint8_t*>(a_d);
  const int rc = gemm_check("pq_gemm_i8", a8, asg_d, rs_d, M, K, P, wpk_d, sz_d, N, pb1, pb2, y_d, ldy, ws_d, ws_bytes,
                            pq_gemm_workspace_bytes(M, N, K));
  if (rc != PQ_OK) return rc == 1 ? PQ_OK : rc;
  return gemm_launch<false, true>("pq_gemm_i8", a8, asg_d, rs_d, M, K, P, wpk_d, sz_d, N, pb1, pb2, y_d, ldy, ws_d,
                                  reinterpret_cast<hipStream_t>(stream));
}

}  // extern "C"

// ---------------------------------------------------------------------------------------
// pq_gemm_noalloc: pq_gemm for callers that cannot allocate. The prefill kernel's scratch (the
// zero-point operand and the transposed group scales, sized for the call's own P) lives in this
// file-scope device array instead of a caller workspace. The host side never uses the array's
// name as an address: each device's copy is looked up once with hipGetSymbolAddress and that
// pointer is what the kernels get. Every call on a device shares its copy, so calls that overlap
// on one device (several streams, or threads) race on it.
namespace pq {

constexpr size_t kScratchBytes = size_t(16) << 20;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
static std::mutex g_scratch_mu;
static void* g_scratch_ptr[kMaxDevices] = {};

// The current device's copy of `scratch` (looked up on its first use). Returns PQ_OK or an error.
static int scratch_for_current_device(const char* what, void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return set_error(PQ_ERR_DEVICE, "%s: hipGetDevice failed: %s", what, hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return set_error(PQ_ERR_DEVICE, "%s: device %d out of range", what, dev);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return set_error(PQ_ERR_DEVICE, "%s: hipGetSymbolAddress(scratch) failed: %s", what, hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return PQ_OK;
}

// Scratch bytes pq_gemm_noalloc needs (0 at M <= 16, where the decode kernel uses none).
static size_t noalloc_bytes(int M, int K, int P) {
  if (M <= 16) return 0;
  const int G = K / PQ_GROUP;
  return zpe_act_bytes(M, G, P) + asgt_bytes(M, G, P);
}

}  // namespace pq

extern "C" {

size_t pq_gemm_noalloc_max_scratch_bytes(void) { return pq::kScratchBytes; }

int pq_gemm_noalloc(const uint8_t* a_d, const float* asg_d, const float* rs_d, int M, int K, int P,
                    const void* wpk_d, const uint16_t* sz_d, int N, int pb1, int pb2, uint16_t* y_d,
                    int64_t ldy, pq_stream_t stream) {
  using namespace pq;
  clear_error();
  // the same checks as pq_gemm, with the library's own scratch standing in for the workspace
  const int rc = gemm_check("pq_gemm_noalloc", a_d, asg_d, rs_d, M, K, P, wpk_d, sz_d, N, pb1, pb2, y_d, ldy,
                            nullptr, 0, 0);
  if (rc != PQ_OK) return rc == 1 ? PQ_OK : rc;
  const size_t need = noalloc_bytes(M, K, P);
  if (need > kScratchBytes)
    return set_error(PQ_ERR_SHAPE, "pq_gemm_noalloc: M=%d K=%d P=%d needs %zu scratch bytes, more than the %zu the "
                     "library holds (use pq_gemm with a workspace)", M, K, P, need, kScratchBytes);
  void* ws = nullptr;
  if (need) {
    const int src = scratch_for_current_device("pq_gemm_noalloc", &ws);
    if (src != PQ_OK) return src;
  }
  return gemm_launch<false, false>("pq_gemm_noalloc", a_d, asg_d, rs_d, M, K, P, wpk_d, sz_d, N, pb1, pb2, y_d, ldy,
                                   ws, reinterpret_cast<hipStream_t>(stream), P);
}

}  // extern "C"
