// Device helpers shared by the library's kernels (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <cstdint>

namespace pq {

__device__ __forceinline__ float f16_to_f32(uint32_t h) {
  return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(h & 0xFFFFu)));
}

// fp32 -> bf16 bit pattern, round to nearest even, with gfx950's convert instruction. Its result
// equals the integer rounding (u + 0x7FFF + bit 16 of u) >> 16, a NaN becoming the quiet NaN
// (u >> 16) | 0x40, bit for bit on every one of the 2^32 inputs (compared exhaustively on the
// device): one instruction where the integer form took a compare, a branch and three to four more.
typedef float pq_f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 pq_bf16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}
// Two at once: lo in bits 0-15, hi in bits 16-31 (one packed convert).
__device__ __forceinline__ uint32_t bf16x2_rn(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(pq_f32x2{lo, hi}, pq_bf16x2));
}

__device__ __forceinline__ float bf16_to_f32(uint32_t h) { return __builtin_bit_cast(float, (h & 0xFFFFu) << 16); }

// The prefill GEMM's zero-point operand, activation side: K' = 3G values per row,
// -[a1 | a1 | a2] with ar = asg * rs = a1 + a2 (bf16 pieces), padded with zeros to whole chunks
// of 32. For partition p, 16-row tile mt and chunk c, 1 KiB where lane l (row 16 mt + l % 16)
// holds the 8 bf16 at k' = 32 c + 8 (l / 16) + 0..7 (the bf16 16x16x32 operand).
__host__ __device__ constexpr int zpe_chunks(int G) { return (3 * G + 31) / 32; }

// Element index of k' of row m in that operand (MT = ceil(M / 16) row tiles, KC chunks).
__device__ __forceinline__ size_t zpa_index(int p, int MT, int KC, int m, int kp) {
  const int c = kp >> 5, r = kp & 31;
  return ((static_cast<size_t>(p) * MT + (m >> 4)) * KC + c) * 512 + ((m & 15) + 16 * (r >> 3)) * 8 + (r & 7);
}

// OCP E4M3FN encode of two floats into the low 16 bits (first value in the low byte):
// NaN -> 0, -0 -> +0, clamp to +-448, then the hardware round-to-nearest-even convert.
// The hardware convert alone does not saturate (it yields NaN above 464) and keeps -0 and NaN;
// this wrapper is the encoder of "ParoQuant (PARO) W4A8 on gfx1201 — engineering log",
// section "hardware e4m3 convert in the producers".
__device__ __forceinline__ float e4m3_prep(float q) {
  q = (q == q) ? q : 0.0f;                                   // NaN -> 0
  q = __builtin_fminf(__builtin_fmaxf(q, -448.0f), 448.0f);  // saturate
  return (__builtin_bit_cast(uint32_t, q) == 0x80000000u) ? 0.0f : q;  // -0 -> +0
}

__device__ __forceinline__ uint32_t e4m3_encode2(float q0, float q1) {
  return static_cast<uint32_t>(
             __builtin_amdgcn_cvt_pk_fp8_f32(e4m3_prep(q0), e4m3_prep(q1), 0, false)) & 0xFFFFu;
}

// 512 * D(code) as an integer (exact: every finite E4M3FN value is a multiple of 2^-9).
__device__ __forceinline__ int e4m3_units(uint32_t code) {
  const int e = (code >> 3) & 15, m = code & 7;
  const int mag = (e == 0) ? m : ((8 + m) << (e - 1));
  return (code & 0x80u) ? -mag : mag;
}

}  // namespace pq
