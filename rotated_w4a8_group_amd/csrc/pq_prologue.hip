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
// Launch shape: every wave is an independent unit of work, one (partition, group, token chunk);
// a 256-thread workgroup holds 4 of them and never synchronises. A wave keeps its lane's 8
// rotation records in registers and carries 8 tokens per step as two quads of 4: lane
// (t = lane/16, c = lane%16) loads 16 bytes (channels 8c..8c+7) of token t of each quad, the
// next step's loads in flight while the current step computes. The scaled values go to LDS
// token-minor, channel ch of a quad in the 16-byte row ch + ch/8 (4 tokens, the quad image).
// The layers then move 16 bytes (4 tokens) per LDS access: the first layer reads both channels
// of each lane's pair from the image, each later one keeps one channel of the previous layer's
// output in registers and takes the other from a hand-off row (one read and one write per lane
// and layer instead of two of each; on gfx950 a 16-byte LDS write costs about 2.5x a read), and
// the last layer writes both back to the image (rot_layers). The record lane order and hand-off
// rows (pq_build_records) keep those accesses and the transposing scalar ones free of bank
// conflicts. amax and the row-sum are reductions over the 16 lanes of a token (DPP).
//
// Encoding: fl32(v * inv) + 0 (which turns -0 into +0) goes straight to the hardware convert.
// For |v| <= amax and a finite inv this equals the saturating encoder unless the convert meets
// a NaN or a value past the e4m3 range, and then it writes a NaN code (0x7F/0xFF). A wave that
// finds such a code, or a non-finite inv, re-encodes its two quads with the full encoder.
#include "pq_device.h"
#include "pq_internal.h"

#pragma clang fp contract(off)

namespace pq {

constexpr int kProWaves = 4;                 // waves per workgroup (independent units)
constexpr int kProQuads = 2;                 // token quads per wave step
constexpr int kProStep = 4 * kProQuads;      // tokens per wave step
constexpr int kProQuadBytes = 144 * 16;      // 128 channel rows + 15 pad rows, 16 B each
constexpr int kProUnits = 16384;             // aim for about this many wave units

__device__ __forceinline__ uint32_t lds_row_bytes(uint32_t ch) { return (ch + (ch >> 3)) << 4; }

// Products with binary16 operands read from a half of a 32-bit word (HI selects the upper one),
// as single v_fma_mix_f32 instructions with a -0 addend: the fused operation rounds the exact
// product once, and adding -0 changes no value (-0 + -0 = -0), so each equals the binary32
// multiply of the converted operands bit for bit, without the conversions.
//   mul_hf<HI>(h2, a)       = fl32(f32(half HI of h2) * a)
//   mul_hh<HI>(a2, b2)      = fl32(f32(half HI of a2) * f32(half HI of b2))
template <bool HI>
__device__ __forceinline__ float mul_hf(uint32_t h2, float a) {
  float r;
  if constexpr (HI)
    asm("v_fma_mix_f32 %0, %1, %2, %3 op_sel:[1,0,0] op_sel_hi:[1,0,0]" : "=v"(r) : "v"(h2), "v"(a), "s"(-0.0f));
  else
    asm("v_fma_mix_f32 %0, %1, %2, %3 op_sel_hi:[1,0,0]" : "=v"(r) : "v"(h2), "v"(a), "s"(-0.0f));
  return r;
}
template <bool HI>
__device__ __forceinline__ float mul_hh(uint32_t a2, uint32_t b2) {
  float r;
  if constexpr (HI)
    asm("v_fma_mix_f32 %0, %1, %2, %3 op_sel:[1,1,0] op_sel_hi:[1,1,0]" : "=v"(r) : "v"(a2), "v"(b2), "s"(-0.0f));
  else
    asm("v_fma_mix_f32 %0, %1, %2, %3 op_sel_hi:[1,1,0]" : "=v"(r) : "v"(a2), "v"(b2), "s"(-0.0f));
  return r;
}

// The 8 rotation layers of one token-group, driven by the lane's records (layout in pq.h): on
// entry every channel ch of a quad sits in the 16-byte image row lds_row(ch) (4 tokens), on exit
// the rotated channels are back in those rows. Layer 0 reads both of the lane's channels from the
// image; afterwards a lane keeps one output of each layer in registers (the next layer's first
// operand) and passes the other through a hand-off row of LDS to the lane that needs it, so
// layers 1..6 read and write one row per quad instead of two; layer 7 writes both outputs to the
// image. Per token, with u the first operand and w the second: keep = f1*u + f2*w and
// hand = f1*w - f2*u, every product and sum rounding to binary32 (this TU has contraction off).
// The records fold into f1 and f2 which output is kept and whether w arrives negated, so keep is
// the pair's rotated value bit for bit and hand is the other one, possibly negated; in layer 7
// the lane negates (f1, f2) for hand when the record's bit 7 says w arrived negated, which makes
// it the rotated value too. A negated hand-off can differ from the exact negation only in the
// sign of an exact zero, which no code, scale or row-sum sees.
struct RotRec {
  uint32_t u0, v0;                 // layer 0: image rows of u and v (bytes)
  uint32_t rd[PQ_LAYERS];          // layers 1..7: hand-off row read (bytes)
  uint32_t wr[PQ_LAYERS];          // layers 0..6: hand-off row written (bytes)
  uint32_t u7, v7;                 // layer 7: image rows of u and v (bytes)
  float f1[PQ_LAYERS], f2[PQ_LAYERS];
  float g7, d7;                    // layer 7: (f1, f2) for v's output
};

// Layer 7's sign for v's output: bit 7 of the record word moved to the float sign bit.
__device__ __forceinline__ uint32_t last_layer_sign(uint32_t x) { return (x << 24) & 0x80000000u; }

__device__ __forceinline__ void rot_decode(const uint2 (&q)[PQ_LAYERS], RotRec& R) {
  R.u0 = lds_row_bytes(q[0].x & 0x7Fu);
  R.v0 = lds_row_bytes((q[0].x >> 8) & 0x7Fu);
  R.u7 = lds_row_bytes(q[PQ_LAYERS - 1].x & 0x7Fu);
  R.v7 = lds_row_bytes((q[PQ_LAYERS - 1].x >> 8) & 0x7Fu);
#pragma unroll
  for (int r = 0; r < PQ_LAYERS; ++r) {
    R.rd[r] = ((q[r].x >> 16) & 0xFFu) << 4;
    R.wr[r] = (q[r].x >> 24) << 4;
    R.f1[r] = f16_to_f32(q[r].y);
    R.f2[r] = f16_to_f32(q[r].y >> 16);
  }
  const uint32_t m = last_layer_sign(q[PQ_LAYERS - 1].x);
  R.g7 = __builtin_bit_cast(float, __builtin_bit_cast(uint32_t, R.f1[PQ_LAYERS - 1]) ^ m);
  R.d7 = __builtin_bit_cast(float, __builtin_bit_cast(uint32_t, R.f2[PQ_LAYERS - 1]) ^ m);
}

// NQ quad images at buf + q * QB.
template <int NQ, int QB>
__device__ __forceinline__ void rot_layers(uint8_t* buf, const RotRec& R) {
  float4 reg[NQ];
#pragma unroll
  for (int r = 0; r < PQ_LAYERS; ++r) {
    float4 a[NQ], b[NQ];
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
      a[q] = r == 0 ? *reinterpret_cast<const float4*>(buf + q * QB + R.u0) : reg[q];
      b[q] = *reinterpret_cast<const float4*>(buf + q * QB + (r == 0 ? R.v0 : R.rd[r]));
    }
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
      const float av[4] = {a[q].x, a[q].y, a[q].z, a[q].w}, bv[4] = {b[q].x, b[q].y, b[q].z, b[q].w};
      float kp[4], ot[4];
      const float gg = r + 1 < PQ_LAYERS ? R.f1[r] : R.g7, dd = r + 1 < PQ_LAYERS ? R.f2[r] : R.d7;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const float x1 = R.f1[r] * av[k], x2 = R.f2[r] * bv[k];
        const float y1 = gg * bv[k], y2 = dd * av[k];
        kp[k] = x1 + x2;
        ot[k] = y1 - y2;
      }
      if (r + 1 < PQ_LAYERS) {
        reg[q] = make_float4(kp[0], kp[1], kp[2], kp[3]);
        *reinterpret_cast<float4*>(buf + q * QB + R.wr[r]) = make_float4(ot[0], ot[1], ot[2], ot[3]);
      } else {
        *reinterpret_cast<float4*>(buf + q * QB + R.u7) = make_float4(kp[0], kp[1], kp[2], kp[3]);
        *reinterpret_cast<float4*>(buf + q * QB + R.v7) = make_float4(ot[0], ot[1], ot[2], ot[3]);
      }
    }
    __builtin_amdgcn_wave_barrier();
  }
}

// The same layers on one quad image, each record decoded where its layer runs (for kernels that
// load a group's records just before rotating it).
template <int NQ, int QB>
__device__ __forceinline__ void rot_layers_q(uint8_t* buf, const uint2 (&q)[PQ_LAYERS]) {
  float4 reg[NQ];
#pragma unroll
  for (int r = 0; r < PQ_LAYERS; ++r) {
    const uint32_t x = q[r].x;
    const float f1 = f16_to_f32(q[r].y), f2 = f16_to_f32(q[r].y >> 16);
    const uint32_t m = r + 1 < PQ_LAYERS ? 0u : last_layer_sign(x);
    const float gg = __builtin_bit_cast(float, __builtin_bit_cast(uint32_t, f1) ^ m);
    const float dd = __builtin_bit_cast(float, __builtin_bit_cast(uint32_t, f2) ^ m);
    const uint32_t ra = lds_row_bytes(x & 0x7Fu), rb = lds_row_bytes((x >> 8) & 0x7Fu);
    float4 a[NQ], b[NQ];
#pragma unroll
    for (int qd = 0; qd < NQ; ++qd) {
      a[qd] = r == 0 ? *reinterpret_cast<const float4*>(buf + qd * QB + ra) : reg[qd];
      b[qd] = *reinterpret_cast<const float4*>(buf + qd * QB + (r == 0 ? rb : ((x >> 16) & 0xFFu) << 4));
    }
#pragma unroll
    for (int qd = 0; qd < NQ; ++qd) {
      const float av[4] = {a[qd].x, a[qd].y, a[qd].z, a[qd].w}, bv[4] = {b[qd].x, b[qd].y, b[qd].z, b[qd].w};
      float kp[4], ot[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const float x1 = f1 * av[k], x2 = f2 * bv[k];
        const float y1 = gg * bv[k], y2 = dd * av[k];
        kp[k] = x1 + x2;
        ot[k] = y1 - y2;
      }
      if (r + 1 < PQ_LAYERS) {
        reg[qd] = make_float4(kp[0], kp[1], kp[2], kp[3]);
        *reinterpret_cast<float4*>(buf + qd * QB + ((x >> 24) << 4)) = make_float4(ot[0], ot[1], ot[2], ot[3]);
      } else {
        *reinterpret_cast<float4*>(buf + qd * QB + ra) = make_float4(kp[0], kp[1], kp[2], kp[3]);
        *reinterpret_cast<float4*>(buf + qd * QB + rb) = make_float4(ot[0], ot[1], ot[2], ot[3]);
      }
    }
    __builtin_amdgcn_wave_barrier();
  }
}

// Lane permutation within a 16-lane row (every lane has a source: the bound_ctrl setting never
// applies), in a form the compiler folds into the consuming max or add.
template <int CTRL>
__device__ __forceinline__ int dpp(int v) {
  return __builtin_amdgcn_mov_dpp(v, CTRL, 0xF, 0xF, true);
}

// Reductions over the 16 lanes of a DPP row: swap within pairs, within quads, mirror the
// 8-lane halves, mirror the row. Every lane of the row ends with the result.
__device__ __forceinline__ float row_max(float v) {
  v = __builtin_fmaxf(v, __builtin_bit_cast(float, dpp<0xB1>(__builtin_bit_cast(int, v))));
  v = __builtin_fmaxf(v, __builtin_bit_cast(float, dpp<0x4E>(__builtin_bit_cast(int, v))));
  v = __builtin_fmaxf(v, __builtin_bit_cast(float, dpp<0x141>(__builtin_bit_cast(int, v))));
  v = __builtin_fmaxf(v, __builtin_bit_cast(float, dpp<0x140>(__builtin_bit_cast(int, v))));
  return v;
}

__device__ __forceinline__ int row_sum(int v) {
  v += dpp<0xB1>(v);
  v += dpp<0x4E>(v);
  v += dpp<0x141>(v);
  v += dpp<0x140>(v);
  return v;
}

__device__ __forceinline__ float recip_rn(float a) { return 1.0f / a; }

// Nonzero when a byte of w is 0x7F or 0xFF (an E4M3FN NaN code).
__device__ __forceinline__ uint32_t nan_bytes(uint32_t w) {
  return ((w & 0x7F7F7F7Fu) + 0x01010101u) & 0x80808080u;
}

// fl32 sum of the 8 decoded codes in w0 (low channels) and w1, times 512: an exact integer.
__device__ __forceinline__ int code_units(uint32_t w0, uint32_t w1) {
  float s = 0.0f;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const auto d0 = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(h ? w1 : w0), false);
    const auto d1 = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(h ? w1 : w0), true);
    s = s + d0[0] + d0[1] + d1[0] + d1[1];
  }
  // each decoded code is k * 2^-9 with |k| <= 229376, so 8 of them sum exactly in binary32
  return static_cast<int>(s * 512.0f);
}

__device__ __forceinline__ uint32_t pack4(float a, float b, float c, float d) {
  // the first convert writes bytes 0-1 and keeps the rest of its "old" operand, which the second
  // convert overwrites (bytes 2-3): any register serves as that operand
  const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, __builtin_bit_cast(int, a), false);
  return static_cast<uint32_t>(__builtin_amdgcn_cvt_pk_fp8_f32(c, d, lo, true));
}

__device__ __forceinline__ float half_lo(uint32_t w) { return f16_to_f32(w); }
__device__ __forceinline__ float half_hi(uint32_t w) { return f16_to_f32(w >> 16); }

// Buffer resource for bytes [base, base + bytes) (raw, no swizzle; gfx9 data format word).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, bytes, 0x00020000);
}

template <bool kVec16>
__device__ __forceinline__ uint4 load_x8(const uint16_t* p) {
  if constexpr (kVec16) {
    return *reinterpret_cast<const uint4*>(p);
  } else {
    const uint32_t* q = reinterpret_cast<const uint32_t*>(p);
    return make_uint4(q[0], q[1], q[2], q[3]);
  }
}

// kI8: per-group int8 codes instead of e4m3 (scale amax/127, round half to even, clamp to +-127,
// integer row-sums).
// kWs: also writes what the prefill GEMM derives from (asg, rs) into its workspace: the scales
// transposed to [P][G][M] (asgt) and the zero-point operand -[a1 | a1 | a2] (zpa, zpa_index),
// with the same arithmetic as the GEMM's own pass over ASG and RS (ar = asg * rs rounded once,
// a1 = bf16(ar), a2 = bf16(ar - a1)), so pq_gemm_prepared can skip that pass.
template <bool kVec16, bool kI8, bool kWs = false>
__global__ __launch_bounds__(256) void rotate_quant_kernel(
    const uint16_t* __restrict__ x, int64_t ldx, int M, int K, int P,
    const uint2* __restrict__ rec, const uint16_t* __restrict__ cs, uint8_t* __restrict__ A,
    float* __restrict__ ASG, float* __restrict__ RS, int tok, int chunks,
    uint16_t* __restrict__ zpa = nullptr, float* __restrict__ asgt = nullptr) {
  __shared__ __align__(16) uint8_t sbuf[kProWaves][kProQuads * kProQuadBytes];

  const int G = K >> 7;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  // workgroups go to the 8 XCDs round-robin: give each XCD a contiguous range of workgroups, so
  // that the units of consecutive groups of a token chunk, whose ASG/RS rows (and zero-point
  // operand lines) share cache lines, run behind one L2
  const int nb = gridDim.x, q8 = nb >> 3, b = blockIdx.x;
  const int bx = b < 8 * q8 ? (b & 7) * q8 + (b >> 3) : b;
  const int unit = bx * kProWaves + wave;
  if (unit >= chunks * G * P) return;
  const int g = unit % G;
  const int chunk = (unit / G) % chunks;
  const int p = unit / (G * chunks);
  const int m0 = chunk * tok;
  const int m_end = min(M, m0 + tok);

  const int lane = threadIdx.x & 63;
  const int t = lane >> 4, c = lane & 15;
  const int half = K >> 1;

  RotRec R;
  {
    uint2 q[PQ_LAYERS];
#pragma unroll
    for (int r = 0; r < PQ_LAYERS; ++r) q[r] = rec[(static_cast<size_t>(p) * PQ_LAYERS + r) * half + g * 64 + lane];
    rot_decode(q, R);
  }
  const uint32_t* csp = reinterpret_cast<const uint32_t*>(cs + static_cast<size_t>(p) * K + g * 128 + 8 * c);
  float csf[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t w = csp[i];
    csf[2 * i] = half_lo(w);
    csf[2 * i + 1] = half_hi(w);
  }

  uint8_t* const buf = sbuf[wave];
  // this lane's scalar slot in a quad: channel 8c+j of token t at row 9c+j, dword t
  uint8_t* const slot = buf + (9 * c) * 16 + 4 * t;
  const uint16_t* const xg = x + g * 128 + 8 * c;
  const size_t out_base = static_cast<size_t>(p) * M;

  auto load_step = [&](int mb, uint4 (&dst)[kProQuads]) {
#pragma unroll
    for (int q = 0; q < kProQuads; ++q) {
      const int m = min(mb + 4 * q + t, m_end - 1);   // clamped: always a valid row
      dst[q] = load_x8<kVec16>(xg + static_cast<size_t>(m) * ldx);
    }
  };

  // kWs: this lane's fixed part of its output index (zpa_index at row 0; 32-bit: the operand
  // has 3 M K / 128 < 2^31 elements) and the row tile stride; the scale copy's row base
  const int zkc = zpe_chunks(G);
  const uint32_t zrow = static_cast<uint32_t>(zkc) * 512;
  const uint32_t zbase = kWs && c >= 1 && c < 4 ? static_cast<uint32_t>(zpa_index(p, (M + 15) >> 4, zkc, 0, (c - 1) * G + g)) : 0u;
  const size_t abase = (static_cast<size_t>(p) * G + g) * M;
  auto run_step = [&](int mb, const uint4 (&xs)[kProQuads]) {
    // v = x * cs (exact: 11 x 11 significand bits), transposed into token-minor rows
#pragma unroll
    for (int q = 0; q < kProQuads; ++q) {
      const uint32_t xw[4] = {xs[q].x, xs[q].y, xs[q].z, xs[q].w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        *reinterpret_cast<float*>(slot + q * kProQuadBytes + (2 * i) * 16) = mul_hf<false>(xw[i], csf[2 * i]);
        *reinterpret_cast<float*>(slot + q * kProQuadBytes + (2 * i + 1) * 16) = mul_hf<true>(xw[i], csf[2 * i + 1]);
      }
    }
    __builtin_amdgcn_wave_barrier();
    rot_layers<kProQuads, kProQuadBytes>(buf, R);
    float v[kProQuads][8], inv[kProQuads], asg[kProQuads];
    uint32_t w[kProQuads][2];
    uint32_t bad = 0;
#pragma unroll
    for (int q = 0; q < kProQuads; ++q) {
#pragma unroll
      for (int j = 0; j < 8; ++j) v[q][j] = *reinterpret_cast<const float*>(slot + q * kProQuadBytes + j * 16);
    }
    __builtin_amdgcn_wave_barrier();
    if constexpr (kI8) {
#pragma unroll
      for (int q = 0; q < kProQuads; ++q) {
        float m = __builtin_fabsf(v[q][0]);
#pragma unroll
        for (int j = 1; j < 8; ++j) m = __builtin_fmaxf(m, __builtin_fabsf(v[q][j]));
        const float amax = row_max(m);
        const float sc8 = amax / 127.0f;        // correctly rounded division
        const float iv = recip_rn(sc8);
        int qi[8], sum = 0;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const float r = __builtin_rintf(v[q][j] * iv);       // round half to even
          qi[j] = amax == 0.0f ? 0 : static_cast<int>(__builtin_fminf(__builtin_fmaxf(r, -127.0f), 127.0f));
          sum += qi[j];
        }
        const uint32_t w0 = (qi[0] & 0xFF) | ((qi[1] & 0xFF) << 8) | ((qi[2] & 0xFF) << 16) | (static_cast<uint32_t>(qi[3]) << 24);
        const uint32_t w1 = (qi[4] & 0xFF) | ((qi[5] & 0xFF) << 8) | ((qi[6] & 0xFF) << 16) | (static_cast<uint32_t>(qi[7]) << 24);
        const int units = row_sum(sum);
        const int m8 = mb + 4 * q + t;
        if (m8 < m_end) {
          *reinterpret_cast<uint2*>(A + (out_base + m8) * K + g * 128 + 8 * c) = make_uint2(w0, w1);
          if (c == 0) {
            ASG[(out_base + m8) * G + g] = sc8;
            RS[(out_base + m8) * G + g] = static_cast<float>(units);   // |units| <= 127 * 128: exact
          }
        }
      }
      return;
    }
#pragma unroll
    for (int q = 0; q < kProQuads; ++q) {
      float m = __builtin_fabsf(v[q][0]);
#pragma unroll
      for (int j = 1; j < 8; ++j) m = __builtin_fmaxf(m, __builtin_fabsf(v[q][j]));
      const float amax = row_max(m);
      asg[q] = amax * 0x1.24924ap-9f;   // fl32(1/448) = 0x3B124925
      inv[q] = recip_rn(asg[q]);
      float s[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) s[j] = v[q][j] * inv[q] + 0.0f;
      w[q][0] = pack4(s[0], s[1], s[2], s[3]);
      w[q][1] = pack4(s[4], s[5], s[6], s[7]);
      bad |= nan_bytes(w[q][0]) | nan_bytes(w[q][1]);
      bad |= (__builtin_fabsf(inv[q]) == __builtin_inff()) ? 1u : 0u;
    }
    if (__builtin_amdgcn_ballot_w64(bad != 0)) {
      // rare: a NaN or out-of-range value somewhere in the wave; take the full encoder
#pragma unroll
      for (int q = 0; q < kProQuads; ++q) {
        w[q][0] = e4m3_encode2(v[q][0] * inv[q], v[q][1] * inv[q]) |
                  (e4m3_encode2(v[q][2] * inv[q], v[q][3] * inv[q]) << 16);
        w[q][1] = e4m3_encode2(v[q][4] * inv[q], v[q][5] * inv[q]) |
                  (e4m3_encode2(v[q][6] * inv[q], v[q][7] * inv[q]) << 16);
      }
    }
#pragma unroll
    for (int q = 0; q < kProQuads; ++q) {
      const int units = row_sum(code_units(w[q][0], w[q][1]));
      const int m = mb + 4 * q + t;
      if (m < m_end) {
        *reinterpret_cast<uint2*>(A + (out_base + m) * K + g * 128 + 8 * c) = make_uint2(w[q][0], w[q][1]);
        const float rsv = static_cast<float>(units) * 0x1p-9f;
        if (c == 0) {
          ASG[(out_base + m) * G + g] = asg[q];
          RS[(out_base + m) * G + g] = rsv;
        }
        if constexpr (kWs) {
          // lane c = 0 of the token writes the transposed scale, lanes 1..3 the pieces at
          // k' = g, G + g, 2G + g; the last group's lanes also zero the padding k' >= 3G
          const float ar = asg[q] * rsv;
          const uint32_t a1 = f32_to_bf16(ar), a2 = f32_to_bf16(ar - bf16_to_f32(a1));
          const uint32_t mrow = static_cast<uint32_t>(m >> 4) * zrow + static_cast<uint32_t>(m & 15) * 8;
          if (c == 0) asgt[abase + m] = asg[q];
          else if (c < 4) zpa[zbase + mrow] = static_cast<uint16_t>((c == 3 ? a2 : a1) ^ 0x8000u);
          if (g == G - 1)
            for (int kp = 3 * G + c; kp < 32 * zkc; kp += 16)
              zpa[zpa_index(p, (M + 15) >> 4, zkc, m, kp)] = 0;
        }
      }
    }
  };

  uint4 xa[kProQuads], xb[kProQuads];
  load_step(m0, xa);
  for (int mb = m0;; mb += 2 * kProStep) {
    load_step(mb + kProStep, xb);
    run_step(mb, xa);
    if (mb + kProStep >= m_end) break;
    load_step(mb + 2 * kProStep, xa);
    run_step(mb + kProStep, xb);
    if (mb + 2 * kProStep >= m_end) break;
  }
}

// ---------------------------------------------------------------------------------------
// Per-token variant: one e4m3 scale per (partition, token) = the largest of the token's group
// scales ("Numbers", the per-token prefill bullet; section "2026-09-08: MXFP4-PARO prod decode",
// item 1). The scale needs every group of the row before any code is written, so a 16-wave
// workgroup takes one quad of 4 tokens across all G groups: wave w rotates groups w, w+16, ...
// through its own LDS quad image (the per-group kernel's layout and record lane order) and keeps
// the rotated values in registers (8 per lane per group, at most NPG groups); a workgroup-wide
// max gives the token amax, then every wave encodes its parked groups and writes plain per-group
// code row-sums.
constexpr int kTokWaves = 16;

template <int NPG, bool kVec16>
__global__ __launch_bounds__(64 * kTokWaves) void rotate_quant_tok_kernel(
    const uint16_t* __restrict__ x, int64_t ldx, int M, int K, int P,
    const uint2* __restrict__ rec, const uint16_t* __restrict__ cs, uint8_t* __restrict__ A,
    float* __restrict__ AS, float* __restrict__ RS) {
  __shared__ __align__(16) uint8_t qbuf[kTokWaves][kProQuadBytes];
  __shared__ float tred[kTokWaves][4];

  const int G = K >> 7, half = K >> 1;
  const int quads = (M + 3) >> 2;
  const int p = blockIdx.x / quads, m0 = 4 * (blockIdx.x % quads);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63, t = lane >> 4, c = lane & 15;
  const int m = m0 + t, mld = min(m, M - 1);      // clamped: always a valid row to read
  uint8_t* const buf = qbuf[wave];
  uint8_t* const slot = buf + (9 * c) * 16 + 4 * t;
  const uint16_t* const xrow = x + static_cast<size_t>(mld) * ldx + 8 * c;
  // records and channel scales through buffer loads: the lane's offset is fixed, the layer and
  // group part of the address is wave-uniform and goes in the scalar offset
  const __amdgpu_buffer_rsrc_t rec_rs = make_rsrc(rec + static_cast<size_t>(p) * PQ_LAYERS * half, 64 * half);
  const __amdgpu_buffer_rsrc_t cs_rs = make_rsrc(cs + static_cast<size_t>(p) * K, 2 * K);

  float park[NPG][8];
  float tmax = 0.0f;
#pragma unroll
  for (int j = 0; j < NPG; ++j) {
    const int g = wave + kTokWaves * j;
    if (g < G) {
      uint2 q[PQ_LAYERS];
#pragma unroll
      for (int r = 0; r < PQ_LAYERS; ++r) {
        const auto v = __builtin_amdgcn_raw_buffer_load_b64(rec_rs, 8 * lane, 8 * (r * half + g * 64), 0);
        q[r] = make_uint2(v[0], v[1]);
      }
      const auto cv = __builtin_amdgcn_raw_buffer_load_b128(cs_rs, 16 * c, 256 * g, 0);
      const uint32_t cs4[4] = {cv[0], cv[1], cv[2], cv[3]};
      const uint4 xs = load_x8<kVec16>(xrow + g * 128);
      const uint32_t xw[4] = {xs.x, xs.y, xs.z, xs.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        *reinterpret_cast<float*>(slot + (2 * i) * 16) = mul_hh<false>(xw[i], cs4[i]);
        *reinterpret_cast<float*>(slot + (2 * i + 1) * 16) = mul_hh<true>(xw[i], cs4[i]);
      }
      __builtin_amdgcn_wave_barrier();
      rot_layers_q<1, kProQuadBytes>(buf, q);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        park[j][i] = *reinterpret_cast<const float*>(slot + i * 16);
        tmax = __builtin_fmaxf(tmax, __builtin_fabsf(park[j][i]));
      }
      __builtin_amdgcn_wave_barrier();
    }
  }

  // token amax: over the 16 lanes of the token, then over the waves
  tmax = row_max(tmax);
  if (c == 0) tred[wave][t] = tmax;
  __syncthreads();
  float amax = tred[0][t];
#pragma unroll
  for (int w = 1; w < kTokWaves; ++w) amax = __builtin_fmaxf(amax, tred[w][t]);
  const float as = amax * 0x1.24924ap-9f;   // fl32(1/448)
  const float inv = recip_rn(as);
  const bool inv_bad = __builtin_fabsf(inv) == __builtin_inff();
  const size_t row = static_cast<size_t>(p) * M + m;
  if (wave == 0 && c == 0 && m < M) AS[row] = as;

#pragma unroll
  for (int j = 0; j < NPG; ++j) {
    const int g = wave + kTokWaves * j;
    if (g < G) {
      float s[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) s[i] = park[j][i] * inv + 0.0f;
      uint32_t w0 = pack4(s[0], s[1], s[2], s[3]), w1 = pack4(s[4], s[5], s[6], s[7]);
      const uint32_t bad = (nan_bytes(w0) | nan_bytes(w1)) | (inv_bad ? 1u : 0u);
      if (__builtin_amdgcn_ballot_w64(bad != 0)) {
        // rare: a NaN or out-of-range value in the wave; the full encoder
        w0 = e4m3_encode2(park[j][0] * inv, park[j][1] * inv) | (e4m3_encode2(park[j][2] * inv, park[j][3] * inv) << 16);
        w1 = e4m3_encode2(park[j][4] * inv, park[j][5] * inv) | (e4m3_encode2(park[j][6] * inv, park[j][7] * inv) << 16);
      }
      const int units = row_sum(code_units(w0, w1));
      if (m < M) {
        *reinterpret_cast<uint2*>(A + row * K + g * 128 + 8 * c) = make_uint2(w0, w1);
        if (c == 0) RS[row * G + g] = static_cast<float>(units) * 0x1p-9f;
      }
    }
  }
}

// Sum over the 16 lanes of a row (every lane gets it), in a fixed order.
__device__ __forceinline__ float row_sum_f(float v) {
  v += __builtin_bit_cast(float, dpp<0xB1>(__builtin_bit_cast(int, v)));
  v += __builtin_bit_cast(float, dpp<0x4E>(__builtin_bit_cast(int, v)));
  v += __builtin_bit_cast(float, dpp<0x141>(__builtin_bit_cast(int, v)));
  v += __builtin_bit_cast(float, dpp<0x140>(__builtin_bit_cast(int, v)));
  return v;
}

__device__ __forceinline__ uint32_t pack_f16x2(float lo, float hi) {
  const _Float16 a = static_cast<_Float16>(lo), b = static_cast<_Float16>(hi);   // round to nearest even
  return static_cast<uint32_t>(__builtin_bit_cast(uint16_t, a)) | (static_cast<uint32_t>(__builtin_bit_cast(uint16_t, b)) << 16);
}

// ---------------------------------------------------------------------------------------
// Fused producer: residual add + RMSNorm + the per-group rotate-quant, for all partitions. One
// 16-wave workgroup per quad of 4 tokens (lane: token t = lane/16, 8 channels 8c..8c+7 of each
// group, c = lane%16). The norm needs the whole row before any group is normalised, so each wave
// keeps its groups' residual-added values in registers (packed f16, <= 9 groups per wave, K <=
// 18432) while the row's sum of squares is reduced over the workgroup; it then writes the
// normalised row and runs, per partition, the per-group prologue on it: channel scale, the 8
// rotation layers through the wave's LDS quad image, group amax, e4m3 encode and code-domain
// row-sums, with the arithmetic of rotate_quant_kernel. For few tokens (kChunked) the groups
// of a quad are cut into chunks of 16, one workgroup each: every workgroup reads the whole row for
// the sum of squares (the same fixed order, so every chunk gets the same rstd) and keeps, writes
// and quantises only the group of its chunk that belongs to each wave.
template <int NPG, bool kChunked>
__global__ __launch_bounds__(64 * kTokWaves) void add_rms_rotate_quant_kernel(
    const uint16_t* __restrict__ x, int64_t ldx, const uint16_t* res, int64_t ldr,
    const uint16_t* __restrict__ nw, float eps, int gemma, int M, int K, int P,
    const uint2* __restrict__ rec, const uint16_t* __restrict__ cs, uint16_t* res_out, int64_t ldo,
    uint16_t* __restrict__ hs, uint8_t* __restrict__ A, float* __restrict__ ASG, float* __restrict__ RS) {
  __shared__ __align__(16) uint8_t qbuf[kTokWaves][kProQuadBytes];
  __shared__ float tred[kTokWaves][4];

  const int G = K >> 7, half = K >> 1;
  const int nchunks = kChunked ? (G + kTokWaves - 1) / kTokWaves : 1;
  const int m0 = 4 * (blockIdx.x / nchunks), chunk = blockIdx.x % nchunks;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63, t = lane >> 4, c = lane & 15;
  const int m = m0 + t, mld = min(m, M - 1);      // clamped: always a valid row to read
  uint8_t* const buf = qbuf[wave];
  uint8_t* const slot = buf + (9 * c) * 16 + 4 * t;
  // the group j of this wave that this workgroup keeps (all of them unless kChunked)
  auto mine = [&](int j) { return !kChunked || j == chunk; };

  // residual add; the new residual is stored as the page's producer returns it (res_out may be
  // res itself only in the unchunked form, where each element is read before the same lane writes
  // it; chunks read the whole row, so the launcher never runs them in place)
  uint32_t hp[NPG][4];
  float ss = 0.0f;
#pragma unroll
  for (int j = 0; j < NPG; ++j) {
    const int g = wave + kTokWaves * j;
    if (g < G) {
      const int col = g * 128 + 8 * c;
      const uint4 xs = *reinterpret_cast<const uint4*>(x + static_cast<size_t>(mld) * ldx + col);
      const uint4 rs = *reinterpret_cast<const uint4*>(res + static_cast<size_t>(mld) * ldr + col);
      const uint32_t xw[4] = {xs.x, xs.y, xs.z, xs.w}, rw[4] = {rs.x, rs.y, rs.z, rs.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        hp[j][i] = pack_f16x2(half_lo(xw[i]) + half_lo(rw[i]), half_hi(xw[i]) + half_hi(rw[i]));
        const float a = half_lo(hp[j][i]), b = half_hi(hp[j][i]);
        ss += a * a;
        ss += b * b;
      }
      if (m < M && mine(j))
        *reinterpret_cast<uint4*>(res_out + static_cast<size_t>(m) * ldo + col) = make_uint4(hp[j][0], hp[j][1], hp[j][2], hp[j][3]);
    }
  }
  // mean square over the row: the token's 16 lanes, then the waves in order
  ss = row_sum_f(ss);
  if (c == 0) tred[wave][t] = ss;
  __syncthreads();
  float tot = tred[0][t];
#pragma unroll
  for (int w = 1; w < kTokWaves; ++w) tot += tred[w][t];
  const float rstd = 1.0f / __builtin_sqrtf(tot / static_cast<float>(K) + eps);

  // normalised row: (h * rstd) * w', rounded once to f16
#pragma unroll
  for (int j = 0; j < NPG; ++j) {
    const int g = wave + kTokWaves * j;
    if (g < G && mine(j)) {
      const int col = g * 128 + 8 * c;
      const uint4 ws = *reinterpret_cast<const uint4*>(nw + col);
      const uint32_t ww[4] = {ws.x, ws.y, ws.z, ws.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float wl = gemma ? 1.0f + half_lo(ww[i]) : half_lo(ww[i]);
        const float wh = gemma ? 1.0f + half_hi(ww[i]) : half_hi(ww[i]);
        hp[j][i] = pack_f16x2((half_lo(hp[j][i]) * rstd) * wl, (half_hi(hp[j][i]) * rstd) * wh);
      }
      if (m < M)
        *reinterpret_cast<uint4*>(hs + static_cast<size_t>(m) * K + col) = make_uint4(hp[j][0], hp[j][1], hp[j][2], hp[j][3]);
    }
  }

  // the per-group prologue on the normalised row, for each group and partition
#pragma unroll
  for (int j = 0; j < NPG; ++j) {
    const int g = wave + kTokWaves * j;
    if (g >= G || !mine(j)) continue;
    for (int p = 0; p < P; ++p) {
      const uint2* const recp = rec + static_cast<size_t>(p) * PQ_LAYERS * half + lane + g * 64;
      const size_t row = static_cast<size_t>(p) * M + m;
      uint2 q[PQ_LAYERS];
#pragma unroll
      for (int r = 0; r < PQ_LAYERS; ++r) q[r] = recp[static_cast<size_t>(r) * half];
      const uint32_t* cw = reinterpret_cast<const uint32_t*>(cs + static_cast<size_t>(p) * K + g * 128 + 8 * c);
      const uint32_t cs4[4] = {cw[0], cw[1], cw[2], cw[3]};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        *reinterpret_cast<float*>(slot + (2 * i) * 16) = mul_hh<false>(hp[j][i], cs4[i]);
        *reinterpret_cast<float*>(slot + (2 * i + 1) * 16) = mul_hh<true>(hp[j][i], cs4[i]);
      }
      __builtin_amdgcn_wave_barrier();
      rot_layers_q<1, kProQuadBytes>(buf, q);
      float v[8];
      float gmax = 0.0f;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        v[i] = *reinterpret_cast<const float*>(slot + i * 16);
        gmax = __builtin_fmaxf(gmax, __builtin_fabsf(v[i]));
      }
      __builtin_amdgcn_wave_barrier();
      const float amax = row_max(gmax);               // over the token's 16 lanes: the group
      const float asg = amax * 0x1.24924ap-9f;        // fl32(1/448)
      const float inv = recip_rn(asg);
      const bool inv_bad = __builtin_fabsf(inv) == __builtin_inff();
      float sv[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) sv[i] = v[i] * inv + 0.0f;
      uint32_t w0 = pack4(sv[0], sv[1], sv[2], sv[3]), w1 = pack4(sv[4], sv[5], sv[6], sv[7]);
      const uint32_t bad = (nan_bytes(w0) | nan_bytes(w1)) | (inv_bad ? 1u : 0u);
      if (__builtin_amdgcn_ballot_w64(bad != 0)) {
        // rare: a NaN or out-of-range value in the wave; the full encoder
        w0 = e4m3_encode2(v[0] * inv, v[1] * inv) | (e4m3_encode2(v[2] * inv, v[3] * inv) << 16);
        w1 = e4m3_encode2(v[4] * inv, v[5] * inv) | (e4m3_encode2(v[6] * inv, v[7] * inv) << 16);
      }
      const int units = row_sum(code_units(w0, w1));
      if (m < M) {
        *reinterpret_cast<uint2*>(A + row * K + g * 128 + 8 * c) = make_uint2(w0, w1);
        if (c == 0) {
          ASG[row * G + g] = asg;
          RS[row * G + g] = static_cast<float>(units) * 0x1p-9f;
        }
      }
    }
  }
}

// Verification hook: out[i] = bf16 bits of x[i] with the rounding of the GEMM outputs, two elements per thread
// through the packed convert of the epilogues, a last odd element through the single one.
__global__ void bf16_round_kernel(const float* __restrict__ x, uint16_t* __restrict__ out, int64_t n) {
  const int64_t i = 2 * (static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x);
  if (i + 1 < n) {
    const uint32_t w = bf16x2_rn(x[i], x[i + 1]);
    out[i] = static_cast<uint16_t>(w);
    out[i + 1] = static_cast<uint16_t>(w >> 16);
  } else if (i < n) {
    out[i] = static_cast<uint16_t>(f32_to_bf16(x[i]));
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

// ws_d (kWs): the prefill GEMM's workspace, laid out as pq_gemm_workspace_bytes sizes it.
template <bool kI8, bool kWs = false>
static int rotate_quant_launch(const char* what, const uint16_t* x_d, int64_t ldx, int M, int K, int P,
                               const void* rec_d, const uint16_t* cs_d, uint8_t* a_d, float* asg_d, float* rs_d,
                               pq_stream_t stream, void* ws_d = nullptr) {
  if (M < 0) return set_error(PQ_ERR_SHAPE, "%s: M=%d < 0", what, M);
  if (K <= 0 || K % PQ_GROUP || K > (1 << 24)) return set_error(PQ_ERR_SHAPE, "%s: K=%d must be a positive multiple of 128", what, K);
  if (P < 1 || P > PQ_MAX_PARTITIONS) return set_error(PQ_ERR_PARTITION, "%s: P=%d must be in 1..3", what, P);
  if (ldx < K || (ldx & 1)) return set_error(PQ_ERR_SHAPE, "%s: ldx=%lld must be even and >= K=%d", what, static_cast<long long>(ldx), K);
  if (M == 0) return PQ_OK;
  if (!x_d || !rec_d || !cs_d || !a_d || !asg_d || !rs_d) return set_error(PQ_ERR_NULL, "%s: NULL pointer", what);
  if (!aligned(x_d, 4) || !aligned(rec_d, 8) || !aligned(cs_d, 4) || !aligned(a_d, 16) || !aligned(asg_d, 4) || !aligned(rs_d, 4))
    return set_error(PQ_ERR_ALIGN, "%s: misaligned pointer", what);
  const int G = K / PQ_GROUP;
  // tokens per wave unit: a multiple of the 8-token step, as few as keep the unit count near
  // kProUnits (short units for small M, at most 256 tokens)
  const int64_t rows = static_cast<int64_t>(G) * P;
  const int64_t want = (static_cast<int64_t>(M) * rows + kProUnits - 1) / kProUnits;
  const int tok = static_cast<int>(std::min<int64_t>(256, std::max<int64_t>(kProStep, (want + kProStep - 1) / kProStep * kProStep)));
  const int64_t chunks = (M + tok - 1) / tok;
  const int64_t units = chunks * rows;
  const int64_t blocks = (units + kProWaves - 1) / kProWaves;
  if (units > 0x7FFFFFFF) return set_error(PQ_ERR_SHAPE, "%s: problem too large", what);
  const bool vec16 = aligned(x_d, 16) && (ldx % 8) == 0;
  uint16_t* zpa = nullptr;
  float* asgt = nullptr;
  if constexpr (kWs) {
    zpa = static_cast<uint16_t*>(ws_d);
    asgt = reinterpret_cast<float*>(static_cast<uint8_t*>(ws_d) + zpe_act_bytes(M, G, PQ_MAX_PARTITIONS));
  }
  auto kern = vec16 ? rotate_quant_kernel<true, kI8, kWs> : rotate_quant_kernel<false, kI8, kWs>;
  hipLaunchKernelGGL(kern, dim3(static_cast<unsigned>(blocks)), dim3(256), 0,
                     reinterpret_cast<hipStream_t>(stream), x_d, ldx, M, K, P,
                     static_cast<const uint2*>(rec_d), cs_d, a_d, asg_d, rs_d, tok,
                     static_cast<int>(chunks), zpa, asgt);
  return launch_status(what);
}

}  // namespace pq

extern "C" {

int pq_rotate_quant(const uint16_t* x_d, int64_t ldx, int M, int K, int P, const void* rec_d,
                    const uint16_t* cs_d, uint8_t* a_d, float* asg_d, float* rs_d,
                    pq_stream_t stream) {
  pq::clear_error();
  return pq::rotate_quant_launch<false>("pq_rotate_quant", x_d, ldx, M, K, P, rec_d, cs_d, a_d, asg_d, rs_d, stream);
}

int pq_rotate_quant_for_gemm(const uint16_t* x_d, int64_t ldx, int M, int K, int P, const void* rec_d,
                             const uint16_t* cs_d, uint8_t* a_d, float* asg_d, float* rs_d, void* ws_d,
                             size_t ws_bytes, pq_stream_t stream) {
  using namespace pq;
  clear_error();
  const char* what = "pq_rotate_quant_for_gemm";
  if (M <= 16 || K <= 0 || K % PQ_GROUP)   // no prefill operands: the plain prologue (or its errors)
    return rotate_quant_launch<false>(what, x_d, ldx, M, K, P, rec_d, cs_d, a_d, asg_d, rs_d, stream);
  // the prefill GEMM's own limit (32-bit activation offsets); it also keeps the zero-point
  // operand's element indices (3 M K / 128 per partition) within 32 bits
  if (static_cast<int64_t>(M) * K > 0x7FFFFFFF)
    return set_error(PQ_ERR_SHAPE, "%s: M * K too large for one call (split the rows)", what);
  if (ws_bytes < pq_gemm_workspace_bytes(M, 0, K)) return set_error(PQ_ERR_WORKSPACE, "%s: workspace too small", what);
  if (!ws_d) return set_error(PQ_ERR_NULL, "%s: NULL workspace", what);
  if (!aligned(ws_d, 16)) return set_error(PQ_ERR_ALIGN, "%s: misaligned workspace", what);
  return rotate_quant_launch<false, true>(what, x_d, ldx, M, K, P, rec_d, cs_d, a_d, asg_d, rs_d, stream, ws_d);
}

int pq_rotate_quant_i8(const uint16_t* x_d, int64_t ldx, int M, int K, int P, const void* rec_d,
                       const uint16_t* cs_d, int8_t* a_d, float* asg_d, float* rs_d,
                       pq_stream_t stream) {
  pq::clear_error();
  return pq::rotate_quant_launch<true>("pq_rotate_quant_i8", x_d, ldx, M, K, P, rec_d, cs_d,
                                       reinterpret_cast<uint8_t*>(a_d), asg_d, rs_d, stream);
}

int pq_rotate_quant_tok(const uint16_t* x_d, int64_t ldx, int M, int K, int P, const void* rec_d,
                        const uint16_t* cs_d, uint8_t* a_d, float* as_d, float* rs_d,
                        pq_stream_t stream) {
  using namespace pq;
  clear_error();
  if (M < 0) return set_error(PQ_ERR_SHAPE, "pq_rotate_quant_tok: M=%d < 0", M);
  if (K <= 0 || K % PQ_GROUP || K > kTokWaves * 9 * PQ_GROUP)
    return set_error(PQ_ERR_SHAPE, "pq_rotate_quant_tok: K=%d must be a positive multiple of 128, at most %d", K,
                     kTokWaves * 9 * PQ_GROUP);
  if (P < 1 || P > PQ_MAX_PARTITIONS) return set_error(PQ_ERR_PARTITION, "pq_rotate_quant_tok: P=%d must be in 1..3", P);
  if (ldx < K || (ldx & 1)) return set_error(PQ_ERR_SHAPE, "pq_rotate_quant_tok: ldx=%lld must be even and >= K=%d", static_cast<long long>(ldx), K);
  if (M == 0) return PQ_OK;
  if (!x_d || !rec_d || !cs_d || !a_d || !as_d || !rs_d) return set_error(PQ_ERR_NULL, "pq_rotate_quant_tok: NULL pointer");
  if (!aligned(x_d, 4) || !aligned(rec_d, 8) || !aligned(cs_d, 4) || !aligned(a_d, 16) || !aligned(as_d, 4) || !aligned(rs_d, 4))
    return set_error(PQ_ERR_ALIGN, "pq_rotate_quant_tok: misaligned pointer");
  const int G = K / PQ_GROUP;
  const int64_t blocks = static_cast<int64_t>(P) * ((M + 3) / 4);
  if (blocks > 0x7FFFFFFF) return set_error(PQ_ERR_SHAPE, "pq_rotate_quant_tok: problem too large");
  const bool vec16 = aligned(x_d, 16) && (ldx % 8) == 0;
  const int npg = (G + kTokWaves - 1) / kTokWaves;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const uint2* rec = static_cast<const uint2*>(rec_d);
#define PQ_TOK_LAUNCH(NPG)                                                                          \
  do {                                                                                              \
    auto kern = vec16 ? rotate_quant_tok_kernel<NPG, true> : rotate_quant_tok_kernel<NPG, false>;   \
    hipLaunchKernelGGL(kern, dim3(static_cast<unsigned>(blocks)), dim3(64 * kTokWaves), 0, s, x_d, ldx, \
                       M, K, P, rec, cs_d, a_d, as_d, rs_d);                                        \
  } while (0)
  if (npg <= 1) PQ_TOK_LAUNCH(1);
  else if (npg <= 3) PQ_TOK_LAUNCH(3);
  else if (npg <= 5) PQ_TOK_LAUNCH(5);
  else PQ_TOK_LAUNCH(9);
#undef PQ_TOK_LAUNCH
  return launch_status("pq_rotate_quant_tok");
}

int pq_add_rms_rotate_quant(const uint16_t* x_d, int64_t ldx, const uint16_t* res_d, int64_t ldr,
                            const uint16_t* w_d, float eps, int gemma, int M, int K, int P,
                            const void* rec_d, const uint16_t* cs_d, uint16_t* res_out_d, int64_t ldo,
                            uint16_t* hs_d, uint8_t* a_d, float* asg_d, float* rs_d, pq_stream_t stream) {
  using namespace pq;
  clear_error();
  const char* what = "pq_add_rms_rotate_quant";
  if (M < 0) return set_error(PQ_ERR_SHAPE, "%s: M=%d < 0", what, M);
  if (K <= 0 || K % PQ_GROUP || K > kTokWaves * 9 * PQ_GROUP)
    return set_error(PQ_ERR_SHAPE, "%s: K=%d must be a positive multiple of 128, at most %d", what, K, kTokWaves * 9 * PQ_GROUP);
  if (P < 1 || P > PQ_MAX_PARTITIONS) return set_error(PQ_ERR_PARTITION, "%s: P=%d must be in 1..3", what, P);
  if (ldx < K || ldr < K || ldo < K || ldx % 8 || ldr % 8 || ldo % 8)
    return set_error(PQ_ERR_SHAPE, "%s: row strides must be multiples of 8 and >= K=%d", what, K);
  if (!(eps > 0.0f) || !(eps < __builtin_inff())) return set_error(PQ_ERR_SHAPE, "%s: eps must be positive and finite", what);
  if (M == 0) return PQ_OK;
  if (!x_d || !res_d || !w_d || !rec_d || !cs_d || !res_out_d || !hs_d || !a_d || !asg_d || !rs_d)
    return set_error(PQ_ERR_NULL, "%s: NULL pointer", what);
  if (!aligned(x_d, 16) || !aligned(res_d, 16) || !aligned(w_d, 16) || !aligned(res_out_d, 16) || !aligned(hs_d, 16) ||
      !aligned(rec_d, 8) || !aligned(cs_d, 4) || !aligned(a_d, 16) || !aligned(asg_d, 4) || !aligned(rs_d, 4))
    return set_error(PQ_ERR_ALIGN, "%s: misaligned pointer", what);
  const int G = K / PQ_GROUP;
  const int npg = (G + kTokWaves - 1) / kTokWaves;
  // The new residual may replace the old one in place (res_out_d == res_d, ldo == ldr); any other
  // overlap of the two row ranges is rejected.
  const uintptr_t r0 = reinterpret_cast<uintptr_t>(res_d), o0 = reinterpret_cast<uintptr_t>(res_out_d);
  const uintptr_t r1 = r0 + 2 * (static_cast<uintptr_t>(M - 1) * static_cast<uintptr_t>(ldr) + static_cast<uintptr_t>(K));
  const uintptr_t o1 = o0 + 2 * (static_cast<uintptr_t>(M - 1) * static_cast<uintptr_t>(ldo) + static_cast<uintptr_t>(K));
  const bool inplace = r0 < o1 && o0 < r1;
  if (inplace && (o0 != r0 || ldo != ldr))
    return set_error(PQ_ERR_SHAPE, "%s: res_out overlaps res without being the same rows (res_out == res and ldo == ldr)", what);
  // few tokens: one workgroup per (quad, chunk of 16 groups), each reading the whole row for its
  // sum of squares; many tokens, or an in-place residual: one workgroup per quad. In the chunked
  // form every chunk reads residual elements that other chunks write, so it cannot run in place;
  // with one workgroup per quad each element is read by the lane that later writes it.
  const bool chunked = M <= 64 && !inplace;
  const int64_t blocks = static_cast<int64_t>((M + 3) / 4) * (chunked ? npg : 1);
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const uint2* rec = static_cast<const uint2*>(rec_d);
#define PQ_PROD_LAUNCH(NPG)                                                                           \
  do {                                                                                                \
    auto kern = chunked ? add_rms_rotate_quant_kernel<NPG, true> : add_rms_rotate_quant_kernel<NPG, false>; \
    hipLaunchKernelGGL(kern, dim3(static_cast<unsigned>(blocks)), dim3(64 * kTokWaves), 0, s, x_d, ldx, \
                       res_d, ldr, w_d, eps, gemma ? 1 : 0, M, K, P, rec, cs_d, res_out_d, ldo, hs_d,   \
                       a_d, asg_d, rs_d);                                                             \
  } while (0)
  if (npg <= 1) PQ_PROD_LAUNCH(1);
  else if (npg <= 3) PQ_PROD_LAUNCH(3);
  else if (npg <= 5) PQ_PROD_LAUNCH(5);
  else PQ_PROD_LAUNCH(9);
#undef PQ_PROD_LAUNCH
  return launch_status(what);
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

int pq_bf16_round(const float* x_d, uint16_t* out_d, int64_t n, pq_stream_t stream) {
  using namespace pq;
  clear_error();
  if (n < 0) return set_error(PQ_ERR_SHAPE, "pq_bf16_round: n < 0");
  if (n == 0) return PQ_OK;
  if (!x_d || !out_d) return set_error(PQ_ERR_NULL, "pq_bf16_round: NULL pointer");
  if (!aligned(x_d, 4) || !aligned(out_d, 2)) return set_error(PQ_ERR_ALIGN, "pq_bf16_round: misaligned pointer");
  const int64_t threads = (n + 1) / 2;
  const int64_t blocks = (threads + 255) / 256;
  if (blocks > 0x7FFFFFFF) return set_error(PQ_ERR_SHAPE, "pq_bf16_round: n too large");
  hipLaunchKernelGGL(bf16_round_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0,
                     reinterpret_cast<hipStream_t>(stream), x_d, out_d, n);
  return launch_status("pq_bf16_round");
}

}  // extern "C"
