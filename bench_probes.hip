// Measured ceilings for the bench's roofline fractions on gfx950 (bench tooling, not part of the
// library): a plain HBM read of a buffer far larger than the last-level cache, and a stream of
// independent fp8 16x16x128 matrix-core instructions. bench.py times them with HIP events and
// reports each kernel's fraction against both these and the datasheet peaks.
#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Each thread reads 4 x 16 bytes per step, the four a grid-width apart (coalesced per wave, four
// requests in flight per thread), and folds them with XOR; one word per block keeps the loads
// alive. The buffer length is a whole number of grid steps (checked on the host).
__global__ __launch_bounds__(256) void read_probe_kernel(const u32x4* __restrict__ p, size_t steps,
                                                         uint32_t* __restrict__ out) {
  const size_t width = static_cast<size_t>(gridDim.x) * blockDim.x;
  size_t i = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  u32x4 acc = {0u, 0u, 0u, 0u};
  for (size_t s = 0; s < steps; ++s, i += 4 * width) {
    const u32x4 a = __builtin_nontemporal_load(p + i);
    const u32x4 b = __builtin_nontemporal_load(p + i + width);
    const u32x4 c = __builtin_nontemporal_load(p + i + 2 * width);
    const u32x4 d = __builtin_nontemporal_load(p + i + 3 * width);
    acc ^= a ^ b ^ c ^ d;
  }
  const uint32_t v = acc.x ^ acc.y ^ acc.z ^ acc.w;
  if (threadIdx.x == 0) out[blockIdx.x] = v;
}

// Every wave issues `iters` rounds of 8 independent fp8 16x16x128 products (8 accumulators), no
// other work; operands are fixed e4m3 bytes of ordinary magnitude.
__global__ __launch_bounds__(256) void mfma_probe_kernel(int iters, float* __restrict__ out) {
  const int t = threadIdx.x;
  v8i a, b;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    a[j] = static_cast<int>(0x38303428u + 0x01010101u * static_cast<uint32_t>((t + j) & 7));
    b[j] = static_cast<int>(0x3A322C24u + 0x01010101u * static_cast<uint32_t>((t * 3 + j) & 7));
  }
  v4f c[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) c[j] = v4f{0.f, 0.f, 0.f, 0.f};
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int j = 0; j < 8; ++j) c[j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c[j], 0, 0, 0, 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j) s += c[j][0] + c[j][1] + c[j][2] + c[j][3];
  out[static_cast<size_t>(blockIdx.x) * blockDim.x + t] = s;
}

extern "C" {

// Reads `bytes` from buf_d (16-byte aligned; bytes a multiple of 4 * 16 * 256 * blocks) with
// `blocks` workgroups of 256 threads; out_d holds `blocks` words. Returns 0, or -1 on a bad
// argument (nothing launched), -2 if the launch failed.
int probe_read(const void* buf_d, size_t bytes, int blocks, uint32_t* out_d, hipStream_t stream) {
  const size_t per_step = static_cast<size_t>(blocks) * 256 * 4 * 16;
  if (!buf_d || !out_d || blocks <= 0 || bytes == 0 || bytes % per_step || reinterpret_cast<uintptr_t>(buf_d) % 16)
    return -1;
  hipLaunchKernelGGL(read_probe_kernel, dim3(blocks), dim3(256), 0, stream, static_cast<const u32x4*>(buf_d),
                     bytes / per_step, out_d);
  return hipGetLastError() == hipSuccess ? 0 : -2;
}

// `blocks` workgroups of 4 waves, each wave 8 * iters fp8 16x16x128 products (65536 flops each);
// out_d holds blocks * 256 floats.
int probe_mfma(int blocks, int iters, float* out_d, hipStream_t stream) {
  if (!out_d || blocks <= 0 || iters <= 0) return -1;
  hipLaunchKernelGGL(mfma_probe_kernel, dim3(blocks), dim3(256), 0, stream, iters, out_d);
  return hipGetLastError() == hipSuccess ? 0 : -2;
}

}  // extern "C"
