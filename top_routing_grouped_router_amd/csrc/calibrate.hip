// Calibration kernels: the achievable rates of this device that the layer's kernels are
// compared with (the published peaks assume clocks the chip does not hold under sustained
// matrix load). Neither is part of the layer.
//
//   * mfma_loop_kernel: one workgroup of 8 wavefronts (2 per SIMD, as the GEMMs run) per
//     compute unit; each wavefront issues rounds of 8 independent v_mfma_f32_32x32x16_bf16 on
//     register operands, so the matrix pipes never wait on memory. The operands are fixed
//     per-lane bit patterns of values in [-1, 1) (not zeros: all-zero operands draw less power,
//     and the loop then runs at the published 2.4 GHz peak, which real data does not). Operands
//     are not modified inside the loop: rewriting registers that in-flight MFMAs still read
//     stalls the matrix pipe (a rotating variant measured 1.23 PFLOP/s against 1.97).
//   * mfma_mx_loop_kernel: the same loop on v_mfma_scale_f32_32x32x64_f8f6f4 (E4M3 operands,
//     unit block scales), the product the MXFP8 expert GEMMs run.
//   * copy_kernel: a grid-stride copy, 4 non-temporal 16-byte loads in flight per thread before
//     the stores (one load per thread measured 5.0 TB/s, four 6.0 TB/s of read + write traffic;
//     torch's device copy 5.1 TB/s).
#include <algorithm>

#include "common.hpp"

namespace moe {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef short i16x8 __attribute__((ext_vector_type(8)));

constexpr int kLoopWaves = 8;

__global__ __launch_bounds__(kLoopWaves * kWave) __attribute__((amdgpu_waves_per_eu(2))) void mfma_loop_kernel(
    float* __restrict__ out, int64_t iters) {
  const int lane = threadIdx.x & (kWave - 1);
  i16x8 ra, rb;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    // bf16 bit patterns of values in [-1, 1): sign, exponent 120..126, varied mantissa
    const int u = (lane * 37 + i * 11 + threadIdx.x / kWave * 5) & 127;
    ra[i] = static_cast<short>(((u & 1) << 15) | ((120 + (u >> 4) % 7) << 7) | (u & 0x7f));
    rb[i] = static_cast<short>((((u >> 1) & 1) << 15) | ((121 + (u >> 3) % 6) << 7) | ((u * 3) & 0x7f));
  }
  f32x16 acc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[j][r] = 0.f;
  const bf16x8 a = __builtin_bit_cast(bf16x8, ra), b = __builtin_bit_cast(bf16x8, rb);
  for (int64_t it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[j], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) s += acc[j][r];
  if (lane == 0) out[static_cast<int64_t>(blockIdx.x) * kLoopWaves + threadIdx.x / kWave] = s;
}

typedef int i32x8 __attribute__((ext_vector_type(8)));

// The same loop on the block-scaled FP8 products the MXFP8 expert GEMMs use
// (v_mfma_scale_f32_32x32x64_f8f6f4, E4M3 operands, unit E8M0 scales).
__global__ __launch_bounds__(kLoopWaves * kWave) __attribute__((amdgpu_waves_per_eu(2))) void mfma_mx_loop_kernel(
    float* __restrict__ out, int64_t iters) {
  const int lane = threadIdx.x & (kWave - 1);
  i32x8 ra, rb;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    // four E4M3 codes per dword, each of magnitude in [2^-3, 2^1): exponent field 4..7
    uint32_t wa = 0, wb = 0;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const int u = (lane * 29 + i * 7 + b * 3 + threadIdx.x / kWave) & 63;
      wa |= static_cast<uint32_t>(((u & 1) << 7) | ((4 + (u >> 4) % 4) << 3) | (u & 7)) << (8 * b);
      wb |= static_cast<uint32_t>((((u >> 1) & 1) << 7) | ((4 + (u >> 3) % 4) << 3) | ((u * 5) & 7)) << (8 * b);
    }
    ra[i] = static_cast<int>(wa);
    rb[i] = static_cast<int>(wb);
  }
  f32x16 acc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[j][r] = 0.f;
  for (int64_t it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < 8; ++j)
      acc[j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(ra, rb, acc[j], 0, 0, 0, 127, 0, 127);
  }
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) s += acc[j][r];
  if (lane == 0) out[static_cast<int64_t>(blockIdx.x) * kLoopWaves + threadIdx.x / kWave] = s;
}

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kCopyUnroll = 4;

__global__ __launch_bounds__(256) void copy_kernel(const u32x4* __restrict__ src, u32x4* __restrict__ dst,
                                                   int64_t n16) {
  const int64_t stride = static_cast<int64_t>(gridDim.x) * 256 * kCopyUnroll;
  for (int64_t i0 = static_cast<int64_t>(blockIdx.x) * 256 * kCopyUnroll + threadIdx.x; i0 < n16; i0 += stride) {
    u32x4 v[kCopyUnroll];
#pragma unroll
    for (int u = 0; u < kCopyUnroll; ++u)
      if (i0 + u * 256 < n16) v[u] = __builtin_nontemporal_load(src + i0 + u * 256);
#pragma unroll
    for (int u = 0; u < kCopyUnroll; ++u)
      if (i0 + u * 256 < n16) __builtin_nontemporal_store(v[u], dst + i0 + u * 256);
  }
}

}  // namespace

int64_t mfma_loop_waves() { return static_cast<int64_t>(device_cu_count()) * kLoopWaves; }

double mfma_loop_flops(int64_t iters, bool mx) {
  return static_cast<double>(mfma_loop_waves()) * static_cast<double>(iters) * 8.0 *
         (mx ? 2.0 * 32 * 32 * 64 : 2.0 * 32 * 32 * 16);
}

hipError_t launch_mfma_loop(float* out, int64_t iters, bool mx, hipStream_t s) {
  const dim3 g(static_cast<unsigned>(device_cu_count())), b(kLoopWaves * kWave);
  if (mx)
    hipLaunchKernelGGL(mfma_mx_loop_kernel, g, b, 0, s, out, iters);
  else
    hipLaunchKernelGGL(mfma_loop_kernel, g, b, 0, s, out, iters);
  return hipGetLastError();
}

hipError_t launch_copy(const void* src, void* dst, int64_t bytes, hipStream_t s) {
  const int64_t n16 = bytes / 16;
  const unsigned grid =
      static_cast<unsigned>(std::min<int64_t>((n16 + 256 * kCopyUnroll - 1) / (256 * kCopyUnroll), int64_t(device_cu_count()) * 32));
  hipLaunchKernelGGL(copy_kernel, dim3(grid), dim3(256), 0, s, static_cast<const u32x4*>(src), static_cast<u32x4*>(dst),
                     n16);
  return hipGetLastError();
}

}  // namespace moe
