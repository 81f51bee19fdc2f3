// MXFP8 quantisation of bf16 rows for the expert matmuls.
//
// "Как устроен Olmo-core 3: обучение больших MoE-моделей", sections "Rowwise FP8 и MXFP8" and
// "Как сравнивали и что получилось": the grouped expert matmuls can run in MXFP8. The page does
// not define the format; it is read as the OCP microscaling format: 32 consecutive elements
// along the contraction dimension share one E8M0 scale 2^(s - 127), the elements are FP8 E4M3
// (bias 7, 3 mantissa bits, max 448). s - 127 = floor(log2(amax of the block)) - 8, clamped to
// [-127, 127]; an all-zero block gets s = 0. Elements = value / 2^(s - 127) (an exact
// power-of-two scaling) rounded to nearest-even E4M3, saturating at +-448.
//
// gfx950's v_cvt_pk_fp8_f32 converts to OCP E4M3 with round-to-nearest-even and returns NaN
// above 464, so values are clamped to +-448 first; the result is then the saturating rounding.
// Inputs must be finite.
//
// One thread per block of 32: 64 bytes in, 32 code bytes and one scale byte out.
#include <math.h>

#include "common.hpp"

namespace moe {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256) void mx_quantize_kernel(const uint16_t* __restrict__ x, int64_t rows, int64_t cols,
                                                          uint8_t* __restrict__ codes, uint8_t* __restrict__ scales) {
  const int64_t nb = cols / 32;
  const int64_t blk = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (blk >= rows * nb) return;
  const int64_t r = blk / nb, b = blk - r * nb;
  const u32x4* src = reinterpret_cast<const u32x4*>(x + r * cols + b * 32);
  float v[32];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const u32x4 w = src[q];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[8 * q + 2 * i] = __uint_as_float(w[i] << 16);
      v[8 * q + 2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
    }
  }
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(v[i]));
  const int s = mx_scale_code(amax);
  const int sh = 127 - s;              // multiply by 2^sh: exact
  uint32_t out[8];
#pragma unroll
  for (int i = 0; i < 8; ++i)
    out[i] = pack4_e4m3(ldexpf(v[4 * i], sh), ldexpf(v[4 * i + 1], sh), ldexpf(v[4 * i + 2], sh),
                        ldexpf(v[4 * i + 3], sh));
  u32x4* dst = reinterpret_cast<u32x4*>(codes + r * cols + b * 32);
  dst[0] = u32x4{out[0], out[1], out[2], out[3]};
  dst[1] = u32x4{out[4], out[5], out[6], out[7]};
  scales[r * nb + b] = static_cast<uint8_t>(s);
}

}  // namespace

hipError_t launch_mx_quantize(const void* x, int64_t rows, int64_t cols, uint8_t* codes, uint8_t* scales,
                              hipStream_t s) {
  const int64_t n = rows * (cols / 32);
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(mx_quantize_kernel, dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256), 0, s,
                     static_cast<const uint16_t*>(x), rows, cols, codes, scales);
  return hipGetLastError();
}

}  // namespace moe
