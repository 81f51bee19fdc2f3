// Skinny dense bf16 GEMM for few token rows (M <= 64): the latent projections of a
// decode-sized batch ("Как устроен Olmo-core 3: обучение больших MoE-моделей", section
// "Латентная проекция экспертов": dense down-projection d_model -> latent_dim and
// up-projection back, fp32 accumulation, output in the layer dtype).
//
// With 64 token rows the product is weight streaming: every weight row is read once and meets
// at most 64 tokens, so the bound is HBM and the work has to be spread over the whole chip.
// Design:
//   * A workgroup owns 64 weight rows x all (<= 64) token rows x one k-slice; the contraction
//     is split over S workgroups (k-slices) and, inside a workgroup, over its 4 wavefronts.
//   * No LDS staging of operands: each lane loads its v_mfma_f32_32x32x16_bf16 fragments
//     straight from global memory. The order of k inside a 64-k block is permuted the same way
//     for both operands (lane half h takes the 32 contiguous elements [32h, 32h + 32) of the
//     block, 16 bytes per MFMA step), so each lane reads 64 contiguous bytes of a row and the
//     two halves of a wavefront cover each row's whole 128-byte line.
//   * The four wavefronts' fp32 tiles are added in LDS in wavefront order; with S = 1 the sum
//     is rounded to bf16 and stored, otherwise it goes to fp32 partial plane `split`, and a
//     second kernel adds the S planes in plane order and rounds. Fixed orders throughout, so
//     results are bitwise reproducible.
#include <algorithm>

#include "common.hpp"

namespace moe {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kSkM = 64;     // token rows (padded)
constexpr int kSkN = 64;     // weight rows per workgroup
constexpr int kSkPad = 68;   // LDS row stride in floats: rows start 4 banks apart
constexpr int kSkMaxSplit = 16;

struct SkinnyArgs {
  const uint16_t* A;  // (M, K) token rows
  int64_t lda;
  int64_t M;
  const uint16_t* B;  // (N, K) weight rows
  int64_t ldb;
  int64_t N;
  int64_t K;
  uint16_t* C;        // (M, N)
  int64_t ldc;
  float* partials;    // (S, M, N) fp32 when S > 1
  int S;
};

__global__ __launch_bounds__(256) void gemm_skinny_kernel(SkinnyArgs a) {
  __shared__ __attribute__((aligned(16))) float red[4 * kSkM * kSkPad];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t n0 = static_cast<int64_t>(blockIdx.x) * kSkN;
  const int sp = blockIdx.y;
  const int nk = static_cast<int>(a.K / 64);
  const int kb = static_cast<int>(static_cast<int64_t>(sp) * nk / a.S);
  const int ke = static_cast<int>(static_cast<int64_t>(sp + 1) * nk / a.S);
  const int wb = kb + wave * (ke - kb) / 4, we = kb + (wave + 1) * (ke - kb) / 4;

  const int r = lane & 31, h = lane >> 5;
  // Rows of this lane: weight rows n0 + 32u + r and token rows 32v + r (u, v = 0, 1), clamped
  // into the operands; padded token rows compute values that are never stored.
  const uint16_t* wrow[2];
  const uint16_t* trow[2];
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    wrow[u] = a.B + min(n0 + 32 * u + r, a.N - 1) * a.ldb + 32 * h;
    trow[u] = a.A + min(static_cast<int64_t>(32 * u + r), a.M - 1) * a.lda + 32 * h;
  }

  f32x16 acc[2][2];
#pragma unroll
  for (int u = 0; u < 2; ++u)
#pragma unroll
    for (int v = 0; v < 2; ++v)
#pragma unroll
      for (int q = 0; q < 16; ++q) acc[u][v][q] = 0.f;

  // Two 64-k blocks per iteration: 32 independent 16-byte loads per lane, then 16 MFMAs.
  for (int kt = wb; kt < we; kt += 2) {
    u32x4 fw[2][2][4], ft[2][2][4];
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      const int kk = min(kt + b, we - 1) * 64;  // a lone last block is loaded twice, used once
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          fw[b][u][s] = *reinterpret_cast<const u32x4*>(wrow[u] + kk + 8 * s);
          ft[b][u][s] = *reinterpret_cast<const u32x4*>(trow[u] + kk + 8 * s);
        }
    }
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      if (kt + b >= we) break;
#pragma unroll
      for (int s = 0; s < 4; ++s)
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
          for (int v = 0; v < 2; ++v)
            acc[u][v] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, fw[b][u][s]),
                                                                __builtin_bit_cast(bf16x8, ft[b][v][s]),
                                                                acc[u][v], 0, 0, 0);
    }
  }

  // Lane holds token 32v + r and weight rows 32u + 8g + 4h + {0..3} of register group g.
  float* mine = red + wave * kSkM * kSkPad;
#pragma unroll
  for (int u = 0; u < 2; ++u)
#pragma unroll
    for (int v = 0; v < 2; ++v)
#pragma unroll
      for (int g = 0; g < 4; ++g)
        *reinterpret_cast<float4*>(mine + (32 * v + r) * kSkPad + 32 * u + 8 * g + 4 * h) =
            make_float4(acc[u][v][4 * g], acc[u][v][4 * g + 1], acc[u][v][4 * g + 2], acc[u][v][4 * g + 3]);
  __syncthreads();

  // Thread: token m, columns [c0, c0 + 16) of the tile; wavefront tiles added in order.
  const int m = tid >> 2, c0 = (tid & 3) * 16;
  if (m >= a.M) return;
  float o[16];
#pragma unroll
  for (int q = 0; q < 16; q += 4) {
    float4 acc4 = *reinterpret_cast<const float4*>(red + m * kSkPad + c0 + q);
#pragma unroll
    for (int w = 1; w < 4; ++w) {
      const float4 x = *reinterpret_cast<const float4*>(red + w * kSkM * kSkPad + m * kSkPad + c0 + q);
      acc4.x += x.x;
      acc4.y += x.y;
      acc4.z += x.z;
      acc4.w += x.w;
    }
    o[q] = acc4.x;
    o[q + 1] = acc4.y;
    o[q + 2] = acc4.z;
    o[q + 3] = acc4.w;
  }
  const int64_t col = n0 + c0;
  if (col >= a.N) return;  // N is a multiple of 64: whole 16-column groups are in or out
  if (a.S == 1) {
    uint32_t pk[8];
#pragma unroll
    for (int q = 0; q < 8; ++q)
      pk[q] = f32_to_bf16_bits(o[2 * q]) | (static_cast<uint32_t>(f32_to_bf16_bits(o[2 * q + 1])) << 16);
    u32x4* dst = reinterpret_cast<u32x4*>(a.C + m * a.ldc + col);
    dst[0] = u32x4{pk[0], pk[1], pk[2], pk[3]};
    dst[1] = u32x4{pk[4], pk[5], pk[6], pk[7]};
  } else {
    float4* dst = reinterpret_cast<float4*>(a.partials + (static_cast<int64_t>(sp) * a.M + m) * a.N + col);
#pragma unroll
    for (int q = 0; q < 4; ++q) dst[q] = make_float4(o[4 * q], o[4 * q + 1], o[4 * q + 2], o[4 * q + 3]);
  }
}

// C = bf16(sum over planes s = 0..S-1 of partials[s]), planes added in order. Four columns per
// thread.
__global__ __launch_bounds__(256) void skinny_finish_kernel(const float* __restrict__ partials, int S, int64_t M,
                                                            int64_t N, uint16_t* __restrict__ C, int64_t ldc) {
  const int64_t i4 = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  const int64_t plane4 = M * N / 4;
  if (i4 >= plane4) return;
  const float4* p = reinterpret_cast<const float4*>(partials);
  float4 acc = p[i4];
  for (int s = 1; s < S; ++s) {
    const float4 x = p[s * plane4 + i4];
    acc.x += x.x;
    acc.y += x.y;
    acc.z += x.z;
    acc.w += x.w;
  }
  const int64_t m = (i4 * 4) / N, n = (i4 * 4) % N;
  const uint32_t lo = f32_to_bf16_bits(acc.x) | (static_cast<uint32_t>(f32_to_bf16_bits(acc.y)) << 16);
  const uint32_t hi = f32_to_bf16_bits(acc.z) | (static_cast<uint32_t>(f32_to_bf16_bits(acc.w)) << 16);
  *reinterpret_cast<uint2*>(C + m * ldc + n) = make_uint2(lo, hi);
}

}  // namespace

int gemm_skinny_splits(int64_t N, int64_t K) {
  const int64_t tiles = (N + kSkN - 1) / kSkN;
  const int64_t nk = K / 64;
  int s = 1;
  // about 128 workgroups, each wavefront keeping at least one 64-k block
  while (s * 2 <= kSkMaxSplit && tiles * s < 128 && s * 2 * 4 <= nk) s *= 2;
  return s;
}

size_t gemm_skinny_partial_bytes(int64_t M, int64_t N, int64_t K) {
  const int s = gemm_skinny_splits(N, K);
  return s > 1 ? static_cast<size_t>(s) * M * N * sizeof(float) : 0;
}

hipError_t launch_gemm_skinny(const GemmCall& c, float* partials, size_t partial_bytes, hipStream_t s) {
  if (c.dense_M <= 0 || c.dense_M > kSkM || c.gather || c.scatter || c.swiglu_h > 0 || c.N % kSkN != 0 ||
      c.Kd % 64 != 0)
    return hipErrorInvalidValue;
  SkinnyArgs a;
  a.A = static_cast<const uint16_t*>(c.A);
  a.lda = c.lda;
  a.M = c.dense_M;
  a.B = static_cast<const uint16_t*>(c.B);
  a.ldb = c.ldb;
  a.N = c.N;
  a.K = c.Kd;
  a.C = static_cast<uint16_t*>(c.C);
  a.ldc = c.ldc;
  a.S = gemm_skinny_splits(c.N, c.Kd);
  const size_t need = gemm_skinny_partial_bytes(c.dense_M, c.N, c.Kd);
  if (a.S > 1 && (!partials || partial_bytes < need)) a.S = 1;  // no room for partials: one k-slice
  a.partials = a.S > 1 ? partials : nullptr;
  const dim3 g(static_cast<unsigned>(c.N / kSkN), static_cast<unsigned>(a.S));
  hipLaunchKernelGGL(gemm_skinny_kernel, g, dim3(256), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.S == 1) return e;
  const int64_t n4 = a.M * a.N / 4;
  hipLaunchKernelGGL(skinny_finish_kernel, dim3(static_cast<unsigned>((n4 + 255) / 256)), dim3(256), 0, s,
                     a.partials, a.S, a.M, a.N, a.C, a.ldc);
  return hipGetLastError();
}

}  // namespace moe
