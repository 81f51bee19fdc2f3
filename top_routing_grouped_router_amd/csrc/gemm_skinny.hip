// Skinny dense bf16 GEMM for few token rows (M <= 64): the latent projections of a
// decode-sized batch ("Как устроен Olmo-core 3: обучение больших MoE-моделей", section
// "Латентная проекция экспертов": dense down-projection d_model -> latent_dim and
// up-projection back, fp32 accumulation, output in the layer dtype).
//
// With 64 token rows the product is weight streaming: every weight row is read once and meets
// at most 64 tokens, so the bound is HBM and the work has to be spread over the whole chip.
// Design:
//   * A workgroup owns 64 weight rows x all (<= 64) token rows x one k-slice; the contraction
//     is split over S workgroups (k-slices), about 256 workgroups in all.
//   * Operands reach LDS by DMA (buffer_load ... lds, 16 bytes per lane): each load fills 8
//     rows x one 128-byte line of a 64-k stage, so every request is a whole line. 16-byte
//     chunks are XOR-swizzled by row pair, so the fragment reads are free of bank conflicts.
//     A four-slot ring keeps up to four stages (64 KiB) of a workgroup in flight.
//   * Each of the 4 wavefronts owns a 32 x 32 block of the output (one
//     v_mfma_f32_32x32x16_bf16 accumulator): weight half w & 1, token half w >> 1.
//   * With S = 1 the block is rounded to bf16 and stored; otherwise it goes to fp32 partial
//     plane `split`, and a second kernel adds the S planes in plane order and rounds. Fixed
//     orders throughout, so results are bitwise reproducible.
#include <algorithm>

#include "common.hpp"

namespace moe {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kSkM = 64;      // token rows (padded)
constexpr int kSkN = 64;      // weight rows per workgroup
constexpr int kSkMaxSplit = 16;
constexpr int kSkSlots = 4;   // ring depth (64-k stages)
constexpr int kSkStage = (kSkM + kSkN) * 128;  // bytes per stage: 128 rows of 128 bytes

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

#define SK_LDS(p) ((__attribute__((address_space(3))) void*)(p))

template <int N>
__device__ __forceinline__ void sk_wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt field");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// byte offset of logical 16-byte chunk c of staged row r
__device__ __forceinline__ int sk_swz(int r, int c) { return r * 128 + ((c ^ ((r >> 1) & 7)) << 4); }

__global__ __launch_bounds__(256) void gemm_skinny_kernel(SkinnyArgs a) {
  __shared__ __attribute__((aligned(1024))) unsigned char ring[kSkSlots * kSkStage];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t n0 = static_cast<int64_t>(blockIdx.x) * kSkN;
  const int sp = blockIdx.y;
  const int nk = static_cast<int>(a.K / 64);
  const int kb = static_cast<int>(static_cast<int64_t>(sp) * nk / a.S);
  const int ns = static_cast<int>(static_cast<int64_t>(sp + 1) * nk / a.S) - kb;  // stages of this slice

  // Load q (0..3) of this wavefront fills staged rows [8i, 8i + 8), i = wave + 4q: token rows
  // for i < 8, weight rows after. Lane: row 8i + lane / 8, LDS slot lane % 8, which holds the
  // row's logical chunk (lane % 8) ^ ((row >> 1) & 7). Rows past the operand are clamped to its
  // last row (their products are never stored).
  uint32_t off[4];
  bool is_a[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int i = wave + 4 * q;
    is_a[q] = i < 8;
    const int r = (i & 7) * 8 + (lane >> 3);
    const int ch = (lane & 7) ^ ((r >> 1) & 7);
    const int64_t row = is_a[q] ? min(static_cast<int64_t>(r), a.M - 1) : min(n0 + r, a.N - 1);
    off[q] = static_cast<uint32_t>((row * (is_a[q] ? a.lda : a.ldb) + static_cast<int64_t>(kb) * 64) * 2 + ch * 16);
  }
#if defined(__HIP_DEVICE_COMPILE__)
  // uniform bases in scalar registers, widened from unsigned halves
  auto rsrc = [](const void* p) {
    const uint64_t v = reinterpret_cast<uint64_t>(p);
    const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v));
    const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v >> 32));
    return __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void*>((static_cast<uint64_t>(hi) << 32) | lo),
                                             static_cast<short>(0), -1, 0x00020000);
  };
  const __amdgpu_buffer_rsrc_t ra = rsrc(a.A), rb = rsrc(a.B);
#endif
  // stage s of the slice into ring slot s % kSkSlots (stages past the slice reload its last one)
  auto issue = [&](int s) {
#if defined(__HIP_DEVICE_COMPILE__)
    const int sc = min(s, ns - 1);
    unsigned char* st = ring + (s % kSkSlots) * kSkStage;
#pragma unroll
    for (int q = 0; q < 4; ++q)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(is_a[q] ? ra : rb, SK_LDS(st + (wave + 4 * q) * 1024), 16, off[q],
                                               static_cast<uint32_t>(sc) * 128, 0, 0);
#else
    (void)s;
#endif
  };

  f32x16 acc;
#pragma unroll
  for (int q = 0; q < 16; ++q) acc[q] = 0.f;
  const int wr = 32 * (wave & 1) + (lane & 31);   // this lane's weight row in the tile
  const int tr = 32 * (wave >> 1) + (lane & 31);  // this lane's token row
  const int half = lane >> 5;

  // Every wavefront issues exactly kSkSlots stages up front, then one per stage computed, so
  // the count of loads still in flight after stage s's own is fixed: 4 per later stage issued.
#pragma unroll
  for (int s = 0; s < kSkSlots; ++s) issue(s);
  for (int s = 0; s < ns; ++s) {
    sk_wait_vmcnt<4 * (kSkSlots - 1)>();  // stage s landed (the kSkSlots - 1 later ones may not)
    __builtin_amdgcn_s_barrier();
    const unsigned char* st = ring + (s % kSkSlots) * kSkStage;
    bf16x8 fw[4], ft[4];
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      fw[kk] = *reinterpret_cast<const bf16x8*>(st + kSkM * 128 + sk_swz(wr, 2 * kk + half));
      ft[kk] = *reinterpret_cast<const bf16x8*>(st + sk_swz(tr, 2 * kk + half));
    }
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fw[kk], ft[kk], acc, 0, 0, 0);
    // every wavefront has read slot s % kSkSlots before it is refilled
    __builtin_amdgcn_s_waitcnt((15) | (3 << 14) | (7 << 4) | (0 << 8));
    __builtin_amdgcn_s_barrier();
    issue(s + kSkSlots);
  }
  sk_wait_vmcnt<0>();  // the reloads issued past the slice (never read) land before the exit

  // Lane holds token (lane & 31) of token half (wave >> 1) and weight rows
  // 8g + 4(lane >> 5) + {0..3} of weight half (wave & 1), g = 0..3.
  const int64_t m = tr;
  if (m >= a.M) return;
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    const int64_t col = n0 + 32 * (wave & 1) + 8 * g + 4 * half;
    if (col >= a.N) continue;
    if (a.S == 1) {
      const uint32_t lo = f32_to_bf16_bits(acc[4 * g]) | (static_cast<uint32_t>(f32_to_bf16_bits(acc[4 * g + 1])) << 16);
      const uint32_t hi = f32_to_bf16_bits(acc[4 * g + 2]) | (static_cast<uint32_t>(f32_to_bf16_bits(acc[4 * g + 3])) << 16);
      *reinterpret_cast<uint2*>(a.C + m * a.ldc + col) = make_uint2(lo, hi);
    } else {
      *reinterpret_cast<float4*>(a.partials + (static_cast<int64_t>(sp) * a.M + m) * a.N + col) =
          make_float4(acc[4 * g], acc[4 * g + 1], acc[4 * g + 2], acc[4 * g + 3]);
    }
  }
}

// C = bf16(sum over planes s = 0..S-1 of partials[s]), planes added in order. Four columns per
// thread; the S loads are issued together (S known at compile time), so the pass costs one
// memory round trip.
template <int S>
__global__ __launch_bounds__(256) void skinny_finish_kernel(const float* __restrict__ partials, int64_t M,
                                                            int64_t N, uint16_t* __restrict__ C, int64_t ldc) {
  const int64_t i4 = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  const int64_t plane4 = M * N / 4;
  if (i4 >= plane4) return;
  const float4* p = reinterpret_cast<const float4*>(partials);
  float4 x[S];
#pragma unroll
  for (int s = 0; s < S; ++s) x[s] = p[s * plane4 + i4];
  float4 acc = x[0];
#pragma unroll
  for (int s = 1; s < S; ++s) {
    acc.x += x[s].x;
    acc.y += x[s].y;
    acc.z += x[s].z;
    acc.w += x[s].w;
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
  // about 256 workgroups (one per CU), each k-slice keeping at least one 64-k stage
  while (s * 2 <= kSkMaxSplit && tiles * s < 256 && s * 2 <= nk) s *= 2;
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
  const dim3 fg(static_cast<unsigned>((n4 + 255) / 256));
  switch (a.S) {  // a power of two up to kSkMaxSplit
    case 2: hipLaunchKernelGGL(skinny_finish_kernel<2>, fg, dim3(256), 0, s, a.partials, a.M, a.N, a.C, a.ldc); break;
    case 4: hipLaunchKernelGGL(skinny_finish_kernel<4>, fg, dim3(256), 0, s, a.partials, a.M, a.N, a.C, a.ldc); break;
    case 8: hipLaunchKernelGGL(skinny_finish_kernel<8>, fg, dim3(256), 0, s, a.partials, a.M, a.N, a.C, a.ldc); break;
    case 16: hipLaunchKernelGGL(skinny_finish_kernel<16>, fg, dim3(256), 0, s, a.partials, a.M, a.N, a.C, a.ldc); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace moe
