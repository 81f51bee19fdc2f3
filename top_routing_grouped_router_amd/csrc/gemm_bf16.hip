// bf16 MFMA GEMM for gfx950: the grouped expert GEMMs and the dense latent projections.
//
// What it computes ("Как устроен Olmo-core 3: обучение больших MoE-моделей"):
//   * section "Вычисления экспертов и точность": tokens grouped by expert run through each
//     expert's MLP with a grouped matrix multiply over int32 row offsets; the grouped experts
//     return bf16;
//   * section "SwiGLU с квантизацией": the first matrix's output splits into halves, up then
//     gate, and act = up * gate * sigmoid(gate) in fp32;
//   * section "Латентная проекция экспертов": the dense down-projection d_model -> latent_dim
//     and up-projection latent_dim -> d_model (dense mode: one group, M = tokens).
// All operands are "NT": token rows A (M, Kd) and weight rows B (N, Kd), Kd contiguous, fp32
// accumulation.
//
// Design for CDNA4:
//   * v_mfma_f32_32x32x16_bf16. The weight rows feed the MFMA's first operand and the token
//     rows its second, so each lane ends with 4 consecutive output columns of one token row:
//     the epilogue writes 8-byte packed bf16 and the SwiGLU pairs up/gate in registers.
//   * Tile = (WM*TM*32 token rows) x (WN*TN*32 weight rows) x 64 k, 4 wavefronts. The large
//     variant is 256 x 256 (each wavefront 128 x 128: 16 MFMA accumulators of 16 floats).
//     LDS holds two stages of both tiles (128 KiB for 256 x 256); 16-byte chunks are XOR-
//     swizzled by row so the per-lane 16-byte fragment reads hit distinct banks.
//   * The A loader gathers token rows through the permutation (row = perm[p] / k), so the
//     permuted copy of the tokens is never materialised; the GEMM2 epilogue scatters rows to
//     assignment order, so the combine reads each token's k rows contiguously.
//   * Persistent grid (one workgroup per CU slot). Workgroup i runs on XCD i % 8; the linear
//     tile sequence is cut into 8 contiguous chunks, one per XCD, and inside a chunk tiles go
//     in groups of 4 M-tiles x all N-tiles, so the tiles an XCD runs together share A and B
//     panels in that XCD's L2.
//   * Experts with no tokens have no M-tile and their weights are never read.
#include "common.hpp"

namespace moe {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int BK = 64;         // k per stage
constexpr int ROWB = BK * 2;   // bytes per staged row
constexpr int kXcds = 8;
constexpr int kGroupM = 4;

template <int WM_, int WN_, int TM_, int TN_>
struct Shape {
  static constexpr int WM = WM_, WN = WN_, TM = TM_, TN = TN_;
  static constexpr int NT = WM * WN * kWave;  // threads
  static constexpr int BM = WM * TM * 32;     // token rows
  static constexpr int BN = WN * TN * 32;     // weight rows
  static constexpr int RPP = NT / 8;          // rows staged per pass (8 chunks per row)
  static constexpr int A_CH = BM / RPP;       // 16-byte chunks per thread per stage
  static constexpr int B_CH = BN / RPP;
  static constexpr int STAGE = (BM + BN) * ROWB;
  static_assert(BM % RPP == 0 && BN % RPP == 0, "whole chunks per thread");
  static_assert(TN % 2 == 0, "SwiGLU pairs up/gate sub-tiles inside a wavefront");
};

// 256 x 256 tile, 8 wavefronts (2 x 4), each 128 token rows x 64 weight rows.
using ShapeLarge = Shape<2, 4, 4, 2>;
// 32 x 256 tile, 4 wavefronts (1 x 4): few rows per expert (decode-shaped loads).
using ShapeSmall = Shape<1, 4, 1, 2>;

__device__ __forceinline__ int swz(int row, int chunk) {
  return row * ROWB + ((chunk ^ (row & 7)) << 4);
}

template <class S, bool SWIGLU, bool GATHER, bool SCATTER>
__global__ __launch_bounds__(S::NT) void gemm_bf16_kernel(GemmCall c) {
  __shared__ __attribute__((aligned(16))) unsigned char lds[2 * S::STAGE];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / S::WN, wn = wave % S::WN;
  const int ld_chunk = tid & 7, ld_row = tid >> 3;  // RPP rows per pass

  const int64_t cols_per_tile = SWIGLU ? S::BN / 2 : S::BN;
  const int64_t ntn = (c.N + cols_per_tile - 1) / cols_per_tile;
  const int64_t total_m = c.dense_M > 0 ? (c.dense_M + S::BM - 1) / S::BM
                                        : min(static_cast<int64_t>(*c.tiles.count),
                                              static_cast<int64_t>(c.tiles.cap));
  const int64_t total = total_m * ntn;
  const int xcd = blockIdx.x % kXcds;
  const int per_xcd = gridDim.x / kXcds;
  const int slot = blockIdx.x / kXcds;
  const int64_t chunk = (total + kXcds - 1) / kXcds;
  const int nk = static_cast<int>(c.Kd / BK);
  const uint16_t* Abase = static_cast<const uint16_t*>(c.A);
  uint16_t* Cbase = static_cast<uint16_t*>(c.C);

  for (int64_t it = slot; it < chunk; it += per_xcd) {
    const int64_t lin = xcd * chunk + it;
    if (lin >= total) break;
    const int64_t gsz = kGroupM * ntn;
    const int64_t grp_i = lin / gsz, first_m = grp_i * kGroupM;
    const int64_t gm = min(static_cast<int64_t>(kGroupM), total_m - first_m);
    const int64_t local = lin - grp_i * gsz;
    const int64_t mt = first_m + local % gm;
    const int64_t nt = local / gm;

    int64_t row0, grp;
    int rows;
    if (c.dense_M > 0) {
      row0 = mt * S::BM;
      rows = static_cast<int>(min(static_cast<int64_t>(S::BM), c.dense_M - row0));
      grp = 0;
    } else {
      row0 = c.tiles.row0[mt];
      rows = c.tiles.rows[mt];
      grp = c.tiles.expert[mt];
    }

    // Per-thread 32-bit byte offsets of the rows this thread stages (uniform bases stay in
    // scalar registers; the loads use the scalar-base + vector-offset form).
    uint32_t a_off[S::A_CH];
#pragma unroll
    for (int q = 0; q < S::A_CH; ++q) {
      const int r = ld_row + S::RPP * q;
      int64_t p = row0 + (r < rows ? r : 0);
      p = min(max(p, int64_t(0)), c.rows_bound - 1);
      int64_t src = GATHER ? static_cast<int64_t>(c.gather[p]) / c.gather_div : p;
      src = min(max(src, int64_t(0)), c.a_rows - 1);
      a_off[q] = static_cast<uint32_t>((src * c.lda + ld_chunk * 8) * 2);
    }
    const unsigned char* Bexp =
        reinterpret_cast<const unsigned char*>(static_cast<const uint16_t*>(c.B) + grp * c.b_group_stride);
    uint32_t b_off[S::B_CH];
#pragma unroll
    for (int q = 0; q < S::B_CH; ++q) {
      const int r = ld_row + S::RPP * q;
      int64_t wrow;
      if (SWIGLU) {
        const int wv = r / (S::TN * 32), qq = r % (S::TN * 32);
        const int half = qq / (S::TN * 16);
        int64_t col = nt * (S::BN / 2) + wv * (S::TN * 16) + (qq % (S::TN * 16));
        col = min(col, c.N - 1);
        wrow = col + (half ? c.swiglu_h : 0);
      } else {
        wrow = min(nt * S::BN + r, c.N - 1);
      }
      b_off[q] = static_cast<uint32_t>((wrow * c.ldb + ld_chunk * 8) * 2);
    }
    const unsigned char* Ab = reinterpret_cast<const unsigned char*>(Abase);

    f32x16 acc[S::TM][S::TN];
#pragma unroll
    for (int i = 0; i < S::TM; ++i)
#pragma unroll
      for (int j = 0; j < S::TN; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

    u32x4 ra[S::A_CH], rb[S::B_CH];
    auto gload = [&](int kt) {
#pragma unroll
      for (int q = 0; q < S::A_CH; ++q)
        ra[q] = *reinterpret_cast<const u32x4*>(Ab + (a_off[q] + static_cast<uint32_t>(kt) * ROWB));
#pragma unroll
      for (int q = 0; q < S::B_CH; ++q)
        rb[q] = *reinterpret_cast<const u32x4*>(Bexp + (b_off[q] + static_cast<uint32_t>(kt) * ROWB));
    };
    auto sstore = [&](int buf) {
      unsigned char* la = lds + buf * S::STAGE;
      unsigned char* lb = la + S::BM * ROWB;
#pragma unroll
      for (int q = 0; q < S::A_CH; ++q)
        *reinterpret_cast<u32x4*>(la + swz(ld_row + S::RPP * q, ld_chunk)) = ra[q];
#pragma unroll
      for (int q = 0; q < S::B_CH; ++q)
        *reinterpret_cast<u32x4*>(lb + swz(ld_row + S::RPP * q, ld_chunk)) = rb[q];
    };

    gload(0);
    sstore(0);
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
      const int buf = kt & 1;
      if (kt + 1 < nk) gload(kt + 1);
      const unsigned char* la = lds + buf * S::STAGE;
      const unsigned char* lb = la + S::BM * ROWB;
#pragma unroll
      for (int kk = 0; kk < BK / 16; ++kk) {
        const int ch = 2 * kk + (lane >> 5);
        bf16x8 fw[S::TN], ft[S::TM];
#pragma unroll
        for (int j = 0; j < S::TN; ++j)
          fw[j] = *reinterpret_cast<const bf16x8*>(lb + swz(wn * S::TN * 32 + j * 32 + (lane & 31), ch));
#pragma unroll
        for (int i = 0; i < S::TM; ++i)
          ft[i] = *reinterpret_cast<const bf16x8*>(la + swz(wm * S::TM * 32 + i * 32 + (lane & 31), ch));
#pragma unroll
        for (int i = 0; i < S::TM; ++i)
#pragma unroll
          for (int j = 0; j < S::TN; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fw[j], ft[i], acc[i][j], 0, 0, 0);
      }
      if (kt + 1 < nk) sstore(buf ^ 1);
      __syncthreads();
    }

    // Epilogue. Lane holds token row (lane & 31) of each 32-row sub-tile and weight rows
    // 8*g + 4*(lane >> 5) + {0..3} of each 32-row weight sub-tile (g = 0..3).
    const int quad = 4 * (lane >> 5);
#pragma unroll
    for (int i = 0; i < S::TM; ++i) {
      const int m = wm * S::TM * 32 + i * 32 + (lane & 31);
      if (m >= rows) continue;
      const int64_t p = min(row0 + m, c.rows_bound - 1);
      int64_t orow = SCATTER ? static_cast<int64_t>(c.scatter[p]) : p;
      orow = min(max(orow, int64_t(0)), c.c_rows - 1);
      uint16_t* crow = Cbase + orow * c.ldc;
      if (SWIGLU) {
#pragma unroll
        for (int j = 0; j < S::TN / 2; ++j) {
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const int64_t col = nt * (S::BN / 2) + wn * (S::TN * 16) + j * 32 + 8 * g + quad;
            if (col >= c.N) continue;
            uint16_t o[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const float up = acc[i][j][4 * g + r];
              const float gate = acc[i][j + S::TN / 2][4 * g + r];
              o[r] = f32_to_bf16_bits(up * (gate / (1.f + expf(-gate))));
            }
            *reinterpret_cast<uint2*>(crow + col) =
                make_uint2(o[0] | (static_cast<uint32_t>(o[1]) << 16),
                           o[2] | (static_cast<uint32_t>(o[3]) << 16));
          }
        }
      } else {
#pragma unroll
        for (int j = 0; j < S::TN; ++j) {
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const int64_t col = nt * S::BN + wn * (S::TN * 32) + j * 32 + 8 * g + quad;
            if (col >= c.N) continue;
            uint16_t o[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) o[r] = f32_to_bf16_bits(acc[i][j][4 * g + r]);
            *reinterpret_cast<uint2*>(crow + col) =
                make_uint2(o[0] | (static_cast<uint32_t>(o[1]) << 16),
                           o[2] | (static_cast<uint32_t>(o[3]) << 16));
          }
        }
      }
    }
  }
}

template <class S>
hipError_t launch_shape(const GemmCall& c, hipStream_t s, int wg_per_cu) {
  const int64_t cols_per_tile = c.swiglu_h > 0 ? S::BN / 2 : S::BN;
  const int64_t ntn = (c.N + cols_per_tile - 1) / cols_per_tile;
  const int64_t tiles_upper = c.dense_M > 0 ? ((c.dense_M + S::BM - 1) / S::BM) * ntn
                                            : static_cast<int64_t>(c.tiles.cap) * ntn;
  if (tiles_upper <= 0 || c.rows_bound <= 0) return hipSuccess;
  int64_t grid = std::min<int64_t>(tiles_upper, static_cast<int64_t>(device_cu_count()) * wg_per_cu);
  grid = ((grid + kXcds - 1) / kXcds) * kXcds;  // whole XCD rounds
  const dim3 g(static_cast<unsigned>(grid)), b(S::NT);
  const bool sw = c.swiglu_h > 0, ga = c.gather != nullptr, sc = c.scatter != nullptr;
  if (sw && ga && !sc) hipLaunchKernelGGL((gemm_bf16_kernel<S, true, true, false>), g, b, 0, s, c);
  else if (!sw && !ga && sc) hipLaunchKernelGGL((gemm_bf16_kernel<S, false, false, true>), g, b, 0, s, c);
  else if (!sw && !ga && !sc) hipLaunchKernelGGL((gemm_bf16_kernel<S, false, false, false>), g, b, 0, s, c);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace

int gemm_bf16_tile_m(int variant) { return variant == 0 ? ShapeLarge::BM : ShapeSmall::BM; }

int gemm_bf16_pick_variant(double mean_rows_per_group) { return mean_rows_per_group >= 96.0 ? 0 : 1; }

hipError_t launch_gemm_bf16(const GemmCall& c, int variant, hipStream_t s) {
  if (variant == 0) return launch_shape<ShapeLarge>(c, s, 1);
  return launch_shape<ShapeSmall>(c, s, 2);
}

}  // namespace moe
