// fp32 "NT" GEMM on the vector ALUs: C = A * B^T with fp32 products and fp32 accumulation.
//
// Serves the fp32 router contraction ("Как устроен Olmo-core 3: обучение больших
// MoE-моделей", section "Маршрутизация: как роутер выбирает экспертов": the router input is
// cast to fp32 and multiplied by the (num_experts, d_model) weight) and every contraction of
// an fp32 layer. Grouped mode walks the per-expert M-tile list built on the device; the
// SwiGLU epilogue splits each tile's weight rows into matching up / gate halves (section
// "SwiGLU с квантизацией": up first, then gate; act = up * gate * sigmoid(gate)).
//
// Tile 64 x 64 outputs, 256 threads as 16 x 16, 4 x 4 outputs per thread, k-step 16 staged
// through LDS. It is bound by fp32 FMA issue, not HBM: an fp32 contraction of these shapes
// has arithmetic intensity far above the fp32 ridge point of the chip.
#include "common.hpp"

namespace moe {
namespace {

constexpr int BM = kF32TileM, BN = 64, BK = 16;

template <bool A_BF16, bool SWIGLU>
__global__ __launch_bounds__(256) void gemm_f32_kernel(GemmCall c, const float* __restrict__ col_bias) {
  __shared__ float As[BK][BM + 4];
  __shared__ float Bs[BK][BN + 4];
  const int64_t a_rows = c.a_rows, out_rows = c.c_rows, rows_bound = c.rows_bound;
  const int tid = threadIdx.x;
  const int tx = tid & 15, ty = tid >> 4;
  const int64_t cols_per_tile = SWIGLU ? BN / 2 : BN;
  const int64_t ntn = (c.N + cols_per_tile - 1) / cols_per_tile;
  const int64_t total_m = c.dense_M > 0 ? (c.dense_M + BM - 1) / BM
                                        : min(static_cast<int64_t>(*c.tiles.count),
                                              static_cast<int64_t>(c.tiles.cap));
  const int64_t total = total_m * ntn;
  const int lr = tid >> 2, lk = (tid & 3) * 4;  // load row, first k of 4

  for (int64_t tile = blockIdx.x; tile < total; tile += gridDim.x) {
    const int64_t mt = tile / ntn, nt = tile % ntn;
    int64_t row0, grp;
    int rows;
    if (c.dense_M > 0) {
      row0 = mt * BM;
      rows = static_cast<int>(min(static_cast<int64_t>(BM), c.dense_M - row0));
      grp = 0;
    } else {
      row0 = c.tiles.row0[mt];
      rows = c.tiles.rows[mt];
      grp = c.tiles.expert[mt];
    }
    // Source row of the A tile row this thread loads (rows past the tile's end reuse row 0).
    int64_t p = row0 + (lr < rows ? lr : 0);
    p = min(max(p, int64_t(0)), rows_bound - 1);
    int64_t arow = c.gather ? static_cast<int64_t>(c.gather[p]) / c.gather_div : p;
    arow = min(max(arow, int64_t(0)), a_rows - 1);
    // Weight row this thread loads.
    int64_t wrow;
    if (SWIGLU) {
      const int64_t n = nt * (BN / 2) + (lr & 31);
      wrow = min(n, c.N - 1) + ((lr >= 32) ? c.swiglu_h : 0);
    } else {
      wrow = min(nt * BN + lr, c.N - 1);
    }
    const float* B = static_cast<const float*>(c.B) + grp * c.b_group_stride + wrow * c.ldb;
    const float* Af = static_cast<const float*>(c.A) + arow * c.lda;
    const uint16_t* Ah = static_cast<const uint16_t*>(c.A) + arow * c.lda;

    float acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = 0.f;

    for (int64_t k0 = 0; k0 < c.Kd; k0 += BK) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int64_t k = k0 + lk + q;
        float a = 0.f, b = 0.f;
        if (k < c.Kd) {
          a = A_BF16 ? bf16_bits_to_f32(Ah[k]) : Af[k];
          b = B[k];
        }
        As[lk + q][lr] = a;
        Bs[lk + q][lr] = b;
      }
      __syncthreads();
#pragma unroll
      for (int kk = 0; kk < BK; ++kk) {
        float av[4], bv[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) av[i] = As[kk][ty + 16 * i];
#pragma unroll
        for (int j = 0; j < 4; ++j) bv[j] = Bs[kk][tx + 16 * j];
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(av[i], bv[j], acc[i][j]);
      }
      __syncthreads();
    }

    float* C = static_cast<float*>(c.C);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = ty + 16 * i;
      if (m >= rows) continue;
      int64_t pr = min(row0 + m, rows_bound - 1);
      int64_t orow = c.scatter ? static_cast<int64_t>(c.scatter[pr]) : pr;
      orow = min(max(orow, int64_t(0)), out_rows - 1);
      if (SWIGLU) {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int64_t col = nt * (BN / 2) + tx + 16 * j;
          if (col >= c.N) continue;
          const float up = acc[i][j], gate = acc[i][j + 2];
          C[orow * c.ldc + col] = up * (gate / (1.f + expf(-gate)));
          if (c.h_out) {  // training forward: the pre-activation [up | gate] of sorted row pr
            float* hr = static_cast<float*>(c.h_out) + pr * 2 * c.swiglu_h;
            hr[col] = up;
            hr[c.swiglu_h + col] = gate;
          }
        }
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int64_t col = nt * BN + tx + 16 * j;
          if (col >= c.N) continue;
          float v = acc[i][j];
          if (col_bias) v += col_bias[col];
          C[orow * c.ldc + col] = v;
        }
      }
    }
  }
}

}  // namespace

hipError_t launch_gemm_f32(const GemmCall& c, bool a_is_bf16, const float* col_bias, hipStream_t s) {
  const int64_t cols_per_tile = c.swiglu_h > 0 ? BN / 2 : BN;
  const int64_t ntn = (c.N + cols_per_tile - 1) / cols_per_tile;
  const int64_t tiles_upper = c.dense_M > 0 ? ((c.dense_M + BM - 1) / BM) * ntn
                                            : static_cast<int64_t>(c.tiles.cap) * ntn;
  if (tiles_upper <= 0 || c.rows_bound <= 0) return hipSuccess;
  const int64_t grid = std::min<int64_t>(tiles_upper, static_cast<int64_t>(device_cu_count()) * 8);
  const dim3 g(static_cast<unsigned>(grid)), b(256);
  const bool sw = c.swiglu_h > 0;
  if (a_is_bf16) {
    if (sw) hipLaunchKernelGGL((gemm_f32_kernel<true, true>), g, b, 0, s, c, col_bias);
    else hipLaunchKernelGGL((gemm_f32_kernel<true, false>), g, b, 0, s, c, col_bias);
  } else {
    if (sw) hipLaunchKernelGGL((gemm_f32_kernel<false, true>), g, b, 0, s, c, col_bias);
    else hipLaunchKernelGGL((gemm_f32_kernel<false, false>), g, b, 0, s, c, col_bias);
  }
  return hipGetLastError();
}

}  // namespace moe
