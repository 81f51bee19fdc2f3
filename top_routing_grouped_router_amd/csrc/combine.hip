// Unpermute + weighted combine (+ the latent restore norm).
//
// "Как устроен Olmo-core 3: обучение больших MoE-моделей":
//   * section "Пересылка токенов между экспертами": expert results return to their original
//     positions (a scatter with the saved indices). The grouped GEMM already wrote each
//     result to its assignment row t*k + j, so a token's k results are contiguous here;
//   * the router's weights scale each result and the k results are summed, in j order, in
//     fp32: o[t] = sum_j w[t,j] * Y[t*k+j];
//   * section "Латентная проекция экспертов": with a latent projection, the up-projection
//     input is normalised (bias-free RMSNorm by default: n = o / sqrt(mean(o^2) + eps) * g)
//     and cast to the up-projection weight's dtype.
// 16-byte loads and stores, fp32 math. HBM-bound: it reads k*K and writes K elements per token.
#include <algorithm>

#include "common.hpp"

namespace moe {
namespace {

constexpr int kThreads = 256;

// Expert-output rows are read once: loaded past the caches' retention (non-temporal), so the
// layer's other operands keep their place in L2 and the last-level cache.
typedef uint32_t u32x4v __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 load_once(const void* p) {
  const u32x4v q = __builtin_nontemporal_load(static_cast<const u32x4v*>(p));
  return make_uint4(q.x, q.y, q.z, q.w);
}
constexpr int kMaxChunks = 8;  // per thread: K <= 256 * 8 * (16 / sizeof(T))

template <typename T>
struct Vec16;
template <>
struct Vec16<uint16_t> {
  static constexpr int N = 8;
  __device__ static void load(const uint16_t* p, float* v) {
    const uint4 u = *reinterpret_cast<const uint4*>(p);
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = __uint_as_float(w[i] << 16);
      v[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  }
  __device__ static void store(uint16_t* p, const float* v) {
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      w[i] = f32_to_bf16_bits(v[2 * i]) | (static_cast<uint32_t>(f32_to_bf16_bits(v[2 * i + 1])) << 16);
    *reinterpret_cast<uint4*>(p) = make_uint4(w[0], w[1], w[2], w[3]);
  }
};
template <>
struct Vec16<float> {
  static constexpr int N = 4;
  __device__ static void load(const float* p, float* v) {
    const float4 u = *reinterpret_cast<const float4*>(p);
    v[0] = u.x; v[1] = u.y; v[2] = u.z; v[3] = u.w;
  }
  __device__ static void store(float* p, const float* v) {
    *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
  }
};

// One block per token, sized to the row: NT threads (64..256) each own CH 16-byte chunks of
// the K-element row. The k assignment rows are loaded several at a time (8 / CH) before any of
// them is used, so their loads overlap; accumulation stays in j order.
template <typename T, bool NORM, int CH>
__global__ __launch_bounds__(kThreads) void combine_kernel(const T* __restrict__ y, const float* __restrict__ w,
                                                           const float* __restrict__ g, T* __restrict__ out,
                                                           int k, int K, float eps) {
  constexpr int V = Vec16<T>::N;
  constexpr int kBatch = CH >= 8 ? 1 : 8 / CH;  // rows in flight: 8 x 16 bytes per thread
  const int nt = blockDim.x;
  const int64_t t = blockIdx.x;
  const int nch = K / V;
  float o[CH][V];
#pragma unroll
  for (int c = 0; c < CH; ++c)
#pragma unroll
    for (int q = 0; q < V; ++q) o[c][q] = 0.f;

  for (int j0 = 0; j0 < k; j0 += kBatch) {
    uint4 raw[kBatch][CH];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const T* yr = y + (t * k + j0 + u) * static_cast<int64_t>(K);
#pragma unroll
      for (int c = 0; c < CH; ++c) {
        const int ci = threadIdx.x + c * nt;
        if (j0 + u < k && ci < nch) raw[u][c] = load_once(yr + ci * V);
      }
    }
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      if (j0 + u >= k) break;
      const float wj = w[t * k + j0 + u];
#pragma unroll
      for (int c = 0; c < CH; ++c) {
        const int ci = threadIdx.x + c * nt;
        if (ci < nch) {
          float v[V];
          Vec16<T>::load(reinterpret_cast<const T*>(&raw[u][c]), v);
#pragma unroll
          for (int q = 0; q < V; ++q) o[c][q] = fmaf(wj, v[q], o[c][q]);
        }
      }
    }
  }

  float scale = 1.f;
  if (NORM) {
    __shared__ float red[kThreads / kWave];
    float ss = 0.f;
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      const int ci = threadIdx.x + c * nt;
      if (ci < nch) {
#pragma unroll
        for (int q = 0; q < V; ++q) ss = fmaf(o[c][q], o[c][q], ss);
      }
    }
    ss = wave_sum(ss);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = ss;
    __syncthreads();
    float tot = 0.f;
    for (int i = 0; i < nt / kWave; ++i) tot += red[i];
    scale = 1.f / sqrtf(tot / static_cast<float>(K) + eps);
  }

  T* orow = out + t * static_cast<int64_t>(K);
#pragma unroll
  for (int c = 0; c < CH; ++c) {
    const int ci = threadIdx.x + c * nt;
    if (ci < nch) {
      float v[V];
#pragma unroll
      for (int q = 0; q < V; ++q) {
        float x = o[c][q];
        if (NORM) {
          x = x * scale;
          if (g) x = x * g[ci * V + q];
        }
        v[q] = x;
      }
      Vec16<T>::store(orow + ci * V, v);
    }
  }
}

// One wavefront per token (rows of up to 4 * 64 chunks of 16 bytes), tokens strided over a grid
// of 4 blocks per CU (measured against 1, 2, 8, 16 and 32: fewer, longer-lived wavefronts;
// latent896 -12 % against 16): the whole of a token's k rows is loaded before any is used (16 chunks
// per lane in flight), the norm's sum of squares is a wavefront reduction (no block barrier),
// and the grid is not re-dispatched per token. Accumulation order as above: j ascending.
template <typename T, bool NORM, int CH>
__global__ __launch_bounds__(kThreads) void combine_wave_kernel(const T* __restrict__ y, const float* __restrict__ w,
                                                                const float* __restrict__ g, T* __restrict__ out,
                                                                int64_t ntok, int k, int K, float eps) {
  constexpr int V = Vec16<T>::N;
  constexpr int kBatch = 16 / CH;  // rows in flight
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t nwaves = static_cast<int64_t>(gridDim.x) * (kThreads / kWave);
  const int nch = K / V;
  // the norm weights of this lane's columns, the same for every token
  float gv[NORM ? CH : 1][V];
#pragma unroll
  for (int c = 0; c < (NORM ? CH : 1); ++c) {
    const int ci = lane + c * kWave;
#pragma unroll
    for (int q = 0; q < V; ++q) gv[c][q] = (NORM && g && ci < nch) ? g[ci * V + q] : 1.f;
  }
  for (int64_t t = static_cast<int64_t>(blockIdx.x) * (kThreads / kWave) + (threadIdx.x >> 6); t < ntok;
       t += nwaves) {
    float o[CH][V];
#pragma unroll
    for (int c = 0; c < CH; ++c)
#pragma unroll
      for (int q = 0; q < V; ++q) o[c][q] = 0.f;
    for (int j0 = 0; j0 < k; j0 += kBatch) {
      uint4 raw[kBatch][CH];
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        const T* yr = y + (t * k + min(j0 + u, k - 1)) * static_cast<int64_t>(K);
#pragma unroll
        for (int c = 0; c < CH; ++c) {
          const int ci = lane + c * kWave;
          if (ci < nch) raw[u][c] = *reinterpret_cast<const uint4*>(yr + ci * V);
        }
      }
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        if (j0 + u >= k) break;
        const float wj = w[t * k + j0 + u];
#pragma unroll
        for (int c = 0; c < CH; ++c) {
          const int ci = lane + c * kWave;
          if (ci < nch) {
            float v[V];
            Vec16<T>::load(reinterpret_cast<const T*>(&raw[u][c]), v);
#pragma unroll
            for (int q = 0; q < V; ++q) o[c][q] = fmaf(wj, v[q], o[c][q]);
          }
        }
      }
    }
    float scale = 1.f;
    if (NORM) {
      float ss = 0.f;
#pragma unroll
      for (int c = 0; c < CH; ++c) {
        const int ci = lane + c * kWave;
        if (ci < nch) {
#pragma unroll
          for (int q = 0; q < V; ++q) ss = fmaf(o[c][q], o[c][q], ss);
        }
      }
      ss = wave_sum(ss);
      scale = 1.f / sqrtf(ss / static_cast<float>(K) + eps);
    }
    T* orow = out + t * static_cast<int64_t>(K);
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      const int ci = lane + c * kWave;
      if (ci < nch) {
        float v[V];
#pragma unroll
        for (int q = 0; q < V; ++q) {
          float x = o[c][q];
          if (NORM) {
            x = x * scale;
            if (g) x = x * gv[NORM ? c : 0][q];
          }
          v[q] = x;
        }
        Vec16<T>::store(orow + ci * V, v);
      }
    }
  }
}

template <typename T, bool NORM>
void launch_tn(const Layer& ly, const void* y, const float* w, const float* g, void* out, hipStream_t s) {
  const int K = static_cast<int>(ly.K);
  const int nch = K / Vec16<T>::N;
  if (nch <= 4 * kWave && ly.T >= 2048) {
    // wavefront per token (few tokens keep the block per token: more wavefronts in flight)
    const int64_t blocks = std::min<int64_t>((ly.T + 3) / 4, static_cast<int64_t>(device_cu_count()) * 4);
    const dim3 grid(static_cast<unsigned>(blocks)), block(kThreads);
    const T* yy = static_cast<const T*>(y);
    T* oo = static_cast<T*>(out);
    if (nch <= kWave)
      hipLaunchKernelGGL((combine_wave_kernel<T, NORM, 1>), grid, block, 0, s, yy, w, g, oo, ly.T, ly.k, K, ly.norm_eps);
    else if (nch <= 2 * kWave)
      hipLaunchKernelGGL((combine_wave_kernel<T, NORM, 2>), grid, block, 0, s, yy, w, g, oo, ly.T, ly.k, K, ly.norm_eps);
    else
      hipLaunchKernelGGL((combine_wave_kernel<T, NORM, 4>), grid, block, 0, s, yy, w, g, oo, ly.T, ly.k, K, ly.norm_eps);
    return;
  }
  const int nt = std::min(kThreads, ((nch + kWave - 1) / kWave) * kWave);
  const int ch = (nch + nt - 1) / nt;
  const dim3 grid(static_cast<unsigned>(ly.T)), block(static_cast<unsigned>(nt));
  const T* yy = static_cast<const T*>(y);
  T* oo = static_cast<T*>(out);
  if (ch <= 1) hipLaunchKernelGGL((combine_kernel<T, NORM, 1>), grid, block, 0, s, yy, w, g, oo, ly.k, K, ly.norm_eps);
  else if (ch <= 2) hipLaunchKernelGGL((combine_kernel<T, NORM, 2>), grid, block, 0, s, yy, w, g, oo, ly.k, K, ly.norm_eps);
  else if (ch <= 4) hipLaunchKernelGGL((combine_kernel<T, NORM, 4>), grid, block, 0, s, yy, w, g, oo, ly.k, K, ly.norm_eps);
  else hipLaunchKernelGGL((combine_kernel<T, NORM, kMaxChunks>), grid, block, 0, s, yy, w, g, oo, ly.k, K, ly.norm_eps);
}

template <typename T>
void launch_t(const Layer& ly, const void* y, const float* w, const float* g, bool norm, void* out,
              hipStream_t s) {
  if (norm) launch_tn<T, true>(ly, y, w, g, out, s);
  else launch_tn<T, false>(ly, y, w, g, out, s);
}

}  // namespace

hipError_t launch_combine(const Layer& ly, const void* y_assign, const float* w,
                          const float* norm_weight, bool apply_norm, void* out, hipStream_t s) {
  if (ly.T <= 0) return hipSuccess;
  if (ly.bf16) launch_t<uint16_t>(ly, y_assign, w, norm_weight, apply_norm, out, s);
  else launch_t<float>(ly, y_assign, w, norm_weight, apply_norm, out, s);
  return hipGetLastError();
}

}  // namespace moe
