// Backward of the routed experts: the data movement around the grouped GEMMs, the combine
// backward, and the fp32-layer gradient products.
//
// "Как устроен Olmo-core 3: обучение больших MoE-моделей":
//   * section "Пересылка токенов между экспертами": the experts see the tokens gathered into
//     sorted order (row p takes token perm[p] / k) and their results go back to the original
//     positions; the backward gathers the output gradients into sorted order and sums the
//     input gradients of a token's k copies;
//   * the combine o[t] = sum_j w[t,j] * Y[t*k+j] gives dY[t*k+j] = w[t,j] * dO[t] and
//     dw[t,j] = <dO[t], Y[t*k+j]>;
//   * section "SwiGLU с квантизацией": d_up = d_act * silu(gate), d_gate = d_act * up *
//     silu'(gate) in fp32 (the bf16 layers do this in the input-gradient GEMM's epilogue; the
//     fp32 kernel below does it per element);
//   * section "Вычисления экспертов и точность": each expert's gradients come from its own rows.
// The row kernels move 16 bytes per lane and are HBM-bound. The fp32 product kernels serve the
// fp32 layers (small shapes): one thread per output element, loads coalesced along the output
// columns.
#include "common.hpp"

namespace moe {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// 16 bytes of a row as fp32 values (8 bf16 or 4 fp32) and back.
template <typename T>
struct Chunk;
template <>
struct Chunk<uint16_t> {
  static constexpr int N = 8;
  __device__ static void load(const uint16_t* p, float* v) {
    const u32x4 u = *reinterpret_cast<const u32x4*>(p);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = __uint_as_float(u[i] << 16);
      v[2 * i + 1] = __uint_as_float(u[i] & 0xffff0000u);
    }
  }
  __device__ static void store(uint16_t* p, const float* v) {
    u32x4 u;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      u[i] = f32_to_bf16_bits(v[2 * i]) | (static_cast<uint32_t>(f32_to_bf16_bits(v[2 * i + 1])) << 16);
    *reinterpret_cast<u32x4*>(p) = u;
  }
};
template <>
struct Chunk<float> {
  static constexpr int N = 4;
  __device__ static void load(const float* p, float* v) {
    const float4 u = *reinterpret_cast<const float4*>(p);
    v[0] = u.x;
    v[1] = u.y;
    v[2] = u.z;
    v[3] = u.w;
  }
  __device__ static void store(float* p, const float* v) { *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]); }
};

// dst[p] = src[idx[p] / div] for the kept rows p < offsets[E] (at most n_max), 16 bytes per lane.
__global__ __launch_bounds__(256) void gather_rows_kernel(const unsigned char* __restrict__ src, int64_t src_rows,
                                                          const int32_t* __restrict__ idx, int div,
                                                          const int32_t* __restrict__ n_ptr, int64_t n_max,
                                                          int64_t row_bytes, unsigned char* __restrict__ dst) {
  const int64_t n = min(max(static_cast<int64_t>(*n_ptr), int64_t(0)), n_max);
  const int64_t cpr = row_bytes / 16;
  const int64_t total = n * cpr;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; i < total;
       i += static_cast<int64_t>(gridDim.x) * 256) {
    const int64_t p = i / cpr, c = i - p * cpr;
    const int64_t r = min(max(static_cast<int64_t>(idx[p]) / div, int64_t(0)), src_rows - 1);
    *reinterpret_cast<u32x4*>(dst + p * row_bytes + c * 16) =
        *reinterpret_cast<const u32x4*>(src + r * row_bytes + c * 16);
  }
}

// out[t] = sum_j in[t*k + j] in fp32, j ascending, one rounding to the storage dtype.
template <typename T>
__global__ __launch_bounds__(256) void sum_copies_kernel(const T* __restrict__ in, int k, int64_t T_rows,
                                                         int64_t width, T* __restrict__ out) {
  constexpr int N = Chunk<T>::N;
  const int64_t cpr = width / N;
  const int64_t total = T_rows * cpr;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; i < total;
       i += static_cast<int64_t>(gridDim.x) * 256) {
    const int64_t t = i / cpr, c = i - t * cpr;
    float acc[N];
#pragma unroll
    for (int e = 0; e < N; ++e) acc[e] = 0.f;
    // the token's copies (read once: non-temporal) in batches of 8 whose loads are all issued
    // before any is added
    for (int j0 = 0; j0 < k; j0 += 8) {
      u32x4 raw[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const T* p = in + (t * k + min(j0 + u, k - 1)) * width + c * N;
        raw[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        if (j0 + u >= k) break;
        float v[N];
        Chunk<T>::load(reinterpret_cast<const T*>(&raw[u]), v);
#pragma unroll
        for (int e = 0; e < N; ++e) acc[e] += v[e];
      }
    }
    Chunk<T>::store(out + t * width + c * N, acc);
  }
}

// One wavefront per token: for each j, dY[t*k+j] = w[t,j] * dO[t] (rounded to the storage
// dtype) and dw[t,j] = sum_c dO[t,c] * Y[t*k+j,c] (fp32, lane partials then a fixed
// butterfly, so the result is deterministic).
template <typename T>
__global__ __launch_bounds__(256) void combine_backward_kernel(const T* __restrict__ y, const float* __restrict__ w,
                                                               const T* __restrict__ d_out, int k, int64_t T_rows,
                                                               int64_t width, T* __restrict__ dy,
                                                               float* __restrict__ dw) {
  constexpr int N = Chunk<T>::N;
  const int64_t t = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (t >= T_rows) return;
  const int lane = threadIdx.x & 63;
  const int64_t cpr = width / N;
  const T* dot = d_out + t * width;
  for (int j = 0; j < k; ++j) {
    const int64_t a = t * k + j;
    const float wj = w[a];
    float part = 0.f;
    for (int64_t c = lane; c < cpr; c += 64) {
      float g[N], yv[N], o[N];
      Chunk<T>::load(dot + c * N, g);
      Chunk<T>::load(y + a * width + c * N, yv);
#pragma unroll
      for (int e = 0; e < N; ++e) {
        part += g[e] * yv[e];
        o[e] = wj * g[e];
      }
      Chunk<T>::store(dy + a * width + c * N, o);
    }
    part = wave_sum(part);
    if (lane == 0 && dw) dw[a] = part;
  }
}

__global__ __launch_bounds__(256) void fill_zero_kernel(u32x4* __restrict__ p, int64_t n16) {
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; i < n16;
       i += static_cast<int64_t>(gridDim.x) * 256)
    p[i] = u32x4{0u, 0u, 0u, 0u};
}

// Experts by decreasing row count (ties by index): the rank of expert e is the number of
// experts with more rows, plus those with as many rows and a lower index. One workgroup,
// E <= 1024.
__global__ __launch_bounds__(1024) void expert_order_kernel(const int32_t* __restrict__ offsets, int E,
                                                            int32_t* __restrict__ order) {
  __shared__ int32_t cnt[1024];
  const int e = threadIdx.x;
  if (e < E) cnt[e] = offsets[e + 1] - offsets[e];
  __syncthreads();
  if (e >= E) return;
  const int32_t c = cnt[e];
  int rank = 0;
  for (int f = 0; f < E; ++f) rank += (cnt[f] > c) || (cnt[f] == c && f < e);
  order[rank] = e;
}

// expert of sorted row p: the last e with offsets[e] <= p (offsets non-decreasing)
__device__ int expert_of_row(const int32_t* offsets, int E, int64_t p) {
  int lo = 0, hi = E - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (offsets[mid] <= p) lo = mid;
    else hi = mid - 1;
  }
  return lo;
}

// fp32 input gradients: out(p, n) = sum_c A[p, c] * W[e(p)][c, n] for the kept rows p, W
// stored (contraction, N). Epilogue: SwiGLU backward with the saved H (bwd_h > 0: n < h and
// [d_up | d_gate] to C with ldc = 2h), else rows to scatter[p] (or p).
__global__ __launch_bounds__(256) void dgrad_f32_kernel(GemmCall c) {
  const int64_t p = blockIdx.y;
  const int64_t n = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  const int64_t kept = min(max(static_cast<int64_t>(c.group_offsets[c.groups]), int64_t(0)), c.rows_bound);
  if (p >= kept || n >= c.N) return;
  const int e = expert_of_row(c.group_offsets, c.groups, p);
  const float* a = static_cast<const float*>(c.A) + p * c.lda;
  const float* b = static_cast<const float*>(c.B) + static_cast<int64_t>(e) * c.b_group_stride + n;
  float acc = 0.f;
  for (int64_t q = 0; q < c.Kd; ++q) acc = fmaf(a[q], b[q * c.ldb], acc);
  float* C = static_cast<float*>(c.C);
  if (c.bwd_h > 0) {
    const float* hr = static_cast<const float*>(c.h_in) + p * 2 * c.bwd_h;
    const float up = hr[n], gate = hr[c.bwd_h + n];
    const float sig = 1.f / (1.f + expf(-gate));
    C[p * c.ldc + n] = acc * (gate * sig);
    C[p * c.ldc + c.bwd_h + n] = acc * up * (sig * (1.f + gate * (1.f - sig)));
  } else {
    int64_t orow = c.scatter ? static_cast<int64_t>(c.scatter[p]) : p;
    orow = min(max(orow, int64_t(0)), c.c_rows - 1);
    C[orow * c.ldc + n] = acc;
  }
}

// fp32 weight gradients: C_e(m, n) = sum over rows p of group e of A[p, m] * B[p, n].
__global__ __launch_bounds__(256) void wgrad_f32_kernel(GemmCall c) {
  const int64_t n = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  const int64_t m = blockIdx.y;
  const int e = blockIdx.z;
  if (n >= c.N) return;
  const int64_t kb = min(max(static_cast<int64_t>(c.group_offsets[e]), int64_t(0)), c.rows_bound);
  const int64_t ke = min(max(static_cast<int64_t>(c.group_offsets[e + 1]), kb), c.rows_bound);
  const float* A = static_cast<const float*>(c.A);
  const float* B = static_cast<const float*>(c.B);
  float acc = 0.f;
  for (int64_t p = kb; p < ke; ++p) acc = fmaf(A[p * c.lda + m], B[p * c.ldb + n], acc);
  static_cast<float*>(c.C)[e * c.c_group_stride + m * c.ldc + n] = acc;
}

unsigned grid_of(int64_t work, int64_t per_block) {
  const int64_t blocks = (work + per_block - 1) / per_block;
  return static_cast<unsigned>(std::min<int64_t>(std::max<int64_t>(blocks, 1), int64_t(device_cu_count()) * 16));
}

}  // namespace

hipError_t launch_gather_rows(const void* src, int64_t src_rows, const int32_t* idx, int div, const int32_t* n_ptr,
                              int64_t n_max, int64_t row_bytes, void* dst, hipStream_t s) {
  if (n_max <= 0) return hipSuccess;
  if (row_bytes % 16 != 0 || div <= 0 || src_rows <= 0) return hipErrorInvalidValue;
  hipLaunchKernelGGL(gather_rows_kernel, dim3(grid_of(n_max * (row_bytes / 16), 256)), dim3(256), 0, s,
                     static_cast<const unsigned char*>(src), src_rows, idx, div, n_ptr, n_max, row_bytes,
                     static_cast<unsigned char*>(dst));
  return hipGetLastError();
}

hipError_t launch_sum_copies(const Layer& ly, const void* in, void* out, hipStream_t s) {
  if (ly.T <= 0) return hipSuccess;
  const int64_t n = ly.T * (ly.K / (ly.bf16 ? 8 : 4));
  if (ly.bf16)
    hipLaunchKernelGGL(sum_copies_kernel<uint16_t>, dim3(grid_of(n, 256)), dim3(256), 0, s,
                       static_cast<const uint16_t*>(in), ly.k, ly.T, ly.K, static_cast<uint16_t*>(out));
  else
    hipLaunchKernelGGL(sum_copies_kernel<float>, dim3(grid_of(n, 256)), dim3(256), 0, s,
                       static_cast<const float*>(in), ly.k, ly.T, ly.K, static_cast<float*>(out));
  return hipGetLastError();
}

hipError_t launch_combine_backward(const Layer& ly, const void* y_assign, const float* w, const void* d_out,
                                   void* dy_assign, float* dw, hipStream_t s) {
  if (ly.T <= 0) return hipSuccess;
  const dim3 g(static_cast<unsigned>((ly.T + 3) / 4)), b(256);
  if (ly.bf16)
    hipLaunchKernelGGL(combine_backward_kernel<uint16_t>, g, b, 0, s, static_cast<const uint16_t*>(y_assign), w,
                       static_cast<const uint16_t*>(d_out), ly.k, ly.T, ly.K, static_cast<uint16_t*>(dy_assign), dw);
  else
    hipLaunchKernelGGL(combine_backward_kernel<float>, g, b, 0, s, static_cast<const float*>(y_assign), w,
                       static_cast<const float*>(d_out), ly.k, ly.T, ly.K, static_cast<float*>(dy_assign), dw);
  return hipGetLastError();
}

hipError_t launch_fill_zero(void* p, size_t bytes, hipStream_t s) {
  if (bytes == 0) return hipSuccess;
  if (bytes % 16 != 0) return hipErrorInvalidValue;
  const int64_t n16 = static_cast<int64_t>(bytes / 16);
  hipLaunchKernelGGL(fill_zero_kernel, dim3(grid_of(n16, 256)), dim3(256), 0, s, static_cast<u32x4*>(p), n16);
  return hipGetLastError();
}

hipError_t launch_expert_order(const int32_t* offsets, int E, int32_t* order, hipStream_t s) {
  if (E <= 0 || E > 1024) return hipErrorInvalidValue;
  hipLaunchKernelGGL(expert_order_kernel, dim3(1), dim3(1024), 0, s, offsets, E, order);
  return hipGetLastError();
}

hipError_t launch_dgrad_f32(const GemmCall& c, hipStream_t s) {
  if (!c.group_offsets || c.groups <= 0 || c.rows_bound <= 0 || c.N <= 0) return hipSuccess;
  if (c.rows_bound > 65535) return hipErrorInvalidValue;  // grid y
  const dim3 g(static_cast<unsigned>((c.N + 255) / 256), static_cast<unsigned>(c.rows_bound));
  hipLaunchKernelGGL(dgrad_f32_kernel, g, dim3(256), 0, s, c);
  return hipGetLastError();
}

hipError_t launch_wgrad_f32(const GemmCall& c, hipStream_t s) {
  if (!c.group_offsets || c.groups <= 0 || c.dense_M <= 0 || c.N <= 0) return hipSuccess;
  if (c.dense_M > 65535 || c.groups > 65535) return hipErrorInvalidValue;
  const dim3 g(static_cast<unsigned>((c.N + 255) / 256), static_cast<unsigned>(c.dense_M), static_cast<unsigned>(c.groups));
  hipLaunchKernelGGL(wgrad_f32_kernel, g, dim3(256), 0, s, c);
  return hipGetLastError();
}

}  // namespace moe
