// Load-balancing state of the router: the per-expert count accumulator, the load-imbalance
// metric and the aux-loss-free score_bias update.
//
// "Как устроен Olmo-core 3: обучение больших MoE-моделей", section "Счётчики и
// bias-корректировка": score_bias_batch_size_per_expert accumulates the tokens assigned to
// each expert and is reset after every step; the update adds bias_gamma * sign(ideal -
// actual) to score_bias, ideal being the mean size per expert; load imbalance is the maximum
// of the counter divided by its mean. Section "Управление состоянием между шагами": the
// update runs after the step's last backward, before the optimiser step, and zeroes the
// accumulator.
//
// Exact arithmetic: the sign is taken in integers, sign(total - E * actual), so no rounding
// of total / E can flip it; the imbalance is max * E / total as one fp64 division of exact
// integers (correctly rounded; NaN with no tokens); the bias moves by one fp32 add of
// +-gamma or 0. The reductions are integer sums and maxima, so the results do not depend on
// the order of the reduction.
//
// The work is E <= 1024 integers: one workgroup of 1024 threads, one expert per thread.
#include <math.h>

#include "common.hpp"

namespace moe {
namespace {

constexpr int kBalanceThreads = 1024;

// Sum of vs and maximum of vm over the workgroup (one of each per thread); every thread gets
// both. Ends with a barrier, so the shared slots may be reused right after.
__device__ void block_sum_max_i64(int64_t vs, int64_t vm, int64_t& sum, int64_t& mx) {
  __shared__ int64_t ssum[kBalanceThreads / kWave], smax[kBalanceThreads / kWave];
  int64_t s = vs, m = vm;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    s += __shfl_xor(s, o, kWave);
    const int64_t u = __shfl_xor(m, o, kWave);
    m = u > m ? u : m;
  }
  const int wave = threadIdx.x / kWave, nw = blockDim.x / kWave;
  if ((threadIdx.x & (kWave - 1)) == 0) {
    ssum[wave] = s;
    smax[wave] = m;
  }
  __syncthreads();
  s = ssum[0];
  m = smax[0];
  for (int w = 1; w < nw; ++w) {
    s += ssum[w];
    m = smax[w] > m ? smax[w] : m;
  }
  __syncthreads();
  sum = s;
  mx = m;
}

__device__ double imbalance_of(int64_t total, int64_t mx, int E) {
  if (total == 0) return __longlong_as_double(0x7ff8000000000000ll);  // 0 / 0
  return static_cast<double>(mx * static_cast<int64_t>(E)) / static_cast<double>(total);
}

__global__ __launch_bounds__(256) void accumulate_counts_kernel(int E, const int32_t* __restrict__ counts,
                                                                int64_t* __restrict__ acc) {
  const int e = blockIdx.x * 256 + threadIdx.x;
  if (e < E) acc[e] += counts[e];
}

__global__ __launch_bounds__(kBalanceThreads) void load_imbalance_kernel(int E, const int64_t* __restrict__ counts,
                                                                         double* __restrict__ out) {
  const int e = threadIdx.x;
  const int64_t c = e < E ? counts[e] : 0;
  int64_t total, mx;
  block_sum_max_i64(c, e < E ? c : INT64_MIN, total, mx);
  if (e == 0) *out = imbalance_of(total, mx, E);
}

__global__ __launch_bounds__(kBalanceThreads) void score_bias_update_kernel(int E, float gamma,
                                                                            int64_t* __restrict__ acc,
                                                                            float* __restrict__ bias,
                                                                            double* __restrict__ imbalance) {
  const int e = threadIdx.x;
  const int64_t c = e < E ? acc[e] : 0;
  int64_t total, mx;
  block_sum_max_i64(c, e < E ? c : INT64_MIN, total, mx);
  if (imbalance && e == 0) *imbalance = imbalance_of(total, mx, E);
  if (e < E) {
    const int64_t d = total - static_cast<int64_t>(E) * c;  // sign(ideal - actual) * E
    const float sgn = d > 0 ? 1.f : (d < 0 ? -1.f : 0.f);
    bias[e] = bias[e] + gamma * sgn;
    acc[e] = 0;
  }
}

}  // namespace

hipError_t launch_accumulate_counts(int E, const int32_t* counts, int64_t* acc, hipStream_t s) {
  hipLaunchKernelGGL(accumulate_counts_kernel, dim3((E + 255) / 256), dim3(256), 0, s, E, counts, acc);
  return hipGetLastError();
}

hipError_t launch_load_imbalance(int E, const int64_t* counts, double* out, hipStream_t s) {
  hipLaunchKernelGGL(load_imbalance_kernel, dim3(1), dim3(kBalanceThreads), 0, s, E, counts, out);
  return hipGetLastError();
}

hipError_t launch_score_bias_update(int E, float gamma, int64_t* acc, float* bias, double* imbalance,
                                    hipStream_t s) {
  hipLaunchKernelGGL(score_bias_update_kernel, dim3(1), dim3(kBalanceThreads), 0, s, E, gamma, acc, bias,
                     imbalance);
  return hipGetLastError();
}

}  // namespace moe
