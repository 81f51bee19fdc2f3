// Router of the MoE layer: fp32 logits, gating, top-k selection, expert weights.
//
// Follows "Как устроен Olmo-core 3: обучение больших MoE-моделей", section "Маршрутизация:
// как роутер выбирает экспертов":
//   * logits = fp32(x) * W_r^T (+ bias), W_r of shape (num_experts, d_model);
//   * softmax and topk_softmax score with a softmax over the experts; sigmoid scores each
//     expert alone and adds sigmoid_stability_epsilon when set;
//   * topk_softmax selects on logits (+ score_bias) and weights with a softmax over the chosen
//     logits; the others select on scores (+ score_bias) and gather the original scores
//     (section "Счётчики и bias-корректировка": the bias steers selection only);
//   * weights divided by their p-norm, then scaled by top_k (restore_weight_scale), by
//     expert_weight_scale, and by sqrt(original_top_k / top_k).
// Ties go to the lower expert index (the intent stated in section "Разрешение равенства
// логитов и квантизация"); keys compare as IEEE numbers (-0.0 == +0.0) and NaN keys rank
// after every number.
//
// gate_topk: one 64-lane wavefront per token; each lane holds ceil(E/64) <= 16 experts in
// registers. Selection is k rounds of a wave-wide arg-max over a 64-bit key
// (order-preserving bits of the key, then the complemented expert index), so each round is
// six xor-shuffle steps and the result is exact and deterministic. The logits row is read
// once, coalesced; the kernel is bound by HBM/L2 reads of the logits.
#include <math.h>

#include "common.hpp"

namespace moe {
namespace {

constexpr int kMaxPerLane = MOE_MAX_EXPERTS / kWave;  // 16

// Order-preserving 32-bit code of a selection key: larger key -> larger code; both zeros map
// to one code; NaN maps to 1, below every number (-inf maps to 0x007FFFFF); 0 means "no
// candidate".
__device__ __forceinline__ uint32_t key_code(float key) {
  if (key != key) return 1u;
  if (key == 0.f) key = 0.f;
  const uint32_t u = __float_as_uint(key);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

struct GateArgs {
  const float* in;          // (T, E) logits, or the gating output when from_scores
  const float* score_bias;  // (E) or NULL
  int32_t* idx;             // (T, k)
  float* w;                 // (T, k)
  float* scores_out;        // (T, E) or NULL
  int64_t T;
  int E;
  int k;
  float sig_eps;
  float norm_p;
  int restore_scale;
  float ews;
  int orig_k;
};

template <int GATING, bool FROM_SCORES>
__global__ __launch_bounds__(256) void gate_topk_kernel(GateArgs a) {
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t t = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (t >= a.T) return;  // whole wavefront leaves together
  const int E = a.E;
  const float* row = a.in + t * E;

  float v[kMaxPerLane];  // input values
  float s[kMaxPerLane];  // gating scores (unused for topk_softmax weights)
#pragma unroll
  for (int i = 0; i < kMaxPerLane; ++i) {
    const int e = i * kWave + lane;
    v[i] = (i * kWave < E && e < E) ? row[e] : -INFINITY;
  }

  if (!FROM_SCORES) {
    if (GATING == MOE_GATING_SIGMOID) {
#pragma unroll
      for (int i = 0; i < kMaxPerLane; ++i) {
        float sc = 1.f / (1.f + expf(-v[i]));
        if (a.sig_eps != 0.f) sc = sc + a.sig_eps;
        s[i] = sc;
      }
    } else {
      float m = -INFINITY;
#pragma unroll
      for (int i = 0; i < kMaxPerLane; ++i) m = fmaxf(m, v[i]);
      m = wave_max(m);
      float sum = 0.f;
#pragma unroll
      for (int i = 0; i < kMaxPerLane; ++i) {
        const int e = i * kWave + lane;
        s[i] = (e < E) ? expf(v[i] - m) : 0.f;
        sum += s[i];
      }
      sum = wave_sum(sum);
#pragma unroll
      for (int i = 0; i < kMaxPerLane; ++i) s[i] = s[i] / sum;
    }
    if (a.scores_out) {
#pragma unroll
      for (int i = 0; i < kMaxPerLane; ++i) {
        const int e = i * kWave + lane;
        if (i * kWave < E && e < E) a.scores_out[t * E + e] = s[i];
      }
    }
  } else {
#pragma unroll
    for (int i = 0; i < kMaxPerLane; ++i) s[i] = v[i];
  }

  // 64-bit candidates: (key code << 32) | ~expert. Max = largest key, then lowest index.
  uint64_t cand[kMaxPerLane];
#pragma unroll
  for (int i = 0; i < kMaxPerLane; ++i) {
    const int e = i * kWave + lane;
    if (i * kWave < E && e < E) {
      float key = (GATING == MOE_GATING_TOPK_SOFTMAX) ? v[i] : s[i];
      if (a.score_bias) key = key + a.score_bias[e];
      cand[i] = (static_cast<uint64_t>(key_code(key)) << 32) | static_cast<uint32_t>(~e);
    } else {
      cand[i] = 0;
    }
  }

  int my_sel = 0;
  for (int j = 0; j < a.k; ++j) {
    uint64_t best = 0;
#pragma unroll
    for (int i = 0; i < kMaxPerLane; ++i) best = cand[i] > best ? cand[i] : best;
    best = wave_max_u64(best);
    int e = static_cast<int>(~static_cast<uint32_t>(best));
    e = min(max(e, 0), E - 1);  // k <= E, so a candidate always exists
    if (lane == j) my_sel = e;
    if (lane == (e & (kWave - 1))) {
#pragma unroll
      for (int i = 0; i < kMaxPerLane; ++i)
        if (i == (e >> 6)) cand[i] = 0;
    }
  }

  // Weights: lane j < k holds selection j.
  const bool active = lane < a.k;
  float w;
  if (GATING == MOE_GATING_TOPK_SOFTMAX) {
    const float lv = active ? row[my_sel] : -INFINITY;
    const float m = wave_max(lv);
    const float ex = active ? expf(lv - m) : 0.f;
    const float sum = wave_sum(ex);
    w = ex / sum;
  } else {
    // Fetch the exact score register of the selected expert from its owning lane.
    const int src = my_sel & (kWave - 1), slot = my_sel >> 6;
    w = 0.f;
#pragma unroll
    for (int i = 0; i < kMaxPerLane; ++i) {
      const float sv = __shfl(s[i], src, kWave);
      if (i == slot) w = sv;
    }
    if (!active) w = 0.f;
  }
  if (a.norm_p != 0.f) {
    const float aw = active ? fabsf(w) : 0.f;
    float nrm;
    if (a.norm_p == 1.f) {
      nrm = wave_sum(aw);
    } else if (a.norm_p == 2.f) {
      nrm = sqrtf(wave_sum(aw * aw));
    } else {
      nrm = powf(wave_sum(active ? powf(aw, a.norm_p) : 0.f), 1.f / a.norm_p);
    }
    w = w / nrm;
  }
  if (a.restore_scale) w = w * static_cast<float>(a.k);
  if (a.ews != 0.f) w = w * a.ews;
  if (a.orig_k != 0 && a.orig_k != a.k)
    w = w * sqrtf(static_cast<float>(a.orig_k) / static_cast<float>(a.k));
  if (active) {
    a.idx[t * a.k + lane] = my_sel;
    a.w[t * a.k + lane] = w;
  }
}

template <int GATING>
void launch_gate(const GateArgs& a, bool from_scores, hipStream_t s) {
  const dim3 g(static_cast<unsigned>((a.T + 3) / 4)), b(256);
  if (from_scores) hipLaunchKernelGGL((gate_topk_kernel<GATING, true>), g, b, 0, s, a);
  else hipLaunchKernelGGL((gate_topk_kernel<GATING, false>), g, b, 0, s, a);
}

}  // namespace

hipError_t launch_gate_topk(const Layer& ly, const float* input, bool from_scores,
                            const float* score_bias, int32_t* idx, float* w, float* scores_out,
                            hipStream_t s) {
  if (ly.T <= 0) return hipSuccess;
  GateArgs a;
  a.in = input;
  a.score_bias = score_bias;
  a.idx = idx;
  a.w = w;
  a.scores_out = from_scores ? nullptr : scores_out;
  a.T = ly.T;
  a.E = ly.E;
  a.k = ly.k;
  a.sig_eps = ly.sig_eps;
  a.norm_p = ly.norm_p;
  a.restore_scale = ly.restore_scale ? 1 : 0;
  a.ews = ly.ews;
  a.orig_k = ly.orig_k;
  switch (ly.gating) {
    case MOE_GATING_SOFTMAX: launch_gate<MOE_GATING_SOFTMAX>(a, from_scores, s); break;
    case MOE_GATING_TOPK_SOFTMAX: launch_gate<MOE_GATING_TOPK_SOFTMAX>(a, from_scores, s); break;
    default: launch_gate<MOE_GATING_SIGMOID>(a, from_scores, s); break;
  }
  return hipGetLastError();
}

hipError_t launch_router_logits(const Layer& ly, const void* x, const float* Wr, const float* br,
                                float* logits, hipStream_t s) {
  if (ly.T <= 0) return hipSuccess;
  GemmCall c{};
  c.A = x;
  c.lda = ly.d;
  c.B = Wr;
  c.ldb = ly.d;
  c.C = logits;
  c.ldc = ly.E;
  c.N = ly.E;
  c.Kd = ly.d;
  c.dense_M = ly.T;
  c.a_rows = ly.T;
  c.c_rows = ly.T;
  c.rows_bound = ly.T;
  return launch_gemm_f32(c, ly.bf16, ly.router_bias ? br : nullptr, s);
}

}  // namespace moe
