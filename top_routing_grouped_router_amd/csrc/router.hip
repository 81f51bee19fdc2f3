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
// router_mfma: the fp32 contraction on bf16 matrix cores. Each fp32 router weight is split
// exactly into three bf16 planes (hi = bf16(w), mid = bf16(w - hi), lo = bf16(w - hi - mid):
// 24 significant bits between them); x is bf16, so every product x * plane is exact in fp32
// and the three MFMA products accumulate in fp32 -- an fp32-accurate dot product (3*d terms)
// at bf16 matrix rate. Tile 64 tokens x 64 experts x 64 k (four wavefronts of 32 x 32), or
// 64 tokens x 16 experts for few tokens and many experts, on v_mfma_f32_16x16x32_bf16. The
// contraction can be split over `nsplit` workgroups along d_model for occupancy; the partial
// sums land in separate planes and the gate kernel adds them in a fixed order, so the result
// is deterministic.
//
// gate_topk: one 64-lane wavefront per token; each lane holds ceil(E/64) <= 16 experts in
// registers (the count is a template parameter). Selection is k rounds of a wave-wide
// arg-max: the largest order-preserving key code through DPP row reductions and scalar
// readlanes, the owning lane from a ballot (ties across lanes: the lowest expert index), so
// the result is exact and deterministic. The logits row is read once, coalesced.
#include <math.h>

#include <algorithm>

#include "common.hpp"

namespace moe {
namespace {

constexpr int kMaxSlots = MOE_MAX_EXPERTS / kWave;  // 16 experts per lane at most

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
  const float* in;          // (nsplit, T, E) logit partial sums, or (T, E) gating output
  int nsplit;               // partial-sum planes to add (1 when from_scores)
  const float* router_bias; // (E) or NULL, added to the logits
  float* logits_out;        // (T, E) or NULL
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

// MULTI: the input has split-K partial-sum planes to add (compiled out otherwise: the plane
// batches hold registers).
template <int GATING, bool FROM_SCORES, int PL, bool MULTI>
__global__ __launch_bounds__(256) void gate_topk_kernel(GateArgs a) {
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t t = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (t >= a.T) return;  // whole wavefront leaves together
  const int E = a.E;
  const int64_t plane = a.T * static_cast<int64_t>(E);
  const float* row = a.in + t * E;

  // Logits (or the given gating output): plane 0, then the other partial-sum planes added in
  // plane order. The plane loop is outermost so each batch issues PB * PL independent loads.
  // Padding slots (e >= E) load the last expert's value (clamped index: every load is in
  // bounds and unconditional) and are masked below.
  float v[PL];
#pragma unroll
  for (int i = 0; i < PL; ++i) v[i] = row[min(i * kWave + lane, E - 1)];
  constexpr int PB = 4;  // planes per batch (each batch's loads are issued together)
  for (int p0 = 1; MULTI && p0 < a.nsplit; p0 += PB) {
    float pv[PB][PL];
#pragma unroll
    for (int u = 0; u < PB; ++u)
#pragma unroll
      for (int i = 0; i < PL; ++i)
        pv[u][i] = row[min(p0 + u, a.nsplit - 1) * plane + min(i * kWave + lane, E - 1)];
#pragma unroll
    for (int u = 0; u < PB; ++u)
      if (p0 + u < a.nsplit) {
#pragma unroll
        for (int i = 0; i < PL; ++i) v[i] += pv[u][i];
      }
  }
#pragma unroll
  for (int i = 0; i < PL; ++i) {
    const int e = i * kWave + lane;
    if (e < E) {
      if (!FROM_SCORES && a.router_bias) v[i] += a.router_bias[e];
      if (!FROM_SCORES && a.logits_out) a.logits_out[t * E + e] = v[i];
    } else {
      v[i] = -INFINITY;
    }
  }

  float s[PL];  // gating scores
  if (!FROM_SCORES) {
    if (GATING == MOE_GATING_SIGMOID) {
#pragma unroll
      for (int i = 0; i < PL; ++i) {
        // sigmoid = 1 / (1 + 2^(-v log2 e)) on the hardware exp2 and reciprocal (a few fp32 ulp)
        float sc = __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(-v[i] * 1.44269504088896340736f));
        if (a.sig_eps != 0.f) sc = sc + a.sig_eps;
        s[i] = sc;
      }
    } else {
      float m = -INFINITY;
#pragma unroll
      for (int i = 0; i < PL; ++i) m = fmaxf(m, v[i]);
      m = wave_max_f32_dpp(m);
      float sum = 0.f;
#pragma unroll
      for (int i = 0; i < PL; ++i) {
        const int e = i * kWave + lane;
        s[i] = (e < E) ? expf(v[i] - m) : 0.f;
        sum += s[i];
      }
      sum = wave_sum_f32_dpp(sum);
#pragma unroll
      for (int i = 0; i < PL; ++i) s[i] = s[i] / sum;
    }
    if (a.scores_out) {
#pragma unroll
      for (int i = 0; i < PL; ++i) {
        const int e = i * kWave + lane;
        if (e < E) a.scores_out[t * E + e] = s[i];
      }
    }
  } else {
#pragma unroll
    for (int i = 0; i < PL; ++i) s[i] = v[i];
  }

  // Selection keys as order-preserving codes; 0 marks "no candidate" (padding, or chosen).
  uint32_t code[PL];
#pragma unroll
  for (int i = 0; i < PL; ++i) {
    const int e = i * kWave + lane;
    float key = (GATING == MOE_GATING_TOPK_SOFTMAX) ? v[i] : s[i];
    if (a.score_bias) key = key + a.score_bias[min(e, E - 1)];
    code[i] = e < E ? key_code(key) : 0u;
  }

  // k rounds. Candidates are ordered by (code descending, expert index ascending); lane l
  // holds experts l, l+64, ..., so inside a lane the slot order is the expert order. Each lane
  // keeps its two greatest remaining candidates (b1 > b2, with their slots and weight sources)
  // and a floor: its candidates at or above the floor are taken. A round finds the wave maximum
  // of the lanes' b1 with DPP (usually one lane holds it; on a tie the lowest expert index among
  // the tied lanes wins); the winning lane moves b2 up, or, when it had already used b2, re-scans
  // its slots below the floor for a new pair. The rescan runs for one lane at most per round and
  // only when that lane wins a second time, so a round is a few dozen instructions.
  auto cand_val = [&](int i) __attribute__((always_inline)) { return (GATING == MOE_GATING_TOPK_SOFTMAX) ? v[i] : s[i]; };
  uint32_t b1 = 0, b2 = 0;
  int s1 = 0, s2 = 0;
  float v1 = 0.f, v2 = 0.f;
  // top two of the slots whose (code, slot) lies below (fc, fs) (everything when !floor_set)
  auto top2 = [&](bool floor_set, uint32_t fc, int fs) __attribute__((always_inline)) {
    b1 = 0; b2 = 0; s1 = 0; s2 = 0; v1 = 0.f; v2 = 0.f;
#pragma unroll
    for (int i = 0; i < PL; ++i) {
      uint32_t c = code[i];
      if (floor_set && !(c < fc || (c == fc && i > fs))) c = 0;
      const float cv = cand_val(i);
      // branch-free, so the pairs stay in registers
      const bool gt1 = c > b1, gt2 = c > b2;
      b2 = gt1 ? b1 : (gt2 ? c : b2);
      s2 = gt1 ? s1 : (gt2 ? i : s2);
      v2 = gt1 ? v1 : (gt2 ? cv : v2);
      b1 = gt1 ? c : b1;
      s1 = gt1 ? i : s1;
      v1 = gt1 ? cv : v1;
    }
  };
  top2(false, 0u, 0);
  bool have2 = true;
  int my_sel = 0;
  float my_val = 0.f;
  for (int j = 0; j < a.k; ++j) {
    const uint32_t m = wave_max_u32_dpp(b1);
    const uint64_t ball = __ballot(b1 == m);
    int e;
    if (__popcll(ball) == 1) {
      const int wl = __ffsll(static_cast<unsigned long long>(ball)) - 1;
      e = __builtin_amdgcn_readlane(s1, wl) * kWave + wl;
    } else {
      e = wave_min_i32_dpp(b1 == m ? s1 * kWave + lane : 0x7fffffff);
    }
    e = min(max(e, 0), E - 1);  // k <= E, so a candidate always exists
    const int wl = e & (kWave - 1);
    const float val = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v1), wl));
    if (lane == j) {
      my_sel = e;
      my_val = val;
    }
    // whether the winner still holds its second candidate: uniform, so the rescan is a
    // wave-level branch taken only when needed
    if (__builtin_amdgcn_readlane(have2 ? 1 : 0, wl) != 0) {
      if (lane == wl) {
        b1 = b2; s1 = s2; v1 = v2;
        have2 = false;
      }
    } else {
      const uint32_t fc = b1;
      const int fs = s1;
      if (lane == wl) {
        top2(true, fc, fs);
        have2 = true;
      }
    }
  }

  // Weights: lane j < k holds selection j.
  const bool active = lane < a.k;
  float w;
  if (GATING == MOE_GATING_TOPK_SOFTMAX) {
    const float lv = active ? my_val : -INFINITY;
    const float m = wave_max_f32_dpp(lv);
    const float ex = active ? expf(lv - m) : 0.f;
    const float sum = wave_sum_f32_dpp(ex);
    w = ex / sum;
  } else {
    w = active ? my_val : 0.f;
  }
  if (a.norm_p != 0.f) {
    const float aw = active ? fabsf(w) : 0.f;
    float nrm;
    if (a.norm_p == 1.f) {
      nrm = wave_sum_f32_dpp(aw);
    } else if (a.norm_p == 2.f) {
      nrm = sqrtf(wave_sum_f32_dpp(aw * aw));
    } else {
      nrm = powf(wave_sum_f32_dpp(active ? powf(aw, a.norm_p) : 0.f), 1.f / a.norm_p);
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

template <int GATING, bool FS, bool MULTI>
void launch_gate_pl(const GateArgs& a, hipStream_t s) {
  const dim3 g(static_cast<unsigned>((a.T + 3) / 4)), b(256);
  const int per_lane = (a.E + kWave - 1) / kWave;
  if (per_lane <= 1) hipLaunchKernelGGL((gate_topk_kernel<GATING, FS, 1, MULTI>), g, b, 0, s, a);
  else if (per_lane <= 2) hipLaunchKernelGGL((gate_topk_kernel<GATING, FS, 2, MULTI>), g, b, 0, s, a);
  else if (per_lane <= 4) hipLaunchKernelGGL((gate_topk_kernel<GATING, FS, 4, MULTI>), g, b, 0, s, a);
  else if (per_lane <= 8) hipLaunchKernelGGL((gate_topk_kernel<GATING, FS, 8, MULTI>), g, b, 0, s, a);
  else hipLaunchKernelGGL((gate_topk_kernel<GATING, FS, kMaxSlots, MULTI>), g, b, 0, s, a);
}

template <int GATING>
void launch_gate(const GateArgs& a, bool from_scores, hipStream_t s) {
  if (from_scores) launch_gate_pl<GATING, true, false>(a, s);
  else if (a.nsplit > 1) launch_gate_pl<GATING, false, true>(a, s);
  else launch_gate_pl<GATING, false, false>(a, s);
}

// ------------------------------------------------------------------ router logits on MFMA

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kRT = 64;    // tokens per tile
constexpr int kRBK = 64;   // k per stage
constexpr int kRowB = kRBK * 2;
constexpr int kXBytes = kRT * kRowB;        // 8 KiB

// Expert tiles of the split-K router: 64 experts (2 x 2 wavefronts of 32 tokens x 32 experts)
// when the tokens alone give enough tiles; 16 experts (4 wavefronts of 16 tokens x 16 experts)
// for few tokens, so that a wide expert pool fills the chip with 4x fewer k-splits (fewer
// partial planes for the gate kernel to add).
template <int RE_>
struct RouterTile {
  static constexpr int RE = RE_;
  static constexpr int WN = RE >= 64 ? 2 : 1;   // wavefronts along experts
  static constexpr int WM = 4 / WN;             // wavefronts along tokens
  static constexpr int TI = kRT / (16 * WM);    // 16-token sub-tiles per wavefront
  static constexpr int TJ = RE / (16 * WN);     // 16-expert sub-tiles per wavefront
  static constexpr int kPlaneBytes = RE * kRowB;
  static constexpr int kStage = kXBytes + 3 * kPlaneBytes;
  static constexpr int NWQ = RE * 16 / 256;     // 16-byte fp32 weight chunks per thread per stage
  static_assert(WM * WN == 4 && TI >= 1 && TJ >= 1 && NWQ >= 1, "router tile");
};

// 16-lane passes over 16 consecutive rows: slot = chunk ^ ((row >> 1) & 7) spreads them over
// all 64 LDS banks (a 128-byte row covers half of them).
__device__ __forceinline__ int rswz(int row, int chunk) {
  return row * kRowB + ((chunk ^ ((row >> 1) & 7)) << 4);
}

__device__ __forceinline__ uint32_t pack2(uint16_t a, uint16_t b) {
  return static_cast<uint32_t>(a) | (static_cast<uint32_t>(b) << 16);
}

// w = hi + mid + lo exactly, each a bf16 (8 significant bits): hi = bf16(w), and each next
// plane rounds what the previous ones left (the differences are exact in fp32). The products
// x * plane are then exact in the MFMA's fp32 accumulation, which sums them in fp32.
__device__ __forceinline__ void split3_bf16(float w, uint16_t& hi, uint16_t& mi, uint16_t& lo) {
  hi = f32_to_bf16_bits(w);
  const float r1 = w - bf16_bits_to_f32(hi);
  mi = f32_to_bf16_bits(r1);
  const float r2 = r1 - bf16_bits_to_f32(mi);
  lo = f32_to_bf16_bits(r2);
}

// The router weights (E, d) fp32 as three bf16 planes (3, E, d): hi, mid, lo. Four elements per
// thread, grid-stride.
__global__ __launch_bounds__(256) void split_planes_kernel(const float4* __restrict__ w, uint2* __restrict__ planes,
                                                           int64_t n4) {
  for (int64_t i = blockIdx.x * 256 + threadIdx.x; i < n4; i += static_cast<int64_t>(gridDim.x) * 256) {
    const float4 v = w[i];
    uint16_t h[4], m[4], l[4];
    split3_bf16(v.x, h[0], m[0], l[0]);
    split3_bf16(v.y, h[1], m[1], l[1]);
    split3_bf16(v.z, h[2], m[2], l[2]);
    split3_bf16(v.w, h[3], m[3], l[3]);
    planes[i] = make_uint2(pack2(h[0], h[1]), pack2(h[2], h[3]));
    planes[n4 + i] = make_uint2(pack2(m[0], m[1]), pack2(m[2], m[3]));
    planes[2 * n4 + i] = make_uint2(pack2(l[0], l[1]), pack2(l[2], l[3]));
  }
}

template <class RT>
__global__ __launch_bounds__(256) void router_mfma_kernel(const uint16_t* __restrict__ x,
                                                          const float* __restrict__ Wr,
                                                          float* __restrict__ part, int64_t T, int E,
                                                          int d, int nsplit) {
  __shared__ __attribute__((aligned(16))) unsigned char lds[2 * RT::kStage];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / RT::WN, wn = wave % RT::WN;
  const int64_t t0 = static_cast<int64_t>(blockIdx.x) * kRT;
  const int e0 = blockIdx.y * RT::RE;
  const int sp = blockIdx.z;
  const int nk = d / kRBK;
  const int kb = static_cast<int>(static_cast<int64_t>(sp) * nk / nsplit);
  const int ke = static_cast<int>(static_cast<int64_t>(sp + 1) * nk / nsplit);

  const unsigned char* xb = reinterpret_cast<const unsigned char*>(x);
  const unsigned char* wb = reinterpret_cast<const unsigned char*>(Wr);
  uint32_t xoff[2], woff[RT::NWQ];
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int c = tid + 256 * q, row = c >> 3, ch = c & 7;
    const int64_t t = min(t0 + row, T - 1);
    xoff[q] = static_cast<uint32_t>((t * d + ch * 8) * 2);
  }
#pragma unroll
  for (int q = 0; q < RT::NWQ; ++q) {
    const int c = tid + 256 * q, row = c >> 4, c4 = c & 15;
    const int64_t e = min(e0 + row, E - 1);
    woff[q] = static_cast<uint32_t>((e * d + c4 * 4) * 4);
  }

  u32x4 rx[2];
  f32x4 rw[RT::NWQ];
  auto gload = [&](int kt) {
#pragma unroll
    for (int q = 0; q < 2; ++q)
      rx[q] = *reinterpret_cast<const u32x4*>(xb + (xoff[q] + static_cast<uint32_t>(kt) * kRowB));
#pragma unroll
    for (int q = 0; q < RT::NWQ; ++q)
      rw[q] = *reinterpret_cast<const f32x4*>(wb + (woff[q] + static_cast<uint32_t>(kt) * (kRBK * 4)));
  };
  auto sstore = [&](int buf) {
    unsigned char* base = lds + buf * RT::kStage;
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int c = tid + 256 * q;
      *reinterpret_cast<u32x4*>(base + rswz(c >> 3, c & 7)) = rx[q];
    }
#pragma unroll
    for (int q = 0; q < RT::NWQ; ++q) {
      const int c = tid + 256 * q, row = c >> 4, c4 = c & 15;
      uint16_t hi[4], mi[4], lo[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) split3_bf16(rw[q][r], hi[r], mi[r], lo[r]);
      const int off = rswz(row, c4 >> 1) + (c4 & 1) * 8;
      unsigned char* pl = base + kXBytes;
      *reinterpret_cast<uint2*>(pl + off) = make_uint2(pack2(hi[0], hi[1]), pack2(hi[2], hi[3]));
      *reinterpret_cast<uint2*>(pl + RT::kPlaneBytes + off) = make_uint2(pack2(mi[0], mi[1]), pack2(mi[2], mi[3]));
      *reinterpret_cast<uint2*>(pl + 2 * RT::kPlaneBytes + off) = make_uint2(pack2(lo[0], lo[1]), pack2(lo[2], lo[3]));
    }
  };

  f32x4 acc[RT::TI][RT::TJ];
#pragma unroll
  for (int i = 0; i < RT::TI; ++i)
#pragma unroll
    for (int j = 0; j < RT::TJ; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  if (kb < ke) {
    gload(kb);
    sstore(0);
    __syncthreads();
    for (int kt = kb; kt < ke; ++kt) {
      const int buf = (kt - kb) & 1;
      if (kt + 1 < ke) gload(kt + 1);
      const unsigned char* X = lds + buf * RT::kStage;
      const unsigned char* Wp = X + kXBytes;
#pragma unroll
      for (int s32 = 0; s32 < 2; ++s32) {
        const int ch = 4 * s32 + (lane >> 4);
        bf16x8 xf[RT::TI], wf[3][RT::TJ];
#pragma unroll
        for (int i = 0; i < RT::TI; ++i)
          xf[i] = *reinterpret_cast<const bf16x8*>(X + rswz(16 * (RT::TI * wm + i) + (lane & 15), ch));
#pragma unroll
        for (int p = 0; p < 3; ++p)
#pragma unroll
          for (int j = 0; j < RT::TJ; ++j)
            wf[p][j] = *reinterpret_cast<const bf16x8*>(Wp + p * RT::kPlaneBytes +
                                                       rswz(16 * (RT::TJ * wn + j) + (lane & 15), ch));
#pragma unroll
        for (int i = 0; i < RT::TI; ++i)
#pragma unroll
          for (int j = 0; j < RT::TJ; ++j)
#pragma unroll
            for (int p = 2; p >= 0; --p)
              acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wf[p][j], xf[i], acc[i][j], 0, 0, 0);
      }
      if (kt + 1 < ke) sstore(buf ^ 1);
      __syncthreads();
    }
  }

  // Lane holds token (lane & 15) of each 16-token sub-tile and experts 4*(lane >> 4) + r.
  float* out = part + static_cast<int64_t>(sp) * T * E;
#pragma unroll
  for (int i = 0; i < RT::TI; ++i) {
    const int64_t t = t0 + 16 * (RT::TI * wm + i) + (lane & 15);
    if (t >= T) continue;
#pragma unroll
    for (int j = 0; j < RT::TJ; ++j) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int e = e0 + 16 * (RT::TJ * wn + j) + 4 * (lane >> 4) + r;
        if (e < E) out[t * E + e] = acc[i][j][r];
      }
    }
  }
}

// Expert-tile width of the split-K router for this layer (RouterTile<RE>) and its k-splits.
struct RouterPlan {
  int re;
  int splits;
};

RouterPlan router_plan(const Layer& ly) {
  const int nk = static_cast<int>(ly.d / kRBK);
  const int64_t tm = (ly.T + kRT - 1) / kRT;
  RouterPlan p{64, 1};
  int64_t tiles = tm * ((ly.E + 63) / 64);
  int64_t target = 512;
  if (ly.E > 64 && tiles * 8 < 512) {  // few tokens, wide pool: narrow expert tiles
    p.re = 16;
    tiles = tm * ((ly.E + 15) / 16);
    target = 384;
  }
  // enough workgroups to cover the chip (a fixed target, so the workspace size does not
  // depend on the device), each keeping at least one k-stage
  while (p.splits * 2 <= nk && p.splits < 32 && tiles * p.splits < target) p.splits *= 2;
  return p;
}

}  // namespace

bool router_uses_planes(const Layer& ly) {
  // The planes path runs the router as one large dense MFMA GEMM (tiles of 256 tokens x
  // gemm_bf16_planes_tile_n() experts): worth it once those tiles cover the chip.
  if (!ly.bf16 || ly.E % 4 != 0 || ly.E < 128) return false;
  const int64_t tn = gemm_bf16_planes_tile_n();
  return ((ly.T + 255) / 256) * ((ly.E + tn - 1) / tn) >= 256;
}

size_t router_scratch_bytes(const Layer& ly) {
  return router_uses_planes(ly) ? static_cast<size_t>(3) * ly.E * ly.d * 2 : 0;
}

int router_splits(const Layer& ly) {
  if (!ly.bf16 || router_uses_planes(ly)) return 1;
  return router_plan(ly).splits;
}

hipError_t launch_gate_topk(const Layer& ly, const float* input, int nsplit, bool from_scores,
                            const float* score_bias, const float* router_bias, int32_t* idx, float* w,
                            float* scores_out, float* logits_out, hipStream_t s) {
  if (ly.T <= 0) return hipSuccess;
  GateArgs a;
  a.in = input;
  a.nsplit = from_scores ? 1 : nsplit;
  a.router_bias = from_scores ? nullptr : router_bias;
  a.logits_out = from_scores ? nullptr : logits_out;
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

hipError_t launch_router_logits(const Layer& ly, const void* x, const float* Wr, float* partials,
                                int nsplit, void* scratch, hipStream_t s) {
  if (ly.T <= 0) return hipSuccess;
  if (router_uses_planes(ly)) {
    const int64_t n4 = static_cast<int64_t>(ly.E) * ly.d / 4;
    const unsigned blocks = static_cast<unsigned>(std::min<int64_t>((n4 + 255) / 256, 4096));
    hipLaunchKernelGGL(split_planes_kernel, dim3(blocks), dim3(256), 0, s, reinterpret_cast<const float4*>(Wr),
                       static_cast<uint2*>(scratch), n4);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    GemmCall c{};
    c.A = x;
    c.lda = ly.d;
    c.B = scratch;
    c.ldb = ly.d;
    c.b_plane_stride = static_cast<int64_t>(ly.E) * ly.d;
    c.C = partials;
    c.ldc = ly.E;
    c.N = ly.E;
    c.Kd = ly.d;
    c.dense_M = ly.T;
    c.a_rows = ly.T;
    c.c_rows = ly.T;
    c.rows_bound = ly.T;
    return launch_gemm_bf16_planes_f32(c, s);
  }
  if (ly.bf16) {
    const RouterPlan p = router_plan(ly);
    const dim3 g(static_cast<unsigned>((ly.T + kRT - 1) / kRT), static_cast<unsigned>((ly.E + p.re - 1) / p.re),
                 static_cast<unsigned>(nsplit));
    if (p.re == 16)
      hipLaunchKernelGGL(router_mfma_kernel<RouterTile<16>>, g, dim3(256), 0, s, static_cast<const uint16_t*>(x), Wr,
                         partials, ly.T, ly.E, static_cast<int>(ly.d), nsplit);
    else
      hipLaunchKernelGGL(router_mfma_kernel<RouterTile<64>>, g, dim3(256), 0, s, static_cast<const uint16_t*>(x), Wr,
                         partials, ly.T, ly.E, static_cast<int>(ly.d), nsplit);
    return hipGetLastError();
  }
  GemmCall c{};
  c.A = x;
  c.lda = ly.d;
  c.B = Wr;
  c.ldb = ly.d;
  c.C = partials;
  c.ldc = ly.E;
  c.N = ly.E;
  c.Kd = ly.d;
  c.dense_M = ly.T;
  c.a_rows = ly.T;
  c.c_rows = ly.T;
  c.rows_bound = ly.T;
  return launch_gemm_f32(c, false, nullptr, s);
}

}  // namespace moe
