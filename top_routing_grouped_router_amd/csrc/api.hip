// C ABI of the MoE layer library: validation, parameter counts, workspace layout and the
// launch sequence of the forward pass. Every argument check runs on the host before any HIP
// call, so the error paths are testable without a GPU.
//
// Layer definition: "Как устроен Olmo-core 3: обучение больших MoE-моделей" (sections
// "Как задаётся конфигурация MoE", "Латентная проекция экспертов", "Маршрутизация: как
// роутер выбирает экспертов", "Пересылка токенов между экспертами", "Вычисления экспертов и
// точность", "SwiGLU с квантизацией").
#include <math.h>
#include <stdio.h>

#include <algorithm>
#include <mutex>
#include <string>
#include <vector>

#include "common.hpp"

// Device memory of moe_forward_noalloc: the forward's workspace for callers that cannot
// allocate. One copy per GPU, held until the process ends; host code uses the per-device
// address from hipGetSymbolAddress, never this name (the name is a host-side stand-in).
static __device__ __align__(256) unsigned char scratch[MOE_NOALLOC_SCRATCH_BYTES];

namespace moe {

namespace {

thread_local std::string g_last_error;

moe_status_t fail(moe_status_t st, const std::string& msg) {
  g_last_error = msg;
  return st;
}

moe_status_t ok() {
  g_last_error.clear();
  return MOE_OK;
}

moe_status_t hip_fail(hipError_t e, const char* where) {
  return fail(MOE_ERR_HIP, std::string(where) + ": " + hipGetErrorString(e));
}

#define MOE_TRY_HIP(expr, where)              \
  do {                                        \
    hipError_t e_ = (expr);                   \
    if (e_ != hipSuccess) return hip_fail(e_, where); \
  } while (0)

bool finite(float v) { return isfinite(v); }

moe_status_t validate_config(const moe_config_t* c) {
  if (!c) return fail(MOE_ERR_INVALID_ARG, "config is NULL");
  if (c->struct_size != static_cast<int32_t>(sizeof(moe_config_t)))
    return fail(MOE_ERR_INVALID_ARG, "config struct_size does not match this library's moe_config_t");
  if (c->d_model <= 0) return fail(MOE_ERR_INVALID_ARG, "d_model must be positive");
  if (c->num_experts <= 0) return fail(MOE_ERR_INVALID_ARG, "num_experts must be positive");
  if (c->top_k <= 0) return fail(MOE_ERR_INVALID_ARG, "top_k must be positive");
  if (c->top_k > c->num_experts) return fail(MOE_ERR_INVALID_ARG, "top_k exceeds num_experts");
  if (c->hidden_size <= 0) return fail(MOE_ERR_INVALID_ARG, "hidden_size must be positive");
  if (c->latent_dim < 0) return fail(MOE_ERR_INVALID_ARG, "latent_dim must be >= 0");
  if (c->gating_function < MOE_GATING_SOFTMAX || c->gating_function > MOE_GATING_SIGMOID)
    return fail(MOE_ERR_INVALID_ARG, "unknown gating_function");
  if (c->dtype != MOE_DTYPE_F32 && c->dtype != MOE_DTYPE_BF16)
    return fail(MOE_ERR_INVALID_ARG, "unknown dtype");
  if (!finite(c->capacity_factor) || c->capacity_factor < 0.f)
    return fail(MOE_ERR_INVALID_ARG, "capacity_factor must be finite and >= 0 (0 = dropless)");
  if (!finite(c->sigmoid_stability_epsilon) || c->sigmoid_stability_epsilon < 0.f)
    return fail(MOE_ERR_INVALID_ARG, "sigmoid_stability_epsilon must be finite and >= 0");
  if (!finite(c->normalize_expert_weights) || c->normalize_expert_weights < 0.f)
    return fail(MOE_ERR_INVALID_ARG, "normalize_expert_weights (p) must be finite and >= 0");
  if (!finite(c->expert_weight_scale)) return fail(MOE_ERR_INVALID_ARG, "expert_weight_scale must be finite");
  if (c->original_top_k < 0) return fail(MOE_ERR_INVALID_ARG, "original_top_k must be >= 0");
  if (!finite(c->up_proj_input_norm_eps) || c->up_proj_input_norm_eps < 0.f)
    return fail(MOE_ERR_INVALID_ARG, "up_proj_input_norm_eps must be finite and >= 0");
  if (c->activation != MOE_ACT_SWIGLU)
    return fail(MOE_ERR_UNSUPPORTED, "only the swiglu activation is implemented");
  if (c->num_experts > MOE_MAX_EXPERTS)
    return fail(MOE_ERR_UNSUPPORTED, "num_experts above 1024 is not supported");
  if (c->top_k > MOE_MAX_TOP_K) return fail(MOE_ERR_UNSUPPORTED, "top_k above 16 is not supported");
  const int64_t mult = c->dtype == MOE_DTYPE_BF16 ? 64 : 4;
  const char* mult_msg = c->dtype == MOE_DTYPE_BF16 ? "64 for bf16" : "4 for f32";
  if (c->d_model % mult || c->hidden_size % mult || c->latent_dim % mult)
    return fail(MOE_ERR_UNSUPPORTED,
                std::string("d_model, hidden_size and latent_dim must be multiples of ") + mult_msg);
  const int64_t K = c->latent_dim ? c->latent_dim : c->d_model;
  const int64_t kmax = c->dtype == MOE_DTYPE_BF16 ? 16384 : 8192;
  if (K > kmax)
    return fail(MOE_ERR_UNSUPPORTED, "expert width (latent_dim or d_model) above 16384 (bf16) / 8192 (f32)");
  if (c->d_model > (int64_t(1) << 30) || c->hidden_size > (int64_t(1) << 30))
    return fail(MOE_ERR_UNSUPPORTED, "dimension too large");
  if (c->expert_precision != MOE_PRECISION_BF16 && c->expert_precision != MOE_PRECISION_MXFP8)
    return fail(MOE_ERR_INVALID_ARG, "unknown expert_precision");
  if (c->expert_precision == MOE_PRECISION_MXFP8) {
    if (c->dtype != MOE_DTYPE_BF16) return fail(MOE_ERR_UNSUPPORTED, "MXFP8 experts need a bf16 layer");
    if (K % 128 || c->hidden_size % 128)
      return fail(MOE_ERR_UNSUPPORTED, "MXFP8 experts need the expert width and hidden_size to be multiples of 128");
  }
  return ok();
}

// [OC3 "Ёмкость эксперта и переполнение"]: capacity = 8 * ceil(cf * top_k * T / (8 * E)) at
// expert-parallel degree 1, in exact integer arithmetic: cf = M * 2^(ex - 24) with M its 24-bit
// integer significand. A capacity of at least T drops nothing (no expert receives more than T
// assignments), so larger values are clamped to T rounded up to 8. 0 = dropless.
int64_t expert_capacity(float cf, int32_t k, int64_t T, int32_t E) {
  if (!(cf > 0.f) || T <= 0) return 0;
  const int64_t no_drop = (T + 7) / 8 * 8;
  if (static_cast<double>(cf) * k * static_cast<double>(T) / E >= static_cast<double>(T) + 16.0) return no_drop;
  int ex = 0;
  const double frac = frexp(static_cast<double>(cf), &ex);  // cf = frac * 2^ex, frac in [0.5, 1)
  const __int128 M = static_cast<__int128>(ldexp(frac, 24));  // exact: cf has 24 significant bits
  __int128 num = M * k * T;                                  // < 2^59
  __int128 den = static_cast<__int128>(8) * E;
  const int sh = ex - 24;                                    // value = num * 2^sh / den
  if (sh >= 0) {
    num <<= sh;  // sh is small here: cf * k * T / E < T + 16 bounds it
  } else if (-sh < 64) {
    den <<= -sh;
  } else {
    return 8;  // cf * k * T / E < 2^-20: the quotient rounds up to one block of 8
  }
  const __int128 q = (num + den - 1) / den;
  const int64_t cap = static_cast<int64_t>(q) * 8;
  return cap < no_drop ? cap : no_drop;
}

Layer make_layer(const moe_config_t* c, int64_t T) {
  Layer ly{};
  ly.T = T;
  ly.d = c->d_model;
  ly.E = c->num_experts;
  ly.k = c->top_k;
  ly.h = c->hidden_size;
  ly.L = c->latent_dim;
  ly.K = c->latent_dim ? c->latent_dim : c->d_model;
  ly.gating = c->gating_function;
  ly.bf16 = c->dtype == MOE_DTYPE_BF16;
  ly.sig_eps = c->sigmoid_stability_epsilon;
  ly.norm_p = c->normalize_expert_weights;
  ly.restore_scale = c->restore_weight_scale != 0;
  ly.ews = c->expert_weight_scale;
  ly.orig_k = c->original_top_k;
  ly.router_bias = c->router_bias != 0;
  ly.up_norm = c->up_proj_input_norm != 0;
  ly.norm_eps = c->up_proj_input_norm_eps;
  ly.capacity = expert_capacity(c->capacity_factor, c->top_k, T, c->num_experts);
  ly.mx = c->expert_precision == MOE_PRECISION_MXFP8;
  return ly;
}

moe_status_t check_tokens(const moe_config_t* c, int64_t T) {
  if (T < 0) return fail(MOE_ERR_INVALID_ARG, "num_tokens must be >= 0");
  if (T * static_cast<int64_t>(c->top_k) >= (int64_t(1) << 31))
    return fail(MOE_ERR_INVALID_ARG, "num_tokens * top_k must be below 2^31 (int32 offsets)");
  if (T * static_cast<int64_t>(c->num_experts) >= (int64_t(1) << 40))
    return fail(MOE_ERR_INVALID_ARG, "num_tokens * num_experts too large");
  if (c->dtype == MOE_DTYPE_BF16) {
    // The bf16 MFMA GEMM addresses each operand (and each expert's weights) with 32-bit byte
    // offsets: every one must stay below 4 GiB.
    const int64_t K = c->latent_dim ? c->latent_dim : c->d_model;
    const int64_t A = T * c->top_k;
    const int64_t lim = int64_t(1) << 31;  // elements of 2 bytes
    // (3 * E * d: the router weights split into three bf16 planes for the large-layer router)
    if (T * c->d_model >= lim || T * K >= lim || A * c->hidden_size >= lim || A * K >= lim ||
        2 * c->hidden_size * K >= lim || c->d_model * K >= lim || 3 * c->num_experts * c->d_model >= lim)
      return fail(MOE_ERR_UNSUPPORTED, "a bf16 GEMM operand would exceed 4 GiB; split the batch");
  }
  return MOE_OK;
}

size_t elem_size(const Layer& ly) { return ly.bf16 ? 2 : 4; }

// How the expert GEMMs cut each expert's rows into M-tiles. bf16: the large shape's 256-row
// tiles, with remainders of at most 128 rows in 64-row tiles of the small shape (a second
// launch); fp32 and MXFP8: one list of their single shape.
constexpr int kSmallRemainderMax = 128;
TilePlan tile_plan(const Layer& ly) {
  if (ly.mx) return TilePlan{gemm_mx_tile_m(), gemm_mx_tile_m(), 0};
  if (!ly.bf16) return TilePlan{kF32TileM, kF32TileM, 0};
  return TilePlan{gemm_bf16_tile_m(0), gemm_bf16_tile_m(1), kSmallRemainderMax};
}
// No expert receives more than T rows: with T at most the largest remainder every expert's
// rows go to the remainder list and the main list is empty.
bool main_list_empty(const Layer& ly, const TilePlan& p) { return p.small_max > 0 && ly.T <= p.small_max; }
int dense_variant(int64_t rows) { return gemm_bf16_pick_variant(static_cast<double>(rows)); }
// Latent projections of few tokens run on the skinny weight-streaming GEMM.
bool uses_skinny(const Layer& ly) { return ly.bf16 && ly.L > 0 && ly.T <= kSkinnyMaxRows; }

struct Carve {
  size_t off = 0;
  size_t take(size_t bytes) {
    const size_t at = off;
    off += (bytes + 255) & ~size_t(255);
    return at;
  }
};

struct WsLayout {
  size_t logits, rscratch, idx, w, counts, offsets, perm, inv, scratch, tcount, texpert, trow0, trows, scount,
      sexpert, srow0, srows, z, act, yassign, skinny, skinny_bytes, zq, zs, aq, as, total;
  int32_t tile_cap, small_cap;
};

WsLayout ws_layout(const Layer& ly) {
  WsLayout w{};
  Carve c;
  const size_t T = static_cast<size_t>(ly.T), E = static_cast<size_t>(ly.E), A = T * ly.k;
  const size_t es = elem_size(ly);
  const TilePlan plan = tile_plan(ly);
  w.tile_cap = static_cast<int32_t>((A + plan.bm - 1) / plan.bm + E);
  // at most ceil(small_max / bs) remainder tiles per expert, plus the M-tiles a thin last round
  // of the main list may move there
  w.small_cap = plan.small_max > 0 ? static_cast<int32_t>(E * ((plan.small_max + plan.bs - 1) / plan.bs) +
                                                          tail_small_tiles(plan))
                                   : 0;
  w.logits = c.take(static_cast<size_t>(router_splits(ly)) * T * E * 4);  // logit partial sums
  w.rscratch = c.take(router_scratch_bytes(ly));                            // router weight planes
  w.idx = c.take(A * 4);
  w.w = c.take(A * 4);
  w.counts = c.take(E * 4);
  w.offsets = c.take((E + 1) * 4);
  w.perm = c.take(A * 4);
  w.inv = c.take(A * 4);
  w.scratch = c.take(dispatch_scratch_bytes(ly));
  w.tcount = c.take(8);
  w.texpert = c.take(static_cast<size_t>(w.tile_cap) * 4);
  w.trow0 = c.take(static_cast<size_t>(w.tile_cap) * 4);
  w.trows = c.take(static_cast<size_t>(w.tile_cap) * 4);
  w.scount = c.take(8);
  w.sexpert = c.take(static_cast<size_t>(w.small_cap) * 4);
  w.srow0 = c.take(static_cast<size_t>(w.small_cap) * 4);
  w.srows = c.take(static_cast<size_t>(w.small_cap) * 4);
  w.z = c.take(ly.L ? T * static_cast<size_t>(ly.L) * es : 0);
  w.act = c.take(A * static_cast<size_t>(ly.h) * es);
  w.yassign = c.take(A * static_cast<size_t>(ly.K) * es);
  // split-K partials of the skinny latent projections (few tokens)
  w.skinny_bytes = uses_skinny(ly) ? std::max(gemm_skinny_partial_bytes(ly.T, ly.L, ly.d),
                                              gemm_skinny_partial_bytes(ly.T, ly.d, ly.L))
                                   : 0;
  w.skinny = c.take(w.skinny_bytes);
  // MXFP8 experts: E4M3 codes and E8M0 block scales of z (T, K) and of the activation (A, h)
  w.zq = c.take(ly.mx ? T * static_cast<size_t>(ly.K) : 0);
  w.zs = c.take(ly.mx ? T * static_cast<size_t>(ly.K) / 32 : 0);
  w.aq = c.take(ly.mx ? A * static_cast<size_t>(ly.h) : 0);
  w.as = c.take(ly.mx ? A * static_cast<size_t>(ly.h) / 32 : 0);
  w.total = c.off;
  return w;
}

template <typename P>
P* at(void* ws, size_t off) {
  return reinterpret_cast<P*>(static_cast<unsigned char*>(ws) + off);
}

TileList tiles_of(void* ws, const WsLayout& w) {
  TileList t;
  t.count = at<int32_t>(ws, w.tcount);
  t.expert = at<int32_t>(ws, w.texpert);
  t.row0 = at<int32_t>(ws, w.trow0);
  t.rows = at<int32_t>(ws, w.trows);
  t.cap = w.tile_cap;
  return t;
}

TileList small_tiles_of(void* ws, const WsLayout& w) {
  TileList t;
  t.count = at<int32_t>(ws, w.scount);
  t.expert = at<int32_t>(ws, w.sexpert);
  t.row0 = at<int32_t>(ws, w.srow0);
  t.rows = at<int32_t>(ws, w.srows);
  t.cap = w.small_cap;
  return t;
}

moe_status_t need(const void* p, const char* what) {
  if (!p) return fail(MOE_ERR_INVALID_ARG, std::string(what) + " is NULL");
  return MOE_OK;
}

moe_status_t check_weights(const moe_config_t* c, const moe_weights_t* w, bool router, bool latent,
                           bool experts) {
  moe_status_t st;
  if ((st = need(w, "weights")) != MOE_OK) return st;
  if (router) {
    if ((st = need(w->router_weight, "weights->router_weight")) != MOE_OK) return st;
    if (c->router_bias && (st = need(w->router_bias, "weights->router_bias")) != MOE_OK) return st;
  }
  if (latent && c->latent_dim) {
    if ((st = need(w->down_proj, "weights->down_proj")) != MOE_OK) return st;
    if ((st = need(w->up_proj, "weights->up_proj")) != MOE_OK) return st;
  }
  if (experts && c->expert_precision == MOE_PRECISION_MXFP8) {
    if ((st = need(w->w1_mx, "weights->w1_mx")) != MOE_OK) return st;
    if ((st = need(w->w1_mx_scale, "weights->w1_mx_scale")) != MOE_OK) return st;
    if ((st = need(w->w2_mx, "weights->w2_mx")) != MOE_OK) return st;
    if ((st = need(w->w2_mx_scale, "weights->w2_mx_scale")) != MOE_OK) return st;
  } else if (experts) {
    if ((st = need(w->w1, "weights->w1")) != MOE_OK) return st;
    if ((st = need(w->w2, "weights->w2")) != MOE_OK) return st;
  }
  return MOE_OK;
}

// ------------------------------------------------------------------ launch helpers

hipError_t run_dense(const Layer& ly, int64_t rows, const void* A, int64_t lda, const void* B, int64_t N,
                     int64_t Kd, void* C, float* partials, size_t partial_bytes, hipStream_t s) {
  GemmCall c{};
  c.A = A;
  c.lda = lda;
  c.B = B;
  c.ldb = Kd;
  c.C = C;
  c.ldc = N;
  c.N = N;
  c.Kd = Kd;
  c.dense_M = rows;
  c.a_rows = rows;
  c.c_rows = rows;
  c.rows_bound = rows;
  if (ly.bf16 && rows <= kSkinnyMaxRows && N % 64 == 0) return launch_gemm_skinny(c, partials, partial_bytes, s);
  if (ly.bf16) return launch_gemm_bf16(c, dense_variant(rows), s);
  return launch_gemm_f32(c, false, nullptr, s);
}

// Workspace of the MXFP8 experts: codes and block scales of z and of the activation.
struct MxBuffers {
  uint8_t* zq;
  uint8_t* zs;
  uint8_t* aq;
  uint8_t* as;
};

MxBuffers mx_buffers(void* ws, const WsLayout& L) {
  return MxBuffers{at<uint8_t>(ws, L.zq), at<uint8_t>(ws, L.zs), at<uint8_t>(ws, L.aq), at<uint8_t>(ws, L.as)};
}

// MXFP8 experts: quantise z, GEMM1 (+ SwiGLU, bf16 activation), quantise the activation, GEMM2.
hipError_t run_experts_mx(const Layer& ly, const void* z, const int32_t* perm, const TileList& tiles,
                          const moe_weights_t* w, void* act, void* yassign, const MxBuffers& mb, hipStream_t s) {
  const int64_t A = ly.T * ly.k;
  hipError_t e;
  if ((e = launch_mx_quantize(z, ly.T, ly.K, mb.zq, mb.zs, s)) != hipSuccess) return e;
  GemmCall g1{};
  g1.A = mb.zq;
  g1.lda = ly.K;
  g1.a_scale = mb.zs;
  g1.a_scale_ld = ly.K / 32;
  g1.gather = perm;
  g1.gather_div = ly.k;
  g1.B = w->w1_mx;
  g1.ldb = ly.K;
  g1.b_group_stride = 2 * ly.h * ly.K;
  g1.b_scale = w->w1_mx_scale;
  g1.b_scale_ld = ly.K / 32;
  g1.b_scale_group_stride = 2 * ly.h * (ly.K / 32);
  // the activation leaves GEMM1's epilogue already MX-quantised (codes + block scales); the
  // bf16 activation is never stored
  g1.C = act;
  g1.c_codes = mb.aq;
  g1.c_scales = mb.as;
  g1.ldc = ly.h;
  g1.N = ly.h;
  g1.Kd = ly.K;
  g1.swiglu_h = ly.h;
  g1.tiles = tiles;
  g1.a_rows = ly.T;
  g1.c_rows = A;
  g1.rows_bound = A;
  if ((e = launch_gemm_mx(g1, s)) != hipSuccess) return e;
  GemmCall g2{};
  g2.A = mb.aq;
  g2.lda = ly.h;
  g2.a_scale = mb.as;
  g2.a_scale_ld = ly.h / 32;
  g2.B = w->w2_mx;
  g2.ldb = ly.h;
  g2.b_group_stride = ly.K * ly.h;
  g2.b_scale = w->w2_mx_scale;
  g2.b_scale_ld = ly.h / 32;
  g2.b_scale_group_stride = ly.K * (ly.h / 32);
  g2.C = yassign;
  g2.ldc = ly.K;
  g2.scatter = perm;
  g2.N = ly.K;
  g2.Kd = ly.h;
  g2.tiles = tiles;
  g2.a_rows = A;
  g2.c_rows = A;
  g2.rows_bound = A;
  return launch_gemm_mx(g2, s);
}

// h_out: training forward, GEMM1 also stores the pre-activation H (A, 2h) in sorted order.
hipError_t run_experts(const Layer& ly, const void* z, const int32_t* perm, const TileList& tiles,
                       const TileList& small_tiles, const moe_weights_t* w, void* act, void* yassign,
                       const MxBuffers& mb, hipStream_t s, void* h_out = nullptr) {
  if (ly.mx) return h_out ? hipErrorInvalidValue : run_experts_mx(ly, z, perm, tiles, w, act, yassign, mb, s);
  const void* w1 = w->w1;
  const void* w2 = w->w2;
  const int64_t A = ly.T * ly.k;
  GemmCall g1{};
  g1.A = z;
  g1.lda = ly.K;
  g1.gather = perm;
  g1.gather_div = ly.k;
  g1.B = w1;
  g1.ldb = ly.K;
  g1.b_group_stride = 2 * ly.h * ly.K;
  g1.C = act;
  g1.ldc = ly.h;
  g1.N = ly.h;
  g1.Kd = ly.K;
  g1.swiglu_h = ly.h;
  g1.h_out = h_out;
  g1.tiles = tiles;
  g1.a_rows = ly.T;
  g1.c_rows = A;
  g1.rows_bound = A;
  GemmCall g2{};
  g2.A = act;
  g2.lda = ly.h;
  g2.B = w2;
  g2.ldb = ly.h;
  g2.b_group_stride = ly.K * ly.h;
  g2.C = yassign;
  g2.ldc = ly.K;
  g2.scatter = perm;
  g2.N = ly.K;
  g2.Kd = ly.h;
  g2.tiles = tiles;
  g2.a_rows = A;
  g2.c_rows = A;
  g2.rows_bound = A;
  hipError_t e;
  if (ly.bf16) {
    // main list on the large shape, remainders on the small shape (each GEMM's two launches
    // cover disjoint rows)
    const TilePlan plan = tile_plan(ly);
    const bool run_main = !main_list_empty(ly, plan);
    GemmCall g1s = g1, g2s = g2;
    g1s.tiles = small_tiles;
    g2s.tiles = small_tiles;
    if (run_main && (e = launch_gemm_bf16(g1, 0, s)) != hipSuccess) return e;
    if ((e = launch_gemm_bf16(g1s, 1, s)) != hipSuccess) return e;
    if (run_main && (e = launch_gemm_bf16(g2, 0, s)) != hipSuccess) return e;
    return launch_gemm_bf16(g2s, 1, s);
  }
  if ((e = launch_gemm_f32(g1, false, nullptr, s)) != hipSuccess) return e;
  return launch_gemm_f32(g2, false, nullptr, s);
}

// ------------------------------------------------------------------ backward of the experts

// Workspace of moe_experts_backward: the M-tile lists of the input-gradient GEMMs, dY and z in
// sorted order (the dY buffer later holds the per-assignment input gradients), dH, the two
// weight-gradient tile counters and the weight-gradient group order.
struct BwdLayout {
  size_t tcount, texpert, trow0, trows, scount, sexpert, srow0, srows, dy, zs, dh, counters, order, total;
  int32_t tile_cap, small_cap;
};
constexpr size_t kCounterBytes = 16;  // the two weight-gradient tile counters (cleared together)

BwdLayout bwd_layout(const Layer& ly) {
  BwdLayout b{};
  Carve c;
  const size_t E = static_cast<size_t>(ly.E), A = static_cast<size_t>(ly.T) * ly.k;
  const size_t es = elem_size(ly);
  const TilePlan plan = tile_plan(ly);
  b.tile_cap = static_cast<int32_t>((A + plan.bm - 1) / plan.bm + E);
  b.small_cap = plan.small_max > 0 ? static_cast<int32_t>(E * ((plan.small_max + plan.bs - 1) / plan.bs) +
                                                          tail_small_tiles(plan))
                                   : 0;
  b.tcount = c.take(8);
  b.texpert = c.take(static_cast<size_t>(b.tile_cap) * 4);
  b.trow0 = c.take(static_cast<size_t>(b.tile_cap) * 4);
  b.trows = c.take(static_cast<size_t>(b.tile_cap) * 4);
  b.scount = c.take(8);
  b.sexpert = c.take(static_cast<size_t>(b.small_cap) * 4);
  b.srow0 = c.take(static_cast<size_t>(b.small_cap) * 4);
  b.srows = c.take(static_cast<size_t>(b.small_cap) * 4);
  b.dy = c.take(A * static_cast<size_t>(ly.K) * es);
  b.zs = c.take(A * static_cast<size_t>(ly.K) * es);
  b.dh = c.take(A * 2 * static_cast<size_t>(ly.h) * es);
  b.counters = c.take(kCounterBytes);
  b.order = c.take(E * 4);
  b.total = c.off;
  return b;
}

struct BwdArgs {
  const void* z;
  const int32_t* offsets;
  const int32_t* perm;
  const void* h_saved;
  const void* act_saved;
  const void* dy_assign;
  void* dz;
  void* dw1;
  void* dw2;
};

// dY, z -> sorted order; d_act = dY w2[e] with the SwiGLU backward in its epilogue -> dH;
// dw2[e] = dY^T act; dz_assign = dH w1[e] scattered to assignment order; dw1[e] = dH^T z;
// dz = sum of each token's k rows of dz_assign.
hipError_t run_experts_backward(const Layer& ly, const moe_weights_t* w, const BwdArgs& a, void* ws,
                                const BwdLayout& L, hipStream_t s) {
  const int64_t A = ly.T * ly.k;
  const size_t es = elem_size(ly);
  TileList tiles{at<int32_t>(ws, L.tcount), at<int32_t>(ws, L.texpert), at<int32_t>(ws, L.trow0),
                 at<int32_t>(ws, L.trows), L.tile_cap};
  TileList small_tiles{at<int32_t>(ws, L.scount), at<int32_t>(ws, L.sexpert), at<int32_t>(ws, L.srow0),
                       at<int32_t>(ws, L.srows), L.small_cap};
  void* dy_sorted = at<void>(ws, L.dy);
  void* z_sorted = at<void>(ws, L.zs);
  void* dh = at<void>(ws, L.dh);
  void* dz_assign = dy_sorted;  // reused once the two dY products are enqueued
  const TilePlan plan = tile_plan(ly);
  hipError_t e;
  const int32_t* kept = a.offsets + ly.E;
  if ((e = launch_build_tiles(ly, a.offsets, tiles, small_tiles, plan, s)) != hipSuccess) return e;
  if ((e = launch_fill_zero(at<void>(ws, L.counters), kCounterBytes, s)) != hipSuccess) return e;
  int32_t* counters = at<int32_t>(ws, L.counters);
  int32_t* order = at<int32_t>(ws, L.order);
  if (ly.bf16 && (e = launch_expert_order(a.offsets, ly.E, order, s)) != hipSuccess) return e;
  if ((e = launch_gather_rows(a.dy_assign, A, a.perm, 1, kept, A, ly.K * es, dy_sorted, s)) != hipSuccess) return e;
  if ((e = launch_gather_rows(a.z, ly.T, a.perm, ly.k, kept, A, ly.K * es, z_sorted, s)) != hipSuccess) return e;

  // input gradient of the activation, then the SwiGLU backward: dH (A, 2h)
  GemmCall d2{};
  d2.A = dy_sorted;
  d2.lda = ly.K;
  d2.B = w->w2;              // (K, h) per expert: contraction K rows, h columns
  d2.ldb = ly.h;
  d2.b_group_stride = ly.K * ly.h;
  d2.trans = 2;
  d2.C = dh;
  d2.ldc = 2 * ly.h;
  d2.N = ly.h;
  d2.Kd = ly.K;
  d2.bwd_h = ly.h;
  d2.h_in = a.h_saved;
  d2.tiles = tiles;
  d2.a_rows = A;
  d2.c_rows = A;
  d2.rows_bound = A;
  // weight gradient of w2: dw2[e] (K, h) = sum_p dY[p]^T act[p]
  GemmCall g2{};
  g2.A = dy_sorted;
  g2.lda = ly.K;
  g2.B = a.act_saved;
  g2.ldb = ly.h;
  g2.trans = 3;
  g2.C = a.dw2;
  g2.ldc = ly.h;
  g2.N = ly.h;
  g2.dense_M = ly.K;
  g2.group_offsets = a.offsets;
  g2.groups = ly.E;
  g2.c_group_stride = ly.K * ly.h;
  g2.group_order = order;
  g2.tile_counter = counters;
  g2.a_rows = A;
  g2.c_rows = ly.K;
  g2.rows_bound = A;
  // input gradient of z_perm: dz_assign = dH w1[e], scattered to assignment order
  GemmCall d1{};
  d1.A = dh;
  d1.lda = 2 * ly.h;
  d1.B = w->w1;              // (2h, K) per expert: contraction 2h rows, K columns
  d1.ldb = ly.K;
  d1.b_group_stride = 2 * ly.h * ly.K;
  d1.trans = 2;
  d1.C = dz_assign;
  d1.ldc = ly.K;
  d1.scatter = a.perm;
  d1.N = ly.K;
  d1.Kd = 2 * ly.h;
  d1.tiles = tiles;
  d1.a_rows = A;
  d1.c_rows = A;
  d1.rows_bound = A;
  // weight gradient of w1: dw1[e] (2h, K) = sum_p dH[p]^T z[p]
  GemmCall g1{};
  g1.A = dh;
  g1.lda = 2 * ly.h;
  g1.B = z_sorted;
  g1.ldb = ly.K;
  g1.trans = 3;
  g1.C = a.dw1;
  g1.ldc = ly.K;
  g1.N = ly.K;
  g1.dense_M = 2 * ly.h;
  g1.group_offsets = a.offsets;
  g1.groups = ly.E;
  g1.c_group_stride = 2 * ly.h * ly.K;
  g1.group_order = order;
  g1.tile_counter = counters + 1;
  g1.a_rows = A;
  g1.c_rows = 2 * ly.h;
  g1.rows_bound = A;

  if (ly.bf16) {
    const bool run_main = !main_list_empty(ly, plan);
    GemmCall d2s = d2, d1s = d1;
    d2s.tiles = small_tiles;
    d1s.tiles = small_tiles;
    if (run_main && (e = launch_gemm_bf16_dgrad(d2, 0, s)) != hipSuccess) return e;
    if ((e = launch_gemm_bf16_dgrad(d2s, 1, s)) != hipSuccess) return e;
    if ((e = launch_gemm_bf16_wgrad(g2, s)) != hipSuccess) return e;
    if (run_main && (e = launch_gemm_bf16_dgrad(d1, 0, s)) != hipSuccess) return e;
    if ((e = launch_gemm_bf16_dgrad(d1s, 1, s)) != hipSuccess) return e;
    if ((e = launch_gemm_bf16_wgrad(g1, s)) != hipSuccess) return e;
  } else {
    // fp32 layers: per-element kernels, the expert of each row found from the offsets
    d2.group_offsets = a.offsets;
    d2.groups = ly.E;
    d1.group_offsets = a.offsets;
    d1.groups = ly.E;
    if ((e = launch_dgrad_f32(d2, s)) != hipSuccess) return e;
    if ((e = launch_wgrad_f32(g2, s)) != hipSuccess) return e;
    if ((e = launch_dgrad_f32(d1, s)) != hipSuccess) return e;
    if ((e = launch_wgrad_f32(g1, s)) != hipSuccess) return e;
  }
  if ((e = launch_zero_dropped(ly, a.offsets, a.perm, dz_assign, s)) != hipSuccess) return e;
  return launch_sum_copies(ly, dz_assign, a.dz, s);
}

// Size limits of the backward on top of check_tokens: 32-bit byte offsets of the bf16 GEMMs
// (dH is A x 2h), and the fp32 kernels' grid (rows and output rows of a group <= 65535).
moe_status_t check_backward(const moe_config_t* c, int64_t T) {
  if (c->expert_precision != MOE_PRECISION_BF16)
    return fail(MOE_ERR_UNSUPPORTED, "the experts backward runs in bf16 precision (MXFP8 training is not built)");
  const int64_t K = c->latent_dim ? c->latent_dim : c->d_model;
  const int64_t A = T * c->top_k;
  if (c->dtype == MOE_DTYPE_BF16) {
    if (A * 2 * c->hidden_size >= (int64_t(1) << 31))
      return fail(MOE_ERR_UNSUPPORTED, "a bf16 backward operand would exceed 4 GiB; split the batch");
  } else if (A > 65535 || K > 65535 || 2 * c->hidden_size > 65535) {
    return fail(MOE_ERR_UNSUPPORTED, "the fp32 experts backward serves up to 65535 assignments and widths");
  }
  return MOE_OK;
}

std::mutex g_dev_mu;
std::vector<int> g_cu_counts;

}  // namespace

int device_cu_count() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  std::lock_guard<std::mutex> lk(g_dev_mu);
  if (static_cast<int>(g_cu_counts.size()) <= dev) g_cu_counts.resize(dev + 1, 0);
  if (g_cu_counts[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    g_cu_counts[dev] = n;
  }
  return g_cu_counts[dev];
}

}  // namespace moe

using namespace moe;

extern "C" {

int moe_abi_version(void) { return MOE_ABI_VERSION; }

const char* moe_status_string(moe_status_t st) {
  switch (st) {
    case MOE_OK: return "ok";
    case MOE_ERR_INVALID_ARG: return "invalid argument";
    case MOE_ERR_UNSUPPORTED: return "unsupported configuration";
    case MOE_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
    case MOE_ERR_HIP: return "HIP runtime error";
  }
  return "unknown status";
}

const char* moe_last_error_message(void) { return g_last_error.c_str(); }

moe_status_t moe_config_default(moe_config_t* cfg) {
  if (!cfg) return fail(MOE_ERR_INVALID_ARG, "config is NULL");
  *cfg = moe_config_t{};
  cfg->struct_size = sizeof(moe_config_t);
  cfg->num_experts = 1;
  cfg->top_k = 1;
  cfg->hidden_size = 256;
  cfg->gating_function = MOE_GATING_SOFTMAX;
  cfg->activation = MOE_ACT_SWIGLU;
  cfg->dtype = MOE_DTYPE_BF16;
  cfg->up_proj_input_norm = 1;
  cfg->up_proj_input_norm_eps = 1e-5f;
  return ok();
}

moe_status_t moe_config_validate(const moe_config_t* cfg) { return validate_config(cfg); }

moe_status_t moe_num_params(const moe_config_t* c, int64_t* total, int64_t* active) {
  moe_status_t st = validate_config(c);
  if (st != MOE_OK) return st;
  const int64_t L = c->latent_dim ? c->latent_dim : c->d_model;
  const int64_t router = c->d_model * c->num_experts + (c->router_bias ? c->num_experts : 0);
  const int64_t up_factor = 2;  // swiglu
  const int64_t per_expert = (up_factor + 1) * L * c->hidden_size;
  const int64_t tot = router + per_expert * c->num_experts;
  if (total) *total = tot;
  if (active) *active = tot - 3 * L * c->hidden_size * c->num_experts + 3 * L * c->hidden_size * c->top_k;
  return ok();
}

moe_status_t moe_expert_capacity(const moe_config_t* c, int64_t T, int64_t* capacity) {
  moe_status_t st = validate_config(c);
  if (st != MOE_OK) return st;
  if ((st = check_tokens(c, T)) != MOE_OK) return st;
  if (!capacity) return fail(MOE_ERR_INVALID_ARG, "capacity is NULL");
  *capacity = make_layer(c, T).capacity;
  return ok();
}

moe_status_t moe_workspace_size(const moe_config_t* c, int64_t T, size_t* bytes) {
  moe_status_t st = validate_config(c);
  if (st != MOE_OK) return st;
  if ((st = check_tokens(c, T)) != MOE_OK) return st;
  if (!bytes) return fail(MOE_ERR_INVALID_ARG, "bytes is NULL");
  *bytes = ws_layout(make_layer(c, T)).total;
  return ok();
}

}  // extern "C"

namespace {

// Argument checks of a whole-layer call (before any HIP call).
moe_status_t check_forward(const moe_config_t* c, const moe_weights_t* w, int64_t T, const void* x, void* y) {
  moe_status_t st = validate_config(c);
  if (st != MOE_OK) return st;
  if ((st = check_tokens(c, T)) != MOE_OK) return st;
  if ((st = check_weights(c, w, true, true, true)) != MOE_OK) return st;
  if (T == 0) return MOE_OK;
  if ((st = need(x, "x")) != MOE_OK) return st;
  return need(y, "y");
}

// The launch sequence of the whole layer on a workspace of at least ws_layout(ly).total bytes.
moe_status_t enqueue_forward(const Layer& ly, const WsLayout& L, const moe_weights_t* w, const void* x, void* y,
                             moe_routing_t* routing, void* ws, hipStream_t s) {
  const int64_t T = ly.T;
  moe_routing_t r{};
  if (routing) r = *routing;
  float* parts = at<float>(ws, L.logits);
  const int nsplit = router_splits(ly);
  int32_t* idx = r.expert_indices ? r.expert_indices : at<int32_t>(ws, L.idx);
  float* wts = r.expert_weights ? r.expert_weights : at<float>(ws, L.w);
  int32_t* counts = r.batch_size_per_expert ? r.batch_size_per_expert : at<int32_t>(ws, L.counts);
  int32_t* offsets = r.expert_offsets ? r.expert_offsets : at<int32_t>(ws, L.offsets);
  int32_t* perm = r.permutation ? r.permutation : at<int32_t>(ws, L.perm);
  int32_t* inv = r.inverse_permutation ? r.inverse_permutation : at<int32_t>(ws, L.inv);
  const TileList tiles = tiles_of(ws, L);
  const TileList small_tiles = small_tiles_of(ws, L);

  MOE_TRY_HIP(launch_router_logits(ly, x, w->router_weight, parts, nsplit, at<void>(ws, L.rscratch), s), "router logits");
  MOE_TRY_HIP(launch_gate_topk(ly, parts, nsplit, false, w->score_bias, ly.router_bias ? w->router_bias : nullptr,
                               idx, wts, r.router_scores, r.router_logits, s),
              "gating/top-k");
  MOE_TRY_HIP(launch_dispatch(ly, idx, counts, offsets, perm, inv, at<void>(ws, L.scratch), tiles, small_tiles,
                              tile_plan(ly), s),
              "dispatch");
  const void* z = x;
  if (ly.L) {
    MOE_TRY_HIP(run_dense(ly, T, x, ly.d, w->down_proj, ly.L, ly.d, at<void>(ws, L.z), at<float>(ws, L.skinny),
                          L.skinny_bytes, s),
                "latent down");
    z = at<void>(ws, L.z);
  }
  MOE_TRY_HIP(run_experts(ly, z, perm, tiles, small_tiles, w, at<void>(ws, L.act), at<void>(ws, L.yassign),
                          mx_buffers(ws, L), s),
              "experts");
  MOE_TRY_HIP(launch_zero_dropped(ly, offsets, perm, at<void>(ws, L.yassign), s), "dropped rows");
  if (ly.L) {
    void* n = at<void>(ws, L.z);  // z is dead after the first expert GEMM
    MOE_TRY_HIP(launch_combine(ly, at<void>(ws, L.yassign), wts, w->up_proj_input_norm_weight, ly.up_norm, n, s),
                "combine");
    MOE_TRY_HIP(run_dense(ly, T, n, ly.L, w->up_proj, ly.d, ly.L, y, at<float>(ws, L.skinny), L.skinny_bytes, s),
                "latent up");
  } else {
    MOE_TRY_HIP(launch_combine(ly, at<void>(ws, L.yassign), wts, nullptr, false, y, s), "combine");
  }
  return ok();
}

// Address of `scratch` on each device, looked up once per device (with that device current)
// on the first allocation-free call there. A fixed table: the lookup allocates nothing.
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_addr[kMaxDevices] = {};

moe_status_t noalloc_scratch(void** out) {
  int dev = 0;
  MOE_TRY_HIP(hipGetDevice(&dev), "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return fail(MOE_ERR_UNSUPPORTED, "device ordinal beyond the scratch table");
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_addr[dev]) {
    void* p = nullptr;
    MOE_TRY_HIP(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)), "hipGetSymbolAddress(scratch)");
    if (!p) return fail(MOE_ERR_HIP, "hipGetSymbolAddress(scratch) gave no address");
    g_scratch_addr[dev] = p;
  }
  *out = g_scratch_addr[dev];
  return MOE_OK;
}

}  // namespace

extern "C" {

moe_status_t moe_forward(const moe_config_t* c, const moe_weights_t* w, int64_t T, const void* x, void* y,
                         moe_routing_t* routing, void* ws, size_t ws_bytes, void* stream) {
  moe_status_t st = check_forward(c, w, T, x, y);
  if (st != MOE_OK) return st;
  if (T == 0) return ok();
  if ((st = need(ws, "workspace")) != MOE_OK) return st;
  const Layer ly = make_layer(c, T);
  const WsLayout L = ws_layout(ly);
  if (ws_bytes < L.total)
    return fail(MOE_ERR_WORKSPACE_TOO_SMALL, "workspace holds " + std::to_string(ws_bytes) + " bytes, needs " +
                                                 std::to_string(L.total));
  return enqueue_forward(ly, L, w, x, y, routing, ws, static_cast<hipStream_t>(stream));
}

moe_status_t moe_forward_noalloc(const moe_config_t* c, const moe_weights_t* w, int64_t T, const void* x, void* y,
                                 moe_routing_t* routing, void* stream) {
  moe_status_t st = check_forward(c, w, T, x, y);
  if (st != MOE_OK) return st;
  if (T == 0) return ok();
  const Layer ly = make_layer(c, T);
  const WsLayout L = ws_layout(ly);
  if (L.total > MOE_NOALLOC_SCRATCH_BYTES)
    return fail(MOE_ERR_WORKSPACE_TOO_SMALL,
                "this layer needs " + std::to_string(L.total) + " bytes of workspace for " + std::to_string(T) +
                    " tokens; the allocation-free forward holds " + std::to_string(MOE_NOALLOC_SCRATCH_BYTES) +
                    ": use moe_forward with a caller workspace, or fewer tokens per call");
  void* ws = nullptr;
  if ((st = noalloc_scratch(&ws)) != MOE_OK) return st;
  return enqueue_forward(ly, L, w, x, y, routing, ws, static_cast<hipStream_t>(stream));
}

moe_status_t moe_router_forward(const moe_config_t* c, const moe_weights_t* w, int64_t T, const void* x,
                                moe_routing_t* routing, void* ws, size_t ws_bytes, void* stream) {
  moe_status_t st = validate_config(c);
  if (st != MOE_OK) return st;
  if ((st = check_tokens(c, T)) != MOE_OK) return st;
  if ((st = check_weights(c, w, true, false, false)) != MOE_OK) return st;
  if ((st = need(routing, "routing")) != MOE_OK) return st;
  if ((st = need(routing->expert_indices, "routing->expert_indices")) != MOE_OK) return st;
  if ((st = need(routing->expert_weights, "routing->expert_weights")) != MOE_OK) return st;
  if (T == 0) return ok();
  if ((st = need(x, "x")) != MOE_OK) return st;
  if ((st = need(ws, "workspace")) != MOE_OK) return st;
  const Layer ly = make_layer(c, T);
  const WsLayout L = ws_layout(ly);
  const int nsplit = router_splits(ly);
  if (ws_bytes < L.logits + static_cast<size_t>(nsplit) * T * ly.E * 4 ||
      ws_bytes < L.rscratch + router_scratch_bytes(ly))
    return fail(MOE_ERR_WORKSPACE_TOO_SMALL, "workspace too small for the router partial sums / weight planes");
  float* parts = at<float>(ws, L.logits);
  hipStream_t s = static_cast<hipStream_t>(stream);
  MOE_TRY_HIP(launch_router_logits(ly, x, w->router_weight, parts, nsplit, at<void>(ws, L.rscratch), s), "router logits");
  MOE_TRY_HIP(launch_gate_topk(ly, parts, nsplit, false, w->score_bias, ly.router_bias ? w->router_bias : nullptr,
                               routing->expert_indices, routing->expert_weights, routing->router_scores,
                               routing->router_logits, s),
              "gating/top-k");
  return ok();
}

moe_status_t moe_route_from_scores(const moe_config_t* c, int64_t T, const float* sel_input,
                                   const float* score_bias, int32_t* expert_indices, float* expert_weights,
                                   void* stream) {
  moe_status_t st = validate_config(c);
  if (st != MOE_OK) return st;
  if ((st = check_tokens(c, T)) != MOE_OK) return st;
  if ((st = need(expert_indices, "expert_indices")) != MOE_OK) return st;
  if ((st = need(expert_weights, "expert_weights")) != MOE_OK) return st;
  if (T == 0) return ok();
  if ((st = need(sel_input, "sel_input")) != MOE_OK) return st;
  const Layer ly = make_layer(c, T);
  MOE_TRY_HIP(launch_gate_topk(ly, sel_input, 1, true, score_bias, nullptr, expert_indices, expert_weights,
                               nullptr, nullptr, static_cast<hipStream_t>(stream)),
              "route from scores");
  return ok();
}

moe_status_t moe_permute(const moe_config_t* c, int64_t T, const int32_t* idx, int32_t* counts, int32_t* offsets,
                         int32_t* perm, int32_t* inv, void* ws, size_t ws_bytes, void* stream) {
  moe_status_t st = validate_config(c);
  if (st != MOE_OK) return st;
  if ((st = check_tokens(c, T)) != MOE_OK) return st;
  if ((st = need(counts, "batch_size_per_expert")) != MOE_OK) return st;
  if ((st = need(offsets, "expert_offsets")) != MOE_OK) return st;
  const Layer ly = make_layer(c, T);
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (T == 0) {  // no assignments: permutation buffers are empty (may be NULL)
    MOE_TRY_HIP(launch_zero_counts_offsets(counts, offsets, ly.E, s), "zero counts and offsets");
    return ok();
  }
  if ((st = need(perm, "permutation")) != MOE_OK) return st;
  if ((st = need(inv, "inverse_permutation")) != MOE_OK) return st;
  if ((st = need(ws, "workspace")) != MOE_OK) return st;
  const WsLayout L = ws_layout(ly);
  if (ws_bytes < L.total) return fail(MOE_ERR_WORKSPACE_TOO_SMALL, "workspace too small");
  if ((st = need(idx, "expert_indices")) != MOE_OK) return st;
  MOE_TRY_HIP(launch_dispatch(ly, idx, counts, offsets, perm, inv, at<void>(ws, L.scratch), tiles_of(ws, L),
                              small_tiles_of(ws, L), tile_plan(ly), s),
              "dispatch");
  return ok();
}

moe_status_t moe_latent_down(const moe_config_t* c, const moe_weights_t* w, int64_t T, const void* x, void* z,
                             void* ws, size_t ws_bytes, void* stream) {
  moe_status_t st = validate_config(c);
  if (st != MOE_OK) return st;
  if (!c->latent_dim) return fail(MOE_ERR_UNSUPPORTED, "latent_down needs latent_dim > 0");
  if ((st = check_tokens(c, T)) != MOE_OK) return st;
  if ((st = need(w, "weights")) != MOE_OK) return st;
  if ((st = need(w->down_proj, "weights->down_proj")) != MOE_OK) return st;
  if (T == 0) return ok();
  if ((st = need(x, "x")) != MOE_OK) return st;
  if ((st = need(z, "z")) != MOE_OK) return st;
  const Layer ly = make_layer(c, T);
  const WsLayout L = ws_layout(ly);
  if (ws && ws_bytes < L.total) return fail(MOE_ERR_WORKSPACE_TOO_SMALL, "workspace too small");
  float* parts = ws ? at<float>(ws, L.skinny) : nullptr;
  MOE_TRY_HIP(run_dense(ly, T, x, ly.d, w->down_proj, ly.L, ly.d, z, parts, ws ? L.skinny_bytes : 0,
                        static_cast<hipStream_t>(stream)),
              "latent down");
  return ok();
}

moe_status_t moe_experts_forward(const moe_config_t* c, const moe_weights_t* w, int64_t T, const void* z,
                                 const int32_t* offsets, const int32_t* perm, void* y_assign, void* ws,
                                 size_t ws_bytes, void* stream) {
  moe_status_t st = validate_config(c);
  if (st != MOE_OK) return st;
  if ((st = check_tokens(c, T)) != MOE_OK) return st;
  if ((st = check_weights(c, w, false, false, true)) != MOE_OK) return st;
  if (T == 0) return ok();
  if ((st = need(z, "z")) != MOE_OK) return st;
  if ((st = need(offsets, "expert_offsets")) != MOE_OK) return st;
  if ((st = need(perm, "permutation")) != MOE_OK) return st;
  if ((st = need(y_assign, "y_assign")) != MOE_OK) return st;
  if ((st = need(ws, "workspace")) != MOE_OK) return st;
  const Layer ly = make_layer(c, T);
  const WsLayout L = ws_layout(ly);
  if (ws_bytes < L.total) return fail(MOE_ERR_WORKSPACE_TOO_SMALL, "workspace too small");
  hipStream_t s = static_cast<hipStream_t>(stream);
  const TileList tiles = tiles_of(ws, L);
  const TileList small_tiles = small_tiles_of(ws, L);
  MOE_TRY_HIP(launch_build_tiles(ly, offsets, tiles, small_tiles, tile_plan(ly), s), "tile list");
  MOE_TRY_HIP(run_experts(ly, z, perm, tiles, small_tiles, w, at<void>(ws, L.act), y_assign, mx_buffers(ws, L), s),
              "experts");
  MOE_TRY_HIP(launch_zero_dropped(ly, offsets, perm, y_assign, s), "dropped rows");
  return ok();
}

moe_status_t moe_experts_forward_train(const moe_config_t* c, const moe_weights_t* w, int64_t T, const void* z,
                                       const int32_t* offsets, const int32_t* perm, void* y_assign, void* h_saved,
                                       void* act_saved, void* ws, size_t ws_bytes, void* stream) {
  moe_status_t st = validate_config(c);
  if (st != MOE_OK) return st;
  if ((st = check_tokens(c, T)) != MOE_OK) return st;
  if ((st = check_backward(c, T)) != MOE_OK) return st;
  if ((st = check_weights(c, w, false, false, true)) != MOE_OK) return st;
  if (T == 0) return ok();
  if ((st = need(z, "z")) != MOE_OK) return st;
  if ((st = need(offsets, "expert_offsets")) != MOE_OK) return st;
  if ((st = need(perm, "permutation")) != MOE_OK) return st;
  if ((st = need(y_assign, "y_assign")) != MOE_OK) return st;
  if ((st = need(h_saved, "h_saved")) != MOE_OK) return st;
  if ((st = need(act_saved, "act_saved")) != MOE_OK) return st;
  if ((st = need(ws, "workspace")) != MOE_OK) return st;
  const Layer ly = make_layer(c, T);
  const WsLayout L = ws_layout(ly);
  if (ws_bytes < L.total) return fail(MOE_ERR_WORKSPACE_TOO_SMALL, "workspace too small");
  hipStream_t s = static_cast<hipStream_t>(stream);
  const TileList tiles = tiles_of(ws, L);
  const TileList small_tiles = small_tiles_of(ws, L);
  MOE_TRY_HIP(launch_build_tiles(ly, offsets, tiles, small_tiles, tile_plan(ly), s), "tile list");
  MOE_TRY_HIP(run_experts(ly, z, perm, tiles, small_tiles, w, act_saved, y_assign, mx_buffers(ws, L), s, h_saved),
              "experts");
  MOE_TRY_HIP(launch_zero_dropped(ly, offsets, perm, y_assign, s), "dropped rows");
  return ok();
}

moe_status_t moe_experts_backward_workspace_size(const moe_config_t* c, int64_t T, size_t* bytes) {
  moe_status_t st = validate_config(c);
  if (st != MOE_OK) return st;
  if ((st = check_tokens(c, T)) != MOE_OK) return st;
  if ((st = check_backward(c, T)) != MOE_OK) return st;
  if (!bytes) return fail(MOE_ERR_INVALID_ARG, "bytes is NULL");
  *bytes = bwd_layout(make_layer(c, T)).total;
  return ok();
}

moe_status_t moe_experts_backward(const moe_config_t* c, const moe_weights_t* w, int64_t T, const void* z,
                                  const int32_t* offsets, const int32_t* perm, const void* h_saved,
                                  const void* act_saved, const void* dy_assign, void* dz, void* dw1, void* dw2,
                                  void* ws, size_t ws_bytes, void* stream) {
  moe_status_t st = validate_config(c);
  if (st != MOE_OK) return st;
  if ((st = check_tokens(c, T)) != MOE_OK) return st;
  if ((st = check_backward(c, T)) != MOE_OK) return st;
  if ((st = check_weights(c, w, false, false, true)) != MOE_OK) return st;
  if ((st = need(dw1, "dw1")) != MOE_OK) return st;
  if ((st = need(dw2, "dw2")) != MOE_OK) return st;
  if (T > 0) {
    if ((st = need(offsets, "expert_offsets")) != MOE_OK) return st;
    if ((st = need(ws, "workspace")) != MOE_OK) return st;
    if ((st = need(z, "z")) != MOE_OK) return st;
    if ((st = need(perm, "permutation")) != MOE_OK) return st;
    if ((st = need(h_saved, "h_saved")) != MOE_OK) return st;
    if ((st = need(act_saved, "act_saved")) != MOE_OK) return st;
    if ((st = need(dy_assign, "dy_assign")) != MOE_OK) return st;
    if ((st = need(dz, "dz")) != MOE_OK) return st;
  }
  const Layer ly = make_layer(c, T);
  const BwdLayout L = bwd_layout(ly);
  if (T > 0 && ws_bytes < L.total)
    return fail(MOE_ERR_WORKSPACE_TOO_SMALL, "workspace holds " + std::to_string(ws_bytes) + " bytes, needs " +
                                                 std::to_string(L.total));
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (T == 0) {
    // no rows: the weight gradients are zero
    MOE_TRY_HIP(launch_fill_zero(dw1, static_cast<size_t>(ly.E) * 2 * ly.h * ly.K * elem_size(ly), s), "dw1");
    MOE_TRY_HIP(launch_fill_zero(dw2, static_cast<size_t>(ly.E) * ly.K * ly.h * elem_size(ly), s), "dw2");
    return ok();
  }
  const BwdArgs a{z, offsets, perm, h_saved, act_saved, dy_assign, dz, dw1, dw2};
  MOE_TRY_HIP(run_experts_backward(ly, w, a, ws, L, s), "experts backward");
  return ok();
}

moe_status_t moe_combine_backward(const moe_config_t* c, int64_t T, const void* y_assign,
                                  const float* expert_weights, const void* d_out, void* dy_assign,
                                  float* d_expert_weights, void* stream) {
  moe_status_t st = validate_config(c);
  if (st != MOE_OK) return st;
  if ((st = check_tokens(c, T)) != MOE_OK) return st;
  if (c->latent_dim && c->up_proj_input_norm)
    return fail(MOE_ERR_UNSUPPORTED, "the combine backward through the latent RMSNorm is not built");
  if (T == 0) return ok();
  if ((st = need(y_assign, "y_assign")) != MOE_OK) return st;
  if ((st = need(expert_weights, "expert_weights")) != MOE_OK) return st;
  if ((st = need(d_out, "d_out")) != MOE_OK) return st;
  if ((st = need(dy_assign, "dy_assign")) != MOE_OK) return st;
  const Layer ly = make_layer(c, T);
  MOE_TRY_HIP(launch_combine_backward(ly, y_assign, expert_weights, d_out, dy_assign, d_expert_weights,
                                      static_cast<hipStream_t>(stream)),
              "combine backward");
  return ok();
}

moe_status_t moe_combine(const moe_config_t* c, const moe_weights_t* w, int64_t T, const void* y_assign,
                         const float* expert_weights, void* out, void* stream) {
  moe_status_t st = validate_config(c);
  if (st != MOE_OK) return st;
  if ((st = check_tokens(c, T)) != MOE_OK) return st;
  if (T == 0) return ok();
  if ((st = need(y_assign, "y_assign")) != MOE_OK) return st;
  if ((st = need(expert_weights, "expert_weights")) != MOE_OK) return st;
  if ((st = need(out, "out")) != MOE_OK) return st;
  const Layer ly = make_layer(c, T);
  const bool norm = ly.L && ly.up_norm;
  const float* g = (norm && w) ? w->up_proj_input_norm_weight : nullptr;
  MOE_TRY_HIP(launch_combine(ly, y_assign, expert_weights, g, norm, out, static_cast<hipStream_t>(stream)),
              "combine");
  return ok();
}

moe_status_t moe_latent_up(const moe_config_t* c, const moe_weights_t* w, int64_t T, const void* n, void* y,
                           void* ws, size_t ws_bytes, void* stream) {
  moe_status_t st = validate_config(c);
  if (st != MOE_OK) return st;
  if (!c->latent_dim) return fail(MOE_ERR_UNSUPPORTED, "latent_up needs latent_dim > 0");
  if ((st = check_tokens(c, T)) != MOE_OK) return st;
  if ((st = need(w, "weights")) != MOE_OK) return st;
  if ((st = need(w->up_proj, "weights->up_proj")) != MOE_OK) return st;
  if (T == 0) return ok();
  if ((st = need(n, "n")) != MOE_OK) return st;
  if ((st = need(y, "y")) != MOE_OK) return st;
  const Layer ly = make_layer(c, T);
  const WsLayout L = ws_layout(ly);
  if (ws && ws_bytes < L.total) return fail(MOE_ERR_WORKSPACE_TOO_SMALL, "workspace too small");
  float* parts = ws ? at<float>(ws, L.skinny) : nullptr;
  MOE_TRY_HIP(run_dense(ly, T, n, ly.L, w->up_proj, ly.d, ly.L, y, parts, ws ? L.skinny_bytes : 0,
                        static_cast<hipStream_t>(stream)),
              "latent up");
  return ok();
}

}  // extern "C"

// ------------------------------------------------------------------------ MXFP8

extern "C" moe_status_t moe_mx_quantize(int64_t rows, int64_t cols, const void* x, uint8_t* codes,
                                        uint8_t* scales, void* stream) {
  if (rows < 0) return fail(MOE_ERR_INVALID_ARG, "rows must be >= 0");
  if (cols <= 0 || cols % 32 != 0) return fail(MOE_ERR_INVALID_ARG, "cols must be a positive multiple of 32");
  if (rows == 0) return ok();
  moe_status_t st;
  if ((st = need(x, "x")) != MOE_OK) return st;
  if ((st = need(codes, "codes")) != MOE_OK) return st;
  if ((st = need(scales, "scales")) != MOE_OK) return st;
  MOE_TRY_HIP(launch_mx_quantize(x, rows, cols, codes, scales, static_cast<hipStream_t>(stream)), "mx quantize");
  return ok();
}

// ------------------------------------------------------------------------ calibration

namespace moe {
// csrc/calibrate.hip: the matrix-core loop (one float per wavefront to `out`, mfma_loop_waves()
// of them; mfma_loop_flops(iters) dense flops per launch) and a plain 16-byte-vector copy.
int64_t mfma_loop_waves();
double mfma_loop_flops(int64_t iters, bool mx);
hipError_t launch_mfma_loop(float* out, int64_t iters, bool mx, hipStream_t s);
hipError_t launch_copy(const void* src, void* dst, int64_t bytes, hipStream_t s);
}  // namespace moe

namespace {
moe_status_t calibrate_mfma(int64_t iters, float* out, int64_t* num_waves, double* flops, bool mx, void* stream) {
  if (iters < 1) return fail(MOE_ERR_INVALID_ARG, "iters must be >= 1");
  moe_status_t st;
  if ((st = need(num_waves, "num_waves")) != MOE_OK) return st;
  if ((st = need(flops, "flops")) != MOE_OK) return st;
  *num_waves = mfma_loop_waves();
  *flops = mfma_loop_flops(iters, mx);
  if (!out) return ok();
  MOE_TRY_HIP(launch_mfma_loop(out, iters, mx, static_cast<hipStream_t>(stream)), "mfma loop");
  return ok();
}
}  // namespace

extern "C" moe_status_t moe_calibrate_mfma_bf16(int64_t iters, float* out, int64_t* num_waves, double* flops,
                                                void* stream) {
  return calibrate_mfma(iters, out, num_waves, flops, false, stream);
}

extern "C" moe_status_t moe_calibrate_mfma_mxfp8(int64_t iters, float* out, int64_t* num_waves, double* flops,
                                                 void* stream) {
  return calibrate_mfma(iters, out, num_waves, flops, true, stream);
}

extern "C" moe_status_t moe_calibrate_copy(const void* src, void* dst, int64_t bytes, void* stream) {
  if (bytes <= 0 || bytes % 16 != 0) return fail(MOE_ERR_INVALID_ARG, "bytes must be a positive multiple of 16");
  moe_status_t st;
  if ((st = need(src, "src")) != MOE_OK) return st;
  if ((st = need(dst, "dst")) != MOE_OK) return st;
  MOE_TRY_HIP(launch_copy(src, dst, bytes, static_cast<hipStream_t>(stream)), "copy");
  return ok();
}

// ------------------------------------------------------------------------ balancing state

namespace {
moe_status_t check_experts(int32_t E) {
  if (E < 1 || E > MOE_MAX_EXPERTS)
    return fail(MOE_ERR_INVALID_ARG, "num_experts must be in 1.." + std::to_string(MOE_MAX_EXPERTS));
  return MOE_OK;
}
}  // namespace

extern "C" {

moe_status_t moe_accumulate_expert_counts(int32_t E, const int32_t* counts, int64_t* acc, void* stream) {
  moe_status_t st;
  if ((st = check_experts(E)) != MOE_OK) return st;
  if ((st = need(counts, "batch_size_per_expert")) != MOE_OK) return st;
  if ((st = need(acc, "accumulator")) != MOE_OK) return st;
  MOE_TRY_HIP(launch_accumulate_counts(E, counts, acc, static_cast<hipStream_t>(stream)), "accumulate counts");
  return ok();
}

moe_status_t moe_load_imbalance(int32_t E, const int64_t* counts, double* imbalance, void* stream) {
  moe_status_t st;
  if ((st = check_experts(E)) != MOE_OK) return st;
  if ((st = need(counts, "counts")) != MOE_OK) return st;
  if ((st = need(imbalance, "imbalance")) != MOE_OK) return st;
  MOE_TRY_HIP(launch_load_imbalance(E, counts, imbalance, static_cast<hipStream_t>(stream)), "load imbalance");
  return ok();
}

moe_status_t moe_score_bias_update(int32_t E, float gamma, int64_t* acc, float* score_bias, double* imbalance,
                                   void* stream) {
  moe_status_t st;
  if ((st = check_experts(E)) != MOE_OK) return st;
  if (!finite(gamma)) return fail(MOE_ERR_INVALID_ARG, "bias_gamma must be finite");
  if ((st = need(acc, "accumulator")) != MOE_OK) return st;
  if ((st = need(score_bias, "score_bias")) != MOE_OK) return st;
  MOE_TRY_HIP(launch_score_bias_update(E, gamma, acc, score_bias, imbalance, static_cast<hipStream_t>(stream)),
              "score_bias update");
  return ok();
}

}  // extern "C"
