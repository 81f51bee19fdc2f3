// Internal declarations shared by the HIP translation units of the MoE layer library.
// gfx950 (CDNA4) only: 64-wide wavefronts, MFMA matrix cores, 160 KB LDS per CU, 8 XCDs.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moe_mi355x.h"

namespace moe {

constexpr int kWave = 64;

// ---------------------------------------------------------------- bf16 (bit patterns)

__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// Round-to-nearest-even float -> bf16 (the hardware conversion on gfx950).
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}

// Element access for the two storage dtypes.
template <typename T> struct Elem;
template <> struct Elem<float> {
  using storage = float;
  __device__ static float load(const float* p) { return *p; }
  __device__ static void store(float* p, float v) { *p = v; }
};
template <> struct Elem<uint16_t> {
  using storage = uint16_t;
  __device__ static float load(const uint16_t* p) { return bf16_bits_to_f32(*p); }
  __device__ static void store(uint16_t* p, float v) { *p = f32_to_bf16_bits(v); }
};

// ---------------------------------------------------------------- MXFP8 (OCP microscaling)

// E8M0 scale code of a 32-element block with absolute maximum amax: floor(log2 amax) - 8 + 127,
// clamped to [0, 254]; 0 for an all-zero block.
__device__ __forceinline__ int mx_scale_code(float amax) {
  if (!(amax > 0.f)) return 0;
  int ex;
  frexpf(amax, &ex);  // amax = m * 2^ex with m in [0.5, 1): floor(log2 amax) = ex - 1
  return min(max(ex - 1 - 8 + 127, 0), 254);
}

// Four values, already divided by the block scale, as E4M3 codes in one word (first value in
// byte 0). v_cvt_pk_fp8_f32 rounds to nearest-even and returns NaN above 464, so the values are
// clamped to the largest code, 448, first: the saturating rounding.
__device__ __forceinline__ uint32_t pack4_e4m3(float a, float b, float c, float d) {
  const auto cl = [](float v) { return fminf(fmaxf(v, -448.f), 448.f); };
  uint32_t r = static_cast<uint32_t>(__builtin_amdgcn_cvt_pk_fp8_f32(cl(a), cl(b), 0, false));
  r = static_cast<uint32_t>(__builtin_amdgcn_cvt_pk_fp8_f32(cl(c), cl(d), static_cast<int>(r), true));
  return r;
}

// ---------------------------------------------------------------- wave reductions

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

// Wave-uniform reductions through DPP: four lane-exchange steps reduce each 16-lane row
// (quad_perm [1,0,3,2], quad_perm [2,3,0,1], row_half_mirror, row_mirror: afterwards every lane
// of a row holds the row's result), then the four row results are read into scalar registers
// and combined in a fixed order ((r0 op r1) op (r2 op r3)). No LDS round trips; the result is
// the same on every lane and, for sums, the order is fixed, so it is deterministic. Every lane
// of the wavefront must be active.
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
  return static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), CTRL, 0xF, 0xF, false));
}

template <typename Op>
__device__ __forceinline__ uint32_t wave_reduce_u32(uint32_t v, Op op) {
  v = op(v, dpp_u32<0xB1>(v));
  v = op(v, dpp_u32<0x4E>(v));
  v = op(v, dpp_u32<0x141>(v));
  v = op(v, dpp_u32<0x140>(v));
  const uint32_t r0 = __builtin_amdgcn_readlane(v, 0), r1 = __builtin_amdgcn_readlane(v, 16);
  const uint32_t r2 = __builtin_amdgcn_readlane(v, 32), r3 = __builtin_amdgcn_readlane(v, 48);
  return op(op(r0, r1), op(r2, r3));
}

__device__ __forceinline__ uint32_t wave_max_u32_dpp(uint32_t v) {
  return wave_reduce_u32(v, [](uint32_t a, uint32_t b) { return a > b ? a : b; });
}
__device__ __forceinline__ int32_t wave_min_i32_dpp(int32_t v) {
  return static_cast<int32_t>(wave_reduce_u32(static_cast<uint32_t>(v), [](uint32_t a, uint32_t b) {
    return static_cast<int32_t>(a) < static_cast<int32_t>(b) ? a : b;
  }));
}
__device__ __forceinline__ float wave_max_f32_dpp(float v) {
  return __uint_as_float(wave_reduce_u32(__float_as_uint(v), [](uint32_t a, uint32_t b) {
    return __float_as_uint(fmaxf(__uint_as_float(a), __uint_as_float(b)));
  }));
}
__device__ __forceinline__ float wave_sum_f32_dpp(float v) {
  return __uint_as_float(wave_reduce_u32(__float_as_uint(v), [](uint32_t a, uint32_t b) {
    return __float_as_uint(__uint_as_float(a) + __uint_as_float(b));
  }));
}

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    uint32_t lo = __shfl_xor(static_cast<uint32_t>(v), o, kWave);
    uint32_t hi = __shfl_xor(static_cast<uint32_t>(v >> 32), o, kWave);
    uint64_t w = (static_cast<uint64_t>(hi) << 32) | lo;
    v = w > v ? w : v;
  }
  return v;
}

// ---------------------------------------------------------------- layer description

// Resolved, validated layer description used by the launchers (host side).
struct Layer {
  int64_t T;      // tokens
  int64_t d;      // d_model
  int32_t E;      // experts
  int32_t k;      // top_k
  int64_t h;      // hidden
  int64_t L;      // latent (0 = none)
  int64_t K;      // expert input width (L or d)
  int gating;     // moe_gating_t
  bool bf16;      // storage dtype
  float sig_eps;
  float norm_p;
  bool restore_scale;
  float ews;
  int32_t orig_k;
  bool router_bias;
  bool up_norm;
  float norm_eps;
  int64_t capacity;  // expert capacity (token dropping); 0 = dropless
  bool mx;           // MXFP8 expert matmuls
};

// Per-expert M-tile list consumed by the grouped GEMMs (device memory, built on the device).
struct TileList {
  int32_t* count;   // [2]   number of M-tiles; [1]: spread tile order (see kSpreadMinMTiles)
  int32_t* expert;  // [cap] expert of each M-tile
  int32_t* row0;    // [cap] first sorted row of each M-tile
  int32_t* rows;    // [cap] valid rows (<= BM)
  int32_t cap;
};

// A main tile list whose M-tiles mostly belong to experts of at least this many M-tiles is
// marked (count[1] = 1) for the GEMMs' spread tile order across the XCDs; remainder lists
// never are.
constexpr int kSpreadMinMTiles = 16;

// How an expert's rows are cut into M-tiles: full tiles of bm rows; the remainder r = rows % bm
// goes to one more tile of that list when r > small_max, else to ceil(r / bs) tiles of bs rows
// in a second list, run by the smaller tile shape (small_max = 0: one list only). With the
// large shape's 256-row tiles, an expert of 1 + 4 * 256 rows then adds one 64-row tile to the
// small list instead of a 256-row tile that is almost all padding.
// Thin last round: the large tiles' persistent grid runs tail_round workgroups at a time, and
// each main-list M-tile is tail_ntn tiles of the up/gate GEMM. When the main list would leave
// a last round of at most tail_round / 8 tiles (after at least one whole round), the fewest
// whole M-tiles that remove it go to the remainder list instead, all from one expert: one that
// already has remainder tiles (its weights are streamed by the small tiles anyway) if any
// expert has enough M-tiles, else the lowest-numbered such expert. Outputs do not change: both
// tile shapes accumulate every output element over k in the same order. tail_round = 0 (or no
// remainder list) disables the move.
struct TilePlan {
  int bm;         // rows per tile of the main list
  int bs;         // rows per tile of the remainder list
  int small_max;  // largest remainder sent to the remainder list (0 = none)
  int tail_round = 0;  // workgroups per round of the main-list GEMMs (0: no tail move)
  int tail_ntn = 0;    // tiles per main-list M-tile of the up/gate GEMM
};
// Largest tail_round the dispatch honours, and the remainder-list room it then needs beyond
// ceil(small_max / bs) tiles per expert: at most kTailRoundMax / 8 M-tiles move.
constexpr int kTailRoundMax = 1024;
inline int tail_small_tiles(const TilePlan& p) {
  return p.small_max > 0 ? (kTailRoundMax / 8 + 1) * ((p.bm + p.bs - 1) / p.bs) : 0;
}

// Grid-wide properties cached per device.
int device_cu_count();

// ---------------------------------------------------------------- launchers (host)
// Every launcher enqueues on `s` and returns hipSuccess or the launch error.

// Router logits as nsplit partial-sum planes (nsplit, T, E) f32 of x (T,d) * Wr^T; the gate
// kernel adds the planes (fixed order) and the router bias. x is f32 or bf16 bits.
// Router logits. Large layers (router_uses_planes) split the fp32 weights into three bf16
// planes in `scratch` (router_scratch_bytes) and run one dense MFMA GEMM into a single logits
// plane; otherwise a split-K kernel writes router_splits(ly) partial planes, summed in a fixed
// order by the gate kernel.
bool router_uses_planes(const Layer& ly);
size_t router_scratch_bytes(const Layer& ly);
int router_splits(const Layer& ly);
hipError_t launch_router_logits(const Layer& ly, const void* x, const float* Wr, float* partials,
                                int nsplit, void* scratch, hipStream_t s);

// Gating + top-k + weights from logit partials (from_scores = false) or from the gating output
// (from_scores = true: scores for softmax/sigmoid, logits for topk_softmax; nsplit ignored).
// logits_out / scores_out (T, E) are optional diagnostics.
hipError_t launch_gate_topk(const Layer& ly, const float* input, int nsplit, bool from_scores,
                            const float* score_bias, const float* router_bias, int32_t* idx, float* w,
                            float* scores_out, float* logits_out, hipStream_t s);

// Histogram, stable permutation and the M-tile lists (main and remainder, see TilePlan).
size_t dispatch_scratch_bytes(const Layer& ly);
hipError_t launch_dispatch(const Layer& ly, const int32_t* idx, int32_t* counts, int32_t* offsets,
                           int32_t* perm, int32_t* inv, void* scratch, const TileList& tiles,
                           const TileList& small_tiles, const TilePlan& plan, hipStream_t s);
// With a capacity (ly.capacity > 0): zero the expert-output rows (assignment order, K wide) of
// the dropped assignments, i.e. rows perm[p] for sorted positions p in [offsets[E], T*k).
hipError_t launch_zero_dropped(const Layer& ly, const int32_t* offsets, const int32_t* perm, void* y,
                               hipStream_t s);
// Only the M-tile list, from existing offsets.
hipError_t launch_build_tiles(const Layer& ly, const int32_t* offsets, const TileList& tiles,
                              const TileList& small_tiles, const TilePlan& plan, hipStream_t s);

// GEMM variants. All operands are "NT": A (rows, Kd) and B (N, Kd), Kd contiguous.
struct GemmCall {
  const void* A;            // token rows (f32 or bf16 bits)
  int64_t lda;
  const int32_t* gather;    // logical sorted row p -> A row gather[p] / gather_div (or NULL)
  int32_t gather_div;
  const void* B;            // weight rows
  int64_t ldb;
  int64_t b_group_stride;   // elements between consecutive experts' weights
  int64_t b_plane_stride;   // elements between weight planes (planes kernel only)
  void* C;                  // output
  int64_t ldc;
  const int32_t* scatter;   // logical sorted row p -> output row scatter[p] (or NULL)
  int64_t N;                // output columns (SwiGLU: act columns = h)
  int64_t Kd;               // contraction length
  int64_t swiglu_h;         // > 0: SwiGLU epilogue, gate rows start at +swiglu_h
  int64_t dense_M;          // > 0: dense GEMM with this many rows (tiles ignored)
  TileList tiles;           // grouped mode
  // MXFP8 operands (launch_gemm_mx): E8M0 scale bytes, one per 32 elements along Kd, rows
  // laid out like the operands' rows (scale row stride *_scale_ld = Kd / 32 bytes)
  const uint8_t* a_scale;
  int64_t a_scale_ld;
  const uint8_t* b_scale;
  int64_t b_scale_ld;
  int64_t b_scale_group_stride;  // scale bytes between consecutive experts' weights
  // MXFP8 output of the SwiGLU GEMM: E4M3 codes (c_rows, ldc) and block scales (c_rows, N / 32)
  // instead of C
  uint8_t* c_codes;
  uint8_t* c_scales;
  // Training forward: the SwiGLU GEMM also stores its pre-activation H (rows_bound, 2 *
  // swiglu_h), sorted rows, [up | gate], rounded to bf16 (or NULL).
  void* h_out;
  // Backward operand layouts (bf16 MFMA GEMM). trans bit 0: A is stored contraction-major,
  // A(m, k) at A[k * lda + m]; bit 1: B likewise, B(n, k) at B[k * ldb + n] (per group).
  int trans;
  // SwiGLU-backward epilogue (bwd_h > 0): the product is d_act (rows, bwd_h), rounded to bf16;
  // with the saved H = h_in (rows, 2 * bwd_h) it writes [d_up | d_gate] to C (ldc = 2 * bwd_h).
  int64_t bwd_h;
  const void* h_in;
  // Weight-gradient mode (group_offsets != NULL): for each of `groups` groups g the product
  // C_g (dense_M, N) = sum over the contraction rows p in [group_offsets[g],
  // group_offsets[g + 1]) of A(., p) B(., p)^T, A and B both contraction-major (trans = 3);
  // C_g starts c_group_stride elements after C_{g-1}. Rows past a group's end read as zeros.
  const int32_t* group_offsets;
  int32_t groups;
  int64_t c_group_stride;
  // ... whose tiles are handed out in the order of group_order (groups by decreasing row count;
  // NULL = 0..groups-1) through tile_counter, one int32 that must be 0 at launch.
  const int32_t* group_order;
  int32_t* tile_counter;
  // Bounds used to clamp every row index a kernel derives from device data, so that a
  // corrupt index can never address memory outside the operands.
  int64_t a_rows;           // rows of A
  int64_t c_rows;           // rows of C
  int64_t rows_bound;       // logical (sorted) rows: dense_M or T*k
};

// bf16 MFMA GEMM; returns the M-tile height it was instantiated with for the chosen variant.
int gemm_bf16_tile_m(int variant);
// Workgroups per round of the main-list (large-tile) persistent grid on the current device, and
// output columns per tile of its up/gate GEMM (the SwiGLU halves of a 256-row weight tile).
int gemm_bf16_round_tiles();
int gemm_bf16_swiglu_tile_cols();
int gemm_bf16_pick_variant(double mean_rows_per_group);
hipError_t launch_gemm_bf16(const GemmCall& c, int variant, hipStream_t s);
// Backward GEMMs (bf16). Input gradients: grouped M-tiles of the given variant's tile height,
// B contraction-major (trans = 2), epilogue SwiGLU backward (bwd_h > 0), scatter or plain.
// Weight gradients: trans = 3 with group_offsets (one launch over all groups).
hipError_t launch_gemm_bf16_dgrad(const GemmCall& c, int variant, hipStream_t s);
hipError_t launch_gemm_bf16_wgrad(const GemmCall& c, hipStream_t s);
// Grouped MXFP8 GEMM: A and B are E4M3 codes (1 byte per element, ld in elements = bytes)
// with E8M0 scales; Kd a multiple of 128; M-tile height gemm_mx_tile_m(). Output and
// epilogues as launch_gemm_bf16 (SwiGLU + gather, or scatter).
int gemm_mx_tile_m();
hipError_t launch_gemm_mx(const GemmCall& c, hipStream_t s);
// Dense C(f32) = A(bf16) x sum_p B_p(bf16)^T over planes p = 0..2 (B_p at B + p*b_plane_stride):
// the fp32-exact router contraction. N must be a multiple of 4; N-tile width below.
hipError_t launch_gemm_bf16_planes_f32(const GemmCall& c, hipStream_t s);
int gemm_bf16_planes_tile_n();

// Skinny dense bf16 GEMM for at most 64 token rows (dense mode, no gather/scatter/SwiGLU,
// N a multiple of 64): weight streaming split over the whole chip. The k-splits write fp32
// partial planes to `partials` (gemm_skinny_partial_bytes; with less room it runs unsplit).
int gemm_skinny_splits(int64_t N, int64_t K);
size_t gemm_skinny_partial_bytes(int64_t M, int64_t N, int64_t K);
hipError_t launch_gemm_skinny(const GemmCall& c, float* partials, size_t partial_bytes, hipStream_t s);
constexpr int64_t kSkinnyMaxRows = 64;

// fp32 vector-ALU GEMM (fp32 layers and the fp32 router contraction); M-tile height 64.
constexpr int kF32TileM = 64;
hipError_t launch_gemm_f32(const GemmCall& c, bool a_is_bf16, const float* col_bias,
                           hipStream_t s);

// Load-balancing state (E <= 1024): acc (E) int64 += counts (E) int32; the load imbalance
// max * E / total of counts (E) int64 as fp64 (NaN with no tokens); the score_bias update by
// gamma * sign(total - E * acc[e]), which also zeroes acc and, when `imbalance` is not NULL,
// writes the imbalance of acc before the reset.
hipError_t launch_accumulate_counts(int E, const int32_t* counts, int64_t* acc, hipStream_t s);
hipError_t launch_load_imbalance(int E, const int64_t* counts, double* out, hipStream_t s);
hipError_t launch_score_bias_update(int E, float gamma, int64_t* acc, float* bias, double* imbalance,
                                    hipStream_t s);

// MXFP8 quantisation of bf16 rows: x (rows, cols) -> E4M3 codes (rows, cols) and E8M0 block
// scales (rows, cols / 32); cols a multiple of 32.
hipError_t launch_mx_quantize(const void* x, int64_t rows, int64_t cols, uint8_t* codes, uint8_t* scales,
                              hipStream_t s);

// Backward of the routed experts (backward.hip).
// dst[p] = src[idx[p] / div] for the kept rows p < min(*n_ptr, n_max); rows of row_bytes (a
// multiple of 16) bytes.
hipError_t launch_gather_rows(const void* src, int64_t src_rows, const int32_t* idx, int div, const int32_t* n_ptr,
                              int64_t n_max, int64_t row_bytes, void* dst, hipStream_t s);
// out (T, K) D = sum over j of in (T*k, K) D rows t*k+j, fp32, j ascending.
hipError_t launch_sum_copies(const Layer& ly, const void* in, void* out, hipStream_t s);
// dY (T*k, K) D = w * dO, dw (T, k) f32 = <dO[t], Y[t*k+j]> (dw may be NULL).
hipError_t launch_combine_backward(const Layer& ly, const void* y_assign, const float* w, const void* d_out,
                                   void* dy_assign, float* dw, hipStream_t s);
hipError_t launch_fill_zero(void* p, size_t bytes, hipStream_t s);
// counts (E) and offsets (E + 1) set to zero (an empty batch's histogram)
hipError_t launch_zero_counts_offsets(int32_t* counts, int32_t* offsets, int E, hipStream_t s);
// order (E): the experts by decreasing row count offsets[e+1] - offsets[e], ties by index
// (E <= 1024).
hipError_t launch_expert_order(const int32_t* offsets, int E, int32_t* order, hipStream_t s);
// fp32 layers: input gradients (group_offsets = expert offsets, groups = E, rows_bound <= 65535)
// and weight gradients (dense_M <= 65535 output rows per group), see backward.hip.
hipError_t launch_dgrad_f32(const GemmCall& c, hipStream_t s);
hipError_t launch_wgrad_f32(const GemmCall& c, hipStream_t s);

// Weighted combine (+ RMSNorm): out (T, K) D.
hipError_t launch_combine(const Layer& ly, const void* y_assign, const float* w,
                          const float* norm_weight, bool apply_norm, void* out, hipStream_t s);

}  // namespace moe
