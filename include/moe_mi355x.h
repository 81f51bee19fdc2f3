/*
 * moe_mi355x.h -- C ABI of the routed Mixture-of-Experts layer on MI355X (gfx950): the forward
 * pass, and the backward of the routed experts and of the combine.
 *
 * What the layer computes is defined on the page "Как устроен Olmo-core 3: обучение больших
 * MoE-моделей" (cited below as [OC3 "<section title>"]):
 *   router logits in fp32 from an (E, d_model) weight -> gating (softmax / topk_softmax /
 *   sigmoid + epsilon) -> top-k on score (+ per-expert score_bias), ties to the lower index ->
 *   weight normalisation and scaling -> optional latent down-projection d_model -> latent_dim
 *   -> stable permutation of the token copies by expert -> per-expert SwiGLU MLP (grouped
 *   GEMM, up_factor 2) -> unpermute and weighted combine -> optional bias-free RMSNorm, cast
 *   and up-projection latent_dim -> d_model.
 * The 896-expert latent shapes follow "Architecting Trillion-Scale Sparse Multimodal Models:
 * Design and Training Practices", section 1.
 *
 * Conventions for every entry point:
 *   - All tensor pointers are DEVICE pointers (hipMalloc / torch CUDA memory) of the calling
 *     process's current device, contiguous, row-major, 16-byte aligned. The caller owns every
 *     buffer; the library never allocates, frees or synchronises, and keeps no state between
 *     calls apart from cached device properties.
 *   - `stream` is a hipStream_t (NULL = the default stream). Work is enqueued on it and
 *     MOE_OK means "enqueued"; results are valid once the stream reaches that point.
 *   - Arguments are validated on the host before any HIP call. A failed check returns a
 *     status, enqueues nothing, and moe_last_error_message() (thread-local) says why. A launch
 *     failure returns MOE_ERR_HIP. Nothing aborts or throws across the ABI.
 *   - "D" below is the layer storage dtype (cfg.dtype): float for MOE_DTYPE_F32, bfloat16
 *     (uint16 bit pattern, round-to-nearest-even) for MOE_DTYPE_BF16. The router weight,
 *     biases, routing weights, logits and scores are always float32.
 *   - T = number of tokens; E = num_experts; k = top_k; K = latent_dim if set, else d_model;
 *     h = hidden_size; A = T*k (token-expert assignments). T = 0 is a valid no-op.
 *   - Results are deterministic: no floating-point atomics anywhere, so repeated calls on the
 *     same inputs are bitwise identical.
 */
#ifndef MOE_MI355X_H
#define MOE_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#if defined(__GNUC__) || defined(__clang__)
#define MOE_API __attribute__((visibility("default")))
#else
#define MOE_API
#endif

#define MOE_ABI_VERSION 7
#define MOE_MAX_EXPERTS 1024
#define MOE_MAX_TOP_K 16

typedef enum {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = 1,          /* NULL required pointer, bad size, inconsistent config  */
  MOE_ERR_UNSUPPORTED = 2,          /* valid on the page but not built here (see message)     */
  MOE_ERR_WORKSPACE_TOO_SMALL = 3,  /* ws_bytes below moe_workspace_size()                    */
  MOE_ERR_HIP = 4                   /* a HIP runtime call or kernel launch failed             */
} moe_status_t;

/* [OC3 "Маршрутизация: как роутер выбирает экспертов"]: the three gating functions. */
typedef enum {
  MOE_GATING_SOFTMAX = 0,       /* scores = softmax(logits); pick top-k of scores (+bias); weights = scores */
  MOE_GATING_TOPK_SOFTMAX = 1,  /* pick top-k of logits (+bias); weights = softmax over the k logits        */
  MOE_GATING_SIGMOID = 2        /* scores = sigmoid(logits) (+eps); pick top-k of scores (+bias)            */
} moe_gating_t;

/* [OC3 "Как задаётся конфигурация MoE"]: swiglu has up_factor 2. Only SwiGLU is defined on the
 * pages with its arithmetic ([OC3 "SwiGLU с квантизацией"]); other activations are rejected. */
typedef enum { MOE_ACT_SWIGLU = 0 } moe_activation_t;

typedef enum { MOE_DTYPE_F32 = 0, MOE_DTYPE_BF16 = 1 } moe_dtype_t;

/* Precision of the grouped expert matmuls ([OC3 "Rowwise FP8 и MXFP8"], [OC3 "Как сравнивали
 * и что получилось"]: the page compares MXFP8 against BF16). MXFP8 (see moe_mx_quantize):
 * the expert inputs z and the SwiGLU activation are MX-quantised along the contraction
 * dimension inside the experts stage, the weights come pre-quantised (moe_weights_t.w*_mx),
 * products accumulate in fp32 on the block-scaled matrix cores, outputs are bf16 as before.
 * Requires dtype bf16 and d_model / latent_dim and hidden_size multiples of 128. */
typedef enum { MOE_PRECISION_BF16 = 0, MOE_PRECISION_MXFP8 = 1 } moe_precision_t;

/*
 * Layer configuration. Field names follow MoEConfig / MoERouterConfigV2 / LatentMoEConfig
 * ([OC3 "Как задаётся конфигурация MoE"], [OC3 "Маршрутизация: как роутер выбирает
 * экспертов"], [OC3 "Латентная проекция экспертов"]). Call moe_config_default() first, then
 * set fields; struct_size lets the library reject a caller built against another layout.
 */
typedef struct moe_config_t {
  int32_t struct_size;                /* = sizeof(moe_config_t)                               */
  int32_t num_experts;                /* E, 1..MOE_MAX_EXPERTS (page default 1)               */
  int64_t d_model;                    /* model width, > 0                                      */
  int32_t top_k;                      /* k, 1..min(E, MOE_MAX_TOP_K)                           */
  int32_t gating_function;            /* moe_gating_t                                          */
  float sigmoid_stability_epsilon;    /* added to sigmoid scores; 0 = unset                    */
  float normalize_expert_weights;     /* p of the p-norm the k weights are divided by; 0 = off */
  int32_t restore_weight_scale;       /* nonzero: weights *= top_k                             */
  float expert_weight_scale;          /* weights *= this; 0 = unset                            */
  int32_t original_top_k;             /* != top_k: weights *= sqrt(original_top_k/top_k); 0 = unset */
  int32_t router_bias;                /* nonzero: router linear layer has an (E) bias          */
  int64_t hidden_size;                /* h, expert hidden width (page default 256)             */
  int32_t activation;                 /* moe_activation_t                                      */
  int32_t dtype;                      /* moe_dtype_t: storage dtype D of x, y and expert weights */
  int64_t latent_dim;                 /* L; 0 = no latent projection                           */
  int32_t up_proj_input_norm;         /* with latent: nonzero = bias-free RMSNorm before up-proj */
  float up_proj_input_norm_eps;       /* RMSNorm epsilon (page gives none; default 1e-5)       */
  float capacity_factor;              /* > 0: expert capacity with token dropping
                                         ([OC3 "Ёмкость эксперта и переполнение"]); 0 = dropless.
                                         capacity = 8 * ceil(capacity_factor * top_k * T / (8 * E))
                                         (expert-parallel degree 1, exact arithmetic); each expert
                                         keeps the first `capacity` assignments of the stable
                                         order, a dropped assignment's expert output is 0      */
  int32_t expert_precision;           /* moe_precision_t of the expert matmuls (default BF16)  */
} moe_config_t;

/*
 * Layer weights (device pointers, caller-owned, layouts out_features x in_features with the
 * input dimension contiguous -- the router's (E, d_model) layout of [OC3 "Маршрутизация"]).
 */
typedef struct moe_weights_t {
  const float* router_weight;  /* (E, d_model) fp32, required                                */
  const float* router_bias;    /* (E) fp32; required iff cfg.router_bias                      */
  const float* score_bias;     /* (E) fp32 or NULL: added to the selection keys only
                                  ([OC3 "Счётчики и bias-корректировка"])                      */
  const void* down_proj;       /* (L, d_model) D; required iff latent_dim                      */
  const float* up_proj_input_norm_weight; /* (L) fp32 RMSNorm weight g, or NULL = all ones      */
  const void* up_proj;         /* (d_model, L) D; required iff latent_dim                      */
  const void* w1;              /* (E, 2h, K) D: rows [0, h) = up, rows [h, 2h) = gate
                                  ([OC3 "SwiGLU с квантизацией"] splits up then gate)           */
  const void* w2;              /* (E, K, h) D                                                  */
  /* MXFP8 experts (cfg.expert_precision = MXFP8) read these instead of w1 / w2: the same
   * matrices as E4M3 codes with E8M0 block scales from moe_mx_quantize (blocks of 32 along
   * each row, i.e. along K for w1 and along h for w2).                                       */
  const uint8_t* w1_mx;        /* (E, 2h, K) codes                                             */
  const uint8_t* w1_mx_scale;  /* (E, 2h, K/32) scales                                         */
  const uint8_t* w2_mx;        /* (E, K, h) codes                                              */
  const uint8_t* w2_mx_scale;  /* (E, K, h/32) scales                                          */
} moe_weights_t;

/*
 * Routing outputs and optional diagnostics. Every pointer may be NULL (not wanted); the
 * stage calls below say which ones they require.
 */
typedef struct moe_routing_t {
  float* expert_weights;           /* (T, k) fp32 combine weights, j in key-descending order   */
  int32_t* expert_indices;         /* (T, k) int32 selected experts, key-descending, ties low  */
  int32_t* batch_size_per_expert;  /* (E) int32 token counts per expert, before any capacity
                                      drop ([OC3 "Балансировка нагрузки и вспомогательные
                                      штрафы"])                                                */
  int32_t* expert_offsets;         /* (E+1) int32 exclusive cumsum of the counts; with a
                                      capacity, of the kept counts min(count, capacity)        */
  int32_t* permutation;            /* (A) int32: sorted position p -> assignment t*k+j; with a
                                      capacity, positions >= expert_offsets[E] hold the dropped
                                      assignments (same stable order); positions past the
                                      placed assignments (only when moe_permute is given
                                      entries the routing never produces) hold -1             */
  int32_t* inverse_permutation;    /* (A) int32: assignment t*k+j -> sorted position p          */
  float* router_logits;            /* (T, E) fp32 logits                                       */
  float* router_scores;            /* (T, E) fp32 gating scores (softmax or sigmoid+eps)       */
} moe_routing_t;

/* ------------------------------------------------------------------------ housekeeping */

/* Returns MOE_ABI_VERSION of the built library. */
MOE_API int moe_abi_version(void);

/* Static description of a status code. Never NULL. */
MOE_API const char* moe_status_string(moe_status_t status);

/* Message of the last failed call on this thread ("" if none). Valid until the next call. */
MOE_API const char* moe_last_error_message(void);

/* Fills *cfg with the page defaults ([OC3 "Как задаётся конфигурация MoE"]: num_experts 1,
 * hidden_size 256) plus: top_k 1, softmax gating, SwiGLU, bf16, no latent, RMSNorm eps 1e-5.
 * d_model is left 0 and must be set. INVALID_ARG if cfg is NULL. */
MOE_API moe_status_t moe_config_default(moe_config_t* cfg);

/* Checks a configuration without touching the GPU. INVALID_ARG for values the page rules out
 * (top_k > num_experts, non-positive sizes, unknown enums); UNSUPPORTED for valid settings
 * this build does not implement (E > 1024, k > 16, non-SwiGLU, bf16 widths not multiples of
 * 64: d_model, latent_dim and hidden_size must be multiples of 64 in bf16). */
MOE_API moe_status_t moe_config_validate(const moe_config_t* cfg);

/* [OC3 "Как задаётся конфигурация MoE"]: total = router (d_model*E, +E with bias) +
 * 3*latent_dim*h*E, active = total - 3*latent_dim*h*E + 3*latent_dim*h*top_k, where
 * latent_dim is d_model without a latent projection. Either output pointer may be NULL. */
MOE_API moe_status_t moe_num_params(const moe_config_t* cfg, int64_t* total, int64_t* active);

/* Expert capacity for T tokens ([OC3 "Ёмкость эксперта и переполнение"]): 8 * ceil(
 * capacity_factor * top_k * T / (8 * num_experts)) in exact arithmetic, at expert-parallel
 * degree 1; values of T or more drop nothing and are reported as T rounded up to 8; 0 when
 * capacity_factor is 0 (dropless). No GPU work. */
MOE_API moe_status_t moe_expert_capacity(const moe_config_t* cfg, int64_t num_tokens, int64_t* capacity);

/* Bytes of device workspace moe_forward needs for T tokens (also enough for every stage call
 * with the same cfg and T). T*k must stay below 2^31 (int32 offsets,
 * [OC3 "Вычисления экспертов и точность"]); INVALID_ARG otherwise. */
MOE_API moe_status_t moe_workspace_size(const moe_config_t* cfg, int64_t num_tokens, size_t* bytes);

/* ------------------------------------------------------------------------ full layer */

/*
 * The whole forward pass for T tokens:
 *   x (T, d_model) D  ->  y (T, d_model) D.
 * routing may be NULL; non-NULL fields receive the routing outputs of this call. ws must
 * hold at least moe_workspace_size(cfg, T) bytes; its contents on entry do not matter.
 */
MOE_API moe_status_t moe_forward(const moe_config_t* cfg, const moe_weights_t* weights, int64_t num_tokens,
                         const void* x, void* y, moe_routing_t* routing, void* ws,
                         size_t ws_bytes, void* stream);

/* Device memory of moe_forward_noalloc, per GPU (64 MiB). */
#define MOE_NOALLOC_SCRATCH_BYTES (64ull << 20)

/*
 * moe_forward for callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid allocation): the same kernels and results, with
 * the workspace taken from a library-owned array of MOE_NOALLOC_SCRATCH_BYTES on each GPU,
 * held from the first call on that GPU until the process ends. The caller still passes the
 * inputs, y and the optional routing outputs. The first call on a device looks up that
 * device's copy of the array (with the device current); no call allocates or frees device
 * memory. WORKSPACE_TOO_SMALL (nothing enqueued) when moe_workspace_size(cfg, T) exceeds
 * MOE_NOALLOC_SCRATCH_BYTES (decode-sized batches fit: 64 tokens of an 896-expert latent
 * layer need 5.4 MiB). Every call on a GPU uses that GPU's one array: calls that overlap on
 * one GPU (two streams, two threads) race and must be ordered by the caller. The array keeps
 * the last call's contents; the forward reads nothing it did not write in the same call.
 */
MOE_API moe_status_t moe_forward_noalloc(const moe_config_t* cfg, const moe_weights_t* weights,
                                 int64_t num_tokens, const void* x, void* y, moe_routing_t* routing,
                                 void* stream);

/* ------------------------------------------------------------------------ stage calls */

/*
 * Router: [OC3 "Маршрутизация: как роутер выбирает экспертов"]. x (T, d_model) D is read as
 * fp32; logits = x * router_weight^T (+ router_bias) in fp32; gating; top-k of the keys
 * (scores or logits, + score_bias); weights gathered / re-softmaxed, normalised and scaled.
 * Requires routing->expert_weights and routing->expert_indices; router_logits and
 * router_scores are filled when non-NULL. Uses the workspace (moe_workspace_size bytes) for
 * partial sums of the logits and, on large layers, for the fp32 router weights split into
 * three bf16 planes (hi + mid + lo = the fp32 value exactly) that the MFMA contraction reads.
 */
MOE_API moe_status_t moe_router_forward(const moe_config_t* cfg, const moe_weights_t* weights,
                                int64_t num_tokens, const void* x, moe_routing_t* routing,
                                void* ws, size_t ws_bytes, void* stream);

/*
 * Selection and weights from a given gating output -- the injection point that makes the
 * routing checkable bit for bit. sel_input (T, E) fp32 is the scores for softmax / sigmoid
 * gating and the logits for topk_softmax ([OC3 "Маршрутизация"]: those are what each gating
 * selects on); score_bias (E) fp32 or NULL. Key = sel_input + score_bias (one fp32 add);
 * indices = the k largest keys, largest first, equal keys to the lower index, -0.0 == +0.0,
 * NaN after every number. Writes expert_indices (T, k) and expert_weights (T, k). No
 * workspace.
 */
MOE_API moe_status_t moe_route_from_scores(const moe_config_t* cfg, int64_t num_tokens,
                                   const float* sel_input, const float* score_bias,
                                   int32_t* expert_indices, float* expert_weights, void* stream);

/*
 * Token counts and the stable permutation: [OC3 "Пересылка токенов между экспертами"] (sort
 * the expert indices; bins = cumsum of counts) and [OC3 "Балансировка нагрузки и
 * вспомогательные штрафы"] (per-expert histogram). expert_indices (T, k) int32 in [0, E),
 * distinct within a row (the routing always gives such rows; an entry out of [0, E), or one
 * that repeats an earlier expert of its row, is not counted and gets no position: its inverse
 * is -1 and it occupies no slot below expert_offsets[E]). Outputs (all required): batch_size_per_expert (E), expert_offsets (E+1),
 * permutation (A), inverse_permutation (A); the permutation is the stable sort of t*k+j by
 * expert. With cfg.capacity_factor > 0 ([OC3 "Ёмкость эксперта и переполнение"]) each expert
 * keeps the first `capacity` assignments of that order: the offsets delimit the kept rows, the
 * permutation lists the kept assignments first and the dropped ones after them, and the counts
 * stay the full histogram. Uses the workspace. With T = 0 only the counts and offsets are
 * written (zeros) and the other pointers may be NULL.
 */
MOE_API moe_status_t moe_permute(const moe_config_t* cfg, int64_t num_tokens,
                         const int32_t* expert_indices, int32_t* batch_size_per_expert,
                         int32_t* expert_offsets, int32_t* permutation,
                         int32_t* inverse_permutation, void* ws, size_t ws_bytes, void* stream);

/*
 * Latent down-projection ([OC3 "Латентная проекция экспертов"], prepare_routed_input):
 * z (T, L) D = x (T, d_model) D * down_proj^T, fp32 accumulation. UNSUPPORTED without latent.
 * ws is optional (NULL: none): with few tokens the projection splits its contraction over the
 * chip and keeps fp32 partial sums there; without it the contraction runs unsplit (same
 * result, slower). A non-NULL ws must hold moe_workspace_size(cfg, num_tokens) bytes
 * (WORKSPACE_TOO_SMALL otherwise).
 */
MOE_API moe_status_t moe_latent_down(const moe_config_t* cfg, const moe_weights_t* weights,
                             int64_t num_tokens, const void* x, void* z, void* ws,
                             size_t ws_bytes, void* stream);

/*
 * Routed experts ([OC3 "Вычисления экспертов и точность"], [OC3 "SwiGLU с квантизацией"]):
 * for every expert e, the rows p in [offsets[e], offsets[e+1]) of the sorted order take token
 * t = permutation[p] / k of z (T, K) D, compute H = z_t * w1[e]^T, act = up * gate *
 * sigmoid(gate) (fp32, stored as D), Y = act * w2[e]^T in fp32 accumulation, rounded to D
 * (bf16 for bf16 layers: the grouped experts return bf16), and write Y to row
 * permutation[p] of y_assign (A, K) D -- i.e. y_assign is in assignment order t*k+j. Experts
 * with no rows read no weights. With cfg.capacity_factor > 0 the rows p >= offsets[E] of the
 * permutation are dropped assignments: their y_assign rows are set to 0. Uses the workspace.
 */
MOE_API moe_status_t moe_experts_forward(const moe_config_t* cfg, const moe_weights_t* weights,
                                 int64_t num_tokens, const void* z, const int32_t* expert_offsets,
                                 const int32_t* permutation, void* y_assign, void* ws,
                                 size_t ws_bytes, void* stream);

/*
 * Unpermute + weighted combine (+ latent restore norm): o[t] = sum_{j<k} expert_weights[t,j] *
 * y_assign[t*k+j] in fp32, j ascending ([OC3 "Пересылка токенов между экспертами"]: results
 * return to the original positions). Without latent: out (T, K) D = o. With latent: out
 * (T, L) D = RMSNorm(o) * g if cfg.up_proj_input_norm, else o, cast to D
 * ([OC3 "Латентная проекция экспертов"]). weights may be NULL when no norm weight is needed.
 */
MOE_API moe_status_t moe_combine(const moe_config_t* cfg, const moe_weights_t* weights,
                         int64_t num_tokens, const void* y_assign, const float* expert_weights,
                         void* out, void* stream);

/*
 * Latent up-projection ([OC3 "Латентная проекция экспертов"], restore_routed_output): y
 * (T, d_model) D = n (T, L) D * up_proj^T, fp32 accumulation. UNSUPPORTED without latent.
 * ws as for moe_latent_down.
 */
MOE_API moe_status_t moe_latent_up(const moe_config_t* cfg, const moe_weights_t* weights,
                           int64_t num_tokens, const void* n, void* y, void* ws, size_t ws_bytes,
                           void* stream);

/* ------------------------------------------------------------------------ backward */

/*
 * Training forward of the routed experts: what moe_experts_forward computes (same arguments,
 * same y_assign), plus the two tensors the backward reads ([OC3 "SwiGLU с квантизацией"]: the
 * activation keeps its input for the backward), both in sorted order:
 *   h_saved (A, 2h) D: the pre-activation H = z_t * w1[e]^T = [up | gate] of each kept row
 *     p < expert_offsets[E], rounded to D (act is computed from the unrounded H);
 *   act_saved (A, h) D: the SwiGLU activation of those rows.
 * Rows p >= expert_offsets[E] of both are left unwritten. bf16 expert precision only
 * (UNSUPPORTED with MXFP8). Uses the workspace (moe_workspace_size bytes).
 */
MOE_API moe_status_t moe_experts_forward_train(const moe_config_t* cfg, const moe_weights_t* weights,
                                               int64_t num_tokens, const void* z, const int32_t* expert_offsets,
                                               const int32_t* permutation, void* y_assign, void* h_saved,
                                               void* act_saved, void* ws, size_t ws_bytes, void* stream);

/* Bytes of device workspace moe_experts_backward needs for T tokens: about (2 * K + 2h) * T *
 * top_k elements of D (dY and z in sorted order, dH) plus the M-tile lists. UNSUPPORTED when
 * the backward does not serve the configuration (see moe_experts_backward). */
MOE_API moe_status_t moe_experts_backward_workspace_size(const moe_config_t* cfg, int64_t num_tokens,
                                                         size_t* bytes);

/*
 * Backward of the routed experts ([OC3 "Вычисления экспертов и точность"]: each expert's
 * gradients come from its own rows of the grouped products; [OC3 "SwiGLU с квантизацией"]: the
 * SwiGLU backward; [OC3 "Пересылка токенов между экспертами"]: the gather by the permutation).
 * Inputs: z (T, K) D, expert_offsets (E+1) and permutation (A) as given to the forward, the
 * forward's h_saved and act_saved (moe_experts_forward_train), and dy_assign (A, K) D, the
 * gradient of y_assign (assignment order t*k+j). With dY[p] = dy_assign[permutation[p]] and
 * z_perm[p] = z[permutation[p] / k], for each expert e on its kept rows R:
 *   d_act   = dY[R] * w2[e]                          fp32 accumulation, stored as D;
 *   dH      = [d_act * silu(gate) | d_act * up * silu'(gate)], silu' = sigmoid * (1 + gate *
 *             (1 - sigmoid)), in fp32 from the saved H, stored as D;
 *   dz_perm = dH * w1[e]                             stored as D;
 *   dw2[e]  = dY[R]^T * act[R],  dw1[e] = dH^T * z_perm[R]   fp32 accumulation, stored as D.
 * Outputs: dz (T, K) D = the sum over j (fp32, j ascending) of dz_perm of assignment t*k+j,
 * dropped assignments contributing nothing; dw1 (E, 2h, K) D and dw2 (E, K, h) D, zero for
 * experts without rows. ws: moe_experts_backward_workspace_size bytes. bf16 expert precision
 * only; bf16 layers need A * 2h < 2^31, fp32 layers A, K and 2h at most 65535 (UNSUPPORTED
 * otherwise). With T = 0 only dw1 and dw2 are written (zeros) and the other pointers may be NULL.
 */
MOE_API moe_status_t moe_experts_backward(const moe_config_t* cfg, const moe_weights_t* weights,
                                          int64_t num_tokens, const void* z, const int32_t* expert_offsets,
                                          const int32_t* permutation, const void* h_saved, const void* act_saved,
                                          const void* dy_assign, void* dz, void* dw1, void* dw2, void* ws,
                                          size_t ws_bytes, void* stream);

/*
 * Backward of the weighted combine o[t] = sum_j expert_weights[t,j] * y_assign[t*k+j]
 * ([OC3 "Пересылка токенов между экспертами"]): given d_out (T, K) D, the gradient of o,
 *   dy_assign (A, K) D        = expert_weights[t,j] * d_out[t], rounded to D;
 *   d_expert_weights (T, k) f32 = sum_c d_out[t,c] * y_assign[t*k+j,c] (NULL: not wanted).
 * UNSUPPORTED for a latent layer with the up-projection input norm (its backward is not
 * built). No workspace.
 */
MOE_API moe_status_t moe_combine_backward(const moe_config_t* cfg, int64_t num_tokens, const void* y_assign,
                                          const float* expert_weights, const void* d_out, void* dy_assign,
                                          float* d_expert_weights, void* stream);

/* ------------------------------------------------------------------------ MXFP8 */

/*
 * MXFP8 quantisation of bf16 rows ([OC3 "Rowwise FP8 и MXFP8"]; the page does not define the
 * format, read as OCP microscaling): each block of 32 consecutive elements of a row shares one
 * E8M0 scale byte s (value 2^(s - 127)) with s - 127 = floor(log2(amax of the block)) - 8,
 * clamped to [-127, 127] (an all-zero block gets s = 0); the elements are FP8 E4M3 (OCP: bias
 * 7, 3 mantissa bits, max 448) of value / 2^(s - 127), rounded to nearest-even and saturated
 * at +-448. x (rows, cols) bf16 -> codes (rows, cols) uint8 and scales (rows, cols / 32) uint8,
 * row-major. cols must be a positive multiple of 32 (INVALID_ARG otherwise); inputs must be
 * finite. Used to pre-quantise the expert weights for cfg.expert_precision = MXFP8 (W1 rows
 * along K, W2 rows along h).
 */
MOE_API moe_status_t moe_mx_quantize(int64_t rows, int64_t cols, const void* x, uint8_t* codes, uint8_t* scales,
                                     void* stream);

/* ------------------------------------------------------------------------ balancing state */

/*
 * Router load-balancing state ([OC3 "Счётчики и bias-корректировка"], [OC3 "Управление
 * состоянием между шагами"]). Counters are per-expert int64 device arrays of num_experts
 * entries (1..MOE_MAX_EXPERTS) owned by the caller; everything is integer arithmetic apart
 * from the two results named below, and nothing depends on reduction order.
 */

/* accumulator (E) int64 += batch_size_per_expert (E) int32 -- the step's
 * score_bias_batch_size_per_expert accumulator, fed with the counts of each forward
 * (moe_routing_t.batch_size_per_expert). INVALID_ARG on NULL pointers or E out of range. */
MOE_API moe_status_t moe_accumulate_expert_counts(int32_t num_experts, const int32_t* batch_size_per_expert,
                                                  int64_t* accumulator, void* stream);

/* Load imbalance of a counter: max(counts) / mean(counts) = max * E / total, one fp64 division
 * of the exact integers (correctly rounded), written to *imbalance (one double on the device).
 * No tokens (total 0): NaN, the value of 0 / 0. The page aggregates the local metric over
 * processes with max and the global one with mean; one process computes this value once. */
MOE_API moe_status_t moe_load_imbalance(int32_t num_experts, const int64_t* counts, double* imbalance,
                                        void* stream);

/* The aux-loss-free score_bias update, run once per step: with ideal = total / E the mean
 * size per expert, score_bias[e] (fp32, in place) += bias_gamma * sign(ideal - accumulator[e])
 * (the sign taken exactly, in integers; one fp32 add of +-bias_gamma or 0), then the
 * accumulator is zeroed. imbalance may be NULL; otherwise it receives the load imbalance of
 * the accumulator before the reset. INVALID_ARG on NULL required pointers, E out of range or
 * a non-finite bias_gamma. */
MOE_API moe_status_t moe_score_bias_update(int32_t num_experts, float bias_gamma, int64_t* accumulator,
                                           float* score_bias, double* imbalance, void* stream);

/* ------------------------------------------------------------------------ calibration */

/*
 * Measurement support, not part of the layer: the rates this device achieves, which the layer's
 * kernels are reported against beside the published peaks.
 *
 * moe_calibrate_mfma_bf16: one workgroup of 8 wavefronts per compute unit, each wavefront running
 * `iters` rounds of 8 independent 32x32x16 bf16 matrix-core products (fp32 accumulation) on
 * register operands, with no memory traffic. *num_waves receives the number of wavefronts and
 * *flops the launch's dense flop count (2*32*32*16 per product); the caller times the stream.
 * Each wavefront writes one float (a sum of its accumulators) to out[wave], so out (device, fp32)
 * must hold *num_waves values. out == NULL only fills *num_waves and *flops and enqueues nothing.
 * INVALID_ARG for iters < 1 or NULL num_waves / flops.
 *
 * moe_calibrate_copy: copies `bytes` (a positive multiple of 16) from src to dst (device, 16-byte
 * aligned, not overlapping) with 16-byte vector loads and stores; HBM traffic 2 * bytes.
 * INVALID_ARG for NULL pointers or a bad size.
 */
MOE_API moe_status_t moe_calibrate_mfma_bf16(int64_t iters, float* out, int64_t* num_waves, double* flops,
                                             void* stream);
/* The same for the block-scaled FP8 products of the MXFP8 expert matmuls: rounds of 8 independent
 * 32x32x64 E4M3 products with unit E8M0 scales (2*32*32*64 flops each); same arguments. */
MOE_API moe_status_t moe_calibrate_mfma_mxfp8(int64_t iters, float* out, int64_t* num_waves, double* flops,
                                              void* stream);
MOE_API moe_status_t moe_calibrate_copy(const void* src, void* dst, int64_t bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_MI355X_H */
