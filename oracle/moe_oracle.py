"""Plain CPU oracle of the routed Mixture-of-Experts layer: the forward pass and the backward
of the routed experts (SwiGLU backward, the grouped matmuls' input and weight gradients, the
combine backward).

TEST INFRASTRUCTURE. Only the tests, the smoke check of the package entry file and the
bench's cpu_baseline leg may import or call this module. The HIP path never does, and this
module imports nothing from it: the two share no code, headers, tables or helpers. The
only thing both consume is the seeded input generators in `workloads`.

Sources (cited by page title and section in every function below):
  [OC3]  "Как устроен Olmo-core 3: обучение больших MoE-моделей" -- the authority for what
         the layer computes. Sections used: "Как задаётся конфигурация MoE" (config and
         parameter counts), "Латентная проекция экспертов" (latent projection),
         "Маршрутизация: как роутер выбирает экспертов" (routing), "Разрешение равенства
         логитов и квантизация" (tie intent), "Балансировка нагрузки и вспомогательные
         штрафы" (token counts), "Пересылка токенов между экспертами" (permutation),
         "Вычисления экспертов и точность" (grouped experts, bf16 output), "SwiGLU с
         квантизацией" (up/gate split, gate*sigmoid(gate)).
  [TSM]  "Architecting Trillion-Scale Sparse Multimodal Models: Design and Training
         Practices", section 1 -- the 896-expert latent scale (context only).

Arithmetic. Every floating-point step runs in float64 and is rounded only where the pages
fix a precision (router logits and scores in fp32; expert output in bf16; the restored
output cast to the up-projection's dtype) or where the layer's storage dtype fixes one (the
latent input z and the SwiGLU activation are stored in the layer dtype). bf16 rounding is
round-to-nearest-even of the float64 value, done with frexp so the arithmetic is exact.

Readings where the pages are silent (each is listed with its reason in the design notes):
  * top-k order: key descending, ties to the lower expert index, -0.0 == +0.0, NaN keys
    after every number (ties among NaNs by index);
  * the permutation is a stable sort of the flat assignment index t*k+j by expert;
  * the combine is o[t] = sum_j w[t,j] * Y[t,j], summed in j order, no extra normalisation;
  * latent restore order: combine, then RMSNorm(eps, weight g, no bias), cast, up-projection;
  * down/up projections carry no bias; all weights are stored (out_features, in_features).

Capacity ([OC3 "Ёмкость эксперта и переполнение"]): with a capacity_factor each expert keeps
the first `capacity` assignments of the stable order and drops the rest (their expert output
is 0), capacity = 8 * ceil(capacity_factor * top_k * T / (8 * E)).

Balancing state ([OC3 "Счётчики и bias-корректировка"]): the count accumulator, the load
imbalance metric max/mean, and the score_bias update by bias_gamma * sign(ideal - actual).

Backward ([OC3 "SwiGLU с квантизацией"]: the activation keeps its input H, the backward
splits it into up and gate and forms sigmoid, silu, its derivative and the two gradients in
fp32 or better, concatenated in the storage dtype; [OC3 "Вычисления экспертов и точность"]:
each expert's gradients come from its own rows of the grouped matmuls). Readings: H is saved
in the layer dtype; d_act, dH, the per-copy input gradients and the weight gradients are
stored in the layer dtype; a token's k copies are summed in float64 and rounded once.

Pins of the backward (tests/test_oracle_backward_pins.py): hand-worked cases, torch autograd
of an independent dense per-assignment forward, central finite differences of the oracle's
own forward, and bf16 representability of every stored gradient.

Pins (tests/test_oracle_pins.py): parameter counts against the element counts of the
generated tensors and the golden table; logits against an exactly-rounded fsum dot
product; gating against torch's softmax/sigmoid; selection against brute force over all
k-subsets and against Python's sort; weights against closed forms (golden fixtures);
histogram/permutation against invariants and a brute-force counting sort; the expert path
against a dense evaluation of every expert on every token; special cases against torch's
silu / rms_norm; permutation equivariance and RMSNorm scale invariance; the balancing
state against closed forms (uniform load, one hot expert, fractional ideal) and against
exact rational arithmetic (fractions.Fraction) on random counts; the capacity against
hand-worked values, a first-come-first-kept walk over the assignments and a dense evaluation
with the kept mask.
"""
from __future__ import annotations

from dataclasses import dataclass, fields
from typing import Optional

import numpy as np

GATINGS = ("softmax", "topk_softmax", "sigmoid")
DTYPES = ("f32", "bf16")


@dataclass(frozen=True)
class MoEConfig:
    """Layer fields. [OC3 "Как задаётся конфигурация MoE"]: num_experts defaults to 1 and
    hidden_size to 256; d_model, num_experts and top_k are set on the router config.
    [OC3 "Маршрутизация"]: gating function, sigmoid_stability_epsilon, normalisation order,
    restore_weight_scale, expert_weight_scale, original_top_k. [OC3 "Латентная проекция
    экспертов"]: latent_dim and the up-projection input norm (bias-free RMSNorm default)."""
    d_model: int
    num_experts: int = 1
    top_k: int = 1
    hidden_size: int = 256
    gating_function: str = "softmax"
    sigmoid_stability_epsilon: Optional[float] = None
    normalize_expert_weights: Optional[float] = None
    restore_weight_scale: bool = False
    expert_weight_scale: Optional[float] = None
    original_top_k: Optional[int] = None
    router_bias: bool = False
    latent_dim: Optional[int] = None
    up_proj_input_norm: bool = True
    up_proj_input_norm_eps: float = 1e-5
    dtype: str = "bf16"
    capacity_factor: Optional[float] = None
    expert_precision: str = "bf16"   # "bf16" or "mxfp8" (the expert matmuls)

    @classmethod
    def from_dict(cls, d: dict) -> "MoEConfig":
        names = {f.name for f in fields(cls)}
        return cls(**{k: v for k, v in d.items() if k in names})

    @property
    def expert_dim(self) -> int:
        """Width of the routed payload: latent_dim with a latent projection, else d_model."""
        return self.latent_dim if self.latent_dim else self.d_model


# ----------------------------------------------------------------------------- rounding

def round_f32(a) -> np.ndarray:
    """Round to the nearest float32 (ties to even); returned as float64 holding that value."""
    return np.asarray(a, dtype=np.float64).astype(np.float32).astype(np.float64)


def round_bf16(a) -> np.ndarray:
    """Round to the nearest bfloat16 (8 significant bits, ties to even), as float64.

    a = m * 2**e with 0.5 <= |m| < 1; m * 2**8 is exact in float64, np.round rounds half to
    even, so the result is the correctly rounded bf16 value. Below 2**-126 (bf16's subnormal
    range) the spacing is fixed at 2**-133. (Overflow never occurs in the layer's values.)
    """
    a = np.asarray(a, dtype=np.float64)
    m, e = np.frexp(a)
    normal = np.ldexp(np.round(m * 256.0) / 256.0, e)
    sub = np.ldexp(np.round(np.ldexp(a, 133)), -133)
    return np.where(np.abs(a) < 2.0 ** -126, sub, normal)


def round_to(a, dtype: str) -> np.ndarray:
    if dtype == "f32":
        return round_f32(a)
    if dtype == "bf16":
        return round_bf16(a)
    raise ValueError(dtype)


def _f64(a) -> np.ndarray:
    return np.asarray(a, dtype=np.float64)


def _acc(a, acc) -> np.ndarray:
    """The operand of a contraction in the accumulation dtype: float64 (the default, for
    checking) or float32 (the mode the CPU timing uses; the products then sum in fp32 BLAS)."""
    return np.asarray(a, dtype=acc)


# ----------------------------------------------------------------------------- router

def router_logits(x, router_weight, router_bias=None, acc=np.float64) -> np.ndarray:
    """[OC3 "Маршрутизация"]: the router input is cast to fp32 and a linear layer with an
    (num_experts, d_model) weight gives the (tokens, num_experts) logits. [OC3 "Как задаётся
    конфигурация MoE"]: the router has d_model*num_experts weights plus num_experts bias terms
    when bias is on. The dot products are summed in float64 and rounded to fp32 once.
    Eval mode: the training-only jitter of [OC3 "Jitter при обучении"] is a no-op."""
    l = _acc(x, acc) @ _acc(router_weight, acc).T
    if router_bias is not None:
        l = l + _f64(router_bias)[None, :]
    return round_f32(l)


def gating_scores(cfg: MoEConfig, logits) -> np.ndarray:
    """[OC3 "Маршрутизация"]: softmax and topk_softmax both score with a softmax of the logits
    over the expert axis; sigmoid scores each expert independently and, when
    sigmoid_stability_epsilon is set, adds it to every score. Computed in float64 and rounded
    to fp32; the epsilon is then added as an fp32 addition."""
    l = _f64(logits)
    if cfg.gating_function in ("softmax", "topk_softmax"):
        m = l.max(axis=-1, keepdims=True)
        e = np.exp(l - m)
        return round_f32(e / e.sum(axis=-1, keepdims=True))
    if cfg.gating_function == "sigmoid":
        with np.errstate(over="ignore"):
            s = round_f32(1.0 / (1.0 + np.exp(-l)))
        if cfg.sigmoid_stability_epsilon:
            s = round_f32(s + round_f32(cfg.sigmoid_stability_epsilon))
        return s
    raise ValueError(cfg.gating_function)


def selection_keys(cfg: MoEConfig, logits, scores, score_bias=None) -> np.ndarray:
    """[OC3 "Маршрутизация"] and [OC3 "Счётчики и bias-корректировка"]: topk_softmax picks
    experts by logits (+ score_bias); the other gatings pick by scores (+ score_bias). The
    bias only steers selection. The addition is one fp32 add per element."""
    base = _f64(logits if cfg.gating_function == "topk_softmax" else scores)
    if score_bias is None:
        return base
    return round_f32(base + _f64(score_bias)[None, :])


def select_topk(keys, k: int) -> np.ndarray:
    """Indices of the k largest keys per row, largest first.

    [OC3 "Маршрутизация"] selects with topk (max when k == 1). The page's disabled tie
    branch ([OC3 "Разрешение равенства логитов и квантизация"]) states the intent that equal
    keys go to the lower expert index; that is the rule here. Keys compare as IEEE numbers
    (-0.0 equals +0.0); NaN keys rank after every number, NaNs among themselves by index.
    Implemented as a lexicographic sort on (is_nan, -key, expert index).
    """
    keys = _f64(keys)
    T, E = keys.shape
    nan = np.isnan(keys)
    neg = np.where(nan, 0.0, -keys)
    neg = np.where(neg == 0.0, 0.0, neg)  # one zero: -0.0 and +0.0 are the same key
    eidx = np.broadcast_to(np.arange(E), (T, E))
    order = np.lexsort((eidx, neg, nan), axis=-1)
    return order[:, :k].astype(np.int64)


def expert_weights(cfg: MoEConfig, logits, scores, idx) -> np.ndarray:
    """[OC3 "Маршрутизация"]: topk_softmax weights are a softmax over the selected experts'
    logits (bias not included); otherwise the weights are the original scores gathered at the
    selected experts. Then, in this order: divide by the p-norm over the k weights when
    normalize_expert_weights = p is set; multiply by top_k when restore_weight_scale; by
    expert_weight_scale when set; by sqrt(original_top_k / top_k) when original_top_k differs
    from top_k. float64, rounded to fp32 at the end."""
    T = idx.shape[0]
    k = cfg.top_k
    rows = np.arange(T)[:, None]
    if cfg.gating_function == "topk_softmax":
        sel = _f64(logits)[rows, idx]
        m = sel.max(axis=-1, keepdims=True)
        e = np.exp(sel - m)
        w = e / e.sum(axis=-1, keepdims=True)
    else:
        w = _f64(scores)[rows, idx]
    p = cfg.normalize_expert_weights
    if p:
        w = w / (np.abs(w) ** p).sum(axis=-1, keepdims=True) ** (1.0 / p)
    if cfg.restore_weight_scale:
        w = w * k
    if cfg.expert_weight_scale:
        w = w * cfg.expert_weight_scale
    if cfg.original_top_k and cfg.original_top_k != k:
        w = w * (cfg.original_top_k / k) ** 0.5
    return round_f32(w)


def route(cfg: MoEConfig, logits, score_bias=None) -> dict:
    """Gating, selection and weights from the logits ([OC3 "Маршрутизация"])."""
    scores = gating_scores(cfg, logits)
    keys = selection_keys(cfg, logits, scores, score_bias)
    idx = select_topk(keys, cfg.top_k)
    w = expert_weights(cfg, logits, scores, idx)
    return dict(logits=_f64(logits), scores=scores, keys=keys, idx=idx, w=w)


def route_from_scores(cfg: MoEConfig, sel_input, score_bias=None) -> dict:
    """Selection and weights given the gating output: the scores for softmax/sigmoid, the
    logits for topk_softmax (the input topk_softmax selects on). Same steps as route()."""
    if cfg.gating_function == "topk_softmax":
        logits, scores = sel_input, None
    else:
        logits, scores = None, sel_input
    keys = selection_keys(cfg, logits, scores, score_bias)
    idx = select_topk(keys, cfg.top_k)
    w = expert_weights(cfg, logits, scores, idx)
    return dict(keys=keys, idx=idx, w=w)


# ----------------------------------------------------------------------- dispatch

def expert_counts(idx, num_experts: int) -> np.ndarray:
    """[OC3 "Балансировка нагрузки и вспомогательные штрафы"]: a histogram of the selected
    indices summed over all tokens -- one count per expert."""
    return np.bincount(np.asarray(idx).ravel(), minlength=num_experts).astype(np.int64)


def expert_offsets(counts) -> np.ndarray:
    """[OC3 "Пересылка токенов между экспертами"]: bins are the cumulative sum of the
    per-expert counts; [OC3 "Вычисления экспертов и точность"]: offsets are int32 cumsums.
    Returned with a leading 0 (length E+1)."""
    return np.concatenate([[0], np.cumsum(np.asarray(counts, dtype=np.int64))])


def stable_permutation(idx):
    """[OC3 "Пересылка токенов между экспертами"]: sorting the expert indices orders the
    assignments by expert. Read as a stable sort of the flat assignment index a = t*k + j by
    expert, so inside one expert the assignments keep token order. Returns (perm, inv) with
    perm[p] = the assignment at sorted position p and inv[perm[p]] = p."""
    flat = np.asarray(idx).ravel()
    perm = np.argsort(flat, kind="stable").astype(np.int64)
    inv = np.empty_like(perm)
    inv[perm] = np.arange(flat.size)
    return perm, inv


def expert_capacity(cfg: MoEConfig, num_tokens: int) -> Optional[int]:
    """[OC3 "Ёмкость эксперта и переполнение"]: expert capacity = (expert-parallel degree) x
    (allowed local inputs per expert); the allowed number is capacity_factor x the ideal
    number of inputs, rounded up to a multiple of eight; the ideal number is top_k x
    local_batch_size / num_experts. One process: degree 1, local batch = the num_tokens
    tokens. Exact rational arithmetic on the fp32 capacity_factor. None = no capacity
    (dropless)."""
    if not cfg.capacity_factor:
        return None
    from fractions import Fraction
    import math
    allowed = Fraction(float(np.float32(cfg.capacity_factor))) * Fraction(cfg.top_k * num_tokens, cfg.num_experts)
    return 8 * math.ceil(allowed / 8)


def capacity_permutation(idx, num_experts: int, capacity: Optional[int]):
    """[OC3 "Ёмкость эксперта и переполнение"]: on overflow every expert gets exactly
    `capacity` inputs, the limit being applied when the local permutation gathers the tokens.
    Read as: in the stable order of [OC3 "Пересылка токенов между экспертами"] (assignments
    t*k+j sorted by expert, token order inside an expert) the first `capacity` assignments of
    each expert are kept and the rest are dropped; a dropped assignment's expert output is 0.
    Returns (perm, inv, kept): perm lists the kept assignments in that stable order, then the
    dropped ones in the same order (so it stays a bijection of the A assignments); inv is its
    inverse; kept (A,) bool. capacity None keeps everything (the plain stable permutation)."""
    flat = np.asarray(idx).ravel()
    order = np.argsort(flat, kind="stable").astype(np.int64)
    if capacity is None:
        kept = np.ones(flat.size, dtype=bool)
        perm = order
    else:
        counts = np.bincount(flat, minlength=num_experts)
        first = np.concatenate([[0], np.cumsum(counts)])[:-1]
        rank = np.empty(flat.size, dtype=np.int64)
        rank[order] = np.arange(flat.size) - first[flat[order]]
        kept = rank < capacity
        perm = np.concatenate([order[kept[order]], order[~kept[order]]])
    inv = np.empty_like(perm)
    inv[perm] = np.arange(flat.size)
    return perm, inv, kept


# ------------------------------------------------------------------- MXFP8 (expert GEMMs)
# [OC3 "Rowwise FP8 и MXFP8"] and [OC3 "Как сравнивали и что получилось"]: the grouped expert
# matmuls can run in MXFP8 (the page measures it against BF16). The page does not spell the
# format out; read as the OCP microscaling format: blocks of 32 consecutive elements along the
# contraction dimension share one power-of-two scale (E8M0), elements are FP8 E4M3 (1 sign,
# 4 exponent bits with bias 7, 3 mantissa bits, no infinities, max 448). Scale exponent =
# floor(log2(amax of the block)) - 8 (8 = the largest E4M3 exponent), elements = the block /
# 2^exponent rounded to nearest-even E4M3, saturating at +-448. An all-zero block gets the
# smallest scale, 2^-127 (E8M0 code 0).

MX_BLOCK = 32
E4M3_MAX = 448.0


def e4m3_values() -> np.ndarray:
    """The 256 E4M3 codes as float64 (NaN for the two NaN codes 0x7F, 0xFF)."""
    c = np.arange(256)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 7
    v = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * 2.0 ** (e - 7.0))
    v = np.where((e == 15) & (m == 7), np.nan, v)
    return sign * v


def e4m3_encode(a) -> np.ndarray:
    """Round-to-nearest-even E4M3 codes of float64 values, saturating at +-448 (NaN input ->
    NaN code 0x7F). The sign of zero is kept."""
    a = np.asarray(a, np.float64)
    mag = np.minimum(np.abs(a), E4M3_MAX)
    # exponent of the E4M3 binade (subnormals share the spacing of the smallest normal binade)
    with np.errstate(divide="ignore"):
        ex = np.floor(np.log2(np.where(mag > 0, mag, 1.0)))
    ex = np.clip(ex, -6, 8)
    step = 2.0 ** (ex - 3)                      # spacing of 3 mantissa bits in that binade
    q = mag / step                              # exact: power-of-two division
    r = np.floor(q)
    frac = q - r
    r = np.where((frac > 0.5) | ((frac == 0.5) & (r % 2 == 1)), r + 1, r)
    val = r * step                              # the rounded magnitude, on the E4M3 grid
    # back to a code: biased exponent and mantissa of val
    with np.errstate(divide="ignore"):
        vex = np.floor(np.log2(np.where(val > 0, val, 1.0)))
    normal = val >= 2.0 ** -6
    code = np.where(normal, ((vex + 7).astype(np.int64) << 3) | ((val / 2.0 ** vex - 1.0) * 8).astype(np.int64),
                    (val / 2.0 ** -9).astype(np.int64))
    code = np.where(val == 0, 0, code)
    code = code | np.where(np.signbit(a), 0x80, 0)
    return np.where(np.isnan(a), 0x7F, code).astype(np.uint8)


def mx_quantize(v, block: int = MX_BLOCK):
    """MX quantisation of v (..., K) along its last axis (K a multiple of `block`). Returns
    (codes uint8 (..., K), scale codes uint8 (..., K/block)) with scale = 2^(code - 127)."""
    v = np.asarray(v, np.float64)
    *lead, K = v.shape
    b = v.reshape(*lead, K // block, block)
    amax = np.abs(b).max(axis=-1)
    with np.errstate(divide="ignore"):
        ex = np.floor(np.log2(np.where(amax > 0, amax, 1.0))) - 8.0
    scode = np.where(amax > 0, np.clip(ex + 127.0, 0, 254), 0).astype(np.int64)
    codes = e4m3_encode(b / (2.0 ** (scode - 127.0))[..., None])
    return codes.reshape(*lead, K), scode.astype(np.uint8)


def mx_dequantize(codes, scales, block: int = MX_BLOCK) -> np.ndarray:
    """Values of MX-quantised data: e4m3(code) * 2^(scale - 127), float64."""
    codes = np.asarray(codes)
    *lead, K = codes.shape
    vals = e4m3_values()[codes].reshape(*lead, K // block, block)
    return (vals * (2.0 ** (np.asarray(scales, np.float64) - 127.0))[..., None]).reshape(*lead, K)


def mx_round(v, block: int = MX_BLOCK) -> np.ndarray:
    """v as it is after MX quantisation (quantise, then dequantise)."""
    return mx_dequantize(*mx_quantize(v, block), block)


def expert_mlp_mxfp8(cfg: "MoEConfig", z_rows, w1_e, w2_e) -> np.ndarray:
    """One expert's SwiGLU MLP with both matmuls in MXFP8 ([OC3 "Rowwise FP8 и MXFP8"], [OC3
    "SwiGLU с квантизацией"]: the SwiGLU step yields the activation and its quantised form).
    The operands are MX-quantised along the contraction dimension (z rows and W1 rows along K,
    the activation rows and W2 rows along h); the products and sums are exact (float64); the
    activation is stored in the layer dtype before it is quantised; the output is bf16."""
    h = cfg.hidden_size
    H = mx_round(z_rows) @ mx_round(w1_e).T
    up, gate = H[:, :h], H[:, h:]
    with np.errstate(over="ignore"):
        act = round_to(up * gate / (1.0 + np.exp(-gate)), cfg.dtype)
    return round_to(mx_round(act) @ mx_round(w2_e).T, cfg.dtype)


# ---------------------------------------------------------------------- experts

def prepare_routed_input(cfg: MoEConfig, x, down_proj=None, acc=np.float64) -> np.ndarray:
    """[OC3 "Латентная проекция экспертов"]: without a latent projection the experts get the
    input unchanged; with one, a down-projection maps (*, d_model) to (*, latent_dim). The
    result is stored in the layer dtype."""
    if not cfg.latent_dim:
        return _f64(x)
    return round_to(_acc(x, acc) @ _acc(down_proj, acc).T, cfg.dtype)


def expert_mlp(cfg: MoEConfig, z_rows, w1_e, w2_e, acc=np.float64) -> np.ndarray:
    """One expert's SwiGLU MLP on its rows.

    [OC3 "Как задаётся конфигурация MoE"]: up_factor is 2 for swiglu, so the first matrix
    has 2*hidden_size output rows. [OC3 "SwiGLU с квантизацией"]: the last dimension is split
    in halves, first `up` then `gate`, and the activation is up * gate * sigmoid(gate) in
    fp32 precision or better (float64 here), stored in the layer dtype. [OC3 "Вычисления
    экспертов и точность"]: the grouped experts return bf16 (fp32 for an fp32 layer).
    Weights are (2h, K) and (K, h), out x in."""
    h = cfg.hidden_size
    H = _acc(z_rows, acc) @ _acc(w1_e, acc).T
    up, gate = H[:, :h], H[:, h:]
    with np.errstate(over="ignore"):
        act = round_to(up * gate / (1.0 + np.exp(-gate)), cfg.dtype)
    return round_to(_acc(act, acc) @ _acc(w2_e, acc).T, cfg.dtype)


def run_experts(cfg: MoEConfig, z, idx, w1, w2, capacity: Optional[int] = None, acc=np.float64) -> dict:
    """[OC3 "Вычисления экспертов и точность"]: group the permuted tokens by expert, run each
    expert's MLP, and return the results; Y is kept in sorted (permuted) order here.
    w1/w2 may be arrays (E, ...) or mappings expert -> array (only touched experts needed).
    With a capacity ([OC3 "Ёмкость эксперта и переполнение"]) only the kept assignments run;
    the rows of dropped assignments (after the kept ones in perm) stay 0. counts are the
    router's counts before any drop; offsets delimit the kept rows of each expert."""
    k = cfg.top_k
    counts = expert_counts(idx, cfg.num_experts)
    kept_counts = counts if capacity is None else np.minimum(counts, capacity)
    offsets = expert_offsets(kept_counts)
    perm, inv, kept = capacity_permutation(idx, cfg.num_experts, capacity)
    z_perm = _acc(z, acc)[perm // k]
    Y = np.zeros((perm.size, z_perm.shape[1]), dtype=acc)  # holds layer-dtype values: exact in fp32 too
    for e in np.nonzero(kept_counts)[0]:
        rows = slice(offsets[e], offsets[e + 1])
        if cfg.expert_precision == "mxfp8":
            Y[rows] = expert_mlp_mxfp8(cfg, z_perm[rows], w1[e], w2[e])
        else:
            Y[rows] = expert_mlp(cfg, z_perm[rows], w1[e], w2[e], acc)
    return dict(counts=counts, offsets=offsets, perm=perm, inv=inv, kept=kept, z_perm=z_perm, Y=Y)


def combine(cfg: MoEConfig, Y, inv, w) -> np.ndarray:
    """Unpermute and weight. [OC3 "Пересылка токенов между экспертами"]: results go back to
    the original positions by a scatter with the saved indices. The router's weights have no
    other consumer, so each token's k results are scaled by its weights and summed
    (o[t] = sum_j w[t,j] * Y[inv[t*k+j]], j ascending)."""
    k = cfg.top_k
    w = _f64(w)
    T = w.shape[0]
    inv = np.asarray(inv).reshape(T, k)
    o = np.zeros((T, Y.shape[1]))
    for j in range(k):
        o += w[:, j:j + 1] * Y[inv[:, j]]
    return o


def restore_routed_output(cfg: MoEConfig, o, norm_weight=None, up_proj=None) -> dict:
    """[OC3 "Латентная проекция экспертов"]: without an up-projection the expert output is
    returned as is; with one it is normalised (bias-free RMSNorm unless configured off),
    cast to the up-projection weight's dtype and multiplied by it, giving (*, d_model).
    [OC3 "Вычисления экспертов и точность"]: the cast before the dense up-projection.
    RMSNorm: n = o / sqrt(mean(o**2) + eps) * g."""
    o = _f64(o)
    if not cfg.latent_dim:
        return dict(n=None, y=o)
    if cfg.up_proj_input_norm:
        g = np.ones(o.shape[1]) if norm_weight is None else _f64(norm_weight)
        n = o / np.sqrt((o * o).mean(axis=-1, keepdims=True) + cfg.up_proj_input_norm_eps) * g
    else:
        n = o
    n = round_to(n, cfg.dtype)
    return dict(n=n, y=n @ _f64(up_proj).T)


def forward(cfg: MoEConfig, weights: dict, x, acc=np.float64) -> dict:
    """The whole layer, step by step. `weights` holds numpy arrays (bf16 values as float32):
    router_weight (E,d), router_bias (E)|None, score_bias (E)|None, down_proj (L,d)|None,
    norm_weight (L)|None, up_proj (d,L)|None, w1 (E,2h,K) or {e: (2h,K)}, w2 (E,K,h) or
    {e: (K,h)}. The final y is returned unrounded (float64). acc = np.float32 sums the
    contractions (router, latent down, expert matmuls) in fp32 instead of float64: the mode
    the CPU timing runs in; every rounding point stays where it is."""
    out = {}
    logits = router_logits(x, weights["router_weight"], weights.get("router_bias"), acc)
    out.update(route(cfg, logits, weights.get("score_bias")))
    z = prepare_routed_input(cfg, x, weights.get("down_proj"), acc)
    out["z"] = z
    out["capacity"] = expert_capacity(cfg, np.asarray(x).shape[0])
    out.update(run_experts(cfg, z, out["idx"], weights["w1"], weights["w2"], out["capacity"], acc))
    o = combine(cfg, out["Y"], out["inv"], out["w"])
    out["o"] = o
    out.update(restore_routed_output(cfg, o, weights.get("norm_weight"), weights.get("up_proj")))
    return out


# ------------------------------------------------------------------- backward (experts)

def expert_mlp_train(cfg: MoEConfig, z_rows, w1_e, w2_e) -> dict:
    """One expert's SwiGLU MLP as the training forward runs it: the same H, act and Y as
    expert_mlp, plus what the backward reads. [OC3 "SwiGLU с квантизацией"]: the activation
    function keeps its input for the backward when that input needs a gradient; that input is
    H, stored in the layer dtype like every tensor that leaves a matmul here. act is computed
    from the unrounded H, as in the inference forward, and stored in the layer dtype."""
    h = cfg.hidden_size
    H = _f64(z_rows) @ _f64(w1_e).T
    up, gate = H[:, :h], H[:, h:]
    with np.errstate(over="ignore"):
        act = round_to(up * gate / (1.0 + np.exp(-gate)), cfg.dtype)
    Y = round_to(act @ _f64(w2_e).T, cfg.dtype)
    return dict(H=round_to(H, cfg.dtype), act=act, Y=Y)


def run_experts_train(cfg: MoEConfig, z, idx, w1, w2, capacity: Optional[int] = None) -> dict:
    """run_experts with the saved tensors of the training forward: H (A, 2h) and act (A, h)
    in sorted order, rows of dropped assignments 0."""
    k = cfg.top_k
    counts = expert_counts(idx, cfg.num_experts)
    kept_counts = counts if capacity is None else np.minimum(counts, capacity)
    offsets = expert_offsets(kept_counts)
    perm, inv, kept = capacity_permutation(idx, cfg.num_experts, capacity)
    z_perm = _f64(z)[perm // k]
    A, h = perm.size, cfg.hidden_size
    Y = np.zeros((A, z_perm.shape[1]))
    H = np.zeros((A, 2 * h))
    act = np.zeros((A, h))
    for e in np.nonzero(kept_counts)[0]:
        rows = slice(offsets[e], offsets[e + 1])
        r = expert_mlp_train(cfg, z_perm[rows], w1[e], w2[e])
        H[rows], act[rows], Y[rows] = r["H"], r["act"], r["Y"]
    return dict(counts=counts, offsets=offsets, perm=perm, inv=inv, kept=kept, z_perm=z_perm,
                H=H, act=act, Y=Y)


def swiglu_backward(cfg: MoEConfig, H, d_act) -> np.ndarray:
    """[OC3 "SwiGLU с квантизацией"], the plain backward: the last dimension of the saved
    input splits in halves, up then gate; sigmoid(gate), silu = gate * sigmoid(gate), its
    derivative sigmoid(gate) * (1 + gate * (1 - sigmoid(gate))) and the two gradients
    d_up = d_act * silu and d_gate = d_act * up * silu' are formed in fp32 or better (float64
    here) and concatenated back, [d_up | d_gate], in the layer dtype."""
    h = cfg.hidden_size
    H = _f64(H)
    up, gate = H[:, :h], H[:, h:]
    with np.errstate(over="ignore"):
        sig = 1.0 / (1.0 + np.exp(-gate))
    silu = gate * sig
    dsilu = sig * (1.0 + gate * (1.0 - sig))
    d_act = _f64(d_act)
    return round_to(np.concatenate([d_act * silu, d_act * up * dsilu], axis=1), cfg.dtype)


def experts_backward(cfg: MoEConfig, z, idx, w1, w2, saved: dict, dY_assign,
                     capacity: Optional[int] = None) -> dict:
    """Gradients of the routed experts stage: the input of the stage is z (T, K) and its
    output the per-assignment rows Y (A, K) in assignment order t*k+j; given dY_assign (the
    gradient of those rows) this returns dz (T, K), dw1 (E, 2h, K) and dw2 (E, K, h).

    [OC3 "Вычисления экспертов и точность"]: each expert's rows go through a grouped matmul,
    so each expert's gradients come from its own rows only. Per expert e on its kept rows R
    (sorted order), with the saved H and act of the training forward:
      d_act   = dY[R] @ w2[e]            (the grad of act @ w2[e]^T), stored in the layer dtype;
      dH      = swiglu_backward(H[R], d_act)   ([OC3 "SwiGLU с квантизацией"]);
      dz_perm = dH @ w1[e]               (the grad of z_perm @ w1[e]^T), layer dtype;
      dw2[e]  = dY[R]^T @ act[R],  dw1[e] = dH^T @ z_perm[R], layer dtype (0 without rows).
    [OC3 "Пересылка токенов между экспертами"]: z_perm is z gathered by perm // k, so the
    gradient of z sums its k copies: dz[t] = sum_j dz_perm[inv[t*k+j]], summed in float64 and
    stored once in the layer dtype (reading: one rounding after the sum). Dropped assignments
    ([OC3 "Ёмкость эксперта и переполнение"]) produced 0 and pass no gradient."""
    k = cfg.top_k
    E, h = cfg.num_experts, cfg.hidden_size
    counts = expert_counts(idx, E)
    kept_counts = counts if capacity is None else np.minimum(counts, capacity)
    offsets = expert_offsets(kept_counts)
    perm, inv, kept = capacity_permutation(idx, E, capacity)
    z = _f64(z)
    T, K = z.shape
    z_perm = z[perm // k]
    dY = _f64(dY_assign)[perm]          # sorted order
    dz_perm = np.zeros((perm.size, K))
    dH_all = np.zeros((perm.size, 2 * h))
    dw1 = np.zeros((E, 2 * h, K))
    dw2 = np.zeros((E, K, h))
    for e in np.nonzero(kept_counts)[0]:
        R = slice(offsets[e], offsets[e + 1])
        d_act = round_to(dY[R] @ _f64(w2[e]), cfg.dtype)
        dH = swiglu_backward(cfg, saved["H"][R], d_act)
        dH_all[R] = dH
        dz_perm[R] = round_to(dH @ _f64(w1[e]), cfg.dtype)
        dw2[e] = round_to(dY[R].T @ _f64(saved["act"][R]), cfg.dtype)
        dw1[e] = round_to(dH.T @ z_perm[R], cfg.dtype)
    dz = np.zeros((T, K))
    inv2 = np.asarray(inv).reshape(T, k)
    for j in range(k):
        dz += dz_perm[inv2[:, j]]
    return dict(dz=round_to(dz, cfg.dtype), dw1=dw1, dw2=dw2, dH=dH_all, dz_perm=dz_perm,
                offsets=offsets, perm=perm, inv=inv)


def combine_backward(cfg: MoEConfig, Y_assign, w, d_o) -> dict:
    """Gradients of the weighted combine o[t] = sum_j w[t,j] * Y[t*k+j] ([OC3 "Пересылка
    токенов между экспертами"]) with Y in assignment order: dY[t*k+j] = w[t,j] * d_o[t],
    stored in the layer dtype (Y's), and dw[t,j] = sum_c d_o[t,c] * Y[t*k+j, c], rounded
    to fp32 (the routing weights are fp32)."""
    k = cfg.top_k
    w = _f64(w)
    T = w.shape[0]
    d_o = _f64(d_o)
    Y = _f64(Y_assign).reshape(T, k, -1)
    dY = round_to(w[:, :, None] * d_o[:, None, :], cfg.dtype).reshape(T * k, -1)
    dw = round_f32(np.einsum("tc,tjc->tj", d_o, Y))
    return dict(dY=dY, dw=dw)


# ------------------------------------------------------------------- balancing state

def accumulate_counts(accumulator, counts) -> np.ndarray:
    """[OC3 "Счётчики и bias-корректировка"]: score_bias_batch_size_per_expert accumulates
    the number of tokens assigned to each expert over the step's forward passes (it is summed
    into, then reset after the step). Integer add."""
    return np.asarray(accumulator, dtype=np.int64) + np.asarray(counts, dtype=np.int64)


def load_imbalance(counts) -> float:
    """[OC3 "Счётчики и bias-корректировка"]: the load imbalance metric is the maximum of the
    per-expert counter divided by its mean. mean = total / E, so the ratio is max * E / total,
    formed as one float64 division of the two exact integers (correctly rounded). With no
    tokens the mean is 0 and the ratio 0/0: NaN. The cross-process aggregations the page
    names (max for the local metric, mean for the global one) combine values of this same
    function."""
    c = np.asarray(counts, dtype=np.int64)
    total = int(c.sum())
    if total == 0:
        return float("nan")
    return float(int(c.max()) * c.size) / float(total)


def score_bias_update(score_bias, accumulator, bias_gamma: float) -> np.ndarray:
    """[OC3 "Счётчики и bias-корректировка"] and [OC3 "Управление состоянием между шагами"]:
    after the step, the ideal mean size per expert is computed from the accumulated counts,
    score_bias moves by bias_gamma * sign(ideal - actual), and the accumulator is reset (the
    caller's job here). ideal = total / E; the sign is taken exactly, as sign(total - E *
    actual) in integers. The move is one fp32 add of +-bias_gamma or 0 to the fp32 bias."""
    c = np.asarray(accumulator, dtype=np.int64)
    sgn = np.sign(int(c.sum()) - c.size * c).astype(np.float32)
    step = np.float32(bias_gamma) * sgn
    return (np.asarray(score_bias, dtype=np.float32) + step).astype(np.float32)


# ------------------------------------------------------------------- parameter counts

def num_params(cfg: MoEConfig) -> dict:
    """[OC3 "Как задаётся конфигурация MoE"]: the latent dimension is d_model when there is no
    latent MoE; total = router params + 3*latent_dim*hidden_size*num_experts (+ shared
    modules, none here); active = total - 3*latent_dim*hidden_size*num_experts +
    3*latent_dim*hidden_size*top_k. Router = d_model*num_experts (+num_experts with bias);
    per expert (up_factor + 1)*dim*hidden_size with up_factor = 2 for swiglu, experts being
    built with d_model = latent_dim. The latent projections and norm weight are not in the
    page's formula; they are reported separately as `latent_extra`."""
    L = cfg.latent_dim if cfg.latent_dim else cfg.d_model
    router = cfg.d_model * cfg.num_experts + (cfg.num_experts if cfg.router_bias else 0)
    up_factor = 2
    experts = (up_factor + 1) * L * cfg.hidden_size * cfg.num_experts
    total = router + experts
    active = total - 3 * L * cfg.hidden_size * cfg.num_experts + 3 * L * cfg.hidden_size * cfg.top_k
    extra = 0
    if cfg.latent_dim:
        extra = 2 * cfg.d_model * cfg.latent_dim + (cfg.latent_dim if cfg.up_proj_input_norm else 0)
    return dict(total=total, active=active, latent_extra=extra)
