"""Synthetic workloads for the routed Mixture-of-Experts layer forward pass.

This module holds the five layer shapes the path is measured and checked on, and the seeded
generators that draw their inputs. It contains none of the layer's arithmetic: only shape
tables and random draws (a normal draw scaled by a standard deviation, rounded to the storage
dtype). Both sides of every parity check -- the CPU oracle and the HIP path -- receive the
same generated values; neither side generates anything itself.

Sources: the layer fields mirror the configuration objects described on the page
"Как устроен Olmo-core 3: обучение больших MoE-моделей" (section "Как задаётся конфигурация
MoE" for MoEConfig / MoERouterConfigV2, section "Латентная проекция экспертов" for
LatentMoEConfig). The 896-expert latent shapes follow the scale given on "Architecting
Trillion-Scale Sparse Multimodal Models" (section 1, overall architecture). The pages print
no workload tensors, so every value here is synthetic.

Seeding: every tensor (and every expert's slice of an expert tensor) has its own torch
generator, seeded from numpy's SeedSequence([seed, config_id, tensor_id, expert_id]). Values
depend on the device the draw runs on (torch's CPU and GPU generators differ); each is
deterministic. Small parity cases draw on the CPU and copy to the GPU; full-size cases draw on
the GPU and copy the slices the oracle needs back to the host.
"""
from __future__ import annotations

import math

import numpy as np
import torch

# Layer fields (names as on the page's config objects) + workload fields (tokens, init recipe).
_LAYER_DEFAULTS = dict(
    d_model=None,
    num_experts=1,
    top_k=1,
    hidden_size=256,
    gating_function="softmax",
    sigmoid_stability_epsilon=None,
    normalize_expert_weights=None,
    restore_weight_scale=False,
    expert_weight_scale=None,
    original_top_k=None,
    router_bias=False,
    latent_dim=None,
    up_proj_input_norm=True,
    up_proj_input_norm_eps=1e-5,
    dtype="bf16",
    capacity_factor=None,
    expert_precision="bf16",
)

LAYER_FIELDS = tuple(_LAYER_DEFAULTS)

CONFIGS = {
    # Tiny, fp32 everywhere; weights N(0, 1/fan_in) (variance), inputs N(0, 1).
    "tiny_f32": dict(
        config_id=1, tokens=256, d_model=256, num_experts=8, top_k=2, hidden_size=128,
        gating_function="softmax", dtype="f32", init="fan_in", score_bias=None,
    ),
    # OlmoE-shaped: 64 experts, top-8, L1-normalised softmax weights; bf16, fp32 router.
    "olmoe": dict(
        config_id=2, tokens=8192, d_model=2048, num_experts=64, top_k=8, hidden_size=1024,
        gating_function="softmax", normalize_expert_weights=1.0, dtype="bf16",
        init="std0.02", score_bias=None,
    ),
    # Ultra-sparse latent layer: 896 experts in a 1024-wide latent space, sigmoid + eps gating,
    # score_bias ~ N(0, 0.1).
    "latent896": dict(
        config_id=3, tokens=16384, d_model=4096, latent_dim=1024, num_experts=896, top_k=8,
        hidden_size=512, gating_function="sigmoid", sigmoid_stability_epsilon=1e-6,
        dtype="bf16", init="std0.02", score_bias="normal0.1",
    ),
    # Skewed load: score_bias_e = 2*ln(1/(e+1)) concentrates tokens on the lowest experts.
    "skewed": dict(
        config_id=4, tokens=32768, d_model=4096, num_experts=256, top_k=8, hidden_size=2048,
        gating_function="sigmoid", dtype="bf16", init="std0.02", score_bias="zipf2",
    ),
    # Decode-shaped: 64 tokens against 896 latent experts (weight streaming).
    "decode": dict(
        config_id=5, tokens=64, d_model=4096, latent_dim=1024, num_experts=896, top_k=8,
        hidden_size=512, gating_function="topk_softmax", dtype="bf16", init="std0.02",
        score_bias=None,
    ),
}

CONFIG_ORDER = ("tiny_f32", "olmoe", "latent896", "skewed", "decode")

_TENSOR_IDS = dict(x=0, router_weight=1, router_bias=2, score_bias=3, down_proj=4,
                   up_proj=5, norm_weight=6, w1=7, w2=8, scores=9, indices=10, y=11,
                   weights=12)


def layer_config(name: str, **overrides) -> dict:
    """The layer fields of workload `name` (no token count), with overrides applied."""
    spec = dict(CONFIGS[name])
    spec.update(overrides)
    return {f: spec.get(f, _LAYER_DEFAULTS[f]) for f in LAYER_FIELDS}


def tokens_of(name: str) -> int:
    return CONFIGS[name]["tokens"]


def seed_of(seed: int, config_id: int, tensor: str, expert: int = 0) -> int:
    ss = np.random.SeedSequence([seed, config_id, _TENSOR_IDS[tensor], expert])
    return int(ss.generate_state(1, dtype=np.uint64)[0] & ((1 << 63) - 1))


def _gen(device, seed):
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def _normal(shape, std, device, seed, dtype):
    g = _gen(device, seed)
    t = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    if std != 1.0:
        t.mul_(std)
    return t.to(dtype)


def storage_dtype(cfg: dict) -> torch.dtype:
    return torch.float32 if cfg["dtype"] == "f32" else torch.bfloat16


def make_workload(name: str, tokens: int | None = None, device="cpu", seed: int = 0,
                  **overrides):
    """Draw x and all weights for workload `name`.

    Returns (cfg, weights, x): cfg = layer fields (dict), weights = dict of torch tensors on
    `device`, x = (tokens, d_model) tensor in the layer dtype. Shape overrides (d_model,
    num_experts, ...) give reduced cases with the same init recipe.
    """
    spec = dict(CONFIGS[name])
    spec.update(overrides)
    cfg = layer_config(name, **overrides)
    cid = spec["config_id"]
    T = spec["tokens"] if tokens is None else int(tokens)
    d, E, h = cfg["d_model"], cfg["num_experts"], cfg["hidden_size"]
    L = cfg["latent_dim"]
    K = L if L else d
    D = storage_dtype(cfg)
    init = spec["init"]

    def std_for(fan_in):
        return 1.0 / math.sqrt(fan_in) if init == "fan_in" else 0.02

    w = {}
    x = _normal((T, d), 1.0, device, seed_of(seed, cid, "x"), D)
    w["router_weight"] = _normal((E, d), std_for(d), device, seed_of(seed, cid, "router_weight"),
                                 torch.float32)
    w["router_bias"] = (_normal((E,), std_for(d), device, seed_of(seed, cid, "router_bias"),
                                torch.float32) if cfg["router_bias"] else None)
    sb = spec.get("score_bias")
    if sb is None:
        w["score_bias"] = None
    elif sb == "normal0.1":
        w["score_bias"] = _normal((E,), 0.1, device, seed_of(seed, cid, "score_bias"),
                                  torch.float32)
    elif sb == "zipf2":
        # score_bias_e = 2 * ln(1 / (e + 1)), evaluated in float64 and stored as float32.
        e = np.arange(E, dtype=np.float64)
        w["score_bias"] = torch.tensor(2.0 * np.log(1.0 / (e + 1.0)), dtype=torch.float32,
                                       device=device)
    else:
        raise ValueError(f"unknown score_bias recipe {sb!r}")
    if L:
        w["down_proj"] = _normal((L, d), std_for(d), device, seed_of(seed, cid, "down_proj"), D)
        w["up_proj"] = _normal((d, L), std_for(L), device, seed_of(seed, cid, "up_proj"), D)
        w["norm_weight"] = torch.ones((L,), dtype=torch.float32, device=device)
    else:
        w["down_proj"] = w["up_proj"] = w["norm_weight"] = None
    w1 = torch.empty((E, 2 * h, K), dtype=D, device=device)
    w2 = torch.empty((E, K, h), dtype=D, device=device)
    for e in range(E):
        w1[e] = _normal((2 * h, K), std_for(K), device, seed_of(seed, cid, "w1", e), D)
        w2[e] = _normal((K, h), std_for(h), device, seed_of(seed, cid, "w2", e), D)
    w["w1"], w["w2"] = w1, w2
    return cfg, w, x


def to_numpy_f32(t):
    """Host float32 copy of a tensor (bf16 values are exact in float32); None passes through."""
    if t is None:
        return None
    return t.detach().to("cpu", torch.float32).numpy()


def synthetic_scores(T: int, E: int, kind: str, device="cpu", seed: int = 0) -> torch.Tensor:
    """A (T, E) float32 score/logit matrix for the routing-only checks.

    kind: "normal" -- N(0, 1); "ties" -- values on a coarse grid {-2, -1.75, ..., 2} so that
    equal keys are frequent, with some exact +0.0 / -0.0 pairs; "nan" -- "ties" plus NaN
    entries in a few rows.
    """
    g = _gen(device, seed_of(seed, 0, "scores", T * 1024 + E))
    s = torch.randn((T, E), generator=g, device=device, dtype=torch.float32)
    if kind == "normal":
        return s
    s = torch.clamp(torch.round(s * 4.0) / 4.0, -2.0, 2.0)
    zero = s == 0
    flip = torch.rand((T, E), generator=g, device=device) < 0.5
    s = torch.where(zero & flip, torch.full_like(s, -0.0), s)
    if kind == "ties":
        return s
    if kind == "nan":
        m = torch.rand((T, E), generator=g, device=device) < 0.05
        return torch.where(m, torch.full_like(s, float("nan")), s)
    raise ValueError(kind)


def random_distinct_indices(T: int, E: int, k: int, device="cpu", seed: int = 0,
                            skew: float = 0.0) -> torch.Tensor:
    """(T, k) int32 expert indices, distinct within each row, drawn at random.

    skew > 0 tilts the draw towards low expert indices (probability ~ (e+1)^-skew).
    """
    g = _gen(device, seed_of(seed, 0, "indices", T * 4096 + E * 16 + k))
    u = torch.rand((T, E), generator=g, device=device, dtype=torch.float64)
    key = torch.log(u)  # Gumbel-top-k style: argsort of log(u)/p picks without replacement
    if skew:
        p = torch.arange(1, E + 1, device=device, dtype=torch.float64) ** (-skew)
        key = key / p
    return torch.topk(key, k, dim=1).indices.to(torch.int32)


def synthetic_counts(num_experts: int, kind: str, seed: int = 0, total: int = 65536) -> np.ndarray:
    """Per-expert token counts (int64) for the balancing-state checks: 'uniform' (all equal,
    total rounded down to a multiple of E), 'hot' (all tokens on expert E // 2), 'zipf'
    (counts proportional to 1/(e+1), rounded down), 'random' (uniform integers in
    [0, 2*total/E]), 'sparse' (random with about half the experts at zero), 'zero'."""
    E = num_experts
    rng = np.random.default_rng(np.random.SeedSequence([seed, E, len(kind)]))
    if kind == "uniform":
        return np.full(E, total // E, dtype=np.int64)
    if kind == "hot":
        c = np.zeros(E, dtype=np.int64)
        c[E // 2] = total
        return c
    if kind == "zipf":
        return np.floor(total / (np.arange(E) + 1.0) / np.sum(1.0 / (np.arange(E) + 1.0))).astype(np.int64)
    if kind == "random":
        return rng.integers(0, 2 * max(total // E, 1) + 1, size=E).astype(np.int64)
    if kind == "sparse":
        c = rng.integers(0, 2 * max(total // E, 1) + 1, size=E).astype(np.int64)
        c[rng.random(E) < 0.5] = 0
        return c
    if kind == "zero":
        return np.zeros(E, dtype=np.int64)
    raise ValueError(kind)
