"""Pins of the CPU oracle to facts that do not come from the oracle itself.

Each test names what fixes the expected value: a closed form derived from the page
"Как устроен Olmo-core 3: обучение больших MoE-моделей" (golden fixtures under
tests/golden/), a library routine (torch's softmax / sigmoid / silu / rms_norm / bf16 cast,
Python's sort, math.fsum), brute force over all subsets, or an invariant of the method.
CPU only.
"""
import dataclasses
import itertools
import json
import math
import os

import numpy as np
import pytest
import torch

import workloads
from oracle import moe_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def cfg_of(**kw):
    base = dict(d_model=64, num_experts=4, top_k=2, hidden_size=32, dtype="f32")
    base.update(kw)
    return O.MoEConfig(**base)


def small_workload(name, T, **over):
    cfg, w, x = workloads.make_workload(name, tokens=T, device="cpu", **over)
    wn = {k: workloads.to_numpy_f32(v) for k, v in w.items()}
    return O.MoEConfig.from_dict(cfg), wn, workloads.to_numpy_f32(x)


# ------------------------------------------------------------------ parameter counts

def _golden_params():
    rows = {}
    with open(os.path.join(GOLDEN, "param_counts.txt")) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            p = line.split()
            rows[p[0]] = tuple(int(v) for v in p[1:4])
    return rows


@pytest.mark.parametrize("name", workloads.CONFIG_ORDER)
def test_param_counts_golden(name):
    cfg = O.MoEConfig.from_dict(workloads.layer_config(name))
    got = O.num_params(cfg)
    assert (got["total"], got["active"], got["latent_extra"]) == _golden_params()[name]


@pytest.mark.parametrize("name,over", [
    ("tiny_f32", {}),
    ("olmoe", dict(d_model=128, hidden_size=64, num_experts=6, top_k=3)),
    ("latent896", dict(d_model=128, latent_dim=64, hidden_size=32, num_experts=10, top_k=4)),
])
def test_param_counts_equal_generated_tensor_sizes(name, over):
    """Count the elements of the tensors a layer actually holds: router weight plus every
    expert's two matrices; active = router plus top_k experts' matrices."""
    cfg, w, _ = workloads.make_workload(name, tokens=4, **over)
    c = O.MoEConfig.from_dict(cfg)
    per_expert = w["w1"][0].numel() + w["w2"][0].numel()
    total = w["router_weight"].numel() + w["w1"].numel() + w["w2"].numel()
    active = w["router_weight"].numel() + c.top_k * per_expert
    got = O.num_params(c)
    assert got["total"] == total and got["active"] == active
    if c.latent_dim:
        assert got["latent_extra"] == (w["down_proj"].numel() + w["up_proj"].numel()
                                       + w["norm_weight"].numel())


# ------------------------------------------------------------------ rounding and logits

def test_round_bf16_matches_torch_cast():
    g = np.random.default_rng(1)
    a = np.concatenate([g.standard_normal(200000).astype(np.float32),
                        g.standard_normal(1000).astype(np.float32) * 1e-30,
                        g.standard_normal(1000).astype(np.float32) * 1e30])
    # exact ties between two bf16 neighbours
    ties = (g.integers(1 << 15, 1 << 16, 5000).astype(np.uint32) << 16) | 0x8000
    a = np.concatenate([a, ties.view(np.float32)])
    a = a[np.isfinite(a)]
    ref = torch.from_numpy(a).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(O.round_bf16(a), ref)


def test_logits_exactly_rounded_dot():
    """fp32 x fp32 products are exact in float64; math.fsum returns the correctly rounded sum,
    so round_f32(fsum) is the exactly rounded logit. The oracle's float64 BLAS sum may differ
    only below float64 resolution: at most one fp32 ulp, and almost never."""
    cfg, w, x = small_workload("tiny_f32", 16)
    got = O.router_logits(x, w["router_weight"])
    W = w["router_weight"].astype(np.float64)
    ref = np.array([[np.float32(math.fsum(x[t].astype(np.float64) * W[e]))
                     for e in range(W.shape[0])] for t in range(x.shape[0])], dtype=np.float64)
    ulps = np.abs(got.astype(np.float32).view(np.int32) - ref.astype(np.float32).view(np.int32))
    assert ulps.max() <= 1 and (ulps == 0).mean() > 0.99


def test_logits_bias_added():
    cfg, w, x = small_workload("tiny_f32", 8)
    b = np.linspace(-1, 1, w["router_weight"].shape[0]).astype(np.float32)
    d = O.router_logits(x, w["router_weight"], b) - O.router_logits(x, w["router_weight"])
    assert np.allclose(d, b[None, :], atol=1e-5)


# ------------------------------------------------------------------ gating

def test_softmax_gating_matches_torch():
    g = np.random.default_rng(2)
    l = O.round_f32(g.standard_normal((64, 37)) * 3)
    got = O.gating_scores(cfg_of(gating_function="softmax", num_experts=37), l)
    ref = torch.softmax(torch.from_numpy(l), dim=-1).numpy()
    assert np.allclose(got, ref, rtol=2 ** -23, atol=0)
    assert np.allclose(got.sum(-1), 1.0, atol=37 * 2 ** -24)


def test_sigmoid_gating_matches_torch_and_eps():
    g = np.random.default_rng(3)
    l = O.round_f32(g.standard_normal((64, 19)) * 8)
    l[0, :3] = [-1e4, 1e4, 0.0]
    s = O.gating_scores(cfg_of(gating_function="sigmoid", num_experts=19), l)
    ref = torch.sigmoid(torch.from_numpy(l)).numpy()
    assert np.allclose(s, ref, rtol=2 ** -23, atol=0)
    se = O.gating_scores(cfg_of(gating_function="sigmoid", num_experts=19,
                                sigmoid_stability_epsilon=1e-6), l)
    eps32 = float(np.float32(1e-6))
    assert np.array_equal(se, (s.astype(np.float32) + np.float32(eps32)).astype(np.float64))
    assert se[0, 0] == np.float32(eps32)  # all-negative logit: score is exactly eps, not 0


# ------------------------------------------------------------------ top-k selection

def _valid_topk_set(keys, S):
    """Characterisation of the top-k set: every selected key ranks above every unselected key
    under (NaN last, larger first, lower index first at equal keys)."""
    def rank_above(a, b):
        ka, kb = keys[a], keys[b]
        if math.isnan(ka) or math.isnan(kb):
            if math.isnan(ka) and math.isnan(kb):
                return a < b
            return not math.isnan(ka)
        if ka != kb:
            return ka > kb
        return a < b
    return all(rank_above(a, b) for a in S for b in range(len(keys)) if b not in S)


@pytest.mark.parametrize("E", [4, 5, 6, 7, 8])
def test_select_topk_brute_force_all_subsets(E):
    g = np.random.default_rng(E)
    grid = np.array([-1.0, -0.5, -0.0, 0.0, 0.5, 1.0, np.nan])
    for trial in range(60):
        keys = g.choice(grid, size=E) if trial % 2 else g.standard_normal(E)
        for k in range(1, E + 1):
            valid = [set(S) for S in itertools.combinations(range(E), k)
                     if _valid_topk_set(keys, set(S))]
            assert len(valid) == 1
            got = O.select_topk(keys[None, :], k)[0]
            assert set(got.tolist()) == valid[0]
            # within the row: non-increasing keys, index ascending among equal keys
            order = sorted(range(E), key=lambda e: (math.isnan(keys[e]),
                                                    0.0 if math.isnan(keys[e]) else -keys[e], e))
            assert got.tolist() == order[:k]


def test_select_topk_matches_python_sort_wide():
    s = workloads.synthetic_scores(300, 64, "nan").numpy().astype(np.float64)
    got = O.select_topk(s, 8)
    for t in range(s.shape[0]):
        row = s[t]
        order = sorted(range(64), key=lambda e: (math.isnan(row[e]),
                                                 0.0 if math.isnan(row[e]) else -row[e], e))
        assert got[t].tolist() == order[:8]


def test_signed_zero_ties_go_to_lower_index():
    keys = np.array([[-0.0, 0.0, -1.0], [0.0, -0.0, -1.0]])
    assert O.select_topk(keys, 1)[:, 0].tolist() == [0, 0]


# ------------------------------------------------------------------ weights

def _golden_cases():
    with open(os.path.join(GOLDEN, "routing_closed_forms.jsonl")) as f:
        return [json.loads(line) for line in f if line.strip()]


def _num(v):
    if isinstance(v, str):
        sign = -1.0 if v.startswith("-") else 1.0
        return sign * math.log(float(v.lstrip("-")[2:]))
    return float(v)


@pytest.mark.parametrize("case", _golden_cases(), ids=lambda c: c["name"])
def test_routing_closed_forms(case):
    E = len(case["logits"])
    cfg = cfg_of(num_experts=E, **case["cfg"])
    logits = O.round_f32(np.array([[_num(v) for v in case["logits"]]]))
    bias = None if case["bias"] is None else np.array(case["bias"], dtype=np.float32)
    r = O.route(cfg, logits, bias)
    assert r["idx"][0].tolist() == case["idx"]
    assert np.allclose(r["w"][0], case["w"], rtol=case["tol"], atol=case["tol"])


def test_weight_invariants():
    s = workloads.synthetic_scores(500, 32, "normal").numpy()
    l = O.round_f32(s * 2)
    c1 = cfg_of(num_experts=32, top_k=6, gating_function="softmax", normalize_expert_weights=1.0)
    w1 = O.route(c1, l)["w"]
    assert np.all(np.abs(w1.sum(-1) - 1) <= 6 * 2 ** -23)
    c2 = cfg_of(num_experts=32, top_k=6, gating_function="topk_softmax")
    w2 = O.route(c2, l)["w"]
    assert np.all(np.abs(w2.sum(-1) - 1) <= 6 * 2 ** -23)
    c3 = cfg_of(num_experts=32, top_k=1, gating_function="topk_softmax")
    assert np.all(O.route(c3, l)["w"] == 1.0)
    c4 = cfg_of(num_experts=32, top_k=6, gating_function="softmax")
    w4 = O.route(c4, l)["w"]
    assert np.all((w4 > 0) & (w4 <= 1))
    eps = 1e-6
    c5 = cfg_of(num_experts=32, top_k=6, gating_function="sigmoid", sigmoid_stability_epsilon=eps)
    w5 = O.route(c5, l * 50)["w"]
    assert np.all((w5 >= np.float32(eps)) & (w5 <= 1 + eps))
    # weights are non-increasing along j for gathered scores without bias
    assert np.all(np.diff(w4, axis=-1) <= 0)


def test_topk_softmax_with_all_experts_equals_softmax():
    s = workloads.synthetic_scores(50, 12, "normal").numpy()
    l = O.round_f32(s)
    a = O.route(cfg_of(num_experts=12, top_k=12, gating_function="topk_softmax"), l)
    b = O.route(cfg_of(num_experts=12, top_k=12, gating_function="softmax"), l)
    assert np.array_equal(a["idx"], b["idx"])
    assert np.allclose(a["w"], b["w"], rtol=2 ** -22, atol=0)


# ------------------------------------------------------------------ histogram / permutation

def test_histogram_and_permutation_invariants():
    T, E, k = 777, 50, 6
    idx = workloads.random_distinct_indices(T, E, k, skew=1.2).numpy()
    counts = O.expert_counts(idx, E)
    offsets = O.expert_offsets(counts)
    perm, inv = O.stable_permutation(idx)
    A = T * k
    assert counts.sum() == A and offsets[-1] == A and np.all(np.diff(offsets) >= 0)
    assert sorted(perm.tolist()) == list(range(A))
    assert np.array_equal(inv[perm], np.arange(A))
    flat = idx.ravel()
    assert np.all(np.diff(flat[perm]) >= 0)
    for e in range(E):
        seg = perm[offsets[e]:offsets[e + 1]]
        assert np.all(flat[seg] == e) and np.all(np.diff(seg) > 0)
    # brute-force counting sort: visit experts in order, assignments in order
    brute = [a for e in range(E) for a in range(A) if flat[a] == e]
    assert perm.tolist() == brute
    for e in range(E):
        assert counts[e] == sum(1 for a in range(A) if flat[a] == e)


# ------------------------------------------------------------------ expert path

def _torch_swiglu_mlp(z, w1e, w2e, h, rnd):
    """Independent SwiGLU MLP: torch's silu, float64, rounding by torch's dtype casts."""
    H = torch.from_numpy(np.asarray(z, np.float64)) @ torch.from_numpy(np.asarray(w1e, np.float64)).T
    up, gate = H[:, :h], H[:, h:]
    act = rnd(up * torch.nn.functional.silu(gate))
    return rnd(act @ torch.from_numpy(np.asarray(w2e, np.float64)).T)


def _torch_round(dtype):
    td = torch.float32 if dtype == "f32" else torch.bfloat16
    return lambda t: t.to(td).to(torch.float64)


@pytest.mark.parametrize("name,over,rtol", [
    ("tiny_f32", dict(d_model=64, num_experts=6, top_k=3, hidden_size=32), 1e-6),
    ("olmoe", dict(d_model=64, num_experts=7, top_k=3, hidden_size=64), 2e-2),
    ("latent896", dict(d_model=128, latent_dim=64, num_experts=9, top_k=4, hidden_size=32), 2e-2),
])
def test_dense_bruteforce_equals_permuted_path(name, over, rtol):
    """Evaluate every expert on every token (no permutation), weight and sum; compare with the
    oracle's sort/group/scatter path. Pins the permutation, the unpermute and the combine."""
    T = 41
    cfg, w, x = small_workload(name, T, **over)
    out = O.forward(cfg, w, x)
    rnd = _torch_round(cfg.dtype)
    z = out["z"]
    K = z.shape[1]
    every = np.stack([_torch_swiglu_mlp(z, w["w1"][e], w["w2"][e], cfg.hidden_size, rnd).numpy()
                      for e in range(cfg.num_experts)])  # (E, T, K)
    o = np.zeros((T, K))
    for t in range(T):
        for j in range(cfg.top_k):
            o[t] += out["w"][t, j] * every[out["idx"][t, j], t]
    scale = np.abs(o).max()
    assert np.abs(o - out["o"]).max() <= rtol * scale


def test_single_expert_layer_is_plain_swiglu_mlp():
    cfg, w, x = small_workload("tiny_f32", 33, num_experts=1, top_k=1, d_model=64,
                               hidden_size=48)
    out = O.forward(cfg, w, x)
    assert np.all(out["w"] == 1.0) and np.all(out["idx"] == 0)
    ref = _torch_swiglu_mlp(x, w["w1"][0], w["w2"][0], 48, _torch_round("f32")).numpy()
    assert np.allclose(out["y"], ref, rtol=1e-6, atol=1e-7)


def test_all_experts_softmax_is_dense_soft_mixture():
    E = 5
    cfg, w, x = small_workload("tiny_f32", 29, num_experts=E, top_k=E, d_model=64,
                               hidden_size=32)
    out = O.forward(cfg, w, x)
    s = torch.softmax(torch.from_numpy(O.router_logits(x, w["router_weight"])), -1)
    s = s.to(torch.float32).to(torch.float64).numpy()
    ref = sum(s[:, e:e + 1] * _torch_swiglu_mlp(x, w["w1"][e], w["w2"][e], 32,
                                                 _torch_round("f32")).numpy() for e in range(E))
    assert np.allclose(out["y"], ref, rtol=1e-6, atol=1e-6)


def test_identity_latent_reduces_to_rmsnorm_of_plain_layer():
    d = 64
    cfg, w, x = small_workload("latent896", 21, d_model=d, latent_dim=d, num_experts=6, top_k=2,
                               hidden_size=32, dtype="f32")
    w["down_proj"] = np.eye(d, dtype=np.float32)
    w["up_proj"] = np.eye(d, dtype=np.float32)
    lat = O.forward(cfg, w, x)
    plain_cfg = O.MoEConfig(**{**cfg.__dict__, "latent_dim": None})
    plain = O.forward(plain_cfg, w, x)
    ref = torch.nn.functional.rms_norm(torch.from_numpy(plain["y"]), (d,),
                                       eps=cfg.up_proj_input_norm_eps).to(torch.float32)
    assert np.allclose(lat["y"], ref.to(torch.float64).numpy(), rtol=1e-6, atol=1e-6)


def test_rmsnorm_scale_invariance():
    """Scaling the weights scales o; RMSNorm removes the scale exactly when eps is negligible
    against mean(o^2): fan-in init (o of order 0.1-1) and eps = 1e-12 here."""
    cfg, w, x = small_workload("tiny_f32", 25, d_model=128, latent_dim=64, num_experts=8,
                               top_k=3, hidden_size=32, up_proj_input_norm_eps=1e-12)
    a = O.forward(cfg, w, x)
    assert (a["o"] ** 2).mean(-1).min() > 1e3 * cfg.up_proj_input_norm_eps
    scaled = O.MoEConfig(**{**cfg.__dict__, "expert_weight_scale": 3.0})
    b = O.forward(scaled, w, x)
    assert np.allclose(a["y"], b["y"], rtol=1e-6, atol=1e-6)
    assert np.allclose(b["w"], 3 * a["w"], rtol=1e-6)


def test_token_permutation_equivariance():
    cfg, w, x = small_workload("olmoe", 50, d_model=64, num_experts=8, top_k=2, hidden_size=32,
                               dtype="f32")
    p = np.random.default_rng(5).permutation(50)
    a = O.forward(cfg, w, x)
    b = O.forward(cfg, w, x[p])
    assert np.array_equal(a["idx"][p], b["idx"])
    assert np.allclose(a["y"][p], b["y"], rtol=1e-6, atol=1e-7)


def test_counts_feed_offsets_and_perm_on_full_layer():
    cfg, w, x = small_workload("latent896", 64, d_model=128, latent_dim=64, num_experts=16,
                               top_k=4, hidden_size=32)
    out = O.forward(cfg, w, x)
    assert out["counts"].sum() == 64 * 4
    for t in range(64):
        assert len(set(out["idx"][t].tolist())) == 4


# ----------------------------------------------------------------- balancing state
# [OC3 "Счётчики и bias-корректировка"]: load imbalance = max / mean of the per-expert counter;
# score_bias += bias_gamma * sign(ideal - actual) with ideal the mean size per expert.

from fractions import Fraction  # noqa: E402

BALANCE_E = (1, 2, 7, 64, 256, 896, 1024)
BALANCE_KINDS = ("uniform", "hot", "zipf", "random", "sparse")


def test_load_imbalance_closed_forms():
    assert O.load_imbalance(workloads.synthetic_counts(64, "uniform")) == 1.0
    for E in (1, 8, 896):
        assert O.load_imbalance(workloads.synthetic_counts(E, "hot")) == float(E)
    assert O.load_imbalance([1, 2]) == 4.0 / 3.0  # max 2, mean 3/2
    assert O.load_imbalance([0, 0, 3]) == 3.0
    assert np.isnan(O.load_imbalance(workloads.synthetic_counts(16, "zero")))


@pytest.mark.parametrize("E", BALANCE_E)
@pytest.mark.parametrize("kind", BALANCE_KINDS)
def test_load_imbalance_is_exact_ratio(E, kind):
    c = workloads.synthetic_counts(E, kind, seed=3)
    if c.sum() == 0:
        return
    mean = Fraction(int(c.sum()), E)
    assert O.load_imbalance(c) == float(Fraction(int(c.max())) / mean)  # correctly rounded


def test_score_bias_update_closed_forms():
    g = np.float32(0.125)
    b = np.array([0.5, -1.0, 3.0, 0.25], dtype=np.float32)
    # uniform load: actual == ideal everywhere, sign 0, bias unchanged
    assert np.array_equal(O.score_bias_update(b, [7, 7, 7, 7], g), b)
    # all tokens on expert 2: it moves down by gamma, every other expert up by gamma
    want = np.array([0.625, -0.875, 2.875, 0.375], dtype=np.float32)
    assert np.array_equal(O.score_bias_update(b, [0, 0, 40, 0], g), want)
    # ideal 1.5 is fractional: 1 < 1.5 up, 2 > 1.5 down
    assert np.array_equal(O.score_bias_update(np.zeros(2, np.float32), [1, 2], 0.5),
                          np.array([0.5, -0.5], dtype=np.float32))
    # a single expert always holds the ideal load
    assert np.array_equal(O.score_bias_update(np.array([2.0], np.float32), [12345], 1.0),
                          np.array([2.0], np.float32))
    # no tokens: every expert at the ideal 0
    assert np.array_equal(O.score_bias_update(b, [0, 0, 0, 0], g), b)


@pytest.mark.parametrize("E", BALANCE_E)
@pytest.mark.parametrize("kind", BALANCE_KINDS)
def test_score_bias_update_against_rational_sign(E, kind):
    c = workloads.synthetic_counts(E, kind, seed=5)
    b = (np.random.default_rng(E).standard_normal(E) * 0.1).astype(np.float32)
    g = 1e-3
    ideal = Fraction(int(c.sum()), E)
    got = O.score_bias_update(b, c, g)
    for e in range(E):
        d = ideal - int(c[e])
        step = np.float32(g) if d > 0 else (-np.float32(g) if d < 0 else np.float32(0))
        assert got[e] == np.float32(b[e] + step), e
    # the move is at most one fp32 gamma, plus the rounding of the fp32 sum
    assert np.all(np.abs(got.astype(np.float64) - b) <= float(np.float32(g)) + np.spacing(np.abs(got)))


def test_accumulated_counts_equal_counts_of_all_batches():
    rng = np.random.default_rng(11)
    E, k = 64, 4
    batches = [np.stack([rng.permutation(E)[:k] for _ in range(T)]) for T in (5, 17, 1, 40)]
    acc = np.zeros(E, dtype=np.int64)
    for idx in batches:
        acc = O.accumulate_counts(acc, O.expert_counts(idx, E))
    every = np.concatenate([b.ravel() for b in batches])
    assert np.array_equal(acc, np.array([np.sum(every == e) for e in range(E)]))


# ----------------------------------------------------------------- expert capacity
# [OC3 "Ёмкость эксперта и переполнение"]: capacity = roundup8(capacity_factor * top_k * T / E)
# at expert-parallel degree 1; each expert keeps the first `capacity` assignments of the
# stable order; dropped assignments contribute nothing.

CAPACITY_GOLDEN = [
    # (capacity_factor, top_k, T, E, capacity) -- worked by hand
    (1.0, 8, 8192, 64, 1024),     # ideal 1024, already a multiple of 8
    (1.25, 2, 100, 8, 32),        # ideal 25, x1.25 = 31.25 -> 32
    (1.0, 1, 1, 1024, 8),         # ideal 1/1024 -> rounds up to 8
    (2.0, 8, 32768, 256, 2048),   # ideal 1024, x2
    (0.5, 8, 16384, 896, 80),     # ideal 146.28..., x0.5 = 73.14... -> 80
    (1.5, 4, 96, 32, 24),         # ideal 12, x1.5 = 18 -> 24
    (1.0, 2, 12, 3, 8),           # ideal 8 exactly: stays 8
]


@pytest.mark.parametrize("cf,k,T,E,want", CAPACITY_GOLDEN)
def test_expert_capacity_hand_worked(cf, k, T, E, want):
    cfg = O.MoEConfig(d_model=64, num_experts=E, top_k=k, capacity_factor=cf)
    assert O.expert_capacity(cfg, T) == want
    assert O.expert_capacity(O.MoEConfig(d_model=64, num_experts=E, top_k=k), T) is None


def _first_come_kept(idx, E, C):
    """Walk the assignments in order t*k+j; an expert accepts until it holds C."""
    held = [0] * E
    kept = []
    for e in np.asarray(idx).ravel():
        kept.append(held[e] < C)
        held[e] += 1
    return np.array(kept)


@pytest.mark.parametrize("E,k,T,C", [(4, 2, 37, 8), (16, 4, 100, 16), (7, 7, 9, 8), (32, 8, 300, 40),
                                     (5, 1, 50, 8)])
def test_capacity_permutation_against_first_come_walk(E, k, T, C):
    rng = np.random.default_rng(E * 1000 + T)
    # skewed choices so that some experts overflow
    p = 1.0 / (np.arange(E) + 1.0)
    idx = np.stack([rng.choice(E, size=k, replace=False, p=p / p.sum()) for _ in range(T)])
    perm, inv, kept = O.capacity_permutation(idx, E, C)
    want_kept = _first_come_kept(idx, E, C)
    assert np.array_equal(kept, want_kept)
    flat = idx.ravel()
    nk = int(want_kept.sum())
    # kept assignments first, grouped by expert in token order; then the dropped ones alike
    want_perm = sorted(range(flat.size), key=lambda a: (not want_kept[a], flat[a], a))
    assert perm.tolist() == want_perm
    assert np.array_equal(inv[perm], np.arange(flat.size))
    counts = np.bincount(flat, minlength=E)
    assert nk == int(np.minimum(counts, C).sum())
    assert np.all(np.bincount(flat[perm[:nk]], minlength=E) == np.minimum(counts, C))


def test_large_capacity_is_dropless():
    cfg, w, x = small_workload("olmoe", 41, d_model=64, num_experts=7, top_k=3, hidden_size=64)
    base = O.forward(cfg, w, x)
    big = O.forward(dataclasses.replace(cfg, capacity_factor=1000.0), w, x)
    assert big["capacity"] >= base["counts"].max()
    assert np.array_equal(big["perm"], base["perm"]) and np.all(big["kept"])
    assert np.array_equal(big["y"], base["y"])


@pytest.mark.parametrize("name,over,rtol", [
    ("tiny_f32", dict(d_model=64, num_experts=6, top_k=3, hidden_size=32, capacity_factor=0.5), 1e-6),
    ("latent896", dict(d_model=128, latent_dim=64, num_experts=9, top_k=4, hidden_size=32,
                       capacity_factor=0.75), 2e-2),
])
def test_capacity_dense_bruteforce(name, over, rtol):
    """Every expert on every token, weighted by w and by the first-come kept mask, equals the
    oracle's capacity path (sort, drop, group, zero the dropped rows, combine)."""
    T = 53
    cfg, w, x = small_workload(name, T, **over)
    out = O.forward(cfg, w, x)
    C = out["capacity"]
    kept = _first_come_kept(out["idx"], cfg.num_experts, C).reshape(T, cfg.top_k)
    assert not kept.all(), "the case must drop something"
    rnd = _torch_round(cfg.dtype)
    z = out["z"]
    every = np.stack([_torch_swiglu_mlp(z, w["w1"][e], w["w2"][e], cfg.hidden_size, rnd).numpy()
                      for e in range(cfg.num_experts)])
    o = np.zeros((T, z.shape[1]))
    for t in range(T):
        for j in range(cfg.top_k):
            if kept[t, j]:
                o[t] += out["w"][t, j] * every[out["idx"][t, j], t]
    assert np.abs(o - out["o"]).max() <= rtol * np.abs(o).max()


# ----------------------------------------------------------------- MXFP8
# OCP microscaling read of [OC3 "Rowwise FP8 и MXFP8"]: E4M3 elements, E8M0 block scales,
# blocks of 32 along the contraction dimension.

def _e4m3_ties_and_edges():
    grid = O.e4m3_values()[:0x7F]           # the 127 finite non-negative codes, increasing
    mids = (grid[1:] + grid[:-1]) / 2.0     # exact midpoints: ties
    vals = np.concatenate([grid, mids, np.nextafter(mids, 0.0), np.nextafter(mids, 1e9), [448.0, 0.0]])
    vals = np.concatenate([vals, -vals])
    return vals.astype(np.float32)


def test_e4m3_encode_matches_torch_float8():
    """torch's float8_e4m3fn cast (round to nearest even) on every grid point, every midpoint
    (exact ties), the neighbours of every midpoint, and random values over the whole range."""
    rng = np.random.default_rng(3)
    rand = rng.standard_normal(50000) * np.exp(rng.uniform(-14, 6.1, 50000))
    x = np.concatenate([_e4m3_ties_and_edges(), np.clip(rand, -448, 448).astype(np.float32)])
    want = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(O.e4m3_encode(x), want)
    assert np.signbit(O.e4m3_values()[O.e4m3_encode(np.float32(-0.0))])  # -0 keeps its sign


def test_e4m3_encode_brute_force_and_saturation():
    grid = O.e4m3_values()[:0x7F]
    rng = np.random.default_rng(4)
    for a in np.abs(rng.standard_normal(3000) * 2.0 ** rng.uniform(-10, 8, 3000)):
        d = np.abs(grid - min(a, 448.0))
        best = np.nonzero(d == d.min())[0]
        want = best[0] if len(best) == 1 else [c for c in best if c % 2 == 0][0]  # ties: even mantissa
        assert O.e4m3_encode(a) == want
    assert list(O.e4m3_encode([448.0, 449.0, 1e30, -500.0])) == [0x7E, 0x7E, 0x7E, 0xFE]


@pytest.mark.parametrize("seed", range(4))
def test_mx_quantize_block_scale_definition(seed):
    rng = np.random.default_rng(seed)
    v = rng.standard_normal((7, 256)) * np.exp(rng.uniform(-8, 8, (7, 1)))
    v[2, 64:96] = 0.0                                      # an all-zero block
    codes, scales = O.mx_quantize(v)
    b = v.reshape(7, 8, 32)
    amax = np.abs(b).max(-1)
    nz = amax > 0
    ratio = amax[nz] / 2.0 ** (scales[nz].astype(np.float64) - 127)
    assert np.all((ratio >= 256) & (ratio < 512))          # exponent = floor(log2 amax) - 8
    assert scales[2, 2] == 0 and np.all(codes[2, 64:96] & 0x7F == 0)
    deq = O.mx_dequantize(codes, scales).reshape(7, 8, 32)
    step = 2.0 ** (scales.astype(np.float64) - 127)[..., None] * 2.0 ** (np.floor(np.log2(np.maximum(np.abs(b) / 2.0 ** (scales.astype(np.float64) - 127)[..., None], 2.0 ** -6))) - 3)
    sat = np.abs(b) / 2.0 ** (scales.astype(np.float64) - 127)[..., None] > 448
    assert np.all(np.abs(deq - b)[~sat] <= step[~sat] / 2)  # nearest grid point
    assert np.all(np.abs(deq[sat]) == 448 * 2.0 ** (scales.astype(np.float64) - 127)[..., None].repeat(32, -1)[sat])


def test_mx_round_trip_of_representable_blocks():
    rng = np.random.default_rng(5)
    grid = O.e4m3_values()[:0x7F]
    for e in (-20, -3, 0, 5, 30):
        blk = rng.choice(grid, size=(4, 32)) * rng.choice([-1.0, 1.0], size=(4, 32))
        blk[:, 0] = 256.0 * np.sign(blk[:, 0] + 0.5)       # amax in [256, 512): scale exactly 2^e
        v = blk * 2.0 ** e
        assert np.array_equal(O.mx_round(v), v)


def test_mxfp8_dense_bruteforce_equals_permuted_path():
    """The MXFP8 expert path through sort/group/combine equals every expert's MXFP8 MLP on
    every token (torch's silu, operands rounded through MX independently of the permutation)."""
    T = 37
    cfg, w, x = small_workload("olmoe", T, d_model=128, num_experts=5, top_k=2, hidden_size=64,
                               expert_precision="mxfp8")
    out = O.forward(cfg, w, x)
    z = out["z"]
    every = []
    for e in range(cfg.num_experts):
        H = torch.from_numpy(O.mx_round(z)) @ torch.from_numpy(O.mx_round(w["w1"][e])).T
        up, gate = H[:, :64], H[:, 64:]
        act = _torch_round("bf16")(up * torch.nn.functional.silu(gate))
        every.append(_torch_round("bf16")(torch.from_numpy(O.mx_round(act.numpy())) @
                                          torch.from_numpy(O.mx_round(w["w2"][e])).T).numpy())
    o = np.zeros_like(out["o"])
    for t in range(T):
        for j in range(cfg.top_k):
            o[t] += out["w"][t, j] * every[out["idx"][t, j]][t]
    assert np.abs(o - out["o"]).max() <= 1e-2 * np.abs(o).max()
    # and the MXFP8 layer stays close to the bf16 one (quantisation error only)
    ref = O.forward(dataclasses.replace(cfg, expert_precision="bf16"), w, x)
    assert np.linalg.norm(out["y"] - ref["y"]) <= 0.1 * np.linalg.norm(ref["y"])


@pytest.mark.parametrize("name,over", [
    ("tiny_f32", {}),
    ("olmoe", dict(tokens=300, d_model=256, num_experts=8, top_k=2, hidden_size=128)),
    ("latent896", dict(tokens=200, d_model=256, latent_dim=128, num_experts=16, top_k=4, hidden_size=64)),
])
def test_float32_accumulation_mode_agrees_with_float64(name, over):
    """The mode the CPU timing runs in (acc=float32) changes only the summation dtype of the
    contractions, so it computes the same layer: equal routing except at near-ties, values
    within the layer tolerance of the float64 oracle (fp32 layer: relative 1e-5; bf16 layers:
    max-abs 2e-2 and relative Frobenius 1e-2)."""
    over = dict(over)
    T = over.pop("tokens", None)
    cfg, w, x = workloads.make_workload(name, tokens=T, **over)
    cfgO = O.MoEConfig.from_dict(cfg)
    wo = {k: workloads.to_numpy_f32(v) for k, v in w.items()}
    xs = workloads.to_numpy_f32(x)
    r64 = O.forward(cfgO, wo, xs)
    r32 = O.forward(cfgO, wo, xs, acc=np.float32)
    same = np.all(r64["idx"] == r32["idx"], axis=1)
    assert same.mean() >= 0.99
    d = np.abs(r32["y"][same] - r64["y"][same])
    fro = np.linalg.norm(r32["y"][same] - r64["y"][same]) / np.linalg.norm(r64["y"][same])
    if cfg["dtype"] == "f32":
        assert fro <= 1e-5 and d.max() <= 1e-5 * np.abs(r64["y"]).max()
    else:
        assert fro <= 1e-2 and d.max() <= 2e-2
    # the mode really sums in fp32: the logits differ from the float64 sums somewhere
    l32 = O.router_logits(xs, wo["router_weight"], wo["router_bias"], acc=np.float32)
    assert not np.array_equal(l32, r64["logits"])
