"""Helpers shared by the GPU parity tests: tolerances, comparisons, sampled-oracle evaluation.

Tolerances (stated once, used everywhere):
  * integer / index outputs: bit-exact;
  * bf16 layers: ||gpu - oracle||_F / ||oracle||_F <= 1e-2 and max |gpu - oracle| <= 2e-2 on
    every element but a tiny share (at most 1e-5 of the elements). Those few must be explained
    by rounding the page fixes: the expert outputs Y are bf16 on both sides (the page on
    grouped experts: they return bf16), computed from fp32 accumulation on the GPU and from
    float64 in the oracle, so near a rounding boundary the two can land one bf16 spacing apart;
    such a flip moves y by w * spacing(Y). The outlier bound is therefore 2e-2 + half the bf16
    spacing of y (its own storage) + sum_j |w_j| * spacing(Y_j) (non-latent layers, where y is
    the weighted sum itself);
  * fp32 layers: relative Frobenius <= 1e-5 and max |.| <= 1e-5 * max |oracle|;
  * routing: the GPU's selection is compared bit for bit with the oracle's selection run on the
    GPU's own fp32 gating output (the scores, or the logits for topk_softmax); counts,
    offsets, permutation and inverse bit for bit with the oracle's on those indices;
  * fp32 gating scores and routing weights: within a number of fp32 ulps derived from the
    kernels' fp32 operation counts (gating_ulps / weight_ulps below), against the oracle run
    on the same fp32 inputs;
  * router logits: within the textbook fp32 dot-product bound (logit_bound).
Layer values are compared with the oracle driven by the GPU's routing (its indices and
weights), so every token is compared; the routing itself is checked separately as above.
The oracle's final y is unrounded (float64); the GPU's y is rounded to the layer dtype.
"""
from __future__ import annotations

import numpy as np
import torch

import workloads
from oracle import moe_oracle as O

BF16_MAX_ABS = 2e-2
BF16_REL_FRO = 1e-2
F32_REL_FRO = 1e-5
F32_REL_MAX = 1e-5
BF16_OUTLIER_SHARE = 1e-5


def np32(t):
    return workloads.to_numpy_f32(t)


def assert_close(got, ref, dtype: str, what: str = "", flip_allow=None, budget_share=None):
    """bf16: relative Frobenius <= BF16_REL_FRO, every element within BF16_MAX_ABS + half a bf16
    spacing (+ flip_allow), and at most budget_share (default BF16_OUTLIER_SHARE) of the elements
    beyond BF16_MAX_ABS itself; budget_share=1.0 drops the count (MXFP8, whose per-element
    allowance comes from the matrix cores' summation bound). f32: relative bounds."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    if got.size == 0:
        return
    assert np.all(np.isfinite(got)), f"{what}: non-finite GPU values"
    d = np.abs(got - ref)
    fro = np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-30)
    mx = d.max()
    if dtype == "bf16":
        over = d > BF16_MAX_ABS
        budget = max(1, int((BF16_OUTLIER_SHARE if budget_share is None else budget_share) * d.size))
        allowed = BF16_MAX_ABS + 0.5 * bf16_spacing(ref)
        if flip_allow is not None:
            allowed = allowed + np.asarray(flip_allow, np.float64)
        msg = (f"{what}: max-abs {mx:.3e}, {int(over.sum())} elements above {BF16_MAX_ABS} (budget {budget}), "
               f"worst excess over the rounding bound {float((d - allowed).max()):.3e}, rel-fro {fro:.3e} "
               f"(<= {BF16_REL_FRO}), max|ref| {np.abs(ref).max():.3f}")
        # every comparison reports its max-abs and its count of elements past 2e-2, so that the
        # departures from the stated max-abs that the rounding allowance admits stay visible
        print(f"  {msg}", flush=True)
        assert fro <= BF16_REL_FRO and int(over.sum()) <= budget and np.all(d <= allowed), msg
    else:
        scale = np.abs(ref).max()
        msg = f"{what}: rel-fro {fro:.3e} (<= {F32_REL_FRO}), max-abs {mx:.3e} (<= {F32_REL_MAX}*{scale:.3e})"
        print(f"  {msg}", flush=True)
        assert fro <= F32_REL_FRO and mx <= F32_REL_MAX * max(scale, 1e-30), msg


def flip_allowance(cfgO, out):
    """Per-element sum_j |w_j| * spacing(Y_j) for non-latent bf16 layers (else None)."""
    if cfgO.latent_dim or cfgO.dtype != "bf16":
        return None
    w = np.asarray(out["w"], np.float64)
    T, k = w.shape
    Y = out["Y"][np.asarray(out["inv"]).reshape(T, k)]
    return (np.abs(w)[:, :, None] * bf16_spacing(Y)).sum(axis=1)


def bf16_spacing(a):
    """Distance between consecutive bf16 numbers at |a| (8 significant bits)."""
    a = np.maximum(np.abs(np.asarray(a, np.float64)), 2.0 ** -126)
    return 2.0 ** (np.floor(np.log2(a)) - 7)


def f32_spacing(a):
    """Distance from |a| to the next float32 (the fp32 ulp at |a|), as float64."""
    a = np.abs(np.asarray(a, np.float32))
    return np.spacing(a).astype(np.float64)


def ulp_error(got, ref):
    """|got - ref| in fp32 ulps of ref (NaN where ref is not finite)."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    with np.errstate(invalid="ignore"):
        return np.abs(got - ref) / f32_spacing(ref)


def gating_ulps(cfgO, logits):
    """Allowance, in fp32 ulps of the oracle's score, for the GPU's gating output computed
    from the same fp32 logits. Each term counts roundings relative to the result (an fp32
    ulp is at least 2^-24 of the value, so a relative error of n * 2^-24 is at most n ulps):
      softmax (also the scores of topk_softmax): the argument l - m rounds (|l - m| * 2^-24
        relative change of exp), expf (<= 1 ulp) for the element and for the sum's terms,
        the sum of E positive terms (ceil(E/64) - 1 sequential adds per lane, then a 6-level
        wave tree), the division (1/2) and the oracle's own rounding (1/2);
      sigmoid: the exponent -l * log2(e) rounds (|l| * 2^-24 relative change of exp2), the
        hardware exp2 and reciprocal (<= 1 ulp each), 1 + e (1/2), the epsilon add (1), the
        oracle's rounding (1/2).
    A factor 2 of headroom covers the binade edge (an ulp of a value just above a power of
    two is 2^-23 of it)."""
    l = np.asarray(logits, np.float64)
    E = l.shape[-1]
    if cfgO.gating_function in ("softmax", "topk_softmax"):
        m = np.nanmax(l, axis=-1, keepdims=True)
        spread = np.nanmax(np.abs(l - m), axis=-1, keepdims=True)
        n = np.abs(l - m) + spread + 2 + (-(-E // 64) - 1) + 6 + 1
    else:
        n = np.abs(l) + 2 + 0.5 + 1 + 0.5
    return 2.0 * (n + 2)


def weight_ulps(cfgO, sel_input, idx):
    """Allowance, in fp32 ulps of the oracle's weight, for the GPU's routing weights computed
    from the same fp32 gating output and the same indices: the gathered score is exact; the
    p-norm sums k terms on a 6-level wave tree (6), squares and a root for p = 2 (2), divides
    (1/2); the scales round once each (restore top_k 1/2, expert_weight_scale 1/2,
    sqrt(original_top_k / top_k) 3/2); the oracle rounds once (1/2). topk_softmax adds the
    softmax over the k selected logits: argument rounding |l - m| * 2^-24, two expf (2), the
    6-level sum (6), the division (1/2). Factor 2 for the binade edge, as in gating_ulps."""
    n = 6 + 2 + 0.5 + 0.5 + 0.5 + 1.5 + 0.5
    if cfgO.gating_function == "topk_softmax":
        sel = np.take_along_axis(np.asarray(sel_input, np.float64), np.asarray(idx, np.int64), axis=1)
        spread = np.max(np.abs(sel - sel.max(axis=1, keepdims=True)), axis=1, keepdims=True)
        n = n + spread + 2 + 6 + 0.5
    return 2.0 * (n + 2)


def assert_within_ulps(got, ref, ulps, what):
    """Every finite entry within `ulps` (scalar or broadcastable array) fp32 ulps of ref; the
    non-finite entries must be non-finite in both. Prints the worst case."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    fin = np.isfinite(ref)
    assert np.array_equal(np.isfinite(got), fin), f"{what}: non-finite entries differ"
    if not fin.any():
        return
    err = np.where(fin, ulp_error(np.where(fin, got, 0.0), np.where(fin, ref, 1.0)), 0.0)
    allow = np.broadcast_to(np.asarray(ulps, np.float64), err.shape)
    bad = err > allow
    print(f"  {what}: worst {err.max():.1f} fp32 ulps (allowance at that entry "
          f"{allow.flat[int(np.argmax(err))]:.1f})", flush=True)
    assert not bad.any(), f"{what}: {int(bad.sum())} entries beyond their allowance, worst {err.max():.1f} ulps"


def logit_bound(x, W, bf16_path):
    """|l_gpu - l_exact| <= gamma_n * sum_i |x_i W_ei| with gamma_n = n u / (1 - n u), u = 2^-24,
    for a sum of n fp32-rounded additions: n = d on the fp32 path; n = 3d + 32 on the bf16 path
    (three exact bf16 products per term, up to 32 partial sums added at the end); plus the
    oracle's final fp32 rounding (1/2 ulp)."""
    d = x.shape[1]
    n = 3 * d + 32 if bf16_path else d
    u = 2.0 ** -24
    g = n * u / (1 - n * u)
    return g * (np.abs(x.astype(np.float64)) @ np.abs(W.astype(np.float64)).T)


def check_forward_routing(cfgO, r: dict, score_bias=None):
    """The routing outputs of a whole-layer (or router) call against the oracle run on the
    GPU's own fp32 gating output: the selection bit for bit on every token, the weights within
    weight_ulps, the gating output within gating_ulps of the oracle's gating of the GPU's
    logits, and (when present) counts, offsets, permutation and inverse bit for bit against
    the oracle's on the GPU's indices. Returns the oracle's routing on the GPU's scores."""
    logits = r["router_logits"].cpu().numpy()
    scores = r["router_scores"].cpu().numpy()
    sel = logits if cfgO.gating_function == "topk_softmax" else scores
    sb = None if score_bias is None else np32(score_bias)
    ref = O.route_from_scores(cfgO, sel, sb)
    gi = r["expert_indices"].cpu().numpy()
    bad = np.nonzero(np.any(gi != ref["idx"], axis=1))[0]
    assert bad.size == 0, (f"{bad.size} tokens select differently from the oracle on the GPU's own "
                           f"scores, first {bad[:5].tolist()}")
    assert_within_ulps(r["expert_weights"].cpu().numpy(), ref["w"], weight_ulps(cfgO, sel, gi), "routing weights")
    assert_within_ulps(scores, O.gating_scores(cfgO, logits), gating_ulps(cfgO, logits), "gating scores")
    if "batch_size_per_expert" in r:
        counts = O.expert_counts(gi, cfgO.num_experts)
        assert np.array_equal(r["batch_size_per_expert"].cpu().numpy(), counts)
        if cfgO.capacity_factor is None:
            perm, inv = O.stable_permutation(gi)
            assert np.array_equal(r["expert_offsets"].cpu().numpy(), O.expert_offsets(counts))
            assert np.array_equal(r["permutation"].cpu().numpy(), perm)
            assert np.array_equal(r["inverse_permutation"].cpu().numpy(), inv)
    return ref


def oracle_from_gpu_routing(cfgO, wo: dict, x, idx, wts, capacity=None):
    """The oracle's expert path, combine and restore driven by given indices and weights (the
    GPU's): every token's value can then be compared, whatever the routing of a near-tie."""
    z = O.prepare_routed_input(cfgO, x, wo.get("down_proj"))
    ex = O.run_experts(cfgO, z, idx, wo["w1"], wo["w2"], capacity)
    o = O.combine(cfgO, ex["Y"], ex["inv"], wts)
    out = O.restore_routed_output(cfgO, o, wo.get("norm_weight"), wo.get("up_proj"))
    return dict(ex, z=z, o=o, w=np.asarray(wts), idx=np.asarray(idx), y=out["y"])


def routing_agreement(gpu_idx, ref: dict, gpu_keys):
    """Share of tokens whose GPU selection equals the pure oracle's (selection on the oracle's
    own logits). Where they differ, each expert the GPU took instead of one the oracle took
    must be a near-tie: their oracle keys lie within the two keys' realised GPU-vs-oracle
    differences (what exact selection on the GPU's keys implies). Returns the agreement mask."""
    gpu_idx = np.asarray(gpu_idx)
    same = np.all(gpu_idx == ref["idx"], axis=1)
    keys = np.asarray(ref["keys"], np.float64)
    dk = np.abs(np.asarray(gpu_keys, np.float64) - keys)
    for t in np.nonzero(~same)[0]:
        g, o = set(gpu_idx[t].tolist()), set(ref["idx"][t].tolist())
        assert len(g) == gpu_idx.shape[1], f"token {t}: repeated experts {gpu_idx[t]}"
        for a in g - o:
            for b in o - g:
                assert keys[t, b] - keys[t, a] <= dk[t, a] + dk[t, b], \
                    f"token {t}: gpu picked {a} (key {keys[t, a]}) over {b} (key {keys[t, b]})"
    return same


def to_device_weights(w: dict, device="cuda"):
    return {k: (None if v is None else v.to(device)) for k, v in w.items()}


def oracle_inputs(w: dict, experts=None) -> dict:
    """Host float32 copies of the weights for the oracle; with `experts`, only those experts'
    matrices (a dict e -> array), copied from wherever the tensors live."""
    out = {k: np32(v) for k, v in w.items() if k not in ("w1", "w2")}
    if experts is None:
        out["w1"], out["w2"] = np32(w["w1"]), np32(w["w2"])
    else:
        out["w1"] = {int(e): np32(w["w1"][int(e)]) for e in experts}
        out["w2"] = {int(e): np32(w["w2"][int(e)]) for e in experts}
    return out


def check_routing_invariants(cfg: dict, r: dict, T: int, capacity=None):
    """Properties of the routing outputs that hold at any size (checked on the device). With a
    capacity, the offsets are those of the kept counts min(count, capacity) and the permutation
    holds the kept assignments, then the dropped ones, each part sorted by expert and stable."""
    E, k = cfg["num_experts"], cfg["top_k"]
    idx = r["expert_indices"].long()
    assert idx.shape == (T, k)
    assert int(idx.min()) >= 0 and int(idx.max()) < E
    s, _ = torch.sort(idx, dim=1)
    assert bool((s[:, 1:] != s[:, :-1]).all()), "repeated expert within a token"
    counts = torch.bincount(idx.flatten(), minlength=E)
    assert torch.equal(counts.to(torch.int32), r["batch_size_per_expert"])
    kept = counts if capacity is None else torch.clamp(counts, max=capacity)
    off = torch.zeros(E + 1, dtype=torch.int64, device=idx.device)
    off[1:] = torch.cumsum(kept, 0)
    assert torch.equal(off.to(torch.int32), r["expert_offsets"])
    perm = r["permutation"].long()
    inv = r["inverse_permutation"].long()
    A = T * k
    flat = idx.flatten()
    assert torch.equal(torch.sort(perm).values, torch.arange(A, device=perm.device))
    assert torch.equal(inv[perm], torch.arange(A, device=perm.device))
    # each part sorted by expert, stable (assignment index increasing within an expert)
    nk = int(off[E])
    for part in (perm[:nk], perm[nk:]):
        if part.numel() < 2:
            continue
        ep = flat[part]
        assert bool((ep[1:] >= ep[:-1]).all())
        same_e = ep[1:] == ep[:-1]
        assert bool((part[1:][same_e] > part[:-1][same_e]).all())


def sample_tokens(T: int, n: int, seed: int = 0) -> np.ndarray:
    g = np.random.default_rng(seed)
    if T <= n:
        return np.arange(T)
    s = set(g.choice(T, size=n - 2, replace=False).tolist()) | {0, T - 1}
    return np.array(sorted(s))


# MXFP8 experts: the block-scaled matrix cores sum their products with an error up to about
# 2^-12 of sum_k |a_k b_k| per instruction (measured on gfx950 against exact products), where
# the oracle sums exactly. Allowance per expert-output element: 2^-10 * sum_k |act_q,k| |w2_q,k|
# (the GEMM2 bound with a factor 4 of headroom, which also covers the rare activation codes that
# GEMM1's error moves across an fp8 rounding boundary).
MX_SUM_ERR = 2.0 ** -10


def mx_expert_allowance(cfgO, ex, wo):
    """Per-row allowance (A, K) in sorted order for an oracle run_experts result `ex`."""
    from oracle import moe_oracle as O
    h = cfgO.hidden_size
    out = np.zeros_like(ex["Y"])
    off = ex["offsets"]
    for e in range(cfgO.num_experts):
        rows = slice(off[e], off[e + 1])
        if off[e + 1] == off[e]:
            continue
        H = O.mx_round(ex["z_perm"][rows]) @ O.mx_round(np.asarray(wo["w1"][e], np.float64)).T
        up, gate = H[:, :h], H[:, h:]
        with np.errstate(over="ignore"):
            act = O.round_to(up * gate / (1.0 + np.exp(-gate)), cfgO.dtype)
        out[rows] = MX_SUM_ERR * (np.abs(O.mx_round(act)) @ np.abs(O.mx_round(np.asarray(wo["w2"][e], np.float64))).T)
    return out
