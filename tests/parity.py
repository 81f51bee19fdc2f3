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
  * fp32 routing weights: |gpu - oracle| <= 4e-6 * max(1, |oracle|) (a few fp32 roundings of
    the same fp32 inputs).
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
WEIGHT_TOL = 4e-6
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
        assert fro <= BF16_REL_FRO and int(over.sum()) <= budget and np.all(d <= allowed), msg
        if over.any():
            print(f"  note: {msg}")
    else:
        scale = np.abs(ref).max()
        assert fro <= F32_REL_FRO and mx <= F32_REL_MAX * max(scale, 1e-30), \
            f"{what}: rel-fro {fro:.3e} (<= {F32_REL_FRO}), max-abs {mx:.3e} (<= {F32_REL_MAX}*{scale:.3e})"


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


def assert_weights_close(got, ref, what="weights"):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    tol = WEIGHT_TOL * np.maximum(1.0, np.abs(ref))
    bad = np.abs(got - ref) > tol
    assert not bad.any(), f"{what}: {bad.sum()} entries off, worst {np.abs(got - ref).max():.3e}"


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


def routing_matches(cfgO: O.MoEConfig, gpu_idx, ref: dict, key_tol: float):
    """Tokens whose GPU selection differs from the oracle's must be near-ties: every swapped
    pair of experts has oracle keys within key_tol (the selection is then valid under the
    GPU's own fp32 rounding). Returns the boolean mask of tokens with identical selections."""
    gpu_idx = np.asarray(gpu_idx)
    same = np.all(gpu_idx == ref["idx"], axis=1)
    keys = ref["keys"]
    for t in np.nonzero(~same)[0]:
        g, o = set(gpu_idx[t].tolist()), set(ref["idx"][t].tolist())
        assert len(g) == cfgO.top_k, f"token {t}: repeated experts {gpu_idx[t]}"
        if g == o:  # same set, order differs: only possible on an exact/near tie
            kg = keys[t, gpu_idx[t]]
            assert np.all(np.abs(np.diff(kg)) <= key_tol) or np.all(np.diff(kg) <= key_tol), t
            continue
        for a in g - o:
            for b in o - g:
                assert abs(keys[t, a] - keys[t, b]) <= key_tol, \
                    f"token {t}: gpu picked {a} (key {keys[t, a]}) over {b} (key {keys[t, b]})"
    return same


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
