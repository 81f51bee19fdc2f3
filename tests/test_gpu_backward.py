"""GPU parity of the routed experts' backward (and of the training forward that saves its inputs)
against the CPU oracle, through the C ABI.

Inputs: the seeded workload generators (weights, tokens) and seeded synthetic expert indices;
the permutation, offsets, z and the saved tensors handed to the GPU backward come from the
oracle, so the comparison covers the backward's arithmetic alone.

Tolerances (derived from the arithmetic; the layer tolerance is stated for the forward output):
  * the training forward's h, act and y: the layer tolerance, with one bf16 spacing of flip per
    element (each is one rounding of an fp32 accumulation on the GPU and of a float64 one in
    the oracle);
  * gradients of a bf16 layer: relative Frobenius <= 1e-2, and every element within
    2^-5 * M + 2 spacings of the reference, where M is the same product taken over absolute
    values (|dH| |w1| for dz, |dY|^T |act| for dw2, |dH|^T |z| for dw1). The bf16 values on
    the way (d_act, dH, the per-copy input gradients) are roundings of fp32 sums on the GPU
    and of float64 sums in the oracle; each can land one spacing (at most 2^-7 relative) apart,
    and the SwiGLU derivative carries a flip of d_act or of the saved H into dH, so a few such
    relative deviations per term bound the difference by a small multiple of 2^-7 * M. A wrong
    index, operand, expert or sign moves an element by O(M);
  * fp32 layers: relative Frobenius <= 1e-5 and max-abs <= 1e-5 * max |reference|.
"""
import numpy as np
import pytest
import torch

import workloads
from oracle import moe_oracle as O
from parity import assert_close, bf16_spacing, np32, oracle_inputs, to_device_weights

pytestmark = pytest.mark.gpu

moe = pytest.importorskip("top_routing_grouped_router_amd")

GRAD_REL_FRO = 1e-2
GRAD_REL_M = 2.0 ** -5
F32_REL = 1e-5


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.set_device(0)


def banner(msg):
    print(f"[case] {msg}", flush=True)


def assert_grad_close(got, ref, M, dtype, what):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite GPU values"
    d = np.abs(got - ref)
    nrm = max(np.linalg.norm(ref), 1e-30)
    fro = np.linalg.norm(got - ref) / nrm
    if dtype == "bf16":
        allow = GRAD_REL_M * np.asarray(M, np.float64) + 2.0 * bf16_spacing(ref)
        worst = float((d - allow).max())
        print(f"  {what}: rel-fro {fro:.2e}, max |diff| / M {float((d / np.maximum(M, 1e-30)).max()):.2e}, "
              f"elements off {int((d > 0).sum())}/{d.size}", flush=True)
        assert fro <= GRAD_REL_FRO and worst <= 0, \
            f"{what}: rel-fro {fro:.3e} (<= {GRAD_REL_FRO}), worst excess over 2^-5 M + 2 spacings {worst:.3e}"
    else:
        scale = max(np.abs(ref).max(), 1e-30)
        assert fro <= F32_REL and d.max() <= F32_REL * scale, \
            f"{what}: rel-fro {fro:.3e}, max-abs {d.max():.3e} (scale {scale:.3e})"


def _case_inputs(name, T, over, seed=3, skew=0.0):
    cfg, w, x = workloads.make_workload(name, tokens=T, **over)
    cfgO = O.MoEConfig.from_dict(cfg)
    T = x.shape[0]
    idx = workloads.random_distinct_indices(T, cfg["num_experts"], cfg["top_k"], seed=seed, skew=skew).numpy()
    wo = oracle_inputs(w)
    z = O.prepare_routed_input(cfgO, np32(x), wo["down_proj"])
    C = O.expert_capacity(cfgO, T)
    tr = O.run_experts_train(cfgO, z, idx, wo["w1"], wo["w2"], C)
    D = workloads.storage_dtype(cfg)
    g = torch.Generator().manual_seed(seed + 11)
    dY = torch.randn((T * cfg["top_k"], cfgO.expert_dim), generator=g).mul_(0.5).to(D)
    return cfg, cfgO, w, wo, z, idx, C, tr, dY


def _dev(a, dtype):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(dtype).cuda()


def _idx(a):
    return torch.from_numpy(np.asarray(a, dtype=np.int32)).cuda()


CASES = [
    ("tiny_f32", None, {}, 0.0),
    ("olmoe", 777, dict(d_model=512, num_experts=16, top_k=4, hidden_size=256), 0.0),    # large tiles
    ("olmoe", 130, dict(d_model=512, num_experts=64, top_k=8, hidden_size=192), 0.0),    # small tiles, ragged N
    ("skewed", 600, dict(d_model=256, num_experts=32, top_k=4, hidden_size=320), 1.2),   # hot experts, ragged
    ("latent896", 200, dict(d_model=512, latent_dim=128, num_experts=96, top_k=8, hidden_size=128), 0.0),
    ("olmoe", 5, dict(d_model=256, num_experts=64, top_k=2, hidden_size=128), 0.0),      # most experts empty
    ("olmoe", 300, dict(d_model=256, num_experts=16, top_k=4, hidden_size=128, capacity_factor=0.5), 1.0),
    ("tiny_f32", 100, dict(capacity_factor=0.75), 1.0),
]
IDS = [f"{c[0]}-{c[1]}-{'-'.join(f'{k}{v}' for k, v in c[2].items())}" for c in CASES]


@pytest.mark.parametrize("case", CASES, ids=IDS)
def test_experts_forward_train(case):
    name, T, over, skew = case
    banner(f"forward_train {case}")
    cfg, cfgO, w, wo, z, idx, C, tr, _ = _case_inputs(name, T, over, skew=skew)
    D = workloads.storage_dtype(cfg)
    out = moe.experts_forward_train(cfg, to_device_weights(w), _dev(z, D), _idx(tr["offsets"]), _idx(tr["perm"]))
    torch.cuda.synchronize()
    n = int(tr["offsets"][-1])
    bf = cfg["dtype"] == "bf16"
    for key in ("h", "act"):
        ref = tr["H" if key == "h" else "act"][:n]
        assert_close(np32(out[key])[:n], ref, cfg["dtype"], key, bf16_spacing(ref) if bf else None)
    ref_y = tr["Y"][tr["inv"]]
    assert_close(np32(out["y_assign"]), ref_y, cfg["dtype"], "y_assign", 2.0 * bf16_spacing(ref_y) if bf else None)
    # the training forward's y equals the inference forward's bit for bit
    y_inf = moe.experts_forward(cfg, to_device_weights(w), _dev(z, D), _idx(tr["offsets"]), _idx(tr["perm"]))
    torch.cuda.synchronize()
    assert torch.equal(y_inf, out["y_assign"])


@pytest.mark.parametrize("case", CASES, ids=IDS)
def test_experts_backward(case):
    name, T, over, skew = case
    banner(f"backward {case}")
    cfg, cfgO, w, wo, z, idx, C, tr, dY = _case_inputs(name, T, over, skew=skew)
    D = workloads.storage_dtype(cfg)
    dYn = np32(dY)
    ref = O.experts_backward(cfgO, z, idx, wo["w1"], wo["w2"], tr, dYn, C)
    saved = {"h": _dev(tr["H"], D), "act": _dev(tr["act"], D)}
    got = moe.experts_backward(cfg, to_device_weights(w), _dev(z, D), _idx(tr["offsets"]), _idx(tr["perm"]),
                               saved, dY.cuda())
    torch.cuda.synchronize()
    # magnitudes: the same products over absolute values
    k, E = cfg["top_k"], cfg["num_experts"]
    offs, perm = tr["offsets"], tr["perm"]
    adH = np.abs(ref["dH"])
    adY = np.abs(dYn)[perm]
    az = np.abs(tr["z_perm"])
    aact = np.abs(tr["act"])
    Mzp = np.zeros_like(ref["dz_perm"])
    Mw1 = np.zeros_like(ref["dw1"])
    Mw2 = np.zeros_like(ref["dw2"])
    for e in range(E):
        R = slice(offs[e], offs[e + 1])
        if offs[e + 1] > offs[e]:
            Mzp[R] = adH[R] @ np.abs(np.asarray(wo["w1"][e], np.float64))
            Mw1[e] = adH[R].T @ az[R]
            Mw2[e] = adY[R].T @ aact[R]
    Mdz = Mzp[np.asarray(tr["inv"]).reshape(-1, k)].sum(axis=1)
    assert_grad_close(np32(got["dz"]), ref["dz"], Mdz, cfg["dtype"], "dz")
    assert_grad_close(np32(got["dw1"]), ref["dw1"], Mw1, cfg["dtype"], "dw1")
    assert_grad_close(np32(got["dw2"]), ref["dw2"], Mw2, cfg["dtype"], "dw2")
    # experts without rows: exactly zero
    empty = np.nonzero(np.diff(offs) == 0)[0]
    if empty.size:
        assert not got["dw1"][torch.from_numpy(empty).cuda()].any()
        assert not got["dw2"][torch.from_numpy(empty).cuda()].any()
    # deterministic: a second call is bitwise equal
    again = moe.experts_backward(cfg, to_device_weights(w), _dev(z, D), _idx(tr["offsets"]), _idx(tr["perm"]),
                                 saved, dY.cuda())
    torch.cuda.synchronize()
    for key in ("dz", "dw1", "dw2"):
        assert torch.equal(again[key], got[key]), key


def test_experts_backward_zero_tokens():
    banner("backward T=0")
    cfg, w, x = workloads.make_workload("olmoe", tokens=1, d_model=256, num_experts=8, top_k=2, hidden_size=128)
    D = workloads.storage_dtype(cfg)
    z = torch.empty((0, 256), dtype=D, device="cuda")
    offs = torch.zeros(9, dtype=torch.int32, device="cuda")
    perm = torch.empty(0, dtype=torch.int32, device="cuda")
    saved = {"h": torch.empty((0, 256), dtype=D, device="cuda"), "act": torch.empty((0, 128), dtype=D, device="cuda")}
    out = {"dz": torch.empty((0, 256), dtype=D, device="cuda"),
           "dw1": torch.full((8, 256, 256), 7.0, dtype=D, device="cuda"),
           "dw2": torch.full((8, 256, 128), 7.0, dtype=D, device="cuda")}
    got = moe.experts_backward(cfg, to_device_weights(w), z, offs, perm, saved,
                               torch.empty((0, 256), dtype=D, device="cuda"), out=out)
    torch.cuda.synchronize()
    assert not got["dw1"].any() and not got["dw2"].any()


@pytest.mark.parametrize("case", [("olmoe", 300, dict(d_model=512, num_experts=16, top_k=4, hidden_size=128)),
                                  ("tiny_f32", None, {}),
                                  ("latent896", 100, dict(d_model=512, latent_dim=256, num_experts=32,
                                                          up_proj_input_norm=False))],
                         ids=lambda c: c[0])
def test_combine_backward(case):
    name, T, over = case
    banner(f"combine backward {case}")
    cfg, w, x = workloads.make_workload(name, tokens=T, **over)
    cfgO = O.MoEConfig.from_dict(cfg)
    T = x.shape[0]
    k, K = cfg["top_k"], cfgO.expert_dim
    D = workloads.storage_dtype(cfg)
    g = torch.Generator().manual_seed(5)
    Y = torch.randn((T * k, K), generator=g).mul_(0.3).to(D)
    wts = torch.rand((T, k), generator=g, dtype=torch.float32)
    dO = torch.randn((T, K), generator=g).to(D)
    got = moe.combine_backward(cfg, Y.cuda(), wts.cuda(), dO.cuda())
    torch.cuda.synchronize()
    ref = O.combine_backward(cfgO, np32(Y), wts.numpy(), np32(dO))
    bf = cfg["dtype"] == "bf16"
    # dY: one product rounded once (float64) against fp32-then-D: at most one spacing apart
    assert_close(np32(got["dy_assign"]), ref["dY"], cfg["dtype"], "dY", bf16_spacing(ref["dY"]) if bf else None)
    # dw: an fp32 dot of K terms; bound by K * 2^-24 * sum |dO| |Y| (sequential fp32 summation)
    M = np.einsum("tc,tjc->tj", np.abs(np32(dO)).astype(np.float64),
                  np.abs(np32(Y)).astype(np.float64).reshape(T, k, K))
    dw = got["d_expert_weights"].cpu().numpy().astype(np.float64)
    assert np.all(np.abs(dw - ref["dw"]) <= K * 2.0 ** -24 * M + 1e-30), np.abs(dw - ref["dw"]).max()


@pytest.mark.parametrize("name,skew", [("olmoe", 0.0), ("latent896", 0.0), ("skewed", 1.0)])
def test_full_size_backward_sampled(name, skew):
    """The experts stage at a workload's full size (tokens, experts, top-k, expert width K and
    hidden width), in the launch configuration the bench times: z, the routing and dY drawn by
    seeded generators (skewed: indices tilted towards low experts), the GPU's training forward
    and backward; every gradient finite, 48 sampled tokens' dz and two experts' whole dW1, dW2
    against the oracle, which recomputes everything for those rows from the inputs."""
    banner(f"full-size backward {name}")
    cfg = workloads.layer_config(name)
    cfgO = O.MoEConfig.from_dict(cfg)
    T, k, E, h = workloads.tokens_of(name), cfg["top_k"], cfg["num_experts"], cfg["hidden_size"]
    K = cfgO.expert_dim
    _, w, _ = workloads.make_workload(name, tokens=1, device="cuda")  # weights only
    D = workloads.storage_dtype(cfg)
    g = torch.Generator(device="cuda").manual_seed(21)
    z = torch.randn((T, K), generator=g, device="cuda").to(D)
    dY = torch.randn((T * k, K), generator=g, device="cuda").mul_(0.5).to(D)
    idx = workloads.random_distinct_indices(T, E, k, seed=9, skew=skew).numpy()
    counts = O.expert_counts(idx, E)
    offs = O.expert_offsets(counts)
    perm, inv, _ = O.capacity_permutation(idx, E, None)
    wd = to_device_weights(w)
    fw = moe.experts_forward_train(cfg, wd, z, _idx(offs), _idx(perm))
    got = moe.experts_backward(cfg, wd, z, _idx(offs), _idx(perm), fw, dY)
    torch.cuda.synchronize()
    for key in ("dz", "dw1", "dw2"):
        assert torch.isfinite(got[key].float()).all(), key
    print(f"  T={T} E={E} K={K} h={h} rows per expert min {counts.min()} max {counts.max()}", flush=True)
    rng = np.random.default_rng(4)
    sample = rng.choice(T, 48, replace=False)
    zs = np32(z[torch.from_numpy(sample).cuda()]).astype(np.float64)
    used = np.unique(idx[sample])
    w1 = {int(e): np32(w["w1"][int(e)]).astype(np.float64) for e in used}
    w2 = {int(e): np32(w["w2"][int(e)]).astype(np.float64) for e in used}
    dY_s = np32(dY[torch.from_numpy((sample[:, None] * k + np.arange(k)).ravel()).cuda()]).astype(np.float64)
    dz_ref, Mdz = [], []
    for i, t in enumerate(sample):
        acc, m = np.zeros(K), np.zeros(K)
        for j in range(k):
            e = int(idx[t, j])
            r = O.expert_mlp_train(cfgO, zs[i:i + 1], w1[e], w2[e])
            d_act = O.round_to(dY_s[i * k + j:i * k + j + 1] @ w2[e], "bf16")
            dH = O.swiglu_backward(cfgO, r["H"], d_act)
            acc += O.round_to(dH @ w1[e], "bf16")[0]
            m += (np.abs(dH) @ np.abs(w1[e]))[0]
        dz_ref.append(O.round_to(acc, "bf16"))
        Mdz.append(m)
    assert_grad_close(np32(got["dz"][torch.from_numpy(sample).cuda()]), np.array(dz_ref), np.array(Mdz), "bf16",
                      "dz (sampled tokens)")
    # two experts' weight gradients from all their rows: the smallest non-empty expert and a
    # median one
    nonempty = np.nonzero(counts)[0]
    order = nonempty[np.argsort(counts[nonempty], kind="stable")]
    for e in (int(order[0]), int(order[len(order) // 2])):
        R = perm[offs[e]:offs[e + 1]]
        Rt = torch.from_numpy(R.astype(np.int64)).cuda()
        ze = np32(z[Rt // k]).astype(np.float64)
        dYe = np32(dY[Rt]).astype(np.float64)
        w1e, w2e = np32(w["w1"][e]).astype(np.float64), np32(w["w2"][e]).astype(np.float64)
        r = O.expert_mlp_train(cfgO, ze, w1e, w2e)
        dH = O.swiglu_backward(cfgO, r["H"], O.round_to(dYe @ w2e, "bf16"))
        assert_grad_close(np32(got["dw2"][e]), O.round_to(dYe.T @ r["act"], "bf16"), np.abs(dYe).T @ np.abs(r["act"]),
                          "bf16", f"dw2[{e}] ({R.size} rows)")
        assert_grad_close(np32(got["dw1"][e]), O.round_to(dH.T @ ze, "bf16"), np.abs(dH).T @ np.abs(ze), "bf16",
                          f"dw1[{e}] ({R.size} rows)")
