"""Full-size parity on the five workload layers, in the launch configuration the bench times.

Inputs are drawn on the GPU by the seeded generators. The oracle cannot run whole layers of
this size, so it evaluates a seeded sample of tokens (the layer is token-wise independent:
the oracle's forward on a subset of rows is exactly the full layer's result on those rows),
copying to the host only the experts those tokens use. Every token's routing outputs are
checked against properties that hold at any size (distinct indices, counts = histogram,
offsets = cumsum, permutation stable and inverse consistent).
"""
import time

import numpy as np
import pytest
import torch

import workloads
from oracle import moe_oracle as O
from parity import (assert_close, assert_weights_close, bf16_spacing, check_routing_invariants, flip_allowance,
                    mx_expert_allowance, np32, oracle_inputs, routing_matches, sample_tokens)

pytestmark = pytest.mark.gpu

moe = pytest.importorskip("top_routing_grouped_router_amd")


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.set_device(0)


@pytest.mark.parametrize("name", workloads.CONFIG_ORDER)
def test_full_size_layer(name):
    print(f"[case] full-size {name}", flush=True)
    t0 = time.time()
    cfg, w, x = workloads.make_workload(name, device="cuda")
    T = x.shape[0]
    layer = moe.MoELayer(cfg, w)
    y, r = layer(x, routing=True)
    torch.cuda.synchronize()
    t1 = time.time()
    check_routing_invariants(cfg, r, T)
    counts = r["batch_size_per_expert"].cpu().numpy()
    print(f"  T={T} used experts {int((counts > 0).sum())}/{cfg['num_experts']} "
          f"max/mean load {counts.max() / counts.mean():.2f} max|y| {float(y.float().abs().max()):.3f}",
          flush=True)

    cfgO = O.MoEConfig.from_dict(cfg)
    sample = sample_tokens(T, 96 if T > 96 else T, seed=1)
    xs = np32(x[torch.from_numpy(sample).cuda()])
    wr = np32(w["router_weight"])
    logits = O.router_logits(xs, wr, np32(w["router_bias"]))
    pre = O.route(cfgO, logits, np32(w["score_bias"]))
    experts = np.unique(pre["idx"])
    wo = oracle_inputs(w, experts)
    ref = O.forward(cfgO, wo, xs)
    gi = r["expert_indices"].cpu().numpy()[sample]
    key_tol = 1e-4 * max(1.0, float(np.abs(ref["keys"]).max()))
    same = routing_matches(cfgO, gi, ref, key_tol)
    assert same.mean() >= 0.97, same.mean()
    gw = r["expert_weights"].cpu().numpy()[sample]
    assert_weights_close(gw[same], ref["w"][same])
    ys = np32(y)[sample]
    fa = flip_allowance(cfgO, ref)
    assert_close(ys[same], ref["y"][same], cfg["dtype"], f"full-size {name}",
                 None if fa is None else fa[same])
    print(f"  gpu {t1 - t0:.1f}s oracle+checks {time.time() - t1:.1f}s, {int(same.sum())}/{len(sample)} tokens compared",
          flush=True)


@pytest.mark.parametrize("name", [n for n in workloads.CONFIG_ORDER if n != "tiny_f32"])
def test_full_size_layer_mxfp8(name):
    """The same full-size check with the expert matmuls in MXFP8. MX quantisation is per token
    row (z, activation) and per weight row, so the oracle on a sample of tokens is again the
    full layer on those rows."""
    print(f"[case] full-size mxfp8 {name}", flush=True)
    cfg, w, x = workloads.make_workload(name, device="cuda", expert_precision="mxfp8")
    T = x.shape[0]
    layer = moe.MoELayer(cfg, w)
    y, r = layer(x, routing=True)
    torch.cuda.synchronize()
    check_routing_invariants(cfg, r, T)
    cfgO = O.MoEConfig.from_dict(cfg)
    sample = sample_tokens(T, 64 if T > 64 else T, seed=2)
    xs = np32(x[torch.from_numpy(sample).cuda()])
    logits = O.router_logits(xs, np32(w["router_weight"]), np32(w["router_bias"]))
    pre = O.route(cfgO, logits, np32(w["score_bias"]))
    wo = oracle_inputs(w, np.unique(pre["idx"]))
    ref = O.forward(cfgO, wo, xs)
    gi = r["expert_indices"].cpu().numpy()[sample]
    key_tol = 1e-4 * max(1.0, float(np.abs(ref["keys"]).max()))
    same = routing_matches(cfgO, gi, ref, key_tol)
    assert same.mean() >= 0.97, same.mean()
    allow = None
    if not cfgO.latent_dim:
        a = mx_expert_allowance(cfgO, ref, wo) + bf16_spacing(ref["Y"])
        n = len(sample)
        allow = (np.abs(ref["w"])[:, :, None] * a[np.asarray(ref["inv"]).reshape(n, -1)]).sum(axis=1)[same]
    ys = np32(y)[sample]
    d = np.abs(ys[same] - ref["y"][same])
    print(f"  max-abs {d.max():.3e} rel-fro {np.linalg.norm(ys[same] - ref['y'][same]) / np.linalg.norm(ref['y'][same]):.3e}",
          flush=True)
    assert_close(ys[same], ref["y"][same], "bf16", f"full-size mxfp8 {name}", allow,
                 budget_share=None if allow is None else 1.0)
