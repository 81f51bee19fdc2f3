"""Full-size parity on the five workload layers, in the launch configuration the bench times.

Inputs are drawn on the GPU by the seeded generators. Every token's routing is checked bit for
bit: the selection against the oracle's selection run on the GPU's own fp32 gating output, the
counts, offsets, permutation and inverse against the oracle's on those indices, the weights
and gating scores within derived fp32 ulps (tests/parity.py). The oracle cannot run whole
layers of this size, so the values are compared on a seeded sample of tokens: the layer is
token-wise independent, so the oracle's expert path on those rows, driven by the GPU's
indices and weights, is exactly the full layer's result on those rows; it copies to the
host only the experts those tokens use. The router logits of the sample are held to the fp32
dot-product bound, and the GPU's selection is compared with the pure oracle's (its own
float64-summed logits), which may differ only on near-ties.
"""
import time

import numpy as np
import pytest
import torch

import workloads
from oracle import moe_oracle as O
from parity import (assert_close, bf16_spacing, check_forward_routing, check_routing_invariants, flip_allowance,
                    logit_bound, mx_expert_allowance, np32, oracle_from_gpu_routing, oracle_inputs, routing_agreement,
                    sample_tokens)

pytestmark = pytest.mark.gpu

moe = pytest.importorskip("top_routing_grouped_router_amd")


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.set_device(0)


def _sampled_checks(cfg, w, x, r, sample):
    """Logit bound and pure-oracle agreement on the sampled tokens; returns the oracle driven by
    the GPU's routing on those tokens, and the host weights of the experts they use."""
    cfgO = O.MoEConfig.from_dict(cfg)
    xs = np32(x[torch.from_numpy(sample).cuda()])
    wr = np32(w["router_weight"])
    ref_l = O.router_logits(xs, wr, np32(w["router_bias"]))
    got_l = r["router_logits"][torch.from_numpy(sample).cuda()].cpu().numpy().astype(np.float64)
    bound = logit_bound(xs, wr, cfg["dtype"] == "bf16") + np.abs(ref_l) * 2.0 ** -23
    assert np.all(np.abs(got_l - ref_l) <= bound), np.max(np.abs(got_l - ref_l) / bound)
    sb = np32(w["score_bias"])
    pure = O.route(cfgO, ref_l, sb)
    got_s = r["router_scores"][torch.from_numpy(sample).cuda()].cpu().numpy()
    same = routing_agreement(r["expert_indices"].cpu().numpy()[sample], pure,
                             O.selection_keys(cfgO, got_l, got_s, sb))
    gi = r["expert_indices"].cpu().numpy()[sample]
    gw = r["expert_weights"].cpu().numpy()[sample]
    wo = oracle_inputs(w, np.unique(gi))
    ref = oracle_from_gpu_routing(cfgO, wo, xs, gi, gw)
    print(f"  selection equal to the pure oracle's on {int(same.sum())}/{len(sample)} sampled tokens", flush=True)
    assert same.mean() >= 0.97, same.mean()
    return cfgO, ref, wo


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
    check_forward_routing(O.MoEConfig.from_dict(cfg), r, w["score_bias"])
    sample = sample_tokens(T, 96 if T > 96 else T, seed=1)
    cfgO, ref, _ = _sampled_checks(cfg, w, x, r, sample)
    ys = np32(y)[sample]
    assert_close(ys, ref["y"], cfg["dtype"], f"full-size {name}", flip_allowance(cfgO, ref))
    print(f"  gpu {t1 - t0:.1f}s oracle+checks {time.time() - t1:.1f}s, {len(sample)} tokens compared", flush=True)


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
    check_forward_routing(O.MoEConfig.from_dict(cfg), r, w["score_bias"])
    sample = sample_tokens(T, 64 if T > 64 else T, seed=2)
    cfgO, ref, wo = _sampled_checks(cfg, w, x, r, sample)
    allow = None
    if not cfgO.latent_dim:
        a = mx_expert_allowance(cfgO, ref, wo) + bf16_spacing(ref["Y"])
        n = len(sample)
        allow = (np.abs(ref["w"])[:, :, None] * a[np.asarray(ref["inv"]).reshape(n, -1)]).sum(axis=1)
    ys = np32(y)[sample]
    d = np.abs(ys - ref["y"])
    print(f"  max-abs {d.max():.3e} rel-fro {np.linalg.norm(ys - ref['y']) / np.linalg.norm(ref['y']):.3e}",
          flush=True)
    assert_close(ys, ref["y"], "bf16", f"full-size mxfp8 {name}", allow,
                 budget_share=None if allow is None else 1.0)
