"""GPU parity of the MXFP8 path against the CPU oracle, through the C ABI.

OCP microscaling read of "Как устроен Olmo-core 3: обучение больших MoE-моделей", section
"Rowwise FP8 и MXFP8": E4M3 elements and E8M0 scales over blocks of 32. Quantisation is an
integer decision taken on identical bf16 inputs, so codes and scales are compared bit for bit.
"""
import numpy as np
import pytest
import torch

from oracle import moe_oracle as O

pytestmark = pytest.mark.gpu

moe = pytest.importorskip("top_routing_grouped_router_amd")


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.set_device(0)


def banner(msg):
    print(f"[case] {msg}", flush=True)


QUANT_CASES = [(1, 32, 1.0), (7, 2048, 1.0), (300, 1024, 0.02), (64, 4096, 30.0), (5, 96, 1e-30)]


@pytest.mark.parametrize("rows,cols,std", QUANT_CASES)
def test_mx_quantize_bitexact(rows, cols, std):
    banner(f"mx_quantize {rows}x{cols} std {std}")
    g = torch.Generator().manual_seed(rows * 7 + cols)
    x = (torch.randn(rows, cols, generator=g, dtype=torch.float64) * std)
    x[0, :32] = 0.0                                   # an all-zero block
    if cols >= 64:
        x[0, 32:64] = torch.linspace(-448, 448, 32, dtype=torch.float64) * std  # saturating edges
    xb = x.to(torch.bfloat16)
    codes, scales = moe.mx_quantize(xb.cuda())
    torch.cuda.synchronize()
    want_c, want_s = O.mx_quantize(xb.to(torch.float64).numpy())
    assert np.array_equal(scales.cpu().numpy(), want_s)
    assert np.array_equal(codes.cpu().numpy(), want_c)


from parity import (assert_close, bf16_spacing, check_forward_routing, check_routing_invariants,  # noqa: E402
                    mx_expert_allowance, np32, oracle_from_gpu_routing, oracle_inputs, to_device_weights)
import workloads  # noqa: E402


def mx_error_report(got, ref, what):
    d = np.abs(got - ref)
    fro = np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-30)
    print(f"  {what}: max-abs {d.max():.3e}, rel-fro {fro:.3e}, max|ref| {np.abs(ref).max():.3f}", flush=True)


STAGE_CASES = [
    ("olmoe", 600, dict(d_model=512, num_experts=16, top_k=4, hidden_size=256)),
    ("olmoe", 1000, dict(d_model=2048, num_experts=8, top_k=2, hidden_size=1024)),
    ("latent896", 300, dict(d_model=512, latent_dim=256, num_experts=64, hidden_size=128)),
]


@pytest.mark.parametrize("case", STAGE_CASES, ids=lambda c: f"{c[0]}-{c[1]}")
def test_experts_stage_mxfp8(case):
    """The MXFP8 experts stage against the oracle's MXFP8 expert path on the same z and the same
    routing (no near-tie can differ)."""
    name, T, over = case
    banner(f"experts mxfp8 {case}")
    cfg, w, x = workloads.make_workload(name, tokens=T, expert_precision="mxfp8", **over)
    K = cfg["latent_dim"] or cfg["d_model"]
    wd = moe.quantize_expert_weights(to_device_weights(w))
    g = torch.Generator().manual_seed(T)
    z = torch.randn(T, K, generator=g).to(torch.bfloat16)
    idx = workloads.random_distinct_indices(T, cfg["num_experts"], cfg["top_k"], skew=0.5)
    r = moe.permute(cfg, idx.cuda())
    ya = moe.experts_forward(cfg, wd, z.cuda(), r["expert_offsets"], r["permutation"])
    torch.cuda.synchronize()
    cfgO = O.MoEConfig.from_dict(cfg)
    wo = oracle_inputs(w)
    ex = O.run_experts(cfgO, np32(z), idx.numpy(), wo["w1"], wo["w2"])
    ref = ex["Y"][ex["inv"]]          # assignment order
    allow = mx_expert_allowance(cfgO, ex, wo)[ex["inv"]]
    got = np32(ya)
    mx_error_report(got, ref, f"Y {name}")
    assert_close(got, ref, "bf16", f"experts mxfp8 {name}", allow, budget_share=1.0)


LAYER_MX_CASES = [
    ("olmoe", 700, dict(d_model=512, num_experts=16, top_k=4, hidden_size=256)),
    ("latent896", 400, dict(d_model=1024, latent_dim=256, num_experts=128, hidden_size=128)),
    ("skewed", 600, dict(d_model=512, num_experts=64, top_k=8, hidden_size=256)),
]


@pytest.mark.parametrize("case", LAYER_MX_CASES, ids=lambda c: f"{c[0]}-{c[1]}")
def test_layer_mxfp8(case):
    name, T, over = case
    banner(f"layer mxfp8 {case}")
    cfg, w, x = workloads.make_workload(name, tokens=T, expert_precision="mxfp8", **over)
    cfgO = O.MoEConfig.from_dict(cfg)
    layer = moe.MoELayer(cfg, to_device_weights(w))
    y, r = layer(x.cuda(), routing=True)
    torch.cuda.synchronize()
    check_routing_invariants(cfg, r, T)
    check_forward_routing(cfgO, r, w["score_bias"])
    wo = oracle_inputs(w)
    gi, gw = r["expert_indices"].cpu().numpy(), r["expert_weights"].cpu().numpy()
    ref = oracle_from_gpu_routing(cfgO, wo, np32(x), gi, gw)
    mx_error_report(np32(y), ref["y"], f"layer {name}")
    allow = None
    if not cfgO.latent_dim:
        # through the combine: sum_j |w_j| (allowance of Y_j + one bf16 spacing of Y_j)
        a = mx_expert_allowance(cfgO, ref, wo) + bf16_spacing(ref["Y"])
        allow = (np.abs(ref["w"])[:, :, None] * a[np.asarray(ref["inv"]).reshape(T, -1)]).sum(axis=1)
    assert_close(np32(y), ref["y"], "bf16", f"layer mxfp8 {name}", allow,
                 budget_share=None if allow is None else 1.0)
