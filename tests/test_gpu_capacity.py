"""GPU parity of expert capacity with token dropping against the CPU oracle, through the C ABI.

Page "Как устроен Olmo-core 3: обучение больших MoE-моделей", section "Ёмкость эксперта и
переполнение": capacity = roundup8(capacity_factor * top_k * T / E) at expert-parallel degree 1;
each expert keeps the first `capacity` assignments of the stable order; dropped assignments
contribute nothing. Counts, offsets and permutations are compared bit for bit; layer outputs to
the layer tolerance, with the oracle's expert path driven by the GPU's own routing (a
near-tie that routes one token differently would otherwise change which later tokens an
expert keeps).
"""
import numpy as np
import pytest
import torch

import workloads
from oracle import moe_oracle as O
from parity import assert_close, check_routing_invariants, flip_allowance, np32, oracle_inputs, to_device_weights

pytestmark = pytest.mark.gpu

moe = pytest.importorskip("top_routing_grouped_router_amd")


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.set_device(0)


def banner(msg):
    print(f"[case] {msg}", flush=True)


PERMUTE_CASES = [
    # (T, E, k, skew, capacity_factor); T <= 1024 runs the one-workgroup dispatch
    (1000, 64, 8, 1.0, 1.0),
    (777, 16, 4, 2.0, 0.5),
    (4097, 256, 8, 2.5, 1.25),
    (3000, 8, 2, 1.5, 1.0),
    (50, 1, 1, 0.0, 0.5),
    (2048, 896, 8, 1.0, 2.0),
    (1025, 32, 4, 0.0, 1.0),
    (300, 1024, 16, 0.5, 0.75),
]


@pytest.mark.parametrize("case", PERMUTE_CASES, ids=lambda c: f"T{c[0]}-E{c[1]}-k{c[2]}-skew{c[3]}-cf{c[4]}")
def test_permute_capacity_bitexact(case):
    T, E, k, skew, cf = case
    banner(f"permute capacity {case}")
    idx = workloads.random_distinct_indices(T, E, k, skew=skew)
    cfg = dict(d_model=64, num_experts=E, top_k=k, hidden_size=64, dtype="bf16", capacity_factor=cf)
    C = O.expert_capacity(O.MoEConfig.from_dict(cfg), T)
    r = moe.permute(cfg, idx.cuda())
    torch.cuda.synchronize()
    counts = O.expert_counts(idx.numpy(), E)
    perm, inv, kept = O.capacity_permutation(idx.numpy(), E, C)
    assert np.array_equal(r["batch_size_per_expert"].cpu().numpy(), counts)
    assert np.array_equal(r["expert_offsets"].cpu().numpy(), O.expert_offsets(np.minimum(counts, C)))
    assert np.array_equal(r["permutation"].cpu().numpy(), perm)
    assert np.array_equal(r["inverse_permutation"].cpu().numpy(), inv)


LAYER_CASES = [
    ("tiny_f32", None, dict(capacity_factor=0.5)),
    ("olmoe", 600, dict(d_model=512, num_experts=16, top_k=4, hidden_size=256, capacity_factor=0.75)),
    ("latent896", 400, dict(d_model=1024, latent_dim=256, num_experts=128, hidden_size=128, capacity_factor=1.0)),
    ("skewed", 1500, dict(d_model=512, num_experts=64, top_k=8, hidden_size=256, capacity_factor=1.0)),
    ("decode", None, dict(d_model=1024, latent_dim=256, num_experts=32, hidden_size=128, capacity_factor=0.5)),
    ("olmoe", 300, dict(d_model=256, num_experts=8, top_k=2, hidden_size=128, capacity_factor=100.0)),
]


def oracle_from_gpu_routing(cfg, w, x, idx, wts):
    """The oracle's expert path and restore, driven by the GPU's indices and weights."""
    cfgO = O.MoEConfig.from_dict(cfg)
    wo = oracle_inputs(w)
    T = x.shape[0]
    C = O.expert_capacity(cfgO, T)
    z = O.prepare_routed_input(cfgO, np32(x), wo.get("down_proj"))
    ex = O.run_experts(cfgO, z, idx, wo["w1"], wo["w2"], C)
    o = O.combine(cfgO, ex["Y"], ex["inv"], wts)
    out = O.restore_routed_output(cfgO, o, wo.get("norm_weight"), wo.get("up_proj"))
    return C, ex, out["y"]


@pytest.mark.parametrize("case", LAYER_CASES,
                         ids=lambda c: f"{c[0]}-{c[1]}-{'-'.join(f'{k}{v}' for k, v in c[2].items())}")
def test_layer_capacity(case):
    name, T, over = case
    banner(f"layer capacity {case}")
    cfg, w, x = workloads.make_workload(name, tokens=T, **over)
    layer = moe.MoELayer(cfg, to_device_weights(w))
    y, r = layer(x.cuda(), routing=True)
    torch.cuda.synchronize()
    T = x.shape[0]
    idx = r["expert_indices"].cpu().numpy()
    wts = r["expert_weights"].cpu().numpy()
    C, ex, ref = oracle_from_gpu_routing(cfg, w, x, idx, wts)
    assert moe.expert_capacity(cfg, T) == min(C, (T + 7) // 8 * 8)
    check_routing_invariants(cfg, r, T, capacity=C)
    assert np.array_equal(r["permutation"].cpu().numpy(), ex["perm"])
    if over["capacity_factor"] < 10:
        assert not ex["kept"].all(), "the case must drop something"
    fa = flip_allowance(O.MoEConfig.from_dict(cfg), dict(w=wts, Y=ex["Y"], inv=ex["inv"]))
    assert_close(np32(y), ref, cfg["dtype"], f"layer capacity {name}", fa)


def test_experts_stage_zeroes_dropped_rows():
    banner("experts stage with capacity")
    cfg, w, x = workloads.make_workload("olmoe", tokens=500, d_model=256, num_experts=8, top_k=2, hidden_size=128,
                                        capacity_factor=0.5)
    wd = to_device_weights(w)
    idx = workloads.random_distinct_indices(500, 8, 2, skew=1.5)
    r = moe.permute(cfg, idx.cuda())
    ya = moe.experts_forward(cfg, wd, x.cuda(), r["expert_offsets"], r["permutation"])
    torch.cuda.synchronize()
    cfgO = O.MoEConfig.from_dict(cfg)
    C = O.expert_capacity(cfgO, 500)
    ex = O.run_experts(cfgO, np32(x), idx.numpy(), oracle_inputs(w)["w1"], oracle_inputs(w)["w2"], C)
    got = np32(ya)
    dropped = ~ex["kept"]
    assert dropped.any()
    assert np.all(got[dropped] == 0.0)
    kept_rows = np.nonzero(ex["kept"])[0]
    assert_close(got[kept_rows], ex["Y"][ex["inv"][kept_rows]], "bf16", "experts capacity")
