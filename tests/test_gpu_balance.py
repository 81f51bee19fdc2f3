"""GPU parity of the router's load-balancing state against the CPU oracle, through the C ABI.

Page "Как устроен Olmo-core 3: обучение больших MoE-моделей", section "Счётчики и
bias-корректировка": the count accumulator, the load imbalance max/mean and the score_bias
update by bias_gamma * sign(ideal - actual). Everything is integer arithmetic except the fp64
imbalance (one correctly rounded division on both sides) and the fp32 bias add (one add on both
sides), so every comparison is bit-exact.
"""
import numpy as np
import pytest
import torch

import workloads
from oracle import moe_oracle as O

pytestmark = pytest.mark.gpu

moe = pytest.importorskip("top_routing_grouped_router_amd")

E_CASES = (1, 2, 7, 64, 256, 896, 1024)
KINDS = ("uniform", "hot", "zipf", "random", "sparse", "zero")


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.set_device(0)


def banner(msg):
    print(f"[case] {msg}", flush=True)


def same_double(a, b):
    return (np.isnan(a) and np.isnan(b)) or a == b


@pytest.mark.parametrize("E", E_CASES)
@pytest.mark.parametrize("kind", KINDS)
def test_load_imbalance_bitexact(E, kind):
    banner(f"load_imbalance E={E} {kind}")
    c = workloads.synthetic_counts(E, kind, seed=7)
    got = moe.load_imbalance(torch.from_numpy(c).cuda()).item()
    assert same_double(got, O.load_imbalance(c)), (got, O.load_imbalance(c))


@pytest.mark.parametrize("E", E_CASES)
@pytest.mark.parametrize("kind", KINDS)
def test_score_bias_update_bitexact(E, kind):
    banner(f"score_bias_update E={E} {kind}")
    c = workloads.synthetic_counts(E, kind, seed=9)
    b = (np.random.default_rng(E + 1).standard_normal(E) * 0.1).astype(np.float32)
    b[0] = -0.0  # a signed zero: the fp32 add of +0 on both sides
    gamma = 1e-3
    acc = torch.from_numpy(c).cuda()
    bias = torch.from_numpy(b).cuda()
    imb = moe.score_bias_update(acc, bias, gamma, imbalance=True)
    torch.cuda.synchronize()
    want = O.score_bias_update(b, c, gamma)
    assert np.array_equal(bias.cpu().numpy().view(np.uint32), want.view(np.uint32))
    assert same_double(imb.item(), O.load_imbalance(c))
    assert torch.count_nonzero(acc).item() == 0, "the accumulator is reset after the update"


def test_bias_update_loop_over_layer_forwards():
    """Counts of several forward passes accumulate; the step's update follows; the next step
    starts from zero. Driven by the layer's own routing, checked against the oracle on the same
    counts (the GPU's counts are first checked against the GPU's indices)."""
    banner("score_bias loop over moe_forward")
    cfg, w, _ = workloads.make_workload("latent896", tokens=96, d_model=512, latent_dim=128, num_experts=32,
                                        top_k=4, hidden_size=128)
    E = cfg["num_experts"]
    wd = {k: (None if v is None else v.cuda()) for k, v in w.items()}
    layer = moe.MoELayer(cfg, wd)
    acc = torch.zeros(E, dtype=torch.int64, device="cuda")
    bias = wd["score_bias"].clone()
    acc_ref = np.zeros(E, dtype=np.int64)
    bias_ref = bias.cpu().numpy()
    g = torch.Generator(device="cpu")
    for step in range(3):
        for mb in range(2):
            g.manual_seed(100 * step + mb)
            x = torch.randn(96, cfg["d_model"], generator=g).to(torch.bfloat16).cuda()
            _, r = layer(x, routing=("expert_indices", "batch_size_per_expert"))
            moe.accumulate_expert_counts(r["batch_size_per_expert"], acc)
            counts = r["batch_size_per_expert"].cpu().numpy()
            assert np.array_equal(counts, O.expert_counts(r["expert_indices"].cpu().numpy(), E))
            acc_ref = O.accumulate_counts(acc_ref, counts)
        assert np.array_equal(acc.cpu().numpy(), acc_ref)
        imb = moe.score_bias_update(acc, bias, 1e-2, imbalance=True)
        torch.cuda.synchronize()
        bias_ref = O.score_bias_update(bias_ref, acc_ref, 1e-2)
        assert same_double(imb.item(), O.load_imbalance(acc_ref))
        acc_ref = np.zeros(E, dtype=np.int64)
        assert np.array_equal(bias.cpu().numpy().view(np.uint32), bias_ref.view(np.uint32))
        assert torch.count_nonzero(acc).item() == 0
