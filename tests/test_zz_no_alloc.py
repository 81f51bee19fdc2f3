"""The allocation-free whole-layer entry point (moe_forward_noalloc) against moe_forward.

Both run the same kernels on the same inputs, so every output -- y and all routing outputs --
must be equal bit for bit. Each case makes two calls in a row on the shared per-GPU scratch
array, the second with fewer tokens, so the second call runs on what the first one left
there. A layer whose workspace exceeds the array is refused before any launch.
"""
import numpy as np
import pytest
import torch

import workloads
from oracle import moe_oracle as O
from parity import assert_close, np32, oracle_from_gpu_routing, oracle_inputs, to_device_weights

pytestmark = pytest.mark.gpu

moe = pytest.importorskip("top_routing_grouped_router_amd")


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.set_device(0)


CASES = [
    # (workload, token counts of the two calls, shape overrides)
    ("decode", (64, 17), {}),                                     # the serving shape, full size
    ("olmoe", (1500, 700), dict(d_model=512, num_experts=16, top_k=4, hidden_size=256)),
    ("latent896", (300, 96), dict(d_model=1024, latent_dim=256, num_experts=128, hidden_size=128)),
    ("tiny_f32", (256, 37), {}),
]


def _routing_buffers(cfg, T, device):
    return moe._routing_tensors(moe.MoEConfig.of(cfg), T, device)


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"{c[0]}-{c[1][0]}-{c[1][1]}")
def test_noalloc_matches_forward(case):
    name, token_counts, over = case
    print(f"[case] noalloc {name} {token_counts}", flush=True)
    T0 = max(token_counts)
    cfg, w, x = workloads.make_workload(name, tokens=T0, device="cuda", **over)
    layer = moe.MoELayer(cfg, w)
    for T in token_counts:
        assert moe.workspace_size(cfg, T) <= moe.NOALLOC_SCRATCH_BYTES
        xt = x[:T].contiguous()
        y_ref, r_ref = layer(xt, routing=True)
        y = torch.empty_like(xt)
        r = _routing_buffers(cfg, T, xt.device)
        layer.forward_noalloc(xt, y, routing=r)
        torch.cuda.synchronize()
        assert torch.equal(y, y_ref), f"{name} T={T}: y differs from moe_forward"
        for k in r_ref:
            assert torch.equal(r[k], r_ref[k]), f"{name} T={T}: {k} differs from moe_forward"
        # and the oracle driven by this routing, on a few tokens, to the layer tolerance
        cfgO = O.MoEConfig.from_dict(cfg)
        rows = np.unique(np.linspace(0, T - 1, min(T, 16)).astype(np.int64))
        gi = r["expert_indices"].cpu().numpy()[rows]
        gw = r["expert_weights"].cpu().numpy()[rows]
        ref = oracle_from_gpu_routing(cfgO, oracle_inputs(w, np.unique(gi)), np32(xt)[rows], gi, gw)
        assert_close(np32(y)[rows], ref["y"], cfg["dtype"], f"noalloc {name} T={T}")
    # without routing outputs as well
    y2 = torch.empty_like(x[:token_counts[-1]])
    layer.forward_noalloc(x[:token_counts[-1]].contiguous(), y2)
    torch.cuda.synchronize()
    assert torch.equal(y2, y_ref)


def test_noalloc_refuses_large_workspace():
    cfg, w, x = workloads.make_workload("olmoe", tokens=8, d_model=256, num_experts=8, top_k=2, hidden_size=128)
    layer = moe.MoELayer(cfg, to_device_weights(w))
    T = 200000  # needs far more than the scratch array
    assert moe.workspace_size(cfg, T) > moe.NOALLOC_SCRATCH_BYTES
    xb = torch.empty((T, 256), dtype=torch.bfloat16, device="cuda")
    y = torch.empty_like(xb)
    with pytest.raises(moe.MoEError) as ei:
        layer.forward_noalloc(xb, y)
    assert ei.value.status == 3  # MOE_ERR_WORKSPACE_TOO_SMALL
    # zero tokens: nothing to do
    layer.forward_noalloc(xb[:0], y[:0])
