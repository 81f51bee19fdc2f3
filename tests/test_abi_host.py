"""Host-side checks of the C ABI: the library loads, exports every entry point the header
declares, and validates arguments before any HIP call (so these run without a GPU).
Parameter counts are checked against the CPU oracle and the golden table."""
import ctypes
import os
import re
import subprocess

import pytest

import workloads
from oracle import moe_oracle as O

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe_mi355x.h")

moe = pytest.importorskip("top_routing_grouped_router_amd",
                          reason="HIP library not built (run __graft_entry__.build())")


def declared_symbols():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^MOE_API\s+[\w\s\*]+?\b(moe_\w+)\(", text, flags=re.M)))


def test_header_declares_the_abi():
    syms = declared_symbols()
    for name in ("moe_forward", "moe_forward_noalloc", "moe_router_forward", "moe_route_from_scores", "moe_permute",
                 "moe_experts_forward", "moe_combine", "moe_latent_down", "moe_latent_up",
                 "moe_config_default", "moe_config_validate", "moe_num_params",
                 "moe_workspace_size", "moe_status_string", "moe_last_error_message",
                 "moe_abi_version", "moe_accumulate_expert_counts", "moe_load_imbalance",
                 "moe_score_bias_update", "moe_expert_capacity", "moe_experts_forward_train",
                 "moe_experts_backward", "moe_experts_backward_workspace_size", "moe_combine_backward",
                 "moe_calibrate_mfma_bf16", "moe_calibrate_mfma_mxfp8", "moe_calibrate_copy"):
        assert name in syms


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(moe.LIB_PATH)
    for name in declared_symbols():
        assert hasattr(lib, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", moe.LIB_PATH], capture_output=True,
                         text=True).stdout
    exported = set(re.findall(r"\sT\s(moe_\w+)$", out, flags=re.M))
    assert set(declared_symbols()) <= exported
    # nothing but the ABI is exported from the library's own code
    assert all(s.startswith("moe_") for s in exported)


def test_abi_version_and_struct_size():
    assert moe.abi_version() == 7
    c = moe._CConfig()
    assert moe._config_default(ctypes.byref(c)) == 0
    assert c.struct_size == ctypes.sizeof(moe._CConfig)
    assert c.num_experts == 1 and c.hidden_size == 256 and c.top_k == 1
    assert c.dtype == 1 and c.up_proj_input_norm == 1


def _status(fn, *args):
    return fn(*args)


def test_validation_rejects_bad_configs():
    base = dict(d_model=256, num_experts=8, top_k=2, hidden_size=128)
    moe.validate(base)
    bad = [
        (dict(top_k=9), 1), (dict(d_model=0), 1), (dict(hidden_size=-64), 1),
        (dict(num_experts=2048, top_k=2), 2), (dict(top_k=17, num_experts=32), 2),
        (dict(d_model=100), 2), (dict(hidden_size=96), 2), (dict(latent_dim=96), 2),
        (dict(normalize_expert_weights=-1.0), 1), (dict(sigmoid_stability_epsilon=-1e-6), 1),
        (dict(dtype="f32", d_model=258), 2),
    ]
    for over, status in bad:
        with pytest.raises(moe.MoEError) as ei:
            moe.validate({**base, **over})
        assert ei.value.status == status, over
    moe.validate({**base, "dtype": "f32", "d_model": 260, "hidden_size": 36})
    c = moe.MoEConfig.of(base).to_c()
    c.struct_size = 8
    assert moe._config_validate(ctypes.byref(c)) == 1
    assert b"struct_size" in moe._last_error()
    c = moe.MoEConfig.of(base).to_c()
    c.activation = 3
    assert moe._config_validate(ctypes.byref(c)) == 2
    assert moe._config_validate(None) == 1
    assert moe._status_string(3) == b"workspace too small"


@pytest.mark.parametrize("name", workloads.CONFIG_ORDER)
def test_num_params_matches_oracle(name):
    cfg = workloads.layer_config(name)
    total, active = moe.num_params(cfg)
    ref = O.num_params(O.MoEConfig.from_dict(cfg))
    assert (total, active) == (ref["total"], ref["active"])


def test_workspace_size_limits():
    cfg = workloads.layer_config("olmoe")
    a = moe.workspace_size(cfg, 1024)
    b = moe.workspace_size(cfg, 8192)
    assert 0 < a < b
    assert moe.workspace_size(cfg, 0) >= 0
    with pytest.raises(moe.MoEError):
        moe.workspace_size(cfg, (1 << 31) // 8)
    with pytest.raises(moe.MoEError):
        moe.workspace_size(cfg, -1)


def test_forward_argument_errors_before_any_gpu_call():
    cfg = moe.MoEConfig.of(workloads.layer_config("olmoe"))
    c = cfg.to_c()
    fake = ctypes.c_void_p(0x10000)
    w = moe._CWeights()
    T = 128
    # missing weights
    assert moe._forward(ctypes.byref(c), None, T, fake, fake, None, fake, 1 << 40, None) == 1
    assert b"weights" in moe._last_error()
    w.router_weight = fake
    assert moe._forward(ctypes.byref(c), ctypes.byref(w), T, fake, fake, None, fake, 1 << 40, None) == 1
    assert b"w1" in moe._last_error()
    w.w1 = fake
    w.w2 = fake
    # missing x / workspace
    assert moe._forward(ctypes.byref(c), ctypes.byref(w), T, None, fake, None, fake, 1 << 40, None) == 1
    assert moe._forward(ctypes.byref(c), ctypes.byref(w), T, fake, fake, None, None, 1 << 40, None) == 1
    # short workspace
    need = moe.workspace_size(cfg, T)
    assert moe._forward(ctypes.byref(c), ctypes.byref(w), T, fake, fake, None, fake, need - 1, None) == 3
    # T = 0 is a no-op, T*k too large is rejected
    assert moe._forward(ctypes.byref(c), ctypes.byref(w), 0, None, None, None, None, 0, None) == 0
    assert moe._forward(ctypes.byref(c), ctypes.byref(w), 1 << 29, fake, fake, None, fake, 1 << 62, None) == 1
    # latent layer without its projections
    lat = moe.MoEConfig.of(workloads.layer_config("latent896")).to_c()
    assert moe._forward(ctypes.byref(lat), ctypes.byref(w), T, fake, fake, None, fake, 1 << 40, None) == 1
    assert b"down_proj" in moe._last_error()
    # stage calls
    assert moe._route_from_scores(ctypes.byref(c), T, fake, None, None, fake, None) == 1
    assert moe._latent_down(ctypes.byref(c), ctypes.byref(w), T, fake, fake, None, 0, None) == 2
    assert moe._latent_up(ctypes.byref(c), ctypes.byref(w), T, fake, fake, None, 0, None) == 2
    # a workspace that is given must be whole
    assert moe._latent_down(ctypes.byref(lat), ctypes.byref(w), T, fake, fake, fake, 16, None) == 1
    wl = moe._CWeights()
    wl.down_proj = wl.up_proj = fake
    need_l = moe.workspace_size(workloads.layer_config("latent896"), T)
    assert moe._latent_down(ctypes.byref(lat), ctypes.byref(wl), T, fake, fake, fake, need_l - 1, None) == 3
    assert moe._latent_up(ctypes.byref(lat), ctypes.byref(wl), T, fake, fake, fake, need_l - 1, None) == 3
    assert moe._permute(ctypes.byref(c), T, fake, fake, fake, fake, fake, fake, 16, None) == 3


def test_forward_noalloc_errors_before_any_gpu_call():
    """The allocation-free forward checks its arguments and the scratch size on the host: a
    layer whose workspace exceeds MOE_NOALLOC_SCRATCH_BYTES is refused before any HIP call."""
    cfg = moe.MoEConfig.of(workloads.layer_config("olmoe"))
    c = cfg.to_c()
    fake = ctypes.c_void_p(0x10000)  # never dereferenced: every call below fails on the host
    w = moe._CWeights()
    T = 8192
    assert moe.workspace_size(cfg, T) > moe.NOALLOC_SCRATCH_BYTES
    assert moe._forward_noalloc(ctypes.byref(c), None, T, fake, fake, None, None) == 1
    w.router_weight = w.w1 = w.w2 = fake
    assert moe._forward_noalloc(ctypes.byref(c), ctypes.byref(w), T, None, fake, None, None) == 1
    assert moe._forward_noalloc(ctypes.byref(c), ctypes.byref(w), T, fake, None, None, None) == 1
    assert moe._forward_noalloc(ctypes.byref(c), ctypes.byref(w), T, fake, fake, None, None) == 3
    msg = moe._last_error().decode()
    assert "allocation-free" in msg and str(moe.NOALLOC_SCRATCH_BYTES) in msg
    assert moe._forward_noalloc(ctypes.byref(c), ctypes.byref(w), 0, None, None, None, None) == 0
    assert moe._forward_noalloc(None, ctypes.byref(w), T, fake, fake, None, None) == 1


def test_balancing_entry_points_validate_before_any_gpu_call():
    fake = ctypes.c_void_p(0x1000)  # never dereferenced: every call below fails validation
    for E in (0, -1, 1025):
        assert moe._accumulate_counts(E, fake, fake, None) == 1
        assert moe._load_imbalance(E, fake, fake, None) == 1
        assert moe._score_bias_update(E, 0.1, fake, fake, None, None) == 1
        assert "num_experts" in moe._last_error().decode()
    assert moe._accumulate_counts(8, None, fake, None) == 1
    assert moe._accumulate_counts(8, fake, None, None) == 1
    assert moe._load_imbalance(8, None, fake, None) == 1
    assert moe._load_imbalance(8, fake, None, None) == 1
    assert moe._score_bias_update(8, 0.1, None, fake, None, None) == 1
    assert moe._score_bias_update(8, 0.1, fake, None, None, None) == 1
    for g in (float("nan"), float("inf"), -float("inf")):
        assert moe._score_bias_update(8, g, fake, fake, None, None) == 1
        assert "bias_gamma" in moe._last_error().decode()


CAPACITY_HOST_CASES = [(cf, k, T, E) for cf in (0.25, 0.5, 0.75, 1.0, 1.1, 1.25, 1.5, 2.0, 3.3, 1e-6, 7.0)
                       for (k, T, E) in ((8, 8192, 64), (2, 100, 8), (1, 1, 1024), (8, 16384, 896),
                                         (4, 97, 32), (16, 12345, 1000), (1, 5, 1))]


@pytest.mark.parametrize("cf,k,T,E", CAPACITY_HOST_CASES)
def test_expert_capacity_host_matches_oracle(cf, k, T, E):
    """The library's host-side capacity (exact integer arithmetic) equals the oracle's exact
    rational one; capacities of T or more drop nothing and are reported as T rounded up to 8."""
    cfg = dict(d_model=64, num_experts=E, top_k=min(k, E), hidden_size=64, capacity_factor=cf)
    want = O.expert_capacity(O.MoEConfig.from_dict(cfg), T)
    got = moe.expert_capacity(cfg, T)
    if want >= T:
        assert got == (T + 7) // 8 * 8
    else:
        assert got == want
    assert moe.expert_capacity(dict(cfg, capacity_factor=None), T) == 0


def test_capacity_factor_validation():
    for bad in (-1.0, float("nan"), float("inf")):
        with pytest.raises(moe.MoEError):
            moe.validate(dict(d_model=64, num_experts=4, top_k=2, hidden_size=64, capacity_factor=bad))


def test_backward_entry_points_validate_before_any_gpu_call():
    fake = ctypes.c_void_p(0x10000)  # never dereferenced: every call below fails validation
    cfg = moe.MoEConfig.of(workloads.layer_config("olmoe"))
    c = cfg.to_c()
    w = moe._CWeights()
    w.w1 = w.w2 = fake
    T = 128
    need = moe.experts_backward_workspace_size(cfg, T)
    assert need > T * cfg.top_k * (2 * cfg.expert_dim + 2 * cfg.hidden_size) * 2
    args = [fake] * 9  # z, offsets, perm, h, act, dy, dz, dw1, dw2
    for i, name in enumerate(("z", "expert_offsets", "permutation", "h_saved", "act_saved", "dy_assign",
                              "dz", "dw1", "dw2")):
        bad = list(args)
        bad[i] = None
        assert moe._experts_backward(ctypes.byref(c), ctypes.byref(w), T, *bad, fake, need, None) == 1, name
        assert name in moe._last_error().decode()
    # short workspace
    assert moe._experts_backward(ctypes.byref(c), ctypes.byref(w), T, *args, fake, need - 1, None) == 3
    # missing expert weights
    assert moe._experts_backward(ctypes.byref(c), ctypes.byref(moe._CWeights()), T, *args, fake, need, None) == 1
    # MXFP8 training is not built
    mx = moe.MoEConfig.of(dict(workloads.layer_config("olmoe"), expert_precision="mxfp8"))
    with pytest.raises(moe.MoEError) as e:
        moe.experts_backward_workspace_size(mx, T)
    assert e.value.status == 2
    cm = mx.to_c()
    assert moe._experts_forward_train(ctypes.byref(cm), ctypes.byref(w), T, *([fake] * 6), fake, 1 << 40, None) == 2
    # fp32 layers beyond the fp32 kernels' grid
    big = dict(workloads.layer_config("tiny_f32"))
    with pytest.raises(moe.MoEError):
        moe.experts_backward_workspace_size(big, 70000)
    # bf16 operands above 4 GiB
    with pytest.raises(moe.MoEError):
        moe.experts_backward_workspace_size(workloads.layer_config("skewed"), 65536)
    # training forward needs both saved buffers
    assert moe._experts_forward_train(ctypes.byref(c), ctypes.byref(w), T, fake, fake, fake, fake, None, fake,
                                      fake, 1 << 40, None) == 1
    assert "h_saved" in moe._last_error().decode()
    # combine backward: pointers, and no backward through the latent norm
    assert moe._combine_backward(ctypes.byref(c), T, fake, fake, None, fake, None, None) == 1
    lat = moe.MoEConfig.of(workloads.layer_config("latent896")).to_c()
    assert moe._combine_backward(ctypes.byref(lat), T, fake, fake, fake, fake, None, None) == 2
    # T = 0: only the weight gradients, which must be given
    assert moe._combine_backward(ctypes.byref(c), 0, None, None, None, None, None, None) == 0
    assert moe._experts_backward(ctypes.byref(c), ctypes.byref(w), 0, *([None] * 7), None, None, None, 0,
                                 None) == 1


def test_calibration_entry_points_validate_before_any_gpu_call():
    fake = ctypes.c_void_p(0x10000)  # never dereferenced: every call below fails validation
    waves, flops = ctypes.c_int64(0), ctypes.c_double(0.0)
    assert moe._calibrate_mfma(0, fake, ctypes.byref(waves), ctypes.byref(flops), None) == 1
    assert "iters" in moe._last_error().decode()
    assert moe._calibrate_mfma(10, fake, None, ctypes.byref(flops), None) == 1
    assert moe._calibrate_mfma(10, fake, ctypes.byref(waves), None, None) == 1
    assert moe._calibrate_mfma_mx(0, fake, ctypes.byref(waves), ctypes.byref(flops), None) == 1
    assert moe._calibrate_mfma_mx(10, fake, None, ctypes.byref(flops), None) == 1
    for nbytes in (0, -16, 24):
        assert moe._calibrate_copy(fake, fake, nbytes, None) == 1
    assert moe._calibrate_copy(None, fake, 64, None) == 1
    assert moe._calibrate_copy(fake, None, 64, None) == 1


def test_router_weight_planes_beyond_4gib_are_refused():
    # The large-layer router splits the fp32 router weights into three bf16 planes addressed
    # with 32-bit byte offsets: 3 * E * d_model elements of 2 bytes must stay below 4 GiB.
    ok = dict(workloads.layer_config("latent896"), num_experts=1024, d_model=698048, latent_dim=64)
    assert 3 * 1024 * 698048 < (1 << 31)
    assert moe.workspace_size(ok, 1) > 0
    big = dict(ok, d_model=699072)
    assert 3 * 1024 * 699072 >= (1 << 31)
    with pytest.raises(moe.MoEError) as e:
        moe.workspace_size(big, 1)
    assert e.value.status == 2 and "4 GiB" in str(e.value)
