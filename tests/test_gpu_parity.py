"""GPU parity of every stage of the MoE layer forward against the CPU oracle, through the C ABI.

Stage checks drive each entry point with inputs drawn by the seeded generators (or produced by
the oracle from them) and compare element by element:
  * moe_route_from_scores: indices bit-exact, weights to fp32 rounding (the injection point:
    both sides select on the same fp32 scores);
  * moe_permute: counts, offsets, permutation and inverse bit-exact;
  * moe_router_forward: logits inside the fp32 dot-product error bound; selection bit-exact
    against the oracle run on the GPU's own scores, gating and weights within derived fp32
    ulps;
  * moe_experts_forward / moe_combine / moe_latent_down / moe_latent_up: values to the layer
    tolerance (see tests/parity.py);
  * moe_forward: whole-layer parity at reduced shapes that span several tiles with ragged
    tails: the routing bit-exact on the GPU's own scores, then every token's value against the
    oracle driven by the GPU's routing.
"""
import ctypes

import numpy as np
import pytest
import torch

import workloads
from oracle import moe_oracle as O
from parity import (assert_close, assert_within_ulps, bf16_spacing, check_forward_routing, check_routing_invariants,
                    flip_allowance, logit_bound, np32, oracle_from_gpu_routing, oracle_inputs, routing_agreement,
                    to_device_weights, weight_ulps)

pytestmark = pytest.mark.gpu

moe = pytest.importorskip("top_routing_grouped_router_amd")


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.set_device(0)


def banner(msg):
    print(f"[case] {msg}", flush=True)


# --------------------------------------------------------------------------- routing

ROUTE_CASES = [
    # (gating, T, E, k, kind, bias, extra cfg)
    ("softmax", 1000, 64, 8, "normal", None, dict(normalize_expert_weights=1.0)),
    ("softmax", 777, 8, 2, "ties", None, {}),
    ("softmax", 300, 896, 8, "nan", "normal", {}),
    ("sigmoid", 513, 896, 8, "normal", "normal", dict(sigmoid_stability_epsilon=1e-6)),
    ("sigmoid", 257, 256, 8, "ties", "zipf", {}),
    ("topk_softmax", 64, 896, 8, "normal", None, {}),
    ("topk_softmax", 200, 100, 1, "ties", None, {}),
    ("softmax", 129, 1024, 16, "nan", None, dict(normalize_expert_weights=2.0, restore_weight_scale=True,
                                                  expert_weight_scale=1.5, original_top_k=32)),
    ("sigmoid", 99, 5, 5, "ties", None, {}),
    ("softmax", 1, 1, 1, "normal", None, {}),
]


@pytest.mark.parametrize("case", ROUTE_CASES, ids=lambda c: f"{c[0]}-T{c[1]}-E{c[2]}-k{c[3]}-{c[4]}")
def test_route_from_scores_bitexact(case):
    gating, T, E, k, kind, bias, extra = case
    banner(f"route_from_scores {case}")
    cfg = dict(d_model=64, num_experts=E, top_k=k, hidden_size=64, gating_function=gating, dtype="f32",
               **extra)
    s = workloads.synthetic_scores(T, E, kind).numpy()
    cfgO = O.MoEConfig.from_dict(cfg)
    if gating != "topk_softmax" and kind == "normal":
        # realistic gating output, made by the oracle from synthetic logits
        s = O.gating_scores(cfgO, s).astype(np.float32)
    sb = None
    if bias == "normal":
        sb = (np.random.default_rng(E).standard_normal(E) * 0.1).astype(np.float32)
    elif bias == "zipf":
        sb = (2.0 * np.log(1.0 / (np.arange(E) + 1.0))).astype(np.float32)
    ref = O.route_from_scores(cfgO, s, sb)
    idx, w = moe.route_from_scores(cfg, torch.from_numpy(s).cuda(),
                                   None if sb is None else torch.from_numpy(sb).cuda())
    torch.cuda.synchronize()
    assert np.array_equal(idx.cpu().numpy(), ref["idx"]), "indices differ"
    # NaN scores give NaN weights on both sides; the finite rows are compared
    ref_w, got_w = ref["w"], w.cpu().numpy()
    fin = np.all(np.isfinite(ref_w), axis=1)
    assert np.array_equal(np.isfinite(got_w), np.isfinite(ref_w))
    allow = np.broadcast_to(weight_ulps(cfgO, s, ref["idx"]), ref_w.shape)
    assert_within_ulps(got_w[fin], ref_w[fin], allow[fin], "weights")


# --------------------------------------------------------------------------- dispatch

PERMUTE_CASES = [(1000, 64, 8, 0.0), (777, 896, 8, 1.0), (33, 5, 5, 0.0), (4097, 256, 8, 2.5),
                 (1, 16, 4, 0.0), (300, 1024, 16, 0.5), (256, 1, 1, 0.0)]


@pytest.mark.parametrize("case", PERMUTE_CASES, ids=lambda c: f"T{c[0]}-E{c[1]}-k{c[2]}-skew{c[3]}")
def test_permute_bitexact(case):
    T, E, k, skew = case
    banner(f"permute {case}")
    idx = workloads.random_distinct_indices(T, E, k, skew=skew)
    cfg = dict(d_model=64, num_experts=E, top_k=k, hidden_size=64, dtype="bf16")
    r = moe.permute(cfg, idx.cuda())
    torch.cuda.synchronize()
    counts = O.expert_counts(idx.numpy(), E)
    perm, inv = O.stable_permutation(idx.numpy())
    assert np.array_equal(r["batch_size_per_expert"].cpu().numpy(), counts)
    assert np.array_equal(r["expert_offsets"].cpu().numpy(), O.expert_offsets(counts))
    assert np.array_equal(r["permutation"].cpu().numpy(), perm)
    assert np.array_equal(r["inverse_permutation"].cpu().numpy(), inv)


def test_permute_zero_tokens():
    cfg = dict(d_model=64, num_experts=7, top_k=2, hidden_size=64)
    r = moe.permute(cfg, torch.zeros((0, 2), dtype=torch.int32, device="cuda"))
    torch.cuda.synchronize()
    assert int(r["batch_size_per_expert"].abs().sum()) == 0
    assert int(r["expert_offsets"].abs().sum()) == 0
    # the histogram of an empty batch is written, whatever the buffers held (E = 300: a grid of
    # two blocks for the 301 offsets)
    c = moe.MoEConfig.of(dict(cfg, num_experts=300)).to_c()
    counts = torch.full((300,), 77, dtype=torch.int32, device="cuda")
    offsets = torch.full((301,), -5, dtype=torch.int32, device="cuda")
    assert moe._permute(ctypes.byref(c), 0, None, moe._ptr(counts), moe._ptr(offsets), None, None, None, 0,
                        moe._stream()) == 0
    torch.cuda.synchronize()
    assert int(counts.abs().sum()) == 0 and int(offsets.abs().sum()) == 0


def _expected_dispatch(idx, E, capacity):
    """The stated rule for entries the routing never produces: an index out of [0, E), or one
    repeating an earlier index of its row, is not counted and gets no position (inverse -1);
    the rest are sorted stably by expert, each expert keeping its first `capacity` (kept rows,
    then dropped rows, each grouped by expert), and the positions after them hold -1."""
    T, k = idx.shape
    valid = (idx >= 0) & (idx < E)
    for j in range(1, k):
        valid[:, j] &= ~np.any(idx[:, :j] == idx[:, j:j + 1], axis=1)
    flat, vm = idx.ravel(), valid.ravel()
    counts = np.bincount(flat[vm], minlength=E)
    kept, dropped = [], []
    for e in range(E):
        a = np.nonzero(vm & (flat == e))[0]
        c = len(a) if capacity is None else min(len(a), capacity)
        kept.append(a[:c])
        dropped.append(a[c:])
    kc = np.array([len(x) for x in kept])
    perm = np.concatenate(kept + dropped + [np.full(T * k - vm.sum(), -1)]).astype(np.int64)
    inv = np.full(T * k, -1, dtype=np.int64)
    placed = perm >= 0
    inv[perm[placed]] = np.nonzero(placed)[0]
    return counts, np.concatenate([[0], np.cumsum(kc)]), perm, inv


@pytest.mark.parametrize("T,cf", [(500, None), (3000, None), (700, 0.75), (2600, 0.75)])
def test_permute_invalid_entries(T, cf):
    """Rows with repeated and out-of-range experts: both dispatch paths (one workgroup up to 1024
    tokens, four kernels above) count, place and mark them alike."""
    banner(f"permute invalid entries T={T} cf={cf}")
    E, k = 32, 4
    idx = workloads.random_distinct_indices(T, E, k, seed=3).numpy().copy()
    rng = np.random.default_rng(T)
    for t in rng.choice(T, size=T // 5, replace=False):
        j = int(rng.integers(1, k))
        idx[t, j] = idx[t, int(rng.integers(0, j))]
    for t in rng.choice(T, size=T // 10, replace=False):
        idx[t, int(rng.integers(0, k))] = (-1, E, E + 7)[int(rng.integers(0, 3))]
    cfg = dict(d_model=64, num_experts=E, top_k=k, hidden_size=64, dtype="bf16", capacity_factor=cf)
    r = moe.permute(cfg, torch.from_numpy(idx).cuda())
    torch.cuda.synchronize()
    C = None if cf is None else O.expert_capacity(O.MoEConfig.from_dict(cfg), T)
    counts, offsets, perm, inv = _expected_dispatch(idx, E, C)
    assert np.array_equal(r["batch_size_per_expert"].cpu().numpy(), counts)
    assert np.array_equal(r["expert_offsets"].cpu().numpy(), offsets)
    assert np.array_equal(r["permutation"].cpu().numpy(), perm)
    assert np.array_equal(r["inverse_permutation"].cpu().numpy(), inv)


# --------------------------------------------------------------------------- router

ROUTER_CASES = [
    ("tiny_f32", None, {}),
    ("olmoe", 513, dict(d_model=1024, num_experts=64)),
    ("latent896", 300, dict(d_model=512, latent_dim=256)),
    ("decode", None, dict(d_model=1024)),
    ("skewed", 257, dict(d_model=512, num_experts=256)),
    # large enough for the weight-planes MFMA GEMM (>= 256 tiles of 256 tokens x 128 experts):
    # ragged token tail and a ragged last expert tile (1020 = 7 * 128 + 124)
    ("latent896", 8300, dict(d_model=256, num_experts=1020, latent_dim=64, hidden_size=64)),
    ("skewed", 32768, dict(d_model=512, num_experts=256, hidden_size=64)),
]


@pytest.mark.parametrize("case", ROUTER_CASES, ids=lambda c: c[0])
def test_router_forward(case):
    name, T, over = case
    banner(f"router {case}")
    cfg, w, x = workloads.make_workload(name, tokens=T, **over)
    cfgO = O.MoEConfig.from_dict(cfg)
    wg = to_device_weights(w)
    r = moe.router_forward(cfg, wg, x.cuda())
    torch.cuda.synchronize()
    xr, W = np32(x), np32(w["router_weight"])
    ref_l = O.router_logits(xr, W, np32(w["router_bias"]))
    got_l = r["router_logits"].cpu().numpy().astype(np.float64)
    bound = logit_bound(xr, W, cfg["dtype"] == "bf16") + np.abs(ref_l) * 2.0 ** -23
    assert np.all(np.abs(got_l - ref_l) <= bound), np.max(np.abs(got_l - ref_l) / bound)
    # selection bit-exact on the GPU's own scores, gating and weights within derived ulps
    check_forward_routing(cfgO, r, w["score_bias"])
    # and against the pure oracle (selection on its own float64-summed logits): differences only
    # on near-ties within the realised score differences
    ref = O.route(cfgO, ref_l, np32(w["score_bias"]))
    gpu_keys = O.selection_keys(cfgO, got_l, r["router_scores"].cpu().numpy(), np32(w["score_bias"]))
    same = routing_agreement(r["expert_indices"].cpu().numpy(), ref, gpu_keys)
    print(f"  selection equal to the pure oracle's on {same.mean():.5f} of the tokens", flush=True)
    assert same.mean() > 0.99


# --------------------------------------------------------------------------- experts / combine

EXPERT_CASES = [
    ("tiny_f32", None, {}),
    ("olmoe", 777, dict(d_model=512, num_experts=16, top_k=4, hidden_size=256)),  # large tiles
    ("olmoe", 130, dict(d_model=512, num_experts=64, top_k=8, hidden_size=192)),  # small tiles
    ("skewed", 600, dict(d_model=256, num_experts=32, top_k=4, hidden_size=320)),  # hot experts
    ("latent896", 200, dict(d_model=512, latent_dim=128, num_experts=96, top_k=8, hidden_size=128)),
]


def _oracle_routing(cfg, w, x):
    cfgO = O.MoEConfig.from_dict(cfg)
    wo = oracle_inputs(w)
    l = O.router_logits(np32(x), wo["router_weight"], wo["router_bias"])
    r = O.route(cfgO, l, wo["score_bias"])
    return cfgO, wo, r


@pytest.mark.parametrize("case", EXPERT_CASES, ids=lambda c: f"{c[0]}-{c[1]}")
def test_experts_forward(case):
    name, T, over = case
    banner(f"experts {case}")
    cfg, w, x = workloads.make_workload(name, tokens=T, **over)
    cfgO, wo, r = _oracle_routing(cfg, w, x)
    z = O.prepare_routed_input(cfgO, np32(x), wo["down_proj"])
    ex = O.run_experts(cfgO, z, r["idx"], wo["w1"], wo["w2"])
    D = workloads.storage_dtype(cfg)
    zt = torch.from_numpy(z.astype(np.float32)).to(D).cuda()  # z holds D-representable values
    y = moe.experts_forward(cfg, to_device_weights(w), zt,
                            torch.from_numpy(ex["offsets"].astype(np.int32)).cuda(),
                            torch.from_numpy(ex["perm"].astype(np.int32)).cuda())
    torch.cuda.synchronize()
    ref_assign = ex["Y"][ex["inv"]]  # assignment order t*k+j
    # each expert output is itself a bf16 rounding of an fp32 / float64 accumulation: a flip
    # is one bf16 spacing
    flips = None if cfg["dtype"] != "bf16" else 2.0 * bf16_spacing(ref_assign)
    assert_close(np32(y), ref_assign, cfg["dtype"], "expert outputs", flips)


# Expert row counts whose main tile list (256-row M-tiles, hidden 128: one up/gate tile per
# M-tile) is 260 M-tiles: one whole round of a 256-workgroup grid and a last round of 4 tiles,
# which the dispatch moves to the remainder list (64-row tiles) from one expert -- the one with
# a remainder already; none has one; none has one and the chosen expert's last M-tile is partial;
# no expert has 4 M-tiles to give, so nothing moves.
TAIL_COUNTS = [
    [70 * 256, 70 * 256, 70 * 256, 50 * 256 + 40],
    [130 * 256, 130 * 256],
    [70 * 256 + 200, 70 * 256, 70 * 256, 49 * 256],
    [3 * 256] * 86 + [2 * 256],
]


def _tail_move(counts, round_tiles, ntn=1, bm=256, small_max=128):
    """M-tiles the dispatch's thin-last-round rule moves for these counts (0: none, also when no
    expert has that many)."""
    nb = [c // bm + (1 if c % bm > small_max else 0) for c in counts]
    work = sum(nb) * ntn
    tail = work % round_tiles
    m = -(-tail // ntn) if work > round_tiles and 0 < tail and 8 * tail <= round_tiles else 0
    return m if max(nb) >= m else 0


@pytest.mark.parametrize("counts", TAIL_COUNTS, ids=lambda c: f"E{len(c)}-{sum(c)}")
def test_experts_forward_thin_last_round(counts):
    """Expert outputs when whole M-tiles of the main list run as remainder tiles instead."""
    E, T = len(counts), sum(counts)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    m = _tail_move(counts, (cus + 7) // 8 * 8)
    banner(f"experts thin last round {counts}: {m} M-tiles moved on {cus} CUs")
    cfg, w, x = workloads.make_workload("olmoe", tokens=T, d_model=256, num_experts=E, top_k=1, hidden_size=128)
    cfgO = O.MoEConfig.from_dict(cfg)
    wo = oracle_inputs(w)
    idx = np.repeat(np.arange(E, dtype=np.int64), counts)[np.random.default_rng(11).permutation(T)].reshape(T, 1)
    z = np32(x)
    ex = O.run_experts(cfgO, z, idx, wo["w1"], wo["w2"])
    assert list(ex["counts"]) == counts
    y = moe.experts_forward(cfg, to_device_weights(w), x.cuda(),
                            torch.from_numpy(ex["offsets"].astype(np.int32)).cuda(),
                            torch.from_numpy(ex["perm"].astype(np.int32)).cuda())
    torch.cuda.synchronize()
    ref_assign = ex["Y"][ex["inv"]]
    assert_close(np32(y), ref_assign, cfg["dtype"], "expert outputs", 2.0 * bf16_spacing(ref_assign))


@pytest.mark.parametrize("case", [("olmoe", 300, dict(d_model=512, num_experts=16, top_k=4, hidden_size=128)),
                                  ("latent896", 300, dict(d_model=512, latent_dim=256, num_experts=32)),
                                  ("tiny_f32", None, {}),
                                  ("latent896", 100, dict(d_model=512, latent_dim=256, num_experts=32,
                                                          dtype="f32")),
                                  # from 2048 tokens on: one wavefront per token over a strided grid,
                                  # rows of 1, 2 and 4 x 64 chunks, ragged token counts
                                  ("olmoe", 2501, dict(d_model=512, num_experts=16, top_k=4, hidden_size=128)),
                                  ("olmoe", 2049, dict(d_model=2048, num_experts=16, top_k=4, hidden_size=128)),
                                  ("latent896", 2050, dict(d_model=512, latent_dim=256, num_experts=32)),
                                  ("latent896", 2303, dict(d_model=1024, latent_dim=1024, num_experts=32)),
                                  ("latent896", 2100, dict(d_model=512, latent_dim=256, num_experts=32,
                                                           dtype="f32"))],
                         ids=lambda c: f"{c[0]}-{c[1]}-{c[2].get('dtype', '')}")
def test_combine(case):
    name, T, over = case
    banner(f"combine {case}")
    cfg, w, x = workloads.make_workload(name, tokens=T, **over)
    cfgO = O.MoEConfig.from_dict(cfg)
    T = x.shape[0]
    k, K = cfg["top_k"], (cfg["latent_dim"] or cfg["d_model"])
    D = workloads.storage_dtype(cfg)
    g = torch.Generator().manual_seed(7)
    Y = torch.randn((T * k, K), generator=g).mul_(0.3).to(D)
    wts = torch.rand((T, k), generator=g, dtype=torch.float32)
    nw = None
    if cfg["latent_dim"]:
        nw = (1.0 + 0.1 * torch.randn((K,), generator=g)).to(torch.float32)
    out = moe.combine(cfg, Y.cuda(), wts.cuda(), None if nw is None else nw.cuda())
    torch.cuda.synchronize()
    Yn = np32(Y)
    inv = np.arange(T * k)  # y_assign is already in assignment order
    o = O.combine(cfgO, Yn, inv, wts.numpy())
    if cfg["latent_dim"]:
        ref = O.restore_routed_output(cfgO, o, None if nw is None else nw.numpy(),
                                      np.eye(K, dtype=np.float32))["n"]
    else:
        ref = o
    assert_close(np32(out), ref, cfg["dtype"], "combine")


@pytest.mark.parametrize("T", [1, 64, 333])
def test_latent_projections(T):
    banner(f"latent projections T={T}")
    cfg, w, x = workloads.make_workload("latent896", tokens=T, d_model=1024, latent_dim=256,
                                        num_experts=8)
    cfgO = O.MoEConfig.from_dict(cfg)
    wg = to_device_weights(w)
    z = moe.latent_down(cfg, wg, x.cuda())
    n = torch.randn((T, 256), generator=torch.Generator().manual_seed(3)).to(torch.bfloat16)
    y = moe.latent_up(cfg, wg, n.cuda())
    torch.cuda.synchronize()
    assert_close(np32(z), O.prepare_routed_input(cfgO, np32(x), np32(w["down_proj"])), "bf16", "down")
    assert_close(np32(y), np32(n).astype(np.float64) @ np32(w["up_proj"]).astype(np.float64).T, "bf16", "up")


@pytest.mark.parametrize("T", [1, 17, 64])
def test_latent_projections_few_tokens(T):
    """Decode-shaped projections (d_model 4096, latent 1024): the skinny weight-streaming GEMM,
    split over the chip with a workspace and unsplit without one."""
    banner(f"skinny latent projections T={T}")
    cfg, w, x = workloads.make_workload("decode", tokens=T, num_experts=8)
    cfgO = O.MoEConfig.from_dict(cfg)
    wg = to_device_weights(w)
    L, d = cfg["latent_dim"], cfg["d_model"]
    n = torch.randn((T, L), generator=torch.Generator().manual_seed(5)).to(torch.bfloat16)
    ref_z = O.prepare_routed_input(cfgO, np32(x), np32(w["down_proj"]))
    ref_y = np32(n).astype(np.float64) @ np32(w["up_proj"]).astype(np.float64).T
    c, cw = moe.MoEConfig.of(cfg).to_c(), moe._c_weights(moe.MoEConfig.of(cfg), wg)
    xg, ng = x.cuda(), n.cuda()
    for with_ws in (True, False):
        z = torch.empty((T, L), dtype=torch.bfloat16, device="cuda")
        y = torch.empty((T, d), dtype=torch.bfloat16, device="cuda")
        ws = torch.empty(moe.workspace_size(cfg, T), dtype=torch.uint8, device="cuda") if with_ws else None
        args = (moe._ptr(ws), ws.numel()) if with_ws else (None, 0)
        moe._check(moe._latent_down(ctypes.byref(c), ctypes.byref(cw), T, moe._ptr(xg), moe._ptr(z), *args,
                                    moe._stream()))
        moe._check(moe._latent_up(ctypes.byref(c), ctypes.byref(cw), T, moe._ptr(ng), moe._ptr(y), *args,
                                  moe._stream()))
        torch.cuda.synchronize()
        assert_close(np32(z), ref_z, "bf16", f"down (workspace {with_ws})")
        assert_close(np32(y), ref_y, "bf16", f"up (workspace {with_ws})")


# --------------------------------------------------------------------------- whole layer

# A few experts take most of 24576 assignments (Zipf score bias): experts of 16 or more 256-row
# tiles hold most of the main tile list, so the GEMMs deal its tiles to the XCDs one by one
# (the spread order); test_spread_case_uses_spread_order checks that the case does.
SPREAD_CASE = ("skewed", 12288, dict(d_model=256, num_experts=16, top_k=2, hidden_size=128))

LAYER_CASES = [
    ("tiny_f32", None, {}),
    ("tiny_f32", 37, dict(num_experts=8, top_k=8)),                       # k = E
    ("tiny_f32", 50, dict(num_experts=1, top_k=1)),                       # one expert
    ("olmoe", 600, dict(d_model=512, num_experts=16, top_k=4, hidden_size=256)),
    ("olmoe", 96, dict(d_model=1024, hidden_size=512)),                   # 64 experts, few rows each
    ("latent896", 400, dict(d_model=1024, latent_dim=256, num_experts=128, hidden_size=128)),
    ("skewed", 700, dict(d_model=512, num_experts=64, top_k=8, hidden_size=256)),
    ("decode", 3, dict(d_model=512, latent_dim=128, num_experts=64, hidden_size=64)),
    ("decode", None, dict(d_model=1024, latent_dim=256, num_experts=896, hidden_size=128)),
    ("latent896", 257, dict(d_model=512, latent_dim=128, num_experts=64, hidden_size=64,
                            up_proj_input_norm=False)),
    ("olmoe", 200, dict(d_model=256, num_experts=12, top_k=3, hidden_size=128, gating_function="topk_softmax",
                        restore_weight_scale=True, router_bias=True)),
    SPREAD_CASE,
]


def run_layer_case(name, T, over):
    cfg, w, x = workloads.make_workload(name, tokens=T, **over)
    cfgO = O.MoEConfig.from_dict(cfg)
    layer = moe.MoELayer(cfg, to_device_weights(w))
    y, r = layer(x.cuda(), routing=True)
    torch.cuda.synchronize()
    T = x.shape[0]
    check_routing_invariants(cfg, r, T)
    check_forward_routing(cfgO, r, w["score_bias"])
    wo = oracle_inputs(w)
    xs = np32(x)
    gi, gw = r["expert_indices"].cpu().numpy(), r["expert_weights"].cpu().numpy()
    ref = oracle_from_gpu_routing(cfgO, wo, xs, gi, gw)
    pure = O.route(cfgO, O.router_logits(xs, wo["router_weight"], wo["router_bias"]), wo["score_bias"])
    gpu_keys = O.selection_keys(cfgO, r["router_logits"].cpu().numpy(), r["router_scores"].cpu().numpy(),
                                wo["score_bias"])
    same = routing_agreement(gi, pure, gpu_keys)
    assert same.mean() >= 0.99
    fa = flip_allowance(cfgO, ref)
    assert_close(np32(y), ref["y"], cfg["dtype"], f"layer {name}", fa)
    return cfg, y


@pytest.mark.parametrize("case", LAYER_CASES, ids=lambda c: f"{c[0]}-{c[1]}-{'-'.join(f'{k}{v}' for k, v in c[2].items())}")
def test_layer_parity(case):
    banner(f"layer {case}")
    run_layer_case(*case)


def test_spread_case_uses_spread_order():
    """The rule the dispatch applies to a main tile list (most of its 256-row tiles in experts
    of at least 16 such tiles; a remainder above 128 rows takes one more tile), evaluated on
    the GPU's own expert counts for the spread case."""
    name, T, over = SPREAD_CASE
    cfg, w, x = workloads.make_workload(name, tokens=T, **over)
    layer = moe.MoELayer(cfg, to_device_weights(w))
    _, r = layer(x.cuda(), routing=True)
    counts = r["batch_size_per_expert"].cpu().numpy().astype(np.int64)
    tiles = counts // 256 + (counts % 256 > 128)
    large = tiles[tiles >= 16].sum()
    assert tiles.sum() > 0 and 2 * large >= tiles.sum(), (counts, tiles)


def test_layer_deterministic():
    banner("determinism")
    cfg, w, x = workloads.make_workload("olmoe", tokens=500, d_model=512, num_experts=16, top_k=4,
                                        hidden_size=256)
    layer = moe.MoELayer(cfg, to_device_weights(w))
    xc = x.cuda()
    y1, r1 = layer(xc, routing=True)
    y2, r2 = layer(xc, routing=True)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2)
    for k in r1:
        assert torch.equal(r1[k], r2[k]), k


def test_zero_tokens():
    cfg, w, x = workloads.make_workload("olmoe", tokens=0, d_model=256, num_experts=4, top_k=2,
                                        hidden_size=64)
    layer = moe.MoELayer(cfg, to_device_weights(w))
    y = layer(x.cuda())
    torch.cuda.synchronize()
    assert y.shape == (0, 256)
