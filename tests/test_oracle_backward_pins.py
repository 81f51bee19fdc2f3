"""Pins of the oracle's backward of the routed experts (SwiGLU backward, the grouped matmuls'
input and weight gradients, the sum over a token's copies, the combine backward) to facts
that do not come from the oracle: hand-worked cases (tests/golden/, each citing the page
section and the closed forms used), torch autograd on an independent float64 forward that
evaluates every assignment densely (no permutation, no grouping), central finite differences
of the oracle's own forward, and invariants of the rounding points. CPU only.
"""
import dataclasses
import json
import math
import os

import numpy as np
import pytest
import torch

import workloads
from oracle import moe_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _ev(v):
    if isinstance(v, list):
        return [_ev(u) for u in v]
    if isinstance(v, str):
        return float(eval(v, {"__builtins__": {}}, {"log": math.log}))
    return float(v)


def _hand_cases():
    with open(os.path.join(GOLDEN, "experts_backward_hand_worked.jsonl")) as f:
        return [json.loads(line) for line in f if line.strip()]


@pytest.mark.parametrize("case", _hand_cases(), ids=lambda c: c["name"])
def test_experts_backward_hand_worked(case):
    z = np.array(_ev(case["z"]))
    w1 = np.array(_ev(case["w1"]))
    w2 = np.array(_ev(case["w2"]))
    T, K = z.shape
    E, h = w1.shape[0], w2.shape[2]
    idx = np.array(case.get("idx", [[0]] * T), dtype=np.int64)
    cfg = O.MoEConfig(d_model=K, num_experts=E, top_k=idx.shape[1], hidden_size=h, dtype="f32")
    tr = O.run_experts_train(cfg, z, idx, w1, w2)
    inv = tr["inv"]
    # saved tensors and outputs in assignment order for the comparison
    np.testing.assert_allclose(tr["H"][inv], _ev(case["H"]), rtol=1e-7, atol=1e-7)
    np.testing.assert_allclose(tr["act"][inv], _ev(case["act"]), rtol=1e-7, atol=1e-7)
    np.testing.assert_allclose(tr["Y"][inv], _ev(case["y"]), rtol=1e-7, atol=1e-7)
    g = O.experts_backward(cfg, z, idx, w1, w2, tr, np.array(_ev(case["dy"])))
    np.testing.assert_allclose(g["dH"][inv], _ev(case["dH"]), rtol=1e-7, atol=1e-7)
    np.testing.assert_allclose(g["dz"], _ev(case["dz"]), rtol=1e-7, atol=1e-7)
    np.testing.assert_allclose(g["dw1"], _ev(case["dw1"]), rtol=1e-7, atol=1e-7)
    np.testing.assert_allclose(g["dw2"], _ev(case["dw2"]), rtol=1e-7, atol=1e-7)


def test_swiglu_backward_closed_forms_at_limits():
    """silu'(0) = 1/2; at gate = log 3, sigmoid = 3/4 and silu' = (3/4)(1 + (log 3)/4);
    silu' -> 1 and silu -> gate for large gates; both -> 0 for very negative gates; d_up never
    depends on up, d_gate is linear in up."""
    cfg = O.MoEConfig(d_model=8, hidden_size=5, dtype="f32")
    up = np.array([[1.0, -2.0, 3.0, 0.5, 1.0]])
    gate = np.array([[0.0, 40.0, -40.0, 0.0, math.log(3.0)]])
    d = np.array([[2.0, 1.0, 1.0, -4.0, 1.0]])
    g = O.swiglu_backward(cfg, np.concatenate([up, gate], 1), d)
    d_up, d_gate = g[0, :5], g[0, 5:]
    assert d_up[0] == 0.0 and d_gate[0] == 2.0 * 1.0 * 0.5
    assert d_up[1] == pytest.approx(40.0) and d_gate[1] == pytest.approx(-2.0)
    assert abs(d_up[2]) < 1e-15 and abs(d_gate[2]) < 1e-14
    assert d_up[3] == 0.0 and d_gate[3] == -4.0 * 0.5 * 0.5
    assert d_up[4] == pytest.approx(0.75 * math.log(3.0), rel=1e-7)
    assert d_gate[4] == pytest.approx(0.75 * (1.0 + math.log(3.0) / 4.0), rel=1e-7)


def test_swiglu_backward_matches_torch_autograd():
    rng = np.random.default_rng(3)
    h = 24
    H = rng.normal(0, 2.0, (37, 2 * h))
    d = rng.normal(0, 1.0, (37, h))
    cfg = O.MoEConfig(d_model=8, hidden_size=h, dtype="f32")
    Ht = torch.tensor(H, requires_grad=True)
    act = Ht[:, :h] * torch.nn.functional.silu(Ht[:, h:])
    act.backward(torch.tensor(d))
    np.testing.assert_allclose(O.swiglu_backward(cfg, H, d), Ht.grad.numpy(), rtol=2e-7, atol=1e-7)


def _first_come_kept(idx, E, C):
    held = [0] * E
    kept = []
    for e in np.asarray(idx).ravel():
        kept.append(C is None or held[e] < C)
        held[e] += 1
    return np.array(kept)


def _torch_dense_grads(z, idx, w1, w2, h, dY, kept):
    """Independent forward: every kept assignment (t, j) evaluates its expert's SwiGLU MLP on
    z[t] directly; loss = sum of dY[t*k+j] * y[t*k+j]; torch autograd gives the gradients."""
    T, k = idx.shape
    zt = torch.tensor(z, requires_grad=True)
    w1t = torch.tensor(np.asarray(w1, np.float64), requires_grad=True)
    w2t = torch.tensor(np.asarray(w2, np.float64), requires_grad=True)
    loss = torch.zeros((), dtype=torch.float64)
    for t in range(T):
        for j in range(k):
            a = t * k + j
            if not kept[a]:
                continue
            e = int(idx[t, j])
            H = w1t[e] @ zt[t]
            y = w2t[e] @ (H[:h] * torch.nn.functional.silu(H[h:]))
            loss = loss + (torch.tensor(dY[a]) * y).sum()
    loss.backward()
    return zt.grad.numpy(), w1t.grad.numpy(), w2t.grad.numpy()


def _small(name, T, **over):
    cfg, w, x = workloads.make_workload(name, tokens=T, device="cpu", **over)
    wn = {k: workloads.to_numpy_f32(v) for k, v in w.items()}
    return O.MoEConfig.from_dict(cfg), wn, workloads.to_numpy_f32(x)


@pytest.mark.parametrize("over", [
    dict(d_model=32, num_experts=5, top_k=2, hidden_size=16),
    dict(d_model=16, num_experts=7, top_k=3, hidden_size=8, capacity_factor=0.5),
    dict(d_model=16, num_experts=1, top_k=1, hidden_size=8),
])
def test_experts_backward_matches_autograd_of_dense_forward(over):
    """fp32 layer (roundings at fp32 only): the oracle's sorted/grouped backward equals the
    autograd gradients of the dense per-assignment forward to ~fp32 accuracy. Pins d_act =
    dY W2, the SwiGLU derivative, dz_perm = dH W1, both weight gradients (operand order and
    transposes), the grouping by expert, the sum over a token's copies and the dropped
    assignments."""
    T = 29
    cfg, w, x = _small("tiny_f32", T, **over)
    out = O.forward(cfg, w, x)
    z, idx = out["z"], out["idx"]
    C = out["capacity"]
    tr = O.run_experts_train(cfg, z, idx, w["w1"], w["w2"], C)
    rng = np.random.default_rng(7)
    dY = rng.normal(0, 1.0, (T * cfg.top_k, z.shape[1]))
    g = O.experts_backward(cfg, z, idx, w["w1"], w["w2"], tr, dY, C)
    kept = _first_come_kept(idx, cfg.num_experts, C)
    if C is not None:
        assert not kept.all(), "the case must drop something"
    dz, dw1, dw2 = _torch_dense_grads(z, idx, w["w1"], w["w2"], cfg.hidden_size, dY, kept)
    for got, want in ((g["dz"], dz), (g["dw1"], dw1), (g["dw2"], dw2)):
        scale = np.abs(want).max()
        assert scale > 0
        assert np.abs(got - want).max() <= 1e-5 * scale


def test_experts_backward_bf16_rounding_points():
    """bf16 layer: every returned gradient is bf16-representable, and each lies within a few
    bf16 roundings of the unrounded autograd gradient."""
    T = 23
    cfg, w, x = _small("olmoe", T, d_model=64, num_experts=5, top_k=2, hidden_size=64)
    out = O.forward(cfg, w, x)
    z, idx = out["z"], out["idx"]
    tr = O.run_experts_train(cfg, z, idx, w["w1"], w["w2"])
    dY = O.round_bf16(np.random.default_rng(1).normal(0, 1.0, (T * cfg.top_k, z.shape[1])))
    g = O.experts_backward(cfg, z, idx, w["w1"], w["w2"], tr, dY)
    for name in ("dz", "dw1", "dw2", "dH", "dz_perm"):
        assert np.array_equal(O.round_bf16(g[name]), g[name]), name
    kept = np.ones(T * cfg.top_k, bool)
    dz, dw1, dw2 = _torch_dense_grads(z, idx, w["w1"], w["w2"], cfg.hidden_size, dY, kept)
    for got, want in ((g["dz"], dz), (g["dw1"], dw1), (g["dw2"], dw2)):
        rel = np.linalg.norm(got - want) / np.linalg.norm(want)
        assert rel < 2e-2


def test_experts_backward_finite_differences():
    """Central differences of the oracle's own forward (fp32 layer) on a few coordinates of z
    and of both weights agree with the backward."""
    T = 6
    cfg, w, x = _small("tiny_f32", T, d_model=8, num_experts=3, top_k=2, hidden_size=4)
    out = O.forward(cfg, w, x)
    z, idx = out["z"], out["idx"]
    k = cfg.top_k
    rng = np.random.default_rng(11)
    dY = rng.normal(0, 1.0, (T * k, z.shape[1]))

    def loss(z_, w1_, w2_):
        r = O.run_experts(cfg, z_, idx, w1_, w2_)
        return float((dY * r["Y"][r["inv"]]).sum())

    tr = O.run_experts_train(cfg, z, idx, w["w1"], w["w2"])
    g = O.experts_backward(cfg, z, idx, w["w1"], w["w2"], tr, dY)
    eps = 1e-3
    checks = [("z", (2, 3)), ("z", (5, 0)), ("w1", (int(idx[0, 0]), 1, 2)),
              ("w1", (int(idx[1, 1]), 6, 7)), ("w2", (int(idx[2, 0]), 3, 1))]
    for which, at in checks:
        args = {"z": np.array(z, np.float64), "w1": np.array(w["w1"], np.float64),
                "w2": np.array(w["w2"], np.float64)}
        a = args[which]
        a[at] += eps
        lp = loss(args["z"], args["w1"], args["w2"])
        a[at] -= 2 * eps
        lm = loss(args["z"], args["w1"], args["w2"])
        fd = (lp - lm) / (2 * eps)
        got = {"z": g["dz"], "w1": g["dw1"], "w2": g["dw2"]}[which][at]
        assert got == pytest.approx(fd, rel=2e-3, abs=2e-4), (which, at)


def test_combine_backward_matches_autograd():
    T, k, K = 17, 3, 12
    rng = np.random.default_rng(5)
    Y = rng.normal(0, 1, (T * k, K))
    w = rng.uniform(0, 1, (T, k))
    d_o = rng.normal(0, 1, (T, K))
    cfg = O.MoEConfig(d_model=K, num_experts=4, top_k=k, dtype="f32")
    Yt = torch.tensor(Y, requires_grad=True)
    wt = torch.tensor(w, requires_grad=True)
    o = (wt[:, :, None] * Yt.view(T, k, K)).sum(1)
    o.backward(torch.tensor(d_o))
    g = O.combine_backward(cfg, Y, w, d_o)
    np.testing.assert_allclose(g["dY"], Yt.grad.numpy(), rtol=1e-7, atol=1e-7)
    np.testing.assert_allclose(g["dw"], wt.grad.numpy(), rtol=1e-6, atol=1e-6)


def test_combine_then_experts_backward_is_layer_gradient():
    """Chaining the combine backward into the experts backward gives the gradient of the
    oracle's own layer output o with respect to z (non-latent fp32 layer), by finite
    differences on two coordinates."""
    T = 5
    cfg, w, x = _small("tiny_f32", T, d_model=8, num_experts=3, top_k=2, hidden_size=4)
    out = O.forward(cfg, w, x)
    z, idx = out["z"], out["idx"]
    rng = np.random.default_rng(2)
    d_o = rng.normal(0, 1, (T, z.shape[1]))
    tr = O.run_experts_train(cfg, z, idx, w["w1"], w["w2"])
    cb = O.combine_backward(cfg, tr["Y"][tr["inv"]], out["w"], d_o)
    g = O.experts_backward(cfg, z, idx, w["w1"], w["w2"], tr, cb["dY"])

    def loss(z_):
        r = O.run_experts(cfg, z_, idx, w["w1"], w["w2"])
        return float((d_o * O.combine(cfg, r["Y"], r["inv"], out["w"])).sum())

    eps = 1e-3
    for at in ((0, 1), (4, 7)):
        zp, zm = np.array(z, np.float64), np.array(z, np.float64)
        zp[at] += eps
        zm[at] -= eps
        assert g["dz"][at] == pytest.approx((loss(zp) - loss(zm)) / (2 * eps), rel=2e-3, abs=2e-4)
