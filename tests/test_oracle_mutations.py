"""Planted mistakes in the CPU oracle must each fail at least one pin.

Each case patches one oracle function with a plausible bug (swapped operand, dropped term,
wrong index, wrong order of steps) and runs the pin that should catch it. CPU only; the
patch lives only inside the test.
"""
import numpy as np
import pytest

import test_oracle_pins as P
from oracle import moe_oracle as O


def _swapped_up_gate(cfg, z_rows, w1_e, w2_e, acc=np.float64):
    h = cfg.hidden_size
    H = np.asarray(z_rows, np.float64) @ np.asarray(w1_e, np.float64).T
    gate, up = H[:, :h], H[:, h:]  # halves swapped
    act = O.round_to(up * gate / (1.0 + np.exp(-gate)), cfg.dtype)
    return O.round_to(act @ np.asarray(w2_e, np.float64).T, cfg.dtype)


def _ties_to_higher_index(keys, k):
    keys = np.asarray(keys, np.float64)
    T, E = keys.shape
    nan = np.isnan(keys)
    neg = np.where(nan, 0.0, -keys)
    eidx = np.broadcast_to(-np.arange(E), (T, E))  # reversed tie rule
    return np.lexsort((eidx, neg, nan), axis=-1)[:, :k]


def _combine_with_perm(cfg, Y, inv, w):
    k = cfg.top_k
    w = np.asarray(w, np.float64)
    T = w.shape[0]
    perm = np.argsort(np.asarray(inv))  # uses perm where inv is needed
    perm = perm.reshape(T, k)
    o = np.zeros((T, Y.shape[1]))
    for j in range(k):
        o += w[:, j:j + 1] * Y[perm[:, j]]
    return o


_orig_weights = O.expert_weights


def _weights_from_keys(cfg, logits, scores, idx):
    # gathers the biased keys instead of the original scores
    return _orig_weights(cfg, logits, None if scores is None else scores + 0.5, idx)


def _scale_before_normalise(cfg, logits, scores, idx):
    import dataclasses
    c = dataclasses.replace(cfg, normalize_expert_weights=None)
    w = _orig_weights(c, logits, scores, idx)
    p = cfg.normalize_expert_weights
    if p:
        w = w / (np.abs(w) ** p).sum(-1, keepdims=True) ** (1.0 / p)
    return w


def _norm_without_mean(cfg, o, norm_weight=None, up_proj=None):
    o = np.asarray(o, np.float64)
    if not cfg.latent_dim:
        return dict(n=None, y=o)
    n = o / np.sqrt((o * o).sum(-1, keepdims=True) + cfg.up_proj_input_norm_eps)  # sum, not mean
    n = O.round_to(n, cfg.dtype)
    return dict(n=n, y=n @ np.asarray(up_proj, np.float64).T)


def _golden(name):
    return [c for c in P._golden_cases() if c["name"] == name][0]


MUTATIONS = [
    ("expert_mlp", _swapped_up_gate, lambda: P.test_single_expert_layer_is_plain_swiglu_mlp()),
    ("select_topk", _ties_to_higher_index,
     lambda: P.test_select_topk_brute_force_all_subsets(6)),
    ("combine", _combine_with_perm, lambda: P.test_dense_bruteforce_equals_permuted_path(
        "tiny_f32", dict(d_model=64, num_experts=6, top_k=3, hidden_size=32), 1e-6)),
    ("expert_weights", _weights_from_keys,
     lambda: P.test_routing_closed_forms(_golden("softmax_ln_ratios"))),
    ("expert_weights", _scale_before_normalise,
     lambda: P.test_routing_closed_forms(_golden("softmax_restore_scale"))),
    ("restore_routed_output", _norm_without_mean,
     lambda: P.test_identity_latent_reduces_to_rmsnorm_of_plain_layer()),
]


@pytest.mark.parametrize("target,bad,pin", MUTATIONS,
                         ids=[f"{m[0]}:{m[1].__name__}" for m in MUTATIONS])
def test_planted_mistake_is_caught(monkeypatch, target, bad, pin):
    monkeypatch.setattr(O, target, bad)
    with pytest.raises(AssertionError):
        pin()


def _bias_sign_reversed(score_bias, accumulator, bias_gamma):
    c = np.asarray(accumulator, dtype=np.int64)
    sgn = np.sign(c.size * c - int(c.sum())).astype(np.float32)  # actual - ideal
    return (np.asarray(score_bias, np.float32) + np.float32(bias_gamma) * sgn).astype(np.float32)


def _imbalance_mean_of_used_experts(counts):
    c = np.asarray(counts, dtype=np.int64)
    used = c[c > 0]
    if used.size == 0:
        return float("nan")
    return float(int(used.max()) * used.size) / float(int(used.sum()))  # mean over used experts only


BALANCE_MUTATIONS = [
    ("score_bias_update", _bias_sign_reversed, lambda: P.test_score_bias_update_closed_forms()),
    ("load_imbalance", _imbalance_mean_of_used_experts, lambda: P.test_load_imbalance_closed_forms()),
]


@pytest.mark.parametrize("target,bad,pin", BALANCE_MUTATIONS,
                         ids=[f"{m[0]}:{m[1].__name__}" for m in BALANCE_MUTATIONS])
def test_planted_balance_mistake_is_caught(monkeypatch, target, bad, pin):
    monkeypatch.setattr(O, target, bad)
    with pytest.raises(AssertionError):
        pin()


def _capacity_keeps_last(idx, num_experts, capacity):
    flat = np.asarray(idx).ravel()
    order = np.argsort(flat, kind="stable")
    if capacity is None:
        kept = np.ones(flat.size, dtype=bool)
    else:
        counts = np.bincount(flat, minlength=num_experts)
        last = np.cumsum(counts)
        rank_from_end = np.empty(flat.size, dtype=np.int64)
        rank_from_end[order] = last[flat[order]] - 1 - np.arange(flat.size)
        kept = rank_from_end < capacity  # keeps the last arrivals instead of the first
    perm = np.concatenate([order[kept[order]], order[~kept[order]]])
    inv = np.empty_like(perm)
    inv[perm] = np.arange(flat.size)
    return perm, inv, kept


def _capacity_rounded_down(cfg, num_tokens):
    if not cfg.capacity_factor:
        return None
    return 8 * int(cfg.capacity_factor * cfg.top_k * num_tokens / cfg.num_experts // 8)


CAPACITY_MUTATIONS = [
    ("capacity_permutation", _capacity_keeps_last,
     lambda: P.test_capacity_permutation_against_first_come_walk(16, 4, 100, 16)),
    ("expert_capacity", _capacity_rounded_down,
     lambda: P.test_expert_capacity_hand_worked(1.25, 2, 100, 8, 32)),
]


@pytest.mark.parametrize("target,bad,pin", CAPACITY_MUTATIONS,
                         ids=[f"{m[0]}:{m[1].__name__}" for m in CAPACITY_MUTATIONS])
def test_planted_capacity_mistake_is_caught(monkeypatch, target, bad, pin):
    monkeypatch.setattr(O, target, bad)
    with pytest.raises(AssertionError):
        pin()


_orig_encode = O.e4m3_encode


def _mx_scale_off_by_one(v, block=O.MX_BLOCK):
    v = np.asarray(v, np.float64)
    *lead, K = v.shape
    b = v.reshape(*lead, K // block, block)
    amax = np.abs(b).max(axis=-1)
    with np.errstate(divide="ignore"):
        ex = np.floor(np.log2(np.where(amax > 0, amax, 1.0))) - 7.0  # uses the mantissa-less max 2^7
    scode = np.where(amax > 0, np.clip(ex + 127.0, 0, 254), 0).astype(np.int64)
    codes = _orig_encode(b / (2.0 ** (scode - 127.0))[..., None])
    return codes.reshape(*lead, K), scode.astype(np.uint8)


def _e4m3_ties_away(a):
    a = np.asarray(a, np.float64)
    up = _orig_encode(np.nextafter(np.abs(a), np.inf)) & 0x7F  # nudging up turns ties into round-up
    return (up | np.where(np.signbit(a), 0x80, 0)).astype(np.uint8)


MX_MUTATIONS = [
    ("mx_quantize", _mx_scale_off_by_one, lambda: P.test_mx_quantize_block_scale_definition(0)),
    ("e4m3_encode", _e4m3_ties_away, lambda: P.test_e4m3_encode_matches_torch_float8()),
]


@pytest.mark.parametrize("target,bad,pin", MX_MUTATIONS, ids=[f"{m[0]}:{m[1].__name__}" for m in MX_MUTATIONS])
def test_planted_mx_mistake_is_caught(monkeypatch, target, bad, pin):
    monkeypatch.setattr(O, target, bad)
    with pytest.raises(AssertionError):
        pin()


# ------------------------------------------------------------------ backward of the experts
import test_oracle_backward_pins as B  # noqa: E402

_orig_experts_backward = O.experts_backward


def _swiglu_bwd_halves_swapped(cfg, H, d_act):
    h = cfg.hidden_size
    H = np.asarray(H, np.float64)
    up, gate = H[:, :h], H[:, h:]
    sig = 1.0 / (1.0 + np.exp(-gate))
    d_act = np.asarray(d_act, np.float64)
    # gate gradient first
    return O.round_to(np.concatenate([d_act * up * sig * (1 + gate * (1 - sig)), d_act * gate * sig], 1),
                      cfg.dtype)


def _swiglu_bwd_sigmoid_as_derivative(cfg, H, d_act):
    h = cfg.hidden_size
    H = np.asarray(H, np.float64)
    up, gate = H[:, :h], H[:, h:]
    sig = 1.0 / (1.0 + np.exp(-gate))
    d_act = np.asarray(d_act, np.float64)
    # silu' taken as sigmoid alone (the gate * sigmoid * (1 - sigmoid) term dropped)
    return O.round_to(np.concatenate([d_act * gate * sig, d_act * up * sig], 1), cfg.dtype)


def _dz_from_first_copy_only(cfg, z, idx, w1, w2, saved, dY_assign, capacity=None):
    g = _orig_experts_backward(cfg, z, idx, w1, w2, saved, dY_assign, capacity)
    T = np.asarray(z).shape[0]
    first = np.asarray(g["inv"]).reshape(T, cfg.top_k)[:, 0]
    g["dz"] = O.round_to(g["dz_perm"][first], cfg.dtype)  # copies not summed
    return g


def _dw2_with_act_in_assignment_order(cfg, z, idx, w1, w2, saved, dY_assign, capacity=None):
    g = _orig_experts_backward(cfg, z, idx, w1, w2, saved, dY_assign, capacity)
    perm, offsets = g["perm"], g["offsets"]
    act_assign = np.asarray(saved["act"])[np.asarray(g["inv"])]  # sorted rows read in assignment order
    dY = np.asarray(dY_assign, np.float64)[perm]
    for e in range(cfg.num_experts):
        R = slice(offsets[e], offsets[e + 1])
        if offsets[e + 1] > offsets[e]:
            g["dw2"][e] = O.round_to(dY[R].T @ act_assign[R], cfg.dtype)
    return g


def _combine_bwd_without_weight(cfg, Y_assign, w, d_o):
    k = cfg.top_k
    d_o = np.asarray(d_o, np.float64)
    T = d_o.shape[0]
    Y = np.asarray(Y_assign, np.float64).reshape(T, k, -1)
    dY = O.round_to(np.repeat(d_o[:, None, :], k, axis=1), cfg.dtype).reshape(T * k, -1)  # w dropped
    return dict(dY=dY, dw=O.round_f32(np.einsum("tc,tjc->tj", d_o, Y)))


_DENSE_K2 = dict(d_model=32, num_experts=5, top_k=2, hidden_size=16)

BACKWARD_MUTATIONS = [
    ("swiglu_backward", _swiglu_bwd_halves_swapped, lambda: B.test_swiglu_backward_matches_torch_autograd()),
    ("swiglu_backward", _swiglu_bwd_sigmoid_as_derivative, lambda: B.test_swiglu_backward_closed_forms_at_limits()),
    ("experts_backward", _dz_from_first_copy_only,
     lambda: B.test_experts_backward_matches_autograd_of_dense_forward(_DENSE_K2)),
    ("experts_backward", _dw2_with_act_in_assignment_order,
     lambda: B.test_experts_backward_matches_autograd_of_dense_forward(_DENSE_K2)),
    ("combine_backward", _combine_bwd_without_weight, lambda: B.test_combine_backward_matches_autograd()),
]


@pytest.mark.parametrize("target,bad,pin", BACKWARD_MUTATIONS,
                         ids=[f"{m[0]}:{m[1].__name__}" for m in BACKWARD_MUTATIONS])
def test_planted_backward_mistake_is_caught(monkeypatch, target, bad, pin):
    monkeypatch.setattr(O, target, bad)
    with pytest.raises(AssertionError):
        pin()
