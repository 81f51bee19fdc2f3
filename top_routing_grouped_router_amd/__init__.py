"""Python binding of the MoE layer's C ABI (include/moe_mi355x.h, lib/libmoe_mi355x.so).

Argument marshalling only: tensors become device pointers, the current torch stream becomes
the hipStream_t, and every step of the layer runs in the library's HIP kernels. PyTorch is
used for device memory and streams. Importing this module loads the library and raises
ImportError if it has not been built (see build.py); there is no fallback path.

Names follow the page "Как устроен Olmo-core 3: обучение больших MoE-моделей" (sections
"Как задаётся конфигурация MoE", "Маршрутизация: как роутер выбирает экспертов", "Латентная
проекция экспертов").
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass, fields
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "lib", "libmoe_mi355x.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is missing: build it with "
                      "`python top_routing_grouped_router_amd/build.py` (gfx950)")
_lib = ctypes.CDLL(LIB_PATH)

c_i32, c_i64, c_f32, c_vp = ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_void_p

STATUS = {0: "MOE_OK", 1: "MOE_ERR_INVALID_ARG", 2: "MOE_ERR_UNSUPPORTED",
          3: "MOE_ERR_WORKSPACE_TOO_SMALL", 4: "MOE_ERR_HIP"}
GATING = {"softmax": 0, "topk_softmax": 1, "sigmoid": 2}
DTYPE = {"f32": 0, "bf16": 1}
PRECISION = {"bf16": 0, "mxfp8": 1}
TORCH_DTYPE = {"f32": torch.float32, "bf16": torch.bfloat16}


class _CConfig(ctypes.Structure):
    _fields_ = [
        ("struct_size", c_i32), ("num_experts", c_i32), ("d_model", c_i64), ("top_k", c_i32),
        ("gating_function", c_i32), ("sigmoid_stability_epsilon", c_f32),
        ("normalize_expert_weights", c_f32), ("restore_weight_scale", c_i32),
        ("expert_weight_scale", c_f32), ("original_top_k", c_i32), ("router_bias", c_i32),
        ("hidden_size", c_i64), ("activation", c_i32), ("dtype", c_i32), ("latent_dim", c_i64),
        ("up_proj_input_norm", c_i32), ("up_proj_input_norm_eps", c_f32), ("capacity_factor", c_f32),
        ("expert_precision", c_i32),
    ]


class _CWeights(ctypes.Structure):
    _fields_ = [(n, c_vp) for n in ("router_weight", "router_bias", "score_bias", "down_proj",
                                    "up_proj_input_norm_weight", "up_proj", "w1", "w2",
                                    "w1_mx", "w1_mx_scale", "w2_mx", "w2_mx_scale")]


ROUTING_FIELDS = ("expert_weights", "expert_indices", "batch_size_per_expert", "expert_offsets",
                  "permutation", "inverse_permutation", "router_logits", "router_scores")


class _CRouting(ctypes.Structure):
    _fields_ = [(n, c_vp) for n in ROUTING_FIELDS]


def _sig(name, res, *args):
    f = getattr(_lib, name)
    f.restype = res
    f.argtypes = list(args)
    return f


_P = ctypes.POINTER
_abi_version = _sig("moe_abi_version", c_i32)
_status_string = _sig("moe_status_string", ctypes.c_char_p, c_i32)
_last_error = _sig("moe_last_error_message", ctypes.c_char_p)
_config_default = _sig("moe_config_default", c_i32, _P(_CConfig))
_config_validate = _sig("moe_config_validate", c_i32, _P(_CConfig))
_num_params = _sig("moe_num_params", c_i32, _P(_CConfig), _P(c_i64), _P(c_i64))
_workspace_size = _sig("moe_workspace_size", c_i32, _P(_CConfig), c_i64, _P(ctypes.c_size_t))
_expert_capacity = _sig("moe_expert_capacity", c_i32, _P(_CConfig), c_i64, _P(c_i64))
_forward = _sig("moe_forward", c_i32, _P(_CConfig), _P(_CWeights), c_i64, c_vp, c_vp,
                _P(_CRouting), c_vp, ctypes.c_size_t, c_vp)
_forward_noalloc = _sig("moe_forward_noalloc", c_i32, _P(_CConfig), _P(_CWeights), c_i64, c_vp, c_vp,
                        _P(_CRouting), c_vp)
NOALLOC_SCRATCH_BYTES = 64 << 20  # MOE_NOALLOC_SCRATCH_BYTES
_router_forward = _sig("moe_router_forward", c_i32, _P(_CConfig), _P(_CWeights), c_i64, c_vp,
                       _P(_CRouting), c_vp, ctypes.c_size_t, c_vp)
_route_from_scores = _sig("moe_route_from_scores", c_i32, _P(_CConfig), c_i64, c_vp, c_vp, c_vp,
                          c_vp, c_vp)
_permute = _sig("moe_permute", c_i32, _P(_CConfig), c_i64, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp,
                ctypes.c_size_t, c_vp)
_latent_down = _sig("moe_latent_down", c_i32, _P(_CConfig), _P(_CWeights), c_i64, c_vp, c_vp, c_vp,
                    ctypes.c_size_t, c_vp)
_experts_forward = _sig("moe_experts_forward", c_i32, _P(_CConfig), _P(_CWeights), c_i64, c_vp,
                        c_vp, c_vp, c_vp, c_vp, ctypes.c_size_t, c_vp)
_combine = _sig("moe_combine", c_i32, _P(_CConfig), _P(_CWeights), c_i64, c_vp, c_vp, c_vp, c_vp)
_latent_up = _sig("moe_latent_up", c_i32, _P(_CConfig), _P(_CWeights), c_i64, c_vp, c_vp, c_vp,
                  ctypes.c_size_t, c_vp)
_experts_forward_train = _sig("moe_experts_forward_train", c_i32, _P(_CConfig), _P(_CWeights), c_i64, c_vp,
                              c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, ctypes.c_size_t, c_vp)
_experts_backward_ws = _sig("moe_experts_backward_workspace_size", c_i32, _P(_CConfig), c_i64,
                            _P(ctypes.c_size_t))
_experts_backward = _sig("moe_experts_backward", c_i32, _P(_CConfig), _P(_CWeights), c_i64, c_vp, c_vp, c_vp,
                         c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, ctypes.c_size_t, c_vp)
_combine_backward = _sig("moe_combine_backward", c_i32, _P(_CConfig), c_i64, c_vp, c_vp, c_vp, c_vp, c_vp,
                         c_vp)
_mx_quantize = _sig("moe_mx_quantize", c_i32, c_i64, c_i64, c_vp, c_vp, c_vp, c_vp)
_accumulate_counts = _sig("moe_accumulate_expert_counts", c_i32, c_i32, c_vp, c_vp, c_vp)
_load_imbalance = _sig("moe_load_imbalance", c_i32, c_i32, c_vp, c_vp, c_vp)
_score_bias_update = _sig("moe_score_bias_update", c_i32, c_i32, c_f32, c_vp, c_vp, c_vp, c_vp)
_calibrate_mfma = _sig("moe_calibrate_mfma_bf16", c_i32, c_i64, c_vp, c_vp, c_vp, c_vp)
_calibrate_mfma_mx = _sig("moe_calibrate_mfma_mxfp8", c_i32, c_i64, c_vp, c_vp, c_vp, c_vp)
_calibrate_copy = _sig("moe_calibrate_copy", c_i32, c_vp, c_vp, c_i64, c_vp)


class MoEError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS.get(status, status)}: {message}")
        self.status = status


def _check(status: int) -> None:
    if status != 0:
        raise MoEError(status, _last_error().decode(errors="replace"))


def abi_version() -> int:
    return int(_abi_version())


@dataclass
class MoEConfig:
    """Layer fields (MoEConfig / MoERouterConfigV2 / LatentMoEConfig). None = unset."""
    d_model: int
    num_experts: int = 1
    top_k: int = 1
    hidden_size: int = 256
    gating_function: str = "softmax"
    sigmoid_stability_epsilon: Optional[float] = None
    normalize_expert_weights: Optional[float] = None
    restore_weight_scale: bool = False
    expert_weight_scale: Optional[float] = None
    original_top_k: Optional[int] = None
    router_bias: bool = False
    latent_dim: Optional[int] = None
    up_proj_input_norm: bool = True
    up_proj_input_norm_eps: float = 1e-5
    dtype: str = "bf16"
    capacity_factor: Optional[float] = None
    expert_precision: str = "bf16"

    @classmethod
    def of(cls, cfg) -> "MoEConfig":
        if isinstance(cfg, MoEConfig):
            return cfg
        names = {f.name for f in fields(cls)}
        return cls(**{k: v for k, v in dict(cfg).items() if k in names})

    def to_c(self) -> _CConfig:
        c = _CConfig()
        _check(_config_default(ctypes.byref(c)))
        c.d_model = int(self.d_model)
        c.num_experts = int(self.num_experts)
        c.top_k = int(self.top_k)
        c.hidden_size = int(self.hidden_size)
        c.gating_function = GATING[self.gating_function]
        c.sigmoid_stability_epsilon = float(self.sigmoid_stability_epsilon or 0.0)
        c.normalize_expert_weights = float(self.normalize_expert_weights or 0.0)
        c.restore_weight_scale = int(bool(self.restore_weight_scale))
        c.expert_weight_scale = float(self.expert_weight_scale or 0.0)
        c.original_top_k = int(self.original_top_k or 0)
        c.router_bias = int(bool(self.router_bias))
        c.latent_dim = int(self.latent_dim or 0)
        c.up_proj_input_norm = int(bool(self.up_proj_input_norm))
        c.up_proj_input_norm_eps = float(self.up_proj_input_norm_eps)
        c.dtype = DTYPE[self.dtype]
        c.capacity_factor = float(self.capacity_factor or 0.0)
        c.expert_precision = PRECISION[self.expert_precision]
        return c

    @property
    def expert_dim(self) -> int:
        return int(self.latent_dim) if self.latent_dim else int(self.d_model)

    @property
    def torch_dtype(self) -> torch.dtype:
        return TORCH_DTYPE[self.dtype]


def validate(cfg) -> None:
    c = MoEConfig.of(cfg).to_c()
    _check(_config_validate(ctypes.byref(c)))


def num_params(cfg) -> tuple[int, int]:
    c = MoEConfig.of(cfg).to_c()
    total, active = c_i64(), c_i64()
    _check(_num_params(ctypes.byref(c), ctypes.byref(total), ctypes.byref(active)))
    return int(total.value), int(active.value)


def expert_capacity(cfg, num_tokens: int) -> int:
    """Expert capacity for num_tokens tokens (0 = dropless)."""
    c = MoEConfig.of(cfg).to_c()
    n = c_i64()
    _check(_expert_capacity(ctypes.byref(c), int(num_tokens), ctypes.byref(n)))
    return int(n.value)


def workspace_size(cfg, num_tokens: int) -> int:
    c = MoEConfig.of(cfg).to_c()
    n = ctypes.c_size_t()
    _check(_workspace_size(ctypes.byref(c), int(num_tokens), ctypes.byref(n)))
    return int(n.value)


# --------------------------------------------------------------------------- marshalling

def _ptr(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("tensors must live on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensors must be contiguous")
    return c_vp(t.data_ptr())


def _stream():
    return c_vp(torch.cuda.current_stream().cuda_stream)


def _expect(t, shape, dtype, name):
    if t is None:
        raise ValueError(f"{name} is required")
    if tuple(t.shape) != tuple(shape) or t.dtype != dtype:
        raise ValueError(f"{name}: expected {tuple(shape)} {dtype}, got {tuple(t.shape)} {t.dtype}")


def _c_weights(cfg: MoEConfig, w: dict) -> _CWeights:
    E, d, h, K = cfg.num_experts, cfg.d_model, cfg.hidden_size, cfg.expert_dim
    D = cfg.torch_dtype
    cw = _CWeights()
    checks = {
        "router_weight": ((E, d), torch.float32), "router_bias": ((E,), torch.float32),
        "score_bias": ((E,), torch.float32), "down_proj": ((cfg.latent_dim or 0, d), D),
        "norm_weight": ((cfg.latent_dim or 0,), torch.float32), "up_proj": ((d, cfg.latent_dim or 0), D),
        "w1": ((E, 2 * h, K), D), "w2": ((E, K, h), D),
        "w1_mx": ((E, 2 * h, K), torch.uint8), "w1_mx_scale": ((E, 2 * h, K // 32), torch.uint8),
        "w2_mx": ((E, K, h), torch.uint8), "w2_mx_scale": ((E, K, h // 32), torch.uint8),
    }
    for name, (shape, dt) in checks.items():
        t = w.get(name)
        if t is not None:
            _expect(t, shape, dt, name)
    cw.router_weight = _ptr(w.get("router_weight"))
    cw.router_bias = _ptr(w.get("router_bias"))
    cw.score_bias = _ptr(w.get("score_bias"))
    cw.down_proj = _ptr(w.get("down_proj"))
    cw.up_proj_input_norm_weight = _ptr(w.get("norm_weight"))
    cw.up_proj = _ptr(w.get("up_proj"))
    cw.w1 = _ptr(w.get("w1"))
    cw.w2 = _ptr(w.get("w2"))
    for name in ("w1_mx", "w1_mx_scale", "w2_mx", "w2_mx_scale"):
        setattr(cw, name, _ptr(w.get(name)))
    return cw


def quantize_expert_weights(weights: dict) -> dict:
    """The weights with MXFP8 copies of the expert matrices added (w1_mx / w1_mx_scale: W1 rows
    along K; w2_mx / w2_mx_scale: W2 rows along h), as the MXFP8 experts read them."""
    out = dict(weights)
    out["w1_mx"], out["w1_mx_scale"] = mx_quantize(weights["w1"])
    out["w2_mx"], out["w2_mx_scale"] = mx_quantize(weights["w2"])
    return out


def _routing_tensors(cfg: MoEConfig, T: int, device, want=ROUTING_FIELDS) -> dict:
    E, k = cfg.num_experts, cfg.top_k
    A = T * k
    shapes = {
        "expert_weights": ((T, k), torch.float32), "expert_indices": ((T, k), torch.int32),
        "batch_size_per_expert": ((E,), torch.int32), "expert_offsets": ((E + 1,), torch.int32),
        "permutation": ((A,), torch.int32), "inverse_permutation": ((A,), torch.int32),
        "router_logits": ((T, E), torch.float32), "router_scores": ((T, E), torch.float32),
    }
    return {n: torch.empty(shapes[n][0], dtype=shapes[n][1], device=device) for n in want}


def _c_routing(r: dict) -> _CRouting:
    cr = _CRouting()
    for n in ROUTING_FIELDS:
        setattr(cr, n, _ptr(r.get(n)))
    return cr


class MoELayer:
    """A routed MoE layer bound to device weights, with a cached workspace.

    weights: dict with router_weight (E,d) f32, router_bias (E) f32 | None, score_bias (E) f32 |
    None, down_proj (L,d) D | None, norm_weight (L) f32 | None, up_proj (d,L) D | None,
    w1 (E,2h,K) D, w2 (E,K,h) D.
    """

    def __init__(self, cfg, weights: dict):
        self.cfg = MoEConfig.of(cfg)
        self._c = self.cfg.to_c()
        _check(_config_validate(ctypes.byref(self._c)))
        if self.cfg.expert_precision == "mxfp8" and weights.get("w1_mx") is None:
            weights = quantize_expert_weights(weights)
        self.weights = weights
        self._cw = _c_weights(self.cfg, weights)
        self._ws = None

    def workspace(self, T: int, device) -> torch.Tensor:
        need = workspace_size(self.cfg, T)
        if self._ws is None or self._ws.numel() < need or self._ws.device != device:
            self._ws = torch.empty(max(need, 1), dtype=torch.uint8, device=device)
        return self._ws

    def forward(self, x: torch.Tensor, routing=None, out: Optional[torch.Tensor] = None):
        """y = layer(x). routing: None, True (all routing outputs) or an iterable of
        ROUTING_FIELDS names; returns y or (y, dict)."""
        T = x.shape[0]
        _expect(x, (T, self.cfg.d_model), self.cfg.torch_dtype, "x")
        y = out if out is not None else torch.empty_like(x)
        _expect(y, (T, self.cfg.d_model), self.cfg.torch_dtype, "out")
        want = () if not routing else (ROUTING_FIELDS if routing is True else tuple(routing))
        r = _routing_tensors(self.cfg, T, x.device, want)
        ws = self.workspace(T, x.device)
        cr = _c_routing(r) if want else None
        _check(_forward(ctypes.byref(self._c), ctypes.byref(self._cw), T, _ptr(x), _ptr(y),
                        ctypes.byref(cr) if cr is not None else None, _ptr(ws), ws.numel(), _stream()))
        return (y, r) if want else y

    __call__ = forward

    def forward_noalloc(self, x: torch.Tensor, out: torch.Tensor, routing: Optional[dict] = None) -> None:
        """y = layer(x) into `out` through moe_forward_noalloc: the library's per-GPU scratch
        array is the workspace, and nothing is allocated (routing: an optional dict of
        preallocated ROUTING_FIELDS tensors to fill)."""
        T = x.shape[0]
        _expect(x, (T, self.cfg.d_model), self.cfg.torch_dtype, "x")
        _expect(out, (T, self.cfg.d_model), self.cfg.torch_dtype, "out")
        cr = _c_routing(routing) if routing else None
        _check(_forward_noalloc(ctypes.byref(self._c), ctypes.byref(self._cw), T, _ptr(x), _ptr(out),
                                ctypes.byref(cr) if cr is not None else None, _stream()))


# --------------------------------------------------------------------------- stage calls

def router_forward(cfg, weights: dict, x: torch.Tensor, logits=True, scores=True) -> dict:
    cfg = MoEConfig.of(cfg)
    T = x.shape[0]
    _expect(x, (T, cfg.d_model), cfg.torch_dtype, "x")
    want = ["expert_weights", "expert_indices"] + (["router_logits"] if logits else []) + \
        (["router_scores"] if scores else [])
    r = _routing_tensors(cfg, T, x.device, want)
    c, cw = cfg.to_c(), _c_weights(cfg, weights)
    ws = torch.empty(max(workspace_size(cfg, T), 1), dtype=torch.uint8, device=x.device)
    cr = _c_routing(r)
    _check(_router_forward(ctypes.byref(c), ctypes.byref(cw), T, _ptr(x), ctypes.byref(cr), _ptr(ws),
                           ws.numel(), _stream()))
    return r


def route_from_scores(cfg, sel_input: torch.Tensor, score_bias: Optional[torch.Tensor] = None):
    """Selection + weights from the gating output (scores; logits for topk_softmax)."""
    cfg = MoEConfig.of(cfg)
    T = sel_input.shape[0]
    _expect(sel_input, (T, cfg.num_experts), torch.float32, "sel_input")
    if score_bias is not None:
        _expect(score_bias, (cfg.num_experts,), torch.float32, "score_bias")
    idx = torch.empty((T, cfg.top_k), dtype=torch.int32, device=sel_input.device)
    w = torch.empty((T, cfg.top_k), dtype=torch.float32, device=sel_input.device)
    c = cfg.to_c()
    _check(_route_from_scores(ctypes.byref(c), T, _ptr(sel_input), _ptr(score_bias), _ptr(idx), _ptr(w),
                              _stream()))
    return idx, w


def permute(cfg, expert_indices: torch.Tensor) -> dict:
    cfg = MoEConfig.of(cfg)
    T = expert_indices.shape[0]
    _expect(expert_indices, (T, cfg.top_k), torch.int32, "expert_indices")
    r = _routing_tensors(cfg, T, expert_indices.device,
                         ("batch_size_per_expert", "expert_offsets", "permutation", "inverse_permutation"))
    ws = torch.empty(max(workspace_size(cfg, T), 1), dtype=torch.uint8, device=expert_indices.device)
    c = cfg.to_c()
    _check(_permute(ctypes.byref(c), T, _ptr(expert_indices), _ptr(r["batch_size_per_expert"]),
                    _ptr(r["expert_offsets"]), _ptr(r["permutation"]), _ptr(r["inverse_permutation"]),
                    _ptr(ws), ws.numel(), _stream()))
    return r


def latent_down(cfg, weights: dict, x: torch.Tensor) -> torch.Tensor:
    cfg = MoEConfig.of(cfg)
    T = x.shape[0]
    _expect(x, (T, cfg.d_model), cfg.torch_dtype, "x")
    z = torch.empty((T, cfg.latent_dim or 0), dtype=cfg.torch_dtype, device=x.device)
    c, cw = cfg.to_c(), _c_weights(cfg, weights)
    ws = torch.empty(max(workspace_size(cfg, T), 1), dtype=torch.uint8, device=x.device)
    _check(_latent_down(ctypes.byref(c), ctypes.byref(cw), T, _ptr(x), _ptr(z), _ptr(ws), ws.numel(),
                        _stream()))
    return z


def experts_forward(cfg, weights: dict, z: torch.Tensor, expert_offsets: torch.Tensor,
                    permutation: torch.Tensor) -> torch.Tensor:
    cfg = MoEConfig.of(cfg)
    T, K = z.shape[0], cfg.expert_dim
    _expect(z, (T, K), cfg.torch_dtype, "z")
    _expect(expert_offsets, (cfg.num_experts + 1,), torch.int32, "expert_offsets")
    _expect(permutation, (T * cfg.top_k,), torch.int32, "permutation")
    y = torch.empty((T * cfg.top_k, K), dtype=cfg.torch_dtype, device=z.device)
    ws = torch.empty(max(workspace_size(cfg, T), 1), dtype=torch.uint8, device=z.device)
    c, cw = cfg.to_c(), _c_weights(cfg, weights)
    _check(_experts_forward(ctypes.byref(c), ctypes.byref(cw), T, _ptr(z), _ptr(expert_offsets),
                            _ptr(permutation), _ptr(y), _ptr(ws), ws.numel(), _stream()))
    return y


def combine(cfg, y_assign: torch.Tensor, expert_weights: torch.Tensor,
            norm_weight: Optional[torch.Tensor] = None) -> torch.Tensor:
    cfg = MoEConfig.of(cfg)
    T, K = expert_weights.shape[0], cfg.expert_dim
    _expect(y_assign, (T * cfg.top_k, K), cfg.torch_dtype, "y_assign")
    _expect(expert_weights, (T, cfg.top_k), torch.float32, "expert_weights")
    out = torch.empty((T, K), dtype=cfg.torch_dtype, device=y_assign.device)
    c = cfg.to_c()
    cw = _c_weights(cfg, {"norm_weight": norm_weight})
    _check(_combine(ctypes.byref(c), ctypes.byref(cw), T, _ptr(y_assign), _ptr(expert_weights), _ptr(out),
                    _stream()))
    return out


def latent_up(cfg, weights: dict, n: torch.Tensor) -> torch.Tensor:
    cfg = MoEConfig.of(cfg)
    T = n.shape[0]
    _expect(n, (T, cfg.latent_dim or 0), cfg.torch_dtype, "n")
    y = torch.empty((T, cfg.d_model), dtype=cfg.torch_dtype, device=n.device)
    c, cw = cfg.to_c(), _c_weights(cfg, weights)
    ws = torch.empty(max(workspace_size(cfg, T), 1), dtype=torch.uint8, device=n.device)
    _check(_latent_up(ctypes.byref(c), ctypes.byref(cw), T, _ptr(n), _ptr(y), _ptr(ws), ws.numel(),
                      _stream()))
    return y


# --------------------------------------------------------------------------- backward
# Page "Как устроен Olmo-core 3: обучение больших MoE-моделей", sections "SwiGLU с квантизацией"
# (the saved pre-activation and the SwiGLU backward), "Вычисления экспертов и точность" (per-
# expert gradients of the grouped products) and "Пересылка токенов между экспертами".

def experts_forward_train(cfg, weights: dict, z: torch.Tensor, expert_offsets: torch.Tensor,
                          permutation: torch.Tensor) -> dict:
    """experts_forward plus the saved pre-activation h (A, 2h) and activation act (A, h), sorted
    order, for experts_backward."""
    cfg = MoEConfig.of(cfg)
    T, K = z.shape[0], cfg.expert_dim
    A, h = T * cfg.top_k, cfg.hidden_size
    _expect(z, (T, K), cfg.torch_dtype, "z")
    _expect(expert_offsets, (cfg.num_experts + 1,), torch.int32, "expert_offsets")
    _expect(permutation, (A,), torch.int32, "permutation")
    y = torch.empty((A, K), dtype=cfg.torch_dtype, device=z.device)
    hs = torch.empty((A, 2 * h), dtype=cfg.torch_dtype, device=z.device)
    act = torch.empty((A, h), dtype=cfg.torch_dtype, device=z.device)
    ws = torch.empty(max(workspace_size(cfg, T), 1), dtype=torch.uint8, device=z.device)
    c, cw = cfg.to_c(), _c_weights(cfg, weights)
    _check(_experts_forward_train(ctypes.byref(c), ctypes.byref(cw), T, _ptr(z), _ptr(expert_offsets),
                                  _ptr(permutation), _ptr(y), _ptr(hs), _ptr(act), _ptr(ws), ws.numel(),
                                  _stream()))
    return {"y_assign": y, "h": hs, "act": act}


def experts_backward_workspace_size(cfg, num_tokens: int) -> int:
    c = MoEConfig.of(cfg).to_c()
    n = ctypes.c_size_t(0)
    _check(_experts_backward_ws(ctypes.byref(c), num_tokens, ctypes.byref(n)))
    return int(n.value)


def experts_backward(cfg, weights: dict, z: torch.Tensor, expert_offsets: torch.Tensor,
                     permutation: torch.Tensor, saved: dict, dy_assign: torch.Tensor,
                     workspace: Optional[torch.Tensor] = None, out: Optional[dict] = None) -> dict:
    """Gradients of the routed experts: dz (T, K), dw1 (E, 2h, K), dw2 (E, K, h), from the
    gradient dy_assign (A, K) of y_assign and the saved tensors of experts_forward_train."""
    cfg = MoEConfig.of(cfg)
    T, K = z.shape[0], cfg.expert_dim
    A, h, E = T * cfg.top_k, cfg.hidden_size, cfg.num_experts
    dt = cfg.torch_dtype
    _expect(z, (T, K), dt, "z")
    _expect(expert_offsets, (E + 1,), torch.int32, "expert_offsets")
    _expect(permutation, (A,), torch.int32, "permutation")
    _expect(saved["h"], (A, 2 * h), dt, "saved h")
    _expect(saved["act"], (A, h), dt, "saved act")
    _expect(dy_assign, (A, K), dt, "dy_assign")
    if out is None:
        out = {"dz": torch.empty((T, K), dtype=dt, device=z.device),
               "dw1": torch.empty((E, 2 * h, K), dtype=dt, device=z.device),
               "dw2": torch.empty((E, K, h), dtype=dt, device=z.device)}
    if workspace is None:
        workspace = torch.empty(max(experts_backward_workspace_size(cfg, T), 1), dtype=torch.uint8,
                                device=z.device)
    c, cw = cfg.to_c(), _c_weights(cfg, weights)
    _check(_experts_backward(ctypes.byref(c), ctypes.byref(cw), T, _ptr(z), _ptr(expert_offsets),
                             _ptr(permutation), _ptr(saved["h"]), _ptr(saved["act"]), _ptr(dy_assign),
                             _ptr(out["dz"]), _ptr(out["dw1"]), _ptr(out["dw2"]), _ptr(workspace),
                             workspace.numel(), _stream()))
    return out


def combine_backward(cfg, y_assign: torch.Tensor, expert_weights: torch.Tensor, d_out: torch.Tensor,
                     want_weight_grad: bool = True) -> dict:
    """dY (A, K) = w * d_out per assignment and d_expert_weights (T, k) = <d_out[t], Y[t*k+j]>."""
    cfg = MoEConfig.of(cfg)
    T, K = expert_weights.shape[0], cfg.expert_dim
    _expect(y_assign, (T * cfg.top_k, K), cfg.torch_dtype, "y_assign")
    _expect(expert_weights, (T, cfg.top_k), torch.float32, "expert_weights")
    _expect(d_out, (T, K), cfg.torch_dtype, "d_out")
    dy = torch.empty((T * cfg.top_k, K), dtype=cfg.torch_dtype, device=y_assign.device)
    dw = torch.empty((T, cfg.top_k), dtype=torch.float32, device=y_assign.device) if want_weight_grad else None
    c = cfg.to_c()
    _check(_combine_backward(ctypes.byref(c), T, _ptr(y_assign), _ptr(expert_weights), _ptr(d_out), _ptr(dy),
                             _ptr(dw), _stream()))
    return {"dy_assign": dy, "d_expert_weights": dw}


# --------------------------------------------------------------------------- balancing state
# Page "Как устроен Olmo-core 3: обучение больших MoE-моделей", section "Счётчики и
# bias-корректировка": the per-expert count accumulator, the load-imbalance metric and the
# aux-loss-free score_bias update.

def accumulate_expert_counts(batch_size_per_expert: torch.Tensor, accumulator: torch.Tensor) -> torch.Tensor:
    """accumulator (E) int64 += batch_size_per_expert (E) int32, in place."""
    E = accumulator.shape[0]
    _expect(accumulator, (E,), torch.int64, "accumulator")
    _expect(batch_size_per_expert, (E,), torch.int32, "batch_size_per_expert")
    _check(_accumulate_counts(E, _ptr(batch_size_per_expert), _ptr(accumulator), _stream()))
    return accumulator


def load_imbalance(counts: torch.Tensor) -> torch.Tensor:
    """max(counts) / mean(counts) of an (E) int64 counter, as a 0-dim float64 tensor on the
    counter's device (NaN with no tokens)."""
    E = counts.shape[0]
    _expect(counts, (E,), torch.int64, "counts")
    out = torch.empty((), dtype=torch.float64, device=counts.device)
    _check(_load_imbalance(E, _ptr(counts), _ptr(out), _stream()))
    return out


def score_bias_update(accumulator: torch.Tensor, score_bias: torch.Tensor, bias_gamma: float,
                      imbalance: bool = False) -> Optional[torch.Tensor]:
    """score_bias (E) fp32 += bias_gamma * sign(total / E - accumulator), in place; zeroes the
    accumulator. With imbalance=True returns the accumulator's load imbalance before the
    reset (0-dim float64 tensor)."""
    E = accumulator.shape[0]
    _expect(accumulator, (E,), torch.int64, "accumulator")
    _expect(score_bias, (E,), torch.float32, "score_bias")
    out = torch.empty((), dtype=torch.float64, device=accumulator.device) if imbalance else None
    _check(_score_bias_update(E, float(bias_gamma), _ptr(accumulator), _ptr(score_bias), _ptr(out), _stream()))
    return out


# --------------------------------------------------------------------------- MXFP8

def mx_quantize(x: torch.Tensor):
    """MXFP8 of bf16 rows (..., cols): (E4M3 codes (..., cols) uint8, E8M0 block scales
    (..., cols / 32) uint8); blocks of 32 along the last axis."""
    if x.dtype != torch.bfloat16:
        raise ValueError("mx_quantize takes bfloat16 rows")
    cols = x.shape[-1]
    rows = x.numel() // cols if cols else 0
    codes = torch.empty(x.shape, dtype=torch.uint8, device=x.device)
    scales = torch.empty((*x.shape[:-1], cols // 32), dtype=torch.uint8, device=x.device)
    _check(_mx_quantize(rows, cols, _ptr(x.contiguous()), _ptr(codes), _ptr(scales), _stream()))
    return codes, scales


# --------------------------------------------------------------------------- calibration

def _calibrate(fn, iters, out):
    waves, flops = ctypes.c_int64(0), ctypes.c_double(0.0)
    _check(fn(iters, None, ctypes.byref(waves), ctypes.byref(flops), _stream()))
    if out is None:
        out = torch.empty(waves.value, dtype=torch.float32, device="cuda")
    _expect(out, (waves.value,), torch.float32, "out")
    _check(fn(iters, _ptr(out), ctypes.byref(waves), ctypes.byref(flops), _stream()))
    return out, flops.value


def calibrate_mfma_bf16(iters: int, out: Optional[torch.Tensor] = None):
    """Enqueue the matrix-core loop (measurement support, not part of the layer): every
    wavefront runs `iters` rounds of 8 register-only 32x32x16 bf16 products. Returns (out, flops)
    with out the per-wavefront sums (float32 on the current device) and flops the launch's dense
    flop count; time the current stream around this call."""
    return _calibrate(_calibrate_mfma, iters, out)


def calibrate_mfma_mxfp8(iters: int, out: Optional[torch.Tensor] = None):
    """The same loop on 32x32x64 block-scaled E4M3 products (the MXFP8 expert matmuls')."""
    return _calibrate(_calibrate_mfma_mx, iters, out)


def calibrate_copy(src: torch.Tensor, dst: torch.Tensor) -> None:
    """Enqueue a 16-byte-vector device copy of src's bytes into dst (measurement support)."""
    nbytes = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() != nbytes:
        raise ValueError("src and dst must have the same size in bytes")
    _check(_calibrate_copy(_ptr(src), _ptr(dst), nbytes, _stream()))
