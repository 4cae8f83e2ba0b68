"""Thin ctypes binding of libfwd.so (include/fwd.h). Argument marshalling only.

PyTorch supplies device memory (tensor.data_ptr()) and HIP streams
(torch.cuda.current_stream().cuda_stream); every step of the computation runs in
the library's HIP kernels. If libfwd.so is missing or no gfx950 device is present
the calls raise: there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os
from typing import Dict, Mapping, Optional

import numpy as np

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libfwd.so")

FWD_OK = 0
FWD_E_CONFIG = -1
FWD_E_WEIGHTS = -2
FWD_E_TOKEN_RANGE = -3
FWD_E_TOO_LARGE = -4
FWD_E_NONFINITE = -5
FWD_E_HIP = -6
FWD_E_UNAVAILABLE = -7
FWD_E_ARG = -8
DTYPE = {"f32": 0, "bf16": 1}
EMBED_SCALE = {"none": 0, "bf16_sqrt_hidden": 1}
NORM = {"pre": 0, "sandwich": 1}
LAYER = {"global": 0, "local": 1}
FFN_ACT = {"silu": 0, "gelu_tanh": 1}
ROPE_SCALING = {"none": 0, "llama3": 1, "longrope": 2}
FFN_KIND = {"dense": 0, "moe": 1}

EXPORTS = ("fwd_available", "fwd_create", "fwd_output_sizes", "fwd_prefill", "fwd_gemm", "fwd_gemm_noalloc",
           "fwd_attention",
           "fwd_rmsnorm", "fwd_set_timing", "fwd_get_timing", "fwd_destroy", "fwd_last_error",
           "fwd_session_create", "fwd_session_prefill", "fwd_session_decode", "fwd_session_length",
           "fwd_session_destroy", "fwd_moe_route")
KERNEL_CLASSES = ("embed", "norm", "qkv_rope", "attention", "o_proj", "gate_up", "down_proj", "lm_head", "argmax",
                  "v_transpose", "qk_norm", "moe_route", "moe_experts", "moe_combine")

c_i32, c_i64, c_f32, c_f64, c_vp = ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_double, ctypes.c_void_p


class FwdConfig(ctypes.Structure):
    _fields_ = [("n_layers", c_i32), ("hidden", c_i32), ("n_heads", c_i32), ("n_kv_heads", c_i32),
                ("head_dim", c_i32), ("ffn", c_i32), ("vocab", c_i32), ("rms_eps", c_f32),
                ("final_logit_softcap", c_f32), ("rope_theta", c_f64), ("embed_scale_mode", c_i32),
                ("sliding_window", c_i32), ("layer_kind", ctypes.POINTER(c_i32)), ("norm_placement", c_i32),
                ("dtype", c_i32), ("max_tokens", c_i32),
                ("qk_norm", c_i32), ("norm_gain_offset", c_i32), ("ffn_act", c_i32), ("rope_theta_local", c_f64),
                ("rope_scaling", c_i32), ("rope_factor", c_f32), ("rope_low_freq_factor", c_f32),
                ("rope_high_freq_factor", c_f32), ("rope_original_max_pos", c_i32),
                ("rope_short_factor", ctypes.POINTER(c_f32)), ("rope_long_factor", ctypes.POINTER(c_f32)),
                ("n_experts", c_i32), ("n_experts_per_tok", c_i32), ("moe_ffn", c_i32), ("moe_norm_topk", c_i32),
                ("ffn_kind", ctypes.POINTER(c_i32))]


class FwdLayerWeights(ctypes.Structure):
    _fields_ = [(n, c_vp) for n in ("attn_norm", "wq", "wk", "wv", "wo", "ffn_norm", "w_gate", "w_up", "w_down",
                                    "post_attn_norm", "post_ffn_norm", "q_norm", "k_norm", "router",
                                    "expert_gate", "expert_up", "expert_down")]


class FwdWeights(ctypes.Structure):
    _fields_ = [("embed", c_vp), ("final_norm", c_vp), ("layers", ctypes.POINTER(FwdLayerWeights))]


class FwdOutputs(ctypes.Structure):
    _fields_ = [("logits", c_vp), ("hidden", c_vp), ("argmax", c_vp)]


class FwdSizes(ctypes.Structure):
    _fields_ = [("logits_elems", c_i64), ("hidden_elems", c_i64), ("argmax_elems", c_i64),
                ("weight_bytes", c_i64), ("workspace_bytes", c_i64)]


class FwdError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"fwd error {code}: {msg}")
        self.code = code


_lib = None


def lib() -> ctypes.CDLL:
    """Load libfwd.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with python -m decoder_only_transformer_bf16_amd._build")
        L = ctypes.CDLL(LIB_PATH)
        L.fwd_available.restype = c_i32
        L.fwd_create.argtypes = [ctypes.POINTER(FwdConfig), ctypes.POINTER(FwdWeights), c_vp, ctypes.POINTER(c_vp)]
        L.fwd_create.restype = c_i32
        L.fwd_output_sizes.argtypes = [ctypes.POINTER(FwdConfig), c_i32, c_i32, ctypes.POINTER(FwdSizes)]
        L.fwd_output_sizes.restype = c_i32
        L.fwd_prefill.argtypes = [c_vp, c_vp, c_i32, c_i32, ctypes.POINTER(FwdOutputs)]
        L.fwd_prefill.restype = c_i32
        L.fwd_gemm.argtypes = [c_vp, c_vp, c_vp, c_i32, c_i32, c_i32, c_i32, c_vp]
        L.fwd_gemm.restype = c_i32
        L.fwd_gemm_noalloc.argtypes = [c_vp, c_vp, c_vp, c_i32, c_i32, c_i32, c_i32, c_vp]
        L.fwd_gemm_noalloc.restype = c_i32
        L.fwd_attention.argtypes = [c_vp, c_vp, c_vp, c_vp] + [c_i32] * 7 + [c_vp]
        L.fwd_attention.restype = c_i32
        L.fwd_rmsnorm.argtypes = [c_vp, c_vp, c_vp, c_i32, c_i32, c_f32, c_i32, c_vp]
        L.fwd_rmsnorm.restype = c_i32
        L.fwd_moe_route.argtypes = [c_vp, c_i32, c_i32, c_i32, c_i32, c_vp, c_vp, c_vp]
        L.fwd_moe_route.restype = c_i32
        L.fwd_set_timing.argtypes = [c_vp, c_i32]
        L.fwd_set_timing.restype = c_i32
        L.fwd_get_timing.argtypes = [c_vp, c_i32, ctypes.POINTER(c_f64), ctypes.POINTER(c_i64)]
        L.fwd_get_timing.restype = c_i32
        L.fwd_destroy.argtypes = [c_vp]
        L.fwd_destroy.restype = None
        L.fwd_last_error.restype = ctypes.c_char_p
        L.fwd_session_create.argtypes = [c_vp, c_i32, c_i32, ctypes.POINTER(c_vp)]
        L.fwd_session_create.restype = c_i32
        L.fwd_session_prefill.argtypes = [c_vp, c_vp, c_i32, c_i32, ctypes.POINTER(FwdOutputs)]
        L.fwd_session_prefill.restype = c_i32
        L.fwd_session_decode.argtypes = [c_vp, c_vp, ctypes.POINTER(FwdOutputs)]
        L.fwd_session_decode.restype = c_i32
        L.fwd_session_length.argtypes = [c_vp]
        L.fwd_session_length.restype = c_i32
        L.fwd_session_destroy.argtypes = [c_vp]
        L.fwd_session_destroy.restype = None
        _lib = L
    return _lib


def _check(rc: int) -> None:
    if rc != FWD_OK:
        raise FwdError(rc, lib().fwd_last_error().decode(errors="replace"))


def available() -> bool:
    return bool(lib().fwd_available())


def make_config(cfg, max_tokens: int):
    """FwdConfig from an object with the geometry attributes (see include/fwd.h).

    Returns (FwdConfig, keep-alive array of the layer map)."""
    kinds = cfg.kinds() if hasattr(cfg, "kinds") else tuple(cfg.layer_kind)
    kind_arr = (c_i32 * max(1, len(kinds)))(*[LAYER[k] for k in kinds])
    c = FwdConfig(n_layers=cfg.n_layers, hidden=cfg.hidden, n_heads=cfg.n_heads, n_kv_heads=cfg.n_kv_heads,
                  head_dim=cfg.head_dim, ffn=cfg.ffn, vocab=cfg.vocab, rms_eps=cfg.rms_eps,
                  final_logit_softcap=cfg.final_logit_softcap, rope_theta=cfg.rope_theta,
                  embed_scale_mode=EMBED_SCALE[cfg.embed_scale_mode], sliding_window=cfg.sliding_window,
                  layer_kind=ctypes.cast(kind_arr, ctypes.POINTER(c_i32)),
                  norm_placement=NORM[cfg.norm_placement], dtype=DTYPE[cfg.dtype], max_tokens=max_tokens)
    keep = [kind_arr]
    c.qk_norm = 1 if getattr(cfg, "qk_norm", False) else 0
    c.norm_gain_offset = int(getattr(cfg, "norm_gain_offset", 0))
    c.ffn_act = FFN_ACT[getattr(cfg, "ffn_act", "silu")]
    c.rope_theta_local = float(getattr(cfg, "rope_theta_local", 0.0))
    c.rope_scaling = ROPE_SCALING[getattr(cfg, "rope_scaling", "none")]
    c.rope_factor = float(getattr(cfg, "rope_factor", 1.0))
    c.rope_low_freq_factor = float(getattr(cfg, "rope_low_freq_factor", 1.0))
    c.rope_high_freq_factor = float(getattr(cfg, "rope_high_freq_factor", 4.0))
    c.rope_original_max_pos = int(getattr(cfg, "rope_original_max_pos", 0))
    if getattr(cfg, "n_experts", 0) > 0:
        c.n_experts = int(cfg.n_experts)
        c.n_experts_per_tok = int(cfg.n_experts_per_tok)
        c.moe_ffn = int(cfg.moe_ffn)
        c.moe_norm_topk = 1 if getattr(cfg, "moe_norm_topk", True) else 0
        kinds_ffn = cfg.ffn_kinds() if hasattr(cfg, "ffn_kinds") else tuple(cfg.ffn_kind)
        arr = (c_i32 * max(1, len(kinds_ffn)))(*[FFN_KIND[k] for k in kinds_ffn])
        keep.append(arr)
        c.ffn_kind = ctypes.cast(arr, ctypes.POINTER(c_i32))
    for field in ("rope_short_factor", "rope_long_factor"):
        vals = tuple(getattr(cfg, field, ()) or ())
        if vals:
            arr = (c_f32 * len(vals))(*vals)
            keep.append(arr)
            setattr(c, field, ctypes.cast(arr, ctypes.POINTER(c_f32)))
    return c, keep


def output_sizes(cfg, B: int, S: int, max_tokens: Optional[int] = None) -> Dict[str, int]:
    c, keep = make_config(cfg, max_tokens or max(1, B * S))
    s = FwdSizes()
    _check(lib().fwd_output_sizes(ctypes.byref(c), B, S, ctypes.byref(s)))
    return {f: getattr(s, f) for f, _ in FwdSizes._fields_}


def to_device(arr: np.ndarray):
    """Host array in storage form -> device tensor on the current GPU: float32 stays
    float32, uint16 (bf16 bit patterns) becomes bfloat16 (bits unchanged)."""
    import torch
    if arr.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(arr)).cuda()


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    return getattr(stream, "cuda_stream", stream)


class Model:
    """A model on the current GPU: fwd_create at construction, fwd_destroy on close()."""

    LAYER_FIELDS = ("attn_norm", "wq", "wk", "wv", "wo", "ffn_norm", "w_gate", "w_up", "w_down",
                    "post_attn_norm", "post_ffn_norm", "q_norm", "k_norm", "router", "expert_gate", "expert_up",
                    "expert_down")

    def __init__(self, cfg, weights: Mapping[str, "object"], max_tokens: int, stream=None):
        self.cfg = cfg
        self.max_tokens = max_tokens
        self._stream = _stream(stream)
        c, keep = make_config(cfg, max_tokens)
        layers = (FwdLayerWeights * max(1, cfg.n_layers))()
        for l in range(cfg.n_layers):
            for f in self.LAYER_FIELDS:
                t = weights.get(f"layers.{l}.{f}")
                setattr(layers[l], f, _ptr(t))
        w = FwdWeights(embed=_ptr(weights.get("embed")), final_norm=_ptr(weights.get("final_norm")),
                       layers=ctypes.cast(layers, ctypes.POINTER(FwdLayerWeights)))
        h = c_vp()
        _check(lib().fwd_create(ctypes.byref(c), ctypes.byref(w), self._stream, ctypes.byref(h)))
        self._h = h

    def close(self) -> None:
        if getattr(self, "_h", None) and self._h.value:
            lib().fwd_destroy(self._h)
            self._h = c_vp()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def set_timing(self, enable: bool) -> None:
        """Per-kernel-class HIP-event timing of later prefills (clears the totals)."""
        _check(lib().fwd_set_timing(self._h, 1 if enable else 0))

    def timing(self) -> Dict[str, Dict[str, float]]:
        """{class: {"ms": total milliseconds, "launches": n}} since set_timing(True)."""
        out = {}
        for i, name in enumerate(KERNEL_CLASSES):
            ms, n = c_f64(), c_i64()
            _check(lib().fwd_get_timing(self._h, i, ctypes.byref(ms), ctypes.byref(n)))
            out[name] = {"ms": ms.value, "launches": n.value}
        return out

    def prefill_into(self, ids: np.ndarray, logits=None, hidden=None, argmax=None) -> None:
        """fwd_prefill writing into caller-allocated device tensors (any may be None)."""
        ids = np.ascontiguousarray(ids, dtype=np.int32)
        B, S = ids.shape
        out = FwdOutputs(logits=_ptr(logits), hidden=_ptr(hidden), argmax=_ptr(argmax))
        _check(lib().fwd_prefill(self._h, ids.ctypes.data, B, S, ctypes.byref(out)))

    def prefill(self, ids: np.ndarray, logits: bool = True, hidden: bool = False, argmax: bool = True):
        """Allocate the requested outputs with torch on the current device and run fwd_prefill."""
        import torch
        ids = np.ascontiguousarray(ids, dtype=np.int32)
        B, S = ids.shape
        cfg = self.cfg
        dev = torch.device("cuda", torch.cuda.current_device())
        res = {
            "logits": torch.empty((B, S, cfg.vocab), dtype=torch.float32, device=dev) if logits else None,
            "hidden": torch.empty((cfg.n_layers + 2, B, S, cfg.hidden), dtype=torch.float32, device=dev)
            if hidden else None,
            "argmax": torch.empty((B, S), dtype=torch.int32, device=dev) if argmax else None,
        }
        self.prefill_into(ids, res["logits"], res["hidden"], res["argmax"])
        return res


class Session:
    """A KV-cache session on a Model (fwd_session_*): prefill, then one token per step."""

    def __init__(self, model: Model, max_batch: int, max_seq: int):
        self.model = model
        h = c_vp()
        _check(lib().fwd_session_create(model._h, max_batch, max_seq, ctypes.byref(h)))
        self._h = h

    def close(self) -> None:
        if getattr(self, "_h", None) and self._h.value:
            lib().fwd_session_destroy(self._h)
            self._h = c_vp()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    @property
    def length(self) -> int:
        return int(lib().fwd_session_length(self._h))

    def _outputs(self, B: int, S: int, logits: bool, hidden: bool, argmax: bool):
        import torch
        cfg = self.model.cfg
        dev = torch.device("cuda", torch.cuda.current_device())
        return {
            "logits": torch.empty((B, S, cfg.vocab), dtype=torch.float32, device=dev) if logits else None,
            "hidden": torch.empty((cfg.n_layers + 2, B, S, cfg.hidden), dtype=torch.float32, device=dev)
            if hidden else None,
            "argmax": torch.empty((B, S), dtype=torch.int32, device=dev) if argmax else None,
        }

    def prefill(self, ids: np.ndarray, logits: bool = True, hidden: bool = False, argmax: bool = True):
        """fwd_session_prefill over ids [B, S]; outputs shaped as Model.prefill's."""
        ids = np.ascontiguousarray(ids, dtype=np.int32)
        B, S = ids.shape
        res = self._outputs(B, S, logits, hidden, argmax)
        out = FwdOutputs(logits=_ptr(res["logits"]), hidden=_ptr(res["hidden"]), argmax=_ptr(res["argmax"]))
        _check(lib().fwd_session_prefill(self._h, ids.ctypes.data, B, S, ctypes.byref(out)))
        return res

    def decode(self, ids: np.ndarray, logits: bool = True, hidden: bool = False, argmax: bool = True):
        """fwd_session_decode of one token per sequence, ids [B]; outputs with S = 1."""
        ids = np.ascontiguousarray(np.asarray(ids).reshape(-1), dtype=np.int32)
        res = self._outputs(ids.size, 1, logits, hidden, argmax)
        out = FwdOutputs(logits=_ptr(res["logits"]), hidden=_ptr(res["hidden"]), argmax=_ptr(res["argmax"]))
        _check(lib().fwd_session_decode(self._h, ids.ctypes.data, ctypes.byref(out)))
        return res


def gemm(X, W, Y=None, stream=None, noalloc: bool = False):
    """Y = X·Wᵀ (fwd_gemm; fwd_gemm_noalloc with noalloc=True, which needs Y given to
    allocate nothing). X [P, in], W [out, in] torch tensors (bf16 or f32) on the GPU."""
    import torch
    P, K = X.shape
    N = W.shape[0]
    dt = "bf16" if X.dtype == torch.bfloat16 else "f32"
    if Y is None:
        Y = torch.empty((P, N), dtype=torch.float32, device=X.device)
    call = lib().fwd_gemm_noalloc if noalloc else lib().fwd_gemm
    _check(call(X.data_ptr(), W.data_ptr(), Y.data_ptr(), P, K, N, DTYPE[dt], _stream(stream)))
    return Y


def attention(q, k, v_t, window: int = 0, o=None, stream=None):
    """fwd_attention: q [B,S,Hq,D], k [B,S,Hkv,D], v_t [B,Hkv,D,Sp] (Sp = S rounded up to 8)."""
    import torch
    B, S, Hq, D = q.shape
    Hkv = k.shape[2]
    dt = "bf16" if q.dtype == torch.bfloat16 else "f32"
    if o is None:
        o = torch.empty_like(q)
    _check(lib().fwd_attention(q.data_ptr(), k.data_ptr(), v_t.data_ptr(), o.data_ptr(), B, S, Hq, Hkv, D, window,
                               DTYPE[dt], _stream(stream)))
    return o


def rmsnorm(x, w, eps: float, dtype: str = "bf16", y=None, stream=None):
    """fwd_rmsnorm: x fp32 [rows, H], w fp32 [H] -> y [rows, H] of dtype."""
    import torch
    rows, H = x.shape
    if y is None:
        y = torch.empty((rows, H), dtype=torch.bfloat16 if dtype == "bf16" else torch.float32, device=x.device)
    _check(lib().fwd_rmsnorm(x.data_ptr(), w.data_ptr(), y.data_ptr(), rows, H, eps, DTYPE[dtype], _stream(stream)))
    return y


def moe_route(logits, k: int, norm_topk: bool = True, stream=None):
    """fwd_moe_route: router logits fp32 [T, E] -> (idx int32 [T, k], w fp32 [T, k])."""
    import torch
    T, E = logits.shape
    idx = torch.empty((T, k), dtype=torch.int32, device=logits.device)
    w = torch.empty((T, k), dtype=torch.float32, device=logits.device)
    _check(lib().fwd_moe_route(logits.data_ptr(), T, E, k, 1 if norm_topk else 0, idx.data_ptr(), w.data_ptr(),
                               _stream(stream)))
    return idx, w
