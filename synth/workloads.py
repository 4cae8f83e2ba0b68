"""Workload presets: model geometry, token-batch shapes and weight recipes.

Pure data plus draws from the shared generator. Names of tensors are the keys the
oracle and the library binding both read:

  embed [V, H]                                  (tied LM head)
  layers.{l}.attn_norm / ffn_norm [H]           (RMSNorm gains)
  layers.{l}.post_attn_norm / post_ffn_norm [H] (sandwich norm only)
  layers.{l}.wq [Hq*D, H], wk/wv [Hkv*D, H], wo [H, Hq*D]
  layers.{l}.w_gate / w_up [F, H], w_down [H, F]
  final_norm [H]

Matrices are N(0, 0.02^2); norm gains are 1.0 (gains drawn from N(0, 0.02^2) would
shrink every normalised activation ~50x and make attention scores and RoPE
numerically invisible, so the plainest non-degenerate reading sets them to one).
"""
from __future__ import annotations

import dataclasses
from typing import Dict, List, Optional, Tuple

import numpy as np

from . import SEED_GEMM, SEED_IDS, SEED_WEIGHTS, WEIGHT_SIGMA, bf16_bits_to_f32, normal, to_bf16_bits, token_ids


@dataclasses.dataclass(frozen=True)
class ModelConfig:
    name: str
    n_layers: int
    hidden: int
    n_heads: int
    n_kv_heads: int
    head_dim: int
    ffn: int
    vocab: int
    rms_eps: float = 1e-5
    rope_theta: float = 10000.0
    embed_scale_mode: str = "none"        # "none" | "bf16_sqrt_hidden"
    final_logit_softcap: float = 0.0      # 0 = off
    sliding_window: int = 0               # 0 = none
    layer_kind: Tuple[str, ...] = ()      # "local" | "global" per layer; empty = all global
    norm_placement: str = "pre"           # "pre" | "sandwich"
    dtype: str = "bf16"                   # "f32" | "bf16"
    batch: int = 1
    seq: int = 16
    # architecture variants (family axes: QK-norm, (1 + w) gains, gated-GELU FFN,
    # per-kind RoPE base, RoPE frequency scaling)
    qk_norm: bool = False                 # RMSNorm over each q and k head (gains q_norm / k_norm [D])
    norm_gain_offset: int = 0             # 0: norms scale by w; 1: by (1 + w)
    ffn_act: str = "silu"                 # "silu" | "gelu_tanh"
    rope_theta_local: float = 0.0         # RoPE base of local layers (0 = rope_theta)
    rope_scaling: str = "none"            # "none" | "llama3" | "longrope"
    rope_factor: float = 1.0
    rope_low_freq_factor: float = 1.0     # llama3
    rope_high_freq_factor: float = 4.0    # llama3
    rope_original_max_pos: int = 0        # llama3 / longrope
    rope_short_factor: Tuple[float, ...] = ()  # longrope, D / 2 values
    rope_long_factor: Tuple[float, ...] = ()   # longrope, D / 2 values
    gain_sigma: float = 0.0               # > 0: norm gains drawn as neutral + N(0, sigma^2)
    # mixture-of-experts feed-forward (qwen3moe-style hybrid dense / sparse layers)
    n_experts: int = 0                    # 0: dense feed-forward everywhere
    n_experts_per_tok: int = 0            # top-k
    moe_ffn: int = 0                      # width of each expert's gated FFN
    moe_norm_topk: bool = True            # renormalise the top-k probabilities to sum 1
    ffn_kind: Tuple[str, ...] = ()        # "dense" | "moe" per layer; empty = all "moe" when n_experts > 0
    router_sigma: float = 0.0             # router weight spread (0: the matrix sigma)

    def ffn_kinds(self) -> Tuple[str, ...]:
        if self.n_experts <= 0:
            return ("dense",) * self.n_layers
        return self.ffn_kind if self.ffn_kind else ("moe",) * self.n_layers

    def kinds(self) -> Tuple[str, ...]:
        return self.layer_kind if self.layer_kind else ("global",) * self.n_layers

    def replace(self, **kw) -> "ModelConfig":
        return dataclasses.replace(self, **kw)


def _gemma_layer_map(n_layers: int) -> Tuple[str, ...]:
    # five sliding-window layers, then one global layer, repeated
    return tuple("global" if (l % 6) == 5 else "local" for l in range(n_layers))


TINY_F32 = ModelConfig("tiny-llama-f32", 2, 64, 4, 2, 16, 172, 512, dtype="f32", batch=1, seq=16)
SMOLLM2_135M = ModelConfig("smollm2-135m-shape", 30, 576, 9, 3, 64, 1536, 49152, batch=1, seq=512)
GEMMA3_STYLE = ModelConfig(
    "gemma3-style-48L", 48, 3840, 16, 8, 256, 15360, 262144,
    embed_scale_mode="bf16_sqrt_hidden", final_logit_softcap=30.0, sliding_window=1024,
    layer_kind=_gemma_layer_map(48), norm_placement="sandwich", batch=1, seq=1024)
LLAMA3_8B = ModelConfig("llama3-8b-shape", 32, 4096, 32, 8, 128, 14336, 128256,
                        rope_theta=500000.0, batch=8, seq=2048)

MODELS: Dict[str, ModelConfig] = {c.name: c for c in (TINY_F32, SMOLLM2_135M, GEMMA3_STYLE, LLAMA3_8B)}

# Standalone GEMM sweep Y = X W^T, [P, in, out]; inputs N(0, 1) bf16.
GEMM_SWEEP: List[Tuple[int, int, int]] = [
    (16, 64, 96), (64, 512, 256), (256, 1536, 1536), (4096, 4096, 14336), (8192, 4096, 128256)]


def weight_shapes(cfg: ModelConfig) -> Dict[str, Tuple[Tuple[int, ...], str]]:
    """name -> (shape, kind) with kind 'matrix' (N(0, 0.02^2)), 'router' (N(0, router_sigma^2))
    or 'gain' (ones, or spread by gain_sigma)."""
    H, D, F = cfg.hidden, cfg.head_dim, cfg.ffn
    out = {"embed": ((cfg.vocab, H), "matrix"), "final_norm": ((H,), "gain")}
    for l in range(cfg.n_layers):
        p = f"layers.{l}."
        out[p + "attn_norm"] = ((H,), "gain")
        out[p + "wq"] = ((cfg.n_heads * D, H), "matrix")
        out[p + "wk"] = ((cfg.n_kv_heads * D, H), "matrix")
        out[p + "wv"] = ((cfg.n_kv_heads * D, H), "matrix")
        out[p + "wo"] = ((H, cfg.n_heads * D), "matrix")
        out[p + "ffn_norm"] = ((H,), "gain")
        out[p + "w_gate"] = ((F, H), "matrix")
        out[p + "w_up"] = ((F, H), "matrix")
        out[p + "w_down"] = ((H, F), "matrix")
        if cfg.norm_placement == "sandwich":
            out[p + "post_attn_norm"] = ((H,), "gain")
            out[p + "post_ffn_norm"] = ((H,), "gain")
        if cfg.qk_norm:
            out[p + "q_norm"] = ((D,), "gain")
            out[p + "k_norm"] = ((D,), "gain")
        if cfg.ffn_kinds()[l] == "moe":  # the sparse layer replaces the dense FFN weights
            for n in ("w_gate", "w_up", "w_down"):
                del out[p + n]
            E, Fe = cfg.n_experts, cfg.moe_ffn
            out[p + "router"] = ((E, H), "router")
            out[p + "expert_gate"] = ((E, Fe, H), "matrix")
            out[p + "expert_up"] = ((E, Fe, H), "matrix")
            out[p + "expert_down"] = ((E, H, Fe), "matrix")
    return out


def draw_weight(cfg: ModelConfig, name: str, seed: int = SEED_WEIGHTS) -> np.ndarray:
    """One weight tensor in the config's storage type: float32, or uint16 bf16 bits."""
    shape, kind = weight_shapes(cfg)[name]
    if kind == "gain":
        # the neutral gain is 1 (or 0 when norms scale by 1 + w); gain_sigma > 0 spreads it
        neutral = 0.0 if cfg.norm_gain_offset else 1.0
        if cfg.gain_sigma > 0:
            g = normal(seed, name, shape, cfg.gain_sigma, "f32") + np.float32(neutral)
        else:
            g = np.full(shape, neutral, dtype=np.float32)
        return g if cfg.dtype == "f32" else to_bf16_bits(g)
    if kind == "router":
        return normal(seed, name, shape, cfg.router_sigma or WEIGHT_SIGMA, cfg.dtype)
    return normal(seed, name, shape, WEIGHT_SIGMA, cfg.dtype)


class LazyWeights:
    """Mapping name -> float32 array, drawn on access (bf16 storage widened exactly).

    Large configs hold tens of GB of weights; the oracle reads them layer by layer
    through this mapping, so only a layer's worth is alive at a time.
    """

    def __init__(self, cfg: ModelConfig, seed: int = SEED_WEIGHTS, cache: bool = False):
        self.cfg, self.seed, self._cache = cfg, seed, ({} if cache else None)
        self._names = weight_shapes(cfg)

    def __contains__(self, name):
        return name in self._names

    def keys(self):
        return self._names.keys()

    def __getitem__(self, name):
        if self._cache is not None and name in self._cache:
            return self._cache[name]
        raw = draw_weight(self.cfg, name, self.seed)
        arr = raw if self.cfg.dtype == "f32" else bf16_bits_to_f32(raw)
        if self._cache is not None:
            self._cache[name] = arr
        return arr


class HostWeights:
    """Mapping name -> float32 view of arrays already drawn in storage form
    (bf16 bit patterns are widened exactly on access)."""

    def __init__(self, raw: Dict[str, np.ndarray]):
        self.raw = raw

    def __contains__(self, name):
        return name in self.raw

    def keys(self):
        return self.raw.keys()

    def __getitem__(self, name):
        a = self.raw[name]
        return bf16_bits_to_f32(a) if a.dtype == np.uint16 else a


def draw_all(cfg: ModelConfig, seed: int = SEED_WEIGHTS) -> Dict[str, np.ndarray]:
    """Every weight of cfg in storage form (float32, or uint16 bf16 bits)."""
    return {n: draw_weight(cfg, n, seed) for n in weight_shapes(cfg)}


def draw_ids(cfg: ModelConfig, batch: Optional[int] = None, seq: Optional[int] = None,
             seed: int = SEED_IDS) -> np.ndarray:
    """int32 [B, S] token ids uniform in [0, V). A shorter draw is a prefix of a longer
    one only in the flattened order, so prefix tests slice a full draw instead."""
    return token_ids(seed, "ids", batch or cfg.batch, seq or cfg.seq, cfg.vocab)


def draw_gemm(P: int, K: int, N: int, seed: int = SEED_GEMM):
    """bf16 bits X [P, K], W [N, K], both N(0, 1)."""
    X = normal(seed, f"gemm.X.{P}x{K}", (P, K), 1.0, "bf16")
    W = normal(seed, f"gemm.W.{N}x{K}", (N, K), 1.0, "bf16")
    return X, W
