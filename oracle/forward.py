"""Plain float64 reference of the prefill forward pass (test infrastructure only).

Sources (page title, then the passage):
  [fp]  "N7 · model/forward-parity" — intro (the op list: embedding lookup, decoder
        stack of RMSNorm, RoPE, causal GQA attention, SwiGLU, residuals and
        topology-selected norm placement, final norm, tied LM head, per-layer hidden
        states, per-position logits) and Theorem 1 (hidden slots, argmax, logits).
  [pi]  "pegainfer issue #878" — Description and Proposed Plan (scaled embedding,
        layer map of local/global layers, final-logit softcap, id bounds check,
        bf16-rounded embedding scale, non-finite values fail).
  [mg]  "N9 · metalgemm" — Theorem 1 (Y = X·Wᵀ with W[out, in]; reference GEMM is a
        float64-accumulated f32 triple loop; err/scale error model).

  Architecture variants: [fp] Theorem statement names the family axes the forward
  must cover (qwen3 QK-norm, gemma3 local/global attention with sandwich norm,
  llama3 rope scaling, phi3 longrope) but gives no formula for them. Those functions
  below follow the families' published definitions, each restated where it is used:
  QK-norm, (1 + w) norm gains, the tanh-approximated GELU gate, a separate RoPE base
  for local layers, the llama3 frequency bands and the longrope per-frequency factors;
  and the mixture-of-experts feed-forward of the hybrid dense/sparse family (qwen3moe).

Every function takes float32 arrays, computes in float64 and returns float32.
Where the pages leave a point open this file takes the plainest reading: rotate-half
RoPE pairs, attention scale 1/sqrt(D), a window W keeps keys with 0 <= i - j < W,
the softcap is applied before the argmax, ties go to the lowest index, and every
row of a batch is its own sequence at positions 0..S-1.
"""
from __future__ import annotations

import math

import numpy as np

_ROW_CHUNK = 8192  # output rows of W widened to float64 at a time (bounds memory only)


def _f64(a) -> np.ndarray:
    return np.asarray(a, dtype=np.float64)


def _f32(a) -> np.ndarray:
    return np.asarray(a, dtype=np.float64).astype(np.float32)


def round_bf16(a) -> np.ndarray:
    """float32 -> nearest bf16 (ties to even) -> float32. Used only by the diagnostic
    mode of forward(), which rounds where a bf16 implementation must round, to tell a
    precision deficit from a bug; the reference itself never rounds activations.

    The IEEE conversion: finite values round to nearest, ties to the even neighbour
    (overflowing to infinity past the largest bf16); infinities and zeros keep their
    sign; a NaN stays a NaN (quietened, so that a payload held only in the dropped low
    bits cannot turn into an infinity)."""
    x = np.asarray(a, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16) << 16
    r = np.where(np.isnan(x), (u | 0x400000) >> 16 << 16, r)
    return r.astype(np.uint32).view(np.float32)


# ---------------------------------------------------------------- projections
def gemm(X, W) -> np.ndarray:
    """Y[p, o] = sum_i X[p, i] * W[o, i] — [mg] Theorem 1 (row-major W[out, in]).

    Accumulated in float64 (numpy matmul), rounded once to float32. Output columns
    are produced in independent chunks of W's rows; no sum is split.
    """
    X64 = _f64(X)
    W = np.asarray(W)
    out = np.empty(X64.shape[:-1] + (W.shape[0],), dtype=np.float32)
    for o0 in range(0, W.shape[0], _ROW_CHUNK):
        Wc = _f64(W[o0:o0 + _ROW_CHUNK])
        out[..., o0:o0 + Wc.shape[0]] = _f32(X64 @ Wc.T)
    return out


# ---------------------------------------------------------------- embedding
def embed_scale(mode: str, hidden: int) -> float:
    """Embedding multiplier — [pi] Proposed Plan / Acceptance Criteria.

    "bf16_sqrt_hidden": sqrt(hidden) rounded to the nearest bf16 value (ties to
    even), the recorded bf16-rounded scale the issue asserts against. "none": 1.
    """
    if mode == "none":
        return 1.0
    if mode != "bf16_sqrt_hidden":
        raise ValueError(f"embed_scale_mode {mode!r}")
    r = math.sqrt(hidden)
    m, e = math.frexp(r)              # r = m * 2**e, 0.5 <= m < 1
    ulp = 2.0 ** (e - 8)              # bf16 keeps 8 significant bits
    q = r / ulp
    lo = math.floor(q)
    frac = q - lo
    if frac > 0.5 or (frac == 0.5 and lo % 2 == 1):
        lo += 1
    return lo * ulp


def embed(E, ids, scale: float) -> np.ndarray:
    """x0[b, t, :] = E[ids[b, t], :] * scale — [fp] intro (embedding lookup), [pi] Plan.

    ids are bounds-checked against the embedding's rows first ([pi] Proposed Plan).
    """
    ids = np.asarray(ids)
    V = np.asarray(E).shape[0]
    if ids.size and (ids.min() < 0 or ids.max() >= V):
        raise ValueError("token id outside [0, vocab)")
    return _f32(_f64(np.asarray(E)[ids]) * scale)


# ---------------------------------------------------------------- normalisation
def rmsnorm(x, w, eps: float, offset: float = 0.0) -> np.ndarray:
    """y_i = x_i * (offset + w_i) / sqrt(mean_j x_j^2 + eps) over the last axis — [fp]
    intro, [mg] intro. offset = 1 is the (1 + w) gain of the gemma3 family."""
    x64 = _f64(x)
    ms = np.mean(x64 * x64, axis=-1, keepdims=True)
    return _f32(x64 / np.sqrt(ms + eps) * (offset + _f64(w)))


# ---------------------------------------------------------------- rotary embedding
def rotate(x, positions, inv_freq, mult: float = 1.0) -> np.ndarray:
    """Rotary embedding of x[..., S, nheads, D] with per-pair frequencies inv_freq[D/2]
    — [fp] intro (RoPE). Rotate-half pairing (the HF convention the forward-parity
    oracle exports): the pair (x_k, x_{k+D/2}) at position p turns by p * inv_freq[k],
    and both cos and sin carry the multiplier `mult` (1 except under longrope)."""
    x64 = _f64(x)
    half = x64.shape[-1] // 2
    ang = _f64(positions)[:, None] * _f64(inv_freq)[None, :]    # [S, D/2]
    c = mult * np.cos(ang)[:, None, :]
    s = mult * np.sin(ang)[:, None, :]
    a, b = x64[..., :half], x64[..., half:]
    return _f32(np.concatenate([a * c - b * s, a * s + b * c], axis=-1))


def rope(x, positions, theta: float) -> np.ndarray:
    """Plain RoPE: pair k turns by p * theta^(-2k/D) — [fp] intro (RoPE)."""
    D = np.asarray(x).shape[-1]
    k = np.arange(D // 2, dtype=np.float64)
    return rotate(x, positions, theta ** (-2.0 * k / D))


def rope_frequencies(cfg, kind: str, seq_len: int):
    """(inv_freq [D/2] float64, multiplier) of a layer of `kind` in a forward whose
    sequence is seq_len tokens long.

    Family axes of [fp] Theorem statement, with the published definitions:
    - base: rope_theta, or rope_theta_local on local layers when it is set (gemma3
      local/global layers use different bases);
    - "llama3" scaling of the base frequencies f_k = theta^(-2k/D), with wavelength
      2 pi / f_k, original context L0, factors lo < hi and s: wavelengths below L0 / hi
      keep f_k, wavelengths above L0 / lo become f_k / s, and in between
      t = (L0 / wavelength - lo) / (hi - lo) blends them as (1 - t) f_k / s + t f_k;
    - "longrope" (phi3): f_k = 1 / (e_k theta^(2k/D)) with e the long factors when the
      sequence is longer than L0 and the short factors otherwise; cos and sin are
      scaled by sqrt(1 + ln s / ln L0) when s = rope_factor > 1.
    """
    D = cfg.head_dim
    theta = cfg.rope_theta
    local_base = getattr(cfg, "rope_theta_local", 0.0)
    if kind == "local" and local_base > 0:
        theta = local_base
    k = np.arange(D // 2, dtype=np.float64)
    f = theta ** (-2.0 * k / D)
    mode = getattr(cfg, "rope_scaling", "none")
    if mode == "none":
        return f, 1.0
    L0 = float(cfg.rope_original_max_pos)
    s = float(cfg.rope_factor)
    if mode == "llama3":
        lo, hi = float(cfg.rope_low_freq_factor), float(cfg.rope_high_freq_factor)
        wavelen = 2.0 * math.pi / f
        t = (L0 / wavelen - lo) / (hi - lo)
        blended = (1.0 - t) * f / s + t * f
        out = np.where(wavelen < L0 / hi, f, np.where(wavelen > L0 / lo, f / s, blended))
        return out, 1.0
    if mode == "longrope":
        e = np.asarray(cfg.rope_long_factor if seq_len > L0 else cfg.rope_short_factor, dtype=np.float64)
        if e.shape != (D // 2,):
            raise ValueError("longrope factors need head_dim / 2 values")
        out = 1.0 / (e * theta ** (2.0 * k / D))
        mult = math.sqrt(1.0 + math.log(s) / math.log(L0)) if s > 1.0 else 1.0
        return out, mult
    raise ValueError(f"rope_scaling {mode!r}")


# ---------------------------------------------------------------- attention
def _visible(S: int, window: int) -> np.ndarray:
    """mask[i, j]: key j visible from query i — causal, and i - j < window if window > 0.

    [fp] intro (causal attention); [pi] Description: a 1024-token prompt is "exactly
    the sliding window" and evicts nothing, so a window of W keeps keys with i - j < W.
    """
    i = np.arange(S)[:, None]
    j = np.arange(S)[None, :]
    m = j <= i
    if window > 0:
        m &= (i - j) < window
    return m


def attention_probs(q, k, window: int = 0) -> np.ndarray:
    """Softmax weights p[b, h, i, j] (float64) of causal grouped-query attention.

    q [B, S, Hq, D], k [B, S, Hkv, D]; query head h reads KV head h // (Hq / Hkv)
    ([fp] intro: GQA). Scores are q·k / sqrt(D), softmax over visible keys.
    """
    q64, k64 = _f64(q), _f64(k)
    B, S, Hq, D = q64.shape
    Hkv = k64.shape[2]
    if Hq % Hkv:
        raise ValueError("n_heads must be a multiple of n_kv_heads")
    group = Hq // Hkv
    mask = _visible(S, window)
    p = np.empty((B, Hq, S, S), dtype=np.float64)
    for b in range(B):
        for h in range(Hq):
            g = h // group
            s = (q64[b, :, h, :] @ k64[b, :, g, :].T) / math.sqrt(D)
            s = np.where(mask, s, -np.inf)
            m = np.max(s, axis=-1, keepdims=True)
            e = np.where(mask, np.exp(s - m), 0.0)
            p[b, h] = e / np.sum(e, axis=-1, keepdims=True)
    return p


def attention(q, k, v, window: int = 0) -> np.ndarray:
    """o[b, i, h, :] = sum_j p[b, h, i, j] * v[b, j, h // group, :] — [fp] intro, [mg] Theorem 1.

    Sequences of a batch never attend to each other. Returns float32 [B, S, Hq, D].
    """
    v64 = _f64(v)
    B, S, Hkv, D = v64.shape
    Hq = np.asarray(q).shape[2]
    group = Hq // Hkv
    out = np.empty((B, S, Hq, D), dtype=np.float32)
    for b in range(B):
        p = attention_probs(np.asarray(q)[b:b + 1], np.asarray(k)[b:b + 1], window)[0]
        for h in range(Hq):
            out[b, :, h, :] = _f32(p[h] @ v64[b, :, h // group, :])
    return out


def _attention_rounded(q, k, v, window: int) -> np.ndarray:
    """Diagnostic only: attention with the probabilities rounded to bf16 before the
    value product (the normaliser stays exact)."""
    v64 = _f64(v)
    B, S, Hkv, D = v64.shape
    Hq = np.asarray(q).shape[2]
    out = np.empty((B, S, Hq, D), dtype=np.float32)
    for b in range(B):
        p = attention_probs(np.asarray(q)[b:b + 1], np.asarray(k)[b:b + 1], window)[0]
        for h in range(Hq):
            out[b, :, h, :] = _f32(_f64(round_bf16(p[h].astype(np.float32))) @ v64[b, :, h // (Hq // Hkv), :])
    return out


def _bf16_point(a, point: str, trace) -> np.ndarray:
    """One rounding point of the bf16 diagnostic: round_bf16(a); with a trace dict the
    rounded tensor is also kept as trace["bf16." + point] (a test hook, so that each
    point can be checked as one rounding of the exact value of its inputs)."""
    r = round_bf16(a)
    if trace is not None:
        trace["bf16." + point] = r
    return r


# ---------------------------------------------------------------- feed-forward
def silu(z) -> np.ndarray:
    """silu(z) = z / (1 + e^-z), float64 in and out."""
    z64 = _f64(z)
    with np.errstate(over="ignore"):
        return z64 / (1.0 + np.exp(-z64))


def swiglu(g, u) -> np.ndarray:
    """a = silu(g) * u — [fp] intro (SwiGLU FFN), [mg] intro."""
    return _f32(silu(g) * _f64(u))


def gelu_tanh(z) -> np.ndarray:
    """GELU in its tanh form, 0.5 z (1 + tanh(sqrt(2/pi) (z + 0.044715 z^3))), float64
    (the gated FFN activation of the gemma3 family, published definition)."""
    z64 = _f64(z)
    return 0.5 * z64 * (1.0 + np.tanh(math.sqrt(2.0 / math.pi) * (z64 + 0.044715 * z64 ** 3)))


def gated_ffn(g, u, act: str = "silu") -> np.ndarray:
    """a = act(g) * u with act silu (SwiGLU) or gelu_tanh."""
    if act == "silu":
        return swiglu(g, u)
    if act == "gelu_tanh":
        return _f32(gelu_tanh(g) * _f64(u))
    raise ValueError(f"ffn_act {act!r}")


def moe_route(logits, top_k: int, norm_topk: bool):
    """Expert choice of each token from router logits [..., E] (qwen3moe family axis of
    [fp] Theorem statement; [fp] intro lists the MoE FFN; published definition):
    probabilities p = softmax(logits) over all experts; the top_k experts by p (the
    softmax is monotone, so by logit; lowest index first on ties); their weights p,
    divided by their sum when norm_topk. Returns (idx int32 [..., k], w float64 [..., k])."""
    z = _f64(logits)
    m = z.max(axis=-1, keepdims=True)
    e = np.exp(z - m)
    p = e / e.sum(axis=-1, keepdims=True)
    idx = np.argsort(-z, axis=-1, kind="stable")[..., :top_k].astype(np.int32)
    w = np.take_along_axis(p, idx, axis=-1)
    if norm_topk:
        w = w / w.sum(axis=-1, keepdims=True)
    return idx, w


def moe_ffn(n, router, expert_gate, expert_up, expert_down, top_k: int, norm_topk: bool, act: str = "silu",
            logits_out=None):
    """Mixture-of-experts feed-forward of rows n [..., H]: d = sum over the token's top_k
    experts e of w_e * (act(n W_g,e^T) * (n W_u,e^T)) W_d,e^T, in expert-rank order.
    expert_* are [E, F_e, H] / [E, H, F_e] row-major stacks (published qwen3moe form)."""
    n2 = np.asarray(n).reshape(-1, np.shape(n)[-1])
    z = gemm(n2, router)
    if logits_out is not None:  # (test hook: the router logits that decided the routing)
        logits_out.append(z)
    idx, w = moe_route(z, top_k, norm_topk)
    out = np.zeros((n2.shape[0], np.shape(expert_down)[1]), dtype=np.float64)
    for e in np.unique(idx):
        rows, slot = np.nonzero(idx == e)
        a = gated_ffn(gemm(n2[rows], expert_gate[e]), gemm(n2[rows], expert_up[e]), act)
        out[rows] += w[rows, slot][:, None] * _f64(gemm(a, expert_down[e]))
    return _f32(out).reshape(np.shape(n)[:-1] + (out.shape[-1],))


# ---------------------------------------------------------------- head
def softcap(z, cap: float) -> np.ndarray:
    """z <- cap * tanh(z / cap) when cap > 0 — [pi] Description (final-logit softcap)."""
    if cap == 0.0:
        return np.asarray(z, dtype=np.float32)
    if not (cap > 0.0):
        raise ValueError("final_logit_softcap must be positive or 0 (off)")
    return _f32(cap * np.tanh(_f64(z) / cap))


def argmax(z) -> np.ndarray:
    """Per-position argmax over the last axis, lowest index on ties ([fp] Theorem 1).

    Non-finite values fail outright ([pi] Acceptance Criteria).
    """
    z = np.asarray(z)
    if not np.all(np.isfinite(z)):
        raise FloatingPointError("non-finite logits")
    return np.argmax(z, axis=-1).astype(np.int32)


# ---------------------------------------------------------------- whole forward
def forward(cfg, weights, ids, want_logits: bool = True, want_hidden: bool = True, bf16_points: bool = False,
            trace=None):
    """The prefill forward pass over a batch of prompts.

    cfg: an object with the geometry fields n_layers, hidden, n_heads, n_kv_heads,
    head_dim, ffn, vocab, rms_eps, rope_theta, embed_scale_mode,
    final_logit_softcap, sliding_window, norm_placement and a kinds() method giving
    "local"/"global" per layer (the parsed layer map, [pi] Proposed Plan).
    weights: mapping name -> float32 array (names as documented on the workloads).
    ids: int [B, S]; every row is an independent sequence at positions 0..S-1.

    Returns dict(logits [B,S,V] f32, hidden [L+2,B,S,H] f32, argmax [B,S] i32); with
    want_logits=False the head is skipped and logits / argmax are None.
    bf16_points=True is a diagnostic, not the reference: it rounds every matrix-product
    input (normalised activations, rotated q / k, v, attention probabilities and
    output, SwiGLU output) to bf16, as a bf16 implementation does.
    Slots ([fp] Theorem 1): 0 = embedding, l+1 = after layer l, L+1 = final norm.
    trace: optional dict; receives "moe_logits.<l>" = the router logits [B*S, E] of each
    mixture-of-experts layer (to judge how decided the routing was), and with
    bf16_points every rounded tensor as "bf16.<l>.<point>" (points n_attn, q_proj,
    k_proj (QK-norm only), v, q, k, o, n_ffn, a) and "bf16.h", plus the residual after
    each attention sublayer as "bf16.<l>.x_attn".
    """
    ids = np.asarray(ids)
    B, S = ids.shape
    H, Hq, Hkv, D = cfg.hidden, cfg.n_heads, cfg.n_kv_heads, cfg.head_dim
    L = cfg.n_layers
    eps = cfg.rms_eps
    sandwich = cfg.norm_placement == "sandwich"
    if cfg.norm_placement not in ("pre", "sandwich"):
        raise ValueError("norm_placement")
    kinds = cfg.kinds()
    positions = np.arange(S)
    goff = float(getattr(cfg, "norm_gain_offset", 0))
    act = getattr(cfg, "ffn_act", "silu")
    qk_norm = bool(getattr(cfg, "qk_norm", False))
    ffn_kinds = cfg.ffn_kinds() if hasattr(cfg, "ffn_kinds") else ("dense",) * L

    E = weights["embed"]
    x = embed(E, ids, embed_scale(cfg.embed_scale_mode, H))            # [B, S, H]
    hidden = np.empty((L + 2, B, S, H), dtype=np.float32) if want_hidden else None
    if want_hidden:
        hidden[0] = x

    def rb(a, point):  # a rounding point of the bf16 diagnostic (identity otherwise)
        return _bf16_point(a, point, trace) if bf16_points else a

    for l in range(L):
        p = f"layers.{l}."
        window = cfg.sliding_window if kinds[l] == "local" else 0
        # attention sublayer
        n = rb(rmsnorm(x, weights[p + "attn_norm"], eps, goff), f"{l}.n_attn")
        q = gemm(n, weights[p + "wq"]).reshape(B, S, Hq, D)
        k = gemm(n, weights[p + "wk"]).reshape(B, S, Hkv, D)
        v = rb(gemm(n, weights[p + "wv"]).reshape(B, S, Hkv, D), f"{l}.v")
        if qk_norm:  # each head's q and k normalised over its D dims, before RoPE (qwen3 / gemma3)
            q = rmsnorm(rb(q, f"{l}.q_proj"), weights[p + "q_norm"], eps, goff)
            k = rmsnorm(rb(k, f"{l}.k_proj"), weights[p + "k_norm"], eps, goff)
        f, mult = rope_frequencies(cfg, kinds[l], S)
        q = rb(np.stack([rotate(q[b], positions, f, mult) for b in range(B)]), f"{l}.q")
        k = rb(np.stack([rotate(k[b], positions, f, mult) for b in range(B)]), f"{l}.k")
        o = rb(_attention_rounded(q, k, v, window) if bf16_points else attention(q, k, v, window), f"{l}.o")
        o = o.reshape(B, S, Hq * D)
        u = gemm(o, weights[p + "wo"])
        if sandwich:
            u = rmsnorm(u, weights[p + "post_attn_norm"], eps, goff)
        x = _f32(_f64(x) + _f64(u))
        if bf16_points and trace is not None:
            trace[f"bf16.{l}.x_attn"] = x
        # feed-forward sublayer (dense, or mixture of experts on the layers the map names)
        n = rb(rmsnorm(x, weights[p + "ffn_norm"], eps, goff), f"{l}.n_ffn")
        if ffn_kinds[l] == "moe":
            zs = [] if trace is not None else None
            d = moe_ffn(n, weights[p + "router"], weights[p + "expert_gate"], weights[p + "expert_up"],
                        weights[p + "expert_down"], cfg.n_experts_per_tok, cfg.moe_norm_topk, act, zs)
            if trace is not None:
                trace[f"moe_logits.{l}"] = zs[0]
        else:
            a = rb(gated_ffn(gemm(n, weights[p + "w_gate"]), gemm(n, weights[p + "w_up"]), act), f"{l}.a")
            d = gemm(a, weights[p + "w_down"])
        if sandwich:
            d = rmsnorm(d, weights[p + "post_ffn_norm"], eps, goff)
        x = _f32(_f64(x) + _f64(d))
        if want_hidden:
            hidden[l + 1] = x

    h = rmsnorm(x, weights["final_norm"], eps, goff)
    if want_hidden:
        hidden[L + 1] = h
    if not want_logits:                          # hidden slots only: the head is not needed
        return {"argmax": None, "hidden": hidden, "logits": None}
    z = softcap(gemm(rb(h, "h"), E), cfg.final_logit_softcap)           # tied head
    return {"argmax": argmax(z), "hidden": hidden, "logits": z}


# ---------------------------------------------------------------- greedy continuation
def greedy(cfg, weights, ids, n_tokens: int):
    """Greedy continuation by repeated cacheless forwards ([fp] Theorem 1: the greedy
    continuation ids; the cached session must reproduce the cacheless forward).

    Token i (i = 0 .. n_tokens-1) of every row is the argmax of the last position's
    logits of a forward over the prompt followed by tokens 0 .. i-1. Nothing is cached.
    Returns (tokens int32 [B, n_tokens], logits f32 [n_tokens, B, V]); logits[i] are
    the last-position logits that chose token i.
    """
    seq = np.asarray(ids, dtype=np.int32)
    B = seq.shape[0]
    toks = np.empty((B, n_tokens), dtype=np.int32)
    logits = np.empty((n_tokens, B, cfg.vocab), dtype=np.float32)
    for i in range(n_tokens):
        z = forward(cfg, weights, seq, want_logits=True, want_hidden=False)["logits"][:, -1]
        logits[i] = z
        toks[:, i] = argmax(z)
        seq = np.concatenate([seq, toks[:, i:i + 1]], axis=1)
    return toks, logits
