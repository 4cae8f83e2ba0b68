"""Pins of the CPU oracle against facts fixed by the pages and by mathematics.

Each test is chosen so that a plausible mistake in the oracle (a dropped term, a
wrong sign or index, a transposed operand, a wrong pairing) fails it. None of them
re-types the oracle's own formula: they use closed forms, exact rational
arithmetic, invariants and special cases that reduce to something simpler.
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
from synth import workloads as wl

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page_values.json")))
rng = np.random.default_rng(1234)


# ------------------------------------------------------------------ GEMM
def _exact_gemm(X, W):
    P, K = X.shape
    N = W.shape[0]
    Y = np.empty((P, N), dtype=np.float64)
    for p in range(P):
        for o in range(N):
            s = Fraction(0)
            for i in range(K):
                s += Fraction(float(X[p, i])) * Fraction(float(W[o, i]))
            Y[p, o] = float(s)
    return Y


@pytest.mark.parametrize("P,K,N", [(1, 1, 1), (3, 5, 2), (8, 8, 8), (2, 7, 5)])
def test_gemm_matches_exact_rational_sum(P, K, N):
    X = rng.standard_normal((P, K)).astype(np.float32)
    W = rng.standard_normal((N, K)).astype(np.float32)
    exact = _exact_gemm(X, W)
    got = oracle.gemm(X, W).astype(np.float64)
    # one float32 rounding of the exact sum (plus at most a double-rounding ulp)
    ulp = np.spacing(np.abs(exact).astype(np.float32)).astype(np.float64)
    assert np.all(np.abs(got - exact) <= ulp)


def test_gemm_integer_inputs_are_exact_and_not_transposed():
    X = rng.integers(-4, 5, size=(3, 6)).astype(np.float32)
    W = rng.integers(-4, 5, size=(4, 6)).astype(np.float32)
    exact = _exact_gemm(X, W)
    assert np.array_equal(oracle.gemm(X, W), exact.astype(np.float32))
    assert oracle.gemm(X, W).shape == (3, 4)


def test_gemm_identity_and_one_hot():
    X = rng.standard_normal((5, 7)).astype(np.float32)
    assert np.array_equal(oracle.gemm(X, np.eye(7, dtype=np.float32)), X)
    W = rng.standard_normal((6, 7)).astype(np.float32)
    onehot = np.zeros((1, 7), dtype=np.float32)
    onehot[0, 3] = 1.0
    assert np.array_equal(oracle.gemm(onehot, W)[0], W[:, 3])


def test_gemm_err_over_scale_gate_on_page_shapes():
    # the page's error model: err/scale = max|d| / max|ref| against a float64 product
    bound = GOLD["gemm_err_over_scale_max"]["value"]
    for P, K, N in GOLD["gemm_shapes_P_in_out"]["value"]:
        X = rng.standard_normal((P, K)).astype(np.float32)
        W = rng.standard_normal((N, K)).astype(np.float32)
        ref = X.astype(np.float64) @ W.astype(np.float64).T
        err = np.max(np.abs(oracle.gemm(X, W) - ref)) / np.max(np.abs(ref))
        assert err < 1e-6 < bound


# ------------------------------------------------------------------ RMSNorm
def test_rmsnorm_hand_example_uses_mean_not_sum():
    y = oracle.rmsnorm(np.array([[3.0, 4.0]], np.float32), np.ones(2, np.float32), 0.0)
    ms = (9.0 + 16.0) / 2.0
    assert np.allclose(y, [[3 / math.sqrt(ms), 4 / math.sqrt(ms)]], rtol=1e-7)


def test_rmsnorm_constant_vector_closed_form():
    c, eps, H = 3.0, 1e-5, 64
    y = oracle.rmsnorm(np.full((2, H), c, np.float32), np.ones(H, np.float32), eps)
    assert np.allclose(y, c / math.sqrt(c * c + eps), rtol=1e-7)
    ms = c * c
    assert math.isclose(float(np.mean(y.astype(np.float64) ** 2)), ms / (ms + eps), rel_tol=1e-6)


def test_rmsnorm_gain_is_elementwise_and_scale_invariant():
    x = rng.standard_normal((4, 32)).astype(np.float32)
    w = rng.standard_normal(32).astype(np.float32)
    one = oracle.rmsnorm(x, np.ones(32, np.float32), 1e-5)
    assert np.allclose(oracle.rmsnorm(x, w, 1e-5), one * w, rtol=1e-6, atol=1e-7)
    one0 = oracle.rmsnorm(x, np.ones(32, np.float32), 0.0)
    assert np.allclose(oracle.rmsnorm(x * 1000.0, np.ones(32, np.float32), 0.0), one0, rtol=1e-6)
    # with eps > 0 the output shrinks by sqrt(ms / (ms + eps)) per row
    ms = np.mean(x.astype(np.float64) ** 2, -1, keepdims=True)
    assert np.allclose(one, one0 * np.sqrt(ms / (ms + 1e-5)), rtol=1e-6)
    # eps matters when the row is tiny: y -> x / sqrt(eps)
    tiny = np.full((1, 8), 1e-6, np.float32)
    assert np.allclose(oracle.rmsnorm(tiny, np.ones(8, np.float32), 1.0), 1e-6, rtol=1e-6)


# ------------------------------------------------------------------ RoPE
def test_rope_d2_turns_by_position_radians():
    x = np.array([[[1.0, 0.0]]] * 4, np.float32)          # [S=4, heads=1, D=2]
    y = oracle.rope(x, np.arange(4), 10000.0)
    for p in range(4):
        assert np.allclose(y[p, 0], [math.cos(p), math.sin(p)], atol=1e-7)


def test_rope_rotate_half_pairing_and_frequency():
    # D = 4: dim 1 pairs with dim 3 and turns at theta^(-2/4) = 1/100 rad per position
    x = np.zeros((4, 1, 4), np.float32)
    x[:, 0, 1] = 1.0
    y = oracle.rope(x, np.arange(4), 10000.0)
    p = 3
    assert np.allclose(y[p, 0], [0.0, math.cos(0.03), 0.0, math.sin(0.03)], atol=1e-7)
    # dim 0 pairs with dim 2 and turns at 1 rad per position
    x = np.zeros((4, 1, 4), np.float32)
    x[:, 0, 0] = 1.0
    y = oracle.rope(x, np.arange(4), 10000.0)
    assert np.allclose(y[2, 0], [math.cos(2), 0.0, math.sin(2), 0.0], atol=1e-7)


def test_rope_preserves_pair_norms_and_is_identity_at_zero():
    D = 64
    x = rng.standard_normal((9, 3, D)).astype(np.float32)
    y = oracle.rope(x, np.arange(9), 500000.0)
    n_in = x[..., :32] ** 2 + x[..., 32:] ** 2
    n_out = y[..., :32].astype(np.float64) ** 2 + y[..., 32:].astype(np.float64) ** 2
    assert np.allclose(n_in, n_out, rtol=1e-5)
    assert np.array_equal(y[0], x[0])


def test_rope_scores_depend_only_on_relative_position():
    D = 16
    q = rng.standard_normal((1, 1, D)).astype(np.float32)
    k = rng.standard_normal((1, 1, D)).astype(np.float32)

    def at(v, p):
        return oracle.rope(v, np.array([p]), 10000.0)[0, 0].astype(np.float64)

    for m, n in [(5, 2), (9, 6), (3, 0), (40, 37)]:
        assert math.isclose(at(q, m) @ at(k, n), at(q, m - n) @ k[0, 0].astype(np.float64), rel_tol=1e-5)


# ------------------------------------------------------------------ attention
def _qkv(B, S, Hq, Hkv, D):
    q = rng.standard_normal((B, S, Hq, D)).astype(np.float32)
    k = rng.standard_normal((B, S, Hkv, D)).astype(np.float32)
    v = rng.standard_normal((B, S, Hkv, D)).astype(np.float32)
    return q, k, v


def test_attention_first_position_returns_its_value_row():
    q, k, v = _qkv(2, 7, 4, 2, 8)
    o = oracle.attention(q, k, v)
    for h in range(4):
        assert np.allclose(o[:, 0, h], v[:, 0, h // 2], rtol=1e-6)
    q1, k1, v1 = q[:, :1], k[:, :1], v[:, :1]
    assert np.allclose(oracle.attention(q1, k1, v1)[:, 0, 3], v1[:, 0, 1], rtol=1e-6)


def test_attention_two_key_closed_form_pins_the_scale():
    D = 4
    q = np.zeros((1, 2, 1, D), np.float32)
    k = np.zeros((1, 2, 1, D), np.float32)
    v = np.zeros((1, 2, 1, D), np.float32)
    k[0, 1, 0, 0] = 1.0                       # k0 = 0, k1 = e0
    q[0, 1, 0, 0] = 2.0 * math.log(3.0)       # s10 = 0, s11 = 2 ln3 / sqrt(4) = ln 3
    v[0, 0, 0] = [1, 0, 0, 0]
    v[0, 1, 0] = [0, 1, 0, 0]
    o = oracle.attention(q, k, v)
    assert np.allclose(o[0, 1, 0], [0.25, 0.75, 0, 0], atol=1e-7)


def test_attention_probabilities_causal_rows_sum_to_one():
    q, k, _ = _qkv(1, 11, 4, 2, 8)
    p = oracle.attention_probs(q, k)
    assert np.allclose(p.sum(-1), 1.0, atol=1e-12)
    iu = np.triu_indices(11, 1)
    assert np.all(p[0, :, iu[0], iu[1]] == 0.0)
    pw = oracle.attention_probs(q, k, window=3)
    assert np.allclose(pw.sum(-1), 1.0, atol=1e-12)
    i, j = np.meshgrid(np.arange(11), np.arange(11), indexing="ij")
    assert np.all(pw[0][:, (i - j) >= 3] == 0.0)
    assert np.all(pw[0][:, (i - j < 3) & (j <= i)] > 0.0)


def test_attention_zero_query_averages_visible_values():
    _, k, v = _qkv(1, 6, 2, 1, 4)
    q = np.zeros((1, 6, 2, 4), np.float32)
    o = oracle.attention(q, k, v)
    for i in range(6):
        assert np.allclose(o[0, i, 1], v[0, :i + 1, 0].mean(0), rtol=1e-6)
    ow = oracle.attention(q, k, v, window=2)
    for i in range(1, 6):
        assert np.allclose(ow[0, i, 0], v[0, i - 1:i + 1, 0].mean(0), rtol=1e-6)


def test_attention_window_special_cases():
    q, k, v = _qkv(1, 9, 2, 2, 8)
    full = oracle.attention(q, k, v)
    assert np.array_equal(oracle.attention(q, k, v, window=9), full)
    assert np.array_equal(oracle.attention(q, k, v, window=100), full)
    assert np.allclose(oracle.attention(q, k, v, window=1), v, rtol=1e-6)
    assert not np.allclose(oracle.attention(q, k, v, window=4)[0, 8], full[0, 8])


def test_attention_gqa_equals_mha_with_repeated_kv_heads():
    q, k, v = _qkv(2, 8, 6, 2, 8)
    gqa = oracle.attention(q, k, v)
    mha = oracle.attention(q, np.repeat(k, 3, axis=2), np.repeat(v, 3, axis=2))
    assert np.allclose(gqa, mha, rtol=1e-6, atol=1e-7)


def test_attention_batch_rows_do_not_mix():
    q, k, v = _qkv(3, 5, 2, 1, 4)
    o = oracle.attention(q, k, v)
    o1 = oracle.attention(q[1:2], k[1:2], v[1:2])
    assert np.array_equal(o[1:2], o1)


# ------------------------------------------------------------------ SwiGLU
def test_silu_closed_forms():
    s = oracle.silu(np.array([0.0, 1.0, -1.0, 40.0, -40.0]))
    assert s[0] == 0.0
    assert math.isclose(s[1], 1.0 / (1.0 + math.exp(-1.0)), rel_tol=1e-15)
    assert math.isclose(s[2], -1.0 / (1.0 + math.exp(1.0)), rel_tol=1e-15)
    assert math.isclose(s[3], 40.0, rel_tol=1e-15)
    assert abs(s[4]) < 1e-15


def test_swiglu_gate_and_up_are_not_interchangeable():
    a = oracle.swiglu(np.array([1.0, 2.0, 0.0], np.float32), np.array([2.0, 1.0, 5.0], np.float32))
    assert np.allclose(a, [2.0 / (1.0 + math.exp(-1.0)), 2.0 / (1.0 + math.exp(-2.0)), 0.0], rtol=1e-7)


# ------------------------------------------------------------------ softcap / argmax
def test_softcap_bounds_monotone_and_small_signal():
    z = np.linspace(-200, 200, 4001).astype(np.float32)
    c = oracle.softcap(z, 30.0)
    assert np.all(np.abs(c) <= 30.0) and np.all(np.diff(c) >= 0)
    small = np.array([1e-3, -2e-2, 0.5], np.float32)
    assert np.all(np.abs(oracle.softcap(small, 30.0) - small) <= np.abs(small) ** 3 / (3 * 900) + 1e-8)
    assert math.isclose(float(oracle.softcap(np.float32(30.0 * math.atanh(0.5)), 30.0)), 15.0, rel_tol=1e-6)
    assert np.array_equal(oracle.softcap(z, 0.0), z)
    with pytest.raises(ValueError):
        oracle.softcap(z, -1.0)
    with pytest.raises(ValueError):
        oracle.softcap(z, float("nan"))


def test_argmax_lowest_index_on_ties_and_nonfinite_fails():
    z = np.array([[1.0, 3.0, 3.0, 2.0], [5.0, 5.0, 5.0, 5.0]], np.float32)
    assert list(oracle.argmax(z)) == [1, 0]
    with pytest.raises(FloatingPointError):
        oracle.argmax(np.array([[1.0, np.nan]], np.float32))
    with pytest.raises(FloatingPointError):
        oracle.argmax(np.array([[1.0, np.inf]], np.float32))


# ------------------------------------------------------------------ embedding
def test_embed_scale_is_bf16_rounded_sqrt():
    assert oracle.embed_scale("bf16_sqrt_hidden", 3840) == 62.0      # sqrt = 61.9677...
    assert math.sqrt(3840) != 62.0
    assert oracle.embed_scale("bf16_sqrt_hidden", 576) == 24.0       # exact square
    assert oracle.embed_scale("bf16_sqrt_hidden", 257 ** 2) == 256.0  # tie -> even mantissa
    assert oracle.embed_scale("bf16_sqrt_hidden", 259 ** 2) == 260.0  # tie -> even mantissa
    assert oracle.embed_scale("bf16_sqrt_hidden", 2) == 1.4140625     # 1.41421... -> 1 + 53/128
    assert oracle.embed_scale("none", 3840) == 1.0


def test_embed_gathers_rows_scales_exactly_and_checks_ids():
    E = rng.standard_normal((10, 6)).astype(np.float32)
    E = (E.view(np.uint32) & 0xFFFF0000).view(np.float32)   # bf16-representable
    ids = np.array([[3, 0, 9]])
    x = oracle.embed(E, ids, 62.0)
    assert np.array_equal(x[0], E[[3, 0, 9]] * np.float32(62.0))
    for bad in ([[10]], [[-1]]):
        with pytest.raises(ValueError):
            oracle.embed(E, np.array(bad), 1.0)


# ------------------------------------------------------------------ whole forward
TINY = wl.TINY_F32


def _weights(cfg, seed=7):
    return {n: wl.LazyWeights(cfg, seed)[n] for n in wl.weight_shapes(cfg)}


def test_forward_shapes_and_slot_convention():
    w = _weights(TINY)
    ids = wl.draw_ids(TINY)
    out = oracle.forward(TINY, w, ids)
    L, H, V = TINY.n_layers, TINY.hidden, TINY.vocab
    assert out["hidden"].shape == (L + 2, 1, 16, H)
    assert out["logits"].shape == (1, 16, V)
    assert np.array_equal(out["hidden"][0], w["embed"][ids])
    assert np.allclose(out["hidden"][L + 1], oracle.rmsnorm(out["hidden"][L], w["final_norm"], TINY.rms_eps))
    assert np.array_equal(out["argmax"], np.argmax(out["logits"], -1))


def test_forward_causal_prefix_invariance():
    w = _weights(TINY)
    ids = wl.draw_ids(TINY)
    full = oracle.forward(TINY, w, ids)
    for s in (1, 5, 11):
        pre = oracle.forward(TINY, w, ids[:, :s])
        assert np.allclose(pre["logits"], full["logits"][:, :s], rtol=1e-6, atol=1e-7)
        assert np.allclose(pre["hidden"], full["hidden"][:, :, :s], rtol=1e-6, atol=1e-7)


def test_forward_batch_rows_are_independent():
    cfg = TINY.replace(batch=3)
    w = _weights(cfg)
    ids = wl.draw_ids(cfg)
    full = oracle.forward(cfg, w, ids)
    one = oracle.forward(cfg, w, ids[2:3])
    assert np.allclose(one["logits"][0], full["logits"][2], rtol=1e-6, atol=1e-7)


def test_forward_zero_layers_argmax_is_the_input_token():
    cfg = TINY.replace(n_layers=0)
    w = _weights(cfg)
    ids = wl.draw_ids(cfg)
    out = oracle.forward(cfg, w, ids)
    # self-dot H*rms(e) ~ 1.28 dominates cross terms ~ N(0, 0.16^2) over 512 rows
    assert np.array_equal(out["argmax"], ids)


def test_forward_residual_passthrough_when_branches_vanish():
    w = _weights(TINY)
    for l in range(TINY.n_layers):
        w[f"layers.{l}.wo"] = np.zeros_like(w[f"layers.{l}.wo"])
        w[f"layers.{l}.w_down"] = np.zeros_like(w[f"layers.{l}.w_down"])
    out = oracle.forward(TINY, w, wl.draw_ids(TINY))
    for s in range(1, TINY.n_layers + 1):
        assert np.array_equal(out["hidden"][s], out["hidden"][0])


def test_forward_single_token_ignores_query_and_key_weights():
    cfg = TINY.replace(seq=1)
    w = _weights(cfg)
    ids = wl.draw_ids(cfg)
    a = oracle.forward(cfg, w, ids)
    w2 = dict(w)
    for l in range(cfg.n_layers):
        w2[f"layers.{l}.wq"] = w[f"layers.{l}.wq"] * -3.0
        w2[f"layers.{l}.wk"] = rng.standard_normal(w[f"layers.{l}.wk"].shape).astype(np.float32)
    b = oracle.forward(cfg, w2, ids)
    assert np.array_equal(a["logits"], b["logits"])


def test_forward_sandwich_norm_cancels_branch_scale():
    base = TINY.replace(rms_eps=1e-12)
    sand = base.replace(norm_placement="sandwich")
    ids = wl.draw_ids(base)
    for cfg, invariant in ((sand, True), (base, False)):
        w = _weights(cfg)
        a = oracle.forward(cfg, w, ids)["logits"]
        for l in range(cfg.n_layers):
            w[f"layers.{l}.wo"] = w[f"layers.{l}.wo"] * 7.0
            w[f"layers.{l}.w_down"] = w[f"layers.{l}.w_down"] * 7.0
        b = oracle.forward(cfg, w, ids)["logits"]
        assert np.allclose(a, b, rtol=1e-4, atol=1e-6) == invariant


def test_forward_layer_map_and_window():
    ids = wl.draw_ids(TINY)
    w = _weights(TINY)
    ref = oracle.forward(TINY, w, ids)["logits"]
    glob = TINY.replace(sliding_window=4, layer_kind=("global", "global"))
    assert np.array_equal(oracle.forward(glob, w, ids)["logits"], ref)
    wide = TINY.replace(sliding_window=16, layer_kind=("local", "local"))
    assert np.array_equal(oracle.forward(wide, w, ids)["logits"], ref)
    narrow = TINY.replace(sliding_window=4, layer_kind=("local", "global"))
    out = oracle.forward(narrow, w, ids)["logits"]
    assert np.array_equal(out[:, :4], ref[:, :4])          # first W positions see everything
    assert not np.allclose(out[:, 4:], ref[:, 4:])


def test_forward_softcap_and_embed_scale_compose():
    capped = TINY.replace(final_logit_softcap=2.0, embed_scale_mode="bf16_sqrt_hidden")
    plain = TINY.replace(embed_scale_mode="bf16_sqrt_hidden")
    w = _weights(TINY)
    ids = wl.draw_ids(TINY)
    a = oracle.forward(capped, w, ids)
    b = oracle.forward(plain, w, ids)
    assert np.array_equal(a["hidden"][0], w["embed"][ids] * np.float32(8.0))   # bf16(sqrt 64) = 8
    assert np.allclose(a["logits"], 2.0 * np.tanh(b["logits"].astype(np.float64) / 2.0), rtol=1e-6, atol=1e-7)
    assert np.all(np.abs(a["logits"]) < 2.0)
    assert np.array_equal(a["argmax"], b["argmax"])


def test_greedy_steps_are_cacheless_forwards():
    """Greedy continuation: token i is the argmax of the last position of a forward over
    the prompt plus tokens 0..i-1; pinned against the forward itself, a restart from the
    extended prompt (catches an off-by-one in the append loop) and per-row independence."""
    w = _weights(TINY)
    ids = np.asarray(wl.draw_ids(TINY.replace(batch=2, seq=5)))
    toks, logits = oracle.greedy(TINY, w, ids, 4)
    first = oracle.forward(TINY, w, ids, want_hidden=False)["logits"][:, -1]
    assert np.array_equal(logits[0], first)
    assert np.array_equal(toks[:, 0], np.argmax(first, axis=-1))
    again, again_logits = oracle.greedy(TINY, w, np.concatenate([ids, toks[:, :1]], axis=1), 3)
    assert np.array_equal(again, toks[:, 1:])
    assert np.array_equal(again_logits, logits[1:])
    for b in range(2):
        one, one_logits = oracle.greedy(TINY, w, ids[b:b + 1], 4)
        assert np.array_equal(one[0], toks[b])
        assert np.allclose(one_logits[:, 0], logits[:, b], rtol=0, atol=1e-6)


# ---------------------------------------------------------------- architecture variants
# [fp] Theorem statement names the family axes (qwen3 QK-norm, gemma3 local/global,
# llama3 rope scaling, phi3 longrope) without formulas; these pins fix the structure
# of the published definitions the oracle restates.

def _llama3_cfg(**kw):
    base = dict(rope_theta=500000.0, rope_scaling="llama3", rope_factor=8.0, rope_low_freq_factor=1.0,
                rope_high_freq_factor=4.0, rope_original_max_pos=8192)
    base.update(kw)
    return wl.LLAMA3_8B.replace(**base)


def test_llama3_scaling_bands():
    cfg = _llama3_cfg()
    D = cfg.head_dim
    plain = 500000.0 ** (-2.0 * np.arange(D // 2) / D)
    f, mult = oracle.rope_frequencies(cfg, "global", 16)
    assert mult == 1.0
    wavelen = 2 * math.pi / plain
    hi_band = wavelen < 8192 / 4.0
    lo_band = wavelen > 8192 / 1.0
    mid = ~hi_band & ~lo_band
    assert hi_band.any() and lo_band.any() and mid.any()     # all three bands occur at D = 128
    assert np.array_equal(f[hi_band], plain[hi_band])        # short wavelengths untouched
    np.testing.assert_allclose(f[lo_band], plain[lo_band] / 8.0, rtol=1e-15)
    assert np.all(f[mid] < plain[mid]) and np.all(f[mid] > plain[mid] / 8.0)
    assert np.all(np.diff(f) < 0)                            # still strictly decreasing in k
    # continuity at both band edges: move the edges onto a pair and compare the limits
    k_edge = int(np.argmax(mid))                             # first blended pair
    for L0 in (wavelen[k_edge] * 4.0, wavelen[k_edge] * 1.0):
        a, _ = oracle.rope_frequencies(_llama3_cfg(rope_original_max_pos=L0 * (1 + 1e-12)), "global", 16)
        b, _ = oracle.rope_frequencies(_llama3_cfg(rope_original_max_pos=L0 * (1 - 1e-12)), "global", 16)
        assert abs(a[k_edge] - b[k_edge]) <= 1e-9 * plain[k_edge]
    # factor 1 is the plain RoPE
    g, _ = oracle.rope_frequencies(_llama3_cfg(rope_factor=1.0), "global", 16)
    np.testing.assert_allclose(g, plain, rtol=1e-15)


def test_longrope_factors_divide_each_frequency_and_switch_at_l0():
    D, L0 = 16, 64
    rng = np.random.default_rng(3)
    short = tuple(float(v) for v in rng.uniform(1.0, 3.0, D // 2))
    long = tuple(float(v) for v in rng.uniform(2.0, 9.0, D // 2))
    cfg = wl.TINY_F32.replace(rope_scaling="longrope", rope_factor=4.0, rope_original_max_pos=L0,
                              rope_short_factor=short, rope_long_factor=long)
    fs, m_s = oracle.rope_frequencies(cfg, "global", L0)
    fl, m_l = oracle.rope_frequencies(cfg, "global", L0 + 1)
    plain = 10000.0 ** (-2.0 * np.arange(D // 2) / D)
    np.testing.assert_allclose(fs, plain / np.array(short), rtol=1e-14)
    np.testing.assert_allclose(fl, plain / np.array(long), rtol=1e-14)
    assert m_s == m_l == pytest.approx(math.sqrt(1 + math.log(4.0) / math.log(L0)), rel=1e-15)
    # pair k rotated at position p equals the plain rotation at position p / e_k
    x = rng.standard_normal((1, 1, D)).astype(np.float32)
    p = 37
    got = oracle.rotate(x, np.array([p]), fs, 1.0)
    for k in range(D // 2):
        ref = oracle.rope(x, np.array([p / short[k]]), 10000.0)
        assert got[0, 0, k] == pytest.approx(ref[0, 0, k], abs=1e-6)
        assert got[0, 0, k + D // 2] == pytest.approx(ref[0, 0, k + D // 2], abs=1e-6)
    # the multiplier scales each pair's norm by mult
    y = oracle.rotate(x, np.array([p]), fs, m_s).astype(np.float64)[0, 0]
    x64 = x.astype(np.float64)[0, 0]
    for k in range(D // 2):
        n_in = math.hypot(x64[k], x64[k + D // 2])
        assert math.hypot(y[k], y[k + D // 2]) == pytest.approx(m_s * n_in, rel=1e-6)
    # no extension (s <= 1) means no multiplier
    _, m1 = oracle.rope_frequencies(cfg.replace(rope_factor=1.0), "global", 8)
    assert m1 == 1.0


def test_local_rope_base_applies_to_local_layers_only():
    cfg = wl.TINY_F32.replace(rope_theta=1e6, rope_theta_local=1e4)
    D = cfg.head_dim
    fg, _ = oracle.rope_frequencies(cfg, "global", 8)
    fl, _ = oracle.rope_frequencies(cfg, "local", 8)
    k = np.arange(D // 2)
    np.testing.assert_allclose(fg, 1e6 ** (-2.0 * k / D), rtol=1e-15)
    np.testing.assert_allclose(fl, 1e4 ** (-2.0 * k / D), rtol=1e-15)
    same, _ = oracle.rope_frequencies(cfg.replace(rope_theta_local=0.0), "local", 8)
    np.testing.assert_allclose(same, fg, rtol=1e-15)


def _f32_weights(cfg):
    return {n: np.asarray(a, np.float32) for n, a in wl.draw_all(cfg).items()}


def test_qk_norm_makes_the_forward_invariant_to_query_and_key_scale():
    cfg = wl.TINY_F32.replace(qk_norm=True, gain_sigma=0.2, rms_eps=1e-12, name="tiny-qknorm")
    w = _f32_weights(cfg)
    ids = wl.draw_ids(cfg)
    base = oracle.forward(cfg, w, ids)["logits"]
    w2 = dict(w)
    for l in range(cfg.n_layers):
        w2[f"layers.{l}.wq"] = w[f"layers.{l}.wq"] * np.float32(4.0)
        w2[f"layers.{l}.wk"] = w[f"layers.{l}.wk"] * np.float32(0.5)
    np.testing.assert_allclose(oracle.forward(cfg, w2, ids)["logits"], base, rtol=0, atol=2e-6)
    # without QK-norm the same scaling changes the scores (non-vacuous)
    plain = cfg.replace(qk_norm=False)
    wp = {n: a for n, a in w.items() if "q_norm" not in n and "k_norm" not in n}
    wp2 = {n: a for n, a in w2.items() if "q_norm" not in n and "k_norm" not in n}
    d = np.abs(oracle.forward(plain, wp2, ids)["logits"] - oracle.forward(plain, wp, ids)["logits"]).max()
    assert d > 1e-3
    # the q / k gains matter: unit gains give a different forward
    w3 = dict(w)
    for l in range(cfg.n_layers):
        w3[f"layers.{l}.q_norm"] = np.ones_like(w[f"layers.{l}.q_norm"])
    assert np.abs(oracle.forward(cfg, w3, ids)["logits"] - base).max() > 1e-4


def test_gain_offset_equals_explicit_one_plus_w():
    cfg = wl.TINY_F32.replace(norm_gain_offset=1, gain_sigma=0.3, qk_norm=True, norm_placement="sandwich",
                              name="tiny-offset")
    w = _f32_weights(cfg)
    ids = wl.draw_ids(cfg)
    got = oracle.forward(cfg, w, ids)
    explicit = {n: (np.float64(1.0) + a.astype(np.float64)).astype(np.float32) if a.ndim == 1 else a
                for n, a in w.items()}
    ref = oracle.forward(cfg.replace(norm_gain_offset=0), explicit, ids)
    for s in range(cfg.n_layers + 2):
        np.testing.assert_allclose(got["hidden"][s], ref["hidden"][s], rtol=1e-6, atol=1e-6)


def test_gelu_tanh_closed_forms_and_gate():
    z = np.linspace(-8, 8, 3201)
    g = oracle.gelu_tanh(z)
    np.testing.assert_allclose(g - oracle.gelu_tanh(-z), z, atol=1e-12)   # odd part is z / 2
    assert oracle.gelu_tanh(np.array([0.0]))[0] == 0.0
    erf_gelu = 0.5 * z * (1 + np.array([math.erf(v / math.sqrt(2)) for v in z]))
    assert np.abs(g - erf_gelu).max() < 1e-3                            # tanh approximation of GELU
    assert oracle.gelu_tanh(np.array([30.0]))[0] == pytest.approx(30.0)
    # the gated FFN multiplies by the up projection and is not symmetric in (g, u)
    a = oracle.gated_ffn(np.array([1.5], np.float32), np.array([-2.0], np.float32), "gelu_tanh")
    assert a[0] == pytest.approx(float(oracle.gelu_tanh(np.array([1.5]))[0]) * -2.0, rel=1e-6)
    b = oracle.gated_ffn(np.array([-2.0], np.float32), np.array([1.5], np.float32), "gelu_tanh")
    assert abs(a[0] - b[0]) > 0.1


# ---------------------------------------------------------------- mixture of experts
def test_moe_route_brute_force_and_ties():
    z = np.array([[0.5, 2.0, 2.0, -1.0, 0.0], [3.0, 1.0, 1.0, 1.0, 3.0]], np.float32)
    idx, w = oracle.moe_route(z, 3, False)
    assert idx.tolist() == [[1, 2, 0], [0, 4, 1]]               # equal logits: lowest index first
    z64 = z.astype(np.float64)
    p = np.exp(z64 - z64.max(-1, keepdims=True))
    p /= p.sum(-1, keepdims=True)
    np.testing.assert_allclose(w, np.take_along_axis(p, idx.astype(np.int64), -1), rtol=1e-14)
    _, wn = oracle.moe_route(z, 3, True)
    np.testing.assert_allclose(wn.sum(-1), 1.0, rtol=1e-15)
    np.testing.assert_allclose(wn, w / w.sum(-1, keepdims=True), rtol=1e-15)


def _moe_weights(E=4, H=8, Fe=6, seed=5):
    rng = np.random.default_rng(seed)
    f = lambda *s: rng.standard_normal(s).astype(np.float32) * 0.5
    return f(E, H), f(E, Fe, H), f(E, Fe, H), f(E, H, Fe)


def test_moe_identical_experts_reduce_to_the_dense_ffn():
    r, g, u, d = _moe_weights()
    g[:] = g[0]
    u[:] = u[0]
    d[:] = d[0]
    n = np.random.default_rng(1).standard_normal((7, 8)).astype(np.float32)
    dense = oracle.gemm(oracle.swiglu(oracle.gemm(n, g[0]), oracle.gemm(n, u[0])), d[0])
    for k in (1, 2, 4):
        np.testing.assert_allclose(oracle.moe_ffn(n, r, g, u, d, k, True), dense, rtol=1e-5, atol=1e-6)


def test_moe_top1_normalised_is_the_winning_expert_alone():
    r, g, u, d = _moe_weights()
    n = np.random.default_rng(2).standard_normal((9, 8)).astype(np.float32)
    got = oracle.moe_ffn(n, r, g, u, d, 1, True)
    win = np.argmax(oracle.gemm(n, r), -1)
    for t in range(9):
        e = win[t]
        ref = oracle.gemm(oracle.swiglu(oracle.gemm(n[t:t + 1], g[e]), oracle.gemm(n[t:t + 1], u[e])), d[e])
        np.testing.assert_allclose(got[t], ref[0], rtol=1e-5, atol=1e-6)


def test_moe_joint_expert_permutation_invariance():
    r, g, u, d = _moe_weights(E=6)
    n = np.random.default_rng(3).standard_normal((11, 8)).astype(np.float32)
    base = oracle.moe_ffn(n, r, g, u, d, 2, False)
    perm = np.array([3, 0, 5, 1, 4, 2])
    np.testing.assert_allclose(oracle.moe_ffn(n, r[perm], g[perm], u[perm], d[perm], 2, False), base,
                               rtol=1e-5, atol=1e-6)
    # permuting the experts alone (router unchanged) changes the result: the router matters
    assert np.abs(oracle.moe_ffn(n, r, g[perm], u[perm], d[perm], 2, False) - base).max() > 1e-3


def test_forward_moe_layer_with_dense_copies_equals_dense_forward():
    dense = wl.TINY_F32
    moe = dense.replace(n_experts=3, n_experts_per_tok=2, moe_ffn=dense.ffn, ffn_kind=("moe", "dense"),
                        name="tiny-moe")
    w = {n: np.asarray(a, np.float32) for n, a in wl.draw_all(dense).items()}
    wm = dict(w)
    for n in ("w_gate", "w_up", "w_down"):
        del wm["layers.0." + n]
    wm["layers.0.router"] = np.random.default_rng(4).standard_normal((3, dense.hidden)).astype(np.float32)
    wm["layers.0.expert_gate"] = np.stack([w["layers.0.w_gate"]] * 3)
    wm["layers.0.expert_up"] = np.stack([w["layers.0.w_up"]] * 3)
    wm["layers.0.expert_down"] = np.stack([w["layers.0.w_down"]] * 3)
    ids = wl.draw_ids(dense)
    a, b = oracle.forward(dense, w, ids), oracle.forward(moe, wm, ids)
    for s in range(dense.n_layers + 2):
        np.testing.assert_allclose(b["hidden"][s], a["hidden"][s], rtol=1e-5, atol=1e-6)
    assert set(wl.weight_shapes(moe)) == set(wm)                   # the recipe names the same tensors


# ---------------------------------------------------------------- bf16 diagnostic
# The bf16-rounded forward sets the floor that deep bf16 configurations are gated
# against, so its rounding function and every rounding point are pinned here: the
# function against hand-worked round-to-nearest-even bit patterns, the points against
# one rounding (by torch's own bf16 conversion, an independent implementation) of the
# exact value of each point's rounded inputs.

def _bits(x):
    return np.asarray(x, np.float32).view(np.uint32)


def _f(bits):
    return np.asarray(bits, np.uint32).view(np.float32)


# (input bits, expected bf16 bits << 16): worked by hand from the bf16 grid
_RNE_CASES = [
    (0x3F800000, 0x3F800000),  # 1.0 is a bf16 value: unchanged
    (0x3F808000, 0x3F800000),  # 1 + 2^-8, halfway 1.0 / 1 + 2^-7: tie to the even 1.0 (down)
    (0x3F818000, 0x3F820000),  # 1 + 3 * 2^-8, halfway: tie to the even 1 + 2^-6 (up)
    (0x3F808001, 0x3F810000),  # just above halfway: up
    (0x3F807FFF, 0x3F800000),  # just below halfway: down
    (0x3FFF8000, 0x40000000),  # halfway 1.9921875 / 2.0: tie to even carries into the exponent
    (0x3FFFC000, 0x40000000),  # above halfway under the exponent boundary: 2.0
    (0xBF818000, 0xBF820000),  # negative tie: sign kept, magnitude to even
    (0xBF808000, 0xBF800000),
    (0x7F7F0000, 0x7F7F0000),  # the largest bf16 value stays
    (0x7F7F7FFF, 0x7F7F0000),  # below halfway to the next binade: the largest bf16
    (0x7F7FFFFF, 0x7F800000),  # the largest float32 overflows to infinity
    (0xFF7FFFFF, 0xFF800000),
    (0x7F800000, 0x7F800000),  # infinities pass through
    (0xFF800000, 0xFF800000),
    (0x00000000, 0x00000000),  # zeros keep their sign
    (0x80000000, 0x80000000),
    (0x00008000, 0x00000000),  # subnormal tie between 0 and the smallest bf16: even 0
    (0x00018000, 0x00020000),  # subnormal tie between odd 1 and even 2 ulps: up
]


def test_round_bf16_hand_worked_bit_patterns():
    got = _bits(oracle.round_bf16(_f([c[0] for c in _RNE_CASES])))
    want = np.array([c[1] for c in _RNE_CASES], np.uint32)
    bad = [(hex(c[0]), hex(int(g)), hex(c[1])) for c, g in zip(_RNE_CASES, got) if g != c[1]]
    assert not bad, bad


def test_round_bf16_nan_stays_nan_and_agrees_with_torch():
    import torch
    nan = _f([0x7FC00000, 0x7F800001, 0xFF800001, 0x7FBFFFFF])  # quiet, low-payload and signalling NaNs
    assert np.all(np.isnan(oracle.round_bf16(nan)))
    # random finite values over many binades (subnormals included): same bits as torch's conversion
    x = (rng.standard_normal(200000) * np.exp2(rng.integers(-140, 120, 200000))).astype(np.float32)
    x = x[np.isfinite(x)]
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy()
    assert np.array_equal(_bits(oracle.round_bf16(x)), _bits(ref))
    # idempotent, and the result always has zero low bits
    r = oracle.round_bf16(x)
    assert np.array_equal(_bits(oracle.round_bf16(r)), _bits(r))
    assert not np.any(_bits(r) & 0xFFFF)


def test_attention_rounded_equals_attention_when_probabilities_are_bf16_exact():
    # two visible keys with scores 0 and ln 3 give p = (1/4, 3/4), both bf16 values:
    # rounding the probabilities then changes nothing
    D = 4
    q = np.zeros((1, 2, 1, D), np.float32)
    k = np.zeros((1, 2, 1, D), np.float32)
    q[0, 1, 0, 0] = 1.0
    k[0, 1, 0, 0] = np.float32(math.log(3.0) * math.sqrt(D))
    v = rng.standard_normal((1, 2, 1, D)).astype(np.float32)
    p = oracle.attention_probs(q, k)[0, 0, 1]
    assert abs(p[0] - 0.25) < 1e-7 and abs(p[1] - 0.75) < 1e-7
    a = oracle.attention(q, k, v)
    b = oracle.forward_module._attention_rounded(q, k, v, 0)
    # the rounded probabilities are within 1e-7 of 1/4 and 3/4, which round to exactly them
    np.testing.assert_array_equal(b[0, 1, 0], (0.25 * v[0, 0, 0].astype(np.float64)
                                               + 0.75 * v[0, 1, 0].astype(np.float64)).astype(np.float32))
    np.testing.assert_allclose(a, b, rtol=0, atol=2e-7)


def test_attention_rounded_rounds_probabilities_not_the_normaliser():
    # three equal scores: p = 1/3 each; bf16(1/3) = 0x3EAB = 0.333984375, and the output is
    # 0.333984375 * (v0 + v1 + v2) (the rounded weights are not renormalised to sum 1)
    D = 2
    q = np.zeros((1, 3, 1, D), np.float32)
    k = np.zeros((1, 3, 1, D), np.float32)
    v = np.array([1.0, 2.0, 4.0], np.float32).reshape(1, 3, 1, 1) * np.ones((1, 1, 1, D), np.float32)
    o = oracle.forward_module._attention_rounded(q, k, v, 0)
    assert o[0, 2, 0, 0] == np.float32(0.333984375 * 7.0)
    assert o[0, 1, 0, 0] == np.float32(0.5 * 3.0)     # two keys: 1/2 is exact
    assert o[0, 0, 0, 0] == np.float32(1.0)           # one key: weight 1


def _rne_torch(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(torch.bfloat16).to(torch.float32).numpy()


_POINT_CFG = wl.TINY_F32.replace(n_layers=2, seq=11, batch=2)


def _check_bf16_points(cfg, seed=7):
    """Every rounding point of the diagnostic is one round-to-nearest-even of the exact
    value of that point computed from the previous points' rounded tensors; the
    unrounded tensors (residual, slots, logits) are not on the bf16 grid. Raises
    AssertionError naming the first point that fails."""
    w = wl.LazyWeights(cfg, seed=seed, cache=True)
    ids = wl.draw_ids(cfg)
    tr = {}
    out = oracle.forward(cfg, w, ids, bf16_points=True, trace=tr)
    B, S = ids.shape
    H, Hq, Hkv, D = cfg.hidden, cfg.n_heads, cfg.n_kv_heads, cfg.head_dim
    eps = cfg.rms_eps
    pos = np.arange(S)

    def same(point, got, want):
        assert np.array_equal(_bits(got), _bits(want)), f"point {point}: not one rounding of the exact value"
        assert not np.any(_bits(got) & 0xFFFF), f"point {point}: not on the bf16 grid"

    x = out["hidden"][0]
    for l in range(cfg.n_layers):
        p = f"layers.{l}."
        g = lambda n: tr[f"bf16.{l}.{n}"]  # noqa: E731
        same(f"{l}.n_attn", g("n_attn"), _rne_torch(oracle.rmsnorm(x, w[p + "attn_norm"], eps)))
        n = g("n_attn")
        same(f"{l}.v", g("v"), _rne_torch(oracle.gemm(n, w[p + "wv"]).reshape(B, S, Hkv, D)))
        f, m = oracle.rope_frequencies(cfg, cfg.kinds()[l], S)
        qp = oracle.gemm(n, w[p + "wq"]).reshape(B, S, Hq, D)
        kp = oracle.gemm(n, w[p + "wk"]).reshape(B, S, Hkv, D)
        same(f"{l}.q", g("q"), _rne_torch(np.stack([oracle.rotate(qp[b], pos, f, m) for b in range(B)])))
        same(f"{l}.k", g("k"), _rne_torch(np.stack([oracle.rotate(kp[b], pos, f, m) for b in range(B)])))
        # o: the exact probabilities of the rounded q, k, rounded once, times the rounded v
        # (float64 sum, one float32 rounding), then rounded to bf16
        window = cfg.sliding_window if cfg.kinds()[l] == "local" else 0
        P = oracle.attention_probs(g("q"), g("k"), window)
        o = np.empty((B, S, Hq, D), np.float32)
        for b in range(B):
            for h in range(Hq):
                pr = _rne_torch(P[b, h].astype(np.float32)).astype(np.float64)
                o[b, :, h, :] = (pr @ g("v")[b, :, h // (Hq // Hkv), :].astype(np.float64)).astype(np.float32)
        same(f"{l}.o", g("o"), _rne_torch(o))
        u = oracle.gemm(g("o").reshape(B, S, Hq * D), w[p + "wo"])
        if cfg.norm_placement == "sandwich":  # the post-norm works on the fp32 product: no rounding point
            u = oracle.rmsnorm(u, w[p + "post_attn_norm"], eps)
        xa = (x.astype(np.float64) + u).astype(np.float32)
        assert np.array_equal(_bits(g("x_attn")), _bits(xa)), f"{l}.x_attn"
        assert np.any(_bits(xa) & 0xFFFF), f"{l}.x_attn should stay unrounded"
        same(f"{l}.n_ffn", g("n_ffn"), _rne_torch(oracle.rmsnorm(xa, w[p + "ffn_norm"], eps)))
        a = oracle.swiglu(oracle.gemm(g("n_ffn"), w[p + "w_gate"]), oracle.gemm(g("n_ffn"), w[p + "w_up"]))
        same(f"{l}.a", g("a"), _rne_torch(a))
        d = oracle.gemm(g("a"), w[p + "w_down"])
        if cfg.norm_placement == "sandwich":
            d = oracle.rmsnorm(d, w[p + "post_ffn_norm"], eps)
        x = (xa.astype(np.float64) + d).astype(np.float32)
        assert np.array_equal(_bits(out["hidden"][l + 1]), _bits(x)), f"slot {l + 1}"
        assert np.any(_bits(x) & 0xFFFF), f"slot {l + 1} should stay unrounded"
    hfin = out["hidden"][cfg.n_layers + 1]
    assert np.any(_bits(hfin) & 0xFFFF), "the final-norm slot stays unrounded"
    same("h", tr["bf16.h"], _rne_torch(hfin))
    z = oracle.softcap(oracle.gemm(tr["bf16.h"], w["embed"]), cfg.final_logit_softcap)
    assert np.array_equal(_bits(out["logits"]), _bits(z)), "logits from the rounded final norm"


# the same points on the sandwich / window / softcap / scaled-embedding path
_POINT_CFG_SANDWICH = _POINT_CFG.replace(norm_placement="sandwich", sliding_window=4,
                                         layer_kind=("local", "global"), final_logit_softcap=2.0,
                                         embed_scale_mode="bf16_sqrt_hidden")


@pytest.mark.parametrize("cfg", [_POINT_CFG, _POINT_CFG_SANDWICH], ids=["pre", "sandwich"])
def test_bf16_points_are_single_roundings_of_exact_values(cfg):
    _check_bf16_points(cfg)


def test_bf16_points_pin_fails_on_planted_rounding_mistakes(monkeypatch):
    """Each planted mistake in the diagnostic (a dropped point, a truncating rounding,
    unrounded probabilities, an extra rounding of the residual) fails the point pin."""
    fm = oracle.forward_module
    real_point, real_round, real_attn = fm._bf16_point, fm.round_bf16, fm._attention_rounded

    def dropped(name):
        def f(a, point, trace):
            r = np.asarray(a, np.float32) if point.endswith(name) else real_round(a)
            if trace is not None:
                trace["bf16." + point] = r
            return r
        return f

    def truncate(a):
        u = np.asarray(a, np.float32).view(np.uint32)
        return (u & 0xFFFF0000).view(np.float32)

    plants = [(n, "_bf16_point", dropped(n)) for n in ("n_attn", ".v", ".q", ".k", ".o", "n_ffn", ".a", "h")]
    plants += [("truncate", "round_bf16", truncate), ("exact p", "_attention_rounded",
                                                     lambda q, k, v, window: oracle.attention(q, k, v, window))]
    for label, attr, fn in plants:
        monkeypatch.setattr(fm, attr, fn)
        with pytest.raises(AssertionError):
            _check_bf16_points(_POINT_CFG)
        monkeypatch.setattr(fm, "_bf16_point", real_point)
        monkeypatch.setattr(fm, "round_bf16", real_round)
        monkeypatch.setattr(fm, "_attention_rounded", real_attn)
    # an extra rounding of the residual stream
    real_f32 = fm._f32
    monkeypatch.setattr(fm, "_f32", lambda a: real_round(real_f32(a)))
    with pytest.raises(AssertionError):
        _check_bf16_points(_POINT_CFG)
    monkeypatch.setattr(fm, "_f32", real_f32)
    _check_bf16_points(_POINT_CFG)  # and the real diagnostic passes again


# ---------------------------------------------------------------- longrope / llama3 closed forms
def _longrope_cfg(s, L0=64):
    D = wl.TINY_F32.head_dim
    return wl.TINY_F32.replace(rope_scaling="longrope", rope_factor=float(s), rope_original_max_pos=L0,
                               rope_short_factor=(1.0,) * (D // 2), rope_long_factor=(2.0,) * (D // 2))


@pytest.mark.parametrize("L0", [64, 4096])
def test_longrope_multiplier_special_cases(L0):
    # sqrt(1 + ln s / ln L0): s = L0 gives sqrt 2, s = L0^2 gives sqrt 3, no extension gives 1
    _, m = oracle.rope_frequencies(_longrope_cfg(L0, L0), "global", 8)
    assert m == pytest.approx(math.sqrt(2.0), rel=1e-14)
    _, m = oracle.rope_frequencies(_longrope_cfg(L0 * L0, L0), "global", 8)
    assert m == pytest.approx(math.sqrt(3.0), rel=1e-14)
    for s in (1.0, 0.5):
        _, m = oracle.rope_frequencies(_longrope_cfg(s, L0), "global", 8)
        assert m == 1.0
    # the multiplier grows with the extension and does not depend on the sequence length
    _, a = oracle.rope_frequencies(_longrope_cfg(8.0, L0), "global", 8)
    _, b = oracle.rope_frequencies(_longrope_cfg(8.0, L0), "global", L0 + 5)
    _, c = oracle.rope_frequencies(_longrope_cfg(16.0, L0), "global", 8)
    assert a == b and 1.0 < a < c


def test_longrope_multiplier_pin_fails_on_planted_mistakes(monkeypatch):
    # a multiplier with the logarithms swapped or a missing square root fails the special cases
    real = oracle.forward_module.rope_frequencies

    def planted(variant):
        def f(cfg, kind, seq_len):
            inv, m = real(cfg, kind, seq_len)
            s, L0 = cfg.rope_factor, cfg.rope_original_max_pos
            if s <= 1.0:
                return inv, m
            if variant == "swapped":
                return inv, math.sqrt(1.0 + math.log(L0) / math.log(s))
            return inv, 1.0 + math.log(s) / math.log(L0)
        return f

    for variant in ("swapped", "no_sqrt"):
        monkeypatch.setattr(oracle, "rope_frequencies", planted(variant))
        with pytest.raises(AssertionError):
            test_longrope_multiplier_special_cases(64)
        monkeypatch.setattr(oracle, "rope_frequencies", real)


def test_llama3_band_interior_hand_worked():
    # place the original context so that a chosen pair sits a quarter and a half of the
    # way through the blended band: L0 / wavelength = lo + t (hi - lo) gives
    # f' = (1 - t) f / s + t f, i.e. f (0.75 / s + 0.25) and f (0.5 / s + 0.5)
    D, s, lo, hi = 128, 8.0, 1.0, 4.0
    plain = 500000.0 ** (-2.0 * np.arange(D // 2) / D)
    k = 40
    wavelen = 2 * math.pi / plain[k]
    for t, factor in ((0.25, 0.75 / s + 0.25), (0.5, 0.5 / s + 0.5), (0.75, 0.25 / s + 0.75)):
        L0 = wavelen * (lo + t * (hi - lo))
        f, _ = oracle.rope_frequencies(_llama3_cfg(rope_original_max_pos=L0, rope_factor=s), "global", 16)
        assert f[k] == pytest.approx(plain[k] * factor, rel=1e-12)
