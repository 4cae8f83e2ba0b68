"""Pins of the oracle's whole forward against an independent implementation of the same
published architectures: the decoder model classes of the `transformers` library.

Each HF model is built locally from a config (nothing is downloaded), given the
oracle's own synthetic weights, and run on the CPU in float64 with eager attention.
HF keeps a few float32 islands inside that (RoPE angles, its RMSNorm, the attention
softmax, the router softmax), and the oracle rounds each op's output to float32, so
the two agree to within 1e-6 of scale; the gate is 2e-6. The families are the axes
"N7 · model/forward-parity" (Theorem statement) names: llama (plain and with llama3
frequency bands), qwen3 (QK-norm), gemma3 (sandwich norms, (1 + w) gains, tanh-GELU
gating, QK-norm, local/global layers with their own RoPE bases and a sliding window,
scaled embedding, final-logit softcap), phi3 (longrope, both factor sets) and
qwen3moe (hybrid dense / sparse layers, softmax router, top-k, renormalised weights).

Every case also checks that the pin has teeth: the oracle with that case's feature
switched off (or mis-set) misses HF by far more than the gate.

Slots: HF returns the embedding output, the output of every layer but the last, and
the final norm's output; the last layer's own output (the oracle's slot L) is taken by
a forward hook, so every one of the L + 2 slots is compared.
"""
import numpy as np
import pytest

import oracle
from synth import workloads as wl

TOL = 2e-6          # err/scale gate for slots and logits (observed 1.6e-7 .. 6.8e-7)
TEETH = 500 * TOL    # a switched-off feature must miss by at least this much


@pytest.fixture(scope="module")
def hf():
    torch = pytest.importorskip("torch")
    transformers = pytest.importorskip("transformers")
    transformers.logging.set_verbosity_error()
    return torch, transformers


def _weights(cfg):
    """The synthetic weights, with Wq and Wk ten times larger: at N(0, 0.02^2) the
    scores of a tiny model are nearly flat and RoPE would barely show."""
    w = {n: np.asarray(a, np.float32) for n, a in wl.draw_all(cfg).items()}
    for n in w:
        if n.endswith(".wq") or n.endswith(".wk"):
            w[n] = w[n] * np.float32(10.0)
    return w


def _build(hf, cls_name, cfg_name, state, **kw):
    torch, tr = hf
    config = getattr(tr, cfg_name)(pad_token_id=None, bos_token_id=None, eos_token_id=None, tie_word_embeddings=True,
                                   attn_implementation="eager", **kw)
    model = getattr(tr, cls_name)(config).to(torch.float64).eval()
    params = dict(model.named_parameters())
    for name, arr in state.items():
        p = params[name]
        assert tuple(p.shape) == arr.shape, (name, tuple(p.shape), arr.shape)
        with torch.no_grad():
            p.copy_(torch.from_numpy(np.asarray(arr, np.float64)))
    missing = {n for n in params if n not in state and n != "lm_head.weight"}
    assert not missing, missing                                    # every parameter set
    assert model.lm_head.weight.data_ptr() == model.model.embed_tokens.weight.data_ptr()  # tied head
    return model


def _run(hf, model, ids):
    """(logits, slots): the embedding output, every layer's output (the last one taken
    by a hook on the last decoder layer) and the final norm's output."""
    torch, _ = hf
    last = []
    hook = model.model.layers[-1].register_forward_hook(
        lambda mod, inp, out: last.append((out[0] if isinstance(out, tuple) else out).detach().clone()))
    try:
        with torch.no_grad():
            out = model(input_ids=torch.from_numpy(np.asarray(ids, np.int64)), output_hidden_states=True)
    finally:
        hook.remove()
    hs = [h.numpy() for h in out.hidden_states]
    assert len(last) == 1 and len(hs) == len(model.model.layers) + 1
    return out.logits.numpy(), hs[:-1] + [last[0].numpy(), hs[-1]]


def _err(a, ref):
    ref = np.asarray(ref, np.float64)
    return float(np.max(np.abs(np.asarray(a, np.float64) - ref)) / np.max(np.abs(ref)))


def _compare(cfg, w, ids, logits, hidden):
    """Largest err/scale of the oracle against HF over the shared slots and the logits."""
    o = oracle.forward(cfg, w, ids)
    assert len(hidden) == cfg.n_layers + 2
    errs = [_err(o["hidden"][s], hidden[s]) for s in range(cfg.n_layers + 2)]
    errs.append(_err(o["logits"], logits))
    return max(errs), o


def _llama_state(cfg, w):
    s = {"model.embed_tokens.weight": w["embed"], "model.norm.weight": w["final_norm"]}
    for l in range(cfg.n_layers):
        p, q = f"layers.{l}.", f"model.layers.{l}."
        s.update({q + "input_layernorm.weight": w[p + "attn_norm"],
                  q + "self_attn.q_proj.weight": w[p + "wq"], q + "self_attn.k_proj.weight": w[p + "wk"],
                  q + "self_attn.v_proj.weight": w[p + "wv"], q + "self_attn.o_proj.weight": w[p + "wo"],
                  q + "post_attention_layernorm.weight": w[p + "ffn_norm"]})
        if p + "w_gate" in w:
            s.update({q + "mlp.gate_proj.weight": w[p + "w_gate"], q + "mlp.up_proj.weight": w[p + "w_up"],
                      q + "mlp.down_proj.weight": w[p + "w_down"]})
        if cfg.qk_norm:
            s.update({q + "self_attn.q_norm.weight": w[p + "q_norm"], q + "self_attn.k_norm.weight": w[p + "k_norm"]})
    return s


def _geometry(cfg):
    return dict(vocab_size=cfg.vocab, hidden_size=cfg.hidden, intermediate_size=cfg.ffn,
                num_hidden_layers=cfg.n_layers, num_attention_heads=cfg.n_heads,
                num_key_value_heads=cfg.n_kv_heads, rms_norm_eps=cfg.rms_eps, max_position_embeddings=4096)


# A tiny llama-family geometry with spread gains (so that a dropped gain or a swapped
# norm cannot pass), in float32 so that the oracle and HF read identical weights.
BASE = wl.TINY_F32.replace(gain_sigma=0.3, batch=2, seq=16)


def test_llama_pre_norm_swiglu_gqa(hf):
    cfg = BASE
    w = _weights(cfg)
    ids = wl.draw_ids(cfg)
    model = _build(hf, "LlamaForCausalLM", "LlamaConfig", _llama_state(cfg, w), **_geometry(cfg),
                   head_dim=cfg.head_dim, hidden_act="silu",
                   rope_parameters={"rope_type": "default", "rope_theta": cfg.rope_theta})
    logits, hidden = _run(hf, model, ids)
    err, o = _compare(cfg, w, ids, logits, hidden)
    assert err < TOL, err
    assert np.array_equal(o["argmax"], np.argmax(logits, axis=-1))
    # teeth: another RoPE base, and gains left out, both miss by far more than the gate
    assert _compare(cfg.replace(rope_theta=500.0), w, ids, logits, hidden)[0] > TEETH
    w1 = dict(w, final_norm=np.ones_like(w["final_norm"]))
    assert _compare(cfg, w1, ids, logits, hidden)[0] > TEETH


def test_llama3_frequency_bands(hf):
    # head_dim 16, theta 1e4: wavelengths 6.3 .. 19869 tokens; with L0 = 256 and factors
    # (1, 4) pairs 0-2 keep their frequency, pair 3 (wavelength 199) is blended and
    # pairs 4-7 are divided by the factor, so all three bands are exercised
    cfg = BASE.replace(rope_scaling="llama3", rope_factor=8.0, rope_low_freq_factor=1.0, rope_high_freq_factor=4.0,
                       rope_original_max_pos=256, seq=24)
    w = _weights(cfg)
    ids = wl.draw_ids(cfg)
    model = _build(hf, "LlamaForCausalLM", "LlamaConfig", _llama_state(cfg, w), **_geometry(cfg),
                   head_dim=cfg.head_dim, hidden_act="silu",
                   rope_parameters={"rope_type": "llama3", "rope_theta": cfg.rope_theta, "factor": 8.0,
                                    "low_freq_factor": 1.0, "high_freq_factor": 4.0,
                                    "original_max_position_embeddings": 256})
    logits, hidden = _run(hf, model, ids)
    assert _compare(cfg, w, ids, logits, hidden)[0] < TOL
    assert _compare(cfg.replace(rope_scaling="none"), w, ids, logits, hidden)[0] > TEETH
    # the blended band alone: a mid-band that takes f / s instead of the blend misses too
    assert _compare(cfg.replace(rope_high_freq_factor=1.0 + 1e-9), w, ids, logits, hidden)[0] > TEETH


def test_qwen3_qk_norm(hf):
    cfg = BASE.replace(qk_norm=True)
    w = _weights(cfg)
    ids = wl.draw_ids(cfg)
    model = _build(hf, "Qwen3ForCausalLM", "Qwen3Config", _llama_state(cfg, w), **_geometry(cfg),
                   head_dim=cfg.head_dim, hidden_act="silu", use_sliding_window=False,
                   rope_parameters={"rope_type": "default", "rope_theta": cfg.rope_theta})
    logits, hidden = _run(hf, model, ids)
    assert _compare(cfg, w, ids, logits, hidden)[0] < TOL
    assert _compare(cfg.replace(qk_norm=False), w, ids, logits, hidden)[0] > TEETH


def _gemma3_state(cfg, w):
    s = {"model.embed_tokens.weight": w["embed"], "model.norm.weight": w["final_norm"]}
    for l in range(cfg.n_layers):
        p, q = f"layers.{l}.", f"model.layers.{l}."
        s.update({q + "input_layernorm.weight": w[p + "attn_norm"],
                  q + "post_attention_layernorm.weight": w[p + "post_attn_norm"],
                  q + "pre_feedforward_layernorm.weight": w[p + "ffn_norm"],
                  q + "post_feedforward_layernorm.weight": w[p + "post_ffn_norm"],
                  q + "self_attn.q_proj.weight": w[p + "wq"], q + "self_attn.k_proj.weight": w[p + "wk"],
                  q + "self_attn.v_proj.weight": w[p + "wv"], q + "self_attn.o_proj.weight": w[p + "wo"],
                  q + "self_attn.q_norm.weight": w[p + "q_norm"], q + "self_attn.k_norm.weight": w[p + "k_norm"],
                  q + "mlp.gate_proj.weight": w[p + "w_gate"], q + "mlp.up_proj.weight": w[p + "w_up"],
                  q + "mlp.down_proj.weight": w[p + "w_down"]})
    return s


def test_gemma3_sandwich_local_global_window_softcap(hf):
    # six layers: five local (window 4, RoPE base 1e4) then one global (base 1e6), over
    # 16 tokens so that the window evicts; hidden 64 makes the scaled embedding's bf16
    # rounding of sqrt(64) exact, as in HF's float64 model
    cfg = BASE.replace(n_layers=6, layer_kind=wl._gemma_layer_map(6), sliding_window=4, rope_theta=1e6,
                       rope_theta_local=1e4, norm_placement="sandwich", qk_norm=True, norm_gain_offset=1,
                       ffn_act="gelu_tanh", embed_scale_mode="bf16_sqrt_hidden", final_logit_softcap=0.5)
    w = _weights(cfg)
    ids = wl.draw_ids(cfg)
    model = _build(hf, "Gemma3ForCausalLM", "Gemma3TextConfig", _gemma3_state(cfg, w), **_geometry(cfg),
                   head_dim=cfg.head_dim, hidden_activation="gelu_pytorch_tanh", query_pre_attn_scalar=cfg.head_dim,
                   sliding_window=4, layer_types=["sliding_attention" if k == "local" else "full_attention"
                                                  for k in cfg.kinds()],
                   final_logit_softcapping=0.5, attn_logit_softcapping=None,
                   rope_parameters={"sliding_attention": {"rope_type": "default", "rope_theta": 1e4},
                                    "full_attention": {"rope_type": "default", "rope_theta": 1e6}})
    logits, hidden = _run(hf, model, ids)
    assert _compare(cfg, w, ids, logits, hidden)[0] < TOL
    for wrong in (dict(rope_theta_local=0.0), dict(sliding_window=0), dict(norm_gain_offset=0),
                  dict(ffn_act="silu"), dict(final_logit_softcap=0.0), dict(embed_scale_mode="none"),
                  dict(layer_kind=("local",) * 6)):
        assert _compare(cfg.replace(**wrong), w, ids, logits, hidden)[0] > TEETH, wrong


def _phi3_state(cfg, w):
    s = {"model.embed_tokens.weight": w["embed"], "model.norm.weight": w["final_norm"]}
    for l in range(cfg.n_layers):
        p, q = f"layers.{l}.", f"model.layers.{l}."
        s.update({q + "input_layernorm.weight": w[p + "attn_norm"],
                  q + "post_attention_layernorm.weight": w[p + "ffn_norm"],
                  q + "self_attn.qkv_proj.weight": np.concatenate([w[p + "wq"], w[p + "wk"], w[p + "wv"]]),
                  q + "self_attn.o_proj.weight": w[p + "wo"],
                  q + "mlp.gate_up_proj.weight": np.concatenate([w[p + "w_gate"], w[p + "w_up"]]),
                  q + "mlp.down_proj.weight": w[p + "w_down"]})
    return s


@pytest.mark.parametrize("seq", [6, 12])
def test_phi3_longrope_short_and_long_factors(hf, seq):
    # original context 8, factor 4: 6 tokens take the short factors, 12 the long ones;
    # cos and sin carry sqrt(1 + ln 4 / ln 8) either way
    L0, s = 8, 4.0
    short = tuple(1.0 + 0.07 * k for k in range(8))
    long = tuple(1.0 + 0.9 * k for k in range(8))
    cfg = BASE.replace(rope_scaling="longrope", rope_factor=s, rope_original_max_pos=L0, rope_short_factor=short,
                       rope_long_factor=long, seq=seq)
    w = _weights(cfg)
    ids = wl.draw_ids(cfg)
    geo = dict(_geometry(cfg), max_position_embeddings=int(s * L0))
    model = _build(hf, "Phi3ForCausalLM", "Phi3Config", _phi3_state(cfg, w), **geo, hidden_act="silu",
                   original_max_position_embeddings=L0,
                   rope_parameters={"rope_type": "longrope", "rope_theta": cfg.rope_theta, "short_factor": list(short),
                                    "long_factor": list(long), "original_max_position_embeddings": L0})
    logits, hidden = _run(hf, model, ids)
    assert _compare(cfg, w, ids, logits, hidden)[0] < TOL
    # the other factor set, and the multiplier left out, both miss
    other = dict(rope_short_factor=long) if seq <= L0 else dict(rope_long_factor=short)
    assert _compare(cfg.replace(**other), w, ids, logits, hidden)[0] > TEETH
    assert _compare(cfg.replace(rope_factor=1.0), w, ids, logits, hidden)[0] > TEETH


def _qwen3moe_state(cfg, w):
    s = _llama_state(cfg, w)
    for l, kind in enumerate(cfg.ffn_kinds()):
        if kind != "moe":
            continue
        p, q = f"layers.{l}.", f"model.layers.{l}."
        s.update({q + "mlp.gate.weight": w[p + "router"],
                  q + "mlp.experts.gate_up_proj": np.concatenate([w[p + "expert_gate"], w[p + "expert_up"]], axis=1),
                  q + "mlp.experts.down_proj": w[p + "expert_down"]})
    return s


@pytest.mark.parametrize("k,norm", [(2, True), (2, False), (1, True), (3, False)])
def test_qwen3moe_hybrid_dense_sparse(hf, k, norm):
    # layers 0 and 2 sparse (5 experts of width 48), layer 1 dense; router spread 0.1 so
    # that routing differs between tokens
    cfg = BASE.replace(n_layers=3, qk_norm=True, n_experts=5, n_experts_per_tok=k, moe_ffn=48, moe_norm_topk=norm,
                       ffn_kind=("moe", "dense", "moe"), router_sigma=0.1)
    w = _weights(cfg)
    ids = wl.draw_ids(cfg)
    model = _build(hf, "Qwen3MoeForCausalLM", "Qwen3MoeConfig", _qwen3moe_state(cfg, w), **_geometry(cfg),
                   head_dim=cfg.head_dim, hidden_act="silu", use_sliding_window=False, moe_intermediate_size=48,
                   num_experts=5, num_experts_per_tok=k, norm_topk_prob=norm, decoder_sparse_step=1,
                   mlp_only_layers=[1], rope_parameters={"rope_type": "default", "rope_theta": cfg.rope_theta},
                   experts_implementation="eager")
    logits, hidden = _run(hf, model, ids)
    trace = {}
    oracle.forward(cfg, w, ids, trace=trace)
    z = np.sort(trace["moe_logits.0"], axis=-1)[:, ::-1]
    assert np.min(z[:, k - 1] - z[:, k]) > 1e-4        # no near tie: both sides route alike
    assert _compare(cfg, w, ids, logits, hidden)[0] < TOL
    if k > 1:
        assert _compare(cfg.replace(moe_norm_topk=not norm), w, ids, logits, hidden)[0] > TEETH
    assert _compare(cfg.replace(n_experts_per_tok=k + 1), w, ids, logits, hidden)[0] > TEETH


def test_greedy_matches_hf_generate(hf):
    """The oracle's greedy continuation (repeated cacheless forwards) against HF's
    greedy generate, which runs through HF's own key/value cache."""
    torch, _ = hf
    cfg = BASE.replace(seq=8)
    # value, output and FFN matrices 10x larger: at N(0, 0.02^2) the embedding dominates
    # the residual stream and every row would just repeat its last token
    w = {n: a * np.float32(10.0) if n.rsplit(".", 1)[-1] in ("wv", "wo", "w_gate", "w_up", "w_down") else a
         for n, a in _weights(cfg).items()}
    ids = wl.draw_ids(cfg)
    model = _build(hf, "LlamaForCausalLM", "LlamaConfig", _llama_state(cfg, w), **_geometry(cfg),
                   head_dim=cfg.head_dim, hidden_act="silu",
                   rope_parameters={"rope_type": "default", "rope_theta": cfg.rope_theta})
    toks, logits = oracle.greedy(cfg, w, ids, 6)
    top2 = np.sort(logits, axis=-1)[..., -2:]
    assert np.min(top2[..., 1] - top2[..., 0]) > 1e-4            # no near tie at any step
    assert len(np.unique(toks)) > 6                              # a continuation, not a repeated token
    with torch.no_grad():
        out = model.generate(torch.from_numpy(np.asarray(ids, np.int64)), max_new_tokens=6, do_sample=False,
                             pad_token_id=0, eos_token_id=None)
    assert np.array_equal(out[:, ids.shape[1]:].numpy(), toks)


def test_llama_family_at_the_smollm2_shape(hf):
    """The SmolLM2-135M-shaped config itself (30 layers, hidden 576, 9 / 3 heads of 64,
    FFN 1536, vocab 49152), with its own bf16 synthetic weights widened to float32 as
    the oracle reads them, over 1 x 24 tokens."""
    cfg = wl.SMOLLM2_135M.replace(seq=24)
    w = {n: np.asarray(wl.bf16_bits_to_f32(a) if a.dtype == np.uint16 else a, np.float32)
         for n, a in wl.draw_all(cfg).items()}
    ids = wl.draw_ids(cfg)
    model = _build(hf, "LlamaForCausalLM", "LlamaConfig", _llama_state(cfg, w), **_geometry(cfg),
                   head_dim=cfg.head_dim, hidden_act="silu",
                   rope_parameters={"rope_type": "default", "rope_theta": cfg.rope_theta})
    logits, hidden = _run(hf, model, ids)
    err, o = _compare(cfg, w, ids, logits, hidden)
    assert err < TOL, err
    assert np.array_equal(o["argmax"], np.argmax(logits, axis=-1))
