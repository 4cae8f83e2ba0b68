"""Architecture variants against the oracle ("N7 · model/forward-parity", Theorem
statement: the forward must hold across the families' axes — qwen3 QK-norm, gemma3
local/global attention with sandwich norms, llama3 rope scaling, phi3 longrope).

Each model has two layers and non-neutral norm gains (gain_sigma), so a gain that is
dropped, or applied without its offset, changes the result. The gates are those of
the plain forward ([fp] Theorem 1): hidden-slot cosine >= 0.9999 at every slot,
argmax exact where pinned (near-tie rule), and on the fp32 model logits within 0.05.
"""
import json
import os
import sys

import numpy as np
import pytest

import oracle
from synth import workloads as wl
from tests.gpu_util import argmax_check, band_for, cosine, logit_band_check, upload_weights

pytestmark = pytest.mark.gpu
GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page_values.json")))
COS_MIN = GOLD["hidden_cosine_min"]["value"]
LOGIT_MAX = GOLD["final_logits_max_abs"]["value"]
STEP_COS = GOLD["metal_forward_cosine_min"]["value"]

SMALL = dict(n_layers=2, hidden=512, ffn=1024, vocab=2048, gain_sigma=0.2)
QWEN3 = wl.SMOLLM2_135M.replace(qk_norm=True, name="qwen3-like-2L", **SMALL)
GEMMA3 = wl.GEMMA3_STYLE.replace(n_heads=4, n_kv_heads=2, head_dim=256, sliding_window=16,
                                 layer_kind=("local", "global"), qk_norm=True, norm_gain_offset=1,
                                 ffn_act="gelu_tanh", rope_theta=1e6, rope_theta_local=1e4,
                                 name="gemma3-like-2L", **SMALL)
LLAMA3_SCALED = wl.LLAMA3_8B.replace(n_heads=8, n_kv_heads=2, qk_norm=True, rope_scaling="llama3", rope_factor=8.0,
                                     rope_low_freq_factor=1.0, rope_high_freq_factor=4.0, rope_original_max_pos=64,
                                     name="llama3-scaled-2L", **SMALL)
_rng = np.random.default_rng(11)
LONGROPE = wl.SMOLLM2_135M.replace(rope_scaling="longrope", rope_factor=4.0, rope_original_max_pos=32,
                                   rope_short_factor=tuple(float(v) for v in _rng.uniform(1.0, 2.0, 32)),
                                   rope_long_factor=tuple(float(v) for v in _rng.uniform(2.0, 8.0, 32)),
                                   name="longrope-2L", **SMALL)
TINY_ALL = wl.TINY_F32.replace(qk_norm=True, norm_gain_offset=1, ffn_act="gelu_tanh", rope_theta_local=500.0,
                               sliding_window=4, layer_kind=("local", "global"), rope_scaling="llama3",
                               rope_factor=4.0, rope_original_max_pos=8, gain_sigma=0.2, name="tiny-f32-variants")


@pytest.fixture(scope="module")
def fwd():
    import torch
    from decoder_only_transformer_bf16_amd import fwd as F
    assert torch.cuda.is_available(), "GPU tests need a visible GPU"
    torch.cuda.set_device(0)
    assert F.available(), "libfwd.so sees no gfx950 device"
    return F


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _parity(fwd, cfg, ids, logit_gate=None, model=None, host=None):
    host = host if host is not None else wl.draw_all(cfg)
    own = model is None
    if own:
        model = fwd.Model(cfg, upload_weights(cfg, host), max_tokens=max(ids.size, 64))
    out = model.prefill(ids, logits=True, hidden=True, argmax=True)
    got = {k: v.cpu().numpy() for k, v in out.items()}
    ref = oracle.forward(cfg, wl.HostWeights(host), ids)
    worst = min(cosine(got["hidden"][s], ref["hidden"][s]) for s in range(cfg.n_layers + 2))
    for s in range(cfg.n_layers + 2):
        c = cosine(got["hidden"][s], ref["hidden"][s])
        assert c >= COS_MIN, f"{cfg.name} {ids.shape}: slot {s} cosine {c}"
    dz = float(np.max(np.abs(got["logits"] - ref["logits"])))
    if logit_gate is not None:
        assert dz <= logit_gate, dz
    band = band_for(cfg, wl.HostWeights(host), ids, ref["logits"])
    pinned, near, fails = argmax_check(got["argmax"], ref["logits"], band)
    assert not fails, fails[:5]
    d, b = logit_band_check(got["logits"], ref["logits"], band)
    assert d <= b, f"max|dlogit| {d} over the oracle-side allowance {b}"
    _say(f"  {cfg.name} {ids.shape}: lowest slot cosine {worst:.7f}, max|dlogit| {dz:.3e} (allowance {b:.3e}), "
         f"argmax pinned {pinned} near-tie {near}")
    if own:
        model.close()
    return got, ref


@pytest.mark.parametrize("cfg", [QWEN3, GEMMA3, LLAMA3_SCALED], ids=lambda c: c.name)
def test_bf16_variant_prefill_matches_oracle(fwd, cfg):
    """96 rows (tiled kernels) and 12 rows (the few-row kernel)."""
    host = wl.draw_all(cfg)
    model = fwd.Model(cfg, upload_weights(cfg, host), max_tokens=96)
    ids = np.asarray(wl.draw_ids(cfg, batch=2, seq=48))
    _parity(fwd, cfg, ids, model=model, host=host)
    _parity(fwd, cfg, ids[:1, :12], model=model, host=host)
    model.close()


def test_longrope_short_and_long_factor_sets(fwd):
    """Calls up to 32 tokens use the short factors, longer ones the long factors (and
    both carry the cos/sin multiplier of factor 4)."""
    cfg = LONGROPE
    host = wl.draw_all(cfg)
    model = fwd.Model(cfg, upload_weights(cfg, host), max_tokens=96)
    ids = np.asarray(wl.draw_ids(cfg, batch=2, seq=48))
    _, short = _parity(fwd, cfg, ids[:, :32], model=model, host=host)
    _, long = _parity(fwd, cfg, ids, model=model, host=host)
    # the factor set matters: position 31's logits differ between the 32- and 48-token calls
    assert np.abs(short["logits"][:, 31] - long["logits"][:, 31]).max() > 1e-3
    model.close()


def test_f32_all_variants(fwd):
    cfg = TINY_ALL
    _parity(fwd, cfg, np.asarray(wl.draw_ids(cfg)), logit_gate=LOGIT_MAX)


@pytest.mark.parametrize("cfg", [QWEN3, GEMMA3, LLAMA3_SCALED], ids=lambda c: c.name)
def test_qk_norm_cached_decode(fwd, cfg):
    """Cached session with QK-norm: the normalising pass also fills the cache. Every
    step against the oracle's cacheless forward over the same sequence ([mg] Theorem 1:
    cosine >= 0.999 and argmax parity at every prefill and greedy step), and against the
    library's own cacheless prefill."""
    host = wl.draw_all(cfg)
    model = fwd.Model(cfg, upload_weights(cfg, host), max_tokens=64)
    prompt = np.asarray(wl.draw_ids(cfg, batch=2, seq=20))
    sess = fwd.Session(model, max_batch=2, max_seq=32)
    out = sess.prefill(prompt, logits=True, argmax=True)
    seq = prompt
    tok = out["argmax"][:, -1].cpu().numpy()
    w = wl.HostWeights(host)
    for step in range(4):
        z = out["logits"][:, -1].cpu().numpy()
        full = oracle.forward(cfg, w, seq, want_hidden=False)["logits"]
        ref = full[:, -1]
        c = cosine(z, ref)
        assert c >= STEP_COS, f"step {step}: cosine {c}"
        pinned, near, fails = argmax_check(tok, ref, band_for(cfg, w, seq, full).reshape(seq.shape)[:, -1])
        assert not fails, fails
        plain = model.prefill(seq, logits=True, argmax=False)["logits"][:, -1].cpu().numpy()
        assert cosine(z, plain) >= COS_MIN
        seq = np.concatenate([seq, tok[:, None]], axis=1)
        out = sess.decode(tok, logits=True, argmax=True)
        out = {"logits": out["logits"], "argmax": out["argmax"]}
        tok = out["argmax"][:, -1].cpu().numpy()
    _say(f"  {cfg.name}: 4 cached steps, last cosine vs oracle {c:.6f}")
    sess.close()
    model.close()


# The variant epilogues on the 256 x 256 ping-pong kernel: 4 x 2048 rows with the
# Llama-3-8B layer shape give every projection at least 256 tiles of 256 x 256 (QKV
# 32 x 24, O and down 32 x 16, gate/up 32 x 112, head 32 x 125), which selects it for
# the unrotated q/k of QK-norm, the tanh-GELU gate, the sandwich products and the
# llama3-scaled RoPE tables. Row 3 is compared with the oracle over a prefix of P
# positions (causal prefix invariance), every slot.
BIG = dict(n_layers=2, vocab=32000, gain_sigma=0.2, batch=4, seq=2048)
QWEN3_BIG = wl.LLAMA3_8B.replace(qk_norm=True, name="qwen3-like-2L-4x2048", **BIG)
GEMMA3_BIG = wl.LLAMA3_8B.replace(qk_norm=True, norm_gain_offset=1, ffn_act="gelu_tanh", norm_placement="sandwich",
                                  sliding_window=1024, layer_kind=("local", "global"), rope_theta=1e6,
                                  rope_theta_local=1e4, final_logit_softcap=30.0, embed_scale_mode="bf16_sqrt_hidden",
                                  name="gemma3-like-2L-4x2048", **BIG)
LLAMA3_SCALED_BIG = wl.LLAMA3_8B.replace(rope_scaling="llama3", rope_factor=8.0, rope_low_freq_factor=1.0,
                                         rope_high_freq_factor=4.0, rope_original_max_pos=8192,
                                         name="llama3-scaled-2L-4x2048", **BIG)


def _pp_tiles(M, N):
    return ((M + 255) // 256) * ((N + 255) // 256)


@pytest.mark.parametrize("cfg,P", [(QWEN3_BIG, 512), (GEMMA3_BIG, 1100), (LLAMA3_SCALED_BIG, 512)],
                         ids=lambda v: v.name if hasattr(v, "name") else str(v))
def test_variants_on_the_large_tile_kernel(fwd, cfg, P):
    T = cfg.batch * cfg.seq
    H, F, V = cfg.hidden, cfg.ffn, cfg.vocab
    qkv = (cfg.n_heads + 2 * cfg.n_kv_heads) * cfg.head_dim
    for N in (qkv, H, 2 * F, V):  # every product takes the 256 x 256 kernel (>= 256 such tiles)
        assert _pp_tiles(T, N) >= 256
    host = wl.draw_all(cfg)
    ids = np.asarray(wl.draw_ids(cfg))
    model = fwd.Model(cfg, upload_weights(cfg, host), max_tokens=T)
    out = model.prefill(ids, logits=True, hidden=True, argmax=True)
    got = {"hidden": out["hidden"][:, 3:4, :P].cpu().numpy(), "logits": out["logits"][3:4, :P].cpu().numpy(),
           "argmax": out["argmax"][3:4, :P].cpu().numpy()}
    del out
    model.close()
    w = wl.HostWeights(host)
    ref = oracle.forward(cfg, w, ids[3:4, :P])
    for s in range(cfg.n_layers + 2):
        c = cosine(got["hidden"][s], ref["hidden"][s])
        assert c >= COS_MIN, f"{cfg.name}: slot {s} cosine {c}"
    band = band_for(cfg, w, ids[3:4, :P], ref["logits"])
    pinned, near, fails = argmax_check(got["argmax"], ref["logits"], band)
    assert not fails, fails[:5]
    d, b = logit_band_check(got["logits"], ref["logits"], band)
    assert d <= b, f"max|dlogit| {d} over the oracle-side allowance {b}"
    worst = min(cosine(got["hidden"][s], ref["hidden"][s]) for s in range(cfg.n_layers + 2))
    _say(f"  {cfg.name}: row 3 x {P}: lowest slot cosine {worst:.7f}, max|dlogit| {d:.3e} (allowance {b:.3e}), "
         f"argmax pinned {pinned} near-tie {near}")
