"""Cached sessions (fwd_session_*): a prefill that fills the KV cache, then greedy
decode steps over it.

Gates:
- "N7 · model/forward-parity", Theorem 1: the cached session reproduces the cacheless
  forward's last-position logits within 1e-4 (fp32 configuration), and the greedy
  continuation ids match token for token. For bf16 the cached step and the cacheless
  prefill round differently (attention over the cache runs in fp32), so the gate there
  is the half-precision one below plus argmax parity.
- "N9 · metalgemm", Theorem 1: argmax-exact and cosine >= 0.999 against the CPU
  reference at every prefill and greedy step, 6 prompt + 8 greedy steps.
Near ties follow the same reading as the prefill tests (argmax_check).
"""
import json
import os
import sys

import numpy as np
import pytest

import oracle
from synth import workloads as wl
from tests.gpu_util import F32_LOGIT_BAND, argmax_check, band_for, cosine, upload_weights

pytestmark = pytest.mark.gpu
GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page_values.json")))
CACHED_MAX = GOLD["cached_prefill_logits_max_abs"]["value"]
STEP_COS = GOLD["metal_forward_cosine_min"]["value"]
PROMPT, STEPS = GOLD["greedy_prompt_and_steps"]["value"]


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


def _generate(fwd, model, prompt, steps, max_seq):
    """Session prefill + `steps` decode steps, feeding back the GPU's own argmax.
    Returns (tokens [B, steps + 1], logits [steps + 1, B, V]) like oracle.greedy."""
    B = prompt.shape[0]
    sess = fwd.Session(model, max_batch=B, max_seq=max_seq)
    out = sess.prefill(prompt, logits=True, argmax=True)
    logits = [out["logits"][:, -1].cpu().numpy()]
    toks = [out["argmax"][:, -1].cpu().numpy()]
    for _ in range(steps):
        out = sess.decode(toks[-1], logits=True, argmax=True)
        logits.append(out["logits"][:, 0].cpu().numpy())
        toks.append(out["argmax"][:, 0].cpu().numpy())
    assert sess.length == prompt.shape[1] + steps
    sess.close()
    return np.stack(toks, axis=1), np.stack(logits)


def _check_against_oracle(cfg, host, prompt, toks, logits):
    """Every step: cosine >= 0.999 and argmax parity (near-tie rule) against the
    oracle's cacheless greedy continuation, fed the GPU's tokens so both see the same
    sequence."""
    n = toks.shape[1]
    ref_logits = np.empty_like(logits)
    bands = np.empty(logits.shape[:2])
    seq = prompt
    w = wl.HostWeights(host)
    for i in range(n):
        full = oracle.forward(cfg, w, seq, want_hidden=False)["logits"]
        ref_logits[i] = full[:, -1]
        bands[i] = band_for(cfg, w, seq, full).reshape(seq.shape)[:, -1]
        seq = np.concatenate([seq, toks[:, i:i + 1]], axis=1)
    for i in range(n):
        c = cosine(logits[i], ref_logits[i])
        assert c >= STEP_COS, f"step {i}: cosine {c}"
        pinned, near, fails = argmax_check(toks[:, i], ref_logits[i], bands[i])
        assert not fails, f"step {i}: {fails[:3]}"
    return ref_logits


def _check_cacheless(model, prompt, toks, logits, max_abs=None, min_cos=None):
    """Each decode step against the library's own cacheless prefill over the same
    sequence (last position)."""
    seq = prompt
    for i in range(toks.shape[1]):
        full = model.prefill(seq, logits=True, argmax=False)["logits"][:, -1].cpu().numpy()
        if max_abs is not None:
            d = float(np.max(np.abs(full - logits[i])))
            assert d <= max_abs, f"step {i}: max|cached - cacheless| = {d}"
        if min_cos is not None:
            c = cosine(full, logits[i])
            assert c >= min_cos, f"step {i}: cosine {c}"
        seq = np.concatenate([seq, toks[:, i:i + 1]], axis=1)


def test_f32_cached_steps_match_cacheless_and_oracle(fwd):
    cfg = wl.TINY_F32.replace(batch=2, seq=PROMPT)
    _say(f"session f32 tiny: {PROMPT} prompt + {STEPS} greedy steps, 2 rows")
    host = wl.draw_all(cfg)
    prompt = np.asarray(wl.draw_ids(cfg))
    model = fwd.Model(cfg, upload_weights(cfg, host), max_tokens=2 * (PROMPT + STEPS + 1))
    toks, logits = _generate(fwd, model, prompt, STEPS, max_seq=PROMPT + STEPS + 1)
    _check_cacheless(model, prompt, toks, logits, max_abs=CACHED_MAX)
    _check_against_oracle(cfg, host, prompt, toks, logits)
    # greedy ids token for token against the oracle's own continuation
    ref_toks, ref_logits = oracle.greedy(cfg, wl.HostWeights(host), prompt, STEPS + 1)
    pinned, near, fails = argmax_check(toks.T.ravel(), ref_logits.reshape(-1, cfg.vocab), F32_LOGIT_BAND)
    assert not fails and np.array_equal(toks, ref_toks), (toks, ref_toks)
    model.close()


def test_bf16_cached_steps_match_oracle(fwd):
    cfg = wl.SMOLLM2_135M.replace(n_layers=2, batch=2, seq=PROMPT, name="smol-2L-session")
    _say(f"session bf16 smollm2-shape 2 layers: {PROMPT} prompt + {STEPS} greedy steps, 2 rows")
    host = wl.draw_all(cfg)
    prompt = np.asarray(wl.draw_ids(cfg))
    model = fwd.Model(cfg, upload_weights(cfg, host), max_tokens=2 * (PROMPT + STEPS + 1))
    toks, logits = _generate(fwd, model, prompt, STEPS, max_seq=PROMPT + STEPS + 1)
    _check_against_oracle(cfg, host, prompt, toks, logits)
    _check_cacheless(model, prompt, toks, logits, min_cos=0.9999)
    model.close()


def test_bf16_window_sandwich_decode_evicts(fwd):
    """Local layers with a 64-key window, the prompt already longer than the window, so
    every decode step drops a key; sandwich norms and softcap on."""
    cfg = wl.SMOLLM2_135M.replace(n_layers=2, sliding_window=64, layer_kind=("local", "global"),
                                  norm_placement="sandwich", final_logit_softcap=30.0,
                                  embed_scale_mode="bf16_sqrt_hidden", batch=1, seq=70, name="smol-2L-window-session")
    _say("session bf16 window 64 sandwich: 70 prompt + 6 steps")
    host = wl.draw_all(cfg)
    prompt = np.asarray(wl.draw_ids(cfg))
    model = fwd.Model(cfg, upload_weights(cfg, host), max_tokens=80)
    toks, logits = _generate(fwd, model, prompt, 6, max_seq=80)
    _check_against_oracle(cfg, host, prompt, toks, logits)
    _check_cacheless(model, prompt, toks, logits, min_cos=0.9999)
    model.close()


def test_bf16_decode_over_several_key_chunks(fwd):
    """A 300-token prompt spans two 256-key chunks of the decode attention (merged by the
    second kernel); three rows."""
    cfg = wl.SMOLLM2_135M.replace(n_layers=2, batch=3, seq=300, name="smol-2L-long-session")
    _say("session bf16: 3 x 300 prompt + 3 steps (two key chunks)")
    host = wl.draw_all(cfg)
    prompt = np.asarray(wl.draw_ids(cfg))
    model = fwd.Model(cfg, upload_weights(cfg, host), max_tokens=3 * 304)
    toks, logits = _generate(fwd, model, prompt, 3, max_seq=304)
    _check_cacheless(model, prompt, toks, logits, min_cos=0.9999)
    _check_against_oracle(cfg, host, prompt[:1], toks[:1], logits[:, :1])
    model.close()


def test_session_prefill_outputs_equal_plain_prefill(fwd):
    cfg = wl.SMOLLM2_135M.replace(n_layers=2, batch=2, seq=40, name="smol-2L-prefill-session")
    _say("session prefill vs plain prefill, bitwise")
    host = wl.draw_all(cfg)
    ids = np.asarray(wl.draw_ids(cfg))
    model = fwd.Model(cfg, upload_weights(cfg, host), max_tokens=ids.size)
    plain = model.prefill(ids, logits=True, hidden=True, argmax=True)
    sess = fwd.Session(model, max_batch=2, max_seq=64)
    cached = sess.prefill(ids, logits=True, hidden=True, argmax=True)
    for k in ("logits", "hidden", "argmax"):
        assert np.array_equal(plain[k].cpu().numpy(), cached[k].cpu().numpy()), k
    sess.close()
    model.close()


def test_session_errors(fwd):
    import torch
    cfg = wl.TINY_F32
    host = wl.draw_all(cfg)
    model = fwd.Model(cfg, upload_weights(cfg, host), max_tokens=32)
    sess = fwd.Session(model, max_batch=2, max_seq=8)
    with pytest.raises(fwd.FwdError) as e:
        sess.decode(np.zeros(1, np.int32))
    assert e.value.code == fwd.FWD_E_ARG                      # no prefill yet
    with pytest.raises(fwd.FwdError) as e:
        sess.prefill(np.zeros((3, 4), np.int32))
    assert e.value.code == fwd.FWD_E_TOO_LARGE                # B > max_batch
    with pytest.raises(fwd.FwdError) as e:
        sess.prefill(np.zeros((1, 9), np.int32))
    assert e.value.code == fwd.FWD_E_TOO_LARGE                # S > max_seq
    sess.prefill(np.zeros((1, 7), np.int32))
    bad = np.array([cfg.vocab], np.int32)
    with pytest.raises(fwd.FwdError) as e:
        sess.decode(bad)
    assert e.value.code == fwd.FWD_E_TOKEN_RANGE
    assert sess.length == 7
    sess.decode(np.array([1], np.int32))
    assert sess.length == 8
    with pytest.raises(fwd.FwdError) as e:
        sess.decode(np.array([1], np.int32))
    assert e.value.code == fwd.FWD_E_TOO_LARGE                # full
    with pytest.raises(fwd.FwdError) as e:
        fwd.Session(model, max_batch=33, max_seq=8)
    assert e.value.code == fwd.FWD_E_TOO_LARGE                # above max_tokens
    sess.close()
    model.close()
    torch.cuda.synchronize()


@pytest.mark.parametrize("shape", ["d128_g4", "d256_g2_window", "d64_g8", "d128_g1", "d128_g2_window", "d128_g8"])
def test_bf16_decode_head_shapes(fwd, shape):
    """The decode attention's head geometries: 128-wide heads in groups of 4 (Llama-3
    shape), 256-wide heads in pairs with a 64-key window on local layers (Gemma-style),
    64-wide heads in groups of 8, and the other group sizes of the 128-wide kernel (1;
    2 with a window; 8); a 300-token prompt spans two key chunks."""
    base = {"d128_g4": wl.LLAMA3_8B.replace(n_heads=8, n_kv_heads=2, head_dim=128),
            "d128_g1": wl.LLAMA3_8B.replace(n_heads=4, n_kv_heads=4, head_dim=128),
            "d128_g2_window": wl.LLAMA3_8B.replace(n_heads=4, n_kv_heads=2, head_dim=128, sliding_window=64,
                                                   layer_kind=("local", "global")),
            "d128_g8": wl.LLAMA3_8B.replace(n_heads=16, n_kv_heads=2, head_dim=128),
            "d256_g2_window": wl.GEMMA3_STYLE.replace(n_heads=4, n_kv_heads=2, head_dim=256, sliding_window=64,
                                                      layer_kind=("local", "global")),
            "d64_g8": wl.SMOLLM2_135M.replace(n_heads=16, n_kv_heads=2, head_dim=64)}[shape]
    cfg = base.replace(n_layers=2, hidden=512, ffn=1024, vocab=2048, batch=2, seq=300, name=f"session-{shape}")
    _say(f"session bf16 {shape}: 2 x 300 prompt + 3 steps")
    host = wl.draw_all(cfg)
    prompt = np.asarray(wl.draw_ids(cfg))
    model = fwd.Model(cfg, upload_weights(cfg, host), max_tokens=2 * 304)
    toks, logits = _generate(fwd, model, prompt, 3, max_seq=304)
    _check_cacheless(model, prompt, toks, logits, min_cos=0.9999)
    _check_against_oracle(cfg, host, prompt[:1], toks[:1], logits[:, :1])
    model.close()
