"""Mixture-of-experts feed-forward against the oracle (qwen3moe hybrid dense/sparse
axis of "N7 · model/forward-parity", Theorem statement; the intro lists the MoE FFN).

- The routing decision alone (fwd_moe_route) on the same fp32 logits: expert ids bit
  for bit, with planted exact ties (lowest index first), weights to fp32 rounding.
- Whole forwards with every expert active (k = E: no discrete decision, the weights
  are the softmax) on both the tiled and the few-row path, a MoE layer between dense
  ones, sandwich norms, and a cached decode.
- Top-k < E with the MoE layer last: a token whose k-th and (k+1)-th router logits
  are closer than the bf16 error could legitimately route differently, and no later
  layer mixes tokens, so exactly those tokens are excluded (counted) and every other
  token is held to the gates of the dense forward.
"""
import json
import os
import sys

import numpy as np
import pytest

import oracle
from synth import workloads as wl
from tests.gpu_util import argmax_check, cosine, upload_weights

pytestmark = pytest.mark.gpu
GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page_values.json")))
COS_MIN = GOLD["hidden_cosine_min"]["value"]
STEP_COS = GOLD["metal_forward_cosine_min"]["value"]

BASE = wl.SMOLLM2_135M.replace(n_layers=3, hidden=512, ffn=1024, vocab=2048, n_experts=8, moe_ffn=256,
                               gain_sigma=0.1)
ALL_EXPERTS = BASE.replace(n_experts_per_tok=8, ffn_kind=("dense", "moe", "dense"), name="moe-all-experts")
ALL_SANDWICH = ALL_EXPERTS.replace(norm_placement="sandwich", ffn_kind=("moe", "dense", "moe"),
                                   moe_norm_topk=False, name="moe-all-sandwich")
TOP2_LAST = BASE.replace(n_experts_per_tok=2, ffn_kind=("dense", "dense", "moe"), router_sigma=0.1,
                         name="moe-top2-last")


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


@pytest.mark.parametrize("T,E,k,norm", [(300, 64, 8, True), (77, 256, 8, False), (5, 3, 3, True), (40, 8, 1, True)])
def test_route_op_matches_oracle_decisions(fwd, T, E, k, norm):
    import torch
    rng = np.random.default_rng(T + E)
    z = (rng.standard_normal((T, E)) * 2).astype(np.float32)
    z[::7, 1] = z[::7, 0]                      # exact ties: the lower index must come first
    z[3::11, E - 1] = z[3::11].max(-1)         # a tie at the top
    idx, w = fwd.moe_route(torch.from_numpy(z).cuda(), k, norm)
    ref_idx, ref_w = oracle.moe_route(z, k, norm)
    assert np.array_equal(idx.cpu().numpy(), ref_idx)
    np.testing.assert_allclose(w.cpu().numpy(), ref_w, rtol=2e-6, atol=1e-7)


def _check(cfg, got, ref, rows_mask=None, slots=None):
    L = cfg.n_layers
    for s in (slots if slots is not None else range(L + 2)):
        g, r = got["hidden"][s], ref["hidden"][s]
        if rows_mask is not None:
            g, r = g[rows_mask], r[rows_mask]
        c = cosine(g, r)
        assert c >= COS_MIN, f"{cfg.name}: slot {s} cosine {c}"
    gz, rz, ga = got["logits"], ref["logits"], got["argmax"]
    if rows_mask is not None:
        gz, rz, ga = gz[rows_mask], rz[rows_mask], ga[rows_mask]
    pinned, near, fails = argmax_check(ga, rz, gz)
    assert not fails, fails[:5]
    return pinned, near


@pytest.mark.parametrize("cfg", [ALL_EXPERTS, ALL_SANDWICH], ids=lambda c: c.name)
def test_moe_all_experts_forward(fwd, cfg):
    host = wl.draw_all(cfg)
    model = fwd.Model(cfg, upload_weights(cfg, host), max_tokens=96)
    ids = np.asarray(wl.draw_ids(cfg, batch=2, seq=48))
    for part in (ids, ids[:1, :12]):           # 96 rows: tiled router product; 12: the few-row kernel
        got = {k: v.cpu().numpy() for k, v in model.prefill(part, logits=True, hidden=True, argmax=True).items()}
        ref = oracle.forward(cfg, wl.HostWeights(host), part)
        pinned, near = _check(cfg, got, ref)
        _say(f"  {cfg.name} {part.shape}: argmax pinned {pinned} near-tie {near}")
    # bitwise repeatable (integer counting, fixed summation order)
    a = model.prefill(ids, logits=True, hidden=False, argmax=True)["logits"].cpu().numpy()
    b = model.prefill(ids, logits=True, hidden=False, argmax=True)["logits"].cpu().numpy()
    assert np.array_equal(a, b)
    model.close()


def test_moe_top2_last_layer_on_decided_tokens(fwd):
    cfg = TOP2_LAST
    host = wl.draw_all(cfg)
    model = fwd.Model(cfg, upload_weights(cfg, host), max_tokens=96)
    ids = np.asarray(wl.draw_ids(cfg, batch=2, seq=48))
    got = {k: v.cpu().numpy() for k, v in model.prefill(ids, logits=True, hidden=True, argmax=True).items()}
    w = wl.HostWeights(host)
    tr, trb = {}, {}
    ref = oracle.forward(cfg, w, ids, trace=tr)
    oracle.forward(cfg, w, ids, want_logits=False, bf16_points=True, trace=trb)
    z = tr["moe_logits.2"].astype(np.float64)
    err = np.abs(z - trb["moe_logits.2"]).max()           # logit error of bf16 operands
    zs = -np.sort(-z, axis=-1)
    margin = zs[:, 1] - zs[:, 2]                           # 2nd vs 3rd largest logit
    decided = (margin > 4 * err).reshape(ids.shape)
    assert decided.mean() >= 0.75, (decided.mean(), err)
    L = cfg.n_layers
    # slots before the MoE layer hold every token; from it on, only the decided ones
    _check(cfg, got, ref, slots=range(L))
    pinned, near = _check(cfg, got, ref, rows_mask=decided, slots=(L, L + 1))
    _say(f"  {cfg.name}: {int(decided.sum())} of {decided.size} tokens decided (bf16 logit error {err:.2e}), "
         f"argmax pinned {pinned} near-tie {near}")
    model.close()


def test_moe_cached_decode(fwd):
    cfg = ALL_EXPERTS
    host = wl.draw_all(cfg)
    model = fwd.Model(cfg, upload_weights(cfg, host), max_tokens=64)
    prompt = np.asarray(wl.draw_ids(cfg, batch=2, seq=20))
    sess = fwd.Session(model, max_batch=2, max_seq=32)
    out = sess.prefill(prompt, logits=True, argmax=True)
    seq, w = prompt, wl.HostWeights(host)
    for step in range(4):
        z = out["logits"][:, -1].cpu().numpy()
        tok = out["argmax"][:, -1].cpu().numpy()
        ref = oracle.forward(cfg, w, seq, want_hidden=False)["logits"][:, -1]
        c = cosine(z, ref)
        assert c >= STEP_COS, f"step {step}: cosine {c}"
        pinned, near, fails = argmax_check(tok, ref, z)
        assert not fails, fails
        seq = np.concatenate([seq, tok[:, None]], axis=1)
        out = sess.decode(tok, logits=True, argmax=True)
    _say(f"  {cfg.name}: 4 cached steps, last cosine vs oracle {c:.6f}")
    sess.close()
    model.close()
