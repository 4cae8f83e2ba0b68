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
from tests.gpu_util import argmax_check, band_for, cosine, oracle_band, upload_weights

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


def _check(cfg, got, ref, band, rows_mask=None, slots=None, argmax=True):
    """Hidden slots by cosine on the given rows; with argmax, the argmax on those rows
    under the oracle-side band. Where routing is undecided on some tokens (their k-th and
    (k+1)-th router logits lie within the bf16 error), the argmax is checked on the
    decided tokens only: an undecided token may take other experts and its logits are
    then not comparable."""
    L = cfg.n_layers
    for s in (slots if slots is not None else range(L + 2)):
        g, r = got["hidden"][s], ref["hidden"][s]
        if rows_mask is not None:
            g, r = g[rows_mask], r[rows_mask]
        c = cosine(g, r)
        assert c >= COS_MIN, f"{cfg.name}: slot {s} cosine {c}"
    if not argmax:
        return None, None
    rz, ga, band = ref["logits"], got["argmax"], np.asarray(band).reshape(got["argmax"].shape)
    if rows_mask is not None:
        rz, ga, band = rz[rows_mask], ga[rows_mask], band[rows_mask]
    pinned, near, fails = argmax_check(ga, rz, band)
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
        pinned, near = _check(cfg, got, ref, band_for(cfg, wl.HostWeights(host), part, ref["logits"]))
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
    refb = oracle.forward(cfg, w, ids, want_hidden=False, bf16_points=True, trace=trb)
    band = oracle_band(ref["logits"], refb["logits"])
    z = tr["moe_logits.2"].astype(np.float64)
    err = np.abs(z - trb["moe_logits.2"]).max()           # logit error of bf16 operands
    zs = -np.sort(-z, axis=-1)
    margin = zs[:, 1] - zs[:, 2]                           # 2nd vs 3rd largest logit
    decided = (margin > 4 * err).reshape(ids.shape)
    assert decided.mean() >= 0.75, (decided.mean(), err)
    L = cfg.n_layers
    # slots before the MoE layer hold every token; from it on, only the decided ones
    _check(cfg, got, ref, band, slots=range(L), argmax=False)
    pinned, near = _check(cfg, got, ref, band, rows_mask=decided, slots=(L, L + 1))
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
        full = oracle.forward(cfg, w, seq, want_hidden=False)["logits"]
        ref = full[:, -1]
        c = cosine(z, ref)
        assert c >= STEP_COS, f"step {step}: cosine {c}"
        pinned, near, fails = argmax_check(tok, ref, band_for(cfg, w, seq, full).reshape(seq.shape)[:, -1])
        assert not fails, fails
        seq = np.concatenate([seq, tok[:, None]], axis=1)
        out = sess.decode(tok, logits=True, argmax=True)
    _say(f"  {cfg.name}: 4 cached steps, last cosine vs oracle {c:.6f}")
    sess.close()
    model.close()


def _routing_masks(cfg, w, ids, ref_trace, l):
    """(decided tokens [B, S], per-expert row counts) of MoE layer l: the oracle's routing
    and, against the bf16-rounded oracle's router logits, the tokens whose k-th and
    (k+1)-th logits are more than 4x the bf16 logit error apart."""
    trb = {}
    refb = oracle.forward(cfg, w, ids, want_hidden=False, bf16_points=True, trace=trb)
    z = ref_trace[f"moe_logits.{l}"].astype(np.float64)
    err = np.abs(z - trb[f"moe_logits.{l}"]).max()
    zs = -np.sort(-z, axis=-1)
    k = cfg.n_experts_per_tok
    decided = (zs[:, k - 1] - zs[:, k] > 4 * err).reshape(ids.shape)
    idx, _ = oracle.moe_route(z, k, cfg.moe_norm_topk)
    counts = np.bincount(idx.ravel(), minlength=cfg.n_experts)
    return decided, counts, err, refb


# Top-2 of 8 experts over 2048 tokens: expert segments span up to eight 256-row tiles
# of the grouped products, with ragged ends. Experts 6 and 7 are planted empty:
# dimension 5 of every embedding row is set to 0.5 and no layer reads or writes it, so
# that dimension of the normalised MoE input sits near +17 for every token; the router
# rows of experts 6 and 7 read only that dimension, with weight -1, so their logits stay
# near -17, far below any top-2 choice, and the other experts' rows do not read it.
# (On these weights expert 0 also receives no token.) The grouped products must skip
# the empty experts.
MULTI_TILE = BASE.replace(n_experts_per_tok=2, ffn_kind=("dense", "dense", "moe"), router_sigma=0.1,
                          batch=1, seq=2048, name="moe-top2-multitile")


def _planted_empty_experts(cfg, host):
    from synth import to_bf16_bits
    host = dict(host)
    E = host["embed"].copy()
    E[:, 5] = to_bf16_bits(np.float32(0.5))
    host["embed"] = E
    for l in range(cfg.n_layers):  # no layer reads or writes dimension 5: it stays 0.5 in every row
        p = f"layers.{l}."
        for n in ("wq", "wk", "wv", "w_gate", "w_up"):
            if p + n in host:
                host[p + n] = host[p + n].copy()
                host[p + n][:, 5] = 0
        for n in ("wo", "w_down"):
            if p + n in host:
                host[p + n] = host[p + n].copy()
                host[p + n][5, :] = 0
    r = host["layers.2.router"].copy()
    r[:, 5] = 0                                    # experts 0-5 do not read the planted dimension
    r[6:8] = 0
    r[6:8, 5] = to_bf16_bits(np.float32(-1.0))
    host["layers.2.router"] = r
    return host


def test_moe_multi_tile_segments_and_empty_experts(fwd):
    cfg = MULTI_TILE
    host = _planted_empty_experts(cfg, wl.draw_all(cfg))
    ids = np.asarray(wl.draw_ids(cfg))
    model = fwd.Model(cfg, upload_weights(cfg, host), max_tokens=ids.size)
    got = {k: v.cpu().numpy() for k, v in model.prefill(ids, logits=True, hidden=True, argmax=True).items()}
    w = wl.HostWeights(host)
    tr = {}
    ref = oracle.forward(cfg, w, ids, trace=tr)
    decided, counts, err, refb = _routing_masks(cfg, w, ids, tr, 2)
    _say(f"  {cfg.name}: rows per expert {counts.tolist()}, {int(decided.sum())} of {decided.size} tokens "
         f"decided (bf16 router logit error {err:.2e})")
    assert counts[6] == 0 and counts[7] == 0, "the planted experts must receive no rows"
    assert counts.max() > 512, "an expert segment should span three or more 256-row tiles"
    assert np.any(counts[:6] % 16 != 0), "a segment should end inside a 16-row block"
    assert decided.mean() >= 0.75, decided.mean()
    band = oracle_band(ref["logits"], refb["logits"])
    L = cfg.n_layers
    _check(cfg, got, ref, band, slots=range(L), argmax=False)
    pinned, near = _check(cfg, got, ref, band, rows_mask=decided, slots=(L, L + 1))
    _say(f"  {cfg.name}: argmax pinned {pinned} near-tie {near} on the decided tokens")
    model.close()


def test_moe_128_experts_top8_full_size(fwd):
    """The benchmark's MoE shape (hidden 2048, 32/4 heads x 128 with QK-norm, 128 experts
    of width 768, top-8, vocabulary 151936) with one MoE layer over 8 x 2048 tokens, so the
    grouped products run at their production size (about 1024 rows per expert, four
    256-row tiles each). Row 0 is compared at every position on the decided tokens (the
    layer is the last, so an undecided token affects only itself)."""
    cfg = wl.ModelConfig("moe-128e-top8-1L", 1, 2048, 32, 4, 128, 6144, 151936, rope_theta=1e6, qk_norm=True,
                         n_experts=128, n_experts_per_tok=8, moe_ffn=768, batch=8, seq=2048)
    host = wl.draw_all(cfg)
    ids = np.asarray(wl.draw_ids(cfg))
    model = fwd.Model(cfg, upload_weights(cfg, host), max_tokens=ids.size)
    out = model.prefill(ids, logits=True, hidden=True, argmax=True)
    got = {"hidden": out["hidden"][:, :1].cpu().numpy(), "logits": out["logits"][:1].cpu().numpy(),
           "argmax": out["argmax"][:1].cpu().numpy()}
    del out
    model.close()
    w = wl.HostWeights(host)
    tr = {}
    _say(f"  {cfg.name}: oracle over row 0 (2048 tokens)")
    ref = oracle.forward(cfg, w, ids[:1], trace=tr)
    decided, counts, err, refb = _routing_masks(cfg, w, ids[:1], tr, 0)
    _say(f"  {cfg.name}: row 0 rows per expert min {counts.min()} max {counts.max()}, {int(decided.sum())} of "
         f"{decided.size} tokens decided (bf16 router logit error {err:.2e})")
    # 128 logits leave small gaps between the 8th and 9th: about a fifth of the tokens are
    # decided beyond four times the bf16 router-logit error
    assert decided.mean() >= 0.15, decided.mean()
    band = oracle_band(ref["logits"], refb["logits"])
    _check(cfg, got, ref, band, slots=(0,), argmax=False)
    pinned, near = _check(cfg, got, ref, band, rows_mask=decided, slots=(1, 2))
    _say(f"  {cfg.name}: argmax pinned {pinned} near-tie {near} on the decided tokens")
