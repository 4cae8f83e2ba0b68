"""Parity at the full workload sizes, in the launch configuration the benchmark times.

The oracle cannot run whole 8 x 2048-token Llama-3-8B-shaped batches or the
48-layer 1024-token Gemma-style prompt in test time, so it recomputes sampled
positions: by causal prefix invariance (pinned in the oracle tests) the first P
positions of any row depend only on that row's first P tokens. Properties that
hold at any size (finite logits, argmax consistent with the logits, batch rows
reproduced alone) are checked on the whole output.
"""
import json
import os
import sys
import time

import numpy as np
import pytest

import oracle
from synth import workloads as wl
from tests.gpu_util import (COS_HALF_PRECISION, FLOOR_SLACK, argmax_check, cosine, distributional_gate,
                            logit_band_check, oracle_band, slot_parity, to_device)

pytestmark = pytest.mark.gpu
GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page_values.json")))
COS_MIN = GOLD["hidden_cosine_min"]["value"]


@pytest.fixture(scope="module")
def fwd():
    import torch
    from decoder_only_transformer_bf16_amd import fwd as F
    assert torch.cuda.is_available(), "GPU tests need a visible GPU"
    torch.cuda.set_device(0)
    assert F.available(), "libfwd.so sees no gfx950 device"
    return F


def _say(msg):
    print(f"[{time.strftime('%H:%M:%S')}] {msg}", flush=True)
    sys.stdout.flush()


def _build(fwd, cfg, max_tokens):
    """Draw every weight once (host, storage form), upload tensor by tensor, pack."""
    host, dev = {}, {}
    for n in wl.weight_shapes(cfg):
        host[n] = wl.draw_weight(cfg, n)
        dev[n] = to_device(host[n])
    model = fwd.Model(cfg, dev, max_tokens=max_tokens)
    del dev
    import torch
    torch.cuda.empty_cache()
    return model, wl.HostWeights(host)


def _compare(cfg, hid, logits, am, ref, refb, label):
    """Hidden slots, logits and argmax of one sample against the oracle (ref) with the
    oracle rounded at the bf16 points (refb: the precision floor of the slots and the
    logit allowance of the argmax gate). hid [L+2, R, P, H], logits [R, P, V], am [R, P]."""
    worst = (1.0, -1, None)
    for s in range(cfg.n_layers + 2):
        ok, c, floor = slot_parity(hid[s], ref["hidden"][s], lambda s=s: refb["hidden"][s])
        assert ok, f"{label}: slot {s}: cosine {c} (bf16 floor {floor})"
        worst = min(worst, (c, s, floor))
    _say(f"  {label}: lowest slot cosine {worst[0]:.6f} at slot {worst[1]} (bf16-rounded oracle there: {worst[2]})")
    band = oracle_band(ref["logits"], refb["logits"])
    pinned, near, fails = argmax_check(am, ref["logits"], band)
    assert not fails, fails[:5]
    d, b = logit_band_check(logits, ref["logits"], band)
    assert d <= b, f"{label}: max|dlogit| {d} over the oracle-side allowance {b}"
    # how closely the GPU follows the oracle rounded at its own bf16 points
    zb = np.asarray(refb["logits"], np.float64).reshape(-1, cfg.vocab)
    same_b = float(np.mean(np.asarray(am).ravel() == np.argmax(zb, -1)))
    d_b = float(np.max(np.abs(np.asarray(logits, np.float64).reshape(zb.shape) - zb)))
    same_o = float(np.mean(np.argmax(zb, -1) == np.asarray(ref["argmax"]).ravel()))
    _say(f"  {label}: max|dlogit| {d:.3e} (allowance {b:.3e}), argmax pinned {pinned} near-tie {near}; "
         f"vs the bf16-rounded oracle: max|dlogit| {d_b:.3e}, same argmax {same_b:.4f} "
         f"(bf16-rounded oracle vs oracle: {same_o:.4f})")
    return pinned, near


def _compare_sampled(cfg, out, rows, P, host, ids):
    import torch
    idx_r = torch.as_tensor(rows, device="cuda")
    hid = out["hidden"][:, idx_r, :P].cpu().numpy()
    logits = out["logits"][idx_r, :P].cpu().numpy()
    am = out["argmax"][idx_r, :P].cpu().numpy()
    ref = oracle.forward(cfg, host, ids[rows, :P])
    refb = oracle.forward(cfg, host, ids[rows, :P], bf16_points=True)
    return _compare(cfg, hid, logits, am, ref, refb, f"rows {rows} x {P} positions")


def _whole_output_properties(out):
    import torch
    z = out["logits"]
    assert torch.isfinite(z).all().item()
    am = out["argmax"].long()
    picked = torch.gather(z, -1, am.unsqueeze(-1)).squeeze(-1)
    assert torch.equal(picked, z.max(-1).values), "argmax is not a maximiser of its row"


@pytest.fixture(scope="module")
def llama(fwd):
    """The Llama-3-8B-shaped model, its host weights and the batch's ids, shared by the
    tests below (results they hand on go in `state`)."""
    import torch
    cfg = wl.LLAMA3_8B
    _say("llama3-8b-shape: drawing and uploading 7.5e9 weights")
    model, host = _build(fwd, cfg, cfg.batch * cfg.seq)
    ids = wl.draw_ids(cfg)
    yield {"cfg": cfg, "model": model, "host": host, "ids": ids, "state": {}}
    model.close()
    torch.cuda.empty_cache()


def test_llama3_8b_full_batch(fwd, llama):
    """The benchmark's launch: 8 x 2048 with every output. Properties that hold at any
    size on the whole output; row 0 in full and the first 256 positions of rows 1-7 are
    kept for the oracle comparisons below (causal prefix invariance makes a prefix of a
    row a forward of its own)."""
    import torch
    cfg, model, ids, st = llama["cfg"], llama["model"], llama["ids"], llama["state"]
    _say("prefill 8 x 2048 (the benchmark's launch)")
    out = model.prefill(ids, logits=True, hidden=True, argmax=True)
    torch.cuda.synchronize()
    _whole_output_properties(out)
    st["row0"] = (out["hidden"][:, :1].cpu().numpy(), out["logits"][:1].cpu().numpy(),
                  out["argmax"][:1].cpu().numpy())
    st["rows1_7"] = (out["hidden"][:, 1:, :PREFIX].cpu().numpy(), out["logits"][1:, :PREFIX].cpu().numpy(),
                     out["argmax"][1:, :PREFIX].cpu().numpy())
    # a row alone reproduces the same row of the batch, bit for bit
    again = model.prefill(ids[7:8], logits=True, hidden=False, argmax=True)
    assert torch.equal(again["logits"][0], out["logits"][7])
    st["cacheless_z"] = out["logits"][:, 2046:].cpu().numpy()   # positions 2046 and 2047
    del out, again
    torch.cuda.empty_cache()


PREFIX = 256  # positions of rows 1-7 compared with the oracle


def test_llama3_8b_row0_oracle(fwd, llama):
    """The oracle over all 2048 positions of row 0 (a 32-layer host forward)."""
    cfg, host, ids, st = llama["cfg"], llama["host"], llama["ids"], llama["state"]
    _say("  oracle: row 0, all 2048 positions, every slot (host forward, about a minute)")
    st["ref0"] = oracle.forward(cfg, host, ids[:1])


def test_llama3_8b_row0_every_position(fwd, llama):
    """Row 0 at every position and slot against the oracle ("N7 · model/forward-parity",
    Theorem 1: cosine at every slot, argmax at every position). The oracle rounded at
    the bf16 points gives each slot's precision floor and each position's logit
    allowance."""
    cfg, host, ids, st = llama["cfg"], llama["host"], llama["ids"], llama["state"]
    _say("  oracle rounded at the bf16 points: row 0, all 2048 positions (about a minute)")
    refb = oracle.forward(cfg, host, ids[:1], bf16_points=True)
    hid, logits, am = st["row0"]
    ref = st["ref0"]
    pinned, near = _compare(cfg, hid, logits, am, ref, refb, "row 0, all 2048 positions")
    assert pinned + near == 2048
    # the allowance at the decode positions, for the cached-step check below
    st["band_2046"] = oracle_band(ref["logits"], refb["logits"])[2046:].max()
    st["oracle_z"], st["bf16_z"] = ref["logits"][:, 2046], refb["logits"][:, 2046]
    st.pop("row0")


def test_llama3_8b_cached_decode(fwd, llama):
    """Cached session at full size: prefill the first 2046 tokens of every row, then
    decode tokens 2046 and 2047 (teacher-forced) over the 8-chunk cache. Both this and
    the cacheless prefill are bf16 computations that round at different points (the
    cached step keeps the probabilities in fp32), so between them the half-precision
    gate applies, with argmax parity inside twice the oracle-side allowance of row 0 at
    those positions. Row 0 at position 2046 is also compared with the oracle: within the
    floor of the bf16-rounded oracle there."""
    model, ids, st = llama["model"], llama["ids"], llama["state"]
    ref_z = st["cacheless_z"]
    band = 2 * st["band_2046"]
    _say("session: prefill 8 x 2046, decode positions 2046 and 2047")
    sess = fwd.Session(model, max_batch=8, max_seq=2048)
    sess.prefill(ids[:, :2046], logits=False, argmax=False)
    cached = []
    for i, pos in enumerate((2046, 2047)):
        step = sess.decode(ids[:, pos], logits=True, argmax=True)
        z = step["logits"][:, 0].cpu().numpy()
        cached.append(z)
        worst = min(cosine(z[b], ref_z[b, i]) for b in range(8))
        assert worst >= COS_HALF_PRECISION, f"position {pos}: cosine {worst}"
        pinned, near, fails = argmax_check(step["argmax"][:, 0].cpu().numpy(), ref_z[:, i], band)
        assert not fails, fails[:5]
        _say(f"  position {pos}: lowest row cosine cached vs cacheless {worst:.6f}, "
             f"max|d| {np.abs(z - ref_z[:, i]).max():.3e}, argmax pinned {pinned} near-tie {near}")
    sess.close()
    zo, zb = st["oracle_z"], st["bf16_z"]
    floor = cosine(zb, zo)
    c_cached, c_plain = cosine(cached[0][:1], zo), cosine(ref_z[:1, 0], zo)
    _say(f"  row 0 position 2046 vs oracle: cached {c_cached:.6f}, cacheless {c_plain:.6f}, "
         f"bf16-rounded oracle {floor:.6f}")
    for c in (c_cached, c_plain):
        assert (1.0 - c) <= FLOOR_SLACK * (1.0 - floor) + 2e-6, (c, floor)
    pinned, near, fails = argmax_check(np.argmax(cached[0][:1], -1), zo, oracle_band(zo, zb))
    assert not fails, fails


def test_llama3_8b_rows1_7_oracle(fwd, llama):
    cfg, host, ids, st = llama["cfg"], llama["host"], llama["ids"], llama["state"]
    _say(f"  oracle: rows 1-7, first {PREFIX} positions (host forward, about a minute)")
    st["ref17"] = oracle.forward(cfg, host, ids[1:, :PREFIX])


def test_llama3_8b_rows1_7_prefix(fwd, llama):
    cfg, host, ids, st = llama["cfg"], llama["host"], llama["ids"], llama["state"]
    _say(f"  oracle rounded at the bf16 points: rows 1-7, first {PREFIX} positions")
    refb = oracle.forward(cfg, host, ids[1:, :PREFIX], bf16_points=True)
    hid, logits, am = st.pop("rows1_7")
    pinned, near = _compare(cfg, hid, logits, am, st.pop("ref17"), refb, f"rows 1-7 x {PREFIX} positions")
    assert pinned + near == 7 * PREFIX


def test_gemma3_style_full_model(fwd):
    import torch
    cfg = wl.GEMMA3_STYLE
    _say("gemma3-style 48 layers: drawing and uploading 1.18e10 weights")
    model, host = _build(fwd, cfg, 1100)
    ids = wl.draw_ids(cfg, seq=1100)
    # the page's three case lengths (one token, nine tokens, the full window) and S = 1100 > W
    for S in (1, 9):
        _say(f"prefill 1 x {S}")
        out = model.prefill(ids[:, :S], logits=True, hidden=True, argmax=True)
        _compare_sampled(cfg, out, [0], S, host, ids)
        x0 = oracle.embed(host["embed"], ids[:, :S], oracle.embed_scale(cfg.embed_scale_mode, cfg.hidden))
        assert np.array_equal(out["hidden"][0].cpu().numpy(), x0)   # scale 62.0 is exact
    for S in (1024, 1100):
        _say(f"prefill 1 x {S} (window 1024 on 40 local layers)")
        out = model.prefill(ids[:, :S], logits=True, hidden=True, argmax=True)
        torch.cuda.synchronize()
        _whole_output_properties(out)
        assert torch.all(out["logits"].abs() <= 30.0).item()
        _compare_sampled(cfg, out, [0], 12, host, ids)
    model.close()


def test_gemma3_style_window_evicts(fwd):
    """One full 5:1 period (6 layers) at S = 1100 > W = 1024: positions >= 1024 lose
    their oldest keys on the 5 local layers. The oracle runs all 1100 positions; the
    hidden slots take the cosine gates, the logits the window-edge distributional gate
    ("pegainfer issue #878": top-64 log-probabilities, global and per-quarter top-1
    floor, log-probability ceiling), and the window is checked to matter."""
    import torch
    cfg = wl.GEMMA3_STYLE.replace(n_layers=6, layer_kind=wl.GEMMA3_STYLE.layer_kind[:6], name="gemma3-6L")
    _say("gemma3-style 6 layers at 1 x 1100")
    model, host = _build(fwd, cfg, 1100)
    ids = wl.draw_ids(cfg, seq=1100)
    out = model.prefill(ids, logits=True, hidden=True, argmax=True)
    got = out["hidden"].cpu().numpy()
    got_z = out["logits"].cpu().numpy()
    got_am = out["argmax"].cpu().numpy()
    del out
    _say("  oracle, all 1100 positions, 6 layers and the head")
    ref = oracle.forward(cfg, host, ids)
    n, of = GOLD["window_edge_top1_floor"]["value"]
    for name, sl in (("all 1100 positions", slice(None)), ("the 76 evicting positions", slice(1024, None))):
        st = distributional_gate(got_z[:, sl], ref["logits"][:, sl], GOLD["window_edge_top_ids"]["value"],
                                 n / of, GOLD["window_edge_logprob_ceiling"]["value"])
        _say(f"  distributional gate, {name}: top-1 {st['top1']:.4f}, quarters "
             f"{[round(q, 4) for q in st['quarters']]}, max |dlogprob| {st['max_gap']:.3e}")
    _say("  oracle rounded at the bf16 points, all 1100 positions")
    refb = oracle.forward(cfg, host, ids, bf16_points=True)
    band = oracle_band(ref["logits"], refb["logits"])
    pinned, near, fails = argmax_check(got_am, ref["logits"], band)
    assert not fails, fails[:5]
    p_tail, n_tail, _ = argmax_check(got_am[:, 1024:], ref["logits"][:, 1024:], band.reshape(ids.shape)[:, 1024:])
    _say(f"  argmax at all 1100 positions: pinned {pinned} near-tie {near} "
         f"(the 76 evicting positions: pinned {p_tail} near-tie {n_tail})")

    def bf16_slot(s, tail=False):
        h = refb["hidden"][s]
        return h[:, 1024:] if tail else h

    for s in range(cfg.n_layers + 2):
        ok, c, floor = slot_parity(got[s], ref["hidden"][s], lambda s=s: bf16_slot(s))
        assert ok, f"slot {s}: cosine {c} (bf16 floor {floor})"
        ok, c, floor = slot_parity(got[s][:, 1024:], ref["hidden"][s][:, 1024:], lambda s=s: bf16_slot(s, True))
        assert ok, f"slot {s}: cosine past the window {c} (bf16 floor {floor})"
    nowin = oracle.forward(cfg.replace(sliding_window=0), host, ids[:, :1100], want_logits=False)
    delta = np.abs(nowin["hidden"][cfg.n_layers][:, 1024:] - ref["hidden"][cfg.n_layers][:, 1024:]).max()
    assert delta > 1e-3, "the window must change positions past it"
    _say(f"  window effect past position 1024: max|d hidden| {delta:.3e}")
    model.close()
