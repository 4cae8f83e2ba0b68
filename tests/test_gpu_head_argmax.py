"""Per-position argmax folded into the tied LM head's epilogue (bf16, more than 64 rows).

Gates ("N7 · model/forward-parity", Theorem 1: per-position argmax; "pegainfer issue
#878", Acceptance Criteria: lowest index on ties, any non-finite logit fails the call):
- exact ties planted by duplicating embedding rows resolve to the lowest index, in
  both the 128 x 128 and the 256 x 256 tile configurations of the head product;
- the argmax-only call (no logits written) returns the same ids as the call that also
  writes logits, and those ids are the first maximum of the written logits;
- the ids agree with the oracle wherever its top-1 margin pins them;
- a single non-finite logit column raises FWD_E_NONFINITE;
- a vocabulary that ends inside a tile and a row count just past a tile boundary
  (ragged edges of the head product and of its argmax chunks).
"""
import sys

import numpy as np
import pytest

import oracle
from synth import workloads as wl
from tests.gpu_util import argmax_check, band_for, upload_weights

pytestmark = pytest.mark.gpu


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


def _duplicated_head(cfg):
    """Weights whose embedding rows [V/2, V) repeat rows [0, V/2): every logit column
    v >= V/2 equals column v - V/2, so the lowest-index rule must pick the lower half."""
    host = wl.draw_all(cfg)
    E = host["embed"].copy()
    half = cfg.vocab // 2
    E[half:2 * half] = E[:half]
    host["embed"] = E
    return host


@pytest.mark.parametrize("seq", [100, 300])  # head grid of 192 and 384 tiles of 256 x 256
def test_planted_ties_take_lowest_index(fwd, seq):
    cfg = wl.SMOLLM2_135M.replace(n_layers=2, batch=1, seq=seq, name=f"smol-2L-ties-{seq}")
    _say(f"head argmax planted ties: {cfg.name}")
    host = _duplicated_head(cfg)
    ids = wl.draw_ids(cfg)
    model = fwd.Model(cfg, upload_weights(cfg, host), max_tokens=ids.size)
    out = model.prefill(ids, logits=True, argmax=True)
    z = out["logits"].cpu().numpy()[0]
    am = out["argmax"].cpu().numpy()[0]
    half = cfg.vocab // 2
    top = z.max(-1)
    tied = (z[:, :half] == top[:, None]) & (z[:, half:2 * half] == top[:, None])
    assert tied.any(-1).all(), "every row's maximum should occur in both halves"
    assert np.array_equal(am, np.argmax(z, -1)), "argmax must be the first maximum of the logits"
    assert (am < half).all()
    only = model.prefill(ids, logits=False, argmax=True)["argmax"].cpu().numpy()[0]
    assert np.array_equal(only, am), "argmax-only call must match the call that writes logits"
    ref = oracle.forward(cfg, wl.HostWeights(host), ids, want_hidden=False)
    pinned, near, fails = argmax_check(am[None], ref["logits"], band_for(cfg, wl.HostWeights(host), ids, ref["logits"]))
    assert not fails, fails[:5]
    _say(f"  pinned {pinned} near-tie {near}")
    model.close()


def test_argmax_only_matches_full_outputs(fwd):
    cfg = wl.SMOLLM2_135M.replace(n_layers=3, batch=2, seq=257, name="smol-3L-2x257")
    _say(f"head argmax, argmax-only vs full outputs: {cfg.name}")
    host = wl.draw_all(cfg)
    ids = wl.draw_ids(cfg)
    model = fwd.Model(cfg, upload_weights(cfg, host), max_tokens=ids.size)
    full = model.prefill(ids, logits=True, hidden=True, argmax=True)
    z = full["logits"].cpu().numpy()
    am = full["argmax"].cpu().numpy()
    assert np.array_equal(am, np.argmax(z, -1))
    only = model.prefill(ids, logits=False, argmax=True)["argmax"].cpu().numpy()
    assert np.array_equal(only, am)
    # a prefix of 65 tokens (still above the few-row limit) reproduces those positions' ids
    pre = model.prefill(ids[:, :65], logits=False, argmax=True)["argmax"].cpu().numpy()
    assert np.array_equal(pre, am[:, :65])
    model.close()


def test_single_nonfinite_column_fails(fwd):
    cfg = wl.SMOLLM2_135M.replace(n_layers=1, batch=1, seq=96, name="smol-1L-inf")
    _say(f"head argmax non-finite column: {cfg.name}")
    host = wl.draw_all(cfg)
    ids = wl.draw_ids(cfg)
    v = int(np.setdiff1d(np.arange(1000, 2000), ids)[0])  # a column no input token embeds
    E = host["embed"].copy()
    E[v] = np.uint16(0x7F7F)  # bf16 3.39e38: the dot product overflows
    host["embed"] = E
    model = fwd.Model(cfg, upload_weights(cfg, host), max_tokens=ids.size)
    with pytest.raises(fwd.FwdError) as e:
        model.prefill(ids, logits=False, argmax=True)
    assert e.value.code == fwd.FWD_E_NONFINITE
    with pytest.raises(fwd.FwdError) as e:
        model.prefill(ids, logits=True, argmax=True)
    assert e.value.code == fwd.FWD_E_NONFINITE
    model.close()


@pytest.mark.parametrize("vocab,seq", [(1000, 257), (4097, 96), (40001, 257)])  # 128 x 128, 128 x 128, 256 x 256 tiles
def test_ragged_vocab_and_rows(fwd, vocab, seq):
    cfg = wl.SMOLLM2_135M.replace(n_layers=1, batch=1, seq=seq, vocab=vocab, name=f"smol-1L-v{vocab}-s{seq}")
    _say(f"head argmax ragged edges: {cfg.name}")
    host = wl.draw_all(cfg)
    ids = wl.draw_ids(cfg)
    model = fwd.Model(cfg, upload_weights(cfg, host), max_tokens=ids.size)
    out = model.prefill(ids, logits=True, argmax=True)
    z = out["logits"].cpu().numpy()
    am = out["argmax"].cpu().numpy()
    assert np.isfinite(z).all()
    assert np.array_equal(am, np.argmax(z, -1))
    only = model.prefill(ids, logits=False, argmax=True)["argmax"].cpu().numpy()
    assert np.array_equal(only, am)
    ref = oracle.forward(cfg, wl.HostWeights(host), ids, want_hidden=False)
    err = float(np.max(np.abs(z - ref["logits"])) / np.max(np.abs(ref["logits"])))
    assert err < 1e-2, err
    pinned, near, fails = argmax_check(am, ref["logits"], band_for(cfg, wl.HostWeights(host), ids, ref["logits"]))
    assert not fails, fails[:5]
    _say(f"  err/scale {err:.2e}, pinned {pinned} near-tie {near}")
    model.close()
