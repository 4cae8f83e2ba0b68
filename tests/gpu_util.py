"""Helpers shared by the GPU tests and the smoke check: move seeded host arrays to
the device as torch tensors, and compare results. No step of the forward pass."""
from __future__ import annotations

import numpy as np


def to_device(arr: np.ndarray):
    """float32 array -> float32 tensor; uint16 (bf16 bits) -> bfloat16 tensor; on cuda."""
    from decoder_only_transformer_bf16_amd import fwd
    return fwd.to_device(arr)


def upload_weights(cfg, host: dict) -> dict:
    return {n: to_device(a) for n, a in host.items()}


def bf16_to_f32(t) -> np.ndarray:
    """bfloat16 tensor -> float32 numpy (exact widening on the host)."""
    import torch
    bits = t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    return (bits.astype(np.uint32) << 16).view(np.float32)


def cosine(a, b) -> float:
    a = np.asarray(a, np.float64).ravel()
    b = np.asarray(b, np.float64).ravel()
    return float(a @ b / (np.linalg.norm(a) * np.linalg.norm(b)))


def err_over_scale(got, ref) -> float:
    """max|got - ref| / max|ref| ("N9 · metalgemm", Theorem 1 error model)."""
    ref = np.asarray(ref, np.float64)
    return float(np.max(np.abs(np.asarray(got, np.float64) - ref)) / np.max(np.abs(ref)))


# Allowed logit error of the fp32 path: ~100x the fp32 rounding of these dot products
# (observed 1e-6 and below), far inside the pages' 0.05 fp32 logit gate.
F32_LOGIT_BAND = 1e-4


def oracle_band(ref_logits, ref_bf16_logits=None, slack: float = None):
    """Per-position allowed logit error, fixed by the oracle alone (never by the GPU's
    result): for a bf16 computation, `slack` times the largest deviation over the
    vocabulary of the oracle rounded at the GPU's bf16 points from the exact oracle at
    that position; for the fp32 path (ref_bf16_logits None), F32_LOGIT_BAND."""
    r = np.asarray(ref_logits, np.float64)
    r = r.reshape(-1, r.shape[-1])
    if ref_bf16_logits is None:
        return np.full(r.shape[0], F32_LOGIT_BAND)
    b = np.asarray(ref_bf16_logits, np.float64).reshape(r.shape)
    return (FLOOR_SLACK if slack is None else slack) * np.max(np.abs(b - r), axis=-1)


def argmax_check(got_ids, ref_logits, band):
    """Argmax parity under the near-tie reading ("N7 · model/forward-parity", Theorem 1:
    the argmax the oracle pins). band[t] is the allowed logit error at position t (from
    oracle_band, or a scalar). Where the oracle's top-1 margin exceeds 2 band[t] the GPU
    id must equal the oracle's; otherwise (a near tie) it must lie within 2 band[t] of
    the oracle's maximum. Returns (n_pinned, n_near_tie, failures)."""
    ref = np.asarray(ref_logits, np.float64)
    ref = ref.reshape(-1, ref.shape[-1])
    ids = np.asarray(got_ids).ravel()
    band = np.asarray(band, np.float64)
    band = np.full(ref.shape[0], float(band)) if band.ndim == 0 else band.reshape(-1)
    if band.shape != (ref.shape[0],):  # one value per position (a logits array is not a band)
        raise ValueError(f"band of {band.size} values for {ref.shape[0]} positions")
    assert ids.shape == (ref.shape[0],)
    pinned = near = 0
    fails = []
    for t in range(ref.shape[0]):
        top2 = np.partition(ref[t], -2)[-2:]
        margin = float(top2[1] - top2[0])
        best = int(np.argmax(ref[t]))
        if margin > 2 * band[t]:
            pinned += 1
            if ids[t] != best:
                fails.append((t, int(ids[t]), best, margin, float(band[t])))
        else:
            near += 1
            if ref[t, ids[t]] < ref[t, best] - 2 * band[t]:
                fails.append((t, int(ids[t]), best, margin, float(band[t])))
    return pinned, near, fails


def band_for(cfg, host, ids, ref_logits):
    """oracle_band of a forward over `ids`: for bf16 configurations the oracle is run
    again, rounded at the bf16 points (host: name -> float32 weights)."""
    if cfg.dtype != "bf16":
        return oracle_band(ref_logits)
    import oracle
    refb = oracle.forward(cfg, host, ids, want_hidden=False, bf16_points=True)
    return oracle_band(ref_logits, refb["logits"])


def logit_band_check(got_logits, ref_logits, band):
    """The GPU's logits within the oracle-side allowance: the largest |d logit| over the
    compared positions must not exceed the largest band over them (a per-position match
    of the rounding noise is not expected). Returns (max |d|, max band)."""
    ref = np.asarray(ref_logits, np.float64)
    ref = ref.reshape(-1, ref.shape[-1])
    d = float(np.max(np.abs(np.asarray(got_logits, np.float64).reshape(ref.shape) - ref)))
    return d, float(np.max(band))


COS_PRIMARY = 0.9999        # "N7 · model/forward-parity", Theorem 1 proof (f32 forward vs f32 reference)
COS_HALF_PRECISION = 0.999  # "N9 · metalgemm", Theorem 1 proof (half-precision device forward vs CPU reference)
FLOOR_SLACK = 1.25


def slot_parity(got, ref, ref_bf16_fn):
    """Hidden-slot gate. Primary: cosine >= 0.9999 against the float64 oracle. Where
    bf16 operands cannot reach that (deep configurations), the slot must instead be
    no farther from the oracle than FLOOR_SLACK times the distance of the oracle
    itself rounded to bf16 at the GPU's rounding points (ref_bf16_fn() -> that slot),
    and never below the pages' half-precision gate of 0.999. Returns (ok, cos, floor)."""
    c = cosine(got, ref)
    if c >= COS_PRIMARY:
        return True, c, None
    floor = cosine(ref_bf16_fn(), ref)
    ok = c >= COS_HALF_PRECISION and (1.0 - c) <= FLOOR_SLACK * (1.0 - floor) + 2e-6
    return ok, c, floor


def distributional_gate(got_logits, ref_logits, top: int, top1_floor: float, logprob_ceiling: float):
    """Window-edge gate of "pegainfer issue #878" (Description, Proposed Plan): log-
    probabilities compared at the reference's top-`top` ids per position, a global
    top-1 agreement floor, the same floor on each quarter of the positions (a failed
    quarter cannot hide inside a passing global rate) and a ceiling on the largest
    log-probability gap. Non-finite values fail outright. Returns the statistics;
    raises AssertionError when a gate fails."""
    g = np.asarray(got_logits, np.float64).reshape(-1, np.shape(got_logits)[-1])
    r = np.asarray(ref_logits, np.float64).reshape(-1, np.shape(ref_logits)[-1])
    assert np.isfinite(g).all() and np.isfinite(r).all(), "non-finite logits"

    def log_softmax(z):
        m = z.max(-1, keepdims=True)
        return z - m - np.log(np.exp(z - m).sum(-1, keepdims=True))

    lg, lr = log_softmax(g), log_softmax(r)
    ids = np.argsort(-r, axis=-1, kind="stable")[:, :top]
    gap = np.abs(np.take_along_axis(lg, ids, -1) - np.take_along_axis(lr, ids, -1))
    agree = np.argmax(g, -1) == np.argmax(r, -1)
    quarters = [float(q.mean()) for q in np.array_split(agree, 4)]
    stats = {"top1": float(agree.mean()), "quarters": quarters, "max_gap": float(gap.max())}
    assert stats["top1"] >= top1_floor, stats
    assert min(quarters) >= top1_floor, stats
    assert stats["max_gap"] <= logprob_ceiling, stats
    return stats
