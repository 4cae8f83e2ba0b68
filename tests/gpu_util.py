"""Helpers shared by the GPU tests and the smoke check: move seeded host arrays to
the device as torch tensors, and compare results. No step of the forward pass."""
from __future__ import annotations

import numpy as np


def to_device(arr: np.ndarray):
    """float32 array -> float32 tensor; uint16 (bf16 bits) -> bfloat16 tensor; on cuda."""
    import torch
    if arr.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(arr)).cuda()


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


def argmax_check(got_ids, ref_logits, got_logits):
    """Argmax parity under the near-tie reading: where the oracle's top-1 margin exceeds
    twice the row's max logit error the id must match exactly; otherwise the GPU id must
    lie within 2 * error of the oracle's max. Returns (n_pinned, n_near_tie, failures)."""
    ref = np.asarray(ref_logits, np.float64).reshape(-1, ref_logits.shape[-1])
    got = np.asarray(got_logits, np.float64).reshape(ref.shape)
    ids = np.asarray(got_ids).ravel()
    pinned = near = 0
    fails = []
    for t in range(ref.shape[0]):
        eps = float(np.max(np.abs(got[t] - ref[t])))
        top2 = np.partition(ref[t], -2)[-2:]
        margin = float(top2[1] - top2[0])
        best = int(np.argmax(ref[t]))
        if margin > 2 * eps:
            pinned += 1
            if ids[t] != best:
                fails.append((t, int(ids[t]), best, margin, eps))
        else:
            near += 1
            if ref[t, ids[t]] < ref[t, best] - 2 * eps:
                fails.append((t, int(ids[t]), best, margin, eps))
    return pinned, near, fails


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
