"""Kernel-level parity of the HIP library against the CPU oracle, through the C ABI.

Gates follow the pages' error model ("N9 · metalgemm", Theorem 1): err/scale =
max|d| / max|ref| < 1e-2 for bf16 operands, plus cosine >= 0.9999. Because the GEMM
inputs are bf16-exact and only the fp32 accumulation order differs from the
float64 oracle, the GEMM also meets an internal gate of 1e-5 (one dropped K term
would show as ~1e-3).
"""
import json
import os
import sys

import numpy as np
import pytest

import oracle
import synth
from synth import workloads as wl
from tests.gpu_util import bf16_to_f32, cosine, err_over_scale, to_device

pytestmark = pytest.mark.gpu
GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page_values.json")))
PAGE_BOUND = GOLD["gemm_err_over_scale_max"]["value"]


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


# ------------------------------------------------------------------ GEMM
SMALL_SHAPES = [tuple(s) for s in GOLD["gemm_shapes_P_in_out"]["value"]] + [
    (1, 64, 96), (7, 576, 960), (300, 576, 576), (513, 1536, 3072), (100, 8, 24), (33, 4104, 200),
    # 320 tiles of 256 x 256 on the row-major 64-wide-slice kernel, ragged in rows, columns and K
    (2000, 96, 10000)]


@pytest.mark.parametrize("P,K,N", SMALL_SHAPES)
def test_gemm_bf16_matches_oracle(fwd, P, K, N):
    _say(f"gemm bf16 P={P} in={K} out={N}")
    X, W = wl.draw_gemm(P, K, N)
    Y = fwd.gemm(to_device(X), to_device(W)).cpu().numpy()
    ref = oracle.gemm(synth.bf16_bits_to_f32(X), synth.bf16_bits_to_f32(W))
    e = err_over_scale(Y, ref)
    assert e < PAGE_BOUND and e < 1e-5, e


@pytest.mark.parametrize("P,K,N", [(16, 64, 96), (16, 172, 64), (5, 4, 7), (130, 68, 190)])
def test_gemm_f32_matches_oracle(fwd, P, K, N):
    _say(f"gemm f32 P={P} in={K} out={N}")
    X = synth.normal(0x1234567, f"f32.X.{P}x{K}", (P, K), 1.0, "f32")
    W = synth.normal(0x1234567, f"f32.W.{N}x{K}", (N, K), 1.0, "f32")
    Y = fwd.gemm(to_device(X), to_device(W)).cpu().numpy()
    ref = oracle.gemm(X, W)
    assert err_over_scale(Y, ref) < 1e-6


@pytest.mark.parametrize("P,K,N", [(4096, 4096, 14336), (8192, 4096, 128256)])
def test_gemm_bf16_large_sampled_rows(fwd, P, K, N):
    """Full-size launch; the oracle recomputes a sample of rows (incl. first/last)."""
    import torch
    _say(f"gemm bf16 large P={P} in={K} out={N}")
    X, W = wl.draw_gemm(P, K, N)
    Xd, Wd = to_device(X), to_device(W)
    Y = fwd.gemm(Xd, Wd)
    rows = np.unique(np.concatenate([[0, 1, P - 1], np.random.default_rng(5).integers(0, P, 13)]))
    got = Y[torch.as_tensor(rows, device=Y.device)].cpu().numpy()
    assert torch.isfinite(Y).all().item()
    ref = oracle.gemm(synth.bf16_bits_to_f32(X[rows]), synth.bf16_bits_to_f32(W))
    e = err_over_scale(got, ref)
    assert e < PAGE_BOUND and e < 1e-5, e


def test_gemm_rejects_bad_arguments(fwd):
    import torch
    X = torch.zeros((4, 7), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(fwd.FwdError) as e:
        fwd.gemm(X, X)
    assert e.value.code == fwd.FWD_E_ARG


# ------------------------------------------------------------------ RMSNorm
@pytest.mark.parametrize("rows,H,dt", [(1, 64, "f32"), (37, 576, "bf16"), (300, 4096, "bf16"), (5, 3840, "bf16"),
                                       (16, 64, "f32"),
                                       # more rows than the capped grid has wavefronts: grid-stride rows
                                       (9001, 576, "bf16")])
def test_rmsnorm_matches_oracle(fwd, rows, H, dt):
    _say(f"rmsnorm rows={rows} H={H} {dt}")
    x = synth.normal(11, f"rms.x.{rows}.{H}", (rows, H), 1.5, "f32")
    w = synth.normal(11, f"rms.w.{H}", (H,), 1.0, "f32")
    y = fwd.rmsnorm(to_device(x), to_device(w), 1e-5, dt)
    got = bf16_to_f32(y) if dt == "bf16" else y.cpu().numpy()
    ref = oracle.rmsnorm(x, w, 1e-5)
    tol = 2.0 ** -8 if dt == "bf16" else 2e-6
    assert np.all(np.abs(got - ref) <= tol * np.abs(ref) + 1e-6)


# ------------------------------------------------------------------ attention
def _attn_inputs(B, S, Hq, Hkv, D, dt, seed=3):
    tag = f"attn.{B}.{S}.{Hq}.{Hkv}.{D}"
    q = synth.normal(seed, tag + ".q", (B, S, Hq, D), 1.0, dt)
    k = synth.normal(seed, tag + ".k", (B, S, Hkv, D), 1.0, dt)
    v = synth.normal(seed, tag + ".v", (B, S, Hkv, D), 1.0, dt)
    return q, k, v


def _vt(v):
    """values transposed to [B, Hkv, D, Sp] with Sp = S rounded up to 8; the padding holds
    a large finite value (bf16 / f32 1000.0) that must not leak into the output."""
    B, S, Hkv, D = v.shape
    Sp = (S + 7) // 8 * 8
    out = np.full((B, Hkv, D, Sp), 0x447A if v.dtype == np.uint16 else 1000.0, dtype=v.dtype)
    out[..., :S] = np.transpose(v, (0, 2, 3, 1))
    return out


ATTN_CASES = [
    # B, S, Hq, Hkv, D, window
    (1, 1, 4, 2, 64, 0), (2, 9, 9, 3, 64, 0), (1, 100, 4, 4, 64, 0), (1, 257, 8, 2, 128, 0),
    (2, 130, 32, 8, 128, 0), (1, 300, 4, 1, 128, 64), (1, 97, 2, 1, 256, 0), (1, 200, 16, 8, 256, 33),
    (1, 64, 2, 2, 64, 4), (1, 65, 2, 1, 64, 64), (1, 65, 2, 1, 64, 65), (1, 65, 2, 1, 64, 66),
    (1, 1536, 3, 1, 64, 256),
    (1, 1100, 16, 8, 256, 1024), (1, 2048, 2, 1, 128, 0),
    # many heads: grids of 512 or more workgroups, as in the large forwards
    (2, 256, 128, 16, 64, 0), (1, 512, 128, 16, 128, 100), (1, 384, 176, 16, 256, 0),
    # heads x 256-query blocks >= 512: two 32-query tiles per wavefront at D = 64
    (4, 256, 128, 16, 64, 0), (2, 512, 128, 16, 128, 0), (2, 500, 128, 16, 128, 100),
]


@pytest.mark.parametrize("B,S,Hq,Hkv,D,W", ATTN_CASES)
def test_attention_bf16_matches_oracle(fwd, B, S, Hq, Hkv, D, W):
    _say(f"attention bf16 B={B} S={S} Hq={Hq} Hkv={Hkv} D={D} W={W}")
    q, k, v = _attn_inputs(B, S, Hq, Hkv, D, "bf16")
    o = fwd.attention(to_device(q), to_device(k), to_device(_vt(v)), window=W)
    got = bf16_to_f32(o)
    f = synth.bf16_bits_to_f32
    ref = oracle.attention(f(q), f(k), f(v), W)
    assert np.isfinite(got).all()
    assert err_over_scale(got, ref) < PAGE_BOUND
    assert cosine(got, ref) >= 0.9999


@pytest.mark.parametrize("B,S,Hq,Hkv,D,W", [(1, 16, 4, 2, 16, 0), (2, 16, 4, 2, 16, 4), (1, 70, 2, 1, 32, 0),
                                            (1, 5, 2, 2, 64, 0)])
def test_attention_f32_matches_oracle(fwd, B, S, Hq, Hkv, D, W):
    _say(f"attention f32 B={B} S={S} Hq={Hq} Hkv={Hkv} D={D} W={W}")
    q, k, v = _attn_inputs(B, S, Hq, Hkv, D, "f32")
    o = fwd.attention(to_device(q), to_device(k), to_device(_vt(v)), window=W)
    ref = oracle.attention(q, k, v, W)
    assert err_over_scale(o.cpu().numpy(), ref) < 1e-5


def test_bf16_output_rounding_is_nearest_even(fwd):
    """rows of +-0.5 with eps = 0.75 give mean(x^2) + eps = 1 exactly, so y = x * w is
    exact in fp32 and the stored bf16 must be its round-to-nearest-even value."""
    rows, H = 64, 256
    rng = np.random.default_rng(9)
    x = np.where(rng.random((rows, H)) < 0.5, -0.5, 0.5).astype(np.float32)
    w = rng.standard_normal(H).astype(np.float32)
    w[:4] = np.array([1 + 2 ** -8, 1 + 3 * 2 ** -8, 1 + 2 ** -9, -(1 + 2 ** -8)], np.float32)  # ties / halfway
    y = bf16_to_f32(fwd.rmsnorm(to_device(x), to_device(w), 0.75, "bf16"))
    exact = x * w                                   # exact products of 0.5 and w
    u = exact.view(np.uint32).astype(np.uint64)
    rne = (((u + 0x7FFF + ((u >> 16) & 1)) >> 16) << 16).astype(np.uint32).view(np.float32)
    assert np.array_equal(y, rne)
