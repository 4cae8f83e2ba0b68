"""The seeded generator: the C implementation matches its numpy twin, draws are
stateless (any slice can be regenerated), and the distributions are as stated."""
import numpy as np

import synth
from synth import workloads as wl


def test_c_generator_matches_numpy_definition():
    for name, sigma in (("layers.0.wq", 0.02), ("gemm.X.16x64", 1.0)):
        c = synth.normal(7, name, (5000,), sigma, "f32")
        ref = synth.normal_numpy(7, name, 5000, sigma).astype(np.float32)
        assert np.array_equal(c, ref)


def test_bf16_is_round_to_nearest_even_of_f32_draw():
    f = synth.normal(7, "x", (20000,), 0.02, "f32")
    b = synth.normal(7, "x", (20000,), 0.02, "bf16")
    wide = synth.bf16_bits_to_f32(b)
    # nearest: |f - wide| <= half a bf16 ulp of f
    ulp = np.abs(f).view(np.uint32) & 0x7F800000
    half = (ulp.astype(np.uint32) - (8 << 23)).view(np.float32)
    assert np.all(np.abs(f - wide) <= half * (1 + 1e-6))


def test_offsets_regenerate_slices():
    full = synth.normal(7, "slice", (1000,), 1.0, "f32")
    key = synth.key_of(7, "slice")
    part = np.empty(100, np.float32)
    synth._load().synth_normal_f32(key, 500, 100, 1.0, part.ctypes.data)
    assert np.array_equal(part, full[500:600])


def test_normal_and_uniform_statistics():
    x = synth.normal(7, "stats", (200000,), 0.02, "f32").astype(np.float64)
    assert abs(x.mean()) < 3 * 0.02 / np.sqrt(len(x)) * 2
    assert abs(x.std() / 0.02 - 1) < 0.01
    ids = synth.token_ids(99, "ids", 4, 50000, 1000)
    assert ids.min() >= 0 and ids.max() < 1000
    counts = np.bincount(ids.ravel(), minlength=1000)
    chi2 = float(((counts - 200.0) ** 2 / 200.0).sum())
    assert chi2 < 1000 + 5 * np.sqrt(2000)


def test_workload_shapes():
    c = wl.LLAMA3_8B
    shapes = wl.weight_shapes(c)
    assert shapes["layers.0.wq"][0] == (4096, 4096)
    assert shapes["layers.0.wk"][0] == (1024, 4096)
    assert shapes["layers.31.w_down"][0] == (4096, 14336)
    g = wl.GEMMA3_STYLE
    assert g.kinds().count("global") == 8 and g.kinds()[5] == "global" and g.kinds()[0] == "local"
    assert "layers.0.post_ffn_norm" in wl.weight_shapes(g)
