"""Host-side checks of the C ABI (no GPU needed): the library loads, exports every
entry point include/fwd.h declares, validates configurations, and refuses to run
compute without a gfx950 device instead of falling back to anything."""
import ctypes
import math
import os
import re

import numpy as np
import pytest

from decoder_only_transformer_bf16_amd import fwd
from synth import workloads as wl

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = open(os.path.join(ROOT, "include", "fwd.h")).read()


def _declared():
    return sorted(set(re.findall(r"^\s*(?:int|int32_t|void|const char\*)\s+(fwd_\w+)\s*\(", HEADER, re.M)))


def test_header_declares_the_binding_exports():
    assert _declared() == sorted(fwd.EXPORTS)


def test_library_exports_every_declared_symbol():
    L = fwd.lib()
    for name in _declared():
        assert hasattr(L, name), name


def _c_layout(struct, fields):
    """(sizeof, [offsetof ...]) of a header struct, from a C program compiled against fwd.h."""
    import shutil
    import subprocess
    import tempfile
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no C compiler")
    src = "#include <stdio.h>\n#include <stddef.h>\n#include \"fwd.h\"\nint main(void) {\n"
    src += f'  printf("%zu\\n", sizeof({struct}));\n'
    for f in fields:
        src += f'  printf("%zu\\n", offsetof({struct}, {f}));\n'
    src += "  return 0;\n}\n"
    with tempfile.TemporaryDirectory() as d:
        c_path, exe = os.path.join(d, "layout.c"), os.path.join(d, "layout")
        open(c_path, "w").write(src)
        subprocess.run([cc, "-I", os.path.join(ROOT, "include"), c_path, "-o", exe], check=True)
        out = [int(v) for v in subprocess.run([exe], stdout=subprocess.PIPE, check=True).stdout.split()]
    return out[0], out[1:]


@pytest.mark.parametrize("struct,ctype", [("fwd_config", "FwdConfig"), ("fwd_layer_weights", "FwdLayerWeights"),
                                          ("fwd_weights", "FwdWeights"), ("fwd_outputs", "FwdOutputs"),
                                          ("fwd_sizes", "FwdSizes")])
def test_struct_layouts_match_header(struct, ctype):
    cls = getattr(fwd, ctype)
    names = [f for f, _ in cls._fields_]
    size, offsets = _c_layout(struct, names)
    assert size == ctypes.sizeof(cls)
    assert offsets == [getattr(cls, f).offset for f in names]


def test_no_device_here_means_unavailable_not_fallback():
    if fwd.available():
        pytest.skip("a gfx950 device is visible")
    cfg, keep = fwd.make_config(wl.TINY_F32, 16)
    w = fwd.FwdWeights(embed=1, final_norm=1, layers=None)
    cfg0, keep0 = fwd.make_config(wl.TINY_F32.replace(n_layers=0), 16)
    h = fwd.c_vp()
    assert fwd.lib().fwd_create(ctypes.byref(cfg0), ctypes.byref(w), None, ctypes.byref(h)) == fwd.FWD_E_UNAVAILABLE
    assert not h.value
    # non-null (never dereferenced) pointers: the device check comes before any access
    assert fwd.lib().fwd_gemm(16, 16, 16, 4, 8, 4, fwd.DTYPE["bf16"], None) == fwd.FWD_E_UNAVAILABLE
    assert b"gfx950" in fwd.lib().fwd_last_error()


def _create_rc(cfg, max_tokens=16):
    c, keep = fwd.make_config(cfg, max_tokens)
    s = fwd.FwdSizes()
    return fwd.lib().fwd_output_sizes(ctypes.byref(c), 1, 16, ctypes.byref(s))


@pytest.mark.parametrize("bad", [
    dict(final_logit_softcap=-1.0), dict(final_logit_softcap=float("nan")), dict(final_logit_softcap=float("inf")),
    dict(n_kv_heads=3), dict(head_dim=24), dict(rms_eps=0.0), dict(rope_theta=1.0), dict(sliding_window=-1),
    dict(dtype="bf16"),  # tiny geometry is not a supported bf16 shape (head_dim 16)
    dict(rope_theta_local=0.5),
    dict(rope_scaling="llama3", rope_factor=8.0, rope_original_max_pos=0),
    dict(rope_scaling="llama3", rope_factor=8.0, rope_original_max_pos=64, rope_low_freq_factor=4.0,
         rope_high_freq_factor=1.0),
    dict(rope_scaling="llama3", rope_factor=0.0, rope_original_max_pos=64),
    dict(rope_scaling="longrope", rope_factor=2.0, rope_original_max_pos=64),  # no factor arrays
    dict(rope_scaling="longrope", rope_factor=2.0, rope_original_max_pos=64,
         rope_short_factor=(1.0,) * 7 + (0.0,), rope_long_factor=(2.0,) * 8),
])
def test_bad_configs_are_rejected(bad):
    assert _create_rc(wl.TINY_F32.replace(**bad)) == fwd.FWD_E_CONFIG


@pytest.mark.parametrize("field,value", [("qk_norm", 2), ("norm_gain_offset", -1), ("ffn_act", 7),
                                         ("rope_scaling", 9)])
def test_out_of_range_variant_fields_are_rejected(field, value):
    c, keep = fwd.make_config(wl.TINY_F32, 16)
    setattr(c, field, value)
    s = fwd.FwdSizes()
    assert fwd.lib().fwd_output_sizes(ctypes.byref(c), 1, 16, ctypes.byref(s)) == fwd.FWD_E_CONFIG


def test_variant_configs_are_accepted():
    for kw in (dict(qk_norm=True, norm_gain_offset=1, ffn_act="gelu_tanh", rope_theta_local=1e4,
                    layer_kind=("local", "global")),
               dict(rope_scaling="llama3", rope_factor=8.0, rope_original_max_pos=64),
               dict(rope_scaling="longrope", rope_factor=2.0, rope_original_max_pos=64,
                    rope_short_factor=(1.0,) * 8, rope_long_factor=(2.0,) * 8)):
        assert _create_rc(wl.TINY_F32.replace(**kw)) == fwd.FWD_OK, kw


def test_output_sizes_are_the_one_source_of_truth():
    for cfg in wl.MODELS.values():
        s = fwd.output_sizes(cfg, cfg.batch, cfg.seq)
        T = cfg.batch * cfg.seq
        assert s["logits_elems"] == T * cfg.vocab
        assert s["hidden_elems"] == (cfg.n_layers + 2) * T * cfg.hidden
        assert s["argmax_elems"] == T
        n_weights = sum(int(np.prod(shape)) for shape, kind in wl.weight_shapes(cfg).values() if kind == "matrix")
        esize = 2 if cfg.dtype == "bf16" else 4
        assert s["weight_bytes"] >= n_weights * esize
    with pytest.raises(fwd.FwdError) as e:
        fwd.output_sizes(wl.TINY_F32, -1, 4)
    assert e.value.code == fwd.FWD_E_ARG


def test_null_handle_and_empty_calls():
    L = fwd.lib()
    assert L.fwd_prefill(None, None, 1, 1, None) == fwd.FWD_E_ARG
    L.fwd_destroy(None)
    # empty problems are no-ops even without a device
    assert L.fwd_gemm(None, None, None, 0, 8, 4, fwd.DTYPE["bf16"], None) == fwd.FWD_OK
    assert L.fwd_gemm(None, None, None, 4, 7, 4, fwd.DTYPE["bf16"], None) == fwd.FWD_E_ARG


def test_session_entry_points_reject_null_handles():
    L = fwd.lib()
    h = ctypes.c_void_p()
    assert L.fwd_session_create(None, 1, 16, ctypes.byref(h)) == fwd.FWD_E_ARG
    assert not h.value
    assert L.fwd_session_create(None, 1, 16, None) == fwd.FWD_E_ARG
    ids = np.zeros(4, dtype=np.int32)
    out = fwd.FwdOutputs()
    assert L.fwd_session_prefill(None, ids.ctypes.data, 1, 4, ctypes.byref(out)) == fwd.FWD_E_ARG
    assert L.fwd_session_decode(None, ids.ctypes.data, ctypes.byref(out)) == fwd.FWD_E_ARG
    assert L.fwd_session_length(None) == -1
    L.fwd_session_destroy(None)
