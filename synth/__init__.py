"""Seeded synthetic inputs shared by the tests, the smoke check and the benchmark.

Both sides of every parity check (the CPU oracle and the HIP library) consume
arrays drawn here; neither side imports the other. This module holds no step of
the transformer's arithmetic: it draws normal and uniform numbers from a
stateless counter-based generator (``synth.c``) and describes workload shapes.

Generator (also implemented in numpy below for cross-checking small draws):
element ``i`` of stream ``(seed, tag)`` is splitmix64 output ``i`` from state
``mix64(seed ^ mix64(tag))``; two 32-bit halves feed a Box-Muller transform.
``tag`` is the 64-bit FNV-1a hash of the tensor's name.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import sys

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "synth.c")
_LIB = os.path.join(_HERE, "libsynth.so")
_lib = None

SEED_WEIGHTS = 7          # rand source 7 on the metalgemm page (Theorem 1)
SEED_IDS = 99             # lcg seed 99, same passage
SEED_GEMM = 0x1234567     # lcg seed 0x1234567, same passage
WEIGHT_SIGMA = 0.02


def build(force: bool = True) -> str:
    """Compile libsynth.so with gcc (OpenMP); returns its path."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        cmd = ["gcc", "-O3", "-fopenmp", "-fPIC", "-shared", "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=False)
        lib = ctypes.CDLL(_LIB)
        u64, i64, i32, dbl = ctypes.c_uint64, ctypes.c_int64, ctypes.c_int32, ctypes.c_double
        p = ctypes.c_void_p
        lib.synth_key.restype = u64
        lib.synth_key.argtypes = [u64, u64]
        lib.synth_bits.argtypes = [u64, u64, i64, p]
        lib.synth_normal_f32.argtypes = [u64, u64, i64, dbl, p]
        lib.synth_normal_bf16.argtypes = [u64, u64, i64, dbl, p]
        lib.synth_ids.argtypes = [u64, u64, i64, i32, p]
        _lib = lib
    return _lib


def tag_of(name: str) -> int:
    """64-bit FNV-1a hash of a tensor name."""
    h = 0xCBF29CE484222325
    for b in name.encode("ascii"):
        h ^= b
        h = (h * 0x100000001B3) & 0xFFFFFFFFFFFFFFFF
    return h


def key_of(seed: int, name: str) -> int:
    return int(_load().synth_key(seed & 0xFFFFFFFFFFFFFFFF, tag_of(name)))


def normal(seed: int, name: str, shape, sigma: float, dtype: str, offset: int = 0) -> np.ndarray:
    """N(0, sigma^2) draw of ``shape``; dtype 'f32' -> float32, 'bf16' -> uint16 bf16 bits."""
    n = int(np.prod(shape)) if len(shape) else 1
    key = key_of(seed, name)
    lib = _load()
    if dtype == "f32":
        out = np.empty(n, dtype=np.float32)
        lib.synth_normal_f32(key, offset, n, float(sigma), out.ctypes.data)
    elif dtype == "bf16":
        out = np.empty(n, dtype=np.uint16)
        lib.synth_normal_bf16(key, offset, n, float(sigma), out.ctypes.data)
    else:
        raise ValueError(f"dtype {dtype!r}")
    return out.reshape(shape)


def token_ids(seed: int, name: str, batch: int, seq: int, vocab: int) -> np.ndarray:
    """int32 [batch, seq] ids, uniform in [0, vocab)."""
    n = batch * seq
    out = np.empty(n, dtype=np.int32)
    _load().synth_ids(key_of(seed, name), 0, n, int(vocab), out.ctypes.data)
    return out.reshape(batch, seq)


def raw_bits(seed: int, name: str, n: int, offset: int = 0) -> np.ndarray:
    out = np.empty(n, dtype=np.uint64)
    _load().synth_bits(key_of(seed, name), offset, n, out.ctypes.data)
    return out


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> uint16 bf16 bits, round to nearest, ties to even (finite inputs)."""
    u = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to float32."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


# --- numpy re-implementation of the same generator, for cross-checking small draws ---

_M64 = np.uint64(0xFFFFFFFFFFFFFFFF)


def _mix64_np(z: np.ndarray) -> np.ndarray:
    with np.errstate(over="ignore"):
        z = (z ^ (z >> np.uint64(30))) * np.uint64(0xBF58476D1CE4E5B9)
        z = (z ^ (z >> np.uint64(27))) * np.uint64(0x94D049BB133111EB)
        return z ^ (z >> np.uint64(31))


def normal_numpy(seed: int, name: str, n: int, sigma: float, offset: int = 0) -> np.ndarray:
    """float64 values before the f32/bf16 rounding (slow path, small n only)."""
    tag = np.array([tag_of(name)], dtype=np.uint64)
    key = _mix64_np(np.array([seed], dtype=np.uint64) ^ _mix64_np(tag))[0]
    i = np.arange(offset, offset + n, dtype=np.uint64)
    with np.errstate(over="ignore"):
        b = _mix64_np(key + (i + np.uint64(1)) * np.uint64(0x9E3779B97F4A7C15))
    u1 = ((b >> np.uint64(32)).astype(np.float64) + 0.5) * 2.0 ** -32
    u2 = ((b & np.uint64(0xFFFFFFFF)).astype(np.float64) + 0.5) * 2.0 ** -32
    return sigma * np.sqrt(-2.0 * np.log(u1)) * np.cos(2.0 * np.pi * u2)
