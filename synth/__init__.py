"""Seeded synthetic inputs for the int4 routed-expert MoE layer.

Harness code: the tests, the benchmark and the oracle's callers draw their
inputs here.  Nothing in this package computes any part of the layer; it makes
random bytes, normals and fp16/bf16 encodings (see ``gen.c``), and knows the
shapes of the five workloads (``configs.py``).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SO = os.path.join(_HERE, "libsynth.so")
_lib = None

T_X, T_XNOISE, T_WR, T_NIB, T_SCALE, T_H0 = 1, 2, 3, 4, 5, 6
SCALE_LO, SCALE_HI = 0.005, 0.02


def build(force: bool = False) -> str:
    """Compile gen.c into libsynth.so (gcc, OpenMP)."""
    if force or not os.path.exists(_SO):
        tmp = _SO + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-fPIC", "-shared", "-fopenmp", "-o", tmp,
                               os.path.join(_HERE, "gen.c"), "-lm"])
        os.replace(tmp, _SO)
    return _SO


def lib():
    global _lib
    if _lib is None:
        build()
        L = ctypes.CDLL(_SO)
        u64, u32, i64 = ctypes.c_uint64, ctypes.c_uint32, ctypes.c_int64
        vp = ctypes.c_void_p
        L.synth_key.restype = u64
        L.synth_key.argtypes = [u64, u32, u32, u32]
        L.synth_draw.restype = u64
        L.synth_draw.argtypes = [u64, u64]
        L.synth_normal_f32.argtypes = [u64, i64, ctypes.c_double, ctypes.c_double, vp]
        L.synth_bytes.argtypes = [u64, i64, vp]
        L.synth_f64_to_f16.restype = ctypes.c_uint16
        L.synth_f64_to_f16.argtypes = [ctypes.c_double]
        L.synth_uniform_f16.argtypes = [u64, i64, ctypes.c_double, ctypes.c_double, vp]
        L.synth_f32_to_bf16.argtypes = [vp, i64, vp]
        L.synth_expert_blob.argtypes = [u64, u32, u32, i64, i64, ctypes.c_double, ctypes.c_double, vp]
        L.synth_layer_blobs.argtypes = [u64, u32, u32, u32, i64, i64, ctypes.c_double,
                                        ctypes.c_double, vp]
        _lib = L
    return _lib


def _ptr(a: np.ndarray) -> int:
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data


def key(seed: int, layer: int, tensor: int, expert: int = 0) -> int:
    return lib().synth_key(seed, layer, tensor, expert)


def draws(k: int, n: int) -> np.ndarray:
    L = lib()
    return np.array([L.synth_draw(k, i) for i in range(n)], dtype=np.uint64)


def normal(seed: int, layer: int, tensor: int, n: int, std: float = 1.0, mean: float = 0.0,
           expert: int = 0) -> np.ndarray:
    out = np.empty(n, dtype=np.float32)
    lib().synth_normal_f32(key(seed, layer, tensor, expert), n, mean, std, _ptr(out))
    return out


def random_bytes(seed: int, layer: int, tensor: int, n: int, expert: int = 0) -> np.ndarray:
    out = np.empty(n, dtype=np.uint8)
    lib().synth_bytes(key(seed, layer, tensor, expert), n, _ptr(out))
    return out


def f64_to_f16_bits(v: float) -> int:
    return lib().synth_f64_to_f16(v)


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.shape, dtype=np.uint16)
    lib().synth_f32_to_bf16(_ptr(x), x.size, _ptr(out))
    return out


def blob_sizes(d: int, f: int, group: int = 64, bits: int = 4):
    """(code bytes, number of fp16 scales) of one expert: three matrices of
    f*d weights, `bits`-wide codes (8, 4 or 2: 1, 2 or 4 per byte), one scale
    per `group` consecutive weights of a row, or (group 0) one scale per row:
    2f + d."""
    nib = 3 * f * d * bits // 8
    nsc = 3 * f * d // group if group else 2 * f + d
    return nib, nsc


def expert_blob(seed: int, layer: int, expert: int, d: int, f: int, out=None,
                group: int = 64, bits: int = 4) -> np.ndarray:
    nib, nsc = blob_sizes(d, f, group, bits)
    if out is None:
        out = np.empty(nib + 2 * nsc, dtype=np.uint8)
    lib().synth_expert_blob(seed, layer, expert, nib, nsc, SCALE_LO, SCALE_HI, _ptr(out))
    return out


def layer_blobs(seed: int, layer: int, n_experts: int, d: int, f: int, e0: int = 0,
                out=None, group: int = 64, bits: int = 4) -> np.ndarray:
    nib, nsc = blob_sizes(d, f, group, bits)
    if out is None:
        out = np.empty((n_experts, nib + 2 * nsc), dtype=np.uint8)
    lib().synth_layer_blobs(seed, layer, e0, n_experts, nib, nsc, SCALE_LO, SCALE_HI, _ptr(out))
    return out


def zipf_bias(n_experts: int, s: float = 1.1) -> np.ndarray:
    """Router bias skewing selection toward low expert ids: the logarithm of an
    un-normalised Zipf(s) mass over rank = id + 1, i.e. -s * ln(id + 1)."""
    e = np.arange(n_experts, dtype=np.float64)
    return (-s * np.log(e + 1.0)).astype(np.float32)
