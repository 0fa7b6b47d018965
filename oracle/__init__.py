"""CPU oracle of the int4 routed-expert MoE layer (ctypes binding of moe_ref.c).

TEST INFRASTRUCTURE: only the test suite, ``__graft_entry__.smoke()`` and the
benchmark's ``cpu_baseline`` leg may import this package.  The product path
(``int4_routed_expert_softmax_amd``) never imports it.

Everything here is argument marshalling; the arithmetic is in moe_ref.c.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SO = os.path.join(_HERE, "libmoeref.so")
_lib = None

PRENORM = 1
RESIDUAL = 2
I8ACT = 8  # integer activations (moe_ref.c, ref_expert_ffn_i8act)


def build(force: bool = False) -> str:
    if force or not os.path.exists(_SO):
        tmp = _SO + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-fPIC", "-shared", "-fopenmp", "-std=c11",
                               "-o", tmp, os.path.join(_HERE, "moe_ref.c"), "-lm"])
        os.replace(tmp, _SO)
    return _SO


def build_sanitized(out_dir: str) -> str:
    """Build moe_ref.c with sanitize_check.c under AddressSanitizer and
    UndefinedBehaviorSanitizer (every report fatal) into an executable in
    out_dir; returns its path."""
    exe = os.path.join(out_dir, "moe_ref_sanitized")
    subprocess.check_call(["gcc", "-O1", "-g", "-fno-omit-frame-pointer", "-fopenmp", "-std=c11",
                           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                           "-o", exe, os.path.join(_HERE, "moe_ref.c"),
                           os.path.join(_HERE, "sanitize_check.c"), "-lm"])
    return exe


def omp_threads(n: int | None = None) -> int:
    """Threads the oracle's OpenMP loops use (the process's libgomp, which
    the oracle library links); with n, set them first."""
    lib()
    gomp = ctypes.CDLL("libgomp.so.1")
    if n is not None:
        gomp.omp_set_num_threads(int(n))
    return int(gomp.omp_get_max_threads())


def lib():
    global _lib
    if _lib is None:
        build()
        L = ctypes.CDLL(_SO)
        vp, i32, i64, u32 = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_uint32
        dbl = ctypes.c_double
        L.ref_nibble.restype = i32
        L.ref_nibble.argtypes = [vp, i64]
        L.ref_f16.restype = dbl
        L.ref_f16.argtypes = [ctypes.c_uint16]
        L.ref_bf16.restype = dbl
        L.ref_bf16.argtypes = [ctypes.c_uint16]
        L.ref_code.restype = i32
        L.ref_code.argtypes = [vp, i64, i32]
        L.ref_blob_bytes.restype = i64
        L.ref_blob_bytes.argtypes = [i32, i32, i32, i32]
        L.ref_dequant.argtypes = [vp, i32, i32, i32, i32, i32, vp]
        L.ref_silu.restype = dbl
        L.ref_silu.argtypes = [dbl]
        L.ref_expert_ffn.argtypes = [i32, i32, i32, i32, vp, vp, i32, vp]
        L.ref_quant_i8.argtypes = [vp, i32, vp, vp]
        L.ref_expert_ffn_i8act.argtypes = [i32, i32, i32, i32, vp, vp, i32, vp]
        L.ref_route.argtypes = [i32, i32, i32, vp, i32, i32, vp, vp, vp, vp, vp]
        L.ref_union.restype = i32
        L.ref_union.argtypes = [i32, i32, i32, vp, vp, vp, vp]
        L.ref_rmsnorm.argtypes = [i32, vp, dbl, vp]
        L.ref_layer_forward.restype = i32
        L.ref_layer_forward.argtypes = [i32, i32, i32, i32, i32, i32, vp, i32, i32, vp, vp, vp,
                                        u32, dbl, vp, vp, vp, vp, vp, vp, vp]
        _lib = L
    return _lib


def _p(a):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"], "oracle inputs must be C-contiguous"
    return a.ctypes.data


def nibble(row_codes: np.ndarray, c: int) -> int:
    return lib().ref_nibble(_p(np.ascontiguousarray(row_codes, dtype=np.uint8)), c)


def code(row_codes: np.ndarray, c: int, bits: int = 4) -> int:
    """Weight c of a row of `bits`-wide two's-complement codes (8, 4 or 2)."""
    return lib().ref_code(_p(np.ascontiguousarray(row_codes, dtype=np.uint8)), c, bits)


def f16(bits: int) -> float:
    return lib().ref_f16(bits)


def bf16(bits: int) -> float:
    return lib().ref_bf16(bits)


# group: 64 (one fp16 scale per 64 consecutive weights of a row) or 0 (one
# scale per row); bits: code width, 4 (int4), 8 (int8) or 2 (int2)
def blob_bytes(d: int, f: int, group: int = 64, bits: int = 4) -> int:
    return lib().ref_blob_bytes(d, f, group, bits)


def dequant(blob: np.ndarray, d: int, f: int, which: int, group: int = 64,
            bits: int = 4) -> np.ndarray:
    rows, cols = (d, f) if which == 2 else (f, d)
    W = np.empty((rows, cols), dtype=np.float64)
    lib().ref_dequant(_p(blob), d, f, group, bits, which, _p(W))
    return W


def silu(v: float) -> float:
    return lib().ref_silu(v)


def expert_ffn(blob: np.ndarray, x: np.ndarray, d: int, f: int, group: int = 64,
               bits: int = 4) -> np.ndarray:
    x = np.ascontiguousarray(np.atleast_2d(x), dtype=np.float64)
    n = x.shape[0]
    y = np.empty((n, d), dtype=np.float64)
    lib().ref_expert_ffn(d, f, group, bits, _p(blob), _p(x), n, _p(y))
    return y


def quant_i8(v: np.ndarray):
    """One activation row (fp32, a multiple of 64 columns) -> (q int8 [cols],
    s float32 [cols / 64])."""
    v = np.ascontiguousarray(v, dtype=np.float32)
    q = np.empty(v.shape[-1], dtype=np.int8)
    s = np.empty(v.shape[-1] // 64, dtype=np.float32)
    lib().ref_quant_i8(_p(v), v.shape[-1], _p(q), _p(s))
    return q, s


def expert_ffn_i8act(blob: np.ndarray, x: np.ndarray, d: int, f: int, group: int = 64,
                     bits: int = 4) -> np.ndarray:
    """The expert FFN with integer activations; x rows are taken as fp32."""
    x = np.ascontiguousarray(np.atleast_2d(x), dtype=np.float32)
    n = x.shape[0]
    y = np.empty((n, d), dtype=np.float64)
    lib().ref_expert_ffn_i8act(d, f, group, bits, _p(blob), _p(x), n, _p(y))
    return y


def _xarg(x: np.ndarray, x_bf16: bool):
    if x_bf16:
        return np.ascontiguousarray(x, dtype=np.uint16)
    return np.ascontiguousarray(x, dtype=np.float32)


def route(x, Wr, bias, k, x_bf16=False):
    """-> idx [T][k] int32, w [T][k] float64, z [T][E] float64."""
    x = _xarg(x, x_bf16)
    T, d = x.shape
    E = Wr.shape[0]
    Wr = np.ascontiguousarray(Wr, dtype=np.float32)
    b = None if bias is None else np.ascontiguousarray(bias, dtype=np.float32)
    idx = np.empty((T, k), dtype=np.int32)
    w = np.empty((T, k), dtype=np.float64)
    z = np.empty((T, E), dtype=np.float64)
    lib().ref_route(d, E, k, _p(x), int(x_bf16), T, _p(Wr), _p(b), _p(idx), _p(w), _p(z))
    return idx, w, z


def union(idx: np.ndarray, E: int):
    """-> (uniq [U], offsets [U+1], rows [T*k]) int32."""
    idx = np.ascontiguousarray(idx, dtype=np.int32)
    T, k = idx.shape
    cap = min(E, T * k)
    uniq = np.empty(cap, dtype=np.int32)
    offsets = np.empty(cap + 1, dtype=np.int32)
    rows = np.empty(T * k, dtype=np.int32)
    U = lib().ref_union(E, k, T, _p(idx), _p(uniq), _p(offsets), _p(rows))
    return uniq[:U].copy(), offsets[:U + 1].copy(), rows


def rmsnorm(h: np.ndarray, eps: float = 1e-6) -> np.ndarray:
    h = np.ascontiguousarray(h, dtype=np.float32)
    xn = np.empty_like(h)
    lib().ref_rmsnorm(h.shape[-1], _p(h), eps, _p(xn))
    return xn


def layer_forward(x, Wr, bias, table, d, f, k, x_bf16=False, flags=0, eps=1e-6, group=64,
                  bits=4):
    """table: sequence of E uint8 blobs (or None for experts nobody picks).
    -> dict(out [T][d] f64, idx, w, uniq, offsets, rows, reads [E])."""
    x = _xarg(x, x_bf16)
    T = x.shape[0]
    E = len(table)
    Wr = np.ascontiguousarray(Wr, dtype=np.float32)
    b = None if bias is None else np.ascontiguousarray(bias, dtype=np.float32)
    ptrs = (ctypes.c_void_p * E)(*[None if t is None else _p(t) for t in table])
    cap = min(E, T * k)
    out = np.empty((T, d), dtype=np.float64)
    idx = np.empty((T, k), dtype=np.int32)
    w = np.empty((T, k), dtype=np.float64)
    uniq = np.empty(cap, dtype=np.int32)
    offsets = np.empty(cap + 1, dtype=np.int32)
    rows = np.empty(T * k, dtype=np.int32)
    reads = np.zeros(E, dtype=np.int32)
    U = lib().ref_layer_forward(d, f, group, bits, E, k, _p(x), int(x_bf16), T, _p(Wr), _p(b),
                                ctypes.cast(ptrs, ctypes.c_void_p), flags, eps, _p(out),
                                _p(idx), _p(w), _p(uniq), _p(offsets), _p(rows), _p(reads))
    if U < 0:
        raise ValueError("a selected expert has no blob in the table")
    return dict(out=out, idx=idx, w=w, uniq=uniq[:U].copy(), offsets=offsets[:U + 1].copy(),
                rows=rows, reads=reads, U=U)
