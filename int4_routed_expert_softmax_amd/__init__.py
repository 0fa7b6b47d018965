"""Python binding of libmoe.so, the gfx950 int4 routed-expert MoE layer.

Thin ctypes marshalling over the C ABI in include/moe.h: the functions below
carry the same names as the C entry points, take torch tensors (device memory
owned by the caller) and pass their pointers, sizes and the current HIP
stream.  Every step of the layer runs in the library's HIP kernels; there is no
Python or CPU fallback, and importing this package fails if the library has not
been built (``python -m int4_routed_expert_softmax_amd.build``).
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

_HERE = os.path.dirname(os.path.abspath(__file__))
# MOE_PHASE_TRACE=1 in the environment loads lib/libmoe_trace.so instead: the
# same library with the phase trace compiled in (moe_trace_read), for
# measurement only.
LIB_PATH = os.path.join(_HERE, "lib", "libmoe_trace.so" if os.environ.get("MOE_PHASE_TRACE") == "1"
                        else "libmoe.so")

MOE_F32, MOE_BF16 = 0, 1
MOE_PRENORM_RMS, MOE_RESIDUAL, MOE_BATCH_INVARIANT, MOE_INT8_ACT = 1, 2, 4, 8
MOE_OK, MOE_EINVAL, MOE_EUNSUPPORTED, MOE_ENOSPC, MOE_EHIP = 0, -1, -2, -3, -4

# Every function include/moe.h declares.
EXPORTS = ("moe_expert_blob_bytes", "moe_workspace_bytes", "moe_workspace_routing",
           "moe_strerror", "moe_route",
           "moe_union", "moe_expert_ffn", "moe_layer_forward", "moe_cache_state_bytes",
           "moe_layer_forward_cached", "moe_layer_forward_noalloc", "moe_timing_arm",
           "moe_trace_read", "moe_trace_reset", "moe_hbm_read_probe")

# Bytes of the library's own per-GPU workspace behind moe_layer_forward_noalloc.
NOALLOC_SCRATCH_BYTES = 32 << 20

# Traced kernels for moe_trace_read (records of 8 uint64 words per workgroup).
TRACES = {"gateup_gemv": 0, "route_small": 1, "down_t1": 2, "router_front": 3,
          "gateup_thin": 4, "down_thin": 5, "gateup_mixed": 6, "down_mixed": 7}
TRACE_RECORDS, TRACE_WORDS = 32768, 8

# Kernel ids for moe_timing_arm.
KERNELS = {"rmsnorm": 0, "logits": 1, "topk": 2, "union": 3, "digitize": 4, "gateup": 5,
           "down": 6, "combine": 7, "read_probe": 8, "gateup_thin": 9, "down_thin": 10}


class MoeError(RuntimeError):
    def __init__(self, code: int, where: str):
        super().__init__(f"{where}: {strerror(code)} (code {code})")
        self.code = code


class moe_routing_offsets(ctypes.Structure):
    _fields_ = [(n, ctypes.c_size_t) for n in
                ("topk_idx", "topk_w", "uniq", "n_uniq", "offsets", "rows")]


class moe_dims(ctypes.Structure):
    _fields_ = [("d", ctypes.c_int32), ("f", ctypes.c_int32), ("n_experts", ctypes.c_int32),
                ("top_k", ctypes.c_int32), ("group_size", ctypes.c_int32),
                ("code_bits", ctypes.c_int32)]


@dataclass(frozen=True)
class Dims:
    d: int
    f: int
    n_experts: int
    top_k: int
    group_size: int = 64
    code_bits: int = 4

    def c(self) -> moe_dims:
        return moe_dims(self.d, self.f, self.n_experts, self.top_k, self.group_size,
                        self.code_bits)


def _hip_runtimes():
    """Paths of every HIP runtime mapped into this process."""
    try:
        with open("/proc/self/maps") as fh:
            return sorted({l.split()[-1] for l in fh if "libamdhip64" in l})
    except OSError:
        return []


def _load():
    # torch ships its own HIP runtime (soname libamdhip64.so.7).  Loading torch
    # first makes libmoe.so bind to that same runtime, so the library and torch
    # share one set of streams and allocations.
    try:
        import torch  # noqa: F401
    except ImportError:
        pass
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with "
                          "`python -m int4_routed_expert_softmax_amd.build` (hipcc, gfx950)")
    L = ctypes.CDLL(LIB_PATH)
    vp, i32, sz, u32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t, ctypes.c_uint32
    dp = ctypes.POINTER(moe_dims)
    L.moe_expert_blob_bytes.restype = sz
    L.moe_expert_blob_bytes.argtypes = [dp]
    L.moe_workspace_bytes.restype = sz
    L.moe_workspace_bytes.argtypes = [dp, i32]
    L.moe_workspace_routing.restype = ctypes.c_int
    L.moe_workspace_routing.argtypes = [dp, i32, ctypes.POINTER(moe_routing_offsets)]
    L.moe_strerror.restype = ctypes.c_char_p
    L.moe_strerror.argtypes = [ctypes.c_int]
    L.moe_route.restype = ctypes.c_int
    L.moe_route.argtypes = [dp, vp, ctypes.c_int, i32, vp, vp, vp, vp, vp, sz, vp]
    L.moe_union.restype = ctypes.c_int
    L.moe_union.argtypes = [dp, vp, i32, vp, vp, vp, vp, vp]
    L.moe_expert_ffn.restype = ctypes.c_int
    L.moe_expert_ffn.argtypes = [dp, vp, vp, ctypes.c_int, vp, i32, vp, vp, sz, vp]
    L.moe_layer_forward.restype = ctypes.c_int
    L.moe_layer_forward.argtypes = [dp, vp, ctypes.c_int, i32, vp, vp, vp, vp, u32,
                                    ctypes.c_float, vp, vp, sz, vp]
    L.moe_cache_state_bytes.restype = sz
    L.moe_cache_state_bytes.argtypes = [dp, i32]
    L.moe_layer_forward_cached.restype = ctypes.c_int
    L.moe_layer_forward_cached.argtypes = [dp, vp, ctypes.c_int, i32, vp, vp, vp, vp, i32, vp, vp,
                                           u32, ctypes.c_float, vp, vp, sz, vp]
    L.moe_layer_forward_noalloc.restype = ctypes.c_int
    L.moe_layer_forward_noalloc.argtypes = [dp, vp, ctypes.c_int, i32, vp, vp, vp, vp, u32,
                                            ctypes.c_float, vp, vp]
    L.moe_timing_arm.restype = ctypes.c_int
    L.moe_timing_arm.argtypes = [ctypes.c_int, vp, vp, ctypes.c_int]
    L.moe_trace_read.restype = ctypes.c_int
    L.moe_trace_read.argtypes = [ctypes.c_int, vp, sz]
    L.moe_trace_reset.restype = ctypes.c_int
    L.moe_trace_reset.argtypes = []
    L.moe_hbm_read_probe.restype = ctypes.c_int
    L.moe_hbm_read_probe.argtypes = [vp, sz, vp, i32, vp]
    rt = _hip_runtimes()
    if len(rt) > 1:
        raise ImportError(f"more than one HIP runtime is loaded: {rt}")
    return L


lib = _load()


def strerror(code: int) -> str:
    return lib.moe_strerror(code).decode()


def _check(code: int, where: str):
    if code != MOE_OK:
        raise MoeError(code, where)


def _ptr(t):
    return None if t is None else t.data_ptr()


def _stream(stream):
    if stream is not None:
        return stream
    import torch
    return torch.cuda.current_stream().cuda_stream


def _xdtype(x) -> int:
    import torch
    if x.dtype == torch.float32:
        return MOE_F32
    if x.dtype == torch.bfloat16:
        return MOE_BF16
    raise TypeError(f"x must be float32 or bfloat16, got {x.dtype}")


def expert_blob_bytes(dims: Dims) -> int:
    return lib.moe_expert_blob_bytes(ctypes.byref(dims.c()))


def workspace_bytes(dims: Dims, T_max: int) -> int:
    return lib.moe_workspace_bytes(ctypes.byref(dims.c()), T_max)


def make_workspace(dims: Dims, T_max: int, device="cuda"):
    """A zero-filled workspace (the library keeps its counters at zero)."""
    import torch
    return torch.zeros(workspace_bytes(dims, T_max), dtype=torch.uint8, device=device)


def moe_workspace_routing(dims: Dims, T: int) -> dict:
    """Byte offsets in a workspace of the routing results a layer call on T
    tokens leaves there."""
    o = moe_routing_offsets()
    _check(lib.moe_workspace_routing(ctypes.byref(dims.c()), T, ctypes.byref(o)),
           "moe_workspace_routing")
    return {n: getattr(o, n) for n, _ in moe_routing_offsets._fields_}


def workspace_routing(dims: Dims, T: int, ws) -> dict:
    """Views into the workspace ws (uint8 device tensor) of the routing of
    the last layer call on T tokens: topk_idx [T][k] int32, topk_w [T][k]
    f32, uniq [cap] int32, n_uniq [1] int32, offsets [cap + 1] int32, rows
    [T*k] int32, cap = min(E, T*k)."""
    import torch
    off = moe_workspace_routing(dims, T)
    k, cap = dims.top_k, min(dims.n_experts, T * dims.top_k)

    def view(name, n, dt):
        nb = n * 4
        return ws[off[name]:off[name] + nb].view(dt)

    return {"topk_idx": view("topk_idx", T * k, torch.int32).view(T, k),
            "topk_w": view("topk_w", T * k, torch.float32).view(T, k),
            "uniq": view("uniq", cap, torch.int32),
            "n_uniq": view("n_uniq", 1, torch.int32),
            "offsets": view("offsets", cap + 1, torch.int32),
            "rows": view("rows", T * k, torch.int32)}


def moe_route(dims: Dims, x, w_router, bias, topk_idx, topk_w, ws, stream=None):
    T = x.shape[0]
    _check(lib.moe_route(ctypes.byref(dims.c()), _ptr(x), _xdtype(x), T, _ptr(w_router),
                         _ptr(bias), _ptr(topk_idx), _ptr(topk_w), _ptr(ws), ws.numel(),
                         _stream(stream)), "moe_route")


def moe_union(dims: Dims, topk_idx, uniq, n_uniq, offsets, rows, stream=None):
    T = topk_idx.shape[0]
    _check(lib.moe_union(ctypes.byref(dims.c()), _ptr(topk_idx), T, _ptr(uniq), _ptr(n_uniq),
                         _ptr(offsets), _ptr(rows), _stream(stream)), "moe_union")


def moe_expert_ffn(dims: Dims, expert_blob, x, rows, n, y, ws, stream=None):
    """expert_blob: a uint8 tensor, or an int device/host-mapped address."""
    blob = expert_blob if isinstance(expert_blob, int) else _ptr(expert_blob)
    _check(lib.moe_expert_ffn(ctypes.byref(dims.c()), blob, _ptr(x), _xdtype(x), _ptr(rows), n,
                              _ptr(y), _ptr(ws), ws.numel(), _stream(stream)), "moe_expert_ffn")


def moe_layer_forward(dims: Dims, x, w_router, bias, expert_table, out, flags=0, rms_eps=1e-6,
                      stats=None, ws=None, stream=None):
    """expert_table: int64 device tensor of E blob addresses."""
    T = x.shape[0]
    _check(lib.moe_layer_forward(ctypes.byref(dims.c()), _ptr(x), _xdtype(x), T, _ptr(w_router),
                                 _ptr(bias), _ptr(expert_table), _ptr(out), flags, rms_eps,
                                 _ptr(stats), _ptr(ws), ws.numel(), _stream(stream)),
           "moe_layer_forward")


def moe_layer_forward_noalloc(dims: Dims, x, w_router, bias, expert_table, out, flags=0,
                              rms_eps=1e-6, stats=None, stream=None):
    """moe_layer_forward on the library's own per-GPU workspace (no ws
    argument; nothing is allocated).  Calls needing more than
    NOALLOC_SCRATCH_BYTES of workspace raise MoeError (MOE_ENOSPC)."""
    T = x.shape[0]
    _check(lib.moe_layer_forward_noalloc(ctypes.byref(dims.c()), _ptr(x), _xdtype(x), T,
                                         _ptr(w_router), _ptr(bias), _ptr(expert_table), _ptr(out),
                                         flags, rms_eps, _ptr(stats), _stream(stream)),
           "moe_layer_forward_noalloc")


def cache_state_bytes(dims: Dims, n_slots: int) -> int:
    return lib.moe_cache_state_bytes(ctypes.byref(dims.c()), n_slots)


def make_cache_state(dims: Dims, n_slots: int, device="cuda"):
    """A zero-filled cache state (every slot empty)."""
    import torch
    n = cache_state_bytes(dims, n_slots)
    if n == 0:
        raise ValueError(f"no cache state for {n_slots} slots of {dims}")
    return torch.zeros(n // 4, dtype=torch.int32, device=device)


def cache_header(state) -> dict:
    """The state's header counters (reads the device buffer)."""
    h = state[:5].cpu().tolist()
    return dict(zip(("clock", "hits", "misses", "last_hits", "last_misses"), h))


def moe_layer_forward_cached(dims: Dims, x, w_router, bias, home_table, slots, n_slots,
                             cache_state, out, flags=0, rms_eps=1e-6, stats=None, ws=None,
                             stream=None):
    """home_table: int64 device tensor of E blob addresses (e.g. host-mapped
    pinned memory); slots: device memory for n_slots blobs."""
    T = x.shape[0]
    _check(lib.moe_layer_forward_cached(
        ctypes.byref(dims.c()), _ptr(x), _xdtype(x), T, _ptr(w_router), _ptr(bias),
        _ptr(home_table), _ptr(slots), n_slots, _ptr(cache_state), _ptr(out), flags, rms_eps,
        _ptr(stats), _ptr(ws), ws.numel(), _stream(stream)), "moe_layer_forward_cached")


def moe_timing_arm(kernel: str, start_events, stop_events):
    """Arm kernel timing: launch i of `kernel` records start_events[i] and
    stop_events[i] (torch.cuda.Event objects with timing enabled; they are
    recorded once here so that their HIP handles exist).  Returns a handle
    that keeps the handle arrays alive; pass it to moe_timing_disarm."""
    import torch
    n = len(start_events)
    assert len(stop_events) == n
    for ev in (*start_events, *stop_events):
        if ev.cuda_event == 0:
            ev.record()
    torch.cuda.synchronize()
    arr_t = ctypes.c_void_p * n
    starts = arr_t(*[ev.cuda_event for ev in start_events])
    stops = arr_t(*[ev.cuda_event for ev in stop_events])
    kid = KERNELS[kernel]
    lib.moe_timing_arm(kid, ctypes.cast(starts, ctypes.c_void_p), ctypes.cast(stops, ctypes.c_void_p), n)
    return (kid, starts, stops)


def moe_timing_disarm(handle) -> int:
    """Disarm; returns how many launches were recorded."""
    return lib.moe_timing_arm(handle[0], None, None, 0)


def moe_trace_read(kernel: str, records: int = TRACE_RECORDS):
    """The first `records` phase-trace records of `kernel` as a uint64 array
    [records][8] (libmoe_trace.so only; MoeError MOE_EUNSUPPORTED otherwise)."""
    import numpy as np
    out = np.zeros((records, TRACE_WORDS), dtype=np.uint64)
    _check(lib.moe_trace_read(TRACES[kernel], out.ctypes.data, out.nbytes), "moe_trace_read")
    return out


def moe_trace_reset():
    _check(lib.moe_trace_reset(), "moe_trace_reset")


def moe_hbm_read_probe(buf, sink, blocks: int, stream=None):
    """Stream all bytes of the device tensor buf (a plain read kernel: the
    measured HBM ceiling); sink: int32 device tensor of blocks * 256 words."""
    assert sink.numel() * sink.element_size() >= blocks * 256 * 4
    _check(lib.moe_hbm_read_probe(_ptr(buf), buf.numel() * buf.element_size(), _ptr(sink), blocks,
                                  _stream(stream)), "moe_hbm_read_probe")
