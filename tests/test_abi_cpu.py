"""The C ABI without a GPU: the library loads, exports every function the
header declares, sizes blobs and workspaces, and rejects invalid arguments
before touching any device (the validation paths make no HIP call)."""
import ctypes
import os
import re

import pytest

import int4_routed_expert_softmax_amd as moe
import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe.h")

GLM = moe.Dims(6144, 2048, 256, 8)
TINY = moe.Dims(256, 128, 16, 2)
FAKE = 1 << 20  # an aligned non-null address that is never dereferenced


def declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z_]+)\s*\(", src)))


def test_header_declarations_are_exported():
    names = declared()
    assert set(names) == set(moe.EXPORTS)
    L = ctypes.CDLL(moe.LIB_PATH)
    for n in names:
        assert hasattr(L, n), n


def test_only_the_abi_is_exported():
    import subprocess
    out = subprocess.run(["nm", "-D", "--defined-only", moe.LIB_PATH], capture_output=True,
                         text=True).stdout
    ours = {l.split()[-1] for l in out.splitlines() if l.split()[-1].startswith("moe_")}
    assert ours == set(moe.EXPORTS)


def test_blob_and_workspace_sizes():
    assert moe.expert_blob_bytes(GLM) == 20054016
    assert moe.expert_blob_bytes(TINY) == 52224
    assert moe.expert_blob_bytes(moe.Dims(6144, 2048, 256, 8, group_size=32)) == 0
    # per-row scales: the codes, then 2f + d scales
    assert moe.expert_blob_bytes(moe.Dims(6144, 2048, 256, 8, group_size=0)) == 18894848
    assert moe.expert_blob_bytes(moe.Dims(256, 128, 16, 2, group_size=0)) == \
        oracle.blob_bytes(256, 128, group=0)
    w1 = moe.workspace_bytes(GLM, 1)
    w512 = moe.workspace_bytes(GLM, 512)
    assert 0 < w1 < 4 << 20 and w512 > w1
    assert moe.workspace_bytes(GLM, 0) == 0


@pytest.mark.parametrize("T,k", [(1, 32), (3, 32), (8, 9), (9, 1), (64, 8)])
def test_workspace_holds_split_logits(T, k):
    # Batches past the small-batch path (T > 8 or T * k > 64 picks) keep 8
    # fp64 partial sums per logit; narrow d and f so nothing else hides it.
    dims = moe.Dims(64, 64, 1024, k)
    small = T <= 8 and T * k <= 64
    need = T * 1024 * 8 * (1 if small else 8)
    assert moe.workspace_bytes(dims, T) >= need


def call_route(dims, x=FAKE, dtype=moe.MOE_F32, T=1, wr=FAKE, idx=FAKE, w=FAKE, ws=FAKE,
               ws_bytes=None):
    if ws_bytes is None:
        ws_bytes = max(1, moe.workspace_bytes(dims, max(T, 1)))
    return moe.lib.moe_route(ctypes.byref(dims.c()), x, dtype, T, wr, None, idx, w, ws, ws_bytes,
                             None)


@pytest.mark.parametrize("dims,code", [
    (moe.Dims(6144, 2048, 256, 8, 32), moe.MOE_EUNSUPPORTED),
    (moe.Dims(6100, 2048, 256, 8), moe.MOE_EUNSUPPORTED),
    (moe.Dims(6144, 2000, 256, 8), moe.MOE_EUNSUPPORTED),
    (moe.Dims(6144, 2048, 2048, 8), moe.MOE_EUNSUPPORTED),
    (moe.Dims(6144, 2048, 256, 33), moe.MOE_EUNSUPPORTED),
    (moe.Dims(6144, 2048, 4, 8), moe.MOE_EINVAL),
    (moe.Dims(0, 2048, 256, 8), moe.MOE_EINVAL),
])
def test_route_rejects_bad_dims(dims, code):
    assert call_route(dims, ws_bytes=1 << 30) == code


def test_route_rejects_bad_arguments():
    assert call_route(GLM, T=0) == moe.MOE_EINVAL
    assert call_route(GLM, x=None) == moe.MOE_EINVAL
    assert call_route(GLM, x=FAKE + 4) == moe.MOE_EINVAL  # misaligned
    assert call_route(GLM, dtype=7) == moe.MOE_EUNSUPPORTED
    assert call_route(GLM, ws=None) == moe.MOE_EINVAL
    assert call_route(GLM, ws=FAKE + 8) == moe.MOE_EINVAL  # workspace not 16-byte aligned
    assert call_route(GLM, ws_bytes=16) == moe.MOE_ENOSPC
    assert moe.lib.moe_route(None, FAKE, 0, 1, FAKE, None, FAKE, FAKE, FAKE, 1 << 30,
                             None) == moe.MOE_EINVAL


def test_union_rejects_bad_arguments():
    d = GLM.c()
    assert moe.lib.moe_union(ctypes.byref(d), None, 1, FAKE, FAKE, FAKE, FAKE, None) == moe.MOE_EINVAL
    assert moe.lib.moe_union(ctypes.byref(d), FAKE, 0, FAKE, FAKE, FAKE, FAKE, None) == moe.MOE_EINVAL


def test_expert_ffn_rejects_bad_arguments():
    d = GLM.c()
    ws = moe.workspace_bytes(GLM, 4)
    f = moe.lib.moe_expert_ffn
    assert f(ctypes.byref(d), None, FAKE, 0, None, 4, FAKE, FAKE, ws, None) == moe.MOE_EINVAL
    assert f(ctypes.byref(d), FAKE + 8, FAKE, 0, None, 4, FAKE, FAKE, ws, None) == moe.MOE_EINVAL
    assert f(ctypes.byref(d), FAKE, FAKE, 0, None, 0, FAKE, FAKE, ws, None) == moe.MOE_EINVAL
    assert f(ctypes.byref(d), FAKE, FAKE, 0, None, 4, FAKE, FAKE, ws - 1, None) == moe.MOE_ENOSPC
    assert f(ctypes.byref(d), FAKE, FAKE, 3, None, 4, FAKE, FAKE, ws, None) == moe.MOE_EUNSUPPORTED


def test_layer_forward_rejects_bad_arguments():
    d = GLM.c()
    ws = moe.workspace_bytes(GLM, 2)
    f = moe.lib.moe_layer_forward

    def call(**kw):
        a = dict(x=FAKE, dt=moe.MOE_F32, T=2, wr=FAKE, table=FAKE, out=FAKE, flags=0, eps=1e-6,
                 ws=FAKE, wsb=ws)
        a.update(kw)
        return f(ctypes.byref(d), a["x"], a["dt"], a["T"], a["wr"], None, a["table"], a["out"],
                 a["flags"], a["eps"], None, a["ws"], a["wsb"], None)

    assert call(table=None) == moe.MOE_EINVAL
    assert call(out=None) == moe.MOE_EINVAL
    assert call(T=-1) == moe.MOE_EINVAL
    assert call(flags=16) == moe.MOE_EUNSUPPORTED  # no such flag
    # batch invariance covers the single-token family's batch limits only
    ws9 = moe.workspace_bytes(GLM, 9)
    assert call(flags=moe.MOE_BATCH_INVARIANT, T=9, wsb=ws9) == moe.MOE_EUNSUPPORTED
    d32 = moe.Dims(6144, 2048, 256, 32).c()
    assert f(ctypes.byref(d32), FAKE, moe.MOE_F32, 3, FAKE, None, FAKE, FAKE,
             moe.MOE_BATCH_INVARIANT, 1e-6, None, FAKE,
             moe.workspace_bytes(moe.Dims(6144, 2048, 256, 32), 3), None) == moe.MOE_EUNSUPPORTED
    assert call(flags=moe.MOE_RESIDUAL, dt=moe.MOE_BF16) == moe.MOE_EUNSUPPORTED
    assert call(flags=moe.MOE_PRENORM_RMS, eps=-1.0) == moe.MOE_EINVAL
    assert call(wsb=ws - 256) == moe.MOE_ENOSPC


def test_cache_state_sizes():
    # header (8 words) + slot_of[E] + expert_of[S] + stamp[S], rounded to 256 B
    assert moe.cache_state_bytes(GLM, 8) == (32 + 4 * 256 + 8 * 8 + 255) // 256 * 256
    assert moe.cache_state_bytes(GLM, 256) == (32 + 4 * 256 + 8 * 256 + 255) // 256 * 256
    assert moe.cache_state_bytes(GLM, 0) == 0
    assert moe.cache_state_bytes(GLM, 257) == 0  # more slots than experts


def test_cached_layer_rejects_bad_arguments():
    d = GLM.c()
    f = moe.lib.moe_layer_forward_cached
    ws = moe.workspace_bytes(GLM, 1)

    def call(**kw):
        a = dict(x=FAKE, dt=moe.MOE_F32, T=1, wr=FAKE, home=FAKE, slots=FAKE, S=8, state=FAKE,
                 out=FAKE, flags=0, ws=FAKE, wsb=ws)
        a.update(kw)
        return f(ctypes.byref(d), a["x"], a["dt"], a["T"], a["wr"], None, a["home"], a["slots"],
                 a["S"], a["state"], a["out"], a["flags"], 1e-6, None, a["ws"], a["wsb"], None)

    assert call(home=None) == moe.MOE_EINVAL
    assert call(slots=None) == moe.MOE_EINVAL
    assert call(state=None) == moe.MOE_EINVAL
    assert call(slots=FAKE + 16) == moe.MOE_EINVAL       # slots must be 256-byte aligned
    assert call(S=7) == moe.MOE_EUNSUPPORTED               # fewer slots than a union can hold
    assert call(T=2, S=15, wsb=moe.workspace_bytes(GLM, 2)) == moe.MOE_EUNSUPPORTED
    assert call(S=257) == moe.MOE_EUNSUPPORTED             # more slots than experts
    assert call(T=9, S=72, wsb=moe.workspace_bytes(GLM, 9)) == moe.MOE_EUNSUPPORTED  # past the small-batch limits
    assert call(flags=16) == moe.MOE_EUNSUPPORTED  # no such flag
    assert call(wsb=ws - 256) == moe.MOE_ENOSPC


def test_read_probe_rejects_bad_arguments():
    # validation happens before anything touches a device
    L = moe.lib
    assert L.moe_hbm_read_probe(None, 1 << 20, 16, 4, None) == moe.MOE_EINVAL
    assert L.moe_hbm_read_probe(64, 1 << 20, None, 4, None) == moe.MOE_EINVAL
    assert L.moe_hbm_read_probe(64, 0, 16, 4, None) == moe.MOE_EINVAL
    assert L.moe_hbm_read_probe(64, 1000, 16, 4, None) == moe.MOE_EINVAL
    assert L.moe_hbm_read_probe(64, 1 << 20, 16, 0, None) == moe.MOE_EINVAL
    assert L.moe_hbm_read_probe(72, 1 << 20, 16, 4, None) == moe.MOE_EINVAL


def test_strerror():
    for c in (0, -1, -2, -3, -4, 99):
        assert isinstance(moe.strerror(c), str) and moe.strerror(c)


def test_one_hip_runtime_in_process():
    assert len(moe._hip_runtimes()) == 1


@pytest.mark.parametrize("dims,T", [(GLM, 1), (GLM, 8), (GLM, 512), (TINY, 4),
                                    (moe.Dims(256, 128, 1024, 32), 2)])
def test_workspace_routing_offsets_lie_inside_the_workspace(dims, T):
    off = moe.moe_workspace_routing(dims, T)
    k, cap = dims.top_k, min(dims.n_experts, T * dims.top_k)
    sizes = {"topk_idx": 4 * T * k, "topk_w": 4 * T * k, "uniq": 4 * cap, "n_uniq": 4,
             "offsets": 4 * (cap + 1), "rows": 4 * T * k}
    total = moe.workspace_bytes(dims, T)
    spans = sorted((off[n], off[n] + sizes[n]) for n in sizes)
    for (a0, a1), (b0, _) in zip(spans, spans[1:]):
        assert a1 <= b0, "routing arrays overlap"
    assert spans[-1][1] <= total
    assert all(off[n] % 4 == 0 for n in off)
    # a smaller call on a larger workspace: offsets of its own T, still inside
    if T > 1:
        assert moe.moe_workspace_routing(dims, 1)["rows"] < total


def test_workspace_routing_rejects_bad_arguments():
    o = moe.moe_routing_offsets()
    assert moe.lib.moe_workspace_routing(ctypes.byref(GLM.c()), 0, ctypes.byref(o)) == moe.MOE_EINVAL
    assert moe.lib.moe_workspace_routing(ctypes.byref(GLM.c()), 1, None) == moe.MOE_EINVAL
    bad = moe.Dims(6144, 2048, 256, 8, 32)
    assert moe.lib.moe_workspace_routing(ctypes.byref(bad.c()), 1, ctypes.byref(o)) == \
        moe.MOE_EUNSUPPORTED


def test_trace_calls_are_refused_by_the_product_library():
    # libmoe.so carries no trace code: both calls say so before touching the GPU
    import numpy as np
    buf = np.zeros((4, moe.TRACE_WORDS), dtype=np.uint64)
    assert moe.lib.moe_trace_read(0, buf.ctypes.data, buf.nbytes) == moe.MOE_EUNSUPPORTED
    assert moe.lib.moe_trace_reset() == moe.MOE_EUNSUPPORTED
    assert moe.lib.moe_trace_read(-1, buf.ctypes.data, buf.nbytes) == moe.MOE_EINVAL
    assert moe.lib.moe_trace_read(8, buf.ctypes.data, buf.nbytes) == moe.MOE_EINVAL
    assert moe.lib.moe_trace_read(0, None, buf.nbytes) == moe.MOE_EINVAL


def test_trace_library_exports_the_same_abi():
    import subprocess
    path = os.path.join(os.path.dirname(moe.LIB_PATH), "libmoe_trace.so")
    out = subprocess.run(["nm", "-D", "--defined-only", path], capture_output=True, text=True,
                         check=True).stdout
    ours = {l.split()[-1] for l in out.splitlines() if l.split()[-1].startswith("moe_")}
    assert ours == set(moe.EXPORTS)
