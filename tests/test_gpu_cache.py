"""GPU: the HBM slot cache in front of the experts' home memory
(moe_layer_forward_cached).

Where an expert's bytes live may decide only the speed (README 工作原理 ›
绝不为同一次磁盘读取等待两遍).  So over a sequence of calls, with the
experts at home in pinned host memory mapped into the device or in other
device memory, every output row and the per-expert counts must be
bit-identical to moe_layer_forward with the blobs resident: with any flags
for one token, with MOE_BATCH_INVARIANT for batches.  The placement policy is
pinned exactly: after every call the whole device state (clock, hit and miss
counters, slot of every expert, expert of every slot, last-use stamps) must
equal a host replay of the rule written out below, and a slot must hold its
expert's blob byte for byte.  Every cached call is also held to the oracle
directly: its routing and union lists (as the call left them in its
workspace) bit-exact, its output within 2e-3 * max|ref|.
"""
import ctypes

import numpy as np
import pytest
import torch

import int4_routed_expert_softmax_amd as moe
import oracle
from synth import configs

from moe_harness import DEV, DeviceLayer, assert_close, check_layer_routing, say

pytestmark = pytest.mark.gpu

INV = moe.MOE_BATCH_INVARIANT
NORM_RES = moe.MOE_PRENORM_RMS | moe.MOE_RESIDUAL


class LruReplay:
    """The placement rule on the host.  Per call the clock advances; union
    experts already in a slot keep it and take the new clock; the others, in
    ascending id, take the slots with the lowest (last use, slot index) and
    evict what those held."""

    def __init__(self, E, S):
        self.slot_of, self.expert_of, self.stamp = [0] * E, [0] * S, [0] * S
        self.clock = self.hits = self.misses = self.last_hits = self.last_misses = 0

    def call(self, union):
        self.clock += 1
        hits = [e for e in union if self.slot_of[e]]
        misses = sorted(e for e in union if not self.slot_of[e])
        for e in hits:
            self.stamp[self.slot_of[e] - 1] = self.clock
        free = sorted(range(len(self.stamp)), key=lambda s: (self.stamp[s], s))
        for e, v in zip(misses, free):
            if self.expert_of[v]:
                self.slot_of[self.expert_of[v] - 1] = 0
            self.expert_of[v], self.slot_of[e], self.stamp[v] = e + 1, v + 1, self.clock
        self.hits += len(hits)
        self.misses += len(misses)
        self.last_hits, self.last_misses = len(hits), len(misses)

    def words(self):
        head = [self.clock, self.hits, self.misses, self.last_hits, self.last_misses, 0, 0, 0]
        return np.array(head + self.slot_of + self.expert_of + self.stamp, dtype=np.int64)


class HostHome:
    """All E blobs of a layer in pinned host memory mapped into the device."""

    def __init__(self, blobs: np.ndarray):
        self.hip = ctypes.CDLL("libamdhip64.so.7")  # the runtime torch already loaded
        self.h = ctypes.c_void_p()
        n = blobs.nbytes
        assert self.hip.hipHostMalloc(ctypes.byref(self.h), ctypes.c_size_t(n), ctypes.c_uint(2)) == 0
        ctypes.memmove(self.h, blobs.ctypes.data, n)
        dptr = ctypes.c_void_p()
        assert self.hip.hipHostGetDevicePointer(ctypes.byref(dptr), self.h, ctypes.c_uint(0)) == 0
        bb = blobs.shape[1]
        self.table = torch.tensor([dptr.value + e * bb for e in range(blobs.shape[0])],
                                  dtype=torch.int64, device=DEV)

    def free(self):
        torch.cuda.synchronize()
        self.hip.hipHostFree(self.h)


class Cache:
    def __init__(self, L: DeviceLayer, home_table, S: int):
        self.L, self.home, self.S = L, home_table, S
        self.bb = moe.expert_blob_bytes(L.dims)
        self.slots = torch.empty(S * self.bb, dtype=torch.uint8, device=DEV)
        self.state = moe.make_cache_state(L.dims, S, DEV)
        self.replay = LruReplay(L.w.n_experts, S)

    def forward(self, xd, flags, out=None):
        L = self.L
        T = xd.shape[0]
        out = torch.empty(T, L.w.d, dtype=torch.float32, device=DEV) if out is None else out
        stats = torch.zeros(1 + L.w.n_experts, dtype=torch.int32, device=DEV)
        ws = moe.make_workspace(L.dims, T, DEV)
        moe.moe_layer_forward_cached(L.dims, xd, L.Wr_d, L.bias_d, self.home, self.slots, self.S,
                                     self.state, out, flags=flags, stats=stats, ws=ws)
        torch.cuda.synchronize()
        self.last_ws = ws
        return out, stats

    def check_state(self, union):
        self.replay.call(union)
        E, S = self.L.w.n_experts, self.S
        got = self.state.cpu().numpy()[:8 + E + 2 * S].astype(np.int64)
        assert np.array_equal(got, self.replay.words()), "cache state differs from the replay"

    def check_slots(self):
        held = self.state.cpu().numpy()[8 + self.L.w.n_experts:][:self.S]
        slots = self.slots.view(self.S, self.bb).cpu().numpy()
        for v, e1 in enumerate(held):
            if e1:
                assert np.array_equal(slots[v], self.L.blobs[e1 - 1]), f"slot {v} != expert {e1 - 1}"


def run_sequence(L: DeviceLayer, cache: Cache, steps, T, flags, bf16=False, in_place=False):
    w = L.w
    for step in steps:
        x, bf = configs.tokens(w, step=step, T=T)
        x = np.ascontiguousarray(x)
        xd = L.x_device(x, bf)
        ref, rst = L.forward(xd.clone(), flags=flags | (INV if T > 1 else 0))
        xc = xd.clone()
        out, st = cache.forward(xc, flags, out=xc if in_place else None)
        orc = oracle.layer_forward(x, L.Wr, L.bias, L.oracle_table(), w.d, w.f, w.top_k,
                                   x_bf16=bf, flags=flags, group=w.group, bits=w.bits)
        check_layer_routing(L.dims, cache.last_ws, T, orc, f"{w.name} cached step {step}")
        assert_close(out.cpu().numpy(), orc["out"], f"{w.name} cached step {step}",
                     case=f"{w.name} cached T={T} S={cache.S} flags={flags}")
        assert np.array_equal(out.cpu().numpy().view(np.uint32), ref.cpu().numpy().view(np.uint32)), \
            f"step {step}: cached output differs from the resident one"
        s, r = st.cpu().numpy(), rst.cpu().numpy()
        assert np.array_equal(s, r), f"step {step}: counts differ"
        union = [int(e) for e in np.nonzero(s[1:])[0]]
        cache.check_state(union)
    h = moe.cache_header(cache.state)
    say(f"cache: {w.name} T={T} S={cache.S} flags={flags}: {h['hits']} hits, {h['misses']} misses "
        f"over {h['clock']} calls")
    return h


@pytest.fixture(scope="module")
def glm():
    return DeviceLayer(configs.WORKLOADS["decode1"])


def test_decode_from_host_memory(glm):
    # the GLM-5.2-shaped layer at home in pinned host memory, 12 HBM slots
    say("cache: pinning 256 GLM experts in host memory")
    home = HostHome(glm.blobs)
    try:
        cache = Cache(glm, home.table, 12)
        h = run_sequence(glm, cache, range(10), 1, 0)
        assert h["hits"] > 0 and h["misses"] >= 8
        run_sequence(glm, cache, range(10, 14), 1, NORM_RES)
    finally:
        home.free()


def test_batches_from_device_home(glm):
    # batches of 4 (RMSNorm + residual, in place) with the home in other HBM
    cache = Cache(glm, glm.table, 32)
    run_sequence(glm, cache, range(6), 4, NORM_RES, in_place=True)


@pytest.mark.parametrize("w,S,T,bf16", [
    # slots exactly as many as a union can hold: every miss evicts
    (configs.Workload("cache_tight", d=512, f=512, n_experts=64, top_k=8, T=2, seed=41), 16, 2, False),
    # every expert fits: later calls hit only
    (configs.Workload("cache_all", d=256, f=128, n_experts=16, top_k=4, T=3, seed=42), 16, 3, False),
    (configs.Workload("cache_bf16", d=512, f=512, n_experts=32, top_k=4, T=1, seed=43,
                      x_kind="bf16"), 6, 1, True),
    # per-row int4 experts (one scale per row): slots of their own blob size
    (configs.Workload("cache_perrow", d=512, f=512, n_experts=64, top_k=8, T=2, seed=44,
                      group=0), 16, 2, False),
], ids=lambda v: v.name if hasattr(v, "name") else str(v))
def test_small_layers(w, S, T, bf16):
    L = DeviceLayer(w)
    home = HostHome(L.blobs)
    try:
        cache = Cache(L, home.table, S)
        run_sequence(L, cache, range(12), T, 0)
        cache.check_slots()
        if w.name == "cache_all":
            before = moe.cache_header(cache.state)
            run_sequence(L, cache, range(12), T, 0)
            after = moe.cache_header(cache.state)
            assert after["misses"] == before["misses"], "a repeated sequence missed with every expert resident"
    finally:
        home.free()


def test_int8_activations_from_device_home(glm):
    """MOE_INT8_ACT through the slot cache: bit-identical to the resident
    layer's integer-activation call (batch-invariant for batches)."""
    cache = Cache(glm, glm.table, 32)  # a batch of 4 can hold 32 distinct experts
    run_sequence(glm, cache, range(6), 1, moe.MOE_INT8_ACT)
    run_sequence(glm, cache, range(6, 10), 4, moe.MOE_INT8_ACT | NORM_RES, in_place=True)


def test_glm_perrow_decode_from_device_home():
    """The GLM-shaped layer with per-row experts, a new token per call, 12 slots."""
    L = DeviceLayer(configs.WORKLOADS["decode1_perrow"])
    cache = Cache(L, L.table, 12)
    run_sequence(L, cache, range(6), 1, 0)
    cache.check_slots()
