"""The five synthetic workloads of the MoE layer, and their seeded inputs.

Shapes follow the GLM-5.2 layer the pages describe: 256 routed experts per
MoE layer with 8 chosen per token, about 19 MB of int4 weights per expert
(colibrì README (简体中文), 核心概念; colibri 技术解读 (linlog.top), "MoE 的稀疏性").
d = 6144 and f = 2048 give 3*d*f/2 = 18.87 MB of 4-bit codes per expert, which
is that figure; the gs64 fp16 scales add 1.18 MB.

Distributions (every draw seeded and counter based, see gen.c):
  x      ~ N(0, 1) fp32; the verify batch is base + 0.3*noise with a shared base;
           the prefill chunk is rounded to bf16 (round to nearest even)
  W_r    ~ N(0, 0.02) fp32, [E][d]
  bias   none for the tiny layer; -1.1*ln(e+1) (a Zipf(1.1) skew) otherwise
  codes  random bytes: every code uniform on its values (int4 on [-8, 7]; the
         int8 and int2 variants on [-128, 127] and [-2, 1])
  scales fp16 uniform on [0.005, 0.02)
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

from . import (T_H0, T_WR, T_X, T_XNOISE, blob_sizes, layer_blobs, normal, to_bf16_bits,
               zipf_bias, expert_blob)


@dataclass(frozen=True)
class Workload:
    name: str
    d: int
    f: int
    n_experts: int
    top_k: int
    T: int
    seed: int
    x_kind: str = "normal"      # normal | shared_base | bf16
    zipf: bool = True
    layers: int = 1
    steps: int = 1
    group: int = 64             # scale group: 64, or 0 for one scale per row
    bits: int = 4               # code width: 4 (int4), 8 (int8) or 2 (int2)

    @property
    def blob_bytes(self) -> int:
        nib, nsc = blob_sizes(self.d, self.f, self.group, self.bits)
        return nib + 2 * nsc

    @property
    def x_bf16(self) -> bool:
        return self.x_kind == "bf16"


WORKLOADS = {
    "tiny": Workload("tiny", d=256, f=128, n_experts=16, top_k=2, T=4, seed=1000, zipf=False),
    "decode1": Workload("decode1", d=6144, f=2048, n_experts=256, top_k=8, T=1, seed=1001),
    "verify8": Workload("verify8", d=6144, f=2048, n_experts=256, top_k=8, T=8, seed=1002,
                        x_kind="shared_base"),
    "prefill512": Workload("prefill512", d=6144, f=2048, n_experts=256, top_k=8, T=512,
                           seed=1003, x_kind="bf16"),
    "chain48": Workload("chain48", d=6144, f=2048, n_experts=256, top_k=8, T=1, seed=1004,
                        layers=48, steps=64),
    # the same layer with per-row int4 experts (one fp16 scale per weight row)
    "decode1_perrow": Workload("decode1_perrow", d=6144, f=2048, n_experts=256, top_k=8, T=1,
                               seed=1005, group=0),
    "verify8_perrow": Workload("verify8_perrow", d=6144, f=2048, n_experts=256, top_k=8, T=8,
                               seed=1006, x_kind="shared_base", group=0),
    "prefill512_perrow": Workload("prefill512_perrow", d=6144, f=2048, n_experts=256, top_k=8,
                                  T=512, seed=1007, x_kind="bf16", group=0),
    # the same layer with int8 and int2 codes (gs64 scales)
    "decode1_int8": Workload("decode1_int8", d=6144, f=2048, n_experts=256, top_k=8, T=1,
                             seed=1008, bits=8),
    "verify8_int8": Workload("verify8_int8", d=6144, f=2048, n_experts=256, top_k=8, T=8,
                             seed=1009, x_kind="shared_base", bits=8),
    "prefill512_int8": Workload("prefill512_int8", d=6144, f=2048, n_experts=256, top_k=8,
                                T=512, seed=1010, x_kind="bf16", bits=8),
    "decode1_int2": Workload("decode1_int2", d=6144, f=2048, n_experts=256, top_k=8, T=1,
                             seed=1011, bits=2),
    "verify8_int2": Workload("verify8_int2", d=6144, f=2048, n_experts=256, top_k=8, T=8,
                             seed=1012, x_kind="shared_base", bits=2),
    "prefill512_int2": Workload("prefill512_int2", d=6144, f=2048, n_experts=256, top_k=8,
                                T=512, seed=1013, x_kind="bf16", bits=2),
}


def router(w: Workload, layer: int = 0):
    """(W_r [E][d] fp32, bias [E] fp32 or None)."""
    wr = normal(w.seed, layer, T_WR, w.n_experts * w.d, std=0.02).reshape(w.n_experts, w.d)
    bias = zipf_bias(w.n_experts) if w.zipf else None
    return wr, bias


def tokens(w: Workload, step: int = 0, T: int | None = None):
    """Layer input for one step.  Returns (x, is_bf16): x is fp32 [T][d], or the
    uint16 bf16 bit patterns [T][d] for the prefill chunk."""
    T = w.T if T is None else T
    n = T * w.d
    if w.x_kind == "shared_base":
        base = normal(w.seed, step, T_X, w.d)
        noise = normal(w.seed, step, T_XNOISE, n).reshape(T, w.d)
        x = (base[None, :].astype(np.float64) + 0.3 * noise.astype(np.float64)).astype(np.float32)
        return x, False
    x = normal(w.seed, step, T_X if w.layers == 1 else T_H0, n).reshape(T, w.d)
    if w.x_kind == "bf16":
        return to_bf16_bits(x), True
    return x, False


def experts(w: Workload, layer: int = 0, e0: int = 0, ne: int | None = None):
    """Expert blobs [ne][blob_bytes] uint8 of one layer."""
    ne = w.n_experts - e0 if ne is None else ne
    return layer_blobs(w.seed, layer, ne, w.d, w.f, e0=e0, group=w.group, bits=w.bits)


def one_expert(w: Workload, layer: int, e: int):
    return expert_blob(w.seed, layer, e, w.d, w.f, group=w.group, bits=w.bits)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (b.astype(np.uint32) << 16).view(np.float32)
