"""Writes tiny_layer.json: the oracle's result on the tiny workload (d=256,
f=128, 16 experts, top-2, 4 tokens).  It calls only the oracle and the seeded
input generator; nothing here comes from the GPU path.  Run from the repo root:
    python tests/golden/make_golden.py
"""
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
from synth import configs  # noqa: E402


def main():
    w = configs.WORKLOADS["tiny"]
    Wr, bias = configs.router(w)
    x, _ = configs.tokens(w)
    r = oracle.layer_forward(x, Wr, bias, list(configs.experts(w)), w.d, w.f, w.top_k)
    g = dict(workload="tiny", seed=w.seed, idx=r["idx"].tolist(), w=r["w"].tolist(),
             uniq=r["uniq"].tolist(), offsets=r["offsets"].tolist(), rows=r["rows"].tolist(),
             out=r["out"].tolist())
    with open(os.path.join(os.path.dirname(os.path.abspath(__file__)), "tiny_layer.json"), "w") as fh:
        json.dump(g, fh)


if __name__ == "__main__":
    main()
