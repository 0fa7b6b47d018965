"""Markdown table of the parity margins a GPU test run logged.

    MOE_PARITY_LOG=margins.jsonl python -m pytest tests -m gpu ...
    python tests/summarize_margins.py margins.jsonl

Each line of the log is one comparison of a GPU output with the CPU oracle
(tests/moe_harness.py: case, rel_err = max-abs-error / max|ref|, tol).  The
table lists every case once, in the order the suite ran it, with the number of
comparisons and the worst ratio, then the headline workloads.
"""
import json
import sys

HEADLINE = [
    ("decode1 flags=0", "int8-digit GEMV (T=1)"),
    ("verify8 flags=0", "fp16 MFMA thin grouped GEMM"),
    ("verify8 INV flags=0", "batch-invariant GEMV"),
    ("prefill512 flags=0", "fp16 MFMA grouped GEMM, all 512 tokens"),
    ("prefill512 worst token (own max|ref|)", "worst single token against its own max|ref|"),
    ("chain48 step 0 worst of 48 layers", "GEMV, RMSNorm + residual, in place"),
    ("chain48 step 1 worst of 48 layers", "same"),
    ("chain48 step 63 worst of 48 layers", "same"),
    ("decode1 cached T=1 S=12 flags=0", "slot cache, host-mapped home"),
    ("decode1_int8 flags=0", "int8 codes, digit GEMV (T=1)"),
    ("verify8_int8 flags=0", "int8 codes, thin GEMM"),
    ("prefill512_int8 flags=0", "int8 codes, thin GEMM, all 512 tokens"),
    ("decode1_int2 flags=0", "int2 codes, digit GEMV (T=1)"),
    ("verify8_int2 flags=0", "int2 codes, thin GEMM"),
    ("prefill512_int2 flags=0", "int2 codes, thin GEMM, all 512 tokens"),
    ("decode1 flags=8", "integer activations, GEMV with int8 digits (T=1)"),
    ("verify8 flags=8", "integer activations, int8 matrix cores"),
    ("prefill512 flags=8", "integer activations, int8 matrix cores, all 512 tokens"),
]


def cell(text):
    return str(text).replace("|", "\\|")


def main(path):
    """Parity comparisons (against the oracle, bar REL_TOL) and the other
    bounded quantities (a `tol` of their own, such as the integer-activation
    layer's distance from the unquantised one) are tabulated apart."""
    worst, count, tols = {}, {}, {}
    with open(path) as fh:
        for line in fh:
            r = json.loads(line)
            c = r["case"]
            count[c] = count.get(c, 0) + 1
            worst[c] = max(worst.get(c, 0.0), r["rel_err"])
            tols[c] = r.get("tol")
    bar = min(t for t in tols.values() if t is not None)
    parity = [c for c in worst if tols[c] == bar]
    other = [c for c in worst if tols[c] != bar]
    wp = max(parity, key=worst.get)
    print(f"{len(parity)} parity cases, {sum(count[c] for c in parity)} comparisons, bar {bar:g}; "
          f"worst {worst[wp]:.2e} ({wp})\n")
    print("| case | comparisons | worst rel. error |")
    print("|---|---|---|")
    for c in parity:
        print(f"| {cell(c)} | {count[c]} | {worst[c]:.2e} |")
    if other:
        print("\nOther bounded quantities (each against its own bound):\n")
        print("| case | comparisons | worst | bound |")
        print("|---|---|---|---|")
        for c in other:
            print(f"| {cell(c)} | {count[c]} | {worst[c]:.2e} | {tols[c]:g} |")
    print("\nHeadline workloads:\n")
    print("| workload | path | rel. error |")
    print("|---|---|---|")
    for c, what in HEADLINE:
        if c in worst:
            print(f"| {cell(c)} | {cell(what)} | {worst[c]:.2e} |")


if __name__ == "__main__":
    main(sys.argv[1])
