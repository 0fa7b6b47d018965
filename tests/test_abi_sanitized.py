"""The C ABI's host-side argument validation under AddressSanitizer and
UndefinedBehaviorSanitizer: the library's sources built with the sanitizers on
the host code only (the device code is built as usual and never runs: every
call in tests/abi_validation_check.c is refused before any HIP call, so no GPU
is involved), every sanitizer report fatal."""
import glob
import os
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "int4_routed_expert_softmax_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not installed")
def test_abi_validation_clean_under_asan_and_ubsan(tmp_path):
    exe = str(tmp_path / "abi_validation_check")
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=all"]
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip"))) + [os.path.join(CSRC, "moe_abi.cpp")]
    objs = [str(tmp_path / (os.path.basename(src) + ".o")) for src in srcs]

    def compile_one(src_obj):
        src, obj = src_obj
        subprocess.check_call([HIPCC, "--offload-arch=gfx950", "-O1", "-g",
                               "-fno-omit-frame-pointer", "-std=c++17", *san,
                               "-I", os.path.join(ROOT, "include"), "-c", src, "-o", obj])

    with ThreadPoolExecutor(max_workers=4) as pool:
        list(pool.map(compile_one, zip(srcs, objs)))
    drv = str(tmp_path / "drv.o")
    subprocess.check_call([HIPCC, "-x", "c", "-O1", "-g", *san, "-I", os.path.join(ROOT, "include"),
                           "-c", os.path.join(ROOT, "tests", "abi_validation_check.c"), "-o", drv])
    subprocess.check_call([HIPCC, *san, "-o", exe, drv, *objs])
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:halt_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120, env=env)
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-4000:]
    assert "abi validation: all ok" in r.stdout
