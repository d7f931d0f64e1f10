"""The ABI shim's host code under AddressSanitizer and UndefinedBehaviorSanitizer
(CPU only): every library source is rebuilt with the sanitizers on its host
side, linked with tests/c/abi_args.cpp, and run.  That program drives every
entry point's argument checks (the same cases as test_abi.py, plus sizes at
and beyond every limit) and sweeps the workspace-size calls over the largest
admitted sizes, so an out-of-bounds host access or an overflowing signed
product in the size arithmetic stops it.  No call reaches a launch: no GPU
is used."""
import os
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "diffusion_speculative_verification_amd", "csrc")
SOURCES = ["abi", "accept", "attn", "commit", "coupled", "route", "states"]
# the sanitizers instrument the host side only (device code is built as usual)
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]
COMMON = ["-O1", "-std=c++17", "-Xarch_host", "-g", "-I" + os.path.join(ROOT, "include")]


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, " ".join(cmd) + "\n" + r.stdout[-3000:] + r.stderr[-3000:]
    return r


@pytest.mark.timeout(900)
def test_abi_checks_under_sanitizers(tmp_path):
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc):
        pytest.skip("hipcc not found")
    objs = []

    def compile_one(name):
        obj = str(tmp_path / (name + ".o"))
        _run([hipcc, "--offload-arch=gfx950", "-fPIC", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
              *COMMON, *SAN, "-c", os.path.join(CSRC, name + ".hip"), "-o", obj])
        return obj

    with ThreadPoolExecutor(max_workers=4) as ex:
        objs = list(ex.map(compile_one, SOURCES))
    main_obj = str(tmp_path / "abi_args.o")
    _run([hipcc, *COMMON, *SAN, "-c", os.path.join(ROOT, "tests", "c", "abi_args.cpp"), "-o", main_obj])
    exe = str(tmp_path / "abi_args")
    _run([hipcc, *SAN, main_obj, *objs, "-o", exe])
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=env)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "runtime error" not in out and "AddressSanitizer" not in out, out[-4000:]
    assert " 0 failures" in r.stdout, out[-4000:]
    print(r.stdout.strip().splitlines()[-1])
