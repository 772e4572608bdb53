"""AddressSanitizer + UndefinedBehaviorSanitizer runs of the host code.

* The fp64 oracle (oracle/oracle.c) built with gcc under both sanitizers
  and driven by tests/sanitize/oracle_driver.c: exact-size buffers around
  every tensor, per-head window array and row list; ragged and empty
  shapes, streaming tiles, row subsets, key chunks merged by
  oracle_combine, and each invalid-argument return.
* The C-ABI layer (online_softmax_tiled_amd/csrc/fa_api.hip) built with
  hipcc, sanitizers on the host pass only, linked with stand-ins for the
  kernel launchers that abort when reached, and driven by
  tests/sanitize/abi_driver.cpp: every entry point with arguments its
  checks must refuse, plus empty requests it must accept without a launch.
  No call reaches the HIP runtime, so no GPU is needed or touched.

Both drivers exit non-zero on a sanitizer report or a failed check.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = os.path.join(ROOT, "tests", "sanitize")
CSRC = os.path.join(ROOT, "online_softmax_tiled_amd", "csrc")
INCLUDE = os.path.join(ROOT, "include")


def _run(exe, leaks, cwd):
    env = dict(os.environ)
    env["ASAN_OPTIONS"] = f"detect_leaks={1 if leaks else 0}:abort_on_error=0:halt_on_error=1"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120, env=env, cwd=cwd)
    assert r.returncode == 0, f"{os.path.basename(exe)} exited {r.returncode}\n{r.stdout[-3000:]}\n{r.stderr[-6000:]}"
    assert "all checks passed" in r.stdout


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_oracle_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "oracle_driver")
    cmd = ["gcc", "-O1", "-g", "-std=c11", "-pthread", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-static-libasan",
           "-o", exe, os.path.join(ROOT, "oracle", "oracle.c"), os.path.join(SAN, "oracle_driver.c"), "-lm"]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-4000:]
    _run(exe, leaks=True, cwd=str(tmp_path))


def _hipcc():
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    return None


@pytest.mark.skipif(_hipcc() is None, reason="hipcc not available")
def test_abi_validation_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "abi_driver")
    # Sanitizers on the host pass only (each flag behind -Xarch_host); the
    # device pass of fa_api.hip holds no kernel, only the static scratch array.
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=all"]
    cmd = [_hipcc(), "--offload-arch=gfx950", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", *san,
           f"-I{INCLUDE}", f"-I{CSRC}", "-o", exe,
           os.path.join(CSRC, "fa_api.hip"), os.path.join(SAN, "launch_stubs.cpp"),
           os.path.join(SAN, "abi_driver.cpp")]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stderr[-4000:]
    # The HIP runtime library, loaded with the driver, keeps allocations of
    # its own until exit: leak detection is for the oracle run only.
    _run(exe, leaks=False, cwd=str(tmp_path))
