"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

* The C-ABI library is rebuilt with the sanitizers on its host side (hipcc
  `-Xarch_host -fsanitize=...`; the gfx950 device code is unchanged and never
  runs here) and driven by tests/sanitize/abi_check_main.c through every
  *_check entry point with valid and invalid descriptors.
* The C oracle (oracle/ref.c) is built with gcc's sanitizers and driven by
  tests/sanitize/oracle_main.c over every mask kind and sink mode on small
  inputs in exact-size heap buffers.

Both programs exit non-zero on an unexpected result, and the sanitizers abort
on any invalid access or undefined operation."""
from __future__ import annotations

import glob
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "sanitize")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def _run(cmd, env=None, cwd=None):
    r = subprocess.run(cmd, capture_output=True, text=True, env=env, cwd=cwd)
    noise = "is not a recognized feature for this target"
    msgs = "\n".join(ln for ln in (r.stdout + r.stderr).splitlines() if noise not in ln)
    assert r.returncode == 0, f"{cmd[0]} exited {r.returncode}:\n{msgs[-4000:]}"
    assert "runtime error" not in msgs and "AddressSanitizer" not in msgs, msgs[-4000:]
    return msgs


def test_oracle_under_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle_san")
    _run(["gcc", "-std=c11", "-O1", "-g", "-fopenmp", "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
          "-fno-omit-frame-pointer", os.path.join(ROOT, "oracle", "ref.c"), os.path.join(HERE, "oracle_main.c"),
          "-o", exe, "-lm"])
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1", OMP_NUM_THREADS="2")
    assert "all cases clean" in _run([exe], env=env)


@pytest.mark.skipif(not os.path.exists(os.path.join(ROCM, "bin", "hipcc")), reason="hipcc not installed")
def test_abi_validation_under_sanitizers(tmp_path):
    lib = str(tmp_path / "libattn_sink_san.so")
    srcs = sorted(glob.glob(os.path.join(ROOT, "sink_aware_masked_amd", "csrc", "*.hip"))) + \
        sorted(glob.glob(os.path.join(ROOT, "sink_aware_masked_amd", "csrc", "*.cpp")))
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]
    _run([os.path.join(ROCM, "bin", "hipcc"), "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC", "-shared",
          "-fvisibility=hidden", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", *san,
          "-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROOT, "sink_aware_masked_amd", "csrc"),
          *srcs, "-o", lib])
    cc = os.path.join(ROCM, "bin", "amdclang")
    cc = cc if os.path.exists(cc) else shutil.which("clang")
    exe = str(tmp_path / "abi_san")
    _run([cc, "-std=c11", "-g", "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROCM, "include"),
          "-I", os.path.join(ROOT, "include"), "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
          os.path.join(HERE, "abi_check_main.c"), "-o", exe, lib, f"-Wl,-rpath,{tmp_path}"])
    # the HIP runtime keeps allocations for the process lifetime: leaks are not checked
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1")
    assert "all statuses as expected" in _run([exe], env=env)
