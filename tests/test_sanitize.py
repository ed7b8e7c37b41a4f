"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU
only; any report aborts the run):
  * oracle/oracle.c, every routine driven once by tests/native/oracle_sanitize.c
    (gcc -fsanitize=address,undefined);
  * the C ABI's argument layer, fa_api.hip, compiled for the host with the
    sanitizers and linked against stub launchers that record each launch
    (tests/native/abi_sanitize.hip): valid calls reach one launcher with the
    caller's sizes, invalid ones return an error and launch nothing.
The device side of fa_api.hip is built as usual (no GPU sanitizer)."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
NATIVE = os.path.join(ROOT, "tests", "native")


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, (" ".join(cmd)) + "\n" + r.stdout + r.stderr
    return r


def test_oracle_under_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle_sanitize")
    _run(["gcc", "-O1", "-g", "-std=gnu11", "-fsanitize=address,undefined",
          "-fno-sanitize-recover=all", "-pthread", os.path.join(ROOT, "oracle", "oracle.c"),
          os.path.join(NATIVE, "oracle_sanitize.c"), "-o", exe, "-lm"])
    r = _run([exe], timeout=120)
    assert r.stdout.strip() == "ok"


def test_abi_layer_under_sanitizers(tmp_path):
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    clangxx = "/opt/rocm/llvm/bin/clang++"
    if not os.path.exists(hipcc) or not os.path.exists(clangxx):
        pytest.fail("ROCm hipcc and clang++ are required")
    # host-side sanitizers only: each -fsanitize= goes after -Xarch_host
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=all"]
    common = ["--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC", *san, "-I",
              os.path.join(ROOT, "include")]
    api = str(tmp_path / "fa_api.o")
    drv = str(tmp_path / "drv.o")
    exe = str(tmp_path / "abi_sanitize")
    _run([hipcc, *common, "-c", os.path.join(ROOT, "flashattention_online_softmax_fa_amd",
                                             "csrc", "fa_api.hip"), "-o", api])
    _run([hipcc, *common, "-c", os.path.join(NATIVE, "abi_sanitize.hip"), "-o", drv])
    _run([clangxx, "-fsanitize=address,undefined", api, drv, "-L/opt/rocm/lib", "-lamdhip64",
          "-Wl,-rpath,/opt/rocm/lib", "-o", exe])
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0")  # the HIP runtime's own allocations
    r = _run([exe], timeout=120, env=env)
    assert r.stdout.strip() == "ok"
