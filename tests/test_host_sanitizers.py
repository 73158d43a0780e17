"""The library's host layer (argument checks, workspace layout, dispatch
readout) under AddressSanitizer and UndefinedBehaviorSanitizer, on the CPU.

The sources are built once more with the sanitizers on the host side only
(GPU code is built as usual but never runs here), and the C-ABI tests of
tests/test_abi.py run in a child process against that build with the
sanitizer runtime preloaded; any report ends the child with an error."""

from __future__ import annotations

import glob
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = "/opt/rocm/bin/hipcc"


def _asan_runtime():
    found = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return found[-1] if found else None


@pytest.mark.skipif(not os.path.exists(HIPCC) or _asan_runtime() is None,
                    reason="hipcc or the sanitizer runtime is not installed")
def test_abi_checks_clean_under_host_sanitizers(tmp_path):
    lib = tmp_path / "libmoe_sanitized.so"
    src = sorted(glob.glob(os.path.join(ROOT, "mixture_experts_ffn_renorm_amd", "csrc", "*.hip")))
    host_san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                "-Xarch_host", "-fno-omit-frame-pointer", "-shared-libsan"]
    cmd = [HIPCC, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC", "-shared",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", *host_san,
           "-I", os.path.join(ROOT, "include"),
           "-I", os.path.join(ROOT, "mixture_experts_ffn_renorm_amd", "csrc"), *src, "-o", str(lib)]
    b = subprocess.run(cmd, capture_output=True, text=True, timeout=900)
    assert b.returncode == 0, b.stderr[-2000:]

    driver = (
        "import sys\n"
        f"sys.path.insert(0, {ROOT!r})\n"
        "import mixture_experts_ffn_renorm_amd as m\n"
        f"m.LIB_PATH = {str(lib)!r}\n"
        "import pytest\n"
        "sys.exit(pytest.main(['-q', '-p', 'no:cacheprovider', '-m', 'not gpu', "
        f"{os.path.join(ROOT, 'tests', 'test_abi.py')!r}]))\n")
    env = dict(os.environ)
    env["LD_PRELOAD"] = _asan_runtime()
    env["ASAN_OPTIONS"] = "detect_leaks=0:halt_on_error=1:abort_on_error=0"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    r = subprocess.run([sys.executable, "-c", driver], capture_output=True, text=True,
                       timeout=900, cwd=ROOT, env=env)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "passed" in r.stdout
    assert "ERROR: AddressSanitizer" not in out and "runtime error:" not in out
