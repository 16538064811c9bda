"""libsdpa's host layer under AddressSanitizer and UndefinedBehaviorSanitizer
(CPU only).  head_attention_fwd_amd/csrc/sdpa_api.hip (argument checks, launch
planning, workspace sizing, the per-device scratch lookup) is built with the
sanitizers on its host code only (-Xarch_host before each -fsanitize=) and
linked with stand-ins for the kernel launchers (tests/abi_launcher_stubs.cpp);
the whole CPU ABI battery then runs against it in a fresh process with clang's
ASan runtime preloaded.  Any out-of-bounds access or undefined behaviour aborts
the child, and so does a call that reaches a launcher where none should."""
import glob
import os
import subprocess
import sys

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(ROOT, "head_attention_fwd_amd", "csrc")
HIPCC = "/opt/rocm/bin/hipcc"
SAN = ["-Xarch_host", "-fsanitize=address,undefined", "-Xarch_host", "-fno-omit-frame-pointer",
       "-Xarch_host", "-fno-sanitize-recover=all", "-shared-libsan"]

PLANTED = r"""
#include <stdlib.h>
extern "C" int planted_overrun(int n)
{
    int *a = (int *)malloc(n * sizeof(int));
    for (int i = 0; i <= n; ++i) a[i] = i;   // one element past the end
    int s = a[n - 1];
    free(a);
    return s;
}
"""


def _asan_runtime():
    found = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not found or not os.path.exists(HIPCC):
        pytest.skip("no ROCm clang ASan runtime in this image")
    return found[-1]


def _hipcc(sources, out):
    cmd = [HIPCC, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC", "-shared",
           "-Wno-unused-command-line-argument", "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"] + SAN + sources + ["-o", out]
    res = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
    assert res.returncode == 0, res.stderr[-4000:]


def _child(args, runtime):
    env = dict(os.environ)
    env["LD_PRELOAD"] = runtime
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    return subprocess.run([sys.executable, os.path.join(HERE, "sanitized_abi_child.py")] + args,
                          capture_output=True, text=True, env=env, timeout=600)


@pytest.fixture(scope="module")
def sanitized(tmp_path_factory):
    runtime = _asan_runtime()
    d = tmp_path_factory.mktemp("abi_san")
    lib = str(d / "libsdpa_host_san.so")
    _hipcc([os.path.join(CSRC, "sdpa_api.hip"), os.path.join(HERE, "abi_launcher_stubs.cpp")], lib)
    return runtime, lib, d


def test_sanitizer_catches_a_planted_overrun(sanitized):
    """Control: host code built by the same command with a one-past-the-end heap
    write must be stopped with a heap buffer overflow report."""
    runtime, lib, d = sanitized
    src = d / "planted.cpp"
    src.write_text(PLANTED)
    ctl = str(d / "libplanted.so")
    _hipcc([str(src)], ctl)
    res = _child([lib, ctl], runtime)
    assert res.returncode != 0
    assert "heap-buffer-overflow" in res.stderr
    assert "planted overrun returned" not in res.stdout


def test_host_layer_under_asan_and_ubsan(sanitized):
    runtime, lib, _ = sanitized
    res = _child([lib], runtime)
    assert res.returncode == 0, res.stdout[-3000:] + res.stderr[-4000:]
    assert "sanitized host layer: launcher calls 0" in res.stdout
    assert "ERROR: AddressSanitizer" not in res.stderr
    assert "runtime error" not in res.stderr
