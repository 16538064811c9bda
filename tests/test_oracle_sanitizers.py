"""The oracle's C code under AddressSanitizer and UndefinedBehaviorSanitizer
(CPU only): built with -fsanitize=address,undefined, it runs the whole pin
battery and exhaustive tiny cases (every key length, both masks, several
radii, the row and multi-head variants) in a fresh Python process with the
ASan runtime preloaded.  Any out-of-bounds access, use of freed memory or
undefined behaviour aborts the child and fails the test."""
import os
import subprocess
import sys

import oracle

HERE = os.path.dirname(os.path.abspath(__file__))


def _runtime(name):
    path = subprocess.run(["gcc", "-print-file-name=" + name], capture_output=True, text=True,
                          check=True).stdout.strip()
    assert os.path.isabs(path) and os.path.exists(path), "gcc has no %s" % name
    return path


def _run_sanitized(src, lib):
    subprocess.run(["gcc", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
                    "-fno-sanitize-recover=all", "-fopenmp", "-shared", "-fPIC", "-std=c11",
                    "-Wall", "-Wextra", "-o", lib, src, "-lm"], check=True)
    env = dict(os.environ)
    env["LD_PRELOAD"] = _runtime("libasan.so")
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    env["OMP_NUM_THREADS"] = "4"
    return subprocess.run([sys.executable, os.path.join(HERE, "sanitized_oracle_child.py"), lib],
                          capture_output=True, text=True, env=env, timeout=600)


def test_sanitizer_catches_a_planted_overrun(tmp_path):
    """Control: the same harness on an oracle copy whose normalisation loop writes
    one element past its scratch row must report a heap buffer overflow."""
    src = open(oracle.SOURCE, encoding="utf-8").read()
    line = "for (int64_t j = 0; j < Lk; ++j) w[j] = w[j] / Z;"
    assert line in src
    bad = tmp_path / "sdpa_oracle_overrun.c"
    bad.write_text(src.replace(line, "for (int64_t j = 0; j <= Lk; ++j) w[j] = w[j] / Z;"))
    res = _run_sanitized(str(bad), str(tmp_path / "libsdpa_oracle_overrun.so"))
    assert res.returncode != 0
    assert "heap-buffer-overflow" in res.stderr


def test_oracle_under_asan_and_ubsan(tmp_path):
    res = _run_sanitized(oracle.SOURCE, str(tmp_path / "libsdpa_oracle_asan.so"))
    assert res.returncode == 0, res.stdout[-2000:] + res.stderr[-4000:]
    assert "sanitized oracle:" in res.stdout
    assert "ERROR: AddressSanitizer" not in res.stderr
    assert "runtime error" not in res.stderr
