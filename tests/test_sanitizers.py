"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

- The oracle (plain C) is built with gcc and both sanitizers and driven
  through every entry point on small caches (tests/oracle_sanitize_driver.c).
- The library's host side (validation, layout, split planning, argument
  packing) is built into tests/split_replay.cpp with the sanitizers on the
  host half of the compilation only, and replays its plans.
Any sanitizer report aborts the program, which fails the test.
"""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
           UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")


def test_oracle_under_asan_ubsan(tmp_path):
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc not available")
    exe = str(tmp_path / "oracle_san")
    san = ["-fsanitize=address", "-fsanitize=undefined", "-fno-sanitize-recover=all"]
    build = subprocess.run(
        [gcc, "-std=c11", "-O1", "-g", "-ffp-contract=off", *san,
         os.path.join(HERE, "oracle_sanitize_driver.c"), os.path.join(ROOT, "oracle", "kvq_oracle.c"),
         "-o", exe, "-lm"], capture_output=True, text=True, timeout=300)
    assert build.returncode == 0, build.stderr[-3000:]
    run = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=ENV)
    assert run.returncode == 0 and run.stdout.strip().endswith("ok"), (run.stdout + run.stderr)[-3000:]


def _hipcc():
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    return None


def test_host_planner_under_asan_ubsan(tmp_path):
    cc = _hipcc()
    if cc is None:
        pytest.skip("hipcc not available")
    exe = str(tmp_path / "split_replay_san")
    host_san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                "-Xarch_host", "-fno-sanitize-recover=all"]
    build = subprocess.run(
        [cc, "-O1", "-g", "-std=c++17", "-x", "hip", "--offload-arch=gfx950", *host_san,
         "-I", os.path.join(ROOT, "include"),
         "-I", os.path.join(ROOT, "quantized_decode_attention_quantize_amd", "csrc"),
         os.path.join(HERE, "split_replay.cpp"), "-o", exe],
        capture_output=True, text=True, timeout=600)
    assert build.returncode == 0, build.stderr[-3000:]
    run = subprocess.run([exe], capture_output=True, text=True, timeout=600, env=ENV)
    assert run.returncode == 0 and run.stdout.strip().endswith("ok"), (run.stdout + run.stderr)[-3000:]
