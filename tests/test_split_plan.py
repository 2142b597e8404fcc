"""Host-side check of the matrix-core decode split (no GPU).

Builds tests/split_replay.cpp -- the library's planning code with recording
stubs in place of the kernel launchers -- and runs it: every token of every
(layer, seq, head) must be processed by exactly one wave or piece, and every
partial index must fit the workspace.
"""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)


def _hipcc():
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    return None


def test_split_covers_every_token_once(tmp_path):
    cc = _hipcc()
    if cc is None:
        pytest.skip("hipcc not available")
    exe = str(tmp_path / "split_replay")
    build = subprocess.run(
        [cc, "-O1", "-std=c++17", "-x", "hip", "--offload-arch=gfx950",
         "-I", os.path.join(ROOT, "include"),
         "-I", os.path.join(ROOT, "quantized_decode_attention_quantize_amd", "csrc"),
         os.path.join(HERE, "split_replay.cpp"), "-o", exe],
        capture_output=True, text=True, timeout=300)
    assert build.returncode == 0, build.stderr[-2000:]
    run = subprocess.run([exe], capture_output=True, text=True, timeout=300)
    assert run.returncode == 0 and run.stdout.strip().endswith("ok"), run.stdout[-3000:]
