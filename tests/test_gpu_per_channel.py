"""GPU parity of per-channel K groups with a bf16 residual window (MI355X).

Stored bytes must equal the oracle's (the block kernel writes coded K rows
and per-block META rows; every other row goes through the per-token
kernel); decode outputs must be within the output tolerance of the oracle's
fp64 attention on the same stored cache, in the default split and in fixed
chunks.  Every case prints its name before touching the GPU.
"""
import sys

import numpy as np
import pytest

from quantized_decode_attention_quantize_amd import kvq, synth

from kvq_testlib import Pair, assert_close, kernel_error

pytestmark = pytest.mark.gpu


def _say(*a):
    print("[case]", *a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    kvq.lib()
    yield


def _pc(w):
    w.k_per_channel = True
    return w


def _decode_check(p, lens, chunk=0, what=""):
    w = p.w
    out, q = p.decode(lens, chunk=chunk)
    got, ref = [], []
    for l in range(w.num_layers):
        for s in range(w.batch):
            for i in range(w.num_q_heads):
                ref.append(p.oracle_decode(l, s, i, lens[s], q[l, s, i]))
                got.append(out[l, s, i])
    got, ref = np.array(got), np.array(ref)
    assert_close(got, ref, what)
    return got, ref


def test_pc_quantize_tiny_bitexact():
    _say("per-channel quantize tiny (fp32 source, residual 10)")
    w = _pc(synth.tiny())
    w.vis_end = [250]  # coded [16, 240), residual [240, 250)
    p = Pair(w)
    p.store()
    assert p.mismatches() == 0


@pytest.mark.parametrize("D,g", [(64, 32), (64, 64), (128, 32), (128, 64), (128, 128)])
def test_pc_quantize_widths_and_groups_bitexact(D, g):
    _say("per-channel quantize D/g", D, g)
    kb = np.array([4, 2, 8, 16], dtype=np.uint8)
    vb = np.array([2, 4, 8, 16], dtype=np.uint8)
    w = _pc(synth.Workload(f"pc{D}_{g}", 1, 3, 4, 4, D, g, [300, 1, 700], [5, 0, 20],
                           [290, 1, 700], [300, 1, 700], kb, vb, seed=D + g))
    p = Pair(w)
    p.store()
    assert p.mismatches() == 0


def test_pc_quantize_llava_layer_bitexact():
    _say("per-channel quantize llava layer (bf16 source, residual 1)")
    p = Pair(_pc(synth.llava_layer(kbits=4, vbits=2)))
    p.store()
    assert p.mismatches() == 0


def test_pc_decode_tiny():
    _say("per-channel decode tiny")
    w = _pc(synth.tiny())
    w.vis_end = [250]
    p = Pair(w)
    p.store()
    got, ref = _decode_check(p, [256], what="pc tiny")
    assert kernel_error(got, ref, "pc tiny") <= 8e-4


@pytest.mark.parametrize("chunk", [0, 256, 1024])
def test_pc_decode_llava_layer(chunk):
    _say("per-channel decode llava layer, chunk", chunk)
    p = Pair(_pc(synth.llava_layer(seed=3, kbits=4, vbits=2)))
    p.store()
    got, ref = _decode_check(p, [6287], chunk=chunk, what=f"pc llava chunk {chunk}")
    assert kernel_error(got, ref, f"pc llava chunk {chunk}") <= 8e-4


def test_pc_decode_multiseq_mixed_widths():
    """Three sequences with spans starting off the 32-token grid (so the
    decode's step grid is shifted per sequence), per-head widths including
    bf16 heads, two layers, shorter attended lengths."""
    _say("per-channel decode multi-sequence mixed widths")
    kb = np.array([4, 16, 2, 8], dtype=np.uint8)
    vb = np.array([2, 16, 4, 8], dtype=np.uint8)
    w = _pc(synth.Workload("pcmix", 2, 3, 14, 2, 128, 64, [700, 90, 1500], [5, 0, 37],
                           [690, 64, 1500], [700, 90, 1500], kb, vb, seed=9))
    p = Pair(w)
    p.store()
    _decode_check(p, [700, 77, 1333], what="pc multi-seq")
    _decode_check(p, [700, 77, 1333], chunk=256, what="pc multi-seq chunk 256")
