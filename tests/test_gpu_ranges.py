"""GPU parity of bf16 ranges inside the visual spans (MI355X).

Positions in a range are stored bf16 in the text plane, the coded positions
around them keep taking visual rows in order.  Stored bytes must equal the
oracle's, also when a store starts or ends inside a range; decode outputs
must be within the output tolerance of the oracle's fp64 attention on the
same stored cache, for sequences with ranges (static split) next to
sequences without (claimed steps), in the default split and in fixed
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


def _tiny_ranges():
    w = synth.tiny()
    w.bf16_ranges = [[(16, 17), (40, 72), (100, 101), (255, 256)]]
    return w


def _mixed(seed=11):
    """Three sequences, two layers, per-head widths with bf16 heads; the
    first and last sequences carry ranges, the middle one none."""
    kb = np.array([4, 16, 2, 8], dtype=np.uint8)
    vb = np.array([2, 16, 4, 8], dtype=np.uint8)
    w = synth.Workload("rngmix", 2, 3, 14, 2, 128, 64, [700, 90, 1500], [5, 0, 37],
                       [690, 64, 1500], [700, 90, 1500], kb, vb, seed=seed)
    w.bf16_ranges = [[(5, 6), (300, 333), (689, 690)], [],
                     synth.protected_tokens(seed, 37, 1500, 20) + [(1499, 1500)]]
    w.bf16_ranges[2] = sorted(set(w.bf16_ranges[2]))
    return w


def test_rng_quantize_tiny_bitexact():
    _say("bf16 ranges quantize tiny (fp32 source)")
    p = Pair(_tiny_ranges())
    p.store()
    assert p.mismatches() == 0


def test_rng_quantize_cut_inside_ranges_bitexact():
    """Stores in pieces whose edges fall inside ranges and coded pieces."""
    _say("bf16 ranges quantize in pieces")
    p = Pair(_tiny_ranges())
    for t0, t1 in ((0, 50), (50, 100), (100, 101), (101, 256)):
        p.store(t0=t0, t1=t1)
    assert p.mismatches() == 0


def test_rng_quantize_mixed_bitexact():
    _say("bf16 ranges quantize multi-sequence mixed widths")
    p = Pair(_mixed())
    p.store()
    assert p.mismatches() == 0


def test_rng_quantize_ragged_matches_per_sequence():
    """kvq_quantize_ragged over all sequences, each from its own start (one
    inside a range, one before the span, one inside the coded part), writes
    the oracle's bytes."""
    _say("bf16 ranges ragged quantize")
    import torch
    import oracle
    from kvq_testlib import as_f32, to_device_src
    w = _mixed(seed=12)
    p = Pair(w)
    starts, n = [310, 0, 700], 80
    for l in range(w.num_layers):
        k = np.stack([w.sources(l, [s], t, t + n, "k")[0] for s, t in enumerate(starts)])
        v = np.stack([w.sources(l, [s], t, t + n, "v")[0] for s, t in enumerate(starts)])
        kvq.kvq_quantize_ragged(p.cfg, p.cache, l, 1, [0, 1, 2], starts, n,
                                to_device_src(k[None]), to_device_src(v[None]))
        for s, t in enumerate(starts):
            for h in range(w.num_kv_heads):
                oracle.store_rows(p.ocfg, p.ocache, l, s, h, 0, t, t + n, as_f32(k[s, h]))
                oracle.store_rows(p.ocfg, p.ocache, l, s, h, 1, t, t + n, as_f32(v[s, h]))
    torch.cuda.synchronize()
    assert p.mismatches() == 0


def test_rng_decode_tiny():
    _say("bf16 ranges decode tiny")
    p = Pair(_tiny_ranges())
    p.store()
    got, ref = _decode_check(p, [256], what="rng tiny")
    assert kernel_error(got, ref, "rng tiny") <= 8e-4
    _decode_check(p, [73], what="rng tiny, length inside a range")


@pytest.mark.parametrize("chunk", [0, 1024])
def test_rng_decode_two_images(chunk):
    _say("bf16 ranges decode two images + protected tokens, chunk", chunk)
    p = Pair(synth.two_images())
    p.store()
    got, ref = _decode_check(p, p.w.capacity, chunk=chunk, what=f"two images chunk {chunk}")
    assert kernel_error(got, ref, f"two images chunk {chunk}") <= 8e-4


def test_rng_decode_mixed_static_and_claimed():
    _say("bf16 ranges decode multi-sequence mixed widths")
    p = Pair(_mixed())
    p.store()
    _decode_check(p, [700, 77, 1333], what="rng multi-seq")
    _decode_check(p, [690, 90, 1500], chunk=256, what="rng multi-seq chunk 256")


def test_rng_decode_36_ranges_rotated():
    """The most ranges a sequence may have, with rotated K codes."""
    _say("bf16 ranges decode 36 ranges, rotated K")
    kb, vb = np.full(2, 4, dtype=np.uint8), np.full(2, 2, dtype=np.uint8)
    w = synth.Workload("rng36", 1, 2, 8, 2, 128, 64, [2400, 2400], [10, 10], [2390, 2390],
                       [2400, 2400], kb, vb, seed=13, rotate_k=True)
    w.bf16_ranges = [[(20 + 60 * i, 21 + 60 * i + i % 5) for i in range(36)], [(10, 2390)]]
    p = Pair(w)
    p.store()
    assert p.mismatches() == 0
    got, ref = _decode_check(p, [2400, 2400], what="rng 36 rotated")
    assert kernel_error(got, ref, "rng 36 rotated") <= 8e-4
