"""GPU parity of query-head subgroups together with every cache feature.

A KV head whose (query head, group) columns exceed one 16-wide matrix-core
tile is decoded in several launches, one per subgroup of its query heads.
These cases run that path with rotated K, per-channel K and bf16 ranges, and
check every output against the oracle.  Every case prints its name before
touching the GPU.
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


def _wide(name, hq, hkv, g, seed, **features):
    """Two layers, two sequences; 28/4 heads at g = 32 is two subgroups of 4
    and 3 query heads, 16/1 at g = 32 four subgroups of 4."""
    kb = np.array([4, 8, 2, 4] * 2, np.uint8)[: 2 * hkv]
    vb = np.array([2, 4, 4, 8] * 2, np.uint8)[: 2 * hkv]
    w = synth.Workload(name, 2, 2, hq, hkv, 128, g, [900, 333], [14, 0], [894, 320],
                       [900, 333], kb, vb, seed=seed)
    for k, v in features.items():
        setattr(w, k, v)
    return w


CASES = [
    ("plain 28/4", dict(hq=28, hkv=4, g=32)),
    ("rotated 28/4", dict(hq=28, hkv=4, g=32, rotate_k=True)),
    ("per-channel 28/4", dict(hq=28, hkv=4, g=32, k_per_channel=True)),
    ("ranges 28/4", dict(hq=28, hkv=4, g=32,
                         bf16_ranges=[[(14, 15), (400, 420), (893, 894)], [(0, 1), (100, 164)]])),
    ("per-channel 16/1", dict(hq=16, hkv=1, g=32, k_per_channel=True)),
    ("ranges 16/1", dict(hq=16, hkv=1, g=32, bf16_ranges=[[(30, 31)], [(5, 9), (300, 320)]])),
]


@pytest.mark.parametrize("name,spec", CASES, ids=[c[0] for c in CASES])
def test_subgroup_decode_with_features(name, spec):
    _say("subgroups:", name)
    spec = dict(spec)
    hq, hkv, g = spec.pop("hq"), spec.pop("hkv"), spec.pop("g")
    w = _wide(name, hq, hkv, g, seed=hq * 7 + g, **spec)
    p = Pair(w)
    p.store()
    assert p.mismatches() == 0
    for lens, chunk in (([900, 333], 0), ([777, 200], 256)):
        out, q = p.decode(lens, chunk=chunk)
        jobs = [(l, s, i, lens[s], q[l, s, i]) for l in range(w.num_layers)
                for s in range(w.batch) for i in range(w.num_q_heads)]
        ref = np.array(p.oracle_decode_many(jobs))
        got = np.array([out[l, s, i] for (l, s, i, _, _) in jobs])
        assert_close(got, ref, f"{name} chunk {chunk}")
        assert kernel_error(got, ref, f"{name} chunk {chunk}") <= 8e-4
