"""kvq_decode_attention_noalloc (the decode with the library's own scratch)
against kvq_decode_attention on the same caches, through the C ABI.

Fixed chunks assign every token statically, so the two entry points must give
identical bytes; the library's default split (steps handed to waves as they
finish) must agree within the output tolerance.  Calls run back to back on
one device with shapes that shrink from call to call, so each call finds the
scratch as the previous, larger one left it.
"""
import sys

import numpy as np
import pytest

from quantized_decode_attention_quantize_amd import kvq, synth

from kvq_testlib import Pair, assert_close, bf16_device, bf16_to_f64

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


def _both(p, lens, chunk, nl=None):
    """(workspace entry point's output, no-alloc entry point's output) as f64."""
    import torch
    w = p.w
    nl = w.num_layers if nl is None else nl
    q = bf16_device(np.stack([w.q_bits(i) for i in range(nl)]))
    lens_d = torch.tensor(np.asarray(lens, dtype=np.int32), device="cuda")
    out_ws, out_na = torch.empty_like(q), torch.empty_like(q)
    ws = torch.zeros(kvq.workspace_bytes(p.cfg, nl, chunk), dtype=torch.uint8, device="cuda")
    kvq.kvq_decode_attention(p.cfg, p.cache, 0, nl, lens_d, q, out_ws, w.sm_scale, chunk, ws)
    kvq.kvq_decode_attention_noalloc(p.cfg, p.cache, 0, nl, lens_d, q, out_na, w.sm_scale, chunk)
    torch.cuda.synchronize()
    return bf16_to_f64(out_ws), bf16_to_f64(out_na)


def test_noalloc_matches_workspace_decode_shrinking_calls():
    # first call: one LLaVA layer with a split that merges partials (7 per
    # (seq, KV head) at 1,024-token chunks), then the default split
    _say("noalloc: llava layer, chunks 1024 then default")
    big = Pair(synth.llava_layer(kbits=4, vbits=2))
    big.store(oracle_too=False)
    lens_big = [big.w.capacity[0]]
    a, b = _both(big, lens_big, 1024)
    assert np.array_equal(a, b)
    a, b = _both(big, lens_big, 0)
    assert_close(b, a, "noalloc vs workspace, llava layer default split")
    # second call, smaller: the tiny case (one KV head, 256 tokens, D = 64)
    _say("noalloc: tiny, chunks 64 then default")
    small = Pair(synth.tiny())
    small.store(oracle_too=False)
    for chunk in (64, 0):
        a, b = _both(small, [256], chunk)
        assert np.array_equal(a, b) if chunk else True
        assert_close(b, a, f"noalloc vs workspace, tiny chunk {chunk}")
    # a shorter attended length on the first cache again, after the small call
    _say("noalloc: llava layer again, 3000 tokens, chunks 512")
    a, b = _both(big, [3000], 512)
    assert np.array_equal(a, b)


def test_noalloc_refuses_beyond_its_scratch():
    """A call whose partials exceed the fixed scratch is refused before any
    launch (batched serving at 32-token chunks needs about 477 MB)."""
    import torch
    w = synth.ragged_serving()
    cfg = kvq.Config.from_workload(w)
    cache = torch.zeros(kvq.kvq_cache_bytes(cfg)["total_bytes"], dtype=torch.uint8, device="cuda")
    q = torch.zeros(1, w.batch, w.num_q_heads, w.head_dim, dtype=torch.bfloat16, device="cuda")
    lens = torch.tensor(w.capacity, dtype=torch.int32, device="cuda")
    with pytest.raises(kvq.KvqError) as e:
        kvq.kvq_decode_attention_noalloc(cfg, cache, 0, 1, lens, q, torch.empty_like(q),
                                         w.sm_scale, 32)
    assert e.value.status == kvq.KVQ_ERR_WORKSPACE
