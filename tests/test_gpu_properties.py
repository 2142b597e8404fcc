"""Properties of the GPU path that hold whatever the data (MI355X).

- GQA: query head i reads KV head floor(i * Hkv / Hq).  Permuting the KV
  heads of a cache (their rows and widths) together with the query-head
  groups that read them permutes the groups of the output and changes
  nothing else.
- Checkpoint: the compressed cache is a position-independent byte string
  fully described by its kvq_config.  Saving its bytes to a file and loading
  them into a fresh device buffer gives bit-identical decode output.
Every case prints its name before touching the GPU.
"""
import sys

import numpy as np
import pytest

from quantized_decode_attention_quantize_amd import kvq, synth

from kvq_testlib import assert_close, bf16_device, bf16_to_f64, to_device_src

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


def _store_and_decode(w, k_src, v_src, q_bits, chunk):
    """Store [0, capacity) of every sequence from explicit sources
    [L][B] -> [Hkv, T, D] and decode all layers; returns (out f64, cache)."""
    import torch
    cfg = kvq.Config.from_workload(w)
    cache = torch.zeros(kvq.kvq_cache_bytes(cfg)["total_bytes"], dtype=torch.uint8, device="cuda")
    for l in range(w.num_layers):
        for s in range(w.batch):
            T = w.capacity[s]
            kvq.kvq_quantize(cfg, cache, l, 1, [s], 0, T, to_device_src(k_src[l][s][None, None]),
                             to_device_src(v_src[l][s][None, None]))
    return _decode(w, cfg, cache, q_bits, chunk), cache


def _decode(w, cfg, cache, q_bits, chunk):
    import torch
    q = bf16_device(q_bits)
    out = torch.empty_like(q)
    lens = torch.tensor(w.capacity, dtype=torch.int32, device="cuda")
    ws = torch.zeros(kvq.workspace_bytes(cfg, w.num_layers, chunk), dtype=torch.uint8,
                     device="cuda")
    kvq.kvq_decode_attention(cfg, cache, 0, w.num_layers, lens, q, out, w.sm_scale, chunk, ws)
    torch.cuda.synchronize()
    return bf16_to_f64(out)


@pytest.mark.parametrize("widths", ["uniform", "mixed"])
def test_decode_gqa_head_permutation(widths):
    _say("gqa permutation", widths)
    w = synth.llava_layer(seed=13, kbits=4, vbits=2)  # 28 query heads, 4 KV heads
    w.capacity, w.vis_end, w.seq_lens = [1500], [1500], [1500]
    if widths == "mixed":
        w.k_bits[:] = [4, 2, 16, 8]
        w.v_bits[:] = [2, 4, 16, 4]
    perm = [2, 0, 3, 1]  # new KV head h holds old KV head perm[h]
    G = w.num_q_heads // w.num_kv_heads
    k = [[w.sources(l, [s], 0, w.capacity[s], "k")[0] for s in range(w.batch)]
         for l in range(w.num_layers)]
    v = [[w.sources(l, [s], 0, w.capacity[s], "v")[0] for s in range(w.batch)]
         for l in range(w.num_layers)]
    q = np.stack([w.q_bits(l) for l in range(w.num_layers)])
    out, _ = _store_and_decode(w, k, v, q, 512)

    wp = synth.llava_layer(seed=13, kbits=4, vbits=2)
    wp.capacity, wp.vis_end, wp.seq_lens = w.capacity, w.vis_end, w.seq_lens
    wp.k_bits[:] = w.k_bits[perm]
    wp.v_bits[:] = w.v_bits[perm]
    kp = [[x[perm] for x in row] for row in k]
    vp = [[x[perm] for x in row] for row in v]
    qidx = np.concatenate([np.arange(p * G, (p + 1) * G) for p in perm])
    qp = q[:, :, qidx]
    outp, _ = _store_and_decode(wp, kp, vp, qp, 512)
    got = outp
    ref = out[:, :, qidx]
    diff = float(np.max(np.abs(got - ref)))
    print(f"[perm] {widths}: max |diff| = {diff:.3e}", flush=True)
    if widths == "uniform":
        assert np.array_equal(got, ref)  # one kernel instance, one static split
    else:
        assert_close(got, ref, "gqa permutation, mixed widths")


def test_cache_checkpoint_round_trip(tmp_path):
    """Cache bytes -> file -> fresh device buffer: identical decode bytes at
    fixed chunks (and the reloaded bytes equal the saved ones)."""
    import torch
    _say("checkpoint round trip")
    w = synth.llava_layer(seed=21, kbits=4, vbits=2)
    w.capacity, w.vis_end, w.seq_lens = [2000], [1990], [2000]
    w.k_bits[:] = [4, 16, 2, 8]
    k = [[w.sources(0, [0], 0, 2000, "k")[0]]]
    v = [[w.sources(0, [0], 0, 2000, "v")[0]]]
    q = np.stack([w.q_bits(0)])
    out1, cache = _store_and_decode(w, k, v, q, 256)
    path = tmp_path / "cache.npy"
    np.save(path, cache.cpu().numpy())
    del cache
    torch.cuda.synchronize()
    host = np.load(path)  # plain uint8 array, no pickled objects
    pad = torch.zeros(4096, dtype=torch.uint8, device="cuda")  # the reload lands elsewhere
    cache2 = torch.from_numpy(host).to("cuda")
    cfg = kvq.Config.from_workload(w)
    out2 = _decode(w, cfg, cache2, q, 256)
    assert np.array_equal(cache2.cpu().numpy(), host)
    assert np.array_equal(out1, out2)
    del pad
