"""GPU parity of kvq_decode_attention_append: the decode-time append and the
decode in one launch.

Each case stores a history, then appends the token at position T (text, so
bf16 rows) and attends over [0, T + 1) of every sequence.  The fused call
must leave the cache byte-identical to the separate path (kvq_quantize, then
kvq_decode_attention), give the same output (bit-identical with fixed
chunks), and match the oracle, which stores the row and decodes.  Every case
prints its name before touching the GPU.
"""
import sys

import numpy as np
import pytest

import oracle
from quantized_decode_attention_quantize_amd import kvq, synth

from kvq_testlib import (Pair, as_f32, assert_close, bf16_device, bf16_to_f64, kernel_error,
                         to_device_src)

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


def _new_rows(w, pos, which):
    """Source rows of position pos[s] of every (layer, seq, KV head):
    [L, B, Hkv, D] in the source dtype."""
    return np.stack([np.stack([w.sources(l, [s], pos[s], pos[s] + 1, which)[0, :, 0]
                               for s in range(w.batch)]) for l in range(w.num_layers)])


def _run(w, pos, chunk, budget=8e-4):
    """History [0, pos[s]) stored on both sides; then the fused call and the
    separate path on copies of the GPU cache; the oracle stores pos[s] and
    decodes.  Returns (fused cache, separate cache, fused out, separate out,
    oracle out)."""
    import torch
    p = Pair(w)
    for s in range(w.batch):
        p.store(seqs=[s], t0=0, t1=pos[s])
    kn, vn = _new_rows(w, pos, "k"), _new_rows(w, pos, "v")
    kd, vd = to_device_src(kn), to_device_src(vn)
    lens = [x + 1 for x in pos]
    lens_d = torch.tensor(np.asarray(lens, dtype=np.int32), device="cuda")
    L = w.num_layers
    q_bits = np.stack([w.q_bits(l) for l in range(L)])
    q = bf16_device(q_bits)
    ws_bytes = kvq.workspace_bytes(p.cfg, L, chunk)

    fused = p.cache.clone()
    out_f = torch.empty_like(q)
    ws = torch.zeros(ws_bytes, dtype=torch.uint8, device="cuda")
    kvq.kvq_decode_attention_append(p.cfg, fused, 0, L, lens_d, kd, vd, q, out_f, w.sm_scale,
                                    chunk, ws)

    sep = p.cache.clone()
    out_s = torch.empty_like(q)
    ws2 = torch.zeros(ws_bytes, dtype=torch.uint8, device="cuda")
    kvq.kvq_quantize_ragged(p.cfg, sep, 0, L, list(range(w.batch)), list(pos), 1,
                            kd[:, :, :, None], vd[:, :, :, None])
    kvq.kvq_decode_attention(p.cfg, sep, 0, L, lens_d, q, out_s, w.sm_scale, chunk, ws2)
    torch.cuda.synchronize()

    for l in range(L):
        for s in range(w.batch):
            for h in range(w.num_kv_heads):
                oracle.store_rows(p.ocfg, p.ocache, l, s, h, 0, pos[s], pos[s] + 1,
                                  as_f32(kn[l, s, h][None]))
                oracle.store_rows(p.ocfg, p.ocache, l, s, h, 1, pos[s], pos[s] + 1,
                                  as_f32(vn[l, s, h][None]))
    jobs = [(l, s, i, lens[s], q_bits[l, s, i]) for l in range(L) for s in range(w.batch)
            for i in range(w.num_q_heads)]
    ref = np.array(p.oracle_decode_many(jobs)).reshape(L, w.batch, w.num_q_heads, w.head_dim)
    got_f, got_s = bf16_to_f64(out_f), bf16_to_f64(out_s)
    assert_close(got_f, ref, f"{w.name} fused append, chunk {chunk}")
    assert kernel_error(got_f, ref, f"{w.name} fused append, chunk {chunk}") <= budget
    # the appended rows on the GPU are the oracle's
    p.cache.copy_(fused)
    assert p.mismatches() == 0
    return fused.cpu().numpy(), sep.cpu().numpy(), got_f, got_s


def _wl(name, L, B, hq, hkv, D, g, vb, ve, cap, kb, vb_bits, **kw):
    w = synth.Workload(name, L, B, hq, hkv, D, g, list(cap), list(vb), list(ve), list(cap),
                       np.asarray(kb, np.uint8), np.asarray(vb_bits, np.uint8), **kw)
    return w


CASES = [
    # name, workload factory, appended positions
    ("tiny bf16", lambda: _wl("app_tiny", 1, 1, 4, 1, 64, 32, [16], [256], [260], [4], [4]),
     [256]),
    ("tiny fp32 source", lambda: _wl("app_tiny32", 1, 1, 4, 1, 64, 32, [16], [256], [260], [4],
                                     [4], src="f32"), [256]),
    ("four layers, protected heads", lambda: _wl(
        "app_prot", 4, 1, 28, 4, 128, 64, [14], [1500], [1600],
        [4, 16, 2, 4, 16, 4, 4, 2, 8, 4, 4, 16, 2, 2, 4, 4],
        [2, 16, 2, 4, 16, 2, 4, 2, 4, 2, 4, 16, 2, 4, 2, 8]), [1520]),
    ("ragged batch", lambda: _wl("app_rag", 2, 3, 8, 2, 128, 64, [14, 0, 30], [900, 333, 40],
                                 [1000, 400, 2100], [4, 2, 8, 4], [2, 4, 4, 8]),
     [930, 333, 2047]),
    ("text prefix position", lambda: _wl("app_pre", 1, 2, 8, 2, 64, 32, [200, 64], [700, 300],
                                         [800, 400], [4, 2], [4, 4]), [150, 350]),
    ("two query-head subgroups", lambda: _wl("app_sub", 2, 1, 28, 4, 128, 32, [14], [1100],
                                             [1200], [4] * 8, [2] * 8), [1150]),
    ("rotated K", lambda: _wl("app_rot", 2, 1, 8, 2, 128, 64, [14], [1000], [1100], [4] * 4,
                              [2] * 4, rotate_k=True), [1010]),
    ("per-channel K", lambda: _wl("app_pc", 1, 2, 8, 2, 128, 64, [14, 30], [1038, 700],
                                  [1100, 800], [4, 2], [4, 4], k_per_channel=True), [1038, 720]),
]


@pytest.mark.parametrize("name,make,pos", CASES, ids=[c[0] for c in CASES])
@pytest.mark.parametrize("chunk", [64, 0])
def test_fused_append_matches_separate_and_oracle(name, make, pos, chunk):
    w = make()
    if chunk and w.k_per_channel:
        chunk = 256  # per-channel K takes fixed chunks in multiples of 256 tokens
    _say("fused append:", name, "chunk", chunk)
    fused, sep, got_f, got_s = _run(w, pos, chunk)
    assert np.array_equal(fused, sep)  # the whole cache, padding included
    if chunk:
        assert np.array_equal(got_f, got_s)  # static steps: the same summation order
    else:
        np.testing.assert_allclose(got_f, got_s, rtol=2.0 ** -7, atol=1e-4 * np.abs(got_s).max())


def test_fused_append_position_in_bf16_range():
    """A position inside a bf16 range of the visual span is a text row: the
    fused call stores it like kvq_quantize does."""
    _say("fused append: position inside a bf16 range")
    w = _wl("app_rng", 1, 1, 8, 2, 128, 64, [14], [700], [800], [4, 4], [2, 2],
            bf16_ranges=[[(300, 320), (600, 650)]])
    fused, sep, got_f, got_s = _run(w, [640], 64)
    assert np.array_equal(fused, sep)
    assert np.array_equal(got_f, got_s)


def test_fused_append_coded_position_is_not_stored():
    """A position the cache stores coded is not written: the cache keeps its
    bytes, and the output is the plain decode's."""
    import torch
    _say("fused append: coded position left alone")
    w = _wl("app_coded", 1, 1, 8, 2, 128, 64, [14], [700], [800], [4, 4], [2, 2])
    p = Pair(w)
    p.store(oracle_too=False)
    before = p.cache.clone()
    pos = [500]
    kd, vd = to_device_src(_new_rows(w, pos, "k")), to_device_src(_new_rows(w, pos, "v"))
    lens_d = torch.tensor([501], dtype=torch.int32, device="cuda")
    q = bf16_device(np.stack([w.q_bits(0)]))
    out_f, out_p = torch.empty_like(q), torch.empty_like(q)
    ws = torch.zeros(kvq.workspace_bytes(p.cfg, 1, 64), dtype=torch.uint8, device="cuda")
    kvq.kvq_decode_attention_append(p.cfg, p.cache, 0, 1, lens_d, kd, vd, q, out_f, w.sm_scale,
                                    64, ws)
    kvq.kvq_decode_attention(p.cfg, p.cache, 0, 1, lens_d, q, out_p, w.sm_scale, 64, ws)
    torch.cuda.synchronize()
    assert torch.equal(p.cache, before)
    assert torch.equal(out_f, out_p)


def test_fused_append_headguard_step_sampled():
    """The 28-layer step with its appended token: fused and separate paths
    leave identical caches and, at fixed chunks, identical outputs; three
    layers against the oracle."""
    import torch
    _say("fused append: 28-layer step")
    w = synth.headguard_step(extra_capacity=1)
    T = w.seq_lens[0]
    p = Pair(w)
    p.store(t0=0, t1=T, oracle_too=False)
    pos = [T]
    kn, vn = _new_rows(w, pos, "k"), _new_rows(w, pos, "v")
    kd, vd = to_device_src(kn), to_device_src(vn)
    lens_d = torch.tensor([T + 1], dtype=torch.int32, device="cuda")
    L = w.num_layers
    q_bits = np.stack([w.q_bits(l) for l in range(L)])
    q = bf16_device(q_bits)
    outs, caches = [], []
    for fused in (True, False):
        c = p.cache.clone()
        out = torch.empty_like(q)
        ws = torch.zeros(kvq.workspace_bytes(p.cfg, L, 1024), dtype=torch.uint8, device="cuda")
        if fused:
            kvq.kvq_decode_attention_append(p.cfg, c, 0, L, lens_d, kd, vd, q, out, w.sm_scale,
                                            1024, ws)
        else:
            kvq.kvq_quantize(p.cfg, c, 0, L, [0], T, T + 1, kd[:, :, :, None],
                             vd[:, :, :, None])
            kvq.kvq_decode_attention(p.cfg, c, 0, L, lens_d, q, out, w.sm_scale, 1024, ws)
        torch.cuda.synchronize()
        outs.append(bf16_to_f64(out))
        caches.append(c)
    assert torch.equal(caches[0], caches[1])
    assert np.array_equal(outs[0], outs[1])
    layers = [0, 13, 27]
    p.cache.copy_(caches[0])
    p.store(layers=layers, t0=0, t1=T, oracle_too=True)  # oracle history (GPU bytes unchanged)
    for l in layers:
        for h in range(w.num_kv_heads):
            oracle.store_rows(p.ocfg, p.ocache, l, 0, h, 0, T, T + 1, as_f32(kn[l, 0, h][None]))
            oracle.store_rows(p.ocfg, p.ocache, l, 0, h, 1, T, T + 1, as_f32(vn[l, 0, h][None]))
    jobs = [(l, 0, i, T + 1, q_bits[l, 0, i]) for l in layers for i in range(w.num_q_heads)]
    ref = np.array(p.oracle_decode_many(jobs))
    got = np.array([outs[0][l, 0, i] for l in layers for i in range(w.num_q_heads)])
    assert_close(got, ref, "28-layer step, fused append")
    assert kernel_error(got, ref, "28-layer step, fused append") <= 8e-4


def test_fused_append_layer_range_and_70_sequences():
    """A call over layers [1, 3) of a 3-layer cache with 70 sequences (two
    launches of the sequence table): every appended row lands where
    kvq_quantize_ragged puts it, and the outputs agree at fixed chunks."""
    import torch
    _say("fused append: layers 1..2 of 3, 70 sequences")
    B = 70
    rng = np.random.default_rng(11)
    caps = [int(c) for c in rng.integers(96, 400, B)]
    vbs = [int(rng.integers(0, 20)) for _ in range(B)]
    ves = [vb + int(rng.integers(0, c // 2)) for vb, c in zip(vbs, caps)]
    w = _wl("app_many", 3, B, 8, 2, 64, 32, vbs, ves, caps, [4, 2, 8, 4, 2, 2], [2, 4, 4, 8, 4, 2])
    pos = [int(rng.integers(ve, c)) for ve, c in zip(ves, caps)]
    p = Pair(w)
    for s in range(B):
        p.store(seqs=[s], t0=0, t1=pos[s], oracle_too=False)
    lb, nl = 1, 2
    kn = np.stack([np.stack([w.sources(l, [s], pos[s], pos[s] + 1, "k")[0, :, 0]
                             for s in range(B)]) for l in range(lb, lb + nl)])
    vn = np.stack([np.stack([w.sources(l, [s], pos[s], pos[s] + 1, "v")[0, :, 0]
                             for s in range(B)]) for l in range(lb, lb + nl)])
    kd, vd = to_device_src(kn), to_device_src(vn)
    lens_d = torch.tensor([x + 1 for x in pos], dtype=torch.int32, device="cuda")
    q = bf16_device(np.stack([w.q_bits(l) for l in range(lb, lb + nl)]))
    outs, caches = [], []
    for fused in (True, False):
        c = p.cache.clone()
        out = torch.empty_like(q)
        ws = torch.zeros(kvq.workspace_bytes(p.cfg, nl, 64), dtype=torch.uint8, device="cuda")
        if fused:
            kvq.kvq_decode_attention_append(p.cfg, c, lb, nl, lens_d, kd, vd, q, out, w.sm_scale,
                                            64, ws)
        else:
            kvq.kvq_quantize_ragged(p.cfg, c, lb, nl, list(range(B)), pos, 1, kd[:, :, :, None],
                                    vd[:, :, :, None])
            kvq.kvq_decode_attention(p.cfg, c, lb, nl, lens_d, q, out, w.sm_scale, 64, ws)
        torch.cuda.synchronize()
        outs.append(out)
        caches.append(c)
    assert torch.equal(caches[0], caches[1])
    assert torch.equal(outs[0], outs[1])
    assert not torch.equal(caches[0], p.cache)  # rows were appended
