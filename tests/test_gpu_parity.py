"""GPU parity of libkvq against the CPU oracle (MI355X).

Stored bytes must be identical to the oracle's (codes, fp16 scale/min, bf16
rows; padding between planes excluded).  Attention outputs (bf16) must be
within max-abs 5e-3 and relative L2 2e-3 of the oracle's fp64 result on the
same stored cache.  Every case prints its name before touching the GPU.
"""
import sys

import numpy as np
import pytest

from quantized_decode_attention_quantize_amd import kvq, synth

from kvq_testlib import Pair, assert_close, errors, kernel_error

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


# --------------------------------------------------------------------------
# quantize: bit-exact


def test_quantize_tiny_bitexact():
    _say("quantize tiny fp32 source")
    p = Pair(synth.tiny())
    p.store()
    assert p.mismatches() == 0


def test_quantize_llava_layer_bitexact():
    _say("quantize llava layer bf16 source")
    p = Pair(synth.llava_layer())
    p.store()
    assert p.mismatches() == 0


@pytest.mark.parametrize("kb,vb", [(8, 2), (2, 8), (16, 4), (4, 16), (8, 8)])
def test_quantize_widths_bitexact(kb, vb):
    _say("quantize widths", kb, vb)
    w = synth.llava_layer(seed=11, kbits=kb, vbits=vb)
    w.capacity = [700]
    w.vis_end = [650]
    w.seq_lens = [700]
    p = Pair(w)
    p.store()
    assert p.mismatches() == 0


def test_quantize_headguard_sampled_layers_bitexact():
    _say("quantize headguard 28 layers, compare sampled layers")
    w = synth.headguard_step()
    prot_layers = sorted({int(i) // 4 for i in w.protected})
    layers = sorted({0, 27, prot_layers[0], prot_layers[-1]})
    p = Pair(w)
    p.store(oracle_too=False)
    p.store(layers=layers)  # overwrite sampled layers on both sides (same bytes on GPU)
    assert p.mismatches(layers=layers) == 0


def test_quantize_appending_matches_full_store():
    """Storing one position at a time (decode-time appends) writes the same
    bytes as storing the whole range at once."""
    _say("quantize append vs full")
    w = synth.tiny(seed=5)
    w.capacity = [300]
    w.vis_begin = [20]
    w.vis_end = [260]
    p = Pair(w)
    p.store(t0=0, t1=250)
    for t in range(250, 300):
        p.store(t0=t, t1=t + 1)
    assert p.mismatches() == 0


def test_quantize_d64_d128_groups():
    for D, g in [(64, 32), (64, 64), (128, 32), (128, 128)]:
        _say("quantize D/g", D, g)
        kb = np.array([4, 2], dtype=np.uint8)
        vb = np.array([8, 16], dtype=np.uint8)
        w = synth.Workload(f"dg{D}_{g}", 1, 2, 4, 2, D, g, [90, 130], [5, 0], [85, 100],
                           [90, 130], kb, vb, seed=D + g)
        p = Pair(w)
        p.store()
        assert p.mismatches() == 0


# --------------------------------------------------------------------------
# decode: within tolerance of the oracle


def _check_decode(p: Pair, lens, layers=None, chunk=0, what=""):
    w = p.w
    out, q = p.decode(lens, chunk=chunk)
    layers = range(w.num_layers) if layers is None else layers
    jobs = [(l, s, i, lens[s], q[l, s, i]) for l in layers for s in range(w.batch)
            for i in range(w.num_q_heads)]
    ref = p.oracle_decode_many(jobs)
    got = [out[l, s, i] for (l, s, i, _, _) in jobs]
    return assert_close(np.array(got), np.array(ref), what)


def _decode_vs_oracle(p: Pair, lens, chunk=0):
    w = p.w
    out, q = p.decode(lens, chunk=chunk)
    got = np.array([out[0, s, i] for s in range(w.batch) for i in range(w.num_q_heads)])
    ref = np.array([p.oracle_decode(0, s, i, lens[s], q[0, s, i])
                    for s in range(w.batch) for i in range(w.num_q_heads)])
    return got, ref


def test_decode_tiny():
    _say("decode tiny")
    p = Pair(synth.tiny())
    p.store()
    got, ref = _decode_vs_oracle(p, [256])
    assert_close(got, ref, "tiny")
    # the kernel's own error, apart from the bf16 rounding of the output
    # (2.5e-4 when measured, against 1.86e-3 for the rounding itself)
    assert kernel_error(got, ref, "tiny") <= 8e-4


def test_decode_llava_layer():
    _say("decode llava layer")
    p = Pair(synth.llava_layer())
    p.store()
    got, ref = _decode_vs_oracle(p, [6287])
    assert_close(got, ref, "llava")
    assert kernel_error(got, ref, "llava") <= 8e-4


@pytest.mark.parametrize("chunk", [32, 64, 224, 1024, 8192])
def test_decode_split_invariance(chunk):
    _say("decode split chunk", chunk)
    w = synth.llava_layer(seed=7, kbits=4, vbits=2)
    p = Pair(w)
    p.store()
    _check_decode(p, [6287], chunk=chunk, what=f"chunk {chunk}")


@pytest.mark.parametrize("length", [1, 2, 13, 14, 15, 47, 3000, 6286, 6287])
def test_decode_lengths(length):
    """len < vis_begin (text only), inside the visual span, full."""
    _say("decode length", length)
    w = synth.llava_layer(seed=3, kbits=8, vbits=4)
    p = Pair(w)
    p.store()
    _check_decode(p, [length], what=f"len {length}")


def test_decode_headguard_step():
    """The whole 28-layer HeadGuard step: every layer, KV head and query head
    against the oracle (the oracle runs on a pool of host threads)."""
    _say("decode headguard 28 layers, every output vs oracle")
    w = synth.headguard_step()
    p = Pair(w)
    p.store()
    _check_decode(p, [6287], what="headguard")


def test_decode_bf16_reference_config():
    _say("decode all-bf16 cache")
    w = synth.llava_layer(seed=9, kbits=16, vbits=16)
    p = Pair(w)
    p.store()
    _check_decode(p, [6287], what="bf16")


def test_decode_mixed_formats_and_d64():
    for D, g, kb, vb in [(64, 32, 4, 2), (64, 64, 16, 2), (128, 32, 2, 16), (128, 128, 8, 8)]:
        _say("decode D/g/kb/vb", D, g, kb, vb)
        w = synth.Workload(f"m{D}", 2, 2, 8, 2, D, g, [300, 170], [10, 0], [290, 170],
                           [300, 170], np.full(4, kb, np.uint8), np.full(4, vb, np.uint8),
                           seed=D + kb)
        p = Pair(w)
        p.store()
        _check_decode(p, [300, 101], what=f"D{D} g{g} k{kb} v{vb}")


@pytest.mark.parametrize("hq,hkv,g", [(28, 4, 32), (16, 1, 64), (16, 1, 32), (8, 8, 128)])
def test_decode_general_kernel_shapes(hq, hkv, g):
    """(head, group) columns beyond one 16-wide tile (28, 32 and 64 here)
    decode in two or four query-head subgroups; G = 1 (no GQA) in one launch."""
    _say("decode heads/group", hq, hkv, g)
    kb = np.full(hkv, 4, np.uint8)
    vb = np.full(hkv, 2, np.uint8)
    w = synth.Workload(f"gen{hq}", 1, 1, hq, hkv, 128, g, [700], [14], [700], [700], kb, vb,
                       seed=hq + g)
    p = Pair(w)
    p.store()
    _check_decode(p, [700], what=f"Hq{hq} Hkv{hkv} g{g}")


@pytest.mark.parametrize("chunk", [64, 128, 256])
def test_decode_wide_group_wave_merge(chunk):
    """G = 16 query heads on one KV head with g = D (16 columns, one launch),
    split into 11, 6 or 3 fixed chunks: both instances of the wave-parallel
    merge (up to 8 and up to 16 partials) on an entry with more than 64
    (partial, head) pairs, each lane reading its own head's (m, l) pairs."""
    _say("decode G 16 wave merge, chunk", chunk)
    w = synth.Workload("wide16", 1, 1, 16, 1, 128, 128, [700], [14], [700], [700],
                       np.full(1, 4, np.uint8), np.full(1, 2, np.uint8), seed=41)
    p = Pair(w)
    p.store()
    _check_decode(p, [700], chunk=chunk, what=f"G16 chunk {chunk}")


def test_decode_empty_visual_span_and_all_visual():
    _say("decode no visual rows / all visual rows")
    kb = np.array([2], np.uint8)
    w = synth.Workload("edge", 1, 3, 4, 1, 128, 64, [100, 90, 64], [40, 0, 0], [40, 90, 64],
                       [100, 90, 64], kb, kb, seed=77)
    p = Pair(w)
    p.store()
    _check_decode(p, [100, 90, 64], what="edge spans")


def test_decode_deterministic():
    """Fixed token chunks (chunk_tokens > 0) assign every token statically, so
    repeated calls give identical bytes.  (The default split hands steps out
    dynamically: the summation order, and so the last bits of the output, may
    differ between calls.)"""
    _say("decode determinism")
    p = Pair(synth.tiny(seed=8))
    p.store(oracle_too=False)
    a, _ = p.decode([256], chunk=64)
    b, _ = p.decode([256], chunk=64)
    assert np.array_equal(a, b)
    p = Pair(synth.llava_layer(seed=8, kbits=4, vbits=2))
    p.store(oracle_too=False)
    a, _ = p.decode([6287], chunk=512)
    b, _ = p.decode([6287], chunk=512)
    assert np.array_equal(a, b)


def test_decode_per_head_formats_in_one_call():
    """(layer, head) pairs of one call with different visual widths: the call is
    split into one launch per width combination, bf16 heads join the first."""
    _say("decode per-head formats")
    kb = np.array([4, 16, 16, 8, 2, 4, 16, 8], np.uint8)
    vb = np.array([2, 16, 2, 4, 2, 2, 16, 8], np.uint8)
    w = synth.Workload("perhead", 2, 2, 16, 4, 128, 64, [400, 333], [14, 5], [390, 333],
                       [400, 333], kb, vb, seed=21)
    p = Pair(w)
    p.store()
    _check_decode(p, [400, 300], what="per-head formats")
    _check_decode(p, [397, 333], chunk=64, what="per-head formats chunk 64")


def test_decode_wave_granular_pieces():
    """6 layers x 4 KV heads, four of them bf16 among INT4/INT2 ones, over five
    ragged sequences (77 to 2,000 rows).  The balanced split gives entries
    wave counts that are not multiples of 8 (1,548 waves in all), so
    workgroups hold up to three entries' pieces, an entry has up to 11
    partials, and the last workgroup is partly idle.  Every output is compared
    with the oracle, at full and at shortened lengths."""
    _say("decode wave-granular pieces (mixed bf16 / INT4-INT2, ragged)")
    kb = np.full(24, 4, np.uint8)
    vb = np.full(24, 2, np.uint8)
    kb[[1, 6, 11, 19]] = 16
    vb[[1, 6, 11, 19]] = 16
    caps = [300, 1200, 77, 2000, 640]
    w = synth.Workload("pieces", 6, 5, 16, 4, 128, 64, caps, [14, 5, 0, 30, 0],
                       [290, 1200, 77, 1990, 600], caps, kb, vb, seed=33)
    p = Pair(w)
    p.store()
    _check_decode(p, caps, what="pieces full length")
    _check_decode(p, [1, 1199, 40, 1500, 33], what="pieces shortened")


def test_decode_workspace_reuse_across_shapes():
    """The merge's arrival counters return to zero after every call and sit
    where no call's partials go, so one workspace serves consecutive calls
    with other lengths, layer ranges and split sizes."""
    _say("decode workspace reuse")
    import torch
    from kvq_testlib import bf16_device, bf16_to_f64
    w = synth.llava_layer(seed=13, kbits=4, vbits=2)
    p = Pair(w)
    p.store()
    ws = torch.zeros(max(kvq.workspace_bytes(p.cfg, 1, c) for c in (0, 32, 64, 1024)),
                     dtype=torch.uint8, device="cuda")
    q_bits = w.q_bits(0)[None]
    q = bf16_device(q_bits)
    # 32-token chunks fill ~2.8 MB with partials; the balanced call after them
    # must still find its arrival counters at zero
    for n, chunk in [(6287, 0), (6287, 32), (6287, 0), (1000, 64), (6287, 1024), (37, 0),
                     (6287, 0)]:
        out = torch.empty_like(q)
        lens = torch.tensor([n], dtype=torch.int32, device="cuda")
        kvq.kvq_decode_attention(p.cfg, p.cache, 0, 1, lens, q, out, w.sm_scale, chunk, ws)
        torch.cuda.synchronize()
        got = bf16_to_f64(out)[0, 0]
        ref = np.stack([p.oracle_decode(0, 0, i, n, q_bits[0, 0, i]) for i in range(w.num_q_heads)])
        assert_close(got, ref, f"reuse len {n} chunk {chunk}")


def test_decode_long_context_full_size_sampled():
    """B=4 x 32,768-token GQA cache (32 query / 8 KV heads, K INT4 / V INT2) at
    full size, decoded in the default (balanced) split as the benchmark runs it;
    every sequence and query head against the oracle (run on a pool of host
    threads)."""
    _say("decode long context 4 x 32768 vs oracle")
    w = synth.long_gqa()
    p = Pair(w)
    p.store()
    assert p.mismatches(seqs=[0, 3]) == 0
    lens = [32768, 20000, 32768, 31999]
    out, q = p.decode(lens)
    jobs = [(0, s, i, lens[s], q[0, s, i]) for s in range(w.batch) for i in range(w.num_q_heads)]
    ref = np.array(p.oracle_decode_many(jobs))
    got = np.array([out[0, s, i] for (_, s, i, _, _) in jobs])
    assert_close(got, ref, "long context")
    assert kernel_error(got, ref, "long context") <= 1.2e-3


def test_decode_ragged_batch_full_size_sampled():
    """B=64 ragged lengths in [1024, 16384], K INT8 / V INT4, at full size.
    Every sequence holds real rows: sampled sequences (shortest, longest and
    six others) come from the seeded generator on both sides and are compared
    with the oracle on every query head; the others are filled with device
    random rows through the same store (generating all 64 on the host would
    take about a minute) and are checked for finite outputs inside the range
    their V rows allow."""
    _say("decode ragged batch of 64, sampled sequences vs oracle")
    import torch
    w = synth.ragged_serving()
    p = Pair(w)
    caps = np.array(w.capacity)
    sampled = sorted({int(np.argmin(caps)), int(np.argmax(caps)), 5, 17, 29, 40, 51, 63})
    p.store(seqs=sampled)
    assert p.mismatches(seqs=sampled) == 0
    gen = torch.Generator(device="cuda").manual_seed(1234)
    others = [s for s in range(w.batch) if s not in sampled]
    for s in others:
        k = torch.randn((1, 1, w.num_kv_heads, w.capacity[s], w.head_dim), generator=gen,
                        device="cuda").to(torch.bfloat16)
        v = torch.randn(k.shape, generator=gen, device="cuda").to(torch.bfloat16)
        kvq.kvq_quantize(p.cfg, p.cache, 0, 1, [s], 0, w.capacity[s], k, v)
    lens = [c if s % 3 else max(1, c - 777) for s, c in enumerate(w.capacity)]
    out, q = p.decode(lens)
    jobs = [(0, s, i, lens[s], q[0, s, i]) for s in sampled for i in range(w.num_q_heads)]
    ref = p.oracle_decode_many(jobs)
    got = [out[0, s, i] for (_, s, i, _, _) in jobs]
    assert_close(np.array(got), np.array(ref), "ragged batch")
    rest = out[0, others]
    assert np.all(np.isfinite(rest))
    # a convex combination of V rows: |out| stays below the largest stored
    # |v| (bf16 normals here stay below 6.5; codes add at most half a step)
    assert float(np.max(np.abs(rest))) < 8.0
    assert float(np.std(rest)) > 0.0


def test_decode_merge_of_many_partials():
    """32-token chunks over 32,768 tokens: 1,024 partials per (layer, seq, head),
    more than the merging workgroup can stage in LDS, so the merge reads them
    from memory directly."""
    _say("decode 1024 partials per head (merge from memory)")
    w = synth.llava_layer(seed=17, kbits=4, vbits=2)
    w.capacity = [32768]
    w.vis_end = [32768]
    w.seq_lens = [32768]
    p = Pair(w)
    p.store()
    _check_decode(p, [32768], chunk=32, what="1024 partials")
    _check_decode(p, [32000], chunk=0, what="balanced, same cache")


# --------------------------------------------------------------------------
# Walsh-Hadamard rotated K rows (include/kvq.h; gist.science 2604.02570,
# section 2-C)


def test_quantize_rotated_bitexact():
    """Coded K rows rotated before quantisation: every stored byte equals the
    oracle's (fp32 D=64 g32 INT4, bf16 D=128 g64 INT2 and INT8)."""
    for w in (synth.tiny(), synth.llava_layer(kbits=2, vbits=4),
              synth.llava_layer(kbits=8, vbits=2)):
        _say("quantize rotated", w.name, int(w.k_bits[0]))
        w.rotate_k = True
        p = Pair(w)
        p.store()
        assert p.mismatches() == 0


def test_decode_rotated():
    """Decode over a rotated cache against the oracle (which undoes the
    rotation of the stored rows in binary64): tiny, the full LLaVA layer in
    the balanced split and in 1,024-token chunks (wave-parallel merge), and a
    call mixing coded and bf16 K heads (only the coded ones are rotated)."""
    _say("decode rotated tiny")
    w = synth.tiny()
    w.rotate_k = True
    p = Pair(w)
    p.store()
    _check_decode(p, [256], what="rotated tiny")
    _say("decode rotated llava layer")
    w = synth.llava_layer(seed=9, kbits=4, vbits=2)
    w.rotate_k = True
    p = Pair(w)
    p.store()
    _check_decode(p, [6287], what="rotated llava")
    _check_decode(p, [5000], chunk=1024, what="rotated llava chunk 1024")
    _say("decode rotated per-head formats")
    kb = np.array([4, 16, 16, 8, 2, 4, 16, 8], np.uint8)
    vb = np.array([2, 16, 2, 4, 2, 2, 16, 8], np.uint8)
    w = synth.Workload("perhead_rot", 2, 2, 16, 4, 128, 64, [400, 333], [14, 5], [390, 333],
                       [400, 333], kb, vb, seed=23, rotate_k=True)
    p = Pair(w)
    p.store()
    _check_decode(p, [400, 300], what="rotated per-head formats")


@pytest.mark.parametrize("bits", [2, 4, 8])
def test_quantize_grid_points_and_ties_bitexact(bits):
    """Values exactly on the code grid and exactly halfway between two codes
    (ties go to the even code): the cases where the kernel's reciprocal
    estimate of the quotient defers to the IEEE divide.  Every group holds its
    own fp16 min and scale (element 0 = min, element 1 = min + n * scale, so
    both are stored exactly); stored bytes equal the oracle's."""
    import torch
    import oracle
    from kvq_testlib import to_device_src
    _say("quantize grid points and ties", bits)
    D, g, T = 128, 64, 512
    n = (1 << bits) - 1
    rng = np.random.default_rng(bits)
    x = np.empty((T, D), np.float64)
    for t in range(T):
        for j in range(D // g):
            # multiples of 1/16 and of 2^-6: every value below is a multiple
            # of 2^-7 under 2^13, exact in fp32 and the min and scale in fp16
            mn = -float(rng.integers(0, 64)) / 16.0
            sc = float(2.0 ** rng.integers(-6, 0) * rng.integers(1, 64))
            k = rng.integers(0, n, g).astype(np.float64)
            half = rng.integers(0, 2, g) * 0.5  # ties on about half of the values
            grp = mn + (k + half) * sc
            grp[0], grp[1] = mn, mn + n * sc
            x[t, j * g:(j + 1) * g] = grp
    xs = x.astype(np.float32)
    assert np.array_equal(xs.astype(np.float64), x)  # every value exact in fp32
    w = synth.Workload("ties", 1, 1, 4, 1, D, g, [T], [0], [T], [T],
                       np.array([bits], np.uint8), np.array([bits], np.uint8), src="f32")
    cfg = kvq.Config.from_workload(w)
    ocfg = oracle.Config.from_workload(w)
    cache = torch.zeros(kvq.kvq_cache_bytes(cfg)["total_bytes"], dtype=torch.uint8,
                        device="cuda")
    src = to_device_src(xs[None, None, None])
    kvq.kvq_quantize(cfg, cache, 0, 1, [0], 0, T, src, src)
    ocache = oracle.new_cache(ocfg)
    for X in (0, 1):
        oracle.store_rows(ocfg, ocache, 0, 0, 0, X, 0, T, xs)
    torch.cuda.synchronize()
    got = cache.cpu().numpy()
    info = kvq.kvq_cache_bytes(cfg)
    for X in (0, 1):
        vis, meta, _ = oracle.plane_offsets(ocfg, 0, 0, X)
        for a, b in ((vis, vis + T * D * bits // 8), (meta, meta + T * (D // g) * 4)):
            assert np.array_equal(got[a:b], ocache[a:b]), (bits, X, a)
    assert info["quantized_values"] == 2 * T * D


def test_quantize_ragged_append_bitexact():
    """A ragged batch appends its next tokens in one call, each sequence at
    its own position (kvq_quantize_ragged): after a prefix store, one token
    per sequence and then three more, across a visual span end and into the
    text suffix; every stored byte equals the oracle's per-sequence stores,
    and the decode that follows matches the oracle."""
    import oracle
    from kvq_testlib import to_device_src, as_f32
    from quantized_decode_attention_quantize_amd.synth import TAG_APPEND_K, TAG_APPEND_V
    _say("quantize ragged append")
    caps = [300, 180, 257, 90, 400]
    vb = [14, 0, 5, 10, 14]
    ve = [290, 170, 250, 88, 390]  # sequence 3's appends cross its span end
    w = synth.Workload("ragged_app", 2, 5, 8, 2, 128, 64, caps, vb, ve, caps,
                       np.array([4, 16, 8, 2], np.uint8), np.array([2, 16, 4, 2], np.uint8),
                       seed=31)
    p = Pair(w)
    T = [c - 5 for c in caps]  # history before the appends
    for s in range(w.batch):
        p.store(seqs=[s], t0=0, t1=T[s])
    seqs = list(range(w.batch))
    for t_off, n in ((0, 1), (1, 3)):
        t0 = [T[s] + t_off for s in seqs]
        k = np.stack([np.stack([np.stack([w.k_rows(l, s, h, t0[s], t0[s] + n, TAG_APPEND_K)
                                          for h in range(w.num_kv_heads)]) for s in seqs])
                      for l in range(w.num_layers)])
        v = np.stack([np.stack([np.stack([w.v_rows(l, s, h, t0[s], t0[s] + n, TAG_APPEND_V)
                                          for h in range(w.num_kv_heads)]) for s in seqs])
                      for l in range(w.num_layers)])
        kvq.kvq_quantize_ragged(p.cfg, p.cache, 0, w.num_layers, seqs, t0, n,
                                to_device_src(k), to_device_src(v))
        for l in range(w.num_layers):
            for s in seqs:
                for h in range(w.num_kv_heads):
                    oracle.store_rows(p.ocfg, p.ocache, l, s, h, 0, t0[s], t0[s] + n,
                                      as_f32(k[l, s, h]))
                    oracle.store_rows(p.ocfg, p.ocache, l, s, h, 1, t0[s], t0[s] + n,
                                      as_f32(v[l, s, h]))
    assert p.mismatches() == 0
    _check_decode(p, [T[s] + 4 for s in seqs], what="after ragged append")


@pytest.mark.parametrize("bits", [2, 4, 8])
def test_quantize_degenerate_groups_bitexact(bits):
    """Groups that stress the fp16 directed roundings and the zero-scale path:
    all zeros, -0, one non-zero constant (its fp16 min may sit below it, so the
    scale rounds up to a tiny non-zero value), a tiny range on a large offset,
    values near the fp16 limit, and values far below the fp16 subnormal step.
    Stored bytes equal the oracle's."""
    import torch
    import oracle
    from kvq_testlib import to_device_src
    _say("quantize degenerate groups", bits)
    D, g = 128, 64
    rng = np.random.default_rng(100 + bits)
    rows = []
    for kind in range(7):
        for rep in range(16):
            r = np.empty(D, np.float64)
            for j in range(D // g):
                c = rng.standard_normal()
                grp = {0: np.zeros(g),
                       1: -np.zeros(g),
                       2: np.full(g, c * 10),
                       3: 100.0 + 1e-3 * rng.standard_normal(g),
                       4: rng.uniform(-65000, 65000, g),
                       5: 1e-9 * rng.standard_normal(g),
                       6: np.concatenate([[c], np.full(g - 1, c + 2.0 ** -20)])}[kind]
                r[j * g:(j + 1) * g] = grp
            rows.append(r)
    xs = np.array(rows, dtype=np.float32)
    T = len(rows)
    w = synth.Workload("degen", 1, 1, 4, 1, D, g, [T], [0], [T], [T],
                       np.array([bits], np.uint8), np.array([bits], np.uint8), src="f32")
    cfg = kvq.Config.from_workload(w)
    ocfg = oracle.Config.from_workload(w)
    cache = torch.zeros(kvq.kvq_cache_bytes(cfg)["total_bytes"], dtype=torch.uint8,
                        device="cuda")
    src = to_device_src(xs[None, None, None])
    kvq.kvq_quantize(cfg, cache, 0, 1, [0], 0, T, src, src)
    ocache = oracle.new_cache(ocfg)
    for X in (0, 1):
        oracle.store_rows(ocfg, ocache, 0, 0, 0, X, 0, T, xs)
    torch.cuda.synchronize()
    got = cache.cpu().numpy()
    for X in (0, 1):
        vis, meta, _ = oracle.plane_offsets(ocfg, 0, 0, X)
        for a, b in ((vis, vis + T * D * bits // 8), (meta, meta + T * (D // g) * 4)):
            bad = np.flatnonzero(got[a:b] != ocache[a:b])
            assert bad.size == 0, (bits, X, a, bad[:8])


def test_calls_split_over_several_launches():
    """Calls larger than one launch's tables: 70 sequences (over the 64 a
    launch holds) and 40 layers x 4 KV heads = 160 (layer, head) pairs (over
    the 128 a launch holds) are stored and decoded in several launches; every
    output and every stored byte matches the oracle."""
    _say("calls over several launches: 70 sequences")
    rng = np.random.default_rng(77)
    caps = [int(c) for c in rng.integers(40, 260, 70)]
    vb = [min(14, c) for c in caps]
    ve = [max(b, c - int(rng.integers(0, 3))) for b, c in zip(vb, caps)]
    w = synth.Workload("seqs70", 1, 70, 8, 2, 128, 64, caps, vb, ve, caps,
                       np.array([4, 16], np.uint8), np.array([2, 16], np.uint8), seed=41)
    p = Pair(w)
    p.store()
    assert p.mismatches() == 0
    _check_decode(p, caps, what="70 sequences")
    _check_decode(p, [max(1, c - 7) for c in caps], what="70 sequences shortened")
    _say("calls over several launches: 160 (layer, head) pairs")
    kb = np.where(np.arange(160) % 9 == 0, 16, 4).astype(np.uint8)
    vbits = np.where(np.arange(160) % 9 == 0, 16, 2).astype(np.uint8)
    w = synth.Workload("pairs160", 40, 1, 16, 4, 128, 64, [150], [5], [140], [150], kb, vbits,
                       seed=43)
    p = Pair(w)
    p.store()
    assert p.mismatches() == 0
    _check_decode(p, [150], what="160 pairs")
