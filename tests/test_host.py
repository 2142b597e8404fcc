"""Host-side checks of libkvq that need no GPU.

The library loads, exports every function include/kvq.h declares, reports
storage exactly as the oracle computes it, and rejects every malformed call
before launching anything (validation runs on the host before the first HIP
call, so these calls never reach a device).
"""
import ctypes as C
import os
import re
import subprocess

import numpy as np
import pytest

from quantized_decode_attention_quantize_amd import kvq, synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kvq.h")


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(kvq.LIB_PATH):
        from quantized_decode_attention_quantize_amd import build
        build.build()
    return kvq.lib()


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(kvq_[a-z_]+)\s*\(", text)))


def test_exports_every_declared_symbol(L):
    names = _declared_functions()
    assert set(names) == set(kvq.EXPORTS)
    for n in names:
        assert hasattr(L, n), n
    out = subprocess.run(["nm", "-D", "--defined-only", kvq.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\bT (kvq_\w+)", out))
    assert set(names) <= exported


def test_status_strings(L):
    for s in range(9):
        assert kvq.status_string(s)
    assert kvq.status_string(kvq.KVQ_ERR_WORKSPACE) == "workspace too small"


def _configs():
    yield synth.tiny()
    yield synth.llava_layer()
    yield synth.headguard_step()
    yield synth.long_gqa()
    yield synth.ragged_serving()
    yield synth.visual_block()
    rng = np.random.default_rng(0)
    for i in range(20):
        L_, B, Hkv = int(rng.integers(1, 4)), int(rng.integers(1, 6)), int(rng.integers(1, 5))
        D = int(rng.choice([64, 128]))
        g = int(rng.choice([g for g in (32, 64, 128) if g <= D]))
        cap = rng.integers(1, 300, B)
        vb = np.array([rng.integers(0, c + 1) for c in cap])
        ve = np.array([rng.integers(b, c + 1) for b, c in zip(vb, cap)])
        kb = rng.choice([2, 4, 8, 16], L_ * Hkv)
        vbits = rng.choice([2, 4, 8, 16], L_ * Hkv)
        w = synth.Workload(f"rand{i}", L_, B, Hkv * 2, Hkv, D, g, list(cap), list(vb),
                           list(ve), list(cap), kb.astype(np.uint8), vbits.astype(np.uint8))
        w.k_per_channel = bool(i % 2)  # per-channel K: coded spans in whole blocks
        if i % 4 == 2:  # bf16 ranges inside the visual spans
            w.bf16_ranges = [_random_ranges(rng, int(b), int(e)) for b, e in zip(vb, ve)]
        yield w


def _random_ranges(rng, vb, ve, most=5):
    """Sorted, disjoint, non-empty ranges inside [vb, ve)."""
    if ve - vb < 2:
        return []
    cuts = np.sort(rng.choice(np.arange(vb, ve + 1), size=min(2 * most, ve - vb + 1),
                              replace=False))
    out = [(int(cuts[j]), int(cuts[j + 1])) for j in range(0, len(cuts) - 1, 2)]
    return out[:int(rng.integers(0, most + 1))]


def test_cache_bytes_matches_oracle(L, orc):
    for w in _configs():
        got = kvq.kvq_cache_bytes(kvq.Config.from_workload(w))
        ref = orc.cache_info(orc.Config.from_workload(w))
        assert got == ref, w.name


def _cfg(**over):
    base = dict(num_layers=1, batch=1, num_q_heads=4, num_kv_heads=1, head_dim=64,
                group_size=32, capacity=[256], vis_begin=[16], vis_end=[256], k_bits=[4],
                v_bits=[4])
    base.update(over)
    return kvq.Config(**base)


@pytest.mark.parametrize("over,status", [
    (dict(head_dim=96), kvq.KVQ_ERR_UNSUPPORTED),
    (dict(group_size=16), kvq.KVQ_ERR_UNSUPPORTED),
    (dict(head_dim=64, group_size=128), kvq.KVQ_ERR_UNSUPPORTED),
    (dict(k_bits=[3]), kvq.KVQ_ERR_UNSUPPORTED),
    (dict(v_bits=[1]), kvq.KVQ_ERR_UNSUPPORTED),
    (dict(num_q_heads=6, num_kv_heads=4, k_bits=[4] * 4, v_bits=[4] * 4),
     kvq.KVQ_ERR_UNSUPPORTED),
    (dict(vis_begin=[20], vis_end=[10]), kvq.KVQ_ERR_SHAPE),
    (dict(vis_end=[300]), kvq.KVQ_ERR_SHAPE),
    (dict(vis_begin=[-1]), kvq.KVQ_ERR_SHAPE),
    (dict(capacity=[0], vis_begin=[0], vis_end=[0]), kvq.KVQ_ERR_SHAPE),
    (dict(num_layers=0), kvq.KVQ_ERR_SHAPE),
])
def test_cache_bytes_rejects(L, over, status):
    with pytest.raises(kvq.KvqError) as e:
        kvq.kvq_cache_bytes(_cfg(**over))
    assert e.value.status == status


def test_cache_bytes_null_pointers(L):
    info = kvq._Info()
    assert L.kvq_cache_bytes(None, C.byref(info)) == kvq.KVQ_ERR_NULL
    c = _cfg()
    assert L.kvq_cache_bytes(c.ref, None) == kvq.KVQ_ERR_NULL
    c.c.k_bits = C.POINTER(C.c_uint8)()
    assert L.kvq_cache_bytes(c.ref, C.byref(info)) == kvq.KVQ_ERR_NULL


# Fake, never-dereferenced "device" addresses: every call below fails host
# validation before any HIP call is made.
A256 = 0x7F0000000000
A16 = A256 + 16


def _quant(L, cfg, cache=A256, layer_begin=0, num_layers=1, seq_ids=(0,), t0=0, t1=8,
           k=A16, v=A16, dtype=kvq.KVQ_SRC_BF16):
    ids = np.ascontiguousarray(seq_ids, dtype=np.int32)
    return L.kvq_quantize(cfg.ref, C.c_void_p(cache) if cache else None, layer_begin,
                          num_layers, len(ids), ids.ctypes.data_as(C.POINTER(C.c_int32)),
                          t0, t1, C.c_void_p(k) if k else None, C.c_void_p(v) if v else None,
                          dtype, None)


def test_quantize_validation(L):
    cfg = _cfg(batch=2, capacity=[256, 100], vis_begin=[16, 0], vis_end=[256, 50])
    assert _quant(L, cfg, layer_begin=1) == kvq.KVQ_ERR_RANGE
    assert _quant(L, cfg, num_layers=2) == kvq.KVQ_ERR_RANGE
    assert _quant(L, cfg, layer_begin=-1) == kvq.KVQ_ERR_RANGE
    assert _quant(L, cfg, seq_ids=(2,)) == kvq.KVQ_ERR_RANGE
    assert _quant(L, cfg, seq_ids=(0, 0)) == kvq.KVQ_ERR_SHAPE
    assert _quant(L, cfg, seq_ids=(1,), t0=90, t1=101) == kvq.KVQ_ERR_RANGE
    assert _quant(L, cfg, t0=-1) == kvq.KVQ_ERR_SHAPE
    assert _quant(L, cfg, t0=9, t1=8) == kvq.KVQ_ERR_SHAPE
    assert _quant(L, cfg, cache=None) == kvq.KVQ_ERR_NULL
    assert _quant(L, cfg, k=None) == kvq.KVQ_ERR_NULL
    assert _quant(L, cfg, cache=A256 + 128) == kvq.KVQ_ERR_ALIGN
    assert _quant(L, cfg, v=A16 + 4) == kvq.KVQ_ERR_ALIGN
    assert _quant(L, cfg, dtype=7) == kvq.KVQ_ERR_UNSUPPORTED
    # empty work is a no-op that touches nothing
    assert _quant(L, cfg, t0=5, t1=5) == kvq.KVQ_OK
    assert _quant(L, cfg, seq_ids=()) == kvq.KVQ_OK
    assert _quant(L, _cfg(head_dim=80)) == kvq.KVQ_ERR_UNSUPPORTED


def _quant_ragged(L, cfg, seq_ids=(0, 1), t0=(3, 7), n=1, cache=A256, k=A16, v=A16):
    ids = np.ascontiguousarray(seq_ids, dtype=np.int32)
    tb = np.ascontiguousarray(t0, dtype=np.int32)
    return L.kvq_quantize_ragged(cfg.ref, C.c_void_p(cache) if cache else None, 0, 1, len(ids),
                                 ids.ctypes.data_as(C.POINTER(C.c_int32)),
                                 tb.ctypes.data_as(C.POINTER(C.c_int32)), n,
                                 C.c_void_p(k) if k else None, C.c_void_p(v) if v else None,
                                 kvq.KVQ_SRC_BF16, None)


def test_quantize_ragged_validation(L):
    """Per-sequence start positions are checked against each sequence's own
    capacity before any launch."""
    cfg = _cfg(batch=2, capacity=[256, 100], vis_begin=[16, 0], vis_end=[256, 50])
    assert _quant_ragged(L, cfg, t0=(255, 100)) == kvq.KVQ_ERR_RANGE   # seq 1 ends at 100
    assert _quant_ragged(L, cfg, t0=(250, 90), n=11) == kvq.KVQ_ERR_RANGE
    assert _quant_ragged(L, cfg, t0=(-1, 3)) == kvq.KVQ_ERR_SHAPE
    assert _quant_ragged(L, cfg, seq_ids=(1, 1)) == kvq.KVQ_ERR_SHAPE
    assert _quant_ragged(L, cfg, seq_ids=(0, 2)) == kvq.KVQ_ERR_RANGE
    assert _quant_ragged(L, cfg, n=-1) == kvq.KVQ_ERR_SHAPE
    assert _quant_ragged(L, cfg, cache=None) == kvq.KVQ_ERR_NULL
    assert _quant_ragged(L, cfg, cache=A256 + 64) == kvq.KVQ_ERR_ALIGN
    assert _quant_ragged(L, cfg, n=0) == kvq.KVQ_OK        # nothing to store
    assert _quant_ragged(L, cfg, seq_ids=(), t0=()) == kvq.KVQ_OK


def _dec(L, cfg, cache=A256, layer_begin=0, num_layers=1, lens=A16, q=A16, out=A16 + 4096,
         chunk=0, ws=A256 + 4096, ws_bytes=1 << 30):
    n = C.c_size_t(ws_bytes)
    st = L.kvq_decode_attention(cfg.ref, C.c_void_p(cache) if cache else None, layer_begin,
                                num_layers, C.c_void_p(lens) if lens else None,
                                C.c_void_p(q) if q else None, C.c_void_p(out) if out else None,
                                0.125, chunk, C.c_void_p(ws) if ws else None, C.byref(n), None)
    return st, n.value


def test_decode_workspace_query(L):
    w = synth.long_gqa()
    cfg = kvq.Config.from_workload(w)
    for chunk in (32, 1024, 4096, 32768):
        st, n = _dec(L, cfg, ws=None, chunk=chunk)
        assert st == kvq.KVQ_OK
        entries = 1 * 4 * 8 * (-(-32768 // chunk))
        G = 4
        expect = (256 + (-(-(entries * G * 128 * 4) // 256) * 256)
                  + (-(-(entries * G * 2 * 4) // 256) * 256)
                  + 256)  # arrivals, partials, (m, l) pairs, partial counts
        assert n == expect == kvq.workspace_bytes(cfg, 1, chunk)
    st, n = _dec(L, cfg, ws=None, chunk=0)
    assert st == kvq.KVQ_OK and n > 0


def test_decode_query_head_subgroups(L):
    """More than 16 (head, group) columns per KV head: the decode runs in
    query-head subgroups (launches of at most 16 columns), so every feature
    is available and the workspace holds one subgroup's partials."""
    # G = 7 query heads per KV head, 4 groups per row: 28 columns, two subgroups
    # of 4 and 3 heads
    wide = kvq.Config(1, 1, 28, 4, 128, 32, [256], [16], [256], [4] * 4, [2] * 4)
    narrow = kvq.Config(1, 1, 16, 4, 128, 32, [256], [16], [256], [4] * 4, [2] * 4)  # 16
    st, n_wide = _dec(L, wide, ws=None, chunk=64)
    st2, n_narrow = _dec(L, narrow, ws=None, chunk=64)
    assert st == st2 == kvq.KVQ_OK and n_wide == n_narrow
    for extra in (dict(rotate_k=True), dict(k_per_channel=True),
                  dict(bf16_ranges=[[(20, 30)]])):
        c = kvq.Config(1, 1, 28, 4, 128, 32, [256], [16], [256], [4] * 4, [2] * 4, **extra)
        assert _dec(L, c, ws=None)[0] == kvq.KVQ_OK, extra
    # 16 query heads per KV head at g = 32: 64 columns, four subgroups
    g16 = kvq.Config(1, 1, 16, 1, 128, 32, [256], [16], [256], [4], [2])
    assert _dec(L, g16, ws=None)[0] == kvq.KVQ_OK


def test_decode_validation(L):
    cfg = _cfg()
    need = kvq.workspace_bytes(cfg, 1, 64)
    assert _dec(L, cfg, chunk=48)[0] == kvq.KVQ_ERR_SHAPE
    assert _dec(L, cfg, chunk=-32)[0] == kvq.KVQ_ERR_SHAPE
    assert _dec(L, cfg, layer_begin=1)[0] == kvq.KVQ_ERR_RANGE
    assert _dec(L, cfg, num_layers=0)[0] == kvq.KVQ_ERR_SHAPE
    assert _dec(L, cfg, chunk=64, ws_bytes=need - 1)[0] == kvq.KVQ_ERR_WORKSPACE
    assert _dec(L, cfg, cache=None)[0] == kvq.KVQ_ERR_NULL
    assert _dec(L, cfg, lens=None)[0] == kvq.KVQ_ERR_NULL
    assert _dec(L, cfg, q=None)[0] == kvq.KVQ_ERR_NULL
    assert _dec(L, cfg, out=None)[0] == kvq.KVQ_ERR_NULL
    assert _dec(L, cfg, q=A16 + 2)[0] == kvq.KVQ_ERR_ALIGN
    assert _dec(L, cfg, ws=A256 + 64)[0] == kvq.KVQ_ERR_ALIGN
    assert _dec(L, cfg, cache=A256 + 16)[0] == kvq.KVQ_ERR_ALIGN
    big_g = _cfg(num_q_heads=32, num_kv_heads=1)
    assert _dec(L, big_g)[0] == kvq.KVQ_ERR_UNSUPPORTED
    n = C.c_size_t(0)
    assert L.kvq_decode_attention(cfg.ref, None, 0, 1, None, None, None, 1.0, 0, None, None,
                                  None) == kvq.KVQ_ERR_NULL
    assert L.kvq_decode_attention(None, None, 0, 1, None, None, None, 1.0, 0, None,
                                  C.byref(n), None) == kvq.KVQ_ERR_NULL


def test_decode_append_validation(L):
    """kvq_decode_attention_append: the size query equals the decode's, and
    the append sources are checked (null, alignment, dtype) before any
    launch."""
    cfg = _cfg()

    def app(k=A16 + 8192, v=A16 + 12288, dt=kvq.KVQ_SRC_BF16, ws=A256 + 4096, chunk=64,
            ws_bytes=1 << 30, layer_begin=0):
        n = C.c_size_t(ws_bytes)
        st = L.kvq_decode_attention_append(
            cfg.ref, C.c_void_p(A256), layer_begin, 1, C.c_void_p(A16),
            C.c_void_p(k) if k else None, C.c_void_p(v) if v else None, dt, C.c_void_p(A16),
            C.c_void_p(A16 + 4096), 0.125, chunk, C.c_void_p(ws) if ws else None, C.byref(n),
            None)
        return st, n.value
    st, n = app(ws=None)
    assert st == kvq.KVQ_OK and n == kvq.workspace_bytes(cfg, 1, 64)
    assert app(k=None)[0] == kvq.KVQ_ERR_NULL
    assert app(v=None)[0] == kvq.KVQ_ERR_NULL
    assert app(k=A16 + 8)[0] == kvq.KVQ_ERR_ALIGN
    assert app(v=A16 + 4)[0] == kvq.KVQ_ERR_ALIGN
    assert app(dt=7)[0] == kvq.KVQ_ERR_UNSUPPORTED
    assert app(ws_bytes=n - 1)[0] == kvq.KVQ_ERR_WORKSPACE
    assert app(layer_begin=1)[0] == kvq.KVQ_ERR_RANGE
    assert app(chunk=48)[0] == kvq.KVQ_ERR_SHAPE


def _headguard_like(num_layers):
    return kvq.Config(num_layers, 1, 28, 4, 128, 64, [6288], [14], [6287], [4] * 4 * num_layers,
                      [2] * 4 * num_layers)


def test_workspace_size_depends_on_cache_layer_count(L):
    """The arrival counters are sized by the cache's layer count, so two caches
    that differ only in it need different workspaces, whatever was planned
    before in the same process (the plans are cached per call shape)."""
    code = ("from quantized_decode_attention_quantize_amd import kvq\n"
            "def h(n): return kvq.Config(n, 1, 28, 4, 128, 64, [6288], [14], [6287], "
            "[4] * 4 * n, [2] * 4 * n)\n"
            "print(kvq.workspace_bytes(h(28), 1), kvq.workspace_bytes(h(1), 1))")
    fresh = subprocess.run(["python", "-c", code], capture_output=True, text=True, check=True,
                           cwd=ROOT).stdout.split()
    a1 = kvq.workspace_bytes(_headguard_like(1), 1)
    a28 = kvq.workspace_bytes(_headguard_like(28), 1)
    b1 = kvq.workspace_bytes(_headguard_like(1), 1)
    assert [str(a28), str(a1)] == fresh
    assert a1 == b1 and a28 > a1


def test_binding_rejects_wrong_dtypes_and_sizes(L):
    """The Python binding checks dtypes and element counts against the config
    before it hands any pointer to the library (CPU tensors: every check below
    fires before the device check)."""
    import torch
    cfg = _cfg(batch=2, capacity=[64, 40], vis_begin=[8, 0], vis_end=[64, 20])
    need = kvq.kvq_cache_bytes(cfg)["total_bytes"]
    cache = torch.zeros(need, dtype=torch.uint8)
    lens = torch.tensor([64, 40], dtype=torch.int32)
    q = torch.zeros(1, 2, 4, 64, dtype=torch.bfloat16)
    out = torch.zeros_like(q)
    ws = torch.zeros(1 << 16, dtype=torch.uint8)

    def dec(**over):
        a = dict(cache=cache, seq_lens=lens, q=q, out=out, workspace=ws)
        a.update(over)
        kvq.kvq_decode_attention(cfg, a["cache"], 0, 1, a["seq_lens"], a["q"], a["out"], 0.125,
                                 0, a["workspace"])

    bad = [dict(cache=torch.zeros(need - 1, dtype=torch.uint8)),
           dict(cache=torch.zeros(need, dtype=torch.int32)),
           dict(seq_lens=lens.long()), dict(seq_lens=lens[:1]),
           dict(q=q.float()), dict(q=q[:, :1]), dict(out=out.half()),
           dict(out=torch.zeros(1, 2, 4, 32, dtype=torch.bfloat16))]
    for over in bad:
        with pytest.raises(ValueError):
            dec(**over)
    with pytest.raises(ValueError, match="device tensor"):
        dec()  # everything well-formed but on the host
    k = torch.zeros(1, 2, 1, 8, 64, dtype=torch.bfloat16)
    for kk, vv in [(k.float(), k), (k.half(), k.half()), (k[:, :1], k[:, :1]),
                   (torch.zeros(1, 2, 1, 7, 64, dtype=torch.bfloat16),) * 2]:
        with pytest.raises(ValueError):
            kvq.kvq_quantize(cfg, cache, 0, 1, [0, 1], 0, 8, kk, vv)
        with pytest.raises(ValueError):
            kvq.kvq_quantize_ragged(cfg, cache, 0, 1, [0, 1], [0, 3], 8, kk, vv)
    with pytest.raises(ValueError, match="device tensor"):
        kvq.kvq_quantize(cfg, cache, 0, 1, [0, 1], 0, 8, k, k)


def test_per_channel_validation(L):
    """Per-channel K: a store that cuts a block of the coded span, rotation on
    top, fixed chunks off the 256-token grid and coded K with bf16 V are
    refused before any launch; shapes of several query-head subgroups run."""
    cfg = _cfg(capacity=[256], vis_begin=[16], vis_end=[250])  # coded [16, 240), g 32
    pc = kvq.Config(**{**dict(num_layers=1, batch=1, num_q_heads=4, num_kv_heads=1, head_dim=64,
                              group_size=32, capacity=[256], vis_begin=[16], vis_end=[250],
                              k_bits=[4], v_bits=[2]), "k_per_channel": True})
    assert _quant(L, pc, t0=0, t1=40) == kvq.KVQ_ERR_SHAPE      # cuts [16, 48)
    assert _quant(L, pc, t0=20, t1=48) == kvq.KVQ_ERR_SHAPE     # starts inside a block
    assert _quant(L, pc, t0=16, t1=48, cache=None) == kvq.KVQ_ERR_NULL  # whole block: passes shape
    assert _quant(L, pc, t0=240, t1=256, cache=None) == kvq.KVQ_ERR_NULL  # residual + text
    info = kvq.kvq_cache_bytes(pc)
    assert info["quantized_values"] == (240 - 16) * 64 * 2
    assert _dec(L, pc, chunk=64)[0] == kvq.KVQ_ERR_UNSUPPORTED
    assert _dec(L, pc, chunk=256, ws=None)[0] == kvq.KVQ_OK
    assert _dec(L, pc, ws=None)[0] == kvq.KVQ_OK
    bf16v = kvq.Config(1, 1, 4, 1, 64, 32, [256], [16], [250], [4], [16], k_per_channel=True)
    assert _dec(L, bf16v, ws=None)[0] == kvq.KVQ_ERR_UNSUPPORTED
    rot = kvq.Config(1, 1, 4, 1, 64, 32, [256], [16], [250], [4], [2], rotate_k=True,
                     k_per_channel=True)
    with pytest.raises(kvq.KvqError) as e:
        kvq.kvq_cache_bytes(rot)
    assert e.value.status == kvq.KVQ_ERR_UNSUPPORTED
    wide = kvq.Config(1, 1, 28, 4, 128, 32, [256], [16], [256], [4] * 4, [2] * 4,
                      k_per_channel=True)  # 28 (head, group) columns: two subgroups
    assert _dec(L, wide, ws=None)[0] == kvq.KVQ_OK
    del cfg


def test_bf16_range_validation(L):
    """bf16 ranges: malformed tables are shape errors, missing arrays null
    errors, and per-channel K with ranges or more than 36 ranges in a
    sequence are refused."""
    def cfg(ranges, **over):
        base = dict(num_layers=1, batch=2, num_q_heads=4, num_kv_heads=1, head_dim=64,
                    group_size=32, capacity=[256, 300], vis_begin=[16, 0],
                    vis_end=[250, 300], k_bits=[4], v_bits=[2], bf16_ranges=ranges)
        base.update(over)
        return kvq.Config(**base)

    def status(c):
        try:
            kvq.kvq_cache_bytes(c)
            return kvq.KVQ_OK
        except kvq.KvqError as e:
            return e.status

    assert status(cfg([[(16, 17), (100, 250)], [(0, 300)]])) == kvq.KVQ_OK
    assert status(cfg([[], []])) == kvq.KVQ_OK
    assert status(cfg([[(15, 17)], []])) == kvq.KVQ_ERR_SHAPE     # starts before the span
    assert status(cfg([[(16, 251)], []])) == kvq.KVQ_ERR_SHAPE    # ends after it
    assert status(cfg([[(20, 20)], []])) == kvq.KVQ_ERR_SHAPE     # empty
    assert status(cfg([[(30, 40), (20, 25)], []])) == kvq.KVQ_ERR_SHAPE  # unsorted
    assert status(cfg([[(30, 40), (39, 45)], []])) == kvq.KVQ_ERR_SHAPE  # overlapping
    assert status(cfg([[(17, 18)], []], k_per_channel=True)) == kvq.KVQ_ERR_UNSUPPORTED
    assert status(cfg([[], []], k_per_channel=True)) == kvq.KVQ_OK
    many = [(20 + 4 * i, 22 + 4 * i) for i in range(37)]
    assert status(cfg([many, []])) == kvq.KVQ_ERR_UNSUPPORTED
    assert status(cfg([many[:36], many[:36]])) == kvq.KVQ_OK
    c = cfg([[(16, 17)], []])
    c.c.bf16_range_end = C.POINTER(C.c_int32)()
    info = kvq._Info()
    assert L.kvq_cache_bytes(c.ref, C.byref(info)) == kvq.KVQ_ERR_NULL
    c = cfg([[(16, 17)], []])
    c._rng_off[0] = 1
    assert status(c) == kvq.KVQ_ERR_SHAPE
    c = cfg([[(16, 17)], []])
    c._rng_off[1] = 2  # offsets must not decrease
    assert status(c) == kvq.KVQ_ERR_SHAPE
    # storage: ranges move rows from the VIS plane to the TXT plane
    plain = kvq.kvq_cache_bytes(cfg(None))
    moved = kvq.kvq_cache_bytes(cfg([[(16, 17), (100, 250)], [(0, 300)]]))
    assert plain["quantized_values"] - moved["quantized_values"] == (1 + 150 + 300) * 64 * 2
    assert moved["bf16_text_bytes"] - plain["bf16_text_bytes"] == (1 + 150 + 300) * 64 * 2 * 2
    # decode takes ranges in the balanced split and in fixed chunks
    ok = cfg([[(16, 17), (100, 250)], []])
    assert _dec(L, ok, ws=None)[0] == kvq.KVQ_OK
    assert _dec(L, ok, chunk=64, ws=None)[0] == kvq.KVQ_OK


def test_latent_cache_bytes_and_validation(L):
    """Latent cache: sizes equal the oracle layout's, malformed configs and
    calls are refused before any launch."""
    from oracle import latent as olat

    def cfg(**over):
        base = dict(num_layers=2, batch=3, num_q_heads=8, num_kv_heads=2, head_dim=128,
                    rank=96, capacity=[5, 33, 64])
        base.update(over)
        return kvq.LatentConfig(**base)

    def status(c):
        try:
            kvq.kvq_latent_cache_bytes(c)
            return kvq.KVQ_OK
        except kvq.KvqError as e:
            return e.status

    for r, D in ((32, 64), (64, 64), (32, 128), (96, 128), (128, 128)):
        c = cfg(rank=r, head_dim=D)
        assert kvq.kvq_latent_cache_bytes(c) == olat.cache_bytes(2, 2, [5, 33, 64], r)
    assert status(cfg(rank=48)) == kvq.KVQ_ERR_UNSUPPORTED
    assert status(cfg(rank=128, head_dim=64)) == kvq.KVQ_ERR_UNSUPPORTED
    assert status(cfg(head_dim=96)) == kvq.KVQ_ERR_UNSUPPORTED
    assert status(cfg(num_q_heads=7)) == kvq.KVQ_ERR_UNSUPPORTED
    assert status(cfg(num_q_heads=34)) == kvq.KVQ_ERR_UNSUPPORTED   # ratio 17
    assert status(cfg(capacity=[5, 0, 64])) == kvq.KVQ_ERR_SHAPE
    assert status(cfg(num_layers=0)) == kvq.KVQ_ERR_SHAPE
    assert status(cfg(batch=1, capacity=[1 << 23], rank=128)) == kvq.KVQ_ERR_UNSUPPORTED
    c = cfg()
    assert L.kvq_latent_cache_bytes(c.ref, None) == kvq.KVQ_ERR_NULL
    c.c.capacity = C.POINTER(C.c_int32)()
    assert L.kvq_latent_cache_bytes(c.ref, C.byref(C.c_uint64())) == kvq.KVQ_ERR_NULL

    c = cfg()
    ids = np.array([1], dtype=np.int32)
    ip = ids.ctypes.data_as(C.POINTER(C.c_int32))

    def store(layer_begin=0, nl=1, t0=0, t1=8, cache=A256, k=A16, ids_p=ip, n=1):
        return L.kvq_latent_store(c.ref, C.c_void_p(cache) if cache else None, layer_begin, nl,
                                  n, ids_p, t0, t1, C.c_void_p(k) if k else None,
                                  C.c_void_p(A16), None)
    assert store(t1=34) == kvq.KVQ_ERR_RANGE      # past capacity 33
    assert store(t0=-1) == kvq.KVQ_ERR_RANGE
    assert store(layer_begin=1, nl=2) == kvq.KVQ_ERR_RANGE
    assert store(cache=A256 + 16) == kvq.KVQ_ERR_ALIGN
    assert store(k=A16 + 2) == kvq.KVQ_ERR_ALIGN
    assert store(k=None) == kvq.KVQ_ERR_NULL
    assert store(t0=8, t1=4) == kvq.KVQ_ERR_SHAPE
    assert store(t0=3, t1=3) == kvq.KVQ_OK          # empty: no launch
    two = np.array([1, 1], dtype=np.int32)
    assert store(ids_p=two.ctypes.data_as(C.POINTER(C.c_int32)), n=2) == kvq.KVQ_ERR_SHAPE
    bad = np.array([3], dtype=np.int32)
    assert store(ids_p=bad.ctypes.data_as(C.POINTER(C.c_int32))) == kvq.KVQ_ERR_RANGE

    def dec(layer_begin=0, nl=1, chunk=0, ws=A256 + 4096, ws_bytes=1 << 30, q=A16, scale=0.1):
        n = C.c_size_t(ws_bytes)
        st = L.kvq_latent_decode(c.ref, C.c_void_p(A256), layer_begin, nl, C.c_void_p(A16),
                                 C.c_void_p(A16), C.c_void_p(A16), C.c_void_p(q) if q else None,
                                 C.c_void_p(A16 + 4096), scale, chunk,
                                 C.c_void_p(ws) if ws else None, C.byref(n), None)
        return st, n.value
    st, need = dec(ws=None)
    assert st == kvq.KVQ_OK and need > 0
    entries = 1 * 3 * 2 * 1  # one chunk per sequence at these capacities
    counters = 256           # 2 layers * 3 sequences * 2 KV heads int32, padded to 256 B
    assert need == counters + -(-(entries * 4 * 128 * 4) // 256) * 256 + entries * 4 * 2 * 4
    assert dec(ws_bytes=need - 1)[0] == kvq.KVQ_ERR_WORKSPACE
    assert dec(layer_begin=2)[0] == kvq.KVQ_ERR_RANGE
    assert dec(nl=0)[0] == kvq.KVQ_ERR_SHAPE
    assert dec(chunk=48)[0] == kvq.KVQ_ERR_SHAPE
    assert dec(scale=0.0)[0] == kvq.KVQ_ERR_SHAPE
    assert dec(q=None)[0] == kvq.KVQ_ERR_NULL
    assert dec(q=A16 + 4)[0] == kvq.KVQ_ERR_ALIGN
    assert dec(ws=A256 + 64)[0] == kvq.KVQ_ERR_ALIGN
    # 32-token chunks: the longest sequence (64 rows) has 2, so 2 slots per entry
    assert dec(chunk=32, ws=None)[1] == counters + \
        -(-(1 * 3 * 2 * 2 * 4 * 128 * 4) // 256) * 256 + 1 * 3 * 2 * 2 * 4 * 2 * 4
