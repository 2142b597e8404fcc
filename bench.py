"""Decode-step benchmark of libkvq on one MI355X.

One step = the hot path of one decode step over a whole model, in one
launch of kvq_decode_attention_append:
  1. the new token's K/V rows are stored for every layer and KV head
     (position T: a generated token, so a bf16 text row), by the wave that
     attends that position, then
  2. the launch attends over [0, T+1) for every layer, KV head and query head
     (split-K over token chunks + log-sum-exp merge).
The same step with the append as a launch of its own (kvq_quantize, then
kvq_decode_attention) is reported among the extras.
The cache is rotated over several replicas (>= 2 GB in total) so each step
reads HBM, not the 256 MB Infinity Cache: at 2 GB even the bf16 rows of the
protected heads alone (about 40 % of a step's bytes) span far more than that
cache holds.  Inputs are resident in HBM before the timed region.

Printed: one JSON line (rank 0).  `value` is effective HBM GB/s of the whole
step (algorithmic bytes / step time); `roofline` refers to the decode
attention launch, timed with HIP events on the stream it runs on.
`cpu_baseline` times the CPU oracle on all host threads (and on one) over a
bounded sample of the same workload, scaled to one step.  Extras: the bf16
reference decode, the long-context (32K) decode, a read-only stream kernel
as the practical HBM ceiling, a device copy, the quantize block, rotated K,
per-channel K, the latent decode, the two-launch step and the layer-by-layer
launch pattern.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time
import types

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0  # MI355X HBM3E, vendor figure


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="headguard_step",
                    choices=["headguard_step", "long_gqa", "llava_layer", "ragged_serving"])
    ap.add_argument("--chunk", type=int, default=0, help="split chunk in tokens (0 = library)")
    ap.add_argument("--replica-mb", type=int, default=2048)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU-oracle baseline")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the bf16 reference, quantize block and copy measurements")
    ap.add_argument("--k-per-channel", action="store_true",
                    help="cache with K grouped per channel over token blocks (chunk 0 or a "
                         "multiple of 256)")
    ap.add_argument("--protected", type=int, default=14,
                    help="HeadGuard protected (bf16) heads of the 28-layer step")
    ap.add_argument("--eager", action="store_true",
                    help="time plain launches instead of a replayed HIP graph")
    ap.add_argument("--copy-only", action="store_true",
                    help="only run a plain 1 GiB device copy (counter calibration)")
    return ap.parse_args()


def workload(name, protected=14):
    from quantized_decode_attention_quantize_amd import synth
    if name == "headguard_step":
        return synth.headguard_step(num_protected=protected, extra_capacity=1)
    if name == "long_gqa":
        w = synth.long_gqa()
    elif name == "llava_layer":
        w = synth.llava_layer(kbits=4, vbits=2)
    else:
        w = synth.ragged_serving()
    w.capacity = [c + 1 for c in w.capacity]
    return w


def describe(w):
    return {
        "headguard_step": "LLaVA-OneVision-7B-shaped full decode step: 28 layers x 4 KV heads "
                          "(28 query heads, D=128), 14 text + 6273 visual + 1 appended token; "
                          "14 seeded protected heads bf16, others K INT4 / V INT2, group 64",
        "long_gqa": "B=4 x 32768 tokens, 32 query / 8 KV heads, D=128, K INT4 / V INT2 g64",
        "llava_layer": "one LLaVA-shaped layer, 6287+1 tokens, K INT4 / V INT2 g64",
        "ragged_serving": "B=64 ragged 1024..16384 tokens, 28/4 heads, K INT8 / V INT4 g64",
    }[w.name]


def stored_row_bytes(w, l, h, X, t, s):
    D, g = w.head_dim, w.group_size
    b = int((w.v_bits if X else w.k_bits)[l * w.num_kv_heads + h])
    visual = w.vis_begin[s] <= t < w.vis_end[s]
    if visual and b < 16:
        return D * b // 8 + (D // g) * 4
    return 2 * D


def algorithmic_bytes(w, lens):
    """Stored K/V bytes every attended position costs, plus q and out.  With
    per-channel K the coded span is its whole blocks of group_size tokens;
    the residual tail is stored, and counted, as bf16 rows."""
    D, g = w.head_dim, w.group_size
    vis_end = list(w.vis_end)
    if getattr(w, "k_per_channel", False):
        vis_end = [w.vis_begin[s] + (w.vis_end[s] - w.vis_begin[s]) // g * g
                   for s in range(w.batch)]
    total = 0
    for l in range(w.num_layers):
        for h in range(w.num_kv_heads):
            for X in (0, 1):
                b = int((w.v_bits if X else w.k_bits)[l * w.num_kv_heads + h])
                for s in range(w.batch):
                    n = lens[s]
                    nv = max(0, min(n, vis_end[s]) - w.vis_begin[s])
                    nt = n - nv
                    vis_row = (D * b // 8 + (D // g) * 4) if b < 16 else 2 * D
                    total += nv * vis_row + nt * 2 * D
    total += 2 * w.num_layers * w.batch * w.num_q_heads * D * 2  # q in, out
    return total


KERNEL_SOURCES = ["kvq_decode_mfma.hip", "kvq_internal.h", "kvq_api.hip"]


def counted_traffic(name):
    """HBM bytes per decode launch (scaled FETCH_SIZE + WRITE_SIZE) from the
    committed rocprofv3 summary of this workload, or None when there is none
    or the kernel sources have changed since the counters were taken."""
    import hashlib
    import re
    path = os.path.join(ROOT, "profiles", f"decode_mfma_{name}.md")
    if not os.path.exists(path):
        return None, None
    m = re.search(r"traffic_bytes_per_launch=(\d+) kernel_source_sha256_16=([0-9a-f]+)",
                  open(path).read())
    if not m:
        return None, None
    csrc = os.path.join(ROOT, "quantized_decode_attention_quantize_amd", "csrc")
    sha = hashlib.sha256(b"".join(open(os.path.join(csrc, f), "rb").read()
                                  for f in KERNEL_SOURCES)).hexdigest()[:16]
    if sha != m.group(2):
        return None, os.path.relpath(path, ROOT) + " (kernel changed since; not used)"
    return int(m.group(1)), os.path.relpath(path, ROOT)


def timed(torch, args, enqueue):
    """Milliseconds per call of `enqueue(i)`, i = 0..K-1, measured with HIP
    events on the current stream.  By default the K calls are captured once
    into a HIP graph (the library's host-side planning runs at capture) and
    the graph is replayed; a spin kernel ahead of the start event keeps the
    host's graph submission out of the measured interval.  --eager times
    plain launches instead (host-bound for short kernels)."""
    stream = torch.cuda.current_stream()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    if args.eager:
        torch.cuda.synchronize()
        t0.record(stream)
        for i in range(args.steps):
            enqueue(i)
        t1.record(stream)
        torch.cuda.synchronize()
        return t0.elapsed_time(t1) / args.steps
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(args.steps):
            enqueue(i)
    g.replay()  # first replay uploads the graph
    torch.cuda.synchronize()
    torch.cuda._sleep(20_000_000)
    t0.record(stream)
    g.replay()
    t1.record(stream)
    torch.cuda.synchronize()
    return t0.elapsed_time(t1) / args.steps


class Events:
    def __init__(self, torch, n):
        self.s = [torch.cuda.Event(enable_timing=True) for _ in range(n)]
        self.e = [torch.cuda.Event(enable_timing=True) for _ in range(n)]

    def times_ms(self):
        return np.array([a.elapsed_time(b) for a, b in zip(self.s, self.e)])


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for {args.gpus}); the library has no "
              "multi-GPU path: the decode kernel runs on one GPU's share and sharding is "
              "left to the caller (independent (layer, sequence, KV head) entries)", file=sys.stderr)
        sys.exit(2)
    import torch
    from quantized_decode_attention_quantize_amd import kvq, synth

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.copy_only:
        print(json.dumps({"copy_ceiling": copy_ceiling(torch, dev, torch.cuda.current_stream())}))
        return
    kvq.lib()
    stream = torch.cuda.current_stream()

    w = workload(args.workload, args.protected)
    w.k_per_channel = args.k_per_channel
    T = [c - 1 for c in w.capacity]          # history length before the step
    lens = [t + 1 for t in T]                # attended after appending
    cfg = kvq.Config.from_workload(w)
    info = kvq.kvq_cache_bytes(cfg)
    nbytes = info["total_bytes"]
    R = max(2, math.ceil(args.replica_mb * 2 ** 20 / nbytes))
    log(f"workload {w.name}: cache {nbytes / 1e6:.1f} MB x {R} replicas")

    ref_cfg = None
    if not args.no_extras:
        rw = workload(args.workload, args.protected)
        rw.k_bits[:] = 16
        rw.v_bits[:] = 16
        ref_cfg = kvq.Config.from_workload(rw)
        ref_bytes = kvq.kvq_cache_bytes(ref_cfg)["total_bytes"]
        R_ref = max(2, math.ceil(args.replica_mb * 2 ** 20 / ref_bytes))

    # ---- fill caches (untimed) ------------------------------------------
    t_gen = time.time()
    cache0 = torch.zeros(nbytes, dtype=torch.uint8, device=dev)
    ref0 = torch.zeros(ref_bytes, dtype=torch.uint8, device=dev) if ref_cfg else None

    def to_dev(a):
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(a).to(dev)

    for l in range(w.num_layers):
        for s in range(w.batch):
            k = to_dev(w.sources(l, [s], 0, T[s], "k")[None])
            v = to_dev(w.sources(l, [s], 0, T[s], "v")[None])
            kvq.kvq_quantize(cfg, cache0, l, 1, [s], 0, T[s], k, v)
            if ref0 is not None:
                kvq.kvq_quantize(ref_cfg, ref0, l, 1, [s], 0, T[s], k, v)
        if l % 7 == 0:
            log(f"stored layer {l}")
    torch.cuda.synchronize()
    caches = [cache0] + [cache0.clone() for _ in range(R - 1)]
    refs = ([ref0] + [ref0.clone() for _ in range(R_ref - 1)]) if ref0 is not None else []
    log(f"caches ready in {time.time() - t_gen:.1f} s")

    # new token's K/V (bf16) for all layers: [L, B, Hkv, 1, D]
    from quantized_decode_attention_quantize_amd.synth import TAG_APPEND_K, TAG_APPEND_V
    kn = np.stack([np.stack([np.stack([w.k_rows(l, s, h, T[s], T[s] + 1, TAG_APPEND_K)
                                        for h in range(w.num_kv_heads)])
                              for s in range(w.batch)]) for l in range(w.num_layers)])
    vn = np.stack([np.stack([np.stack([w.v_rows(l, s, h, T[s], T[s] + 1, TAG_APPEND_V)
                                        for h in range(w.num_kv_heads)])
                              for s in range(w.batch)]) for l in range(w.num_layers)])
    k_new, v_new = to_dev(kn), to_dev(vn)
    q_bits = np.stack([w.q_bits(l) for l in range(w.num_layers)])
    q = to_dev(q_bits)
    out = torch.empty_like(q)
    lens_d = torch.tensor(lens, dtype=torch.int32, device=dev)
    seq_ids = list(range(w.batch))
    ws = torch.zeros(kvq.workspace_bytes(cfg, w.num_layers, args.chunk), dtype=torch.uint8,
                     device=dev)
    same_T = len(set(T)) == 1

    def step(i):
        # the appended token (position T[s], a text row) is stored by the
        # decode launch itself, by the wave that attends it
        kvq.kvq_decode_attention_append(cfg, caches[i % R], 0, w.num_layers, lens_d, k_new,
                                        v_new, q, out, w.sm_scale, args.chunk, ws)

    def step_separate(i):
        c = caches[i % R]
        if same_T:
            kvq.kvq_quantize(cfg, c, 0, w.num_layers, seq_ids, T[0], T[0] + 1, k_new, v_new)
        else:  # ragged batch: every sequence appends at its own length, one launch
            kvq.kvq_quantize_ragged(cfg, c, 0, w.num_layers, seq_ids, T, 1, k_new, v_new)
        kvq.kvq_decode_attention(cfg, c, 0, w.num_layers, lens_d, q, out, w.sm_scale,
                                 args.chunk, ws)

    def decode_only(i):
        kvq.kvq_decode_attention(cfg, caches[i % R], 0, w.num_layers, lens_d, q, out,
                                 w.sm_scale, args.chunk, ws)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    ms_step = timed(torch, args, lambda i: step(args.warmup + i))
    dec_avg = timed(torch, args, decode_only)

    alg = algorithmic_bytes(w, lens)
    append_bytes = 2 * w.num_layers * w.batch * w.num_kv_heads * w.head_dim * 2 * 2
    step_bytes = alg + append_bytes
    value = step_bytes / (ms_step * 1e-3) / 1e9
    dec_gbs = alg / (dec_avg * 1e-3) / 1e9
    log(f"step {ms_step * 1e3:.1f} us, decode {dec_avg * 1e3:.1f} us per launch, "
        f"{dec_gbs:.0f} GB/s")

    extras = {}
    if not args.no_extras:
        # the same step with the append as a launch of its own (kvq_quantize
        # or kvq_quantize_ragged, then kvq_decode_attention)
        sep_ms = timed(torch, args, step_separate)
        extras["separate_append_step"] = {
            "us": round(sep_ms * 1e3, 2), "launches": 2,
            "gbps": round(step_bytes / (sep_ms * 1e-3) / 1e9, 1)}
    if not args.no_extras and w.num_layers > 1:
        # the same step as a layer-by-layer serving loop issues it: one
        # decode launch per layer, back to back
        def per_layer(i):
            c = caches[i % R]
            for l in range(w.num_layers):
                kvq.kvq_decode_attention(cfg, c, l, 1, lens_d, q[l:l + 1], out[l:l + 1],
                                         w.sm_scale, args.chunk, ws)
        pl_ms = timed(torch, args, per_layer)
        extras["per_layer_launches"] = {
            "launches": w.num_layers, "us": round(pl_ms * 1e3, 2),
            "us_per_layer": round(pl_ms * 1e3 / w.num_layers, 2),
            "vs_one_launch": round(pl_ms / dec_avg, 3)}
    if not args.no_extras:
        # bf16 reference: same shapes, every row bf16 (bandwidth reference)
        ref_alg = algorithmic_bytes(_bf16_like(w), lens)
        wsr = torch.zeros(kvq.workspace_bytes(ref_cfg, w.num_layers, args.chunk),
                          dtype=torch.uint8, device=dev)
        for i in range(args.warmup):
            kvq.kvq_decode_attention(ref_cfg, refs[i % R_ref], 0, w.num_layers, lens_d, q, out,
                                     w.sm_scale, args.chunk, wsr)
        r_ms = timed(torch, args, lambda i: kvq.kvq_decode_attention(
            ref_cfg, refs[i % R_ref], 0, w.num_layers, lens_d, q, out, w.sm_scale, args.chunk,
            wsr))
        extras["bf16_reference_decode"] = {
            "us": round(r_ms * 1e3, 2), "algorithmic_bytes": ref_alg,
            "gbps": round(ref_alg / (r_ms * 1e-3) / 1e9, 1),
            "speedup_of_quantized": round(r_ms / dec_avg, 3)}
        del refs, wsr
        if not args.k_per_channel:  # rotation and per-channel K do not combine
            extras["rotated_k_decode"] = rotated_decode(torch, kvq, w, args, dev, T, lens_d, q,
                                                        out, to_dev, dec_avg, alg)
        if args.chunk == 0 and not args.k_per_channel:
            extras["per_channel_k_decode"] = per_channel_decode(torch, kvq, w, args, dev, T, lens_d,
                                                                q, out, to_dev, dec_avg)
        extras["quantize_block"] = quantize_block(torch, kvq, synth, dev, stream, args)
        extras["copy_ceiling"] = copy_ceiling(torch, dev, stream)
        extras["read_stream_ceiling"] = read_stream_ceiling(torch, dev, args, alg, dec_avg)
        if w.name != "long_gqa" and args.chunk == 0:
            extras["long_gqa_decode"] = long_context_decode(torch, kvq, args, dev)
        extras["latent_decode"] = latent_decode(torch, kvq, synth, args, dev)

    cpu = None if args.no_cpu else cpu_baseline(w, lens, q_bits, alg)
    profiled = (args.chunk == 0 and not args.k_per_channel and
                (w.name != "headguard_step" or args.protected == 14))
    traffic, traffic_src = counted_traffic(w.name) if profiled else (None, None)

    line = {
        "metric": "decode-attn µs/step + effective HBM GB/s (% of MI355X peak), INT4/INT2 KV",
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "us_per_step": round(ms_step * 1e3, 2),
        "pct_of_peak": round(100 * value / PEAK_HBM_GBS, 1),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16/bf16 MFMA operands, fp32 accumulate",
        "data": "synthetic",
        "config": {"workload": describe(w) + ("; K grouped per channel over blocks of the group "
                                              "size" if args.k_per_channel else ""),
                   "name": w.name, "layers": w.num_layers,
                   "batch": w.batch, "q_heads": w.num_q_heads, "kv_heads": w.num_kv_heads,
                   "head_dim": w.head_dim, "group": w.group_size, "tokens": lens,
                   "cache_replicas": R, "chunk_tokens": args.chunk,
                   "step_bytes": step_bytes} if w.batch <= 4 else
                  {"workload": describe(w), "name": w.name, "cache_replicas": R,
                   "step_bytes": step_bytes},
        "decode": {"us_per_launch": round(dec_avg * 1e3, 2), "algorithmic_bytes": alg,
                   "gbps": round(dec_gbs, 1),
                   "timing": "eager launches" if args.eager else
                             "HIP graph of K back-to-back launches, events around the replay"},
        "roofline": {"bound": "hbm", "achieved": round(dec_gbs, 1), "peak": PEAK_HBM_GBS,
                     "unit": "GB/s", "frac": round(dec_gbs / PEAK_HBM_GBS, 4),
                     "traffic": traffic, "traffic_source": traffic_src,
                     "algorithmic_bytes": alg,
                     "kernel": "decode_mfma_kernel (split-K, merge fused)"},
        "cpu_baseline": cpu,
    }
    line.update(extras)
    print(json.dumps(line), flush=True)


def rotated_decode(torch, kvq, w, args, dev, T, lens_d, q, out, to_dev, dec_avg, alg):
    """The same workload stored with Walsh-Hadamard rotated K codes (rotate_k):
    same bytes, plus the query rotation inside the kernel."""
    import copy
    rw = copy.deepcopy(w)
    rw.rotate_k = True
    cfg = kvq.Config.from_workload(rw)
    nbytes = kvq.kvq_cache_bytes(cfg)["total_bytes"]
    R = max(2, math.ceil(args.replica_mb * 2 ** 20 / nbytes))
    c0 = torch.zeros(nbytes, dtype=torch.uint8, device=dev)
    for l in range(rw.num_layers):
        for s in range(rw.batch):
            k = to_dev(rw.sources(l, [s], 0, T[s] + 1, "k")[None])
            v = to_dev(rw.sources(l, [s], 0, T[s] + 1, "v")[None])
            kvq.kvq_quantize(cfg, c0, l, 1, [s], 0, T[s] + 1, k, v)
    caches = [c0] + [c0.clone() for _ in range(R - 1)]
    ws = torch.zeros(kvq.workspace_bytes(cfg, rw.num_layers, args.chunk), dtype=torch.uint8,
                     device=dev)

    def dec(i):
        kvq.kvq_decode_attention(cfg, caches[i % R], 0, rw.num_layers, lens_d, q, out,
                                 rw.sm_scale, args.chunk, ws)

    for i in range(args.warmup):
        dec(i)
    ms = timed(torch, args, dec)
    del caches, ws
    return {"us": round(ms * 1e3, 2), "algorithmic_bytes": alg,
            "gbps": round(alg / (ms * 1e-3) / 1e9, 1),
            "vs_unrotated": round(ms / dec_avg, 3)}


def per_channel_decode(torch, kvq, w, args, dev, T, lens_d, q, out, to_dev, dec_avg):
    """The same workload with K grouped per channel over blocks of group_size
    visual tokens (k_per_channel): the coded span shrinks to whole blocks and
    the residual tail is bf16, so its algorithmic bytes are counted anew."""
    import copy
    pw = copy.deepcopy(w)
    pw.k_per_channel = True
    cfg = kvq.Config.from_workload(pw)
    nbytes = kvq.kvq_cache_bytes(cfg)["total_bytes"]
    R = max(2, math.ceil(args.replica_mb * 2 ** 20 / nbytes))
    c0 = torch.zeros(nbytes, dtype=torch.uint8, device=dev)
    for l in range(pw.num_layers):
        for s in range(pw.batch):
            k = to_dev(pw.sources(l, [s], 0, T[s] + 1, "k")[None])
            v = to_dev(pw.sources(l, [s], 0, T[s] + 1, "v")[None])
            kvq.kvq_quantize(cfg, c0, l, 1, [s], 0, T[s] + 1, k, v)
    caches = [c0] + [c0.clone() for _ in range(R - 1)]
    ws = torch.zeros(kvq.workspace_bytes(cfg, pw.num_layers, args.chunk), dtype=torch.uint8,
                     device=dev)

    def dec(i):
        kvq.kvq_decode_attention(cfg, caches[i % R], 0, pw.num_layers, lens_d, q, out,
                                 pw.sm_scale, args.chunk, ws)

    for i in range(args.warmup):
        dec(i)
    ms = timed(torch, args, dec)
    g = pw.group_size
    coded = [pw.vis_begin[s] + (pw.vis_end[s] - pw.vis_begin[s]) // g * g for s in range(pw.batch)]
    bw = copy.deepcopy(pw)
    bw.vis_end = coded  # the residual window counts as bf16 rows
    alg = algorithmic_bytes(bw, [t + 1 for t in T])
    del caches, ws
    return {"us": round(ms * 1e3, 2), "algorithmic_bytes": alg,
            "gbps": round(alg / (ms * 1e-3) / 1e9, 1), "vs_per_token": round(ms / dec_avg, 3)}


def _bf16_like(w):
    import copy
    r = copy.deepcopy(w)
    r.k_bits[:] = 16
    r.v_bits[:] = 16
    return r


def quantize_block(torch, kvq, synth, dev, stream, args):
    """Quantize path: a fresh 6273-token visual block (bf16 in) for 8
    sequences, K INT8 / V INT4 group 64 -> packed codes + meta."""
    w = synth.visual_block()
    cfg = kvq.Config.from_workload(w)
    cache = torch.zeros(kvq.kvq_cache_bytes(cfg)["total_bytes"], dtype=torch.uint8, device=dev)
    vb, ve = w.vis_begin[0], w.vis_end[0]
    seqs = list(range(w.batch))

    def to_dev(a):
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)

    k = to_dev(np.stack([w.sources(0, [s], vb, ve, "k")[0] for s in seqs])[None])
    v = to_dev(np.stack([w.sources(0, [s], vb, ve, "v")[0] for s in seqs])[None])
    R = 4
    ks = [k] + [k.clone() for _ in range(R - 1)]
    vs = [v] + [v.clone() for _ in range(R - 1)]
    n = ve - vb
    rd = 2 * w.batch * w.num_kv_heads * n * w.head_dim * 2
    wr = w.batch * w.num_kv_heads * n * (w.head_dim * 8 // 8 + w.head_dim * 4 // 8 + 2 * 8)
    for i in range(10):
        kvq.kvq_quantize(cfg, cache, 0, 1, seqs, vb, ve, ks[i % R], vs[i % R])
    torch.cuda.synchronize()
    # back-to-back launches in a graph, timed like the decode (see timed())
    qargs = types.SimpleNamespace(eager=False, steps=50)
    ms = timed(torch, qargs, lambda i: kvq.kvq_quantize(cfg, cache, 0, 1, seqs, vb, ve,
                                                         ks[i % R], vs[i % R]))
    return {"workload": "8 seqs x 6273 visual tokens x 4 KV heads, bf16 in, K INT8 / V INT4 g64",
            "us": round(ms * 1e3, 2), "read_bytes": rd, "write_bytes": wr,
            "gbps": round((rd + wr) / (ms * 1e-3) / 1e9, 1)}


def copy_ceiling(torch, dev, stream):
    """A plain device-to-device copy of 1 GiB: the practical HBM ceiling."""
    n = 2 ** 30
    a = torch.empty(n, dtype=torch.uint8, device=dev)
    b = torch.empty_like(a)
    a.fill_(1)
    for _ in range(3):
        b.copy_(a)
    ev = Events(torch, 10)
    for i in range(10):
        ev.s[i].record(stream)
        b.copy_(a)
        ev.e[i].record(stream)
    torch.cuda.synchronize()
    ms = float(np.median(ev.times_ms()))
    return {"bytes_moved": 2 * n, "gbps": round(2 * n / (ms * 1e-3) / 1e9, 1)}


def read_stream_ceiling(torch, dev, args, decode_bytes, decode_ms):
    """The practical HBM ceiling: a hand-written read-only stream kernel
    (libkvqbench.so) timed like the decode, once reading as many bytes per
    launch as the decode's algorithmic bytes and once 1 GiB per launch, each
    launch reading the next region of a >= 2 GiB buffer so the reads come
    from HBM."""
    import ctypes as C
    from quantized_decode_attention_quantize_amd import build
    lib = C.CDLL(build.BENCH_LIB)
    lib.kvqb_read_stream.restype = C.c_int
    lib.kvqb_read_stream.argtypes = [C.c_void_p, C.c_uint64, C.c_int, C.c_void_p, C.c_void_p]
    total = max(2 << 30, 4 * (1 << 30))
    buf = torch.ones(total, dtype=torch.uint8, device=dev)
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    out = {}
    for name, nbytes, grid in (("decode_bytes", decode_bytes // 16 * 16, 4096),
                               ("one_gib", 1 << 30, 4096)):
        R = total // nbytes

        def launch(i):
            # the stream current at the call: under graph capture, the capturing one
            st = torch.cuda.current_stream().cuda_stream
            rc = lib.kvqb_read_stream(C.c_void_p(buf.data_ptr() + (i % R) * nbytes), nbytes, grid,
                                      C.c_void_p(sink.data_ptr()), C.c_void_p(st))
            assert rc == 0, rc
        for i in range(5):
            launch(i)
        torch.cuda.synchronize()
        ms = timed(torch, types.SimpleNamespace(eager=False, steps=50 if nbytes < 1 << 28 else 10),
                   launch)
        gbs = nbytes / (ms * 1e-3) / 1e9
        out[name] = {"bytes": nbytes, "us": round(ms * 1e3, 2), "gbps": round(gbs, 1),
                     "frac_of_peak": round(gbs / PEAK_HBM_GBS, 4)}
    d = out["decode_bytes"]
    out["decode_vs_stream"] = round(d["us"] / (decode_ms * 1e3), 4)
    out["kernel"] = "kvqb_read_stream: 4096 workgroups x 512 threads, 8 x 16-byte loads in flight"
    del buf
    return out


def long_context_decode(torch, kvq, args, dev):
    """Decode-only timing of the long-context workload (B=4 x 32K tokens,
    32/8 heads, K INT4 / V INT2), the second configuration the bandwidth
    target names, with its roofline fraction and counted traffic."""
    w = workload("long_gqa")
    T = [c - 1 for c in w.capacity]
    lens = [t + 1 for t in T]
    cfg = kvq.Config.from_workload(w)
    nbytes = kvq.kvq_cache_bytes(cfg)["total_bytes"]
    R = max(2, math.ceil(args.replica_mb * 2 ** 20 / nbytes))
    c0 = torch.zeros(nbytes, dtype=torch.uint8, device=dev)

    def to_dev(a):
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)

    for s in range(w.batch):
        k = to_dev(w.sources(0, [s], 0, lens[s], "k")[None])
        v = to_dev(w.sources(0, [s], 0, lens[s], "v")[None])
        kvq.kvq_quantize(cfg, c0, 0, 1, [s], 0, lens[s], k, v)
    torch.cuda.synchronize()
    caches = [c0] + [c0.clone() for _ in range(R - 1)]
    q = to_dev(np.stack([w.q_bits(0)]))
    out = torch.empty_like(q)
    lens_d = torch.tensor(lens, dtype=torch.int32, device=dev)
    ws = torch.zeros(kvq.workspace_bytes(cfg, 1, 0), dtype=torch.uint8, device=dev)

    def dec(i):
        kvq.kvq_decode_attention(cfg, caches[i % R], 0, 1, lens_d, q, out, w.sm_scale, 0, ws)

    for i in range(args.warmup):
        dec(i)
    ms = timed(torch, args, dec)
    alg = algorithmic_bytes(w, lens)
    gbs = alg / (ms * 1e-3) / 1e9
    traffic, src = counted_traffic(w.name)
    # fixed splits: about S chunks per (sequence, KV head), S = 16, 32, 64
    sweep = {}
    for S in (16, 32, 64):
        chunk = 32 * math.ceil(max(lens) / (32 * S))
        wss = torch.zeros(kvq.workspace_bytes(cfg, 1, chunk), dtype=torch.uint8, device=dev)

        def dec_s(i, chunk=chunk, wss=wss):
            kvq.kvq_decode_attention(cfg, caches[i % R], 0, 1, lens_d, q, out, w.sm_scale, chunk,
                                     wss)

        for i in range(args.warmup):
            dec_s(i)
        sweep[str(S)] = {"chunk_tokens": chunk, "us": round(timed(torch, args, dec_s) * 1e3, 2)}
        del wss
    del caches, ws
    return {"workload": describe(w), "us": round(ms * 1e3, 2), "algorithmic_bytes": alg,
            "gbps": round(gbs, 1), "frac": round(gbs / PEAK_HBM_GBS, 4), "traffic": traffic,
            "traffic_source": src, "cache_replicas": R, "fixed_split_sweep": sweep}


def latent_decode(torch, kvq, synth, args, dev):
    """Decode over a per-head low-rank latent cache (rank 96) of the same
    28-layer LLaVA-shaped step: latents stream from HBM, the query is
    projected once per workgroup and B_V applied after the merge."""
    w = synth.llava_latent()
    cfg = kvq.LatentConfig(w.num_layers, w.batch, w.num_q_heads, w.num_kv_heads, w.head_dim,
                           w.rank, w.capacity)
    nbytes = kvq.kvq_latent_cache_bytes(cfg)
    R = max(2, math.ceil(args.replica_mb * 2 ** 20 / nbytes))

    def to_dev(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(
            torch.bfloat16).to(dev)

    c0 = torch.zeros(nbytes, dtype=torch.uint8, device=dev)
    T = w.capacity[0]
    for l in range(w.num_layers):
        kv = [to_dev(np.stack([w.latents(l, 0, h, X, 0, T) for h in range(w.num_kv_heads)])
                     [None, None]) for X in (0, 1)]
        kvq.kvq_latent_store(cfg, c0, l, 1, [0], 0, T, kv[0], kv[1])
    torch.cuda.synchronize()
    caches = [c0] + [c0.clone() for _ in range(R - 1)]
    up = [to_dev(np.stack([np.stack([w.up(l, h, X) for h in range(w.num_kv_heads)])
                           for l in range(w.num_layers)])) for X in (0, 1)]
    q = to_dev(np.stack([w.q_bits(l) for l in range(w.num_layers)]))
    out = torch.empty_like(q)
    lens_d = torch.tensor(w.seq_lens, dtype=torch.int32, device=dev)
    ws = torch.zeros(kvq.latent_workspace_bytes(cfg, w.num_layers, 0), dtype=torch.uint8,
                     device=dev)

    def dec(i):
        kvq.kvq_latent_decode(cfg, caches[i % R], 0, w.num_layers, lens_d, up[0], up[1], q, out,
                              w.sm_scale, 0, ws)

    for i in range(args.warmup):
        dec(i)
    ms = timed(torch, args, dec)
    L, H, r, D = w.num_layers, w.num_kv_heads, w.rank, w.head_dim
    alg = (2 * L * H * sum(w.seq_lens) * r * 2 + 2 * L * H * r * D * 2 +
           2 * L * w.batch * w.num_q_heads * D * 2)
    gbs = alg / (ms * 1e-3) / 1e9
    del caches, ws
    return {"workload": "28 layers x 4 KV heads (28 query heads, D=128), 6288 tokens, "
                        "bf16 latents of rank 96 with per-head up-projections",
            "us": round(ms * 1e3, 2), "algorithmic_bytes": alg, "gbps": round(gbs, 1),
            "frac": round(gbs / PEAK_HBM_GBS, 4), "cache_replicas": R,
            "kernels": "latent_decode_kernel (merge by the last chunk to finish)"}


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def host_threads():
    """Worker threads for the all-core timing: the CPUs this process may run
    on, at most 16 (the host share of one GPU on the boxes this runs on)."""
    try:
        n = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def cpu_baseline(w, lens, q_bits, alg_bytes, budget_s=8.0):
    """Time the CPU oracle decoding the step, on one thread and on all host
    threads.  A work unit is one (layer, sequence, KV head): its query heads
    over the full history.  The per-unit oracle stays single-threaded (the C
    calls release the GIL, so Python threads run units side by side).  Storing the
    rows is not timed.  One thread decodes units until about budget_s seconds
    are timed; the all-thread run then takes as many units as fill about
    budget_s seconds of wall time at that rate (every unit when the step fits)
    and both figures are scaled to one step."""
    import oracle
    from concurrent.futures import ThreadPoolExecutor
    cfg = oracle.Config.from_workload(w)
    cache = oracle.new_cache(cfg)
    G = w.num_q_heads // w.num_kv_heads
    units = [(l, s, h) for l in range(w.num_layers) for s in range(w.batch)
             for h in range(w.num_kv_heads)]
    stored = set()

    def store(l, s):
        T = lens[s] - 1
        for h in range(w.num_kv_heads):
            oracle.store_rows(cfg, cache, l, s, h, 0, 0, T, _f32(w.k_rows(l, s, h, 0, T)))
            oracle.store_rows(cfg, cache, l, s, h, 1, 0, T, _f32(w.v_rows(l, s, h, 0, T)))
            zero = np.zeros((1, w.head_dim), np.float32)
            oracle.store_rows(cfg, cache, l, s, h, 0, T, T + 1, zero)
            oracle.store_rows(cfg, cache, l, s, h, 1, T, T + 1, zero)
        stored.add((l, s))

    def decode(unit):
        l, s, h = unit
        for i in range(h * G, (h + 1) * G):
            oracle.decode_one(cfg, cache, l, s, i, lens[s], q_bits[l, s, i], w.sm_scale)

    # one thread
    dt1, n1 = 0.0, 0
    for u in units:
        if u[:2] not in stored:
            store(*u[:2])
        t0 = time.perf_counter()
        decode(u)
        dt1 += time.perf_counter() - t0
        n1 += 1
        if dt1 >= budget_s:
            break
    step1 = dt1 * len(units) / n1
    # every host thread, over as many units as fill about budget_s of wall time
    nt = host_threads()
    n_all = min(len(units), max(nt, int(budget_s * nt / (dt1 / n1))))
    sample = units[:n_all]
    for u in sample:
        if u[:2] not in stored:
            store(*u[:2])
    t0 = time.perf_counter()
    with ThreadPoolExecutor(nt) as ex:
        list(ex.map(decode, sample))
    dtn = time.perf_counter() - t0
    stepn = dtn * len(units) / n_all
    return {"value": round(alg_bytes / stepn / 1e9, 4), "unit": "GB/s", "cores": nt,
            "kind": "oracle", "cpu_model": cpu_model(),
            "seconds_per_step": round(stepn, 3),
            "sample": f"{n_all} of {len(units)} (layer, seq, KV head) units, their query heads "
                      f"over the full history, {dtn:.2f} s wall on {nt} threads, scaled "
                      f"x{len(units) / n_all:.2f} to one step",
            "one_thread": {"value": round(alg_bytes / step1 / 1e9, 4), "cores": 1,
                           "seconds_per_step": round(step1, 3),
                           "sample": f"{n1} units, {dt1:.2f} s, scaled x{len(units) / n1:.2f}"}}


def _f32(a):
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << np.uint32(16)).view(np.float32)
    return a.astype(np.float32)


if __name__ == "__main__":
    main()
