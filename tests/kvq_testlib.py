"""Helpers shared by the GPU tests: build the same cache on the GPU (libkvq)
and on the CPU (oracle) from the same seeded sources, compare stored bytes
outside the inter-plane padding, and compare attention outputs."""
from __future__ import annotations

from typing import Iterable, List, Optional, Sequence

import os

import numpy as np

import oracle
from quantized_decode_attention_quantize_amd import kvq, synth

# Tolerances on the bf16 attention output against the unrounded fp64 oracle
# (max abs error and relative L2 error over the whole compared tensor).
MAX_ABS = 5e-3
REL_L2 = 2e-3


def torch():
    import torch as _t
    return _t


def to_device_src(arr: np.ndarray, device="cuda"):
    t = torch()
    if arr.dtype == np.uint16:
        return t.from_numpy(np.ascontiguousarray(arr).view(np.int16)).view(t.bfloat16).to(device)
    return t.from_numpy(np.ascontiguousarray(arr, dtype=np.float32)).to(device)


def bf16_device(bits: np.ndarray, device="cuda"):
    t = torch()
    return t.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(t.bfloat16).to(device)


def bf16_to_f64(x) -> np.ndarray:
    t = torch()
    return x.detach().to(t.float64).cpu().numpy()


def as_f32(rows: np.ndarray) -> np.ndarray:
    if rows.dtype == np.uint16:
        return synth.bf16_bits_to_f32(rows)
    return rows.astype(np.float32)


def coded_count(w: synth.Workload, s: int) -> int:
    """Positions of sequence s stored as codes: the visual span (whole
    g-token blocks of it with per-channel K) minus its bf16 ranges."""
    n = w.vis_end[s] - w.vis_begin[s]
    if getattr(w, "k_per_channel", False):
        n -= n % w.group_size
    for b, e in (getattr(w, "bf16_ranges", None) or [[]] * w.batch)[s]:
        n -= e - b
    return int(n)


class Pair:
    """The same workload stored by libkvq on the GPU and by the oracle."""

    def __init__(self, w: synth.Workload, device="cuda"):
        t = torch()
        self.w = w
        self.cfg = kvq.Config.from_workload(w)
        self.ocfg = oracle.Config.from_workload(w)
        self.info = kvq.kvq_cache_bytes(self.cfg)
        self.cache = t.zeros(self.info["total_bytes"], dtype=t.uint8, device=device)
        self.ocache = oracle.new_cache(self.ocfg)
        self.device = device

    # --- storing ---------------------------------------------------------
    def store(self, layers: Optional[Sequence[int]] = None, seqs: Optional[Sequence[int]] = None,
              t0: int = 0, t1: Optional[int] = None, oracle_too: bool = True):
        """Store positions [t0, t1) (default: whole capacity) on both sides,
        one kvq_quantize call per (layer, sequence)."""
        w = self.w
        layers = range(w.num_layers) if layers is None else layers
        seqs = range(w.batch) if seqs is None else seqs
        for l in layers:
            for s in seqs:
                e = w.capacity[s] if t1 is None else t1
                k = w.sources(l, [s], t0, e, "k")
                v = w.sources(l, [s], t0, e, "v")
                kvq.kvq_quantize(self.cfg, self.cache, l, 1, [s], t0, e,
                                 to_device_src(k[None]), to_device_src(v[None]))
                if oracle_too:
                    for h in range(w.num_kv_heads):
                        oracle.store_rows(self.ocfg, self.ocache, l, s, h, 0, t0, e, as_f32(k[0, h]))
                        oracle.store_rows(self.ocfg, self.ocache, l, s, h, 1, t0, e, as_f32(v[0, h]))

    def gpu_bytes(self) -> np.ndarray:
        torch().cuda.synchronize()
        return self.cache.cpu().numpy()

    # --- byte regions ------------------------------------------------------
    def regions(self, layers: Optional[Iterable[int]] = None,
                seqs: Optional[Iterable[int]] = None) -> List[tuple]:
        """(start, end) byte ranges of stored rows (no padding), restricted to
        the given layers and sequences."""
        w = self.w
        D, g = w.head_dim, w.group_size
        layers = range(w.num_layers) if layers is None else layers
        seqs = range(w.batch) if seqs is None else seqs
        out = []
        vrow0, trow0, rv, rt = [], [], 0, 0
        coded = [coded_count(w, s) for s in range(w.batch)]
        for s in range(w.batch):
            nv = coded[s]
            vrow0.append(rv)
            trow0.append(rt)
            rv += nv
            rt += w.capacity[s] - nv
        for l in layers:
            for h in range(w.num_kv_heads):
                for X in (0, 1):
                    b = int((w.v_bits if X else w.k_bits)[l * w.num_kv_heads + h])
                    vis, meta, txt = oracle.plane_offsets(self.ocfg, l, h, X)
                    vrb = 2 * D if b == 16 else D * b // 8
                    for s in seqs:
                        nv = coded[s]
                        nt = w.capacity[s] - nv
                        if nv:
                            out.append((vis + vrow0[s] * vrb, vis + (vrow0[s] + nv) * vrb))
                            if b < 16:
                                mrb = (D // g) * 4
                                out.append((meta + vrow0[s] * mrb, meta + (vrow0[s] + nv) * mrb))
                        if nt:
                            out.append((txt + trow0[s] * 2 * D, txt + (trow0[s] + nt) * 2 * D))
        return out

    def mismatches(self, layers=None, seqs=None) -> int:
        g = self.gpu_bytes()
        bad = 0
        for a, b in self.regions(layers, seqs):
            bad += int(np.count_nonzero(g[a:b] != self.ocache[a:b]))
        return bad

    # --- decoding ----------------------------------------------------------
    def decode(self, lens: Sequence[int], layer_begin=0, num_layers=None, chunk=0, q_bits=None):
        """Run kvq_decode_attention; returns (out float64 [nl, B, Hq, D], q_bits)."""
        t = torch()
        w = self.w
        nl = w.num_layers - layer_begin if num_layers is None else num_layers
        if q_bits is None:
            q_bits = np.stack([w.q_bits(layer_begin + i) for i in range(nl)])
        q = bf16_device(q_bits, self.device)
        out = t.empty_like(q)
        lens_d = t.tensor(np.asarray(lens, dtype=np.int32), device=self.device)
        ws = t.zeros(kvq.workspace_bytes(self.cfg, nl, chunk), dtype=t.uint8, device=self.device)
        kvq.kvq_decode_attention(self.cfg, self.cache, layer_begin, nl, lens_d, q, out,
                                 w.sm_scale, chunk, ws)
        t.cuda.synchronize()
        return bf16_to_f64(out), q_bits

    def oracle_decode(self, layer: int, seq: int, qhead: int, length: int, q_bits_row):
        out, _ = oracle.decode_one(self.ocfg, self.ocache, layer, seq, qhead, length,
                                   q_bits_row, self.w.sm_scale)
        return out

    def oracle_decode_many(self, jobs):
        """oracle_decode over (layer, seq, qhead, length, q_bits_row) jobs on a
        pool of host threads (the C oracle runs without the interpreter lock),
        results in job order."""
        from concurrent.futures import ThreadPoolExecutor
        workers = max(1, min(16, os.cpu_count() or 1))
        with ThreadPoolExecutor(workers) as ex:
            return list(ex.map(lambda j: self.oracle_decode(*j), jobs))


def bf16_half_ulp(x: np.ndarray) -> np.ndarray:
    """Half the bf16 spacing at |x| (normal range): 2^(floor(log2|x|) - 8)."""
    _, e = np.frexp(np.abs(x))
    return np.where(x == 0, 0.0, np.ldexp(1.0, e - 9))


def errors(got: np.ndarray, ref: np.ndarray):
    """(max abs error beyond the output's own bf16 rounding, rel L2 error)."""
    diff = got - ref
    excess = float(np.max(np.abs(diff) - bf16_half_ulp(ref)))
    rel = float(np.linalg.norm(diff) / max(np.linalg.norm(ref), 1e-300))
    return excess, rel


def assert_close(got: np.ndarray, ref: np.ndarray, what: str = ""):
    """bf16 output vs unrounded fp64 oracle: every element within 5e-3 plus
    half a bf16 ulp of the reference (rounding the exact value to bf16 alone
    costs up to that half ulp), and relative L2 error <= 2e-3."""
    max_abs, rel = errors(got, ref)
    print(f"[close] {what}: max_abs={max_abs:.3e} rel_l2={rel:.3e}", flush=True)
    assert np.all(np.isfinite(got)), what
    assert max_abs <= MAX_ABS and rel <= REL_L2, f"{what}: max_abs={max_abs:.3e} rel_l2={rel:.3e}"
    return max_abs, rel


def kernel_error(got: np.ndarray, ref: np.ndarray, what: str = ""):
    """Split the output error into the bf16 rounding of the output itself and
    the kernel's own arithmetic (f16/bf16 operands, fp32 accumulation):
    relative L2 of got vs the exact reference, of the exact reference rounded
    to bf16 vs itself, of got vs that rounded reference (zero when every
    element rounds to the same bf16 the exact value does), and the excess of
    the first over the second in quadrature.  Returns the last: the part of
    the error the kernel adds to what rounding the exact output to bf16
    costs by itself."""
    t = torch()
    ref16 = t.from_numpy(np.ascontiguousarray(ref)).to(t.bfloat16).double().numpy()
    nr = max(float(np.linalg.norm(ref)), 1e-300)
    tot = float(np.linalg.norm(got - ref)) / nr
    rnd = float(np.linalg.norm(ref16 - ref)) / nr
    k16 = float(np.linalg.norm(got - ref16)) / nr
    exc = max(0.0, tot * tot - rnd * rnd) ** 0.5
    print(f"[err] {what}: total={tot:.3e} bf16_rounding={rnd:.3e} vs_rounded_ref={k16:.3e} "
          f"excess_in_quadrature={exc:.3e}", flush=True)
    return exc
