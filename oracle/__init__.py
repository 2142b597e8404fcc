"""CPU oracle for the compressed-KV decode path -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, the smoke check and the benchmark's CPU-baseline leg use
this package.  The product library never imports, links or calls it, and
it shares no code with the GPU path: the C source ``kvq_oracle.c`` is a
plain, single-threaded implementation of the definitions (see its header
comment for the pages each step follows).

This module wraps the C library with numpy-friendly helpers.  ``build()``
compiles it with gcc (``-ffp-contract=off``, no fast-math).
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess
from typing import Dict, Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "kvq_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile ``liboracle.so`` next to this file; returns its path."""
    if force or not os.path.exists(_LIB):
        cmd = ["gcc", "-std=c11", "-O2", "-ffp-contract=off", "-fno-fast-math",
               "-Wall", "-Wextra", "-fPIC", "-shared", _SRC, "-o", _LIB + ".tmp", "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(_LIB + ".tmp", _LIB)
    return _LIB


class _Cfg(C.Structure):
    _fields_ = [("num_layers", C.c_int32), ("batch", C.c_int32),
                ("num_q_heads", C.c_int32), ("num_kv_heads", C.c_int32),
                ("head_dim", C.c_int32), ("group_size", C.c_int32),
                ("capacity", C.POINTER(C.c_int32)), ("vis_begin", C.POINTER(C.c_int32)),
                ("vis_end", C.POINTER(C.c_int32)), ("k_bits", C.POINTER(C.c_uint8)),
                ("v_bits", C.POINTER(C.c_uint8)), ("rotate_k", C.c_int32),
                ("k_per_channel", C.c_int32),
                ("bf16_range_offsets", C.POINTER(C.c_int32)),
                ("bf16_range_begin", C.POINTER(C.c_int32)),
                ("bf16_range_end", C.POINTER(C.c_int32))]


class _Info(C.Structure):
    _fields_ = [(n, C.c_uint64) for n in (
        "total_bytes", "payload_bytes", "code_bytes", "meta_bytes",
        "bf16_visual_bytes", "bf16_text_bytes", "quantized_values", "stored_values")]


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        L = C.CDLL(_LIB)
        P = C.c_void_p
        L.orc_f16_round_down.restype = C.c_uint16
        L.orc_f16_round_down.argtypes = [C.c_float]
        L.orc_f16_round_up.restype = C.c_uint16
        L.orc_f16_round_up.argtypes = [C.c_float]
        L.orc_f16_value.restype = C.c_double
        L.orc_f16_value.argtypes = [C.c_uint16]
        L.orc_bf16_round_nearest_even.restype = C.c_uint16
        L.orc_bf16_round_nearest_even.argtypes = [C.c_float]
        L.orc_bf16_value.restype = C.c_double
        L.orc_bf16_value.argtypes = [C.c_uint16]
        L.orc_round_half_even.restype = C.c_double
        L.orc_round_half_even.argtypes = [C.c_double]
        L.orc_quantize_group.restype = None
        L.orc_quantize_group.argtypes = [P, C.c_int, C.c_int, P, P, P]
        L.orc_validate.argtypes = [C.POINTER(_Cfg)]
        L.orc_cache_bytes.argtypes = [C.POINTER(_Cfg), C.POINTER(_Info)]
        L.orc_plane_offsets.argtypes = [C.POINTER(_Cfg), C.c_int, C.c_int, C.c_int,
                                        C.POINTER(C.c_uint64), C.POINTER(C.c_uint64),
                                        C.POINTER(C.c_uint64)]
        L.orc_row_of.argtypes = [C.POINTER(_Cfg), C.c_int, C.c_int, C.POINTER(C.c_int),
                                 C.POINTER(C.c_int64)]
        L.orc_coded_end.argtypes = [C.POINTER(_Cfg), C.c_int]
        L.orc_is_coded.argtypes = [C.POINTER(_Cfg), C.c_int, C.c_int]
        L.orc_store_rows.argtypes = [C.POINTER(_Cfg), P, C.c_int, C.c_int, C.c_int,
                                     C.c_int, C.c_int, C.c_int, P]
        L.orc_load_row.argtypes = [C.POINTER(_Cfg), P, C.c_int, C.c_int, C.c_int,
                                   C.c_int, C.c_int, P]
        L.orc_load_row_stored.argtypes = [C.POINTER(_Cfg), P, C.c_int, C.c_int, C.c_int,
                                          C.c_int, C.c_int, P]
        L.orc_hadamard_rotate.restype = None
        L.orc_hadamard_rotate.argtypes = [P, C.c_int]
        L.orc_hadamard_unrotate.restype = None
        L.orc_hadamard_unrotate.argtypes = [P, C.c_int]
        L.orc_attention.restype = None
        L.orc_attention.argtypes = [P, P, P, C.c_int, C.c_int, C.c_double, P, P]
        L.orc_decode_one.argtypes = [C.POINTER(_Cfg), P, C.c_int, C.c_int, C.c_int,
                                     C.c_int, P, C.c_float, P, P, P]
        L.orc_decode_all.argtypes = [C.POINTER(_Cfg), P, C.c_int, C.c_int, P, P,
                                     C.c_float, P]
        L.orc_kl_logits.restype = C.c_double
        L.orc_kl_logits.argtypes = [P, P, C.c_int]
        _lib = L
    return _lib


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(C.c_void_p)


class Config:
    """Holds a C config plus the numpy arrays it points into."""

    def __init__(self, num_layers, batch, num_q_heads, num_kv_heads, head_dim,
                 group_size, capacity, vis_begin, vis_end, k_bits, v_bits, rotate_k=False,
                 k_per_channel=False, bf16_ranges=None):
        """bf16_ranges: None, or one list of (begin, end) position pairs per
        sequence (ranges inside the visual span stored bf16)."""
        self.capacity = np.ascontiguousarray(capacity, dtype=np.int32)
        self.vis_begin = np.ascontiguousarray(vis_begin, dtype=np.int32)
        self.vis_end = np.ascontiguousarray(vis_end, dtype=np.int32)
        self.k_bits = np.ascontiguousarray(k_bits, dtype=np.uint8)
        self.v_bits = np.ascontiguousarray(v_bits, dtype=np.uint8)
        if bf16_ranges is not None:
            offs = np.cumsum([0] + [len(r) for r in bf16_ranges]).astype(np.int32)
            flat = [p for r in bf16_ranges for p in r]
            self.rng_off = np.ascontiguousarray(offs)
            self.rng_b = np.ascontiguousarray([p[0] for p in flat] or [0], dtype=np.int32)
            self.rng_e = np.ascontiguousarray([p[1] for p in flat] or [0], dtype=np.int32)
            ptrs = [a.ctypes.data_as(C.POINTER(C.c_int32))
                    for a in (self.rng_off, self.rng_b, self.rng_e)]
        else:
            ptrs = [C.POINTER(C.c_int32)()] * 3
        self.c = _Cfg(num_layers, batch, num_q_heads, num_kv_heads, head_dim, group_size,
                      self.capacity.ctypes.data_as(C.POINTER(C.c_int32)),
                      self.vis_begin.ctypes.data_as(C.POINTER(C.c_int32)),
                      self.vis_end.ctypes.data_as(C.POINTER(C.c_int32)),
                      self.k_bits.ctypes.data_as(C.POINTER(C.c_uint8)),
                      self.v_bits.ctypes.data_as(C.POINTER(C.c_uint8)), int(bool(rotate_k)),
                      int(bool(k_per_channel)), *ptrs)

    @classmethod
    def from_workload(cls, w) -> "Config":
        a = w.config_arrays()
        return cls(w.num_layers, w.batch, w.num_q_heads, w.num_kv_heads, w.head_dim,
                   w.group_size, a["capacity"], a["vis_begin"], a["vis_end"],
                   a["k_bits"], a["v_bits"], getattr(w, "rotate_k", False),
                   getattr(w, "k_per_channel", False), getattr(w, "bf16_ranges", None))

    @property
    def ref(self):
        return C.byref(self.c)


# ---- scalar helpers -------------------------------------------------------

def f16_round_down(x: float) -> int:
    return int(lib().orc_f16_round_down(float(x)))


def f16_round_up(x: float) -> int:
    return int(lib().orc_f16_round_up(float(x)))


def f16_value(h: int) -> float:
    return float(lib().orc_f16_value(int(h)))


def bf16_round(x: float) -> int:
    return int(lib().orc_bf16_round_nearest_even(float(x)))


def bf16_value(b: int) -> float:
    return float(lib().orc_bf16_value(int(b)))


def round_half_even(v: float) -> float:
    return float(lib().orc_round_half_even(float(v)))


def quantize_group(x: np.ndarray, bits: int):
    """-> (codes uint8 [g], scale16 bits, min16 bits)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    codes = np.zeros(x.size, dtype=np.uint8)
    s = np.zeros(1, dtype=np.uint16)
    m = np.zeros(1, dtype=np.uint16)
    lib().orc_quantize_group(_ptr(x), x.size, bits, _ptr(codes), _ptr(s), _ptr(m))
    return codes, int(s[0]), int(m[0])


# ---- layout ------------------------------------------------------------------

def cache_info(cfg: Config) -> Dict[str, int]:
    info = _Info()
    rc = lib().orc_cache_bytes(cfg.ref, C.byref(info))
    if rc:
        raise ValueError(f"invalid config (oracle code {rc})")
    return {n: int(getattr(info, n)) for n, _ in _Info._fields_}


def plane_offsets(cfg: Config, layer: int, head: int, X: int):
    v, m, t = C.c_uint64(), C.c_uint64(), C.c_uint64()
    rc = lib().orc_plane_offsets(cfg.ref, layer, head, X, C.byref(v), C.byref(m),
                                 C.byref(t))
    if rc:
        raise ValueError(rc)
    return int(v.value), int(m.value), int(t.value)


def coded_end(cfg: Config, seq: int) -> int:
    """End of the coded part of the visual span (see kvq_oracle.h)."""
    return int(lib().orc_coded_end(cfg.ref, seq))


def is_coded(cfg: Config, seq: int, t: int) -> bool:
    return bool(lib().orc_is_coded(cfg.ref, seq, t))


def row_of(cfg: Config, seq: int, t: int):
    p, r = C.c_int(), C.c_int64()
    if lib().orc_row_of(cfg.ref, seq, t, C.byref(p), C.byref(r)):
        raise ValueError("position out of range")
    return int(p.value), int(r.value)


# ---- store / load -------------------------------------------------------------

def store_rows(cfg: Config, cache: np.ndarray, layer: int, seq: int, head: int, X: int,
               t0: int, t1: int, src_f32: np.ndarray) -> None:
    src = np.ascontiguousarray(src_f32, dtype=np.float32)
    assert src.shape == (t1 - t0, cfg.c.head_dim)
    rc = lib().orc_store_rows(cfg.ref, _ptr(cache), layer, seq, head, X, t0, t1, _ptr(src))
    if rc:
        raise ValueError(f"store_rows failed ({rc})")


def load_row(cfg: Config, cache: np.ndarray, layer: int, seq: int, head: int, X: int,
             t: int) -> np.ndarray:
    out = np.zeros(cfg.c.head_dim, dtype=np.float64)
    if lib().orc_load_row(cfg.ref, _ptr(cache), layer, seq, head, X, t, _ptr(out)):
        raise ValueError("load_row failed")
    return out


def load_row_stored(cfg: Config, cache: np.ndarray, layer: int, seq: int, head: int, X: int,
                    t: int) -> np.ndarray:
    """The row's dequantised values as stored (rotated domain for rotated K rows)."""
    out = np.zeros(cfg.c.head_dim, dtype=np.float64)
    if lib().orc_load_row_stored(cfg.ref, _ptr(cache), layer, seq, head, X, t, _ptr(out)):
        raise ValueError("load_row_stored failed")
    return out


def hadamard_rotate(x: np.ndarray) -> np.ndarray:
    """Forward Walsh-Hadamard rotation of one row in binary32 (see kvq_oracle.h)."""
    y = np.ascontiguousarray(x, dtype=np.float32).copy()
    lib().orc_hadamard_rotate(_ptr(y), y.size)
    return y


def hadamard_unrotate(y: np.ndarray) -> np.ndarray:
    """Inverse rotation of one row in binary64."""
    x = np.ascontiguousarray(y, dtype=np.float64).copy()
    lib().orc_hadamard_unrotate(_ptr(x), x.size)
    return x


def new_cache(cfg: Config) -> np.ndarray:
    return np.zeros(cache_info(cfg)["total_bytes"], dtype=np.uint8)


def _as_f32(rows: np.ndarray) -> np.ndarray:
    if rows.dtype == np.uint16:  # bf16 bit patterns -> exact float32
        return (rows.astype(np.uint32) << np.uint32(16)).view(np.float32)
    return np.ascontiguousarray(rows, dtype=np.float32)


def build_cache(w, cfg: Optional[Config] = None, layers: Optional[Sequence[int]] = None,
                cache: Optional[np.ndarray] = None) -> np.ndarray:
    """Quantise/store every position of every sequence of workload ``w``."""
    cfg = cfg or Config.from_workload(w)
    if cache is None:
        cache = new_cache(cfg)
    for l in (range(w.num_layers) if layers is None else layers):
        for s in range(w.batch):
            T = w.capacity[s]
            for h in range(w.num_kv_heads):
                store_rows(cfg, cache, l, s, h, 0, 0, T, _as_f32(w.k_rows(l, s, h, 0, T)))
                store_rows(cfg, cache, l, s, h, 1, 0, T, _as_f32(w.v_rows(l, s, h, 0, T)))
    return cache


# ---- attention ---------------------------------------------------------------

def attention(q: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float):
    q = np.ascontiguousarray(q, dtype=np.float64)
    K = np.ascontiguousarray(K, dtype=np.float64)
    V = np.ascontiguousarray(V, dtype=np.float64)
    T, D = K.shape
    out = np.zeros(D, dtype=np.float64)
    lse = np.zeros(1, dtype=np.float64)
    lib().orc_attention(_ptr(q), _ptr(K), _ptr(V), T, D, float(scale), _ptr(out), _ptr(lse))
    return out, float(lse[0])


def decode_one(cfg: Config, cache: np.ndarray, layer: int, seq: int, qhead: int,
               length: int, q_bits: np.ndarray, sm_scale: float, want_scores=False):
    D = cfg.c.head_dim
    q = np.ascontiguousarray(q_bits, dtype=np.uint16)
    out = np.zeros(D, dtype=np.float64)
    lse = np.zeros(1, dtype=np.float64)
    sc = np.zeros(length, dtype=np.float64) if want_scores else None
    rc = lib().orc_decode_one(cfg.ref, _ptr(cache), layer, seq, qhead, length, _ptr(q),
                              float(sm_scale), _ptr(out), _ptr(lse),
                              _ptr(sc) if sc is not None else None)
    if rc:
        raise ValueError(f"decode_one failed ({rc})")
    return (out, float(lse[0]), sc) if want_scores else (out, float(lse[0]))


def decode_all(cfg: Config, cache: np.ndarray, l0: int, nl: int, lens: np.ndarray,
               q_bits: np.ndarray, sm_scale: float) -> np.ndarray:
    """q_bits [nl, batch, Hq, D] bf16 bits -> out float64 [nl, batch, Hq, D]."""
    q = np.ascontiguousarray(q_bits, dtype=np.uint16)
    lens = np.ascontiguousarray(lens, dtype=np.int32)
    out = np.zeros(q.shape, dtype=np.float64)
    rc = lib().orc_decode_all(cfg.ref, _ptr(cache), l0, nl, _ptr(lens), _ptr(q),
                              float(sm_scale), _ptr(out))
    if rc:
        raise ValueError("decode_all failed")
    return out


def kl_logits(s_p: np.ndarray, s_q: np.ndarray) -> float:
    a = np.ascontiguousarray(s_p, dtype=np.float64)
    b = np.ascontiguousarray(s_q, dtype=np.float64)
    return float(lib().orc_kl_logits(_ptr(a), _ptr(b), a.size))
