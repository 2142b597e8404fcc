"""ctypes binding of libkvq (include/kvq.h), same call names as the C ABI.

Argument marshalling only: torch tensors become device pointers, the current
torch stream becomes the HIP stream, host arrays become C arrays.  Every step
of the computation runs in libkvq's HIP kernels; there is no fallback path.
If ``libkvq.so`` has not been built the first call raises.
"""
from __future__ import annotations

import ctypes as C
import os
from typing import Dict, Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libkvq.so")

KVQ_OK = 0
KVQ_ERR_NULL = 1
KVQ_ERR_SHAPE = 2
KVQ_ERR_UNSUPPORTED = 3
KVQ_ERR_RANGE = 4
KVQ_ERR_WORKSPACE = 5
KVQ_ERR_ALIGN = 6
KVQ_ERR_HIP = 7
KVQ_ERR_INTERNAL = 8
KVQ_SRC_F32 = 0
KVQ_SRC_BF16 = 1

EXPORTS = ("kvq_cache_bytes", "kvq_quantize", "kvq_quantize_ragged", "kvq_decode_attention",
           "kvq_decode_attention_append", "kvq_decode_attention_noalloc",
           "kvq_latent_cache_bytes", "kvq_latent_store",
           "kvq_latent_decode", "kvq_status_string")


class KvqError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_string(status)} (status {status})")


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


class _LatentCfg(C.Structure):
    _fields_ = [("num_layers", C.c_int32), ("batch", C.c_int32),
                ("num_q_heads", C.c_int32), ("num_kv_heads", C.c_int32),
                ("head_dim", C.c_int32), ("rank", C.c_int32),
                ("capacity", C.POINTER(C.c_int32))]


class _Info(C.Structure):
    _fields_ = [(n, C.c_uint64) for n in (
        "total_bytes", "payload_bytes", "code_bytes", "meta_bytes",
        "bf16_visual_bytes", "bf16_text_bytes", "quantized_values", "stored_values")]


_lib = None


def lib(path: str = LIB_PATH):
    """Load libkvq.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(path):
            raise RuntimeError(f"libkvq.so not found at {path}; build it with "
                               "`python -m quantized_decode_attention_quantize_amd.build`")
        L = C.CDLL(path)
        P = C.c_void_p
        L.kvq_cache_bytes.restype = C.c_int
        L.kvq_cache_bytes.argtypes = [C.POINTER(_Cfg), C.POINTER(_Info)]
        L.kvq_quantize.restype = C.c_int
        L.kvq_quantize.argtypes = [C.POINTER(_Cfg), P, C.c_int32, C.c_int32, C.c_int32,
                                   C.POINTER(C.c_int32), C.c_int32, C.c_int32, P, P,
                                   C.c_int, P]
        L.kvq_quantize_ragged.restype = C.c_int
        L.kvq_quantize_ragged.argtypes = [C.POINTER(_Cfg), P, C.c_int32, C.c_int32, C.c_int32,
                                          C.POINTER(C.c_int32), C.POINTER(C.c_int32),
                                          C.c_int32, P, P, C.c_int, P]
        L.kvq_decode_attention.restype = C.c_int
        L.kvq_decode_attention.argtypes = [C.POINTER(_Cfg), P, C.c_int32, C.c_int32, P, P, P,
                                           C.c_float, C.c_int32, P, C.POINTER(C.c_size_t), P]
        L.kvq_decode_attention_noalloc.restype = C.c_int
        L.kvq_decode_attention_noalloc.argtypes = [C.POINTER(_Cfg), P, C.c_int32, C.c_int32, P,
                                                   P, P, C.c_float, C.c_int32, P]
        L.kvq_decode_attention_append.restype = C.c_int
        L.kvq_decode_attention_append.argtypes = [C.POINTER(_Cfg), P, C.c_int32, C.c_int32, P,
                                                  P, P, C.c_int, P, P, C.c_float, C.c_int32,
                                                  P, C.POINTER(C.c_size_t), P]
        L.kvq_latent_cache_bytes.restype = C.c_int
        L.kvq_latent_cache_bytes.argtypes = [C.POINTER(_LatentCfg), C.POINTER(C.c_uint64)]
        L.kvq_latent_store.restype = C.c_int
        L.kvq_latent_store.argtypes = [C.POINTER(_LatentCfg), P, C.c_int32, C.c_int32, C.c_int32,
                                       C.POINTER(C.c_int32), C.c_int32, C.c_int32, P, P, P]
        L.kvq_latent_decode.restype = C.c_int
        L.kvq_latent_decode.argtypes = [C.POINTER(_LatentCfg), P, C.c_int32, C.c_int32, P, P, P,
                                        P, P, C.c_float, C.c_int32, P, C.POINTER(C.c_size_t), P]
        L.kvq_status_string.restype = C.c_char_p
        L.kvq_status_string.argtypes = [C.c_int]
        _lib = L
    return _lib


def status_string(status: int) -> str:
    return lib().kvq_status_string(int(status)).decode()


class Config:
    """A kvq_config plus the host arrays it points into."""

    def __init__(self, num_layers: int, batch: int, num_q_heads: int, num_kv_heads: int,
                 head_dim: int, group_size: int, capacity, vis_begin, vis_end, k_bits, v_bits,
                 rotate_k: bool = False, k_per_channel: bool = False, bf16_ranges=None):
        """bf16_ranges: None, or per sequence a list of (begin, end) position
        pairs inside its visual span whose rows are stored bf16."""
        self.capacity = np.ascontiguousarray(capacity, dtype=np.int32)
        self.vis_begin = np.ascontiguousarray(vis_begin, dtype=np.int32)
        self.vis_end = np.ascontiguousarray(vis_end, dtype=np.int32)
        self.k_bits = np.ascontiguousarray(k_bits, dtype=np.uint8)
        self.v_bits = np.ascontiguousarray(v_bits, dtype=np.uint8)
        self.num_layers, self.batch = num_layers, batch
        self.num_q_heads, self.num_kv_heads = num_q_heads, num_kv_heads
        self.head_dim, self.group_size = head_dim, group_size
        self.rotate_k = bool(rotate_k)
        self.k_per_channel = bool(k_per_channel)
        i32p = C.POINTER(C.c_int32)
        self.bf16_ranges = bf16_ranges
        if bf16_ranges is None:
            rng = (i32p(), i32p(), i32p())
        else:
            if len(bf16_ranges) != batch:
                raise ValueError(f"bf16_ranges needs one list per sequence ({batch})")
            pairs = [(int(b), int(e)) for seq in bf16_ranges for (b, e) in seq]
            self._rng_off = np.zeros(batch + 1, dtype=np.int32)
            self._rng_off[1:] = np.cumsum([len(seq) for seq in bf16_ranges])
            # one spare element so an empty table still has an address
            self._rng_b = np.array([b for b, _ in pairs] + [0], dtype=np.int32)
            self._rng_e = np.array([e for _, e in pairs] + [0], dtype=np.int32)
            rng = tuple(x.ctypes.data_as(i32p) for x in (self._rng_off, self._rng_b, self._rng_e))
        self.c = _Cfg(num_layers, batch, num_q_heads, num_kv_heads, head_dim, group_size,
                      self.capacity.ctypes.data_as(C.POINTER(C.c_int32)),
                      self.vis_begin.ctypes.data_as(C.POINTER(C.c_int32)),
                      self.vis_end.ctypes.data_as(C.POINTER(C.c_int32)),
                      self.k_bits.ctypes.data_as(C.POINTER(C.c_uint8)),
                      self.v_bits.ctypes.data_as(C.POINTER(C.c_uint8)), int(self.rotate_k),
                      int(self.k_per_channel), *rng)

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


def _check(status: int, where: str) -> None:
    if status != KVQ_OK:
        raise KvqError(status, where)


def _dev_ptr(t, name: str):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return C.c_void_p(t.data_ptr())


def _nbytes(t) -> int:
    return t.numel() * t.element_size()


def _check_cache(cfg: "Config", cache) -> None:
    import torch
    if cache.dtype != torch.uint8:
        raise ValueError("cache must be a uint8 tensor")
    need = kvq_cache_bytes(cfg)["total_bytes"]
    if cache.numel() < need:
        raise ValueError(f"cache holds {cache.numel()} bytes, the config needs {need}")


def _check_sources(cfg: "Config", k_src, v_src, num_layers: int, num_seqs: int,
                   num_tokens: int):
    """-> the source dtype code; shapes must be [num_layers, num_seqs, Hkv, num_tokens, D]."""
    import torch
    if k_src.dtype != v_src.dtype:
        raise ValueError("k_src and v_src must share a dtype")
    if k_src.dtype == torch.bfloat16:
        dt = KVQ_SRC_BF16
    elif k_src.dtype == torch.float32:
        dt = KVQ_SRC_F32
    else:
        raise ValueError("sources must be float32 or bfloat16")
    want = (num_layers, num_seqs, cfg.num_kv_heads, num_tokens, cfg.head_dim)
    for name, t in (("k_src", k_src), ("v_src", v_src)):
        if tuple(t.shape) != want:
            raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {want}")
    return dt


def _check_decode_args(cfg: "Config", cache, num_layers: int, seq_lens, q, out) -> None:
    import torch
    _check_cache(cfg, cache)
    if seq_lens.dtype != torch.int32 or seq_lens.numel() != cfg.batch:
        raise ValueError(f"seq_lens must be int32 [{cfg.batch}]")
    want = (num_layers, cfg.batch, cfg.num_q_heads, cfg.head_dim)
    for name, t in (("q", q), ("out", out)):
        if t.dtype != torch.bfloat16 or t.numel() != int(np.prod(want)):
            raise ValueError(f"{name} must be bfloat16 with {want} elements in that layout")


def _stream(stream) -> Optional[C.c_void_p]:
    if stream is None:
        import torch
        stream = torch.cuda.current_stream()
    return C.c_void_p(stream.cuda_stream)


def kvq_cache_bytes(cfg: Config) -> Dict[str, int]:
    info = _Info()
    _check(lib().kvq_cache_bytes(cfg.ref, C.byref(info)), "kvq_cache_bytes")
    return {n: int(getattr(info, n)) for n, _ in _Info._fields_}


def kvq_quantize(cfg: Config, cache, layer_begin: int, num_layers: int,
                 seq_ids: Sequence[int], tok_begin: int, tok_end: int, k_src, v_src,
                 stream=None) -> None:
    """k_src/v_src: device float32 or bfloat16 [num_layers, len(seq_ids), Hkv, n_tok, D]."""
    ids = np.ascontiguousarray(seq_ids, dtype=np.int32)
    _check_cache(cfg, cache)
    dt = _check_sources(cfg, k_src, v_src, num_layers, len(ids), max(0, tok_end - tok_begin))
    _check(lib().kvq_quantize(cfg.ref, _dev_ptr(cache, "cache"), layer_begin, num_layers,
                              len(ids), ids.ctypes.data_as(C.POINTER(C.c_int32)),
                              tok_begin, tok_end, _dev_ptr(k_src, "k_src"),
                              _dev_ptr(v_src, "v_src"), dt, _stream(stream)), "kvq_quantize")


def kvq_quantize_ragged(cfg: Config, cache, layer_begin: int, num_layers: int,
                        seq_ids: Sequence[int], tok_begin: Sequence[int], num_tokens: int,
                        k_src, v_src, stream=None) -> None:
    """Sequence seq_ids[i] stores positions [tok_begin[i], tok_begin[i] + num_tokens);
    k_src/v_src: device float32 or bfloat16 [num_layers, len(seq_ids), Hkv, num_tokens, D]."""
    ids = np.ascontiguousarray(seq_ids, dtype=np.int32)
    t0 = np.ascontiguousarray(tok_begin, dtype=np.int32)
    if t0.shape != ids.shape:
        raise ValueError("one start position per sequence")
    _check_cache(cfg, cache)
    dt = _check_sources(cfg, k_src, v_src, num_layers, len(ids), max(0, num_tokens))
    _check(lib().kvq_quantize_ragged(cfg.ref, _dev_ptr(cache, "cache"), layer_begin, num_layers,
                                     len(ids), ids.ctypes.data_as(C.POINTER(C.c_int32)),
                                     t0.ctypes.data_as(C.POINTER(C.c_int32)), num_tokens,
                                     _dev_ptr(k_src, "k_src"), _dev_ptr(v_src, "v_src"), dt,
                                     _stream(stream)), "kvq_quantize_ragged")


def workspace_bytes(cfg: Config, num_layers: int, chunk_tokens: int = 0) -> int:
    n = C.c_size_t(0)
    _check(lib().kvq_decode_attention(cfg.ref, None, 0, num_layers, None, None, None, 1.0,
                                      chunk_tokens, None, C.byref(n), None),
           "kvq_decode_attention(size query)")
    return int(n.value)


def kvq_decode_attention(cfg: Config, cache, layer_begin: int, num_layers: int, seq_lens,
                         q, out, sm_scale: float, chunk_tokens: int = 0, workspace=None,
                         stream=None) -> None:
    """seq_lens: device int32 [batch]; q/out: device bf16 [num_layers, batch, Hq, D].
    workspace: device uint8 tensor of at least workspace_bytes(...) bytes, zero-filled
    before its first use (e.g. torch.zeros); each call leaves it ready for reuse."""
    if workspace is None:
        raise ValueError("workspace tensor required (see workspace_bytes)")
    _check_decode_args(cfg, cache, num_layers, seq_lens, q, out)
    n = C.c_size_t(_nbytes(workspace))
    _check(lib().kvq_decode_attention(cfg.ref, _dev_ptr(cache, "cache"), layer_begin,
                                      num_layers, _dev_ptr(seq_lens, "seq_lens"),
                                      _dev_ptr(q, "q"), _dev_ptr(out, "out"), float(sm_scale),
                                      chunk_tokens, _dev_ptr(workspace, "workspace"),
                                      C.byref(n), _stream(stream)), "kvq_decode_attention")


def kvq_decode_attention_append(cfg: Config, cache, layer_begin: int, num_layers: int, seq_lens,
                                k_new, v_new, q, out, sm_scale: float, chunk_tokens: int = 0,
                                workspace=None, stream=None) -> None:
    """Stores the token at position seq_lens[s] - 1 of every (layer, sequence, KV
    head) from k_new / v_new (device float32 or bfloat16 [num_layers, batch, Hkv,
    D]; a text position), then decodes as kvq_decode_attention, in one launch."""
    if workspace is None:
        raise ValueError("workspace tensor required (see workspace_bytes)")
    _check_decode_args(cfg, cache, num_layers, seq_lens, q, out)
    dt = _check_sources(cfg, k_new.reshape(num_layers, cfg.batch, cfg.num_kv_heads, 1,
                                           cfg.head_dim),
                        v_new.reshape(num_layers, cfg.batch, cfg.num_kv_heads, 1, cfg.head_dim),
                        num_layers, cfg.batch, 1)
    n = C.c_size_t(_nbytes(workspace))
    _check(lib().kvq_decode_attention_append(
        cfg.ref, _dev_ptr(cache, "cache"), layer_begin, num_layers,
        _dev_ptr(seq_lens, "seq_lens"), _dev_ptr(k_new, "k_new"), _dev_ptr(v_new, "v_new"), dt,
        _dev_ptr(q, "q"), _dev_ptr(out, "out"), float(sm_scale), chunk_tokens,
        _dev_ptr(workspace, "workspace"), C.byref(n), _stream(stream)),
        "kvq_decode_attention_append")


def kvq_decode_attention_noalloc(cfg: Config, cache, layer_begin: int, num_layers: int,
                                 seq_lens, q, out, sm_scale: float, chunk_tokens: int = 0,
                                 stream=None) -> None:
    """kvq_decode_attention with the library's own per-device scratch instead of a
    workspace (for callers that cannot allocate).  Calls that overlap in time on
    one device race; calls ordered on one stream are safe."""
    _check_decode_args(cfg, cache, num_layers, seq_lens, q, out)
    _check(lib().kvq_decode_attention_noalloc(cfg.ref, _dev_ptr(cache, "cache"), layer_begin,
                                              num_layers, _dev_ptr(seq_lens, "seq_lens"),
                                              _dev_ptr(q, "q"), _dev_ptr(out, "out"),
                                              float(sm_scale), chunk_tokens, _stream(stream)),
           "kvq_decode_attention_noalloc")


# ---- low-rank latent cache ------------------------------------------------

class LatentConfig:
    """A kvq_latent_config plus the host array it points into."""

    def __init__(self, num_layers: int, batch: int, num_q_heads: int, num_kv_heads: int,
                 head_dim: int, rank: int, capacity):
        self.capacity = np.ascontiguousarray(capacity, dtype=np.int32)
        self.num_layers, self.batch = num_layers, batch
        self.num_q_heads, self.num_kv_heads = num_q_heads, num_kv_heads
        self.head_dim, self.rank = head_dim, rank
        self.c = _LatentCfg(num_layers, batch, num_q_heads, num_kv_heads, head_dim, rank,
                            self.capacity.ctypes.data_as(C.POINTER(C.c_int32)))

    @property
    def ref(self):
        return C.byref(self.c)


def kvq_latent_cache_bytes(cfg: LatentConfig) -> int:
    n = C.c_uint64(0)
    _check(lib().kvq_latent_cache_bytes(cfg.ref, C.byref(n)), "kvq_latent_cache_bytes")
    return int(n.value)


def _check_bf16(t, name: str, shape) -> None:
    import torch
    if t.dtype != torch.bfloat16:
        raise ValueError(f"{name} must be bfloat16")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


def kvq_latent_store(cfg: LatentConfig, cache, layer_begin: int, num_layers: int,
                     seq_ids: Sequence[int], tok_begin: int, tok_end: int, k_latent, v_latent,
                     stream=None) -> None:
    """k_latent/v_latent: device bf16 [num_layers, len(seq_ids), Hkv, tok_end - tok_begin, r]."""
    import torch
    ids = np.ascontiguousarray(seq_ids, dtype=np.int32)
    if cache.dtype != torch.uint8 or cache.numel() < kvq_latent_cache_bytes(cfg):
        raise ValueError("cache must be a uint8 tensor of kvq_latent_cache_bytes bytes")
    want = (num_layers, len(ids), cfg.num_kv_heads, max(0, tok_end - tok_begin), cfg.rank)
    _check_bf16(k_latent, "k_latent", want)
    _check_bf16(v_latent, "v_latent", want)
    _check(lib().kvq_latent_store(cfg.ref, _dev_ptr(cache, "cache"), layer_begin, num_layers,
                                  len(ids), ids.ctypes.data_as(C.POINTER(C.c_int32)), tok_begin,
                                  tok_end, _dev_ptr(k_latent, "k_latent"),
                                  _dev_ptr(v_latent, "v_latent"), _stream(stream)),
           "kvq_latent_store")


def latent_workspace_bytes(cfg: LatentConfig, num_layers: int, chunk_tokens: int = 0) -> int:
    n = C.c_size_t(0)
    _check(lib().kvq_latent_decode(cfg.ref, None, 0, num_layers, None, None, None, None, None,
                                   1.0, chunk_tokens, None, C.byref(n), None),
           "kvq_latent_decode(size query)")
    return int(n.value)


def kvq_latent_decode(cfg: LatentConfig, cache, layer_begin: int, num_layers: int, seq_lens,
                      up_k, up_v, q, out, sm_scale: float, chunk_tokens: int = 0,
                      workspace=None, stream=None) -> None:
    """up_k/up_v: device bf16 [L, Hkv, r, D]; q/out: device bf16 [num_layers, B, Hq, D];
    seq_lens: device int32 [B]; workspace: device uint8 of latent_workspace_bytes(...),
    zero-filled before its first use (the calls leave it reusable)."""
    import torch
    if workspace is None:
        raise ValueError("workspace tensor required (see latent_workspace_bytes)")
    if cache.dtype != torch.uint8 or cache.numel() < kvq_latent_cache_bytes(cfg):
        raise ValueError("cache must be a uint8 tensor of kvq_latent_cache_bytes bytes")
    if seq_lens.dtype != torch.int32 or seq_lens.numel() != cfg.batch:
        raise ValueError(f"seq_lens must be int32 [{cfg.batch}]")
    up = (cfg.num_layers, cfg.num_kv_heads, cfg.rank, cfg.head_dim)
    _check_bf16(up_k, "up_k", up)
    _check_bf16(up_v, "up_v", up)
    io = (num_layers, cfg.batch, cfg.num_q_heads, cfg.head_dim)
    _check_bf16(q, "q", io)
    _check_bf16(out, "out", io)
    n = C.c_size_t(_nbytes(workspace))
    _check(lib().kvq_latent_decode(cfg.ref, _dev_ptr(cache, "cache"), layer_begin, num_layers,
                                   _dev_ptr(seq_lens, "seq_lens"), _dev_ptr(up_k, "up_k"),
                                   _dev_ptr(up_v, "up_v"), _dev_ptr(q, "q"),
                                   _dev_ptr(out, "out"), float(sm_scale), chunk_tokens,
                                   _dev_ptr(workspace, "workspace"), C.byref(n),
                                   _stream(stream)), "kvq_latent_decode")
