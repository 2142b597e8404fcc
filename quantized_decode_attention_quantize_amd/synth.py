"""Seeded synthetic inputs for the compressed-KV decode path.

This module holds no part of the method: no quantizer, no layout, no
attention.  It only draws numbers.  Both the GPU path (tests, bench) and the
CPU oracle take their inputs from here, so the two see identical bits.

Randomness is counter based, so any sub-range of any tensor can be drawn on
its own without generating what comes before it:

* SplitMix64 (Steele, Lea, Flood, "Fast splittable pseudorandom number
  generators", OOPSLA 2014): value ``i`` of the stream with key ``k`` is the
  SplitMix64 finaliser applied to ``k + (i + 1) * 0x9E3779B97F4A7C15``.
* Uniforms take the top 53 bits: ``(z >> 11) * 2**-53`` in ``[0, 1)``.
* Normals use the Box-Muller transform on consecutive uniform pairs
  ``(u1, u2)``: ``r = sqrt(-2 ln(1 - u1))``, values ``r cos(2 pi u2)`` and
  ``r sin(2 pi u2)``.

The workload shapes follow the pages' setting (a LLaVA-OneVision-7B style
video VLM: 28 query / 4 KV heads, head dim 128, ~14 system-text tokens then
32 frames x ~196 = 6,273 visual tokens, K stored after RoPE, V unrotated;
nuiw.github.io "VLM_KV_Quantization", section 2) and the HeadGuard briefing
(about 1/8 of physical KV heads protected).  The values are synthetic:
no model, weights or dataset are involved.

Floating-point outputs are float32 arrays or bfloat16 *bit patterns* held in
uint16 arrays (numpy has no bfloat16); ``bf16_bits_to_f32`` widens the latter
exactly.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np

_MASK64 = (1 << 64) - 1
_GOLDEN = 0x9E3779B97F4A7C15
_M1 = 0xBF58476D1CE4E5B9
_M2 = 0x94D049BB133111EB

# Stream tags: every tensor family draws from its own keyed stream.
TAG_K = 1
TAG_V = 2
TAG_Q = 3
TAG_OUTLIER = 4
TAG_HEADS = 5
TAG_LENS = 6
TAG_APPEND_K = 7
TAG_APPEND_V = 8
TAG_BLOCK_K = 9
TAG_BLOCK_V = 10
TAG_TOKENS = 11
TAG_LATENT = 12
TAG_UP = 13


def _mix64_int(z: int) -> int:
    z &= _MASK64
    z = ((z ^ (z >> 30)) * _M1) & _MASK64
    z = ((z ^ (z >> 27)) * _M2) & _MASK64
    return z ^ (z >> 31)


def stream_key(*parts: int) -> int:
    """Fold integers into one 64-bit stream key (SplitMix64 finaliser chain)."""
    h = 0x243F6A8885A308D3  # arbitrary non-zero start
    for p in parts:
        h = _mix64_int(h ^ (int(p) & _MASK64))
        h = _mix64_int((h + _GOLDEN) & _MASK64)
    return h


def splitmix64(key: int, start: int, count: int) -> np.ndarray:
    """Values ``start .. start+count-1`` of the SplitMix64 stream ``key``."""
    idx = np.arange(start + 1, start + 1 + count, dtype=np.uint64)
    with np.errstate(over="ignore"):
        z = np.uint64(key) + idx * np.uint64(_GOLDEN)
        z = (z ^ (z >> np.uint64(30))) * np.uint64(_M1)
        z = (z ^ (z >> np.uint64(27))) * np.uint64(_M2)
    return z ^ (z >> np.uint64(31))


def uniform(key: int, start: int, count: int) -> np.ndarray:
    """Uniform float64 in [0, 1) with 53 random bits."""
    z = splitmix64(key, start, count)
    return (z >> np.uint64(11)).astype(np.float64) * (2.0 ** -53)


def normal(key: int, start: int, count: int) -> np.ndarray:
    """Standard normals ``start .. start+count-1`` of stream ``key`` (fp64).

    Normal ``i`` comes from uniform pair ``i // 2``; even ``i`` take the
    cosine branch, odd ``i`` the sine branch.
    """
    if count <= 0:
        return np.zeros(0, dtype=np.float64)
    p0 = start // 2
    p1 = (start + count - 1) // 2 + 1
    u = uniform(key, 2 * p0, 2 * (p1 - p0)).reshape(-1, 2)
    r = np.sqrt(-2.0 * np.log1p(-u[:, 0]))
    th = 2.0 * math.pi * u[:, 1]
    z = np.empty(2 * (p1 - p0), dtype=np.float64)
    z[0::2] = r * np.cos(th)
    z[1::2] = r * np.sin(th)
    off = start - 2 * p0
    return z[off:off + count]


def permutation_prefix(key: int, n: int, k: int) -> np.ndarray:
    """First ``k`` entries of a Fisher-Yates shuffle of ``0..n-1``."""
    perm = np.arange(n, dtype=np.int64)
    u = uniform(key, 0, k)
    for i in range(k):
        j = i + int(u[i] * (n - i))
        perm[i], perm[j] = perm[j], perm[i]
    return perm[:k].copy()


def uniform_ints(key: int, lo: int, hi: int, count: int) -> np.ndarray:
    """Integers uniform in the closed range [lo, hi]."""
    u = uniform(key, 0, count)
    return (lo + np.floor(u * (hi - lo + 1))).astype(np.int64)


# ---------------------------------------------------------------------------
# dtype helpers (input preparation only)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns, round to nearest even (finite input)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (u + np.uint64(0x7FFF) + ((u >> np.uint64(16)) & np.uint64(1))) >> np.uint64(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns -> float32 (exact)."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _to_src(x64: np.ndarray, src: str) -> np.ndarray:
    x32 = x64.astype(np.float32)
    if src == "f32":
        return x32
    if src == "bf16":
        return f32_to_bf16_bits(x32)
    raise ValueError(src)


# ---------------------------------------------------------------------------
# workloads


@dataclass
class Workload:
    """One synthetic decode workload (shapes, formats and value recipe).

    Each sequence's history is ``[text prefix][visual span][text suffix]``:
    positions ``[vis_begin, vis_end)`` are visual, everything else is text.
    ``k_bits``/``v_bits`` give the storage format per (layer, KV head); 16 is
    bfloat16 (a protected head), 2/4/8 are integer codes.
    """

    name: str
    num_layers: int
    batch: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    group_size: int
    seq_lens: List[int]
    vis_begin: List[int]
    vis_end: List[int]
    capacity: List[int]
    k_bits: np.ndarray  # uint8 [num_layers * num_kv_heads]
    v_bits: np.ndarray
    src: str = "bf16"  # source dtype of K/V rows: "f32" or "bf16"
    rope: bool = True
    rope_base: float = 1.0e6
    outliers: int = 4
    outlier_scale: float = 8.0
    k_std: float = 1.0
    v_std: float = 1.0
    seed: int = 0
    protected: Optional[np.ndarray] = None  # flat (layer*Hkv + head) ids kept bf16
    rotate_k: bool = False  # coded K rows stored Walsh-Hadamard rotated
    k_per_channel: bool = False  # K codes grouped per channel over token blocks
    # per sequence, (begin, end) ranges inside the visual span stored bf16
    # (protected tokens, or text between two images); None: none
    bf16_ranges: Optional[List[List[Tuple[int, int]]]] = None

    @property
    def group_ratio(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    @property
    def sm_scale(self) -> float:
        """Softmax scale 1/sqrt(D) rounded to float32 (passed as fp32)."""
        return float(np.float32(1.0 / math.sqrt(self.head_dim)))

    # --- value recipe -----------------------------------------------------
    def outlier_channels(self, layer: int, seq: int, head: int) -> np.ndarray:
        if not self.rope or self.outliers <= 0:
            return np.zeros(0, dtype=np.int64)
        key = stream_key(self.seed, TAG_OUTLIER, layer, seq, head)
        return permutation_prefix(key, self.head_dim, self.outliers)

    def _rotate(self, x: np.ndarray, t0: int) -> np.ndarray:
        """Rotate-half RoPE on rows at absolute positions t0, t0+1, ..."""
        D = self.head_dim
        half = D // 2
        i = np.arange(half, dtype=np.float64)
        inv = np.power(self.rope_base, -2.0 * i / D)
        pos = np.arange(t0, t0 + x.shape[0], dtype=np.float64)
        ang = pos[:, None] * inv[None, :]
        c, s = np.cos(ang), np.sin(ang)
        a, b = x[:, :half], x[:, half:]
        return np.concatenate([a * c - b * s, a * s + b * c], axis=1)

    def k_rows64(self, layer: int, seq: int, head: int, t0: int, t1: int,
                 tag: int = TAG_K) -> np.ndarray:
        D = self.head_dim
        key = stream_key(self.seed, tag, layer, seq, head)
        x = normal(key, t0 * D, (t1 - t0) * D).reshape(t1 - t0, D) * self.k_std
        ch = self.outlier_channels(layer, seq, head)
        if ch.size:
            x[:, ch] *= self.outlier_scale
        if self.rope:
            x = self._rotate(x, t0)
        return x

    def v_rows64(self, layer: int, seq: int, head: int, t0: int, t1: int,
                 tag: int = TAG_V) -> np.ndarray:
        D = self.head_dim
        key = stream_key(self.seed, tag, layer, seq, head)
        return normal(key, t0 * D, (t1 - t0) * D).reshape(t1 - t0, D) * self.v_std

    def k_rows(self, layer, seq, head, t0, t1, tag=TAG_K):
        """K source rows in the source dtype (float32, or bf16 bits)."""
        return _to_src(self.k_rows64(layer, seq, head, t0, t1, tag), self.src)

    def v_rows(self, layer, seq, head, t0, t1, tag=TAG_V):
        return _to_src(self.v_rows64(layer, seq, head, t0, t1, tag), self.src)

    def q_bits(self, layer: int) -> np.ndarray:
        """Query for one layer: bf16 bits [batch, Hq, D], N(0,1)."""
        key = stream_key(self.seed, TAG_Q, layer)
        n = self.batch * self.num_q_heads * self.head_dim
        q = normal(key, 0, n).reshape(self.batch, self.num_q_heads, self.head_dim)
        return f32_to_bf16_bits(q.astype(np.float32))

    def sources(self, layer: int, seqs: Sequence[int], t0: int, t1: int,
                which: str = "k", tag: Optional[int] = None) -> np.ndarray:
        """Stacked source rows [len(seqs), Hkv, t1-t0, D] for one layer."""
        fn = self.k_rows if which == "k" else self.v_rows
        tg = tag if tag is not None else (TAG_K if which == "k" else TAG_V)
        return np.stack([np.stack([fn(layer, s, h, t0, t1, tg)
                                   for h in range(self.num_kv_heads)])
                         for s in seqs])

    def config_arrays(self) -> Dict[str, np.ndarray]:
        return dict(
            capacity=np.asarray(self.capacity, dtype=np.int32),
            vis_begin=np.asarray(self.vis_begin, dtype=np.int32),
            vis_end=np.asarray(self.vis_end, dtype=np.int32),
            k_bits=np.asarray(self.k_bits, dtype=np.uint8),
            v_bits=np.asarray(self.v_bits, dtype=np.uint8),
        )


def _bits_table(L: int, H: int, kb: int, vb: int) -> Tuple[np.ndarray, np.ndarray]:
    return (np.full(L * H, kb, dtype=np.uint8), np.full(L * H, vb, dtype=np.uint8))


def protected_heads(seed: int, num_heads_total: int, count: int) -> np.ndarray:
    """Seeded choice of protected physical heads (Fisher-Yates prefix)."""
    key = stream_key(seed, TAG_HEADS, num_heads_total, count)
    return np.sort(permutation_prefix(key, num_heads_total, count))


def ragged_lengths(seed: int, batch: int, lo: int, hi: int) -> np.ndarray:
    return uniform_ints(stream_key(seed, TAG_LENS, batch, lo, hi), lo, hi, batch)


def tiny(seed: int = 0) -> Workload:
    """Tiny reference case: 1 layer, GQA 4:1, D=64, 16 text + 240 visual.

    fp32 N(0,1) K and V without RoPE, INT4 with group 32 along D.
    """
    kb, vb = _bits_table(1, 1, 4, 4)
    return Workload("tiny", 1, 1, 4, 1, 64, 32, [256], [16], [256], [256], kb, vb,
                    src="f32", rope=False, outliers=0, seed=seed)


def llava_layer(seed: int = 1, kbits: int = 4, vbits: int = 4) -> Workload:
    """One LLaVA-OneVision-7B shaped layer: 28/4 heads, D=128, 14 + 6,273 tokens."""
    T = 14 + 6273
    kb, vb = _bits_table(1, 4, kbits, vbits)
    return Workload("llava_layer", 1, 1, 28, 4, 128, 64, [T], [14], [T], [T], kb, vb,
                    seed=seed)


def headguard_step(seed: int = 2, num_protected: int = 14, extra_capacity: int = 0
                   ) -> Workload:
    """Full 28-layer decode step with HeadGuard protection.

    112 physical heads; ``num_protected`` seeded heads keep visual K and V in
    bf16, the others store visual K INT4 / visual V INT2, group 64.
    """
    L, H = 28, 4
    T = 14 + 6273
    prot = protected_heads(seed, L * H, num_protected)
    kb = np.full(L * H, 4, dtype=np.uint8)
    vb = np.full(L * H, 2, dtype=np.uint8)
    kb[prot] = 16
    vb[prot] = 16
    cap = T + extra_capacity
    return Workload("headguard_step", L, 1, 28, 4, 128, 64, [T], [14], [T], [cap],
                    kb, vb, seed=seed, protected=prot)


def long_gqa(seed: int = 3, T: int = 32768) -> Workload:
    """Long-context GQA: B=4, 32/8 heads, D=128, 64 text + rest visual, K4/V2."""
    kb, vb = _bits_table(1, 8, 4, 2)
    B = 4
    return Workload("long_gqa", 1, B, 32, 8, 128, 64, [T] * B, [64] * B, [T] * B,
                    [T] * B, kb, vb, v_std=0.5, seed=seed)


def ragged_serving(seed: int = 4, batch: int = 64, lo: int = 1024, hi: int = 16384
                   ) -> Workload:
    """Batched serving: ragged lengths in [lo, hi], 14 text + rest visual, K8/V4."""
    lens = [int(x) for x in ragged_lengths(seed, batch, lo, hi)]
    kb, vb = _bits_table(1, 4, 8, 4)
    return Workload("ragged_serving", 1, batch, 28, 4, 128, 64, lens, [14] * batch,
                    lens, lens, kb, vb, seed=seed)


def visual_block(seed: int = 4, num_seqs: int = 8, n_vis: int = 6273) -> Workload:
    """Quantize-path workload: ``num_seqs`` sequences receive a fresh visual
    block of ``n_vis`` tokens (bf16 in), K INT8 / V INT4, group 64."""
    T = 14 + n_vis
    kb, vb = _bits_table(1, 4, 8, 4)
    return Workload("visual_block", 1, num_seqs, 28, 4, 128, 64, [T] * num_seqs,
                    [14] * num_seqs, [T] * num_seqs, [T] * num_seqs, kb, vb, seed=seed)


def protected_tokens(seed: int, vb: int, ve: int, count: int) -> List[Tuple[int, int]]:
    """Seeded one-token ranges: the span's first token (an attention sink)
    and ``count - 1`` further distinct positions of [vb, ve)."""
    if ve <= vb or count <= 0:
        return []
    picks = permutation_prefix(stream_key(seed, TAG_TOKENS, vb, ve, count), ve - vb - 1,
                               min(count - 1, ve - vb - 1)) + vb + 1
    return [(int(t), int(t) + 1) for t in sorted({vb, *picks.tolist()})]


def two_images(seed: int = 5, tokens_protected: int = 8) -> Workload:
    """LLaVA-OneVision-7B shaped layer whose prompt holds two images:
    14 text + 3,136 visual + 32 text + 3,136 visual + 14 text tokens.  The
    text between the images is a bf16 range of one visual span, and
    ``tokens_protected`` seeded visual tokens (the first one a sink) are kept
    bf16 too.  K INT4 / V INT2, group 64."""
    n1 = n2 = 3136
    vb, mid = 14, 14 + n1
    ve = mid + 32 + n2
    T = ve + 14
    kb, vbits = _bits_table(1, 4, 4, 2)
    singles = protected_tokens(seed, vb, ve, tokens_protected)
    ranges = sorted([r for r in singles if not (mid <= r[0] < mid + 32)] + [(mid, mid + 32)])
    return Workload("two_images", 1, 1, 28, 4, 128, 64, [T], [vb], [ve], [T], kb, vbits,
                    seed=seed, bf16_ranges=[ranges])


@dataclass
class LatentWorkload:
    """Synthetic low-rank latent decode workload.

    Per (layer, KV head): latent rows c^K_t, c^V_t of width ``rank`` ~ N(0, 1)
    and up-projections B_K, B_V [rank, D] ~ N(0, 1/rank), so reconstructed
    K and V rows have unit variance per element like the quantised
    workloads' sources; queries N(0, 1).  Everything is bf16.
    """

    name: str
    num_layers: int
    batch: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    rank: int
    capacity: List[int]
    seq_lens: List[int]
    seed: int = 0

    @property
    def group_ratio(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    @property
    def sm_scale(self) -> float:
        return float(np.float32(1.0 / math.sqrt(self.head_dim)))

    def latents(self, layer: int, seq: int, head: int, X: int, t0: int, t1: int) -> np.ndarray:
        """bf16 bits [t1 - t0, rank] of K (X = 0) or V (X = 1) latents."""
        key = stream_key(self.seed, TAG_LATENT, layer, seq, head, X)
        x = normal(key, t0 * self.rank, (t1 - t0) * self.rank).reshape(t1 - t0, self.rank)
        return f32_to_bf16_bits(x.astype(np.float32))

    def up(self, layer: int, head: int, X: int) -> np.ndarray:
        """bf16 bits [rank, D] of B_K (X = 0) or B_V (X = 1)."""
        key = stream_key(self.seed, TAG_UP, layer, head, X)
        x = normal(key, 0, self.rank * self.head_dim).reshape(self.rank, self.head_dim)
        return f32_to_bf16_bits((x / math.sqrt(self.rank)).astype(np.float32))

    def q_bits(self, layer: int) -> np.ndarray:
        key = stream_key(self.seed, TAG_Q, layer, 1)
        n = self.batch * self.num_q_heads * self.head_dim
        q = normal(key, 0, n).reshape(self.batch, self.num_q_heads, self.head_dim)
        return f32_to_bf16_bits(q.astype(np.float32))


def llava_latent(seed: int = 6, rank: int = 96, num_layers: int = 28) -> LatentWorkload:
    """A LLaVA-OneVision-7B-shaped decode step over a per-head latent cache:
    28 layers x 4 KV heads (28 query heads, D = 128), 6,288 cached tokens.
    Rank 96: WSVD section 4 reports models keeping 70 % of their parameters
    (rho1); one r x (E + D) factor pair of a 3584 x 128 head projection keeps
    r * 3712 / (3584 * 128) of it, 78 % at r = 96, the smallest multiple of 32
    at or above 70 %."""
    T = 14 + 6273 + 1
    return LatentWorkload("llava_latent", num_layers, 1, 28, 4, 128, rank, [T], [T], seed=seed)


WORKLOADS = {
    "tiny": tiny,
    "llava_layer": llava_layer,
    "headguard_step": headguard_step,
    "long_gqa": long_gqa,
    "ragged_serving": ragged_serving,
    "visual_block": visual_block,
    "two_images": two_images,
}
