"""CPU oracle for low-rank latent decode -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, the smoke check and the benchmark's CPU-baseline leg use
this module; the product library never imports or calls it and shares no
code with it.  Plain numpy in float64.

What it computes follows gist.science paper 2604.02570 (WSVD), section 2:
part 가 gives every attention head its own low-rank factorisation, so the
cache of one (layer, KV head) holds latent rows c_t of width r instead of
K/V rows of width D, and K_t = c^K_t B_K, V_t = c^V_t B_V with per-head
r x D up-projections; part 라 reconstructs K and V on chip inside flash
decoding and then runs ordinary attention.  The oracle does exactly that,
written out: reconstruct every K and V row in float64, then softmax
attention over the first ``length`` positions.

The byte layout of the latent cache is this library's own (the pages fix
none); ``latent_offset`` writes it out one element at a time:

* each sequence's rows start on a multiple of 32 rows: sequence s owns rows
  [row0_s, row0_s + capacity_s) with row0_s the sum of the earlier
  capacities rounded up to 32;
* (layer, KV head, X) planes follow each other, X = 0 (K) then 1 (V), each
  ``align256(R * r * 2)`` bytes with R = the last row0 plus its capacity
  rounded up to 32;
* K and V latents are row-major bf16: element (row, j) of a plane at
  ``(row * r + j) * 2``.
"""
from __future__ import annotations

from typing import List, Sequence

import numpy as np


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> exact float64 values."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


# ---- layout --------------------------------------------------------------

def row_bases(capacity: Sequence[int]) -> List[int]:
    """First row of every sequence (each a multiple of 32), plus R at the end."""
    out, r = [], 0
    for c in capacity:
        out.append(r)
        r += -(-int(c) // 32) * 32
    out.append(r)
    return out


def plane_bytes(capacity: Sequence[int], rank: int) -> int:
    R = row_bases(capacity)[-1]
    return -(-(R * rank * 2) // 256) * 256


def cache_bytes(num_layers: int, num_kv_heads: int, capacity: Sequence[int], rank: int) -> int:
    return num_layers * num_kv_heads * 2 * plane_bytes(capacity, rank)


def latent_offset(num_kv_heads: int, capacity: Sequence[int], rank: int, layer: int,
                  head: int, X: int, seq: int, t: int, j: int) -> int:
    """Byte offset of latent element j of position t of sequence seq."""
    assert 0 <= t < capacity[seq] and 0 <= j < rank and X in (0, 1)
    plane = ((layer * num_kv_heads + head) * 2 + X) * plane_bytes(capacity, rank)
    row = row_bases(capacity)[seq] + t
    return plane + (row * rank + j) * 2


def write_rows(cache: np.ndarray, num_kv_heads: int, capacity: Sequence[int], rank: int,
               layer: int, head: int, X: int, seq: int, t0: int, bits: np.ndarray) -> None:
    """Store bf16 latent rows ``bits`` [n, rank] at positions t0 .. t0 + n - 1,
    element by element."""
    n = bits.shape[0]
    for i in range(n):
        for j in range(rank):
            o = latent_offset(num_kv_heads, capacity, rank, layer, head, X, seq, t0 + i, j)
            v = int(bits[i, j])
            cache[o] = v & 255
            cache[o + 1] = v >> 8


# ---- decode --------------------------------------------------------------

def decode_one(ck: np.ndarray, cv: np.ndarray, up_k: np.ndarray, up_v: np.ndarray,
               q: np.ndarray, length: int, sm_scale: float) -> np.ndarray:
    """One query head over one KV head's history, float64 [D].

    ck, cv: latents [>= length, r]; up_k, up_v: [r, D]; q: [D].
    K and V rows are reconstructed first (WSVD section 2 가), then the
    scores q . K_t * sm_scale go through a softmax over positions
    0 .. length - 1 and weight the V rows.  length 0 gives zeros.
    """
    if length <= 0:
        return np.zeros(up_v.shape[1])
    K = np.asarray(ck[:length], np.float64) @ np.asarray(up_k, np.float64)
    V = np.asarray(cv[:length], np.float64) @ np.asarray(up_v, np.float64)
    s = (K @ np.asarray(q, np.float64)) * float(sm_scale)
    p = np.exp(s - s.max())
    return (p / p.sum()) @ V


def decode(ck: np.ndarray, cv: np.ndarray, up_k: np.ndarray, up_v: np.ndarray,
           q: np.ndarray, lens: Sequence[int], sm_scale: float) -> np.ndarray:
    """Every (layer, sequence, query head): float64 [L, B, Hq, D].

    ck, cv: per (layer, seq, KV head) latents [L, B, Hkv, T, r];
    up_k, up_v: [L, Hkv, r, D]; q: [L, B, Hq, D].  Query head i reads KV
    head i // (Hq / Hkv) (grouped-query attention).
    """
    L, B, Hkv = ck.shape[:3]
    Hq, D = q.shape[2], q.shape[3]
    G = Hq // Hkv
    out = np.zeros((L, B, Hq, D))
    for l in range(L):
        for s in range(B):
            for i in range(Hq):
                h = i // G
                out[l, s, i] = decode_one(ck[l, s, h], cv[l, s, h], up_k[l, h], up_v[l, h],
                                          q[l, s, i], lens[s], sm_scale)
    return out
