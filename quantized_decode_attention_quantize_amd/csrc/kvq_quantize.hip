// kvq_quantize.hip -- store K/V rows into the compressed cache (gfx950).
//
// Visual rows of heads narrower than 16 bits become group-wise asymmetric
// min-max codes with an fp16 (scale, min) pair per group; every other row is
// stored as bf16 (nuiw.github.io "VLM_KV_Quantization" sections 1-2: only
// the historical cache is compressed, Visual/Text and K/V separated;
// HeadGuard briefing: protected heads keep bf16).  The quantiser's exact
// arithmetic is spelled out in include/kvq.h.
//
// Mapping: one row (token) of D values is handled by D/16 consecutive lanes,
// 16 values per lane (two 16-byte bf16 loads or four for fp32).  A
// quantisation group of g values spans g/16 lanes; its min/max is a butterfly
// over those lanes.  Codes of one lane are contiguous in the packed row (16*b
// bits, 2b bytes), so each lane issues one store of 2b bytes; the first lane
// of a group writes the group's 4-byte (scale, min) pair.
#include <hip/hip_runtime.h>

#include "kvq_internal.h"

#pragma clang fp contract(off)

namespace kvq {
namespace {

__device__ inline uint16_t f16_bits(_Float16 h) { return __builtin_bit_cast(uint16_t, h); }
__device__ inline float f16_float(uint16_t b) { return (float)__builtin_bit_cast(_Float16, b); }

// One binary16 step toward -inf / +inf from a finite or infinite pattern.
__device__ inline uint16_t f16_step_down(uint16_t h) {
  if ((h & 0x7FFFu) == 0) return 0x8001u;          // +-0 -> -min subnormal
  return (h & 0x8000u) ? uint16_t(h + 1u) : uint16_t(h - 1u);
}
__device__ inline uint16_t f16_step_up(uint16_t h) {
  if ((h & 0x7FFFu) == 0) return 0x0001u;
  return (h & 0x8000u) ? uint16_t(h - 1u) : uint16_t(h + 1u);
}

// Largest binary16 <= x: convert with round-to-nearest-even (v_cvt_f16_f32,
// default MODE), step down once if that landed above x.  Zero -> +0.
__device__ inline uint16_t f16_round_down(float x) {
  uint16_t h = f16_bits((_Float16)x);
  if (f16_float(h) > x) h = f16_step_down(h);
  return (h & 0x7FFFu) ? h : uint16_t(0);
}
// Smallest binary16 >= x.
__device__ inline uint16_t f16_round_up(float x) {
  uint16_t h = f16_bits((_Float16)x);
  if (f16_float(h) < x) h = f16_step_up(h);
  return (h & 0x7FFFu) ? h : uint16_t(0);
}

__device__ inline uint16_t bf16_rne(float x) { return __builtin_bit_cast(uint16_t, (__bf16)x); }

__device__ inline float bf16_float(uint16_t b) {
  return __builtin_bit_cast(float, uint32_t(b) << 16);
}

// Value of another lane of the same row of 16 (DPP moves; every source lane
// exists): lane l ^ 1, lane l ^ 2, and lane 7 - l of each group of eight.
template <int CTRL>
__device__ inline float dpp_mov(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL,
                                                               0xF, 0xF, true));
}
__device__ inline float lane_xor1(float v) { return dpp_mov<0xB1>(v); }     // quad_perm 1,0,3,2
__device__ inline float lane_xor2(float v) { return dpp_mov<0x4E>(v); }     // quad_perm 2,3,0,1
__device__ inline float lane_mirror8(float v) { return dpp_mov<0x141>(v); }  // row_half_mirror

// Minimum / maximum over aligned groups of LANES (2, 4 or 8) lanes: pairs,
// then quads, then each quad with the mirrored one of its group of eight.
template <int LANES>
__device__ inline float group_min(float v) {
  static_assert(LANES == 2 || LANES == 4 || LANES == 8, "group lanes");
  v = fminf(v, lane_xor1(v));
  if constexpr (LANES >= 4) v = fminf(v, lane_xor2(v));
  if constexpr (LANES == 8) v = fminf(v, lane_mirror8(v));
  return v;
}
template <int LANES>
__device__ inline float group_max(float v) {
  static_assert(LANES == 2 || LANES == 4 || LANES == 8, "group lanes");
  v = fmaxf(v, lane_xor1(v));
  if constexpr (LANES >= 4) v = fmaxf(v, lane_xor2(v));
  if constexpr (LANES == 8) v = fmaxf(v, lane_mirror8(v));
  return v;
}

// Values of one row held by each lane.  The work that depends only on the
// group (its min/max reduction, the two directed fp16 roundings, the scale
// divide, the meta store, the addressing) is shared by a lane's E values, so
// a wave covers twice the values for little more than the instructions of a
// wave holding 8.
constexpr int kE = 16;

// Quantise this lane's kE values (part of a group spanning GL lanes) into
// packed codes (bit i * bits of the lane's kE * bits bits, as 32-bit words;
// bits divides 32, so no code straddles a word).  Writes (scale | min << 16)
// to meta.
constexpr int kWords = kE / 4;  // 32-bit words of an 8-bit lane chunk

// Rounded quotients c, B bits each, packed little-endian.  Every c is an
// integer in [0, 2^B - 1] (d >= 0 and d / sc <= 2^B - 1 for values inside
// the binary16 range), so the codes of one byte combine exactly in binary32
// (c0 + 2^B c1 + ...) and v_cvt_pk_u8_f32 places the byte.
template <int B>
__device__ inline void pack_codes(const float (&c)[kE], uint32_t (&packed)[kWords]) {
  constexpr int kPer = 8 / B;  // codes per byte
#pragma unroll
  for (int byte = 0; byte < kE / kPer; ++byte) {
    float v = c[kPer * byte + kPer - 1];
#pragma unroll
    for (int k = kPer - 2; k >= 0; --k) v = __builtin_fmaf(v, float(1 << B), c[kPer * byte + k]);
    packed[byte / 4] = __builtin_amdgcn_cvt_pk_u8_f32(v, byte % 4, packed[byte / 4]);
  }
}

template <int GL>
__device__ inline void quantize_lane(const float (&x)[kE], int bits, uint32_t (&packed)[kWords],
                                     uint32_t& meta) {
  float lo = x[0], hi = x[0];
#pragma unroll
  for (int i = 1; i < kE; ++i) {
    lo = fminf(lo, x[i]);
    hi = fmaxf(hi, x[i]);
  }
  lo = group_min<GL>(lo);
  hi = group_max<GL>(hi);
  const uint16_t mn16 = f16_round_down(lo);
  const float mn = f16_float(mn16);
  const float n = float((1 << bits) - 1);
  const float range = hi - mn;
  uint16_t sc16 = 0;
  // Each code is rint of the IEEE quotient fl(d / sc).  d * rcp(sc) is within
  // 1.5 * 2^-23 relative of d / sc (rcp within 1 ulp, one rounding), i.e.
  // within 2^-14 for quotients up to 255, and fl(d / sc) within 2^-16 of it:
  // unless the estimate lies within 2^-13 of a half-integer, both round to the
  // same integer.  When any lane of the wave has such a value, the whole wave
  // takes the IEEE divide for its values (a wave-uniform branch).  A
  // zero-range group keeps scale 0 and all-zero codes.
  const bool live = range != 0.0f;
  if (live) sc16 = f16_round_up(range / n);
  const float sc = f16_float(sc16);
  const float r = __builtin_amdgcn_rcpf(live ? sc : 1.0f);
  float d[kE], c[kE];
  bool near = false;
#pragma unroll
  for (int i = 0; i < kE; ++i) {
    d[i] = x[i] - mn;  // >= 0: mn <= every value of the group
    const float q = d[i] * r;
    c[i] = __builtin_rintf(q);
    // within 2^-13 of a half-integer: q - c is exact, and |q - c| <= 1/2
    near |= __builtin_fabsf(q - c[i]) > 0.5f - 0x1p-13f;
  }
  if (__builtin_amdgcn_ballot_w64(live && near) != 0) {
#pragma unroll
    for (int i = 0; i < kE; ++i) c[i] = live ? __builtin_rintf(d[i] / sc) : 0.0f;
  }
#pragma unroll
  for (int k = 0; k < kWords; ++k) packed[k] = 0u;
  if (live) {
    // the width is the same for the whole workgroup: one branch, and each
    // code's word and shift are constants
    if (bits == 2) pack_codes<2>(c, packed);
    else if (bits == 4) pack_codes<4>(c, packed);
    else pack_codes<8>(c, packed);
  }
  meta = uint32_t(sc16) | (uint32_t(mn16) << 16);
}

// Walsh-Hadamard rotation of one row (include/kvq.h; gist.science 2604.02570,
// section 2-C), held as kE values in each of the row's D/kE lanes: butterflies
// of stride 1 .. kE/2 inside the lane, then kE .. D/2 across lanes (the lower
// index of a pair keeps the sum, the upper one lower - upper), then the exact
// scaling by 2^-ceil(log2(D)/2).  Every lane of the row must be active.
template <int D>
__device__ inline void hadamard_row(float (&x)[kE], int lane_in_row) {
#pragma unroll
  for (int s = 1; s < kE; s <<= 1)
#pragma unroll
    for (int i = 0; i < kE; ++i)
      if (!(i & s)) {
        const float lo = x[i], hi = x[i + s];
        x[i] = lo + hi;
        x[i + s] = lo - hi;
      }
#pragma unroll
  for (int m = 1; m < D / kE; m <<= 1) {
    const bool upper = (lane_in_row & m) != 0;
#pragma unroll
    for (int i = 0; i < kE; ++i) {
      const float other = __shfl_xor(x[i], m);
      x[i] = upper ? other - x[i] : x[i] + other;
    }
  }
  constexpr float kScale = D == 128 ? 0.0625f : 0.125f;  // 2^-ceil(log2(D)/2)
#pragma unroll
  for (int i = 0; i < kE; ++i) x[i] = x[i] * kScale;
}

// Stores one row's lane share: this lane's kE values x of position t (row
// r of the call; inactive lanes past the call's rows only join the group
// reductions).
template <int D>
__device__ __forceinline__ void quantize_row(const QuantizeArgs& a, float (&x)[kE], int t,
                                             bool active, int lane_in_row, int sl, int lh,
                                             int X) {
  const int bits = a.bits[lh][X];
  const int vb = a.vb[sl], ve = a.ve[sl];
  // Position t is coded when it lies in the coded span and in none of the
  // sequence's bf16 ranges.  nc = coded positions before t: coded positions
  // take VIS rows in order, all others TXT rows in order.
  bool visual = t >= vb && t < ve;
  int nc = min(max(t, vb), ve) - vb;
  for (int k = a.rng_first[sl]; k < a.rng_first[sl + 1]; ++k) {
    const int b = a.rng_b[k], e = a.rng_e[k];
    nc -= t >= e ? e - b : t > b ? t - b : 0;
    visual = visual && !(t >= b && t < e);
  }
  uint8_t* vis = a.cache + uint64_t(a.base256[lh][X]) * 256u;

  // Coded K rows of a per-channel cache are written by quantize_kblock_kernel.
  if (visual && bits < 16 && X == 0 && a.k_per_channel) return;
  // Every lane of a row takes the same branch; groups never straddle rows.
  if (visual && bits < 16) {
    uint32_t meta;
    uint32_t packed[kWords];
    if (a.rotate_k && X == 0) hadamard_row<D>(x, lane_in_row);
    if (a.g == 32) quantize_lane<32 / kE>(x, bits, packed, meta);
    else if (a.g == 64) quantize_lane<64 / kE>(x, bits, packed, meta);
    else quantize_lane<128 / kE>(x, bits, packed, meta);
    if (!active) return;
    const int64_t row = a.vrow0[sl] + nc;
    uint8_t* rowp = vis + row * (D * bits / 8) + lane_in_row * (kE * bits / 8);
    // the lane's kE * bits / 32 words, in 16-byte pieces where they fill one
    const int words = kE * bits / 32;
    if (words >= 4) {
#pragma unroll
      for (int k = 0; k < kWords / 4; ++k)
        if (4 * k < words)
          reinterpret_cast<uint4*>(rowp)[k] =
              make_uint4(packed[4 * k], packed[4 * k + 1], packed[4 * k + 2], packed[4 * k + 3]);
    } else if (words == 2) {
      *reinterpret_cast<uint2*>(rowp) = make_uint2(packed[0], packed[1]);
    } else {
      *reinterpret_cast<uint32_t*>(rowp) = packed[0];
    }
    const int gl = a.g / kE;
    if (lane_in_row % gl == 0) {
      uint8_t* metap = vis + meta_plane_offset(a.Rvis, D, bits) + row * ((D / a.g) * 4);
      *reinterpret_cast<uint32_t*>(metap + (lane_in_row / gl) * 4) = meta;
    }
  } else {
    if (!active) return;
    uint8_t* rowp;
    if (visual) {  // 16-bit (protected) head: coded position kept bf16 in VIS
      rowp = vis + (a.vrow0[sl] + nc) * int64_t(2 * D);
    } else {
      const int64_t trow = a.trow0[sl] + (t - nc);
      rowp = vis + txt_plane_offset(a.Rvis, D, a.g, bits) + trow * int64_t(2 * D);
    }
#pragma unroll
    for (int k = 0; k < kE / 8; ++k) {
      uint4 o;
      o.x = uint32_t(bf16_rne(x[8 * k + 0])) | (uint32_t(bf16_rne(x[8 * k + 1])) << 16);
      o.y = uint32_t(bf16_rne(x[8 * k + 2])) | (uint32_t(bf16_rne(x[8 * k + 3])) << 16);
      o.z = uint32_t(bf16_rne(x[8 * k + 4])) | (uint32_t(bf16_rne(x[8 * k + 5])) << 16);
      o.w = uint32_t(bf16_rne(x[8 * k + 6])) | (uint32_t(bf16_rne(x[8 * k + 7])) << 16);
      reinterpret_cast<uint4*>(rowp + lane_in_row * (2 * kE))[k] = o;
    }
  }
}

// One row per D/kE lanes, 256 / (D/kE) rows per workgroup.  Instances per
// source dtype: the bf16 one holds half the source registers of the fp32
// one, which keeps more waves resident (the kernel is bound by how many rows
// are in flight, not by its arithmetic).
template <int D, bool BF16>  // BF16: bf16 sources (else fp32)
__global__ __launch_bounds__(256) void quantize_kernel(QuantizeArgs a) {
  constexpr int LPR = D / kE;            // lanes per row
  constexpr int RPB = 256 / LPR;         // rows per workgroup
  const int lane_in_row = threadIdx.x % LPR;
  const int row_in_block = threadIdx.x / LPR;
  const int z = blockIdx.z;              // (lh, X)
  const int lh = z >> 1, X = z & 1;
  const int sl = blockIdx.y;             // sequence within this launch
  const int r = blockIdx.x * RPB + row_in_block;  // row within [0, n_tok)
  const bool active = r < a.n_tok;
  const int rr = active ? r : a.n_tok - 1;  // keep inactive lanes in bounds
  // source element offset: [nl, num_seqs, Hkv, n_tok, D]
  const int glh = a.lh_off + lh;         // layer-local * Hkv + head
  const int l_local = glh / a.Hkv, h = glh % a.Hkv;
  const int64_t src_row =
      ((int64_t(l_local) * a.num_seqs_total + (a.seq_off + sl)) * a.Hkv + h) * a.n_tok + rr;
  const void* src = X ? a.v_src : a.k_src;
  float x[kE];
  if constexpr (BF16) {
    const uint4* p = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(src) +
                                                    src_row * D + lane_in_row * kE);
#pragma unroll
    for (int k = 0; k < kE / 8; ++k) {
      const uint4 v = p[k];
      const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        x[8 * k + 2 * i] = __builtin_bit_cast(float, w[i] << 16);
        x[8 * k + 2 * i + 1] = __builtin_bit_cast(float, w[i] & 0xFFFF0000u);
      }
    }
  } else {
    const float4* p = reinterpret_cast<const float4*>(static_cast<const float*>(src) +
                                                      src_row * D + lane_in_row * kE);
#pragma unroll
    for (int k = 0; k < kE / 4; ++k) {
      const float4 u = p[k];
      x[4 * k] = u.x; x[4 * k + 1] = u.y; x[4 * k + 2] = u.z; x[4 * k + 3] = u.w;
    }
  }
  quantize_row<D>(a, x, a.tok0[sl] + rr, active, lane_in_row, sl, lh, X);
}

// Per-channel K (k_per_channel): one workgroup per (slot, sequence, block of
// g coded tokens), one thread per channel d.  The channel's g values over the
// block form one group, quantised with the same arithmetic as a per-token
// group (the exact IEEE divide for every code); the thread writes the
// channel's (scale, min) pair into the block's META row, and the codes go
// through LDS so that every token row is packed and stored as whole words.
template <int D>
__global__ __launch_bounds__(D) void quantize_kblock_kernel(QuantizeArgs a) {
  __shared__ uint8_t codes[128][D];  // [token in block][channel]
  const int d = threadIdx.x;
  const int lh = blockIdx.z, sl = blockIdx.y, j = blockIdx.x;
  const int g = a.g, bits = a.bits[lh][0];
  if (j >= a.kblkn[sl] || bits >= 16) return;  // workgroup-uniform (bf16 K: no blocks)
  const int blk = a.kblk0[sl] + j;            // block within the sequence
  const int t0 = a.vb[sl] + blk * g;          // its first position
  const int r0 = t0 - a.tok0[sl];             // its first source row
  const int glh = a.lh_off + lh;
  const int l_local = glh / a.Hkv, h = glh % a.Hkv;
  const int64_t src_row0 =
      ((int64_t(l_local) * a.num_seqs_total + (a.seq_off + sl)) * a.Hkv + h) * a.n_tok + r0;
  auto load = [&](int i) {
    const int64_t e = (src_row0 + i) * D + d;
    return a.src_bf16 ? bf16_float(static_cast<const uint16_t*>(a.k_src)[e])
                      : static_cast<const float*>(a.k_src)[e];
  };
  float lo = load(0), hi = lo;
  for (int i = 1; i < g; ++i) {
    const float x = load(i);
    lo = fminf(lo, x);
    hi = fmaxf(hi, x);
  }
  const uint16_t mn16 = f16_round_down(lo);
  const float mn = f16_float(mn16);
  const float n = float((1 << bits) - 1);
  const float range = hi - mn;
  const bool live = range != 0.0f;
  const uint16_t sc16 = live ? f16_round_up(range / n) : uint16_t(0);
  const float sc = f16_float(sc16);
  for (int i = 0; i < g; ++i) {
    const float c = live ? __builtin_rintf((load(i) - mn) / sc) : 0.0f;
    codes[i][d] = uint8_t(__builtin_amdgcn_fmed3f(c, 0.0f, n));
  }
  uint8_t* vis = a.cache + uint64_t(a.base256[lh][0]) * 256u;
  const int64_t row0 = a.vrow0[sl] + int64_t(blk) * g;  // VIS row of t0 (a multiple of g)
  uint8_t* meta = vis + meta_plane_offset(a.Rvis, D, bits) + (row0 / g) * int64_t(4 * D);
  reinterpret_cast<uint32_t*>(meta)[d] = uint32_t(sc16) | (uint32_t(mn16) << 16);
  __syncthreads();
  // row i of the block: D * bits / 32 words, word k holds channels
  // [k * 32 / bits, (k + 1) * 32 / bits), channel c at bit (c * bits) % 32
  const int wpr = D * bits / 32, per = 32 / bits;
  uint32_t* rows = reinterpret_cast<uint32_t*>(vis + row0 * int64_t(D * bits / 8));
  for (int w = d; w < g * wpr; w += D) {
    const int i = w / wpr, k = w % wpr;
    uint32_t word = 0u;
    for (int e = 0; e < per; ++e) word |= uint32_t(codes[i][k * per + e]) << (e * bits);
    rows[w] = word;
  }
}

}  // namespace

hipError_t launch_quantize_kblocks(const QuantizeArgs& a, int n_lh_launch, int n_seq_launch,
                                   int max_blocks, hipStream_t stream) {
  if (max_blocks <= 0) return hipSuccess;
  const dim3 grid(max_blocks, n_seq_launch, n_lh_launch);
  if (a.D == 128)
    hipLaunchKernelGGL(quantize_kblock_kernel<128>, grid, dim3(128), 0, stream, a);
  else
    hipLaunchKernelGGL(quantize_kblock_kernel<64>, grid, dim3(64), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_quantize(const QuantizeArgs& a, int n_lh_launch, int n_seq_launch,
                           hipStream_t stream) {
  const int rpb = 256 / (a.D / kE);  // rows per block
  dim3 grid((a.n_tok + rpb - 1) / rpb, n_seq_launch, n_lh_launch * 2);
  if (a.D == 128 && a.src_bf16)
    hipLaunchKernelGGL((quantize_kernel<128, true>), grid, dim3(256), 0, stream, a);
  else if (a.D == 128)
    hipLaunchKernelGGL((quantize_kernel<128, false>), grid, dim3(256), 0, stream, a);
  else if (a.src_bf16)
    hipLaunchKernelGGL((quantize_kernel<64, true>), grid, dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL((quantize_kernel<64, false>), grid, dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace kvq
