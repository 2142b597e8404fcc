// kvq_decode_mfma.hip -- split-K decode attention on the CDNA4 matrix cores.
//
// Work is split over waves of (layer, sequence, KV head) token ranges; stored
// rows are reconstructed on chip and never written back (gist.science 2604.02570,
// section 2-D: reconstruction fused into flash decoding); K/V widths per
// head and the Visual/Text split follow nuiw.github.io "VLM_KV_Quantization"
// (sections 1-2) and the HeadGuard briefing (bf16 protected heads).
//
// Work of one wave: 32 tokens per step, all contractions on
// v_mfma_f32_16x16x32_{f16,bf16} (wave64, 16x16 tile, K = 32):
//
// A launch decodes a subgroup of G query heads of every KV head (a KV head
// with more than one tile of (head, group) columns takes several launches,
// each reading its rows again); q and out stride by all of the KV head's
// query heads (Gs).
//
//   q.k   S^T[token][c] = sum_k A[token][k] B[k][c] over two 16-token tiles.
//         A = stored K row data of the tile, B = Q' (built once per segment).
//         Column c = (head h, group j) = h * NG + j: Q' holds head h's query
//         restricted to the d of group j, so each column accumulates one
//         group's partial dot product and the group's fp16 scale/min apply
//         after the product: score = sum_j sc_j * acc_j + mn_j * sum_{d in j} q_d.
//         Integer codes enter the MFMA as exact binary16 SUBNORMALS: the code
//         bits are masked into place (value code * w * 2^-24 for a power of two
//         w set by the bit position); Q' carries 1/w, and 2^24 goes into the
//         scale.  bf16 rows enter the bf16 MFMA directly.
//   p.v   O[c][d] = sum_t A[c][t] B[t][d], eight (D=128) 16-column blocks.
//         The q.k result already sits in the A-operand layout (lane = column
//         c, registers = tokens), so no transpose is needed.  Row c of A holds
//         p * scale_V(token, group of c) in f16 (or p as a bf16 hi/lo pair for
//         bf16 V); B holds V codes as subnormals (or bf16 values).  Output
//         column d keeps row (h, group(d)); the min term sum_t p * min_V is an
//         fp32 side sum per row.
//
// Lane layout of v_mfma_f32_16x16x32 (checked on gfx950): A: lane l holds row
// l%16, k = 8(l/16)..+7; B: lane l holds column l%16, same k; C: lane l holds
// column l%16, rows 4(l/16)..+3.
//
// Online softmax in log2 units with a lazy running max: the wave rescales
// only when a column's max grows by more than kLazy, so p <= 2^kLazy.
#include <hip/hip_runtime.h>

#include "kvq_internal.h"

namespace kvq {
namespace {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Eight waves per workgroup and one workgroup per CU: two waves per SIMD,
// both of the same workgroup, so the LDS claim counter below can even out the
// older wave's issue advantage over the younger one.
constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr float kLazy = 6.0f;  // p <= 2^6 between rescales
#ifndef KVQ_RING_DEPTH
#define KVQ_RING_DEPTH 2  // quantised steps in flight per wave
#endif

__device__ inline f32x4 mfma_f16(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}
__device__ inline f32x4 mfma_bf16(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

__device__ inline float f16lo(uint32_t w) { return (float)__builtin_bit_cast(_Float16, uint16_t(w)); }
__device__ inline float f16hi(uint32_t w) { return (float)__builtin_bit_cast(_Float16, uint16_t(w >> 16)); }
__device__ inline float bf16f(uint32_t b) { return __builtin_bit_cast(float, b << 16); }
__device__ inline uint32_t pack_f16(float lo, float hi) {
  return uint32_t(__builtin_bit_cast(uint16_t, (_Float16)lo)) |
         (uint32_t(__builtin_bit_cast(uint16_t, (_Float16)hi)) << 16);
}
__device__ inline uint32_t pack_bf16(float lo, float hi) {
  return uint32_t(__builtin_bit_cast(uint16_t, (__bf16)lo)) |
         (uint32_t(__builtin_bit_cast(uint16_t, (__bf16)hi)) << 16);
}
// Lane l's value from lane l^1 / l^2 (quad permutes; no lane is out of
// bounds, bound_ctrl lets the move fold into the consuming add).
__device__ inline float dpp_xor1(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0xB1,
                                                               0xF, 0xF, true));
}
__device__ inline float dpp_xor2(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x4E,
                                                               0xF, 0xF, true));
}
// Max over lanes {l, l^16, l^32, l^48} (the four row quarters of one MFMA
// column) with the gfx950 cross-row swaps instead of LDS permutes.
// Maximum of two floats.  The NaN-propagating form maps to gfx950's
// v_maximum / v_maximum3, which need no input canonicalisation (fmaxf does
// when the compiler cannot prove its inputs canonical); the two agree on all
// non-NaN values, -inf included.
__device__ inline float fmax2(float a, float b) { return __builtin_elementwise_maximum(a, b); }
__device__ inline float max_over_quarters(float v) {
  const unsigned u = __builtin_bit_cast(unsigned, v);
  const auto r32 = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  const float m = fmax2(__builtin_bit_cast(float, unsigned(r32[0])),
                        __builtin_bit_cast(float, unsigned(r32[1])));
  const unsigned w = __builtin_bit_cast(unsigned, m);
  const auto r16 = __builtin_amdgcn_permlane16_swap(w, w, false, false);
  return fmax2(__builtin_bit_cast(float, unsigned(r16[0])), __builtin_bit_cast(float, unsigned(r16[1])));
}
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
// f16 pair (round to nearest even) of lo * slo, hi * shi.  Written as fmas
// with a zero addend so each half is one mixed-precision fma into its half
// of the result register.
__device__ inline uint32_t pack_f16_mul(float lo, float slo, float hi, float shi) {
  f16x2 r;
  r.x = (_Float16)__builtin_fmaf(lo, slo, 0.0f);
  r.y = (_Float16)__builtin_fmaf(hi, shi, 0.0f);
  return __builtin_bit_cast(uint32_t, r);
}

// ---------------------------------------------------------------------------
// Per-format row geometry.  D elements per row; a K row is split into 4 lane
// quarters of D/4 elements; a V row into 16 lane columns of D/16 elements.
template <int D, int B>
struct Fmt {
  static constexpr int kRowBytes = B == 16 ? 2 * D : D * B / 8;
  static constexpr int kKDwords = kRowBytes / 16;   // per lane quarter
  static constexpr int kVBytes = kRowBytes / 16;    // per lane column
};

// Slot map of the q.k A operand: k-step s, slot e (0..7) -> the head-dim
// offset within the lane's quarter (d - jq * D / 4) and the power-of-two
// weight w of the stored code bits (operand value = code * w * 2^-24).  Must
// mirror k_operand() below.  Every format's slots of k-steps 2i and 2i + 1
// cover quarter offsets [16 i, 16 i + 16) exactly once.
template <int D, int B>
__device__ constexpr int kslot_off(int s, int e) {
  const int kp = e >> 1, hf = e & 1;
  if (B == 16) return 8 * s + e;
  if (B == 8) return 4 * (2 * s + (kp >> 1)) + (kp & 1) + 2 * hf;
  if (B == 4) return 8 * s + kp + 4 * hf;
  return 16 * (s >> 1) + ((s & 1) ? 4 : 0) + kp + 8 * hf;
}
template <int D, int B>
__device__ constexpr float kslot_w(int s, int e) {
  const int kp = e >> 1;
  if (B == 16 || B == 8) return 1.0f;
  if (B == 4) return (kp & 1) ? 16.0f : 1.0f;
  return ((s & 1) == 0 || kp) ? float(1 << (2 * kp)) : 256.0f;
}

// A operand (4 dwords) of k-step s from this lane's raw K dwords.
template <int D, int B>
__device__ inline u32x4 k_operand(const uint32_t* w, int s) {
  u32x4 a;
  if (B == 16) {
    a[0] = w[4 * s]; a[1] = w[4 * s + 1]; a[2] = w[4 * s + 2]; a[3] = w[4 * s + 3];
  } else if (B == 8) {
    const uint32_t x = w[2 * s], y = w[2 * s + 1];
    a[0] = x & 0x00FF00FFu; a[1] = (x >> 8) & 0x00FF00FFu;
    a[2] = y & 0x00FF00FFu; a[3] = (y >> 8) & 0x00FF00FFu;
  } else if (B == 4) {
    const uint32_t x = w[s], t = x >> 8;
    a[0] = x & 0x000F000Fu; a[1] = x & 0x00F000F0u;
    a[2] = t & 0x000F000Fu; a[3] = t & 0x00F000F0u;
  } else {
    const uint32_t x = w[s >> 1];
    if ((s & 1) == 0) {
      a[0] = x & 0x00030003u; a[1] = x & 0x000C000Cu;
      a[2] = x & 0x00300030u; a[3] = x & 0x00C000C0u;
    } else {
      const uint32_t t = x >> 8;
      a[0] = x & 0x03000300u; a[1] = t & 0x000C000Cu;
      a[2] = t & 0x00300030u; a[3] = t & 0x00C000C0u;
    }
  }
  return a;
}

// p.v B operand: for a pair of tokens (a: lo half, b: hi half) the lane's V
// slices are first merged into pair words (vpair_words), then each 16-column
// block mb takes one masked word (v_block).  Value = code * wv(mb) * 2^-24,
// or the bf16 element itself.
template <int D, int B>
struct VPair {
  static constexpr int N = B == 16 ? D / 32 : B == 8 ? D / 64 : 2;
  uint32_t w[N];
};
// Bytes per lane per token of a V row (one of 16 lane columns).
template <int D, int B>
__device__ constexpr int v_lane_bytes() { return (B == 16 ? 2 * D : D * B / 8) / 16; }
// Byte selector that merges this lane's V slice of two tokens (a low, b
// high) into one pair word when the slice is 1 or 2 bytes wide and sits at
// byte offset o of the dword it was read in (o = 0 when loaded on its own).
template <int D, int B>
__device__ inline uint32_t v_pair_selector(int o) {
  constexpr int VBY = v_lane_bytes<D, B>();
  if constexpr (VBY == 2)
    return uint32_t(o) | uint32_t(o + 1) << 8 | uint32_t(o + 4) << 16 | uint32_t(o + 5) << 24;
  else
    return uint32_t(o) | 0x0Cu << 8 | uint32_t(o + 4) << 16 | 0x0Cu << 24;  // 0x0C: zero byte
}
template <int D, int B>
__device__ inline VPair<D, B> vpair_words(const uint32_t* a, const uint32_t* b, uint32_t vsel) {
  VPair<D, B> r;
  if constexpr (B == 16) {  // bf16 elements 2i, 2i+1 of each token
#pragma unroll
    for (int i = 0; i < D / 32; ++i) {
      r.w[i] = a[i];          // kept raw; v_block permutes
    }
  } else if constexpr (B == 8) {
#pragma unroll
    for (int i = 0; i < D / 64; ++i) r.w[i] = a[i];
  } else if constexpr (B == 4 && v_lane_bytes<D, B>() == 4) {
    r.w[0] = __builtin_amdgcn_perm(b[0], a[0], 0x05040100u);  // nibbles 0..3 of a | b
    r.w[1] = __builtin_amdgcn_perm(b[0], a[0], 0x07060302u);  // nibbles 4..7
  } else {  // 1- or 2-byte slices: one selector merge
    r.w[0] = __builtin_amdgcn_perm(b[0], a[0], vsel);
    r.w[1] = r.w[0] >> 8;
  }
  return r;
}
template <int D, int B>
__device__ inline uint32_t v_block(const VPair<D, B>& pw, const uint32_t* a, const uint32_t* b,
                                   int mb) {
  if constexpr (B == 16) {
    return __builtin_amdgcn_perm(b[mb >> 1], a[mb >> 1], (mb & 1) ? 0x07060302u : 0x05040100u);
  } else if constexpr (B == 8) {
    const uint32_t sel = 0x0C000C00u | (uint32_t(4 + (mb & 3)) << 16) | uint32_t(mb & 3);
    return __builtin_amdgcn_perm(b[mb >> 2], a[mb >> 2], sel);
  } else if constexpr (B == 4) {
    const uint32_t x = pw.w[(mb >> 2) & 1];
    const uint32_t t = (mb & 2) ? (x >> 8) : x;
    return t & ((mb & 1) ? 0x00F000F0u : 0x000F000Fu);
  } else {
    if (D == 128 && mb >= 5) return pw.w[1] & (0x00030003u << (2 * (mb - 4)));
    return pw.w[0] & (0x00030003u << (2 * mb));
  }
}
template <int D, int B>
__device__ constexpr float v_weight(int mb) {
  return B == 16 ? 1.0f
       : B == 8  ? 1.0f
       : B == 4  ? ((mb & 1) ? 16.0f : 1.0f)
       : (D == 128 && mb >= 5) ? float(1 << (2 * (mb - 4))) : float(1 << (2 * mb));
}
// Factor by which p.v MFMA outputs of block mb exceed the true value.
template <int D, int B>
__device__ constexpr float v_inflation(int mb) {
  return B == 16 ? 1.0f : v_weight<D, B>(mb) * 5.9604644775390625e-08f;  // * 2^-24
}

template <int D>
struct WaveState {
  static constexpr int NB = D / 16;
  f32x4 o[NB];      // p.v accumulators, scaled per the current V format
  float m;          // running max (log2 units) of this lane's column
  float l;          // partial sum of p over this lane's tokens
  float mt;         // partial sum of p * min_V over this lane's tokens
};

struct Ctx {
  const uint8_t* kvis;  // K planes of this (layer, head)
  const uint8_t* kmeta;
  const uint8_t* ktxt;
  const uint8_t* vvis;
  const uint8_t* vmeta;
  const uint8_t* vtxt;
  u32x4* qq;               // this lane's D/64 16-byte pieces in LDS: quarter jq of
                           // the query of column n's head (head 0 for dead columns)
  uint8_t* stage;          // this wave's LDS stage (BigLds::kStage bytes)
  float qscale;
  int G;
  int64_t kmeta_bytes;     // size of the K META plane (per-channel block loads)
  bool rotate_k;           // coded K rows are stored Walsh-Hadamard rotated
  int lane, n, jq;         // lane, column (l % 16), quarter (l / 16)
};

// The lane's quarter of its head's query (bf16 pairs) -> fp32 values.
template <int D>
__device__ inline void unpack_quarter(const Ctx& c, float (&v)[D / 4]) {
#pragma unroll
  for (int k = 0; k < D / 32; ++k) {
    const u32x4 w = c.qq[k];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[8 * k + 2 * i] = bf16f(w[i] & 0xFFFFu);
      v[8 * k + 2 * i + 1] = bf16f(w[i] >> 16);
    }
  }
}

// The lane's quarter of the query -> the same quarter of the rotated query,
// for K rows stored rotated (include/kvq.h; gist.science 2604.02570, section
// 2-C): the butterflies of the stored rows, then 2^-floor(log2(D)/2), so the
// product with a rotated K row is q.k.  Strides below D/4 run inside the
// lane; strides D/4 and D/2 pair quarter jq with jq ^ 1 and jq ^ 2, which sit
// 16 and 32 lanes away (lane = 16 jq + column).
template <int D>
__device__ inline void rotate_quarter(const Ctx& c, float (&v)[D / 4]) {
  constexpr int Q = D / 4;
#pragma unroll
  for (int st = 1; st < Q; st <<= 1)
#pragma unroll
    for (int i = 0; i < Q; ++i)
      if (!(i & st)) {
        const float lo = v[i], hi = v[i + st];
        v[i] = lo + hi;
        v[i + st] = lo - hi;
      }
#pragma unroll
  for (int m = 1; m <= 2; m <<= 1) {
    const bool upper = (c.jq & m) != 0;
#pragma unroll
    for (int i = 0; i < Q; ++i) {
      const float other = __shfl_xor(v[i], 16 * m);
      v[i] = upper ? other - v[i] : v[i] + other;
    }
  }
#pragma unroll
  for (int i = 0; i < Q; ++i) v[i] *= 0.125f;  // 2^-floor(log2(D)/2), D in {64, 128}
}

// Build Q' for k format KB: per k-step, 8 slots of this lane's column.
// Returns the sum of q over the column's (head, group), times 2^-24 (the unit
// of the code products): each lane's slots cover its quarter of the head dim
// exactly once, so a sum over the four quarters completes it.  qv: the lane's
// quarter of the (possibly rotated) query.
template <int D, int NG, int KB>
__device__ inline float build_q(const Ctx& c, const float (&qv)[D / 4], u32x4 (&qop)[D / 32]) {
  constexpr int g = D / NG;
  const int gj = c.n % NG;
  const bool live = c.n < c.G * NG;
  const int c0 = c.jq * (D / 4);
  float qs = 0.0f;
#pragma unroll
  for (int s = 0; s < D / 32; ++s) {
#pragma unroll
    for (int e2 = 0; e2 < 4; ++e2) {
      float v2[2];
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        const int off = kslot_off<D, KB>(s, 2 * e2 + hf);
        const float w = kslot_w<D, KB>(s, 2 * e2 + hf);
        const float q = qv[off];
        const bool in = live && (c0 + off) / g == gj;
        qs += in ? q : 0.0f;
        v2[hf] = in ? q * (1.0f / w) : 0.0f;  // w: power of two
      }
      qop[s][e2] = KB == 16 ? pack_bf16(v2[0], v2[1]) : pack_f16(v2[0], v2[1]);
    }
  }
  qs += __shfl_xor(qs, 16);
  qs += __shfl_xor(qs, 32);
  return qs * 5.9604644775390625e-08f;  // * 2^-24, exact
}

// Q' of one per-channel K block: the block's META row (D (scale, min) fp16
// pairs, pair d for channel d) at pairs, in LDS.  The channel scale goes into
// the query operand and the min into one constant per column:
//   q.k^ = sum_d q_d (s_d c_d + m_d) = sum_d (q_d s_d) c_d + sum_d q_d m_d.
// The operand is q_d s_d 2^4 / w (the 2^4 keeps small products out of the
// binary16 subnormals), so products with the codes come out in units of
// 2^-20; the returned constant of the lane's column (head, group), summed over
// its four quarters, is in the same units.  q_d s_d needs up to 19
// significant bits (bf16 times fp16), more than binary16 holds, so it is
// carried as a binary16 pair hi + lo (qop, qlo): two products per code, error
// about 2^-22 relative, where one binary16 operand alone (2^-12) cost the
// LLaVA-shaped layer 1.5e-3 of relative L2 error in the output.
template <int D, int NG, int KB>
__device__ inline float build_q_pc(const Ctx& c, const uint32_t* pairs, u32x4 (&qop)[D / 32],
                                   u32x4 (&qlo)[D / 32]) {
  constexpr int g = D / NG;
  const int c0 = c.jq * (D / 4);
  // A lane's quarter [c0, c0 + D/4) lies inside one group (g is a multiple
  // of D/4), so whether the lane's column (head, group) owns its channels is
  // one test per lane; a lane that does not works on a zero query.
  const bool in = c.n < c.G * NG && c0 / g == c.n % NG;
  float mt = 0.0f;
  // k-steps 2i and 2i + 1 cover quarter offsets [16 i, 16 i + 16): read
  // those 16 query values and (scale, min) pairs, then fill both k-steps.
  // The products read the binary16 scale and min straight from the pair
  // words (mixed-precision fmas, one rounding each); q * 16 / w is exact.
#pragma unroll
  for (int i = 0; i < D / 64; ++i) {
    uint32_t qw[8], sm[16];
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const u32x4 w = c.qq[2 * i + k];
      qw[4 * k] = w[0]; qw[4 * k + 1] = w[1]; qw[4 * k + 2] = w[2]; qw[4 * k + 3] = w[3];
    }
#pragma unroll
    for (int k = 0; k < 8; ++k) qw[k] = in ? qw[k] : 0u;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const uint4 w4 = reinterpret_cast<const uint4*>(pairs + c0 + 16 * i)[k];
      sm[4 * k] = w4.x; sm[4 * k + 1] = w4.y; sm[4 * k + 2] = w4.z; sm[4 * k + 3] = w4.w;
    }
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) {
      const int s = 2 * i + s2;
#pragma unroll
      for (int e2 = 0; e2 < 4; ++e2) {
        float v2[2];
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
          const int off = kslot_off<D, KB>(s, 2 * e2 + hf), o16 = off - 16 * i;
          const float w = kslot_w<D, KB>(s, 2 * e2 + hf);
          const float q = bf16f((qw[o16 >> 1] >> (16 * (o16 & 1))) & 0xFFFFu);
          mt = __builtin_fmaf(q, f16hi(sm[o16]), mt);
          v2[hf] = __builtin_fmaf(q * (16.0f / w), f16lo(sm[o16]), 0.0f);  // w: power of two
        }
        const uint32_t hi = pack_f16(v2[0], v2[1]);
        qop[s][e2] = hi;
        // the remainders are exact in fp32 (v minus its binary16 rounding)
        qlo[s][e2] = pack_f16(__builtin_fmaf(f16lo(hi), -1.0f, v2[0]),
                              __builtin_fmaf(f16hi(hi), -1.0f, v2[1]));
      }
    }
  }
  mt += __shfl_xor(mt, 16);
  mt += __shfl_xor(mt, 32);
  return mt * 9.5367431640625e-07f;  // * 2^-20, exact
}

template <int NBYTES>
__device__ inline void load_bytes(const uint8_t* p, uint32_t* out) {
  if constexpr (NBYTES >= 16) {
#pragma unroll
    for (int i = 0; i < NBYTES / 16; ++i) {
      const uint4 v = reinterpret_cast<const uint4*>(p)[i];
      out[4 * i] = v.x; out[4 * i + 1] = v.y; out[4 * i + 2] = v.z; out[4 * i + 3] = v.w;
    }
  } else if constexpr (NBYTES == 8) {
    const uint2 v = *reinterpret_cast<const uint2*>(p);
    out[0] = v.x; out[1] = v.y;
  } else if constexpr (NBYTES == 4) {
    out[0] = *reinterpret_cast<const uint32_t*>(p);
  } else if constexpr (NBYTES == 2) {
    out[0] = *reinterpret_cast<const uint16_t*>(p);
  } else {
    out[0] = *p;
  }
}

// Raw data one lane needs for one 32-token step.
template <int D, int KB, int VB>
struct Step {
  static constexpr int KDW = Fmt<D, KB>::kRowBytes / 16;          // dwords per K quarter-row
  static constexpr int VDW = (Fmt<D, VB>::kVBytes + 3) / 4;       // dwords per V lane slice
  uint32_t k[2][KDW];
  uint32_t km[KB < 16 ? 8 : 1];
  uint32_t vm[VB < 16 ? 8 : 1];
  uint32_t v[8][VDW];
};

// Lane byte offsets of one step, relative to the step's first row.  In full
// steps the per-slot parts are compile-time constants added to three base
// offsets; the tail step clamps every slot's row to the segment end.
template <int D, int NG, int KB, int VB>
struct Offs {
  static constexpr int KR = Fmt<D, KB>::kRowBytes, VR = Fmt<D, VB>::kRowBytes, MR = NG * 4;
  uint32_t k0, m0, v0;   // tile-0 / slot-0 base offsets
  uint32_t k[2], m[8], v[8];  // clamped offsets (tail step only)
  __device__ inline void full(const Ctx& c) {
    k0 = uint32_t(c.n * KR + c.jq * (KR / 4));
    m0 = uint32_t(4 * c.jq * MR + (c.n % NG) * 4);
    v0 = uint32_t(4 * c.jq * VR + c.n * Fmt<D, VB>::kVBytes);
  }
  __device__ inline void clamped(const Ctx& c, int rows_left) {
#pragma unroll
    for (int tau = 0; tau < 2; ++tau) {
      const int r = min(16 * tau + c.n, rows_left - 1);
      k[tau] = uint32_t(r * KR + c.jq * (KR / 4));
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int r = min(16 * (e >> 2) + 4 * c.jq + (e & 3), rows_left - 1);
      m[e] = uint32_t(r * MR + (c.n % NG) * 4);
      v[e] = uint32_t(r * VR + c.n * Fmt<D, VB>::kVBytes);
    }
  }
  static constexpr uint32_t kslot_off(int tau) { return uint32_t(16 * tau * KR); }
  static constexpr uint32_t mslot_off(int e) { return uint32_t((16 * (e >> 2) + (e & 3)) * MR); }
  static constexpr uint32_t vslot_off(int e) { return uint32_t((16 * (e >> 2) + (e & 3)) * VR); }
};

template <int D, int NG, int KB, int VB, bool CLAMPED>
__device__ inline void load_step(const uint8_t* kp, const uint8_t* kmp, const uint8_t* vp,
                                 const uint8_t* vmp, const Offs<D, NG, KB, VB>& o,
                                 Step<D, KB, VB>& st) {
  using O = Offs<D, NG, KB, VB>;
  constexpr int KQ = Fmt<D, KB>::kRowBytes / 4;
#pragma unroll
  for (int tau = 0; tau < 2; ++tau)
    load_bytes<KQ>(kp + (CLAMPED ? o.k[tau] : o.k0 + O::kslot_off(tau)), st.k[tau]);
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const uint32_t mo = CLAMPED ? o.m[e] : o.m0 + O::mslot_off(e);
    const uint32_t vo = CLAMPED ? o.v[e] : o.v0 + O::vslot_off(e);
    if constexpr (KB < 16) st.km[e] = *reinterpret_cast<const uint32_t*>(kmp + mo);
    if constexpr (VB < 16) st.vm[e] = *reinterpret_cast<const uint32_t*>(vmp + mo);
    load_bytes<Fmt<D, VB>::kVBytes>(vp + vo, st.v[e]);
  }
}

// exp, P operand and p.v of one step, given the scaled scores and the
// (possibly just raised) running max.
template <int D, int NG, int KB, int VB>
__device__ inline void finish_step(WaveState<D>& ws, const Step<D, KB, VB>& st,
                                   const float (&sc)[8], float cs, uint32_t vsel) {
  constexpr int NB = D / 16;
  float p[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    p[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[e], cs, -ws.m));
    ws.l += p[e];
  }

  u32x4 pa, pb;  // A operand (and the bf16 low part for bf16 V)
  if constexpr (VB < 16) {
#pragma unroll
    for (int e2 = 0; e2 < 4; ++e2) {
      const float p0 = p[2 * e2], p1 = p[2 * e2 + 1];
      pa[e2] = pack_f16_mul(p0, f16lo(st.vm[2 * e2]), p1, f16lo(st.vm[2 * e2 + 1]));
      ws.mt = __builtin_fmaf(p0, f16hi(st.vm[2 * e2]), ws.mt);
      ws.mt = __builtin_fmaf(p1, f16hi(st.vm[2 * e2 + 1]), ws.mt);
    }
  } else {
#pragma unroll
    for (int e2 = 0; e2 < 4; ++e2) {
      const float p0 = p[2 * e2], p1 = p[2 * e2 + 1];
      pa[e2] = pack_bf16(p0, p1);
      pb[e2] = pack_bf16(p0 - bf16f(pa[e2] & 0xFFFFu), p1 - bf16f(pa[e2] >> 16));
    }
  }
  VPair<D, VB> pw[4];
#pragma unroll
  for (int e2 = 0; e2 < 4; ++e2)
    pw[e2] = vpair_words<D, VB>(st.v[2 * e2], st.v[2 * e2 + 1], vsel);
#pragma unroll
  for (int mb = 0; mb < NB; ++mb) {
    u32x4 b;
#pragma unroll
    for (int e2 = 0; e2 < 4; ++e2) b[e2] = v_block<D, VB>(pw[e2], st.v[2 * e2], st.v[2 * e2 + 1], mb);
    if constexpr (VB == 16) {
      ws.o[mb] = mfma_bf16(pa, b, ws.o[mb]);
      ws.o[mb] = mfma_bf16(pb, b, ws.o[mb]);
    } else {
      ws.o[mb] = mfma_f16(pa, b, ws.o[mb]);
    }
  }
}

// q.k, softmax and p.v of one 32-token step of which the first rows_left
// (1..32, wave-uniform) rows are real.  vsel: see v_pair_selector.
template <int D, int NG, int KB, int VB, bool PC = false>
__device__ inline void compute_step(const Ctx& c, WaveState<D>& ws, const Step<D, KB, VB>& st,
                                    const u32x4 (&qop)[D / 32], float qsr, float c24,
                                    int rows_left, uint32_t vsel,
                                    const u32x4 (*qlo)[D / 32] = nullptr) {
  constexpr int KS = D / 32;
  constexpr int NB = D / 16;
  f32x4 acc[2];
#pragma unroll
  for (int tau = 0; tau < 2; ++tau) {
    acc[tau] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const u32x4 a = k_operand<D, KB>(st.k[tau], s);
      acc[tau] = KB == 16 ? mfma_bf16(a, qop[s], acc[tau]) : mfma_f16(a, qop[s], acc[tau]);
      if constexpr (PC) acc[tau] = mfma_f16(a, (*qlo)[s], acc[tau]);
    }
  }
  // scaled scores v: score (log2 units) = v * cs.  Quantised K: v = sc * acc +
  // mn * qsr with acc in units of 2^-24 (see build_q), so cs = 2^24 * qscale
  // and qsr = 2^-24 * sum(q over the group); per-channel K: v = acc + qsr
  // in units of 2^-20 (see build_q_pc), cs = 2^20 * qscale; bf16 K: v = acc,
  // cs = qscale.
  const float cs = PC ? c24 * 0.0625f : KB < 16 ? c24 : c.qscale;
  float sc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const float a = acc[e >> 2][e & 3];
    float part;
    // (mn * qsr as an fma with a zero addend: the same single rounding, in
    // one mixed-precision instruction that reads mn as f16)
    if constexpr (PC)
      part = a + qsr;
    else if constexpr (KB < 16)
      part = __builtin_fmaf(f16lo(st.km[e]), a, __builtin_fmaf(f16hi(st.km[e]), qsr, 0.0f));
    else part = a;
    if constexpr (NG >= 2) part += dpp_xor1(part);
    if constexpr (NG >= 4) part += dpp_xor2(part);
    sc[e] = part;
  }
  if (rows_left < 32) {  // a segment's last step: rows past its end do not count
#pragma unroll
    for (int e = 0; e < 8; ++e)
      if (16 * (e >> 2) + 4 * c.jq + (e & 3) >= rows_left) sc[e] = -INFINITY;
  }

  // online softmax with a lazy running max: the accumulators are rescaled
  // only when a column's max grows by more than kLazy, so p <= 2^kLazy.
  float mx = fmax2(fmax2(fmax2(sc[0], sc[1]), fmax2(sc[2], sc[3])),
                   fmax2(fmax2(sc[4], sc[5]), fmax2(sc[6], sc[7])));
  mx = max_over_quarters(mx) * cs;
  const float mnew = fmax2(ws.m, mx);
  if (__builtin_amdgcn_ballot_w64(mnew > ws.m + kLazy) != 0) {
    const float alpha = __builtin_amdgcn_exp2f(ws.m - mnew);  // 0 on the first step
    ws.l *= alpha;
    ws.mt *= alpha;
    float ar[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) ar[i] = __shfl(alpha, 4 * c.jq + i);
#pragma unroll
    for (int mb = 0; mb < NB; ++mb)
#pragma unroll
      for (int i = 0; i < 4; ++i) ws.o[mb][i] *= ar[i];
    ws.m = mnew;
  }
  finish_step<D, NG, KB, VB>(ws, st, sc, cs, vsel);
}

// ---------------------------------------------------------------------------
// Cooperative staging of quantised steps through wave-private LDS.
//
// The 32 rows of a step form contiguous tiles in each plane (K codes, K meta,
// V codes, V meta).  Lane l loads bytes [l * RB/2, (l + 1) * RB/2) of a tile
// of row size RB -- row l/2, half l%2 -- with the widest loads the piece
// allows, writes the piece to the same offset of the wave's LDS stage, and
// the operands are then read back in the MFMA layouts.  Versus loading the
// operand layouts straight from memory this issues ~5 wide loads per step
// instead of ~26 narrow ones and keeps ~14 VGPRs per step in flight instead
// of ~32, so two steps stay in flight per wave.
template <int NBYTES>
__device__ inline void store_bytes(uint8_t* p, const uint32_t* in) {
  if constexpr (NBYTES >= 16) {
#pragma unroll
    for (int i = 0; i < NBYTES / 16; ++i)
      reinterpret_cast<uint4*>(p)[i] = make_uint4(in[4 * i], in[4 * i + 1], in[4 * i + 2],
                                                  in[4 * i + 3]);
  } else if constexpr (NBYTES == 8) {
    *reinterpret_cast<uint2*>(p) = make_uint2(in[0], in[1]);
  } else if constexpr (NBYTES == 4) {
    *reinterpret_cast<uint32_t*>(p) = in[0];
  } else {
    *reinterpret_cast<uint16_t*>(p) = uint16_t(in[0]);
  }
}

template <int D, int NG, int KB, int VB>
struct Stage {
  static constexpr int KR = Fmt<D, KB>::kRowBytes, VR = Fmt<D, VB>::kRowBytes, MR = NG * 4;
  static constexpr int KP = KR / 2, VP = VR / 2, MP = MR / 2;  // bytes per lane per tile
  // The K meta region holds either the step's 32 META rows (per-token
  // groups) or its block's META row of D (scale, min) pairs (per-channel K,
  // D / 16 bytes per lane).
  static constexpr int PCP = D / 16;
  static constexpr int KMB = 32 * MR > 4 * D ? 32 * MR : 4 * D;
  static constexpr int kOffKM = 32 * KR, kOffV = kOffKM + KMB, kOffVM = kOffV + 32 * VR;
  static constexpr int kBytes = kOffVM + 32 * MR;
  uint32_t k[KP / 4];
  uint32_t km[((MP > PCP ? MP : PCP) + 3) / 4];
  uint32_t v[VP / 4];
  uint32_t vm[(MP + 3) / 4];
};


// Buffer resource over `bytes` bytes from `base` (raw, unswizzled): loads
// through it take a per-lane 32-bit offset plus a wave-uniform offset, so a
// step's loads need no per-lane address arithmetic.
typedef __amdgpu_buffer_rsrc_t Rsrc;
// Cache-policy operand of buffer loads: sc0 | sc1, i.e. system-coherent (the
// load is served past this XCD's caches).
constexpr int kCoherent = 1 | 16;
// Cache rows are read once per call: the non-temporal bit (nt) lets them
// stream through the caches without evicting what is reused -- the code of
// the tail paths, the argument block, query rows -- so the combine and merge
// at the end of a launch start warm (0.7-1 us per 28-layer step).  Only
// loads whose instruction covers whole lines take it: a line that several
// instructions read in parts is gone before the later ones arrive (64-byte
// lane pieces of 128-byte INT8 K rows: 100 -> 124 us on a 64-sequence batch).
constexpr int kStream = 2;
__device__ inline Rsrc make_rsrc(const void* base, int64_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0,
                                           int(bytes < 0x7FFFFFFF ? bytes : 0x7FFFFFFF),
                                           0x00020000);
}
// A lane's NBYTES at voff; callers lay the lanes' pieces end to end, so one
// instruction covers whole lines only when a piece is one load.
template <int NBYTES>
__device__ inline void buf_load(Rsrc r, uint32_t voff, uint32_t soff, uint32_t* out) {
  constexpr int kAux = NBYTES <= 16 ? kStream : 0;
  if constexpr (NBYTES >= 16) {
#pragma unroll
    for (int i = 0; i < NBYTES / 16; ++i) {
      const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, voff + 16 * i, soff, kAux);
      out[4 * i] = v[0]; out[4 * i + 1] = v[1]; out[4 * i + 2] = v[2]; out[4 * i + 3] = v[3];
    }
  } else if constexpr (NBYTES == 8) {
    const auto v = __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, kAux);
    out[0] = v[0]; out[1] = v[1];
  } else if constexpr (NBYTES == 4) {
    out[0] = __builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, kAux);
  } else {
    out[0] = __builtin_amdgcn_raw_buffer_load_b16(r, voff, soff, kAux);
  }
}

// The four planes of one segment (K codes, K meta, V codes, V meta).
struct SegPlanes {
  Rsrc k, km, v, vm;
};

// Lane l's share of a 32-row tile of row size R (P = R / 2 bytes per lane).
// A 32-byte lane piece is taken as two 16-byte chunks, chunk i at tile
// offset (64 i + l) * 16, so each load instruction covers 1 KB of
// consecutive bytes (0.6 us off the 28-layer HeadGuard step against a
// 32-byte lane stride); other pieces are bytes [l P, (l + 1) P) (for 64-byte
// pieces, INT8 K at D = 128, the chunked form costs registers the kernel does
// not have).  Only the first `rows` (1..32) rows exist: a chunk in a later
// row re-reads the same columns of the last row.  The chunk offsets without
// that clamp say where tile_put stores the data.
template <int R, int P>
__device__ inline void tile_load(Rsrc r, uint32_t soff, int rows, int lane, uint32_t* out) {
  if constexpr (P == 32) {
#pragma unroll
    for (int i = 0; i < P / 16; ++i) {
      const uint32_t off = uint32_t(i * 64 + lane) * 16u;
      const uint32_t row = min(off / R, uint32_t(rows - 1)), col = off % R;
      const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, row * R + col, soff, kStream);
      out[4 * i] = v[0]; out[4 * i + 1] = v[1]; out[4 * i + 2] = v[2]; out[4 * i + 3] = v[3];
    }
  } else {
    const uint32_t row = min(uint32_t(lane >> 1), uint32_t(rows - 1)), half = uint32_t(lane & 1);
    buf_load<P>(r, row * R + half * P, soff, out);
  }
}
template <int P>
__device__ inline void tile_put(uint8_t* lds, int lane, const uint32_t* in) {
  if constexpr (P == 32) {
#pragma unroll
    for (int i = 0; i < P / 16; ++i)
      reinterpret_cast<uint4*>(lds)[i * 64 + lane] =
          make_uint4(in[4 * i], in[4 * i + 1], in[4 * i + 2], in[4 * i + 3]);
  } else {
    store_bytes<P>(lds + lane * P, in);
  }
}

// Lane share of every plane's tile of step `step` (wave-uniform).  PC: the
// K meta is the META row of the step's block, at byte kmblk of the plane.
template <int D, int NG, int KB, int VB, bool PC>
__device__ inline void stage_load(const SegPlanes& pl, int step, int rows, int lane,
                                  Stage<D, NG, KB, VB>& st, uint32_t kmblk) {
  using S = Stage<D, NG, KB, VB>;
  const uint32_t r0 = uint32_t(step) * 32u;
  tile_load<S::KR, S::KP>(pl.k, r0 * S::KR, rows, lane, st.k);
  if constexpr (PC)
    buf_load<S::PCP>(pl.km, uint32_t(lane) * S::PCP, kmblk, st.km);
  else
    tile_load<S::MR, S::MP>(pl.km, r0 * S::MR, rows, lane, st.km);
  tile_load<S::VR, S::VP>(pl.v, r0 * S::VR, rows, lane, st.v);
  tile_load<S::MR, S::MP>(pl.vm, r0 * S::MR, rows, lane, st.vm);
}

// Lanes exchange data through the stage, so the compiler must not move one
// lane's LDS accesses across another's: wave barriers order the previous
// step's reads before these writes, and these writes before the next reads
// (LDS executes one wave's instructions in order).
template <int D, int NG, int KB, int VB, bool PC>
__device__ inline void stage_put(uint8_t* lds, int lane, const Stage<D, NG, KB, VB>& st) {
  using S = Stage<D, NG, KB, VB>;
  __builtin_amdgcn_wave_barrier();
  tile_put<S::KP>(lds, lane, st.k);
  if constexpr (PC)
    store_bytes<S::PCP>(lds + S::kOffKM + lane * S::PCP, st.km);
  else
    tile_put<S::MP>(lds + S::kOffKM, lane, st.km);
  tile_put<S::VP>(lds + S::kOffV, lane, st.v);
  tile_put<S::MP>(lds + S::kOffVM, lane, st.vm);
  __builtin_amdgcn_wave_barrier();
}

// Operand gather from the LDS stage into the layout compute_step expects.
template <int D, int NG, int KB, int VB, bool PC>
__device__ inline void stage_get(const uint8_t* lds, const Ctx& c, Step<D, KB, VB>& st) {
  using S = Stage<D, NG, KB, VB>;
  constexpr int KQ = S::KR / 4, VBY = Fmt<D, VB>::kVBytes;
  const int gj = c.n % NG;
#pragma unroll
  for (int tau = 0; tau < 2; ++tau)
    load_bytes<KQ>(lds + (16 * tau + c.n) * S::KR + c.jq * KQ, st.k[tau]);
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int r = 16 * (e >> 2) + 4 * c.jq + (e & 3);
    if constexpr (!PC)
      st.km[e] = *reinterpret_cast<const uint32_t*>(lds + S::kOffKM + r * S::MR + gj * 4);
    st.vm[e] = *reinterpret_cast<const uint32_t*>(lds + S::kOffVM + r * S::MR + gj * 4);
    if constexpr (VBY <= 2)  // the aligned dword holding the slice; see v_pair_selector
      st.v[e][0] = *reinterpret_cast<const uint32_t*>(lds + S::kOffV + r * S::VR +
                                                     ((c.n * VBY) & ~3));
    else
      load_bytes<VBY>(lds + S::kOffV + r * S::VR + c.n * VBY, st.v[e]);
  }
}

// Dynamic work claiming inside one segment.  Two waves share each SIMD and
// the older one issues first, so with a fixed split the younger wave of every
// SIMD ends several microseconds behind.  Instead the workgroup's share of a
// segment is handed out one 32-token step at a time: each wave starts on a
// few steps of its own, then claims the following steps from a counter in
// LDS shared by the workgroup's waves of the same (layer, seq, head).  A
// claim is issued ahead of its use, so the LDS atomic's latency stays hidden.
struct Claim {
  int* ctr;  // LDS counter; nullptr: the wave takes the whole segment itself
  int wave;  // this wave's index among the waves sharing the counter
  int nw;    // waves sharing the counter
};
// Next step from the counter (claims start after the statically taken ones);
// issued by lane 0, meaningful in lane 0 (read with readlane).
__device__ inline int claim_step(const Claim& cl, int lane, int base) {
  int r = 0;
  if (lane == 0)
    r = base + __hip_atomic_fetch_add(cl.ctr, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
  return r;
}

// One segment [x0, x1) of rows of one format, rows starting at plane row
// row0 (K and V share row numbering).  KB/VB: stored widths (16 = bf16).
// With cl.ctr set the wave processes the steps it claims of the segment,
// otherwise all of it.  PC: coded K rows with per-channel groups over
// g-token blocks; every step then lies inside one block (row0 is a multiple
// of 32 from the block grid, see wave_range), whose META row is staged with
// the step and folded into Q' whenever the block changes.
template <int D, int NG, int KB, int VB, bool PC = false>
__device__ void run_segment(const Ctx& c, WaveState<D>& ws, int x0, int x1, int64_t row0,
                            bool visual, const Claim& cl, const u32x4 (&qreg)[D / 32],
                            bool& q_pending) {
  constexpr int NB = D / 16;
  constexpr int KR = Fmt<D, KB>::kRowBytes, VR = Fmt<D, VB>::kRowBytes, MR = NG * 4;
  const uint8_t* kp = (visual ? c.kvis : c.ktxt) + row0 * KR;
  const uint8_t* vp = (visual ? c.vvis : c.vtxt) + row0 * VR;
  const uint8_t* kmp = c.kmeta + row0 * MR;
  const uint8_t* vmp = c.vmeta + row0 * MR;

  const int rows = x1 - x0;
  const int nsteps = (rows + 31) / 32;
  auto rows_in = [&](int st) { return min(32, rows - 32 * st); };
  constexpr int VBY = Fmt<D, VB>::kVBytes;
  // Quantised steps are small (~14 VGPRs per lane for INT4/INT2): kDepth of
  // them are in flight from memory into registers while earlier ones go
  // through the wave's LDS stage and compute; the first loads are issued
  // before Q' is built so the latencies overlap.  bf16 steps carry 64 VGPRs
  // of data and load straight into operands.
  constexpr bool kStaged = KB < 16 && VB < 16;
  static_assert(!PC || kStaged, "per-channel K runs on the staged path");
  using S = Stage<D, NG, KB, VB>;
  constexpr int g = D / NG;
  // per-channel K: byte offset of the META row of the block of step st
  auto kmblk = [&](int st) {
    return PC ? uint32_t((row0 + 32 * int64_t(st)) / g) * uint32_t(4 * D) : 0u;
  };
  constexpr int kDepth = S::KP + S::VP <= 48 ? KVQ_RING_DEPTH : 2;
  S g_[kDepth];
  SegPlanes pl;
  if constexpr (kStaged) {
    pl.k = make_rsrc(kp, int64_t(rows) * KR);
    pl.km = PC ? make_rsrc(c.kmeta, c.kmeta_bytes) : make_rsrc(kmp, int64_t(rows) * MR);
    pl.v = make_rsrc(vp, int64_t(rows) * VR);
    pl.vm = make_rsrc(vmp, int64_t(rows) * MR);
#pragma unroll
    for (int k = 0; k < kDepth; ++k) {  // this wave's first steps (taken statically)
      const int st = min(cl.ctr ? cl.wave * kDepth + k : k, nsteps - 1);
      stage_load<D, NG, KB, VB, PC>(pl, st, rows_in(st), c.lane, g_[k], kmblk(st));
    }
  }

  // bf16 rows load straight into operands: the first step goes out now
  const uint32_t vsel_mem = v_pair_selector<D, VB>(0);
  Offs<D, NG, KB, VB> of;
  of.full(c);
  Step<D, KB, VB> sa;
  auto load_direct = [&](int st) {
    const int64_t o = int64_t(st) * 32;
    const int rl = rows_in(st);
    if (rl == 32) {
      load_step<D, NG, KB, VB, false>(kp + o * KR, kmp + o * MR, vp + o * VR, vmp + o * MR, of,
                                      sa);
    } else {
      Offs<D, NG, KB, VB> oc;
      oc.clamped(c, rl);
      load_step<D, NG, KB, VB, true>(kp + o * KR, kmp + o * MR, vp + o * VR, vmp + o * MR, oc,
                                     sa);
    }
  };
  int st_d = cl.ctr ? cl.wave : 0;
  if constexpr (!kStaged) {
    if (st_d < nsteps) load_direct(st_d);
  }
  // the wave's query quarter reaches its LDS slot once the first K/V loads
  // are out, so the two latencies overlap
  if (q_pending) {
#pragma unroll
    for (int k = 0; k < D / 32; ++k) c.qq[k] = qreg[k];
    q_pending = false;
  }

  // the query in the operand layout; coded K rows of a rotated cache meet
  // the rotated query
  u32x4 qop[D / 32];
  u32x4 qlo[PC ? D / 32 : 1];  // per-channel K: low binary16 parts of Q'
  float qsr = 0.0f;
  if constexpr (!PC) {  // per-channel K builds Q' per block, in the loop
    float qv[D / 4];
    unpack_quarter<D>(c, qv);
    if (KB < 16 && visual && c.rotate_k) rotate_quarter<D>(c, qv);
    qsr = build_q<D, NG, KB>(c, qv, qop);
  }
  const float c24 = c.qscale * 16777216.0f;  // 2^24 * qscale

#pragma unroll
  for (int mb = 0; mb < NB; ++mb) ws.o[mb] *= v_inflation<D, VB>(mb);

  if constexpr (kStaged) {
    const uint32_t vsel = v_pair_selector<D, VB>((c.n * VBY) & 3);
    // Ring slot k holds step slot[k]; after a slot's step is staged, the
    // slot is refilled with the next claimed step (or, without a counter,
    // the step kDepth further on).  A wave's steps increase, so once slot 0
    // is past the end so is every later one.  Loads stay unconditional
    // (clamped to the last step) so the compiler's wait counts stay exact.
    const int base = cl.nw * kDepth;
    int slot[kDepth];
#pragma unroll
    for (int k = 0; k < kDepth; ++k) slot[k] = cl.ctr ? cl.wave * kDepth + k : k;
    int pend = cl.ctr ? claim_step(cl, c.lane, base) : kDepth;
    int qblk = -1;  // per-channel K: the block Q' was built for
    while (slot[0] < nsteps) {
#pragma unroll
      for (int k = 0; k < kDepth; ++k) {
        const int cur = slot[k];
        stage_put<D, NG, KB, VB, PC>(c.stage, c.lane, g_[k]);
        const int nxt = __builtin_amdgcn_readlane(pend, 0);
        pend = cl.ctr ? claim_step(cl, c.lane, base) : nxt + 1;
        const int la = min(nxt, nsteps - 1);
        stage_load<D, NG, KB, VB, PC>(pl, la, rows_in(la), c.lane, g_[k], kmblk(la));
        slot[k] = nxt;
        stage_get<D, NG, KB, VB, PC>(c.stage, c, sa);
        if constexpr (PC) {
          const int blk = int((row0 + 32 * int64_t(cur)) / g);
          if (cur < nsteps && blk != qblk) {  // wave-uniform
            qsr = build_q_pc<D, NG, KB>(
                c, reinterpret_cast<const uint32_t*>(c.stage + S::kOffKM), qop, qlo);
            qblk = blk;
          }
        }
        if (cur < nsteps) {
          if constexpr (PC)
            compute_step<D, NG, KB, VB, true>(c, ws, sa, qop, qsr, c24, rows_in(cur), vsel, &qlo);
          else
            compute_step<D, NG, KB, VB>(c, ws, sa, qop, qsr, c24, rows_in(cur), vsel);
        }
      }
    }
  } else {
    // bf16 rows (and bf16 K with quantised V): one claimed step at a time
    // (the next claim flies while a step runs), each loaded straight into
    // operands after the previous one is computed
    int pend = cl.ctr ? claim_step(cl, c.lane, cl.nw) : 1;
    while (st_d < nsteps) {
      compute_step<D, NG, KB, VB>(c, ws, sa, qop, qsr, c24, rows_in(st_d), vsel_mem);
      st_d = __builtin_amdgcn_readlane(pend, 0);
      pend = cl.ctr ? claim_step(cl, c.lane, cl.nw) : st_d + 1;
      if (st_d < nsteps) load_direct(st_d);
    }
  }

#pragma unroll
  for (int mb = 0; mb < NB; ++mb) ws.o[mb] *= 1.0f / v_inflation<D, VB>(mb);
}

// The workgroup's large LDS area: the waves' stages during the loop, their
// outputs o_all[wave][16][D] in the combine, the partials in the merge.
// When both fit side by side (small formats), a wave writes its outputs as
// soon as its own loop ends, while the others still stream; otherwise the
// outputs reuse the stages after a barrier.
template <int D, int NG, int KB, int VB>
struct BigLds {
  static constexpr int kStage = KB < 16 && VB < 16 ? (Stage<D, NG, KB, VB>::kBytes + 15) & ~15 : 0;
  static constexpr int kOAll = kWaves * kMaxGroupRatio * D * 4;
  static constexpr bool kApart = kOAll + kWaves * kStage <= 96 * 1024;
  static constexpr int kStageOff = kApart ? kOAll : 0;  // where the stages start
  static constexpr int kBytes = kApart ? kOAll + kWaves * kStage
                                       : (kOAll > kWaves * kStage ? kOAll : kWaves * kStage);
};

// The launch's scalar arguments, wave-uniform.  The kernel reads them from
// its LDS copy of the argument block: the argument segment itself is a slow
// round trip away, and every scalar load from it in the set-up or the tail
// would sit on the critical path.
struct Launch {
  const uint8_t* cache;
  const uint16_t* q;
  uint16_t* out;
  float* ws_o;
  float* ws_ml;
  int32_t* ws_arrive;
  int64_t Rvis;
  float qscale;
  int G, Gs, Hkv, Hq, B, chunk, max_chunks, seq_off, n_lh, n_seq, rotate_k, k_per_channel;
};
// A device pointer read from LDS, made wave-uniform and marked as a global
// (not generic) address, so accesses through it compile to global or buffer
// instructions rather than flat ones (which would also count against the LDS
// wait counter).
template <class T>
__device__ inline T* uniform_ptr(T* p) {
  const uint64_t v = reinterpret_cast<uint64_t>(p);
  // (readfirstlane returns int: go through uint32_t, or a low word with bit
  // 31 set would be sign-extended over the high word)
  const uint64_t lo = uint32_t(__builtin_amdgcn_readfirstlane(uint32_t(v)));
  const uint64_t hi = uint32_t(__builtin_amdgcn_readfirstlane(uint32_t(v >> 32)));
  return (T*)((__attribute__((address_space(1))) T*)(hi << 32 | lo));
}
__device__ inline int uniform_int(int v) { return __builtin_amdgcn_readfirstlane(v); }

// Decode-time append (kvq_decode_attention_append): stores the bf16 row of
// one text position, plane row `row` of the K and V planes, from the call's
// sources, then waits until the stores are complete, so the wave's loads of
// that row, which follow, read it.  The stores are write-through (system
// scope).  Lanes [0, D/2) take two elements each.
template <int D>
__device__ void append_row(const DecodeArgs& t, const uint8_t* kplane, const uint8_t* vplane,
                           int64_t row, int64_t src, int lane) {
  const int mode = __builtin_amdgcn_readfirstlane(int(t.app_mode));
  if (lane < D / 2) {
#pragma unroll
    for (int X = 0; X < 2; ++X) {
      const uint8_t* sp = uniform_ptr(static_cast<const uint8_t*>(X ? t.app_v : t.app_k));
      uint32_t w;
      if (mode == 1) {
        w = reinterpret_cast<const uint32_t*>(sp + src * 2)[lane];
      } else {
        const float2 f = reinterpret_cast<const float2*>(sp + src * 4)[lane];
        w = pack_bf16(f.x, f.y);  // nearest even, as the quantizer stores bf16 rows
      }
      uint32_t* dst =
          reinterpret_cast<uint32_t*>(const_cast<uint8_t*>(X ? vplane : kplane) + row * (2 * D));
      __hip_atomic_store(dst + lane, w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
    }
  }
  __builtin_amdgcn_s_waitcnt(0);      // the row's stores are complete
  __asm__ volatile("" ::: "memory");  // and the compiler keeps the loads after them
}
__device__ inline Launch launch_scalars(const DecodeArgs& t) {
  Launch L;
  L.cache = uniform_ptr(t.cache);
  L.q = uniform_ptr(t.q);
  L.out = uniform_ptr(t.out);
  L.ws_o = uniform_ptr(t.ws_o);
  L.ws_ml = uniform_ptr(t.ws_ml);
  L.ws_arrive = uniform_ptr(t.ws_arrive);
  const uint64_t rv = uint64_t(t.Rvis);
  L.Rvis = int64_t(uint64_t(uint32_t(uniform_int(int(uint32_t(rv >> 32))))) << 32 |
                   uint32_t(uniform_int(int(uint32_t(rv)))));
  L.qscale = __builtin_bit_cast(float, uniform_int(__builtin_bit_cast(int, t.qscale)));
  L.G = uniform_int(t.G);
  L.Gs = uniform_int(int(t.g_stride));
  L.Hkv = uniform_int(t.Hkv);
  L.Hq = uniform_int(t.Hq);
  L.B = uniform_int(t.B);
  L.chunk = uniform_int(t.chunk);
  L.max_chunks = uniform_int(t.max_chunks);
  L.seq_off = uniform_int(t.seq_off);
  L.n_lh = uniform_int(t.n_lh);
  L.n_seq = uniform_int(t.n_seq);
  L.rotate_k = uniform_int(t.rotate_k);
  L.k_per_channel = uniform_int(t.k_per_channel);
  return L;
}

// Split-K merge of one (layer, seq, head) by the workgroup whose partial
// completed its arrival count: the nxs partials (normalised rows o / l with
// their (m, l)) are combined with the log-sum-exp rule, read past the caches,
// and the arrival counter is reset to zero for the next call.  Uses the
// workgroup's reusable LDS (big_lds) and all its threads; the caller ensures
// no thread still uses that LDS.
template <int D, int kBigBytes>
__device__ void merge_entry(const Launch& a, uint8_t* big_lds, int l_local, int s, int h,
                            int nxs) {
  const int G = a.G;
  const int64_t entry = (int64_t(l_local) * a.B + s) * a.Hkv + h;
  uint16_t* outp = a.out + ((int64_t(l_local) * a.B + s) * a.Hq + int64_t(h) * a.Gs) * D;
  // Merge in LDS: the (m, l) pairs of all partials come in with the first
  // batch of partial rows and become weights w[cx][j] = l 2^(m - M_j) (0 for
  // a partial without tokens); the partial rows (normalised, o / l) stream
  // through in batches, each element accumulating sum_cx o w and sum_cx w.
  // All loads are 16- or 4-byte buffer loads that bypass the caches, issued
  // together.  Entries with more partials than LDS holds read memory directly.
  const int64_t p0 = partial_index(l_local, s, h, 0, a.B, a.Hkv, a.max_chunks);
  const float* gml = a.ws_ml + p0 * G * 2;
  const float* go = a.ws_o + p0 * G * D;
  constexpr int kLdsFloats = kBigBytes / 4;  // the whole stage / o_all area
  constexpr int kPer = (kMaxGroupRatio * D + kThreads - 1) / kThreads;  // elements per thread
  const int n_ml = nxs * G * 2;
  float* lml = reinterpret_cast<float*>(big_lds);  // [nxs][G] (m, l)
  float* lw = lml + n_ml;                           // [nxs][G] weights
  const int lo_off = (3 * nxs * G + 3) & ~3;
  float* lo = lml + lo_off;                         // partial rows of the current batch
  const int room = kLdsFloats - lo_off;
  float acc[kPer], wsum[kPer];
#pragma unroll
  for (int k = 0; k < kPer; ++k) {
    acc[k] = 0.0f;
    wsum[k] = 0.0f;
  }
  if (room >= G * D) {
    const int kBatch = room / (G * D);
    const Rsrc rm = make_rsrc(gml, int64_t(n_ml) * 4);
    for (int c0 = 0; c0 < nxs; c0 += kBatch) {
      const int nb = min(kBatch, nxs - c0);
      const int n_o = nb * G * D;
      const Rsrc ro = make_rsrc(go + int64_t(c0) * G * D, int64_t(n_o) * 4);
      if (c0 > 0) __syncthreads();  // the previous batch is consumed
      // Every load of a pass is issued before the first LDS store, so a batch
      // costs one memory round trip per kU * kThreads vectors (the (m, l)
      // pairs, with the first batch, ride along with the first pass).
      constexpr int kU = 4;
      const int n_v = n_o / 4;
      float mlr[2] = {0.0f, 0.0f};
      for (int v0 = 0; v0 < n_v; v0 += kU * kThreads) {
        u32x4 buf[kU];
#pragma unroll
        for (int k = 0; k < kU; ++k) {
          const int v = v0 + int(threadIdx.x) + kThreads * k;
          if (v < n_v) buf[k] = __builtin_amdgcn_raw_buffer_load_b128(ro, uint32_t(v) * 16u, 0, kCoherent);
        }
        if (c0 == 0 && v0 == 0) {
#pragma unroll
          for (int k = 0; k < 2; ++k) {
            const int i = int(threadIdx.x) + kThreads * k;
            if (i < n_ml)
              mlr[k] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                                     rm, uint32_t(i) * 4u, 0, kCoherent));
          }
        }
#pragma unroll
        for (int k = 0; k < kU; ++k) {
          const int v = v0 + int(threadIdx.x) + kThreads * k;
          if (v < n_v) reinterpret_cast<u32x4*>(lo)[v] = buf[k];
        }
      }
      if (c0 == 0) {  // the (m, l) pairs travel with the first batch
#pragma unroll
        for (int k = 0; k < 2; ++k) {
          const int i = int(threadIdx.x) + kThreads * k;
          if (i < n_ml) lml[i] = mlr[k];
        }
        for (int i = int(threadIdx.x) + 2 * kThreads; i < n_ml; i += kThreads)
          lml[i] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                                 rm, uint32_t(i) * 4u, 0, kCoherent));
        __syncthreads();
        // one thread per (partial cx, head j): M_j over all partials (every
        // thread of head j reads the same pairs), then its own weight; the
        // partial rows are normalised (o / l), so the weight is l 2^(m - M_j)
        for (int t = threadIdx.x; t < nxs * G; t += kThreads) {
          const int j = t % G;
          float M = -INFINITY;
#pragma unroll 8
          for (int cx = 0; cx < nxs; ++cx) {
            const float2 ml = reinterpret_cast<const float2*>(lml)[cx * G + j];
            M = ml.y > 0.0f ? fmaxf(M, ml.x) : M;
          }
          const float2 me = reinterpret_cast<const float2*>(lml)[t];
          lw[t] = me.y > 0.0f ? me.y * __builtin_amdgcn_exp2f(me.x - M) : 0.0f;
        }
      }
      __syncthreads();
#pragma unroll
      for (int k = 0; k < kPer; ++k) {
        const int i = threadIdx.x + kThreads * k;
        if (i < G * D) {
          const int j = i / D;
#pragma unroll 4
          for (int cx = 0; cx < nb; ++cx) {
            const float wgt = lw[(c0 + cx) * G + j];
            acc[k] += lo[cx * G * D + i] * wgt;
            wsum[k] += wgt;
          }
        }
      }
    }
#pragma unroll
    for (int k = 0; k < kPer; ++k) acc[k] *= __builtin_amdgcn_rcpf(wsum[k]);
  } else {
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
      const int i = threadIdx.x + kThreads * k;
      if (i >= G * D) break;
      const int j = i / D;
      auto ld = [&](const float* p) {
        return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
      };
      float M = -INFINITY;
      for (int cx = 0; cx < nxs; ++cx)
        M = ld(&gml[(cx * G + j) * 2 + 1]) > 0.0f ? fmaxf(M, ld(&gml[(cx * G + j) * 2])) : M;
      float L = 0.0f, A = 0.0f;
      for (int cx = 0; cx < nxs; ++cx) {
        const float lx = ld(&gml[(cx * G + j) * 2 + 1]);
        const float wgt =
            lx > 0.0f ? lx * __builtin_amdgcn_exp2f(ld(&gml[(cx * G + j) * 2]) - M) : 0.0f;
        L += wgt;
        A += lx > 0.0f ? wgt * ld(&go[int64_t(cx) * G * D + i]) : 0.0f;
      }
      acc[k] = A * __builtin_amdgcn_rcpf(L);
    }
  }
#pragma unroll
  for (int k = 0; k < kPer; ++k) {
    const int i = threadIdx.x + kThreads * k;
    if (i < G * D) outp[i] = __builtin_bit_cast(uint16_t, (__bf16)acc[k]);
  }
  if (threadIdx.x == 0)
    __hip_atomic_store(&a.ws_arrive[entry], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
}

// Split-K merge, wave-parallel form.  The m entries a workgroup completed
// are spread over its waves: wave w merges entry w % m, slice w / m of that
// entry's G * D outputs, so several merges run side by side with no
// workgroup barrier and no LDS.  A lane holds one 16-byte vector of outputs
// per t < kWmT and reads that vector of each of the entry's nxs partials
// together with the (m, l) pair of the vector's head in each partial, all
// loads issued before the first use: one memory round trip and no
// cross-lane traffic.  Entries whose partials do not fit that (nxs > kWmX or
// more than kWmT vectors per lane) go through merge_entry instead.
// Two instances: up to 8 partials (the common case) and up to 16 (a small
// call's 512-token chunks of a 6K-token sequence); the wider one's guarded
// loads and loops cost about 0.5 us on entries the narrow one fits.
constexpr int kWmX = 16, kWmT = 2;
__device__ inline bool wave_merge_fits(int nxs, int G, int D, int waves) {
  const int per_wave = (G * D / 4 + waves - 1) / waves;  // 16-byte vectors per wave
  return nxs <= kWmX && per_wave <= 64 * kWmT;
}
template <int D, int kX>
__device__ void merge_entry_wave(const Launch& a, int l_local, int s, int h, int nxs,
                                 int slice, int waves, int lane) {
  const int G = a.G;
  const int64_t entry = (int64_t(l_local) * a.B + s) * a.Hkv + h;
  const int64_t p0 = partial_index(l_local, s, h, 0, a.B, a.Hkv, a.max_chunks);
  const int nv = G * D / 4;
  const int per_wave = (nv + waves - 1) / waves;
  const int v_lo = slice * per_wave, v_hi = min(nv, v_lo + per_wave);
  const int nt = min(kWmT, (v_hi - v_lo + 63) / 64);  // vector slots this wave uses
  const Rsrc ro = make_rsrc(a.ws_o + p0 * G * D, int64_t(nxs) * G * D * 4);
  const Rsrc rm = make_rsrc(a.ws_ml + p0 * G * 2, int64_t(nxs) * G * 8);
  u32x4 buf[kWmT][kX];
  u32x2 mlv[kWmT][kX];
#pragma unroll
  for (int t = 0; t < kWmT; ++t) {
    const int v = v_lo + lane + 64 * t;
    const int j = min(4 * v / D, G - 1);  // head of this vector (clamped for idle lanes)
#pragma unroll
    for (int cx = 0; cx < kX; ++cx)
      if (t < nt && v < v_hi && cx < nxs) {
        buf[t][cx] = __builtin_amdgcn_raw_buffer_load_b128(
            ro, uint32_t(cx * G * D + 4 * v) * 4u, 0, kCoherent);
        mlv[t][cx] = __builtin_amdgcn_raw_buffer_load_b64(rm, uint32_t(cx * G + j) * 8u, 0,
                                                          kCoherent);
      }
  }
  uint16_t* outp = a.out + ((int64_t(l_local) * a.B + s) * a.Hq + int64_t(h) * a.Gs) * D;
#pragma unroll
  for (int t = 0; t < kWmT; ++t) {
    if (t >= nt) break;
    const int v = v_lo + lane + 64 * t;
    if (v < v_hi) {
      // weights l 2^(m - M) of the partials of this vector's head (0 for
      // one without tokens)
      float mj[kX], lj[kX];
      float M = -INFINITY;
#pragma unroll
      for (int cx = 0; cx < kX; ++cx) {
        // (each element as a value: bit_cast of a vector element reference
        // reads element 0)
        mj[cx] = cx < nxs ? __builtin_bit_cast(float, uint32_t(mlv[t][cx][0])) : 0.0f;
        lj[cx] = cx < nxs ? __builtin_bit_cast(float, uint32_t(mlv[t][cx][1])) : 0.0f;
        if (lj[cx] > 0.0f) M = fmaxf(M, mj[cx]);
      }
      f32x4 acc = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
      float wsum = 0.0f;
#pragma unroll
      for (int cx = 0; cx < kX; ++cx) {
        if (lj[cx] > 0.0f) {
          const float w = lj[cx] * __builtin_amdgcn_exp2f(mj[cx] - M);
          wsum += w;
#pragma unroll
          for (int e = 0; e < 4; ++e)  // (the element as a value: bit_cast of a vector
                                        // element reference reads element 0)
            acc[e] += __builtin_bit_cast(float, uint32_t(buf[t][cx][e])) * w;
        }
      }
      const float r = __builtin_amdgcn_rcpf(wsum);
      uint2 o;
      o.x = uint32_t(__builtin_bit_cast(uint16_t, (__bf16)(acc[0] * r))) |
            (uint32_t(__builtin_bit_cast(uint16_t, (__bf16)(acc[1] * r))) << 16);
      o.y = uint32_t(__builtin_bit_cast(uint16_t, (__bf16)(acc[2] * r))) |
            (uint32_t(__builtin_bit_cast(uint16_t, (__bf16)(acc[3] * r))) << 16);
      *reinterpret_cast<uint2*>(outp + 4 * v) = o;
    }
  }
  if (slice == 0 && lane == 0)
    __hip_atomic_store(&a.ws_arrive[entry], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
}

// One instance per (D, groups per row, visual K/V widths): a launch holds
// only (layer, head) pairs whose visual rows have widths (KB, VB) or are bf16
// (protected heads), so each instance carries two row paths -- the quantised
// one and the bf16 one that text rows use anyway -- and nothing else.
//
// Work layout: the launch's units are waves (see DecodeArgs::mult) and
// workgroup b runs units [8b, 8b + 8).  The waves of a workgroup that belong
// to one (layer, seq, head) form a piece: they share a claim counter, and
// their results are combined in LDS into one partial, or into the output when
// the piece is the whole entry.  The piece that completes an entry's arrival
// count merges the entry's partials.
template <int D, int NG, int KB, int VB, bool PC>
__global__ __launch_bounds__(kThreads, 1) void decode_mfma_kernel(DecodeArgs a) {
  constexpr int NB = D / 16;
  constexpr int g = D / NG;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform

  // The per-slot / per-sequence tables are indexed by values computed here.
  // One cooperative 16-byte pass copies the whole argument block to LDS; the
  // launch's sequence lengths are loaded in the same round trip.
  static_assert(sizeof(DecodeArgs) % 16 == 0, "argument block copied in 16-byte pieces");
  constexpr int kArgVec = int(sizeof(DecodeArgs) / 16);
  static_assert(kArgVec <= kThreads, "one 16-byte piece per thread");
  __shared__ uint4 args_lds[kArgVec];
  __shared__ int lds_claim[kWaves];  // per piece (by its first wave): claim counter
  __shared__ int lens_lds[kMaxSeq];  // attended lengths of the launch's sequences
  __shared__ unsigned lead_lds, split_lds;  // pieces by lowest wave; any split piece
  {
    // branch-free, so both loads go out before the first wait
    const uint4* src = (const uint4*)(__builtin_amdgcn_kernarg_segment_ptr());
    const int ti = int(threadIdx.x);
    const uint4 v = src[min(ti, kArgVec - 1)];
    const int len_v = a.seq_lens[a.seq_off + min(min(ti, kMaxSeq - 1), a.n_seq - 1)];
    if (ti < kWaves) lds_claim[ti] = 0;
    if (ti == 0) lead_lds = split_lds = 0u;
    if (ti < kArgVec) args_lds[ti] = v;
    if (ti < kMaxSeq) lens_lds[ti] = len_v;
  }
  __syncthreads();
  const DecodeArgs& t = *reinterpret_cast<const DecodeArgs*>(args_lds);
  const Launch La = launch_scalars(t);

  // Lane-parallel copies of the launch tables: lane l holds slots l and l + 64
  // and sequence l, read in one batch of independent LDS reads.  Every lookup
  // below is then a ballot or a readlane, not a chain of dependent reads.
  static_assert(kMaxLH <= 128 && kMaxSeq <= 64, "two lanes' worth of slots, one of sequences");
  const int n_lh = La.n_lh, n_seq = La.n_seq;
  const int sA = lane, sB = min(lane + 64, kMaxLH - 1);
  const int mcA = t.mcum[sA], mcB = t.mcum[sB];
  const int mA = t.mult[sA], mB = t.mult[sB];
  const int lhA = t.lh_glob[sA], lhB = t.lh_glob[sB];
  const int bitsA = int(t.bits[sA][0]) | int(t.bits[sA][1]) << 8;
  const int bitsB = int(t.bits[sB][0]) | int(t.bits[sB][1]) << 8;
  const uint32_t kbaseA = t.base256[sA][0], kbaseB = t.base256[sB][0];
  const uint32_t vbaseA = t.base256[sA][1], vbaseB = t.base256[sB][1];
  const int nxc = t.nxcum[lane], nxl = t.nxcum[lane + 1] - nxc;  // nxcum has kMaxSeq + 1 entries
  const int vbl = t.vb[lane], vel = t.ve[lane], capl = t.cap[lane];
  const int vr0l = t.vrow0[lane], tr0l = t.trow0[lane], lenl = lens_lds[lane];
  const int per_mult = t.nxcum[n_seq];  // units of one slot with mult 1
  auto pick = [&](int vA, int vB, int i) {  // slot table value of (uniform) slot i
    return __builtin_amdgcn_readlane(i < 64 ? vA : vB, i & 63);
  };
  // unit b (wave-uniform) -> slot, sequence index within the launch and x,
  // the unit's index among the mult[slot] * nx[seq] units of that pair
  auto unit_of = [&](int b, int& slot_, int& sl_, int& x_) {
    const int cA = __builtin_popcountll(__ballot(lane < n_lh && per_mult * mcA <= b));
    const int cB = __builtin_popcountll(__ballot(lane + 64 < n_lh && per_mult * mcB <= b));
    slot_ = __builtin_amdgcn_readfirstlane(cA + cB - 1);
    const int m = pick(mA, mB, slot_);
    const int r = b - per_mult * pick(mcA, mcB, slot_);
    sl_ = __builtin_amdgcn_readfirstlane(
        __builtin_popcountll(__ballot(lane < n_seq && m * nxc <= r)) - 1);
    x_ = r - m * __builtin_amdgcn_readlane(nxc, sl_);
  };

  // this wave's unit -> (slot, sequence, index u among the entry's ne units).
  // Units b8 + r (positions r) are dealt to the waves so that every piece
  // gets older and younger waves alike: the two waves sharing a SIMD
  // (w, w + 4) do not issue evenly (the older one goes first), and the waves
  // of a piece rebalance only among themselves.  Positions follow the order
  // of waves 0, 4, 1, 5, ...; when the first piece is longer than half the
  // workgroup the positions are rotated so the short piece after it starts at
  // wave 0.
  const int b8 = int(blockIdx.x) * kWaves;
  const int total = per_mult * t.mcum[n_lh];  // the last block may be short
  int rot = 0;
  auto pos_of = [&](int w) { return ((((w & 3) << 1) | (w >> 2)) + rot) & (kWaves - 1); };
  {
    // the first piece's length (units of the block's first entry)
    int s0, l0, u0;
    unit_of(b8, s0, l0, u0);
    const int first = min(kWaves, __builtin_amdgcn_readlane(nxl, l0) * pick(mA, mB, s0) - u0);
    rot = __builtin_amdgcn_readfirstlane(first > kWaves / 2 && first < kWaves ? first : 0);
  }
  int slot = 0, sl = 0, u = 0;
  if (b8 + pos_of(wave) < total) unit_of(b8 + pos_of(wave), slot, sl, u);
  const int pos = pos_of(wave);
  const int gw = b8 + pos;
  const bool active = gw < total;
  const int ne = __builtin_amdgcn_readfirstlane(__builtin_amdgcn_readlane(nxl, sl) *
                                                pick(mA, mB, slot));
  const int w0 = gw - u;  // the entry's first unit
  // the piece: positions [p_lo, p_hi) of this workgroup, i.e. the waves of
  // pmask; the entry's piece px of pn (idle waves form no piece)
  const int p_lo = active ? max(w0, b8) - b8 : 0;
  const int p_hi = active ? min(w0 + ne, b8 + kWaves) - b8 : 0;
  unsigned pmask = 0;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) pmask |= pos_of(w) >= p_lo && pos_of(w) < p_hi ? 1u << w : 0u;
  const int px = int(blockIdx.x) - w0 / kWaves;
  const int pn = (w0 + ne - 1) / kWaves - w0 / kWaves + 1;
  const int lh = __builtin_amdgcn_readfirstlane(pick(lhA, lhB, slot));
  const int l_local = lh / La.Hkv, h = lh % La.Hkv;
  const int s = La.seq_off + sl;
  // piece table for the combine, written now so it is off the tail's path
  __shared__ int winfo[kWaves][8];  // per wave: pmask, -, l_local, s, h, px, pn
  if (lane < 7) winfo[wave][lane] = lane == 0 ? int(pmask) : lane == 1 ? 0 : lane == 2 ? l_local
                                    : lane == 3 ? s : lane == 4 ? h : lane == 5 ? px : pn;
  if (lane == 0 && pmask != 0u && __builtin_ctz(pmask) == wave) {
    __hip_atomic_fetch_or(&lead_lds, 1u << wave, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    if (pn > 1) __hip_atomic_fetch_or(&split_lds, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
  }
  const int cap = __builtin_amdgcn_readlane(capl, sl);
  const int G = La.G;

  __shared__ float ml_lds[kWaves][16][2];
  using Big = BigLds<D, NG, KB, VB>;
  __shared__ __attribute__((aligned(16))) uint8_t big_lds[Big::kBytes];

  // quarter jq of the query of column n's head (head 0 for dead columns):
  // D/4 bf16, 16-byte aligned, loaded now and parked in the lane's own LDS
  // slot once the first K/V loads are out (only this lane reads it back)
  Ctx c;
  __shared__ __attribute__((aligned(16))) u32x4 q_lds[kWaves][64][D / 32];
  u32x4 qreg[D / 32];
  {
    const int qh = (lane & 15) < G * NG ? (lane & 15) / NG : 0;
    const uint16_t* qp = La.q + ((int64_t(l_local) * La.B + s) * La.Hq + int64_t(h) * La.Gs + qh) * D +
                         (lane >> 4) * (D / 4);
#pragma unroll
    for (int k = 0; k < D / 32; ++k)
      qreg[k] = active ? reinterpret_cast<const u32x4*>(qp)[k] : u32x4{0, 0, 0, 0};
  }
  c.qq = q_lds[wave][lane];
  bool q_pending = true;
  int len = __builtin_amdgcn_readlane(lenl, sl);
  len = len < 1 ? 1 : (len > cap ? cap : len);

  const int bits2 = pick(bitsA, bitsB, slot);
  const int kbits = bits2 & 0xFF;
  const int vbits = bits2 >> 8;
  {
    const int kb = kbits, vb = vbits;
    c.kvis = La.cache + uint64_t(uint32_t(pick(int(kbaseA), int(kbaseB), slot))) * 256u;
    c.kmeta = c.kvis + meta_plane_offset(La.Rvis, D, kb);
    c.ktxt = c.kvis + txt_plane_offset(La.Rvis, D, g, kb);
    c.vvis = La.cache + uint64_t(uint32_t(pick(int(vbaseA), int(vbaseB), slot))) * 256u;
    c.vmeta = c.vvis + meta_plane_offset(La.Rvis, D, vb);
    c.vtxt = c.vvis + txt_plane_offset(La.Rvis, D, g, vb);
  }
  c.stage = big_lds + Big::kStageOff + wave * Big::kStage;
  c.qscale = La.qscale;
  c.G = G;
  c.rotate_k = La.rotate_k != 0;
  c.kmeta_bytes = La.Rvis * (D / g) * 4;
  const bool kpc = PC;  // launches of per-channel caches use the PC instances
  c.lane = lane;
  c.n = lane & 15;
  c.jq = lane >> 4;

  WaveState<D> st;
#pragma unroll
  for (int mb = 0; mb < NB; ++mb) st.o[mb] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  st.m = -INFINITY;
  st.l = 0.0f;
  st.mt = 0.0f;

  if (active) {
    // static split: chunk mode gives each workgroup (8 units) one chunk,
    // the balanced mode deals the entry's steps over its ne units
    const int vb = __builtin_amdgcn_readlane(vbl, sl);
    // per-channel K: shift the step grid so steps of the coded span start on
    // multiples of 32 from vis_begin (each then lies inside one block)
    const int phase = kpc ? (32 - vb % 32) % 32 : 0;
    int wa, wb;
    if (La.chunk > 0)
      wave_range(u / kWaves, u % kWaves, ne / kWaves, len, La.chunk, kWaves, wa, wb, phase);
    else
      wave_range(u, 0, ne, len, 0, 1, wa, wb, phase);
    const int ve = __builtin_amdgcn_readlane(vel, sl);
    const int64_t vrow0 = __builtin_amdgcn_readlane(vr0l, sl);
    const int64_t trow0 = __builtin_amdgcn_readlane(tr0l, sl);
    const bool quant_vis = !(KB == 16 && VB == 16) && kbits == KB && vbits == VB;
    // bf16 ranges of this sequence inside its coded span (rows of the text
    // plane); a sequence with ranges takes the static split
    const int r_lo = __builtin_amdgcn_readfirstlane(int(t.rng_first[sl]));
    const int nr = __builtin_amdgcn_readfirstlane(int(t.rng_first[sl + 1])) - r_lo;
    int range_total = 0;  // positions of the span inside bf16 ranges
#pragma clang loop unroll(disable)
    for (int k = 0; k < nr; ++k) range_total += t.rng_e[r_lo + k] - t.rng_b[r_lo + k];
    range_total = __builtin_amdgcn_readfirstlane(range_total);
    // In a balanced split the piece's visual rows (the union of its waves'
    // static ranges) are claimed step by step by its waves, and the entry's
    // text rows all go to one unit of its largest piece (text_unit), first,
    // so the claimed part absorbs them; in the fixed chunk mode and for a
    // sequence with bf16 ranges every row follows the static split [wa, wb).
    const bool dyn = La.chunk == 0 && nr == 0;
    const bool txt_mine = u == text_unit(w0, ne, kWaves);
    int ga, gb, gt;
    wave_range(p_lo + b8 - w0, 0, ne, len, 0, 1, ga, gt, phase);
    wave_range(p_hi - 1 + b8 - w0, 0, ne, len, 0, 1, gt, gb, phase);
    const Claim cl{&lds_claim[p_lo], pos - p_lo, p_hi - p_lo};
    // segments: 0 text prefix [0, vb), 1 text suffix [ve, cap), then for
    // j = 0 .. 2 nr: coded piece j / 2 (even j) or bf16 range (j - 1) / 2
    // (odd j) of the span; rows are consecutive inside a segment.  Kept as a
    // loop so each row path is emitted once.
    int skipped = 0;  // range positions before the current piece or range
#pragma clang loop unroll(disable)
    for (int seg = 0; seg < 3 + 2 * nr; ++seg) {
      const bool vis = seg >= 2 && ((seg - 2) & 1) == 0;
      int f0, f1;
      int64_t frow;  // plane row of position f0
      if (seg == 0) {
        f0 = 0;
        f1 = vb;
        frow = trow0;
      } else if (seg == 1) {  // text rows before it: vb + range_total
        f0 = ve;
        f1 = cap;
        frow = trow0 + vb + range_total;
      } else {
        const int k = (seg - 2) >> 1;
        if (vis) {
          f0 = k == 0 ? vb : t.rng_e[r_lo + k - 1];
          f1 = k < nr ? t.rng_b[r_lo + k] : ve;
          frow = vrow0 + (f0 - vb) - skipped;
        } else {
          f0 = t.rng_b[r_lo + k];
          f1 = t.rng_e[r_lo + k];
          frow = trow0 + vb + skipped;
          skipped += f1 - f0;
        }
      }
      f0 = __builtin_amdgcn_readfirstlane(f0);
      f1 = __builtin_amdgcn_readfirstlane(f1);
      int x0, x1;
      if (vis && dyn) {
        x0 = max(ga, f0);
        x1 = min(gb, f1);
      } else if (dyn) {  // text prefix or suffix: the attended part, on one unit
        x0 = txt_mine ? min(f0, len) : 0;
        x1 = txt_mine ? min(f1, len) : 0;
      } else {
        x0 = max(wa, f0);
        x1 = min(wb, f1);
      }
      if (x0 >= x1) continue;
      const int64_t row0 = frow + (x0 - f0);
      const Claim use = vis && dyn ? cl : Claim{nullptr, 0, 1};
      if (vis && quant_vis) {
        run_segment<D, NG, KB, VB, PC>(c, st, x0, x1, row0, true, use, qreg, q_pending);
      } else {  // text rows, or bf16 visual rows of a protected head
        // decode-time append: the wave whose static rows hold the last
        // attended position stores that position's row first (text
        // positions: the prefix, the suffix and bf16 ranges)
        if (t.app_mode != 0 && !vis && x0 <= len - 1 && len - 1 < x1)
          append_row<D>(t, c.ktxt, c.vtxt, row0 + (len - 1 - x0),
                        ((int64_t(l_local) * La.B + s) * La.Hkv + h) * D, lane);
        run_segment<D, NG, 16, 16>(c, st, x0, x1, row0, vis, use, qreg, q_pending);
      }
    }
  }

  // ---- wave results -> LDS ---------------------------------------------------
  // Row c of every wave's p.v accumulator (column (head, group) c of S) goes
  // to o_all[wave][c][d] with the V-min term added; (m, l) per column to
  // ml_all.  Rows of dead columns and the other groups' d are written too
  // and simply never read.  An idle wave writes zeros and l = 0.
  if constexpr (!Big::kApart) __syncthreads();  // the stages are reused as o_all below
  float l_col = st.l + __shfl_xor(st.l, 16);
  l_col += __shfl_xor(l_col, 32);
  float mt_col = st.mt + __shfl_xor(st.mt, 16);
  mt_col += __shfl_xor(mt_col, 32);
  const int n = lane & 15, jq = lane >> 4;
  float(*o_all)[16][D] = reinterpret_cast<float(*)[16][D]>(big_lds);
  if (jq == 0) {
    ml_lds[wave][n][0] = st.m;
    ml_lds[wave][n][1] = l_col;
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float mt_r = __shfl(mt_col, 4 * jq + i);
    f32x4 v[NB / 4];
#pragma unroll
    for (int mb = 0; mb < NB; ++mb) v[mb / 4][mb % 4] = st.o[mb][i] + mt_r;
#pragma unroll
    for (int k = 0; k < NB / 4; ++k)
      reinterpret_cast<f32x4*>(&o_all[wave][4 * jq + i][NB * n])[k] = v[k];
  }
  __syncthreads();

  // ---- combine each piece's waves; write its partial (or the output) --------
  // Every output element is a weighted sum over its piece's waves: wave w's
  // weight is f_w = 2^(m_w - M) against the piece's maximum M (0 for a wave
  // without tokens), and L = sum l_w f_w.  Each thread forms the weights of
  // its own row from the (m, l) pairs, so one barrier separates the waves'
  // writes from the combine.  Head j's value at d lives in row
  // c = j * NG + (d / g).  The pieces are combined side by side: wave w
  // takes piece w % np (np pieces, by their lowest waves) and slice w / np of
  // its G * D / 4 vectors, so a workgroup holding two pieces spends one pass,
  // not two.
  const unsigned lead = __builtin_amdgcn_readfirstlane(lead_lds);
  const bool any_split = __builtin_amdgcn_readfirstlane(split_lds) != 0u;
  const int GD = G * D;
  if (lead != 0u) {
    const int np = __popc(lead);
    const int kk = wave % np;
    unsigned rest = lead;
    for (int i = 0; i < kk; ++i) rest &= rest - 1u;
    const int wl = __builtin_ctz(rest);
    const int slice = wave / np, nslices = (kWaves - kk + np - 1) / np;
    const unsigned pm = __builtin_amdgcn_readfirstlane(winfo[wl][0]);
    const int pl = __builtin_amdgcn_readfirstlane(winfo[wl][2]);
    const int ps = __builtin_amdgcn_readfirstlane(winfo[wl][3]);
    const int ph = __builtin_amdgcn_readfirstlane(winfo[wl][4]);
    const int ppx = __builtin_amdgcn_readfirstlane(winfo[wl][5]);
    const int ppn = __builtin_amdgcn_readfirstlane(winfo[wl][6]);
    const int64_t pidx = partial_index(pl, ps, ph, ppx, La.B, La.Hkv, La.max_chunks);
    uint16_t* outp = La.out + ((int64_t(pl) * La.B + ps) * La.Hq + int64_t(ph) * La.Gs) * D;
    // four consecutive outputs per thread (one head, one group: D and g are
    // multiples of 4): 16-byte LDS reads and one 16-byte store
    const Rsrc rpo = make_rsrc(La.ws_o + pidx * GD, int64_t(GD) * 4);
    for (int i4 = slice * 64 + lane; i4 < GD / 4; i4 += nslices * 64) {
      const int i = 4 * i4;
      const int j = i / D, d = i % D, cr = j * NG + d / g;
      // every LDS read up front (one round trip); the selects below stay
      // branch-free
      float2 ml[kWaves];
      f32x4 ov[kWaves];
#pragma unroll
      for (int v = 0; v < kWaves; ++v) {
        ml[v] = *reinterpret_cast<const float2*>(ml_lds[v][cr]);
        ov[v] = *reinterpret_cast<const f32x4*>(&o_all[v][cr][d]);
      }
      float M = -INFINITY;
#pragma unroll
      for (int v = 0; v < kWaves; ++v)
        M = (((pm >> v) & 1u) != 0u && ml[v].y > 0.0f) ? fmaxf(M, ml[v].x) : M;
      float L = 0.0f;
      f32x4 acc = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int v = 0; v < kWaves; ++v) {
        const float f = (((pm >> v) & 1u) != 0u && ml[v].y > 0.0f)
                            ? __builtin_amdgcn_exp2f(ml[v].x - M) : 0.0f;
        L += ml[v].y * f;
        acc += ov[v] * f;
      }
      const float rl = L > 0.0f ? __builtin_amdgcn_rcpf(L) : 0.0f;  // 0: no token here
      const f32x4 o = acc * rl;
      if (ppn == 1) {
        uint2 ob;
        ob.x = uint32_t(__builtin_bit_cast(uint16_t, (__bf16)o[0])) |
               (uint32_t(__builtin_bit_cast(uint16_t, (__bf16)o[1])) << 16);
        ob.y = uint32_t(__builtin_bit_cast(uint16_t, (__bf16)o[2])) |
               (uint32_t(__builtin_bit_cast(uint16_t, (__bf16)o[3])) << 16);
        *reinterpret_cast<uint2*>(outp + i) = ob;
      } else {
        // write-through (system-coherent) store: the merging workgroup may
        // sit on another XCD and reads it past its own caches
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, o), rpo,
                                               uint32_t(i) * 4u, 0, kCoherent);
        if (d == 0) {
          __hip_atomic_store(&La.ws_ml[(pidx * G + j) * 2 + 0], M, __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_SYSTEM);
          __hip_atomic_store(&La.ws_ml[(pidx * G + j) * 2 + 1], L, __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_SYSTEM);
        }
      }
    }
  }
  if (!any_split) return;

  // ---- split-K merge by the last piece of each (layer, seq, head) -----------
  // Each workgroup waits until its partials have reached memory, then counts
  // each split piece in; the piece that completes its entry's count has this
  // workgroup merge that entry.  No cache write-back or invalidation is
  // needed.
  __shared__ int is_last[kWaves];
  __builtin_amdgcn_s_waitcnt(0);  // this wave's partial stores are complete
  __syncthreads();
  // the lowest wave of each split piece counts the piece in, with its own
  // (wave-uniform) entry
  if (lane == 0) {
    int last = 0;
    if (((lead >> wave) & 1u) && pn > 1) {
      const int64_t entry = (int64_t(l_local) * La.B + s) * La.Hkv + h;
      last = __hip_atomic_fetch_add(&La.ws_arrive[entry], 1, __ATOMIC_RELAXED,
                                    __HIP_MEMORY_SCOPE_SYSTEM) == pn - 1;
    }
    is_last[wave] = last;
  }
  __syncthreads();
  // the entries this workgroup completed (by their pieces' lowest waves)
  unsigned done = 0u;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) done |= is_last[w] != 0 ? 1u << w : 0u;
  done = __builtin_amdgcn_readfirstlane(done);
  if (done == 0u) return;
  {
    const int m = __popc(done);
    bool fits = true;
    int k = 0;
    for (unsigned rest = done; rest != 0u; rest &= rest - 1u, ++k) {
      const int w = __builtin_ctz(rest);
      fits = fits && wave_merge_fits(winfo[w][6], G, D, (kWaves - k + m - 1) / m);
    }
    if (__builtin_amdgcn_readfirstlane(int(fits))) {
      // wave `wave` takes the (wave % m)-th completed entry, slice wave / m
      const int kk = wave % m;
      unsigned rest = done;
      for (int i = 0; i < kk; ++i) rest &= rest - 1u;
      const int w = __builtin_ctz(rest);
      const int el = __builtin_amdgcn_readfirstlane(winfo[w][2]);
      const int es = __builtin_amdgcn_readfirstlane(winfo[w][3]);
      const int eh = __builtin_amdgcn_readfirstlane(winfo[w][4]);
      const int en = __builtin_amdgcn_readfirstlane(winfo[w][6]);
      if (en <= 8)
        merge_entry_wave<D, 8>(La, el, es, eh, en, wave / m, (kWaves - kk + m - 1) / m, lane);
      else
        merge_entry_wave<D, kWmX>(La, el, es, eh, en, wave / m, (kWaves - kk + m - 1) / m, lane);
      return;
    }
  }
  bool first_merge = true;
#pragma clang loop unroll(disable)
  for (unsigned rest = lead; rest != 0u; rest &= rest - 1u) {
    const int w = __builtin_ctz(rest);
    if (__builtin_amdgcn_readfirstlane(is_last[w])) {
      if (!first_merge) __syncthreads();  // the previous merge is done with the LDS
      first_merge = false;
      merge_entry<D, Big::kBytes>(La, big_lds, __builtin_amdgcn_readfirstlane(winfo[w][2]),
                     __builtin_amdgcn_readfirstlane(winfo[w][3]),
                     __builtin_amdgcn_readfirstlane(winfo[w][4]),
                     __builtin_amdgcn_readfirstlane(winfo[w][6]));
    }
  }
}

}  // namespace

#if !defined(KVQ_MFMA_PART) || KVQ_MFMA_PART == 0
bool mfma_supported(int D, int g, int G) {
  return (D == 64 || D == 128) && G * (D / g) <= 16;
}
int mfma_subgroups(int D, int g, int G) {
  if (!(D == 64 || D == 128) || g < 32 || D % g) return 0;
  return (G * (D / g) + 15) / 16;
}
#endif

// The instances are spread over parts so a build can compile them in
// parallel (-DKVQ_MFMA_PART=0..4, one object each); without the macro one
// object holds every part.
#define KVQ_LAUNCH(DD, NN, K, V)                                                           \
  if (kb == K && vb == V && !pc) {                                                         \
    hipLaunchKernelGGL((decode_mfma_kernel<DD, NN, K, V, false>), grid, dim3(kThreads), 0, \
                       stream, a);                                                         \
    return hipGetLastError();                                                              \
  }
// per-channel K instances exist for coded K with coded V only
#define KVQ_LAUNCH_PC(DD, NN, K, V)                                                        \
  if (kb == K && vb == V && pc) {                                                          \
    hipLaunchKernelGGL((decode_mfma_kernel<DD, NN, K, V, true>), grid, dim3(kThreads), 0,  \
                       stream, a);                                                         \
    return hipGetLastError();                                                              \
  }
#define KVQ_PART_FN(DD, NN)                                                                 \
  hipError_t launch_decode_mfma_##DD##_##NN(const DecodeArgs& a, int kb, int vb,           \
                                            hipStream_t stream) {                           \
    /* one workgroup per kWaves units (waves) of the compact unit list */                \
    const dim3 grid((a.nxcum[a.n_seq] * a.mcum[a.n_lh] + kWaves - 1) / kWaves, 1, 1);      \
    const bool pc = a.k_per_channel != 0;                                                   \
    KVQ_LAUNCH(DD, NN, 2, 2) KVQ_LAUNCH(DD, NN, 2, 4) KVQ_LAUNCH(DD, NN, 2, 8)              \
    KVQ_LAUNCH(DD, NN, 2, 16) KVQ_LAUNCH(DD, NN, 4, 2) KVQ_LAUNCH(DD, NN, 4, 4)             \
    KVQ_LAUNCH(DD, NN, 4, 8) KVQ_LAUNCH(DD, NN, 4, 16) KVQ_LAUNCH(DD, NN, 8, 2)             \
    KVQ_LAUNCH(DD, NN, 8, 4) KVQ_LAUNCH(DD, NN, 8, 8) KVQ_LAUNCH(DD, NN, 8, 16)             \
    KVQ_LAUNCH(DD, NN, 16, 2) KVQ_LAUNCH(DD, NN, 16, 4) KVQ_LAUNCH(DD, NN, 16, 8)           \
    KVQ_LAUNCH(DD, NN, 16, 16)                                                              \
    KVQ_LAUNCH_PC(DD, NN, 2, 2) KVQ_LAUNCH_PC(DD, NN, 2, 4) KVQ_LAUNCH_PC(DD, NN, 2, 8)     \
    KVQ_LAUNCH_PC(DD, NN, 4, 2) KVQ_LAUNCH_PC(DD, NN, 4, 4) KVQ_LAUNCH_PC(DD, NN, 4, 8)     \
    KVQ_LAUNCH_PC(DD, NN, 8, 2) KVQ_LAUNCH_PC(DD, NN, 8, 4) KVQ_LAUNCH_PC(DD, NN, 8, 8)     \
    return hipErrorInvalidValue;                                                            \
  }
#if !defined(KVQ_MFMA_PART) || KVQ_MFMA_PART == 0
KVQ_PART_FN(128, 1)
#endif
#if !defined(KVQ_MFMA_PART) || KVQ_MFMA_PART == 1
KVQ_PART_FN(128, 2)
#endif
#if !defined(KVQ_MFMA_PART) || KVQ_MFMA_PART == 2
KVQ_PART_FN(128, 4)
#endif
#if !defined(KVQ_MFMA_PART) || KVQ_MFMA_PART == 3
KVQ_PART_FN(64, 1)
#endif
#if !defined(KVQ_MFMA_PART) || KVQ_MFMA_PART == 4
KVQ_PART_FN(64, 2)
#endif
#undef KVQ_PART_FN
#undef KVQ_LAUNCH_PC
#undef KVQ_LAUNCH

#if !defined(KVQ_MFMA_PART) || KVQ_MFMA_PART == 0
hipError_t launch_decode_mfma(const DecodeArgs& a, int kb, int vb, hipStream_t stream) {
  const int NG = a.D / a.g;
  if (a.D == 128 && NG == 1) return launch_decode_mfma_128_1(a, kb, vb, stream);
  if (a.D == 128 && NG == 2) return launch_decode_mfma_128_2(a, kb, vb, stream);
  if (a.D == 128 && NG == 4) return launch_decode_mfma_128_4(a, kb, vb, stream);
  if (a.D == 64 && NG == 1) return launch_decode_mfma_64_1(a, kb, vb, stream);
  if (a.D == 64 && NG == 2) return launch_decode_mfma_64_2(a, kb, vb, stream);
  return hipErrorInvalidValue;
}
#endif

}  // namespace kvq
