// kvq_decode_mfma.hip -- split-K decode attention on the CDNA4 matrix cores.
//
// Same contract as the general split kernel (kvq_decode.hip): one workgroup
// per token chunk of one (layer, sequence, KV head); stored rows are
// reconstructed on chip and never written back (gist.science 2604.02570,
// section 2-D: reconstruction fused into flash decoding); K/V widths per
// head and the Visual/Text split follow nuiw.github.io "VLM_KV_Quantization"
// (sections 1-2) and the HeadGuard briefing (bf16 protected heads).
//
// Work of one wave: 32 tokens per step, all contractions on
// v_mfma_f32_16x16x32_{f16,bf16} (wave64, 16x16 tile, K = 32):
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

constexpr int kWaves = 4;
constexpr float kLazy = 6.0f;  // p <= 2^6 between rescales

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
__device__ inline float dpp_xor1(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0xB1,
                                                            0xF, 0xF, false));
}
__device__ inline float dpp_xor2(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x4E,
                                                            0xF, 0xF, false));
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

// Slot map of the q.k A operand: k-step s, lane quarter jq, slot e (0..7) ->
// head-dim index d and the power-of-two weight w of the stored code bits
// (operand value = code * w * 2^-24).  Must mirror k_operand() below.
template <int D, int B>
__device__ inline void kslot(int s, int jq, int e, int& d, float& w) {
  const int c0 = jq * (D / 4);
  const int kp = e >> 1, hf = e & 1;
  if (B == 16) {
    d = c0 + 8 * s + e;
    w = 1.0f;
  } else if (B == 8) {
    const int di = 2 * s + (kp >> 1);
    d = c0 + 4 * di + (kp & 1) + 2 * hf;
    w = 1.0f;
  } else if (B == 4) {
    d = c0 + 8 * s + kp + 4 * hf;
    w = (kp & 1) ? 16.0f : 1.0f;
  } else {  // B == 2
    const int odd = s & 1;
    d = c0 + 16 * (s >> 1) + (odd ? 4 : 0) + kp + 8 * hf;
    w = (!odd || kp) ? float(1 << (2 * kp)) : 256.0f;
  }
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
template <int D, int B>
__device__ inline VPair<D, B> vpair_words(const uint32_t* a, const uint32_t* b) {
  VPair<D, B> r;
  if constexpr (B == 16) {  // bf16 elements 2i, 2i+1 of each token
#pragma unroll
    for (int i = 0; i < D / 32; ++i) {
      r.w[i] = a[i];          // kept raw; v_block permutes
    }
  } else if constexpr (B == 8) {
#pragma unroll
    for (int i = 0; i < D / 64; ++i) r.w[i] = a[i];
  } else if constexpr (B == 4) {
    r.w[0] = __builtin_amdgcn_perm(b[0], a[0], 0x05040100u);  // nibbles 0..3 of a | b
    r.w[1] = __builtin_amdgcn_perm(b[0], a[0], 0x07060302u);  // nibbles 4..7
  } else {
    r.w[0] = (a[0] & 0xFFFFu) | (b[0] << 16);
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
  const uint16_t* q_lds;   // [G][D] bf16 bits of this workgroup's queries
  uint8_t* stage;          // this wave's LDS stage (kStageBytes)
  float qscale;
  int G;
  int lane, n, jq;         // lane, column (l % 16), quarter (l / 16)
};

// Build Q' for k format KB: per k-step, 8 slots of this lane's column.
// Returns the sum of q over the column's (head, group), times qscale: each
// lane's slots cover its quarter of the head dim exactly once, so a sum over
// the four quarters completes it.
template <int D, int NG, int KB>
__device__ inline float build_q(const Ctx& c, u32x4 (&qop)[D / 32]) {
  constexpr int g = D / NG;
  const int h = c.n / NG, gj = c.n % NG;
  const bool live = c.n < c.G * NG;
  float qs = 0.0f;
#pragma unroll
  for (int s = 0; s < D / 32; ++s) {
#pragma unroll
    for (int e2 = 0; e2 < 4; ++e2) {
      float v2[2];
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        int d;
        float w;
        kslot<D, KB>(s, c.jq, 2 * e2 + hf, d, w);
        const float qv = bf16f(c.q_lds[(live ? h : 0) * D + d]);
        const bool in = live && d / g == gj;
        qs += in ? qv : 0.0f;
        v2[hf] = in ? qv * (1.0f / w) : 0.0f;  // w: power of two
      }
      qop[s][e2] = KB == 16 ? pack_bf16(v2[0], v2[1]) : pack_f16(v2[0], v2[1]);
    }
  }
  qs += __shfl_xor(qs, 16);
  qs += __shfl_xor(qs, 32);
  return qs * c.qscale;
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

// q.k, softmax and p.v of one 32-token step.  MASKED: the step may run past
// the segment end (rows_left < 32).
template <int D, int NG, int KB, int VB, bool MASKED>
__device__ inline void compute_step(const Ctx& c, WaveState<D>& ws, const Step<D, KB, VB>& st,
                                    const u32x4 (&qop)[D / 32], float qs, float c24,
                                    int rows_left) {
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
    }
  }
  float sc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const float a = acc[e >> 2][e & 3];
    float part;
    if constexpr (KB < 16) part = a * (f16lo(st.km[e]) * c24) + f16hi(st.km[e]) * qs;
    else part = a * c.qscale;
    if constexpr (NG >= 2) part += dpp_xor1(part);
    if constexpr (NG >= 4) part += dpp_xor2(part);
    if constexpr (MASKED) {
      const int r = 16 * (e >> 2) + 4 * c.jq + (e & 3);
      part = r < rows_left ? part : -INFINITY;
    }
    sc[e] = part;
  }

  // online softmax with a lazy running max
  float mx = fmaxf(fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3])),
                   fmaxf(fmaxf(sc[4], sc[5]), fmaxf(sc[6], sc[7])));
  mx = fmaxf(mx, __shfl_xor(mx, 16));
  mx = fmaxf(mx, __shfl_xor(mx, 32));
  const float mnew = fmaxf(ws.m, mx);
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
  float p[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    p[e] = __builtin_amdgcn_exp2f(sc[e] - ws.m);
    ws.l += p[e];
  }

  u32x4 pa, pb;  // A operand (and the bf16 low part for bf16 V)
  if constexpr (VB < 16) {
#pragma unroll
    for (int e2 = 0; e2 < 4; ++e2) {
      const float p0 = p[2 * e2], p1 = p[2 * e2 + 1];
      pa[e2] = pack_f16(p0 * f16lo(st.vm[2 * e2]), p1 * f16lo(st.vm[2 * e2 + 1]));
      ws.mt += p0 * f16hi(st.vm[2 * e2]) + p1 * f16hi(st.vm[2 * e2 + 1]);
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
  for (int e2 = 0; e2 < 4; ++e2) pw[e2] = vpair_words<D, VB>(st.v[2 * e2], st.v[2 * e2 + 1]);
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
  static constexpr int kOffKM = 32 * KR, kOffV = kOffKM + 32 * MR, kOffVM = kOffV + 32 * VR;
  static constexpr int kBytes = kOffVM + 32 * MR;
  uint32_t k[KP / 4];
  uint32_t km[(MP + 3) / 4];
  uint32_t v[VP / 4];
  uint32_t vm[(MP + 3) / 4];
};

// Wave-private LDS stage large enough for every quantised format.
constexpr int kStageBytes = 2 * (32 * 128 + 32 * 16);  // INT8 K and V at D=128, NG=4

// Lane piece of tile rows [0, 32) of step `step`; rows at or past rows_total
// are clamped to the segment's last row (those lanes re-read cached bytes).
template <int D, int NG, int KB, int VB>
__device__ inline void stage_load(const uint8_t* kp, const uint8_t* kmp, const uint8_t* vp,
                                  const uint8_t* vmp, int step, int rows_total, int lane,
                                  Stage<D, NG, KB, VB>& st) {
  using S = Stage<D, NG, KB, VB>;
  const int row = min(step * 32 + (lane >> 1), rows_total - 1);
  const int half = lane & 1;
  load_bytes<S::KP>(kp + row * S::KR + half * S::KP, st.k);
  load_bytes<S::MP>(kmp + row * S::MR + half * S::MP, st.km);
  load_bytes<S::VP>(vp + row * S::VR + half * S::VP, st.v);
  load_bytes<S::MP>(vmp + row * S::MR + half * S::MP, st.vm);
}

// Lanes exchange data through the stage, so the compiler must not move one
// lane's LDS accesses across another's: wave barriers order the previous
// step's reads before these writes, and these writes before the next reads
// (LDS executes one wave's instructions in order).
template <int D, int NG, int KB, int VB>
__device__ inline void stage_put(uint8_t* lds, int lane, const Stage<D, NG, KB, VB>& st) {
  using S = Stage<D, NG, KB, VB>;
  __builtin_amdgcn_wave_barrier();
  store_bytes<S::KP>(lds + lane * S::KP, st.k);
  store_bytes<S::MP>(lds + S::kOffKM + lane * S::MP, st.km);
  store_bytes<S::VP>(lds + S::kOffV + lane * S::VP, st.v);
  store_bytes<S::MP>(lds + S::kOffVM + lane * S::MP, st.vm);
  __builtin_amdgcn_wave_barrier();
}

// Operand gather from the LDS stage into the layout compute_step expects.
template <int D, int NG, int KB, int VB>
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
    st.km[e] = *reinterpret_cast<const uint32_t*>(lds + S::kOffKM + r * S::MR + gj * 4);
    st.vm[e] = *reinterpret_cast<const uint32_t*>(lds + S::kOffVM + r * S::MR + gj * 4);
    load_bytes<VBY>(lds + S::kOffV + r * S::VR + c.n * VBY, st.v[e]);
  }
}

// One segment [x0, x1) of rows of one format, rows starting at plane row
// row0 (K and V share row numbering).  KB/VB: stored widths (16 = bf16).
template <int D, int NG, int KB, int VB>
__device__ void run_segment(const Ctx& c, WaveState<D>& ws, int x0, int x1, int64_t row0,
                            bool visual) {
  constexpr int NB = D / 16;
  constexpr int KR = Fmt<D, KB>::kRowBytes, VR = Fmt<D, VB>::kRowBytes, MR = NG * 4;
  const uint8_t* kp = (visual ? c.kvis : c.ktxt) + row0 * KR;
  const uint8_t* vp = (visual ? c.vvis : c.vtxt) + row0 * VR;
  const uint8_t* kmp = c.kmeta + row0 * MR;
  const uint8_t* vmp = c.vmeta + row0 * MR;

  u32x4 qop[D / 32];
  const float qs = build_q<D, NG, KB>(c, qop);
  const float c24 = c.qscale * 16777216.0f;  // 2^24 * qscale

#pragma unroll
  for (int mb = 0; mb < NB; ++mb) ws.o[mb] *= v_inflation<D, VB>(mb);

  const int rows = x1 - x0;
  const int nfull = rows / 32;
  Offs<D, NG, KB, VB> of;
  of.full(c);
  // Quantised steps are small (~32 VGPRs of raw data): double-buffer them so
  // the loads of step i+1 fly while step i computes.  bf16 steps carry 64
  // VGPRs of data and run single-buffered.
  constexpr bool kStaged = KB < 16 && VB < 16;
  Step<D, KB, VB> sa;
  int i = 0;
  if constexpr (kStaged) {
    // Two register stages in flight; loads inside the loop are unconditional
    // (clamped to the last full step) so the wait counts stay exact.
    if (nfull > 0) {
      Stage<D, NG, KB, VB> ga, gb;
      stage_load<D, NG, KB, VB>(kp, kmp, vp, vmp, 0, 32 * nfull, c.lane, ga);
      stage_load<D, NG, KB, VB>(kp, kmp, vp, vmp, min(1, nfull - 1), 32 * nfull, c.lane, gb);
      for (; i + 1 < nfull; i += 2) {
        stage_put<D, NG, KB, VB>(c.stage, c.lane, ga);
        stage_load<D, NG, KB, VB>(kp, kmp, vp, vmp, min(i + 2, nfull - 1), 32 * nfull, c.lane, ga);
        stage_get<D, NG, KB, VB>(c.stage, c, sa);
        compute_step<D, NG, KB, VB, false>(c, ws, sa, qop, qs, c24, 32);
        stage_put<D, NG, KB, VB>(c.stage, c.lane, gb);
        stage_load<D, NG, KB, VB>(kp, kmp, vp, vmp, min(i + 3, nfull - 1), 32 * nfull, c.lane, gb);
        stage_get<D, NG, KB, VB>(c.stage, c, sa);
        compute_step<D, NG, KB, VB, false>(c, ws, sa, qop, qs, c24, 32);
      }
      if (i < nfull) {  // odd step count: the last full step sits in ga
        stage_put<D, NG, KB, VB>(c.stage, c.lane, ga);
        stage_get<D, NG, KB, VB>(c.stage, c, sa);
        compute_step<D, NG, KB, VB, false>(c, ws, sa, qop, qs, c24, 32);
        ++i;
      }
    }
  } else {
    for (; i < nfull; ++i) {
      const int64_t o = int64_t(i) * 32;
      load_step<D, NG, KB, VB, false>(kp + o * KR, kmp + o * MR, vp + o * VR, vmp + o * MR, of,
                                      sa);
      compute_step<D, NG, KB, VB, false>(c, ws, sa, qop, qs, c24, 32);
    }
  }
  const int tail = rows - 32 * nfull;
  if (tail > 0) {
    const int64_t o = int64_t(nfull) * 32;
    of.clamped(c, tail);
    load_step<D, NG, KB, VB, true>(kp + o * KR, kmp + o * MR, vp + o * VR, vmp + o * MR, of, sa);
    compute_step<D, NG, KB, VB, true>(c, ws, sa, qop, qs, c24, tail);
  }

#pragma unroll
  for (int mb = 0; mb < NB; ++mb) ws.o[mb] *= 1.0f / v_inflation<D, VB>(mb);
}

template <int D, int NG>
__device__ void dispatch_visual(int kb, int vb, const Ctx& c, WaveState<D>& st, int x0, int x1,
                                int64_t row0) {
#define KVQ_VIS(K, V) \
  if (kb == K && vb == V) { run_segment<D, NG, K, V>(c, st, x0, x1, row0, true); return; }
  KVQ_VIS(2, 2) KVQ_VIS(2, 4) KVQ_VIS(2, 8) KVQ_VIS(2, 16)
  KVQ_VIS(4, 2) KVQ_VIS(4, 4) KVQ_VIS(4, 8) KVQ_VIS(4, 16)
  KVQ_VIS(8, 2) KVQ_VIS(8, 4) KVQ_VIS(8, 8) KVQ_VIS(8, 16)
  KVQ_VIS(16, 2) KVQ_VIS(16, 4) KVQ_VIS(16, 8) KVQ_VIS(16, 16)
#undef KVQ_VIS
}

template <int D, int NG>
__global__ __launch_bounds__(256, 2) void decode_mfma_kernel(DecodeArgs a) {
  constexpr int NB = D / 16;
  constexpr int g = D / NG;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
  int slot, sl, x;
  decode_block(a, blockIdx.x, a.n_seq, slot, sl, x);
  const int lh = a.lh_glob[slot];
  const int l_local = lh / a.Hkv, h = lh % a.Hkv;
  const int s = a.seq_off + sl;
  const int nxs = a.nx[sl] * a.mult[slot];  // workgroups of this (layer, seq, head)
  const int cap = a.cap[sl];
  int len = a.seq_lens[s];
  len = len < 1 ? 1 : (len > cap ? cap : len);
  const int G = a.G;

  __shared__ uint16_t q_lds[kMaxGroupRatio * D];
  __shared__ float ml_lds[kWaves][kMaxGroupRatio][2];
  // wave stages during the loop; per-wave outputs for the final combine after it
  constexpr int kOBytes = kWaves * kMaxGroupRatio * D * 4;
  constexpr int kUnion = kOBytes > kWaves * kStageBytes ? kOBytes : kWaves * kStageBytes;
  __shared__ __attribute__((aligned(16))) uint8_t big_lds[kUnion];
  float(*o_lds)[kMaxGroupRatio][D] = reinterpret_cast<float(*)[kMaxGroupRatio][D]>(big_lds);

  const uint16_t* qp = a.q + ((int64_t(l_local) * a.B + s) * a.Hq + int64_t(h) * G) * D;
  for (int i = threadIdx.x; i < G * D; i += 256) q_lds[i] = qp[i];
  __syncthreads();

  Ctx c;
  {
    const int kb = a.bits[slot][0], vb = a.bits[slot][1];
    c.kvis = a.cache + uint64_t(a.base256[slot][0]) * 256u;
    c.kmeta = c.kvis + meta_plane_offset(a.Rvis, D, kb);
    c.ktxt = c.kvis + txt_plane_offset(a.Rvis, D, g, kb);
    c.vvis = a.cache + uint64_t(a.base256[slot][1]) * 256u;
    c.vmeta = c.vvis + meta_plane_offset(a.Rvis, D, vb);
    c.vtxt = c.vvis + txt_plane_offset(a.Rvis, D, g, vb);
  }
  c.q_lds = q_lds;
  c.stage = big_lds + wave * kStageBytes;
  c.qscale = a.qscale;
  c.G = G;
  c.lane = lane;
  c.n = lane & 15;
  c.jq = lane >> 4;

  WaveState<D> st;
#pragma unroll
  for (int mb = 0; mb < NB; ++mb) st.o[mb] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  st.m = -INFINITY;
  st.l = 0.0f;
  st.mt = 0.0f;

  int wa, wb;
  wave_range(x, wave, nxs, len, a.chunk, kWaves, wa, wb);
  if (wa < wb) {
    const int vb = a.vb[sl], ve = a.ve[sl];
    const int64_t vrow0 = a.vrow0[sl], trow0 = a.trow0[sl];
    const int kb = a.bits[slot][0], vbits = a.bits[slot][1];
    // text prefix [0, vb), visual [vb, ve), text suffix [ve, cap)
    int x0 = wa, x1 = min(wb, vb);
    if (x0 < x1) run_segment<D, NG, 16, 16>(c, st, x0, x1, trow0 + x0, false);
    x0 = max(wa, vb);
    x1 = min(wb, ve);
    if (x0 < x1) dispatch_visual<D, NG>(kb, vbits, c, st, x0, x1, vrow0 + (x0 - vb));
    x0 = max(wa, ve);
    x1 = wb;
    if (x0 < x1) run_segment<D, NG, 16, 16>(c, st, x0, x1, trow0 + (x0 - (ve - vb)), false);
  }

  // ---- wave result -> LDS: per head m, l and unnormalised o[d] ---------------
  __syncthreads();  // stages are reused as o_lds below
  float l_col = st.l + __shfl_xor(st.l, 16);
  l_col += __shfl_xor(l_col, 32);
  float mt_col = st.mt + __shfl_xor(st.mt, 16);
  mt_col += __shfl_xor(mt_col, 32);
  const int n = lane & 15, jq = lane >> 4;
  if (jq == 0 && n < G * NG && n % NG == 0) {
    ml_lds[wave][n / NG][0] = st.m;
    ml_lds[wave][n / NG][1] = l_col;
  }
  float mt_row[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) mt_row[i] = __shfl(mt_col, 4 * jq + i);
#pragma unroll
  for (int mb = 0; mb < NB; ++mb) {
    const int d = NB * n + mb;
    const int gd = d / g;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 4 * jq + i;
      if (r < G * NG && r % NG == gd) o_lds[wave][r / NG][d] = st.o[mb][i] + mt_row[i];
    }
  }
  __syncthreads();

  // ---- combine waves; write the workgroup's partial (or the final output) ----
  const bool single = nxs == 1;
  const int64_t pidx = partial_index(l_local, s, h, x, a.B, a.Hkv, a.max_chunks);
  if (x == 0 && threadIdx.x == 0)
    a.ws_cnt[(int64_t(l_local) * a.B + s) * a.Hkv + h] = nxs;
  for (int i = threadIdx.x; i < G * D; i += 256) {
    const int j = i / D, d = i % D;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWaves; ++w)
      if (ml_lds[w][j][1] > 0.0f) M = fmaxf(M, ml_lds[w][j][0]);
    float L = 0.0f, acc = 0.0f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      if (ml_lds[w][j][1] > 0.0f) {
        const float f = __builtin_amdgcn_exp2f(ml_lds[w][j][0] - M);
        L += ml_lds[w][j][1] * f;
        acc += o_lds[w][j][d] * f;
      }
    }
    const float o = L > 0.0f ? acc / L : 0.0f;  // L == 0: no token in this workgroup
    if (single) {
      a.out[((int64_t(l_local) * a.B + s) * a.Hq + int64_t(h) * G + j) * D + d] =
          __builtin_bit_cast(uint16_t, (__bf16)o);
    } else {
      a.ws_o[(pidx * G + j) * D + d] = o;
      if (d == 0) {
        a.ws_ml[(pidx * G + j) * 2 + 0] = M;
        a.ws_ml[(pidx * G + j) * 2 + 1] = L;
      }
    }
  }
}

}  // namespace

bool mfma_supported(int D, int g, int G) {
  return (D == 64 || D == 128) && G * (D / g) <= 16;
}

hipError_t launch_decode_mfma(const DecodeArgs& a, int n_seq_launch, hipStream_t stream) {
  (void)n_seq_launch;  // a.n_seq
  const dim3 grid(a.nxcum[a.n_seq] * a.mcum[a.n_lh], 1, 1);  // compact block list
  const int NG = a.D / a.g;
#define KVQ_LAUNCH(DD, NN)                                                           \
  if (a.D == DD && NG == NN) {                                                       \
    hipLaunchKernelGGL((decode_mfma_kernel<DD, NN>), grid, dim3(256), 0, stream, a); \
    return hipGetLastError();                                                        \
  }
  KVQ_LAUNCH(128, 1) KVQ_LAUNCH(128, 2) KVQ_LAUNCH(128, 4) KVQ_LAUNCH(64, 1) KVQ_LAUNCH(64, 2)
#undef KVQ_LAUNCH
  return hipErrorInvalidValue;
}

}  // namespace kvq
