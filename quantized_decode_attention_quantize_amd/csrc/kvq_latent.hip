// kvq_latent.hip -- decode-step attention over a low-rank latent cache, and
// the store of latent rows: kvq_latent_cache_bytes, kvq_latent_store and
// kvq_latent_decode of include/kvq.h.
//
// gist.science 2604.02570 (WSVD), section 2-A: every attention head gets its
// own low-rank factorisation, so one (layer, KV head) caches latent rows c_t
// of width r instead of K/V rows of width D, with K_t = c^K_t B_K and
// V_t = c^V_t B_V for per-head r x D up-projections; section 2-D: K and V
// are reconstructed on chip inside flash decoding and never written back.
//
// The kernel never forms a K or V row: q . (c B_K) = (B_K q) . c and
// sum_t p_t (c_t B_V) = (sum_t p_t c_t) B_V, so each workgroup projects its
// query heads once on the matrix cores (q' = B_K q), attends over the
// latents at width r, and the merge applies B_V to the combined latent
// output.  It reads the same bytes as a row-by-row reconstruction and skips
// its r x D product per token.  Precision: q' and the probabilities enter
// the bf16 matrix cores as hi/lo bf16 pairs (about 16 significant bits),
// every sum is fp32, the output is rounded to bf16 once.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <vector>

#include "../../include/kvq.h"
#include "kvq_internal.h"

namespace kvq {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x3 __attribute__((ext_vector_type(3)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __amdgpu_buffer_rsrc_t Rsrc;

// Waves per decode workgroup: eight for narrow latents (a step is few
// bytes, so more waves keep more of them in flight), four for wide ones
// (more waves would cost registers the loop needs and a longer combine).
template <int R>
constexpr int lat_waves() { return R <= 64 ? 8 : 4; }
constexpr float kLLazy = 6.0f;            // p <= 2^6 between rescales
constexpr int kLMaxChunks = 4096;         // partial slots per (layer, seq, head)

struct LatentArgs {
  const uint8_t* cache;
  const int32_t* seq_lens;  // device [batch]
  const uint16_t* q;        // bf16 [nl, B, Hq, D]
  uint16_t* out;            // bf16 [nl, B, Hq, D]
  const uint16_t* up_k;     // bf16 [L, Hkv, r, D]
  const uint16_t* up_v;
  float* ws_o;              // [entries][G][D] unnormalised outputs (B_V applied)
  float* ws_ml;             // [entries][G][2] (max in log2 units, sum)
  int32_t* ws_arrive;       // [cache layers][B][Hkv] arrival counters, zero between calls
  float qscale;             // sm_scale * log2(e)
  int64_t plane_bytes;
  int Hkv, Hq, G, B;
  int layer_begin, nl;
  int chunk;                // tokens per decode workgroup (multiple of 32)
  int claim_steps;          // 1: waves claim their steps (library-chosen chunks)
  int max_chunks;
  int seq_off, n_seq;       // sequences [seq_off, seq_off + n_seq) of this launch
  int32_t row0[kMaxSeq];    // first plane row of each sequence
  int32_t cap[kMaxSeq];
  int32_t nxcum[kMaxSeq + 1];  // sequence i has nxcum[i + 1] - nxcum[i] chunks
};
static_assert(sizeof(LatentArgs) <= 4096, "LatentArgs must fit the kernel argument limit");

struct LatentStoreArgs {
  uint8_t* cache;
  const uint16_t* src[2];   // bf16 [nl, S, Hkv, n, r] for K and V
  int64_t plane_bytes;
  int Hkv, n, S, seq_off, layer_begin, nl;
  int32_t row0[kMaxSeq];    // plane row of the call's first position, per sequence
};

__device__ inline f32x4 mfma_bf16(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}
__device__ inline float bf16_lo(uint32_t w) { return __builtin_bit_cast(float, w << 16); }
__device__ inline float bf16_hi(uint32_t w) { return __builtin_bit_cast(float, w & 0xFFFF0000u); }
__device__ inline uint32_t bf16_bits(float x) {
  return uint32_t(__builtin_bit_cast(uint16_t, (__bf16)x));  // nearest even
}
// hi/lo bf16 pair words of (x0, x1): hi = bf16(x), lo = bf16(x - hi).
__device__ inline void split_pair(float x0, float x1, uint32_t& hi, uint32_t& lo) {
  const uint32_t h0 = bf16_bits(x0), h1 = bf16_bits(x1);
  hi = h0 | (h1 << 16);
  lo = bf16_bits(x0 - bf16_lo(h0)) | (bf16_bits(x1 - bf16_lo(h1)) << 16);
}
__device__ inline Rsrc make_rsrc(const void* base, int64_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, int(bytes), 0x00020000);
}
// Max over lanes {l, l^16, l^32, l^48}: the four row quarters of one column
// of a 16 x 16 accumulator.
__device__ inline float max_quarters(float v) {
  v = fmaxf(v, __shfl_xor(v, 16));
  return fmaxf(v, __shfl_xor(v, 32));
}
__device__ inline float sum_quarters(float v) {
  v += __shfl_xor(v, 16);
  return v + __shfl_xor(v, 32);
}

// One 32-token step of one wave, as loaded: lane (n = lane % 16, j = lane /
// 16) holds, for rows 16 tau + n, the j-th quarter of the K latent row (r/4
// values, r/32 chunks of 8), and for the eight rows 16 (e / 4) + 4 j + e % 4
// the n-th sixteenth of the V latent row (r/16 values).
template <int R>
struct LStep {
  u32x4 k[2][R / 32];
  uint32_t v[8][R / 32];
};

template <int R>
__device__ inline void load_vpiece(Rsrc r, uint32_t off, uint32_t* out) {
  if constexpr (R == 128) {
    const u32x4 x = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
    out[0] = x[0]; out[1] = x[1]; out[2] = x[2]; out[3] = x[3];
  } else if constexpr (R == 96) {
    const u32x3 x = __builtin_amdgcn_raw_buffer_load_b96(r, off, 0, 0);
    out[0] = x[0]; out[1] = x[1]; out[2] = x[2];
  } else if constexpr (R == 64) {
    const u32x2 x = __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0);
    out[0] = x[0]; out[1] = x[1];
  } else {
    out[0] = __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0);
  }
}

// Loads the step whose first plane row is `row`, of which `rows` (1..32)
// exist: rows past them re-read the last one (their scores are masked).
template <int R>
__device__ inline void load_lstep(Rsrc kr, Rsrc vr, int row, int rows, int n, int j,
                                  LStep<R>& st) {
#pragma unroll
  for (int tau = 0; tau < 2; ++tau) {
    const uint32_t off = uint32_t(row + min(16 * tau + n, rows - 1)) * (2 * R) + j * (R / 2);
#pragma unroll
    for (int c = 0; c < R / 32; ++c)
      st.k[tau][c] = __builtin_amdgcn_raw_buffer_load_b128(kr, off + 16 * c, 0, 0);
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int t = 16 * (e >> 2) + 4 * j + (e & 3);
    load_vpiece<R>(vr, uint32_t(row + min(t, rows - 1)) * (2 * R) + n * (R / 8), st.v[e]);
  }
}

template <int R>
struct LWave {
  float m = -INFINITY;  // running max of this lane's column (log2 units)
  float l = 0.0f;       // this lane's share of the column's sum
  f32x4 o[R / 16];      // o[mb][i]: head 4 j + i, latent column n * R / 16 + mb
};

// q' . c, online softmax and p . c^V of one step of `rows` real rows.
template <int R>
__device__ inline void compute_lstep(LWave<R>& w, const LStep<R>& st, const u32x4 (&qhi)[R / 32],
                                     const u32x4 (&qlo)[R / 32], int rows, int j) {
  f32x4 acc[2];
#pragma unroll
  for (int tau = 0; tau < 2; ++tau) {
    acc[tau] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int c = 0; c < R / 32; ++c) {
      acc[tau] = mfma_bf16(st.k[tau][c], qhi[c], acc[tau]);
      acc[tau] = mfma_bf16(st.k[tau][c], qlo[c], acc[tau]);
    }
  }
  // sc[e]: score of row 16 (e / 4) + 4 j + e % 4 for head n (log2 units)
  float sc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    sc[e] = acc[e >> 2][e & 3];
    if (rows < 32 && 16 * (e >> 2) + 4 * j + (e & 3) >= rows) sc[e] = -INFINITY;
  }
  float mx = sc[0];
#pragma unroll
  for (int e = 1; e < 8; ++e) mx = fmaxf(mx, sc[e]);
  mx = max_quarters(mx);
  const float mnew = fmaxf(w.m, mx);
  if (__builtin_amdgcn_ballot_w64(mnew > w.m + kLLazy) != 0) {
    const float alpha = __builtin_amdgcn_exp2f(w.m - mnew);  // 0 on the first step
    w.l *= alpha;
    float ar[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) ar[i] = __shfl(alpha, 4 * j + i);
#pragma unroll
    for (int mb = 0; mb < R / 16; ++mb)
#pragma unroll
      for (int i = 0; i < 4; ++i) w.o[mb][i] *= ar[i];
    w.m = mnew;
  }
  float p[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    p[e] = __builtin_amdgcn_exp2f(sc[e] - w.m);
    w.l += p[e];
  }
  // P as the A operand (rows = heads, k = the lane's eight rows), hi and lo
  u32x4 pa, pb;
#pragma unroll
  for (int e2 = 0; e2 < 4; ++e2) {
    uint32_t hi, lo;
    split_pair(p[2 * e2], p[2 * e2 + 1], hi, lo);
    pa[e2] = hi;
    pb[e2] = lo;
  }
#pragma unroll
  for (int mb = 0; mb < R / 16; ++mb) {
    u32x4 b;
#pragma unroll
    for (int e2 = 0; e2 < 4; ++e2) {
      const uint32_t w0 = st.v[2 * e2][mb >> 1], w1 = st.v[2 * e2 + 1][mb >> 1];
      b[e2] = (mb & 1) ? __builtin_amdgcn_perm(w1, w0, 0x07060302u)
                       : __builtin_amdgcn_perm(w1, w0, 0x05040100u);
    }
    w.o[mb] = mfma_bf16(pa, b, w.o[mb]);
    w.o[mb] = mfma_bf16(pb, b, w.o[mb]);
  }
}

// Loads past this XCD's caches: partials written by workgroups on other
// XCDs (with write-through stores) are read from memory.
__device__ inline float ld_sys(const float* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
}

// Log-sum-exp merge of one (layer, sequence, KV head)'s nx chunk partials
// (D wide, B_V already applied) into its bf16 output, by the whole
// workgroup.  Latency-bound: all loads of a block of up to kMB chunks -- the
// (m, l) pairs and the partial outputs -- are issued before the block's
// first barrier.  kMB * kE = 32 values in flight per thread, so the merge
// needs no more registers than the decode loop before it.
template <int D, int kLThreads>
__device__ void merge_latent_entry(const LatentArgs& a, int l, int s, int h, int nx) {
  constexpr int kE = 16 * D / kLThreads;  // (head, column) elements per thread
  constexpr int kMB = 32 / kE;      // chunks per merge block
  static_assert(kE >= 1 && kMB * 16 <= kLThreads, "merge block shape");
  __shared__ float2 mls[kMB][16];
  __shared__ float fx[kMB][16];
  __shared__ float scl[16];
  __shared__ float Ls[16];
  const int G = a.G;
  const int64_t p0 = ((int64_t(l) * a.B + s) * a.Hkv + h) * a.max_chunks;
  const int tid = threadIdx.x;
  float acc[kE];
#pragma unroll
  for (int k = 0; k < kE; ++k) acc[k] = 0.0f;
  float M = -INFINITY, L = 0.0f;  // running (max, sum) of head tid (threads < 16)
  for (int xb = 0; xb < nx; xb += kMB) {
    const int nb = min(kMB, nx - xb);
    float ov[kMB][kE];
#pragma unroll
    for (int x = 0; x < kMB; ++x)
#pragma unroll
      for (int k = 0; k < kE; ++k) {
        const int idx = tid + kLThreads * k, hh = idx / D;
        ov[x][k] = x < nb && hh < G ? ld_sys(a.ws_o + (p0 + xb + x) * G * D + idx) : 0.0f;
      }
    if (tid < kMB * 16) {
      const int x = tid >> 4, hh = tid & 15;
      const float* m = a.ws_ml + ((p0 + xb + x) * G + hh) * 2;
      mls[x][hh] = x < nb && hh < G ? make_float2(ld_sys(m), ld_sys(m + 1))
                                    : make_float2(-INFINITY, 0.0f);
    }
    __syncthreads();
    if (tid < 16) {  // new running max; this block's weights relative to it
      float Mn = M;
      for (int x = 0; x < nb; ++x)
        if (mls[x][tid].y > 0.0f) Mn = fmaxf(Mn, mls[x][tid].x);
      const float sc = L > 0.0f ? __builtin_amdgcn_exp2f(M - Mn) : 0.0f;
      L *= sc;
      for (int x = 0; x < kMB; ++x) {
        const float2 v = mls[x][tid];
        const float f = x < nb && v.y > 0.0f ? __builtin_amdgcn_exp2f(v.x - Mn) : 0.0f;
        fx[x][tid] = f;
        L = __builtin_fmaf(f, v.y, L);
      }
      scl[tid] = sc;  // factor for the sums of earlier blocks
      M = Mn;
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < kE; ++k) {
      const int hh = (tid + kLThreads * k) / D;
      float o = acc[k] * scl[hh];
#pragma unroll
      for (int x = 0; x < kMB; ++x) o = __builtin_fmaf(fx[x][hh], ov[x][k], o);
      acc[k] = o;
    }
    __syncthreads();  // fx and scl are rewritten by the next block
  }
  if (tid < 16) Ls[tid] = L;
  __syncthreads();
  uint16_t* outp = a.out + ((int64_t(l) * a.B + s) * a.Hq + int64_t(h) * G) * D;
#pragma unroll
  for (int k = 0; k < kE; ++k) {
    const int idx = tid + kLThreads * k, hh = idx / D;
    if (hh < G) outp[idx] = uint16_t(bf16_bits(acc[k] / Ls[hh]));
  }
  if (tid == 0)
    __hip_atomic_store(&a.ws_arrive[(int64_t(a.layer_begin + l) * a.B + s) * a.Hkv + h], 0,
                       __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
}

// One workgroup: one chunk of one (layer, sequence, KV head); its waves take
// the chunk's 32-token steps, then combine into one partial.
template <int D, int R>
__global__ __launch_bounds__(64 * lat_waves<R>()) void latent_decode_kernel(LatentArgs a) {
  constexpr int kLWaves = lat_waves<R>();
  constexpr int kLThreads = 64 * kLWaves;
  __shared__ float q_lds[16][R + 4];  // q'
  __shared__ float o_lds[kLWaves][16][R];  // the waves' latent outputs
  __shared__ float ml_lds[kLWaves][16][2];
  __shared__ uint4 bv_lds[R * D / 8];  // B_V of this (layer, head), bf16
  __shared__ int claim;                // the chunk's next unclaimed step
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n = lane & 15, j = lane >> 4;

  // workgroup -> (layer-local l, head h, sequence index i, chunk x)
  const int per = a.nxcum[a.n_seq];
  const int u = blockIdx.x;
  const int lh = u / per;
  const int rem = u - lh * per;
  int lo = 0, hi = a.n_seq - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (a.nxcum[mid] <= rem) lo = mid; else hi = mid - 1;
  }
  const int i = lo, x = rem - a.nxcum[lo];
  const int l = lh / a.Hkv, h = lh - l * a.Hkv, s = a.seq_off + i, G = a.G;
  const int len = min(max(a.seq_lens[s], 1), a.cap[i]);
  const int t0 = x * a.chunk, t1 = min(t0 + a.chunk, len);
  const int64_t lhg = int64_t(a.layer_begin + l) * a.Hkv + h;
  const uint8_t* kplane = a.cache + 2 * lhg * a.plane_bytes;
  const Rsrc kr = make_rsrc(kplane, a.plane_bytes);
  const Rsrc vr = make_rsrc(kplane + a.plane_bytes, a.plane_bytes);
  const int row0 = a.row0[i];
  const int nsteps = t1 > t0 ? (t1 - t0 + 31) >> 5 : 0;
  auto rows_of = [&](int k) { return min(32, t1 - t0 - 32 * k); };
  auto load = [&](int k, LStep<R>& b) {
    if (k < nsteps) load_lstep<R>(kr, vr, row0 + t0 + 32 * k, rows_of(k), n, j, b);
  };
  // The wave's first step is loaded first: its memory latency overlaps the
  // query projection below, which does not depend on it.
  LStep<R> cur, nxt;
  load(wave, cur);

  // ---- q' = qscale * B_K q for the group's heads, on the matrix cores ----
  // B operand: lane (n, j) holds q_n[32 sd + 8 j .. + 8] (zeros past G);
  // A operand: B_K rows 16 jb + n.  Result lane (n, j), element ii: q'_n at
  // latent index 16 jb + 4 j + ii.  The waves share the r/16 blocks.
  {
    u32x4 qop[D / 32];
    const uint16_t* qrow = a.q + ((int64_t(l) * a.B + s) * a.Hq + int64_t(h) * G + n) * D;
#pragma unroll
    for (int sd = 0; sd < D / 32; ++sd)
      qop[sd] = n < G ? *reinterpret_cast<const u32x4*>(qrow + 32 * sd + 8 * j)
                      : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
    for (int jb = wave; jb < R / 16; jb += kLWaves) {
      const uint16_t* bk = a.up_k + (lhg * R + 16 * jb + n) * D;
      f32x4 c = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int sd = 0; sd < D / 32; ++sd)
        c = mfma_bf16(*reinterpret_cast<const u32x4*>(bk + 32 * sd + 8 * j), qop[sd], c);
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) q_lds[n][16 * jb + 4 * j + ii] = c[ii] * a.qscale;
    }
  }
  if (threadIdx.x == 0) claim = kLWaves;
  __syncthreads();
  // B_V loads go out after the projection (which waits for its own loads)
  // and land during the loop; they reach LDS after it
  constexpr int kBV = (R * D / 8 + kLThreads - 1) / kLThreads;
  uint4 bvt[kBV];
  {
    const uint4* bvg = reinterpret_cast<const uint4*>(a.up_v + lhg * R * D);
#pragma unroll
    for (int k = 0; k < kBV; ++k)
      if (R * D / 8 % kLThreads == 0 || threadIdx.x + kLThreads * k < R * D / 8)
        bvt[k] = bvg[threadIdx.x + kLThreads * k];
  }
  // score B operand, chunk c: lane (n, j) holds q'_n[j r/4 + 8 c .. + 8]
  u32x4 qhi[R / 32], qlo[R / 32];
#pragma unroll
  for (int c = 0; c < R / 32; ++c)
#pragma unroll
    for (int e2 = 0; e2 < 4; ++e2) {
      const int k = j * (R / 4) + 8 * c + 2 * e2;
      uint32_t hw, lw;
      split_pair(q_lds[n][k], q_lds[n][k + 1], hw, lw);
      qhi[c][e2] = hw;
      qlo[c][e2] = lw;
    }

  // ---- the wave's steps ---------------------------------------------------
  // Wave v starts on step v.  With library-chosen chunks later steps are
  // claimed from an LDS counter, so waves that issue later (two share a
  // SIMD) take fewer; fixed chunks take steps v, v + kLWaves, ... (a fixed
  // summation order).  One step is computed while the next one loads.
  LWave<R> w;
#pragma unroll
  for (int mb = 0; mb < R / 16; ++mb) w.o[mb] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  for (int k = wave; k < nsteps;) {
    int kn = k + kLWaves;
    if (a.claim_steps) {
      if (lane == 0)
        kn = __hip_atomic_fetch_add(&claim, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
      kn = __builtin_amdgcn_readfirstlane(kn);
    }
    const bool more = kn < nsteps;
    if (more) load(kn, nxt);
    compute_lstep<R>(w, cur, qhi, qlo, rows_of(k), j);
    if (!more) break;
    cur = nxt;
    k = kn;
  }

#pragma unroll
  for (int k = 0; k < kBV; ++k)
    if (R * D / 8 % kLThreads == 0 || threadIdx.x + kLThreads * k < R * D / 8)
      bv_lds[threadIdx.x + kLThreads * k] = bvt[k];
  // ---- combine the waves, apply B_V, write the chunk's partial ----------
  // The chunk's latent output is projected here, so partials (and the
  // merge) are D wide; a sequence that fits one chunk gets its final output
  // directly and needs no merge.
  const float l_col = sum_quarters(w.l);
#pragma unroll
  for (int mb = 0; mb < R / 16; ++mb)
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) o_lds[wave][4 * j + ii][n * (R / 16) + mb] = w.o[mb][ii];
  if (j == 0) {
    ml_lds[wave][n][0] = w.m;
    ml_lds[wave][n][1] = l_col;
  }
  __syncthreads();
  // Every wave combines the waves' outputs itself, straight into the A
  // operand of the projection below: lane (n, j) weighs the waves' sums of
  // head n (weights 0 for waves without rows) and gathers O[n][32 c + 8 j ..
  // + 8].  (M, L) of head n end up in every lane of column n.
  float fw[kLWaves];
  float M = -INFINITY, L = 0.0f;
#pragma unroll
  for (int v = 0; v < kLWaves; ++v) {
    const float mv = ml_lds[v][n][0], lv = ml_lds[v][n][1];
    M = lv > 0.0f ? fmaxf(M, mv) : M;
    fw[v] = mv;
  }
#pragma unroll
  for (int v = 0; v < kLWaves; ++v) {
    const float lv = ml_lds[v][n][1];
    fw[v] = lv > 0.0f ? __builtin_amdgcn_exp2f(fw[v] - M) : 0.0f;
    L = __builtin_fmaf(fw[v], lv, L);
  }
  // y = O B_V on the matrix cores, O (16 heads x r, rows past G zero) as a
  // hi/lo bf16 pair.  A: lane (n, j) holds O[n][32 c + 8 j .. + 8]; B: lane
  // (n, j) holds B_V[32 c + 8 j + e][16 nb + n] for e = 0..7; the result
  // lane (n, j) holds y[4 j + ii][16 nb + n].  Waves take the D/16 column
  // blocks nb in turn.
  const int64_t p = ((int64_t(l) * a.B + s) * a.Hkv + h) * a.max_chunks + x;
  const int nx = a.nxcum[i + 1] - a.nxcum[i];
  uint16_t* outp = a.out + ((int64_t(l) * a.B + s) * a.Hq + int64_t(h) * G) * D;
  const uint16_t* bv = reinterpret_cast<const uint16_t*>(bv_lds);
  u32x4 ohi[R / 32], olo[R / 32];
#pragma unroll
  for (int c = 0; c < R / 32; ++c) {
    float o[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = 0.0f;
#pragma unroll
    for (int v = 0; v < kLWaves; ++v)
#pragma unroll
      for (int e = 0; e < 8; ++e) o[e] = __builtin_fmaf(fw[v], o_lds[v][n][32 * c + 8 * j + e], o[e]);
#pragma unroll
    for (int e2 = 0; e2 < 4; ++e2) {
      uint32_t hw, lw;
      split_pair(n < G ? o[2 * e2] : 0.0f, n < G ? o[2 * e2 + 1] : 0.0f, hw, lw);
      ohi[c][e2] = hw;
      olo[c][e2] = lw;
    }
  }
  // L of the four heads of this lane's result rows
  float lr[4];
#pragma unroll
  for (int ii = 0; ii < 4; ++ii) lr[ii] = __shfl(L, 4 * j + ii);
  for (int nb = wave; nb < D / 16; nb += kLWaves) {
    const int dd = 16 * nb + n;
    f32x4 y = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int c = 0; c < R / 32; ++c) {
      u32x4 b;
#pragma unroll
      for (int e2 = 0; e2 < 4; ++e2) {
        const int k = 32 * c + 8 * j + 2 * e2;
        b[e2] = uint32_t(bv[k * D + dd]) | uint32_t(bv[(k + 1) * D + dd]) << 16;
      }
      y = mfma_bf16(ohi[c], b, y);
      y = mfma_bf16(olo[c], b, y);
    }
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) {
      const int hh = 4 * j + ii;
      if (hh >= G) continue;
      if (nx == 1) {  // the whole sequence in this chunk: the output itself
        outp[int64_t(hh) * D + dd] = uint16_t(bf16_bits(y[ii] / lr[ii]));
      } else {
        // write-through stores: the merging workgroup may sit on another XCD
        __hip_atomic_store(&a.ws_o[(p * G + hh) * D + dd], y[ii], __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_SYSTEM);
      }
    }
  }
  if (nx > 1 && threadIdx.x < G) {  // wave 0, lanes (n < G, j = 0)
    __hip_atomic_store(&a.ws_ml[(p * G + n) * 2], M, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
    __hip_atomic_store(&a.ws_ml[(p * G + n) * 2 + 1], L, __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_SYSTEM);
  }
  if (nx == 1) return;
  // The workgroup counts its chunk in once its partial has reached memory;
  // the one that completes the count merges the entry (no second launch).
  __shared__ int last;
  __builtin_amdgcn_s_waitcnt(0);  // this thread's partial stores are complete
  __syncthreads();
  if (threadIdx.x == 0)
    last = __hip_atomic_fetch_add(&a.ws_arrive[(int64_t(a.layer_begin + l) * a.B + s) * a.Hkv + h],
                                  1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM) == nx - 1;
  __syncthreads();
  if (last) merge_latent_entry<D, kLThreads>(a, l, s, h, nx);
}

// Copies 16-byte pieces of latent rows into their planes.
template <int R>
__global__ __launch_bounds__(256) void latent_store_kernel(LatentStoreArgs a) {
  constexpr int kPieces = R / 8;  // 16-byte pieces per row
  const int piece = blockIdx.x * 256 + threadIdx.x;
  const int t = piece / kPieces, c = piece - t * kPieces;
  if (t >= a.n) return;
  const int si = blockIdx.y;
  const int z = blockIdx.z;  // (layer-local l, head h, X)
  const int X = z & 1, lh = z >> 1, l = lh / a.Hkv, h = lh - l * a.Hkv;
  const uint16_t* src =
      a.src[X] + ((((int64_t(l) * a.S + a.seq_off + si) * a.Hkv + h) * a.n + t) * R + 8 * c);
  const int64_t lhg = int64_t(a.layer_begin + l) * a.Hkv + h;
  uint8_t* dst = a.cache + (2 * lhg + X) * a.plane_bytes + (int64_t(a.row0[si]) + t) * (2 * R) +
                 16 * c;
  *reinterpret_cast<u32x4*>(dst) = *reinterpret_cast<const u32x4*>(src);
}

// ---- host side ---------------------------------------------------------

bool rank_ok(int r, int D) { return (r == 32 || r == 64 || r == 96 || r == 128) && r <= D; }

std::vector<int64_t> row_bases(const kvq_latent_config* c) {
  std::vector<int64_t> b(size_t(c->batch) + 1, 0);
  for (int s = 0; s < c->batch; ++s) b[s + 1] = b[s] + (int64_t(c->capacity[s]) + 31) / 32 * 32;
  return b;
}

int64_t plane_bytes_of(const kvq_latent_config* c) {
  return (row_bases(c).back() * c->rank * 2 + 255) / 256 * 256;
}

kvq_status check_latent(const kvq_latent_config* c) {
  if (!c || !c->capacity) return KVQ_ERR_NULL;
  if (c->num_layers < 1 || c->batch < 1 || c->num_q_heads < 1 || c->num_kv_heads < 1)
    return KVQ_ERR_SHAPE;
  for (int s = 0; s < c->batch; ++s)
    if (c->capacity[s] < 1) return KVQ_ERR_SHAPE;
  if (c->num_q_heads % c->num_kv_heads) return KVQ_ERR_UNSUPPORTED;
  if (c->num_q_heads / c->num_kv_heads > 16) return KVQ_ERR_UNSUPPORTED;
  if (c->head_dim != 64 && c->head_dim != 128) return KVQ_ERR_UNSUPPORTED;
  if (!rank_ok(c->rank, c->head_dim)) return KVQ_ERR_UNSUPPORTED;
  if (plane_bytes_of(c) > int64_t(0x7FFFFFFF)) return KVQ_ERR_UNSUPPORTED;  // 32-bit offsets
  return KVQ_OK;
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

// Tokens per decode workgroup: the shortest 128-token multiple (at least 256)
// for which the call has at most one workgroup per compute unit.  Long
// chunks measured fastest (the per-workgroup query projection and epilogue
// are paid least often), and a count just above the unit count leaves some
// units with two workgroups and the rest idle at the end.
int latent_chunk(const kvq_latent_config* c, int num_layers, int chunk_tokens) {
  if (chunk_tokens > 0) return chunk_tokens;
  int64_t work = 0;
  int longest = 1;
  for (int s = 0; s < c->batch; ++s) {
    work += c->capacity[s];
    longest = std::max(longest, int(c->capacity[s]));
  }
  const int64_t lh = int64_t(num_layers) * c->num_kv_heads, units = device_cus();
  int64_t ch = (work * lh + units - 1) / units;
  ch = std::max<int64_t>((ch + 127) / 128 * 128, 256);
  auto count = [&](int64_t chunk) {
    int64_t n = 0;
    for (int s = 0; s < c->batch; ++s) n += (c->capacity[s] + chunk - 1) / chunk;
    return n * lh;
  };
  while (ch < longest && count(ch) > units) ch += 128;
  return int(std::min<int64_t>(ch, 1 << 20));
}

int max_chunks_of(const kvq_latent_config* c, int chunk) {
  int m = 1;
  for (int s = 0; s < c->batch; ++s) m = std::max(m, (c->capacity[s] + chunk - 1) / chunk);
  return m;
}

template <int D, int R>
hipError_t launch_latent(const LatentArgs& a, hipStream_t st) {
  const int units = a.nl * a.Hkv * a.nxcum[a.n_seq];
  hipLaunchKernelGGL((latent_decode_kernel<D, R>), dim3(units), dim3(64 * lat_waves<R>()), 0, st,
                     a);
  return hipGetLastError();
}

hipError_t dispatch_latent(int D, int R, const LatentArgs& a, hipStream_t st) {
#define KVQ_LATENT_CASE(d, r) \
  if (D == d && R == r) return launch_latent<d, r>(a, st);
  KVQ_LATENT_CASE(64, 32)
  KVQ_LATENT_CASE(64, 64)
  KVQ_LATENT_CASE(128, 32)
  KVQ_LATENT_CASE(128, 64)
  KVQ_LATENT_CASE(128, 96)
  KVQ_LATENT_CASE(128, 128)
#undef KVQ_LATENT_CASE
  return hipErrorInvalidValue;
}

template <int R>
hipError_t launch_latent_store(const LatentStoreArgs& a, int n_seq, hipStream_t st) {
  const int pieces = a.n * (R / 8);
  const dim3 grid((pieces + 255) / 256, n_seq, a.nl * a.Hkv * 2);
  hipLaunchKernelGGL((latent_store_kernel<R>), grid, dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace
}  // namespace kvq

using namespace kvq;

extern "C" kvq_status kvq_latent_cache_bytes(const kvq_latent_config* cfg, uint64_t* bytes) {
  if (!bytes) return KVQ_ERR_NULL;
  const kvq_status st = check_latent(cfg);
  if (st != KVQ_OK) return st;
  *bytes = uint64_t(cfg->num_layers) * cfg->num_kv_heads * 2 * uint64_t(plane_bytes_of(cfg));
  return KVQ_OK;
}

extern "C" kvq_status kvq_latent_store(const kvq_latent_config* cfg, void* cache,
                                       int32_t layer_begin, int32_t num_layers,
                                       int32_t num_seqs, const int32_t* seq_ids,
                                       int32_t tok_begin, int32_t tok_end, const void* k_latent,
                                       const void* v_latent, void* stream) {
  kvq_status st = check_latent(cfg);
  if (st != KVQ_OK) return st;
  if (num_layers < 0 || num_seqs < 0 || tok_end < tok_begin) return KVQ_ERR_SHAPE;
  if (num_layers == 0 || num_seqs == 0 || tok_end == tok_begin) return KVQ_OK;
  if (!cache || !seq_ids || !k_latent || !v_latent) return KVQ_ERR_NULL;
  if (!aligned(cache, 256) || !aligned(k_latent, 16) || !aligned(v_latent, 16))
    return KVQ_ERR_ALIGN;
  if (layer_begin < 0 || int64_t(layer_begin) + num_layers > cfg->num_layers) return KVQ_ERR_RANGE;
  if (tok_begin < 0) return KVQ_ERR_RANGE;
  std::vector<char> seen(size_t(cfg->batch), 0);
  for (int i = 0; i < num_seqs; ++i) {
    const int s = seq_ids[i];
    if (s < 0 || s >= cfg->batch) return KVQ_ERR_RANGE;
    if (seen[s]) return KVQ_ERR_SHAPE;
    seen[s] = 1;
    if (tok_end > cfg->capacity[s]) return KVQ_ERR_RANGE;
  }
  const std::vector<int64_t> base = row_bases(cfg);
  LatentStoreArgs a{};
  a.cache = static_cast<uint8_t*>(cache);
  a.src[0] = static_cast<const uint16_t*>(k_latent);
  a.src[1] = static_cast<const uint16_t*>(v_latent);
  a.plane_bytes = plane_bytes_of(cfg);
  a.Hkv = cfg->num_kv_heads;
  a.n = tok_end - tok_begin;
  a.S = num_seqs;
  a.layer_begin = layer_begin;
  a.nl = num_layers;
  if (int64_t(num_layers) * cfg->num_kv_heads * 2 > 65535) return KVQ_ERR_UNSUPPORTED;
  for (int s0 = 0; s0 < num_seqs; s0 += kMaxSeq) {
    const int ns = std::min(kMaxSeq, num_seqs - s0);
    a.seq_off = s0;
    for (int i = 0; i < ns; ++i) a.row0[i] = int32_t(base[seq_ids[s0 + i]] + tok_begin);
    hipError_t e;
    switch (cfg->rank) {
      case 32: e = launch_latent_store<32>(a, ns, static_cast<hipStream_t>(stream)); break;
      case 64: e = launch_latent_store<64>(a, ns, static_cast<hipStream_t>(stream)); break;
      case 96: e = launch_latent_store<96>(a, ns, static_cast<hipStream_t>(stream)); break;
      default: e = launch_latent_store<128>(a, ns, static_cast<hipStream_t>(stream)); break;
    }
    if (e != hipSuccess) return KVQ_ERR_HIP;
  }
  return KVQ_OK;
}

extern "C" kvq_status kvq_latent_decode(const kvq_latent_config* cfg, const void* cache,
                                        int32_t layer_begin, int32_t num_layers,
                                        const int32_t* seq_lens, const void* up_k,
                                        const void* up_v, const void* q, void* out,
                                        float sm_scale, int32_t chunk_tokens, void* workspace,
                                        size_t* workspace_bytes, void* stream) {
  kvq_status st = check_latent(cfg);
  if (st != KVQ_OK) return st;
  if (!workspace_bytes) return KVQ_ERR_NULL;
  if (num_layers < 1) return KVQ_ERR_SHAPE;
  if (layer_begin < 0 || int64_t(layer_begin) + num_layers > cfg->num_layers) return KVQ_ERR_RANGE;
  if (chunk_tokens < 0 || chunk_tokens % 32) return KVQ_ERR_SHAPE;
  if (!(sm_scale > 0.0f) || !std::isfinite(sm_scale)) return KVQ_ERR_SHAPE;
  const int D = cfg->head_dim, R = cfg->rank, Hkv = cfg->num_kv_heads;
  const int G = cfg->num_q_heads / Hkv;
  const int chunk = latent_chunk(cfg, num_layers, chunk_tokens);
  const int max_chunks = max_chunks_of(cfg, chunk);
  if (max_chunks > kLMaxChunks) return KVQ_ERR_UNSUPPORTED;
  const int64_t entries = int64_t(num_layers) * cfg->batch * Hkv * max_chunks;
  // arrival counters first, sized by the cache (every layer, sequence and KV
  // head), so calls of any layer range find them at the same offsets
  const int64_t arrive_bytes = (int64_t(cfg->num_layers) * cfg->batch * Hkv * 4 + 255) / 256 * 256;
  const int64_t o_bytes = (entries * G * D * 4 + 255) / 256 * 256;
  const int64_t need = arrive_bytes + o_bytes + entries * G * 2 * 4;
  if (!workspace) {
    *workspace_bytes = size_t(need);
    return KVQ_OK;
  }
  if (int64_t(*workspace_bytes) < need) return KVQ_ERR_WORKSPACE;
  if (!cache || !seq_lens || !up_k || !up_v || !q || !out) return KVQ_ERR_NULL;
  if (!aligned(cache, 256) || !aligned(workspace, 256) || !aligned(up_k, 16) ||
      !aligned(up_v, 16) || !aligned(q, 16) || !aligned(out, 16))
    return KVQ_ERR_ALIGN;
  const std::vector<int64_t> base = row_bases(cfg);
  LatentArgs a{};
  a.cache = static_cast<const uint8_t*>(cache);
  a.seq_lens = seq_lens;
  a.q = static_cast<const uint16_t*>(q);
  a.out = static_cast<uint16_t*>(out);
  a.up_k = static_cast<const uint16_t*>(up_k);
  a.up_v = static_cast<const uint16_t*>(up_v);
  a.ws_arrive = static_cast<int32_t*>(workspace);
  a.ws_o = reinterpret_cast<float*>(static_cast<uint8_t*>(workspace) + arrive_bytes);
  a.ws_ml = reinterpret_cast<float*>(static_cast<uint8_t*>(workspace) + arrive_bytes + o_bytes);
  a.qscale = sm_scale * 1.4426950408889634f;
  a.plane_bytes = plane_bytes_of(cfg);
  a.Hkv = Hkv;
  a.Hq = cfg->num_q_heads;
  a.G = G;
  a.B = cfg->batch;
  a.layer_begin = layer_begin;
  a.nl = num_layers;
  a.chunk = chunk;
  a.claim_steps = chunk_tokens == 0;
  a.max_chunks = max_chunks;
  for (int s0 = 0; s0 < cfg->batch; s0 += kMaxSeq) {
    const int ns = std::min(kMaxSeq, cfg->batch - s0);
    a.seq_off = s0;
    a.n_seq = ns;
    a.nxcum[0] = 0;
    for (int i = 0; i < ns; ++i) {
      a.row0[i] = int32_t(base[s0 + i]);
      a.cap[i] = cfg->capacity[s0 + i];
      a.nxcum[i + 1] = a.nxcum[i] + (a.cap[i] + chunk - 1) / chunk;
    }
    if (int64_t(num_layers) * Hkv * a.nxcum[ns] > int64_t(0x7FFFFFFF)) return KVQ_ERR_UNSUPPORTED;
    if (dispatch_latent(D, R, a, static_cast<hipStream_t>(stream)) != hipSuccess)
      return KVQ_ERR_HIP;
  }
  return KVQ_OK;
}
