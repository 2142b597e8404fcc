// kvq_decode.hip -- split-K decode attention over the compressed cache:
// the general VALU split kernel and the log-sum-exp merge (gfx950).
//
// Flash-decoding pattern with reconstruction on chip: each workgroup takes
// one token chunk of one (layer, sequence, KV head), reconstructs K/V rows in
// registers (code * scale + min, or bf16), and produces for each of the G
// query heads of the group a partial (o / l, m, l) with m the running max of
// the log2-domain scores.  Nothing reconstructed is written to memory
// (gist.science 2604.02570 section 2-D describes this fused pattern for a
// low-rank cache; here the compressed form is the quantised one).  The merge
// kernel combines the chunks of a query head:
//   M = max_c m_c,  w_c = l_c 2^(m_c - M),  out = sum_c w_c o_c / sum_c w_c.
//
// This file's split kernel is the general one: one token per lane for q.k,
// one or two head-dim elements per lane for p.v, plain fp32 FMAs.  The
// matrix-core kernel (kvq_decode_mfma.hip) covers the common shapes faster.
#include <hip/hip_runtime.h>

#include "kvq_internal.h"

namespace kvq {
namespace {

__device__ inline float bf16f(uint32_t b) { return __builtin_bit_cast(float, b << 16); }
__device__ inline float f16f(uint32_t b) { return (float)__builtin_bit_cast(_Float16, uint16_t(b)); }

__device__ inline float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}
__device__ inline float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

// Where the rows of one (layer, head, X) live, and how position t maps.
struct RowSrc {
  const uint8_t* vis;
  const uint8_t* meta;
  const uint8_t* txt;
  int bits;
};

__device__ inline RowSrc row_src(const DecodeArgs& a, int slot, int X) {
  RowSrc r;
  r.vis = a.cache + uint64_t(a.base256[slot][X]) * 256u;
  r.bits = a.bits[slot][X];
  r.meta = r.vis + meta_plane_offset(a.Rvis, a.D, r.bits);
  r.txt = r.vis + txt_plane_offset(a.Rvis, a.D, a.g, r.bits);
  return r;
}

// Reconstruct elements [d0, d0 + n) of the row at position t.
template <int N>
__device__ inline void load_elems(const DecodeArgs& a, const RowSrc& r, int vb, int ve,
                                  int64_t vrow0, int64_t trow0, int t, int d0, float (&v)[N]) {
  const int D = a.D;
  if (t >= vb && t < ve && r.bits < 16) {
    const int64_t row = vrow0 + (t - vb);
    const uint8_t* codes = r.vis + row * (D * r.bits / 8);
    const uint8_t* meta = r.meta + row * ((D / a.g) * 4);
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const int d = d0 + i;
      const int bit = d * r.bits;
      const uint32_t c = (uint32_t(codes[bit >> 3]) >> (bit & 7)) & ((1u << r.bits) - 1u);
      const uint32_t m = *reinterpret_cast<const uint32_t*>(meta + (d / a.g) * 4);
      v[i] = float(c) * f16f(m & 0xFFFFu) + f16f(m >> 16);
    }
  } else {
    const uint16_t* row;
    if (t >= vb && t < ve)
      row = reinterpret_cast<const uint16_t*>(r.vis) + (vrow0 + (t - vb)) * D;
    else
      row = reinterpret_cast<const uint16_t*>(r.txt) + (trow0 + (t < vb ? t : t - (ve - vb))) * D;
#pragma unroll
    for (int i = 0; i < N; ++i) v[i] = bf16f(row[d0 + i]);
  }
}

template <int D>
__global__ __launch_bounds__(256) void decode_simple_kernel(DecodeArgs a) {
  constexpr int DPL = D / 64;  // head-dim elements per lane in p.v
  constexpr int NW = 4;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int slot = blockIdx.y;
  const int lh = a.lh_glob[slot];
  const int l_local = lh / a.Hkv, h = lh % a.Hkv;
  const int sl = blockIdx.z, s = a.seq_off + sl;
  const int nxs = a.nxcum[sl + 1] - a.nxcum[sl];  // workgroups of this (layer, seq, head); chunk mode
  if (int(blockIdx.x) >= nxs) return;
  const int cap = a.cap[sl];
  int len = a.seq_lens[s];
  len = len < 1 ? 1 : (len > cap ? cap : len);
  const int t0 = min(int(blockIdx.x) * a.chunk, len);  // empty when past len
  const int t1 = min(t0 + a.chunk, len);
  const int G = a.G;
  const int vb = a.vb[sl], ve = a.ve[sl];
  const int64_t vrow0 = a.vrow0[sl], trow0 = a.trow0[sl];
  const RowSrc ks = row_src(a, slot, 0), vs = row_src(a, slot, 1);

  __shared__ float q_s[kMaxGroupRatio][D];
  __shared__ float p_s[NW][kMaxGroupRatio][64];
  __shared__ float red_ml[NW][kMaxGroupRatio][2];
  __shared__ float red_o[NW][kMaxGroupRatio][D];

  const uint16_t* qp = a.q + ((int64_t(l_local) * a.B + s) * a.Hq + int64_t(h) * G) * D;
  for (int i = threadIdx.x; i < G * D; i += 256)
    q_s[i / D][i % D] = bf16f(qp[i]) * a.qscale;
  __syncthreads();

  float m[kMaxGroupRatio], l[kMaxGroupRatio], o[kMaxGroupRatio][DPL];
#pragma unroll
  for (int j = 0; j < kMaxGroupRatio; ++j) {
    m[j] = -INFINITY;
    l[j] = 0.0f;
#pragma unroll
    for (int e = 0; e < DPL; ++e) o[j][e] = 0.0f;
  }

  for (int tt = t0 + wave * 64; tt < t1; tt += NW * 64) {
    const int t = tt + lane;
    const bool valid = t < t1;
    const int tc = valid ? t : t1 - 1;
    float sc[kMaxGroupRatio];
#pragma unroll
    for (int j = 0; j < kMaxGroupRatio; ++j) sc[j] = 0.0f;
    for (int d0 = 0; d0 < D; d0 += 8) {
      float kv[8];
      load_elems<8>(a, ks, vb, ve, vrow0, trow0, tc, d0, kv);
#pragma unroll
      for (int j = 0; j < kMaxGroupRatio; ++j) {
        if (j < G) {
#pragma unroll
          for (int i = 0; i < 8; ++i) sc[j] += q_s[j][d0 + i] * kv[i];
        }
      }
    }
#pragma unroll
    for (int j = 0; j < kMaxGroupRatio; ++j) {
      if (j < G) {
        const float sj = valid ? sc[j] : -INFINITY;
        const float mn = fmaxf(m[j], wave_max(sj));
        const float alpha = exp2f(m[j] - mn);
        const float p = valid ? exp2f(sj - mn) : 0.0f;
        l[j] = l[j] * alpha + wave_sum(p);
#pragma unroll
        for (int e = 0; e < DPL; ++e) o[j][e] *= alpha;
        m[j] = mn;
        p_s[wave][j][lane] = p;
      }
    }
    __builtin_amdgcn_wave_barrier();  // p_s is written and read by this wave only
    const int nvalid = min(64, t1 - tt);
    for (int u = 0; u < nvalid; ++u) {
      float vv[DPL];
      load_elems<DPL>(a, vs, vb, ve, vrow0, trow0, tt + u, lane * DPL, vv);
#pragma unroll
      for (int j = 0; j < kMaxGroupRatio; ++j) {
        if (j < G) {
          const float p = p_s[wave][j][u];
#pragma unroll
          for (int e = 0; e < DPL; ++e) o[j][e] += p * vv[e];
        }
      }
    }
    __builtin_amdgcn_wave_barrier();
  }

  // combine the NW waves of the block
#pragma unroll
  for (int j = 0; j < kMaxGroupRatio; ++j) {
    if (j < G) {
      if (lane == 0) {
        red_ml[wave][j][0] = m[j];
        red_ml[wave][j][1] = l[j];
      }
#pragma unroll
      for (int e = 0; e < DPL; ++e) red_o[wave][j][lane * DPL + e] = o[j][e];
    }
  }
  __syncthreads();
  const int64_t pidx = partial_index(l_local, s, h, blockIdx.x, a.B, a.Hkv, a.max_chunks);
  if (blockIdx.x == 0 && threadIdx.x == 0)
    a.ws_cnt[(int64_t(l_local) * a.B + s) * a.Hkv + h] = nxs;
  for (int i = threadIdx.x; i < G * D; i += 256) {
    const int j = i / D, d = i % D;
    float M = -INFINITY;
    for (int w = 0; w < NW; ++w)
      if (red_ml[w][j][1] > 0.0f) M = fmaxf(M, red_ml[w][j][0]);
    float L = 0.0f, acc = 0.0f;
    for (int w = 0; w < NW; ++w) {
      if (red_ml[w][j][1] > 0.0f) {
        const float sc = exp2f(red_ml[w][j][0] - M);
        L += red_ml[w][j][1] * sc;
        acc += red_o[w][j][d] * sc;
      }
    }
    const float o = L > 0.0f ? acc / L : 0.0f;  // L == 0: no token in this workgroup
    if (nxs == 1) {
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

// One block of 64 lanes per (layer-local, sequence, query head).
template <int D>
__global__ __launch_bounds__(64) void decode_merge_kernel(DecodeArgs a) {
  constexpr int DPL = D / 64;
  const int i = blockIdx.x;          // query head
  const int sl = blockIdx.y, s = a.seq_off + sl;
  const int l_local = blockIdx.z;
  const int lane = threadIdx.x;
  const int G = a.G, h = i / G, j = i % G;
  const int nc = a.ws_cnt[(int64_t(l_local) * a.B + s) * a.Hkv + h];
  if (nc <= 1) return;  // one workgroup: the split kernel wrote the output
  const int64_t p0 = partial_index(l_local, s, h, 0, a.B, a.Hkv, a.max_chunks);
  float M = -INFINITY;
  for (int c = 0; c < nc; ++c) {
    const float* ml = a.ws_ml + ((p0 + c) * G + j) * 2;
    if (ml[1] > 0.0f) M = fmaxf(M, ml[0]);
  }
  float W = 0.0f, acc[DPL];
#pragma unroll
  for (int e = 0; e < DPL; ++e) acc[e] = 0.0f;
  for (int c = 0; c < nc; ++c) {
    const float* ml = a.ws_ml + ((p0 + c) * G + j) * 2;
    if (!(ml[1] > 0.0f)) continue;  // empty workgroup
    const float w = ml[1] * exp2f(ml[0] - M);
    W += w;
    const float* op = a.ws_o + ((p0 + c) * G + j) * D + lane * DPL;
#pragma unroll
    for (int e = 0; e < DPL; ++e) acc[e] += w * op[e];
  }
  uint16_t* outp = a.out + ((int64_t(l_local) * a.B + s) * a.Hq + i) * D + lane * DPL;
#pragma unroll
  for (int e = 0; e < DPL; ++e) outp[e] = __builtin_bit_cast(uint16_t, (__bf16)(acc[e] / W));
}

}  // namespace

hipError_t launch_decode_simple(const DecodeArgs& a, int n_seq_launch, hipStream_t stream) {
  dim3 grid(a.max_chunks, a.n_lh, n_seq_launch);
  if (a.D == 128)
    hipLaunchKernelGGL(decode_simple_kernel<128>, grid, dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL(decode_simple_kernel<64>, grid, dim3(256), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_decode_merge(const DecodeArgs& a, int nl, int n_seq_launch,
                               hipStream_t stream) {
  dim3 grid(a.Hq, n_seq_launch, nl);
  if (a.D == 128)
    hipLaunchKernelGGL(decode_merge_kernel<128>, grid, dim3(64), 0, stream, a);
  else
    hipLaunchKernelGGL(decode_merge_kernel<64>, grid, dim3(64), 0, stream, a);
  return hipGetLastError();
}

}  // namespace kvq
