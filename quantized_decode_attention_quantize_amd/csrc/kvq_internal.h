// kvq_internal.h -- launch arguments and device helpers shared by the libkvq
// HIP sources.  Not part of the public ABI (see include/kvq.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kvq {

// Per-launch limits of the by-value kernel arguments.  A call that touches
// more (layer, KV head) pairs or sequences is split into several launches by
// the host code.
constexpr int kMaxLH = 128;   // (layer, KV head) pairs per launch
constexpr int kMaxSeq = 64;   // sequences per launch
constexpr int kMaxGroupRatio = 16;  // Hq / Hkv supported by the decode kernels

// Width codes for the per-(layer, head, X) row formats.
__host__ __device__ constexpr int vis_row_bytes(int D, int bits) {
  return bits == 16 ? 2 * D : D * bits / 8;
}
__host__ __device__ constexpr int64_t align256(int64_t x) { return (x + 255) & ~int64_t(255); }

// Byte offsets of the META and TXT planes of one (layer, head, X) relative to
// its VIS plane.  Rvis is the total number of visual rows (all sequences).
__host__ __device__ inline int64_t meta_plane_offset(int64_t Rvis, int D, int bits) {
  return align256(Rvis * vis_row_bytes(D, bits));
}
__host__ __device__ inline int64_t txt_plane_offset(int64_t Rvis, int D, int g, int bits) {
  return meta_plane_offset(Rvis, D, bits) + (bits < 16 ? align256(Rvis * (D / g) * 4) : 0);
}

struct QuantizeArgs {
  uint8_t* cache;
  const void* k_src;
  const void* v_src;
  int64_t Rvis;
  int D, g, src_bf16;
  int tok_begin, n_tok;   // positions [tok_begin, tok_begin + n_tok)
  int num_seqs_total;     // seq count of the source tensors
  int seq_off;            // first source sequence covered by this launch
  int Hkv;
  int lh_off;             // first (layer-local * Hkv + head) of this launch
  uint32_t base256[kMaxLH][2];  // VIS plane offset / 256 per (lh, X)
  uint8_t bits[kMaxLH][2];
  int32_t vb[kMaxSeq], ve[kMaxSeq], vrow0[kMaxSeq], trow0[kMaxSeq];
};

struct DecodeArgs {
  const uint8_t* cache;
  const int32_t* seq_lens;  // device [batch], global sequence ids
  const uint16_t* q;        // bf16 [nl, B, Hq, D]
  uint16_t* out;            // bf16 [nl, B, Hq, D]
  float* ws_o;              // [entries][G][D] normalised partial outputs
  float* ws_ml;             // [entries][G][2] (running max m in log2 units, sum l)
  float qscale;             // sm_scale * log2(e)
  int64_t Rvis;
  int D, g, G, Hkv, Hq, B;
  int chunk, max_chunks;
  int seq_off;              // first global sequence of this launch
  int n_lh;                 // (layer-local, head) pairs in this launch
  uint16_t lh_glob[kMaxLH];  // grid.y slot -> layer_local * Hkv + head
  uint32_t base256[kMaxLH][2];  // per slot: VIS plane offset / 256 of K and V
  uint8_t bits[kMaxLH][2];
  int32_t vb[kMaxSeq], ve[kMaxSeq], cap[kMaxSeq], vrow0[kMaxSeq], trow0[kMaxSeq];
};

// Index of a split partial: (layer-local l, global seq s, head h, chunk x).
__host__ __device__ inline int64_t partial_index(int l, int s, int h, int x, int B, int Hkv,
                                                 int max_chunks) {
  return ((int64_t(l) * B + s) * Hkv + h) * max_chunks + x;
}

hipError_t launch_quantize(const QuantizeArgs& a, int n_lh_launch, int n_seq_launch,
                           hipStream_t stream);
hipError_t launch_decode_simple(const DecodeArgs& a, int n_seq_launch, hipStream_t stream);
// Matrix-core split kernel: needs (D / g) * G <= 16 (one 16-row MFMA tile of
// (head, group) columns); writes the final output itself when max_chunks == 1.
bool mfma_supported(int D, int g, int G);
hipError_t launch_decode_mfma(const DecodeArgs& a, int n_seq_launch, hipStream_t stream);
hipError_t launch_decode_merge(const DecodeArgs& a, int nl, int n_seq_launch,
                               hipStream_t stream);

}  // namespace kvq
