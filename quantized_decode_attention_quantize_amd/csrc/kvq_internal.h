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
constexpr int kMaxRangesQ = 64;     // bf16 ranges per quantize launch
constexpr int kMaxRangesD = 36;     // bf16 ranges per decode launch (and per sequence)

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
  int rotate_k;           // coded K rows are Walsh-Hadamard rotated first
  int n_tok;              // rows per sequence: positions [tok0[s], tok0[s] + n_tok)
  int num_seqs_total;     // seq count of the source tensors
  int seq_off;            // first source sequence covered by this launch
  int Hkv;
  int lh_off;             // first (layer-local * Hkv + head) of this launch
  uint32_t base256[kMaxLH][2];  // VIS plane offset / 256 per (lh, X)
  uint8_t bits[kMaxLH][2];
  int32_t vb[kMaxSeq], ve[kMaxSeq], vrow0[kMaxSeq], trow0[kMaxSeq];
  int32_t tok0[kMaxSeq];  // per sequence: first position stored (the call's
                          // n_tok rows start there)
  int32_t k_per_channel;  // K codes grouped per channel over g-token blocks
  int32_t kblk0[kMaxSeq];  // per sequence: first per-channel K block stored
  int32_t kblkn[kMaxSeq];  // per sequence: number of such blocks (0: none)
  // bf16 ranges inside the visual spans: sequence i owns ranges
  // [rng_first[i], rng_first[i + 1]) of this launch's table
  int32_t rng_first[kMaxSeq + 1];
  int32_t rng_b[kMaxRangesQ], rng_e[kMaxRangesQ];
};
static_assert(sizeof(QuantizeArgs) <= 4096, "QuantizeArgs must fit the kernel argument limit");

struct DecodeArgs {
  const uint8_t* cache;
  const int32_t* seq_lens;  // device [batch], global sequence ids
  const uint16_t* q;        // bf16 [nl, B, Hq, D]
  uint16_t* out;            // bf16 [nl, B, Hq, D]
  float* ws_o;              // [entries][G][D] normalised partial outputs
  float* ws_ml;             // [entries][G][2] (running max m in log2 units, sum l)
  int32_t* ws_cnt;          // [nl * B * Hkv] partial count of each (layer, seq, head)
  int32_t* ws_arrive;       // [nl * B * Hkv] arrival counters of the fused merge; zero
                            // between calls (the last arriving workgroup resets them)
  float qscale;             // sm_scale * log2(e)
  int64_t Rvis;
  int D, g, G, Hkv, Hq, B;
  int chunk;                // tokens per workgroup; 0 = balanced split (see nx)
  int max_chunks;           // partial slots per (layer, seq, head)
  int seq_off;              // first global sequence of this launch
  int n_lh;                 // (layer-local, head) pairs in this launch
  int n_seq;                // sequences in this launch
  uint16_t lh_glob[kMaxLH];  // grid.y slot -> layer_local * Hkv + head
  uint32_t base256[kMaxLH][2];  // per slot: VIS plane offset / 256 of K and V
  uint8_t bits[kMaxLH][2];
  // Work units (waves): slot i and sequence s get mult[i] * nx[s]
  // consecutive units, slot-major, so unit u of the launch decodes with two
  // searches.
  uint16_t mult[kMaxLH];    // per slot
  uint16_t mcum[kMaxLH + 1];  // per slot: sum of mult over earlier slots
  int32_t vb[kMaxSeq], ve[kMaxSeq], cap[kMaxSeq], vrow0[kMaxSeq], trow0[kMaxSeq];
  // per sequence: units of one slot with mult 1 before it (sequence i has
  // nx_i = nxcum[i + 1] - nxcum[i])
  int32_t nxcum[kMaxSeq + 1];
  int32_t rotate_k;         // coded K rows are stored rotated: rotate q for them
  int32_t k_per_channel;    // coded K rows carry per-channel (scale, min) per block
  // bf16 ranges inside the visual spans: sequence i owns ranges
  // [rng_first[i], rng_first[i + 1]) of this launch's table
  uint8_t rng_first[kMaxSeq + 1];
  uint8_t g_stride;         // query heads per KV head in q / out (G counts this
                            // launch's subgroup of them; q and out point at its first)
  uint8_t app_mode;         // decode-time append: 0 none, 1 bf16 sources, 2 fp32 sources
  uint8_t pad_;
  int32_t rng_b[kMaxRangesD], rng_e[kMaxRangesD];
  // append sources [nl, B, Hkv, D]: the row of position seq_lens[s] - 1 of
  // each (layer, seq, KV head), stored before it is attended
  const void* app_k;
  const void* app_v;
};
static_assert(sizeof(DecodeArgs) % 16 == 0, "DecodeArgs is copied in 16-byte pieces");
static_assert(sizeof(DecodeArgs) <= 4096, "DecodeArgs must fit the kernel argument limit");

// Unit u of a launch (see DecodeArgs::mult) -> slot, the sequence index
// within the launch and x, the unit's index among the mult[slot] * nx[seq]
// units of that (slot, sequence).  The layout leaves no idle units, so the
// round-robin dealing of workgroups to the XCDs stays even.
__device__ inline void decode_block(const DecodeArgs& a, int b, int n_seq, int& slot, int& sl,
                                    int& x) {
  const int per_mult = a.nxcum[n_seq];  // units of one slot with mult 1
  int lo = 0, hi = a.n_lh - 1;          // last slot with per_mult * mcum[slot] <= b
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (per_mult * int(a.mcum[mid]) <= b) lo = mid; else hi = mid - 1;
  }
  slot = lo;
  const int m = a.mult[slot];
  const int r = b - per_mult * int(a.mcum[slot]);
  lo = 0;
  hi = n_seq - 1;                       // last sequence with m * nxcum[seq] <= r
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (m * a.nxcum[mid] <= r) lo = mid; else hi = mid - 1;
  }
  sl = lo;
  x = r - m * a.nxcum[sl];
}

// Token range of wave `w` of workgroup `x` out of `nxs` workgroups of one
// (layer, seq, head) with `len` attended tokens.  chunk > 0: workgroup x takes
// [x * chunk, (x + 1) * chunk) and its waves split that evenly.  chunk == 0
// (balanced): the len tokens form ceil(len / 32) steps dealt into
// waves * nxs nearly equal wave units.
//
// phase (0..31) shifts the grid: ranges are cut from [0, len + phase) and then
// moved down by phase (the first range loses phase tokens), so position p
// starts a 32-token step when p + phase is a multiple of 32.  Per-channel K
// uses phase = (32 - vis_begin % 32) % 32, which starts every step of the
// coded span inside one g-token block.
__host__ __device__ inline void wave_range(int x, int w, int nxs, int len, int chunk,
                                           int waves, int& a, int& b, int phase = 0) {
  const int n = len + phase;
  if (chunk > 0) {
    const int per = chunk / waves;
    a = x * chunk + w * per;
    b = a + per;
    const int e = x * chunk + chunk;
    if (b > e) b = e;
  } else {
    const int64_t nblk = (n + 31) / 32, U = int64_t(waves) * nxs, u = int64_t(x) * waves + w;
    a = int(32 * (u * nblk / U));
    b = int(32 * ((u + 1) * nblk / U));
  }
  if (a > n) a = n;
  if (b > n) b = n;
  a = a < phase ? 0 : a - phase;
  b = b < phase ? 0 : b - phase;
}

// The unit of an entry (units [w0, w0 + ne) of a launch, `waves` units per
// workgroup) that takes all of the entry's text rows in the balanced split:
// the first unit of its largest piece -- the first full workgroup, else the
// larger of its two pieces -- so that the piece's claimed visual steps absorb
// the text steps and the decode-time append, which a piece of one or two
// waves cannot.
__host__ __device__ inline int text_unit(int w0, int ne, int waves) {
  const int room = waves - w0 % waves;
  const int n1 = ne < room ? ne : room;  // units in the entry's first piece
  if (n1 == ne || n1 == waves) return 0;
  if (ne - n1 >= waves) return n1;        // the entry's next workgroup is full
  return n1 >= ne - n1 ? 0 : n1;
}

// Index of a split partial: (layer-local l, global seq s, head h, chunk x).
__host__ __device__ inline int64_t partial_index(int l, int s, int h, int x, int B, int Hkv,
                                                 int max_chunks) {
  return ((int64_t(l) * B + s) * Hkv + h) * max_chunks + x;
}

// Compute units of the current device, read once per device (256 when no
// device can be queried).
int device_cus();

hipError_t launch_quantize(const QuantizeArgs& a, int n_lh_launch, int n_seq_launch,
                           hipStream_t stream);
// Per-channel K blocks of a launch (k_per_channel): one workgroup per
// (layer-head slot, sequence, block); max_blocks = the largest kblkn.
hipError_t launch_quantize_kblocks(const QuantizeArgs& a, int n_lh_launch, int n_seq_launch,
                                   int max_blocks, hipStream_t stream);
// Matrix-core split kernel: one 16-row MFMA tile of (head, group) columns,
// i.e. (D / g) * G <= 16 query heads of each KV head per launch; writes the
// final output itself when max_chunks == 1.
bool mfma_supported(int D, int g, int G);
// Launches (query-head subgroups) a call with G query heads per KV head
// needs, each of at most ceil(G / n) heads: ceil(G * (D / g) / 16).
int mfma_subgroups(int D, int g, int G);
// kb, vb: the visual widths every non-bf16 (layer, head) pair of the launch has.
hipError_t launch_decode_mfma(const DecodeArgs& a, int kb, int vb, hipStream_t stream);
hipError_t launch_decode_mfma_128_1(const DecodeArgs& a, int kb, int vb, hipStream_t stream);
hipError_t launch_decode_mfma_128_2(const DecodeArgs& a, int kb, int vb, hipStream_t stream);
hipError_t launch_decode_mfma_128_4(const DecodeArgs& a, int kb, int vb, hipStream_t stream);
hipError_t launch_decode_mfma_64_1(const DecodeArgs& a, int kb, int vb, hipStream_t stream);
hipError_t launch_decode_mfma_64_2(const DecodeArgs& a, int kb, int vb, hipStream_t stream);
constexpr int kMfmaWaves = 8;      // waves per workgroup of the matrix-core kernel

}  // namespace kvq
