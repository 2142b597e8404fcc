/*
 * kvq_oracle.h -- plain, slow CPU oracle for the compressed-KV decode path.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library links or calls
 * this code; only the tests, the smoke check and the benchmark's CPU-baseline
 * leg do.  It shares no source with the GPU path.
 *
 * What it computes (sources: the pages listed in the functions below):
 *   - historical K/V of one (layer, KV head) stored per token; tokens inside
 *     the sequence's visual span are stored as b-bit codes (b in {2,4,8}) with
 *     one (fp16 scale, fp16 min) pair per group of g values along the head
 *     dimension; text tokens and protected heads (b = 16) keep bfloat16
 *     (nuiw.github.io "VLM_KV_Quantization" sections 1-2: only the historical
 *     cache is compressed, Visual/Text and K/V handled separately; HeadGuard
 *     briefing: ~1/8 of physical KV heads keep image K and optionally V in
 *     bf16);
 *   - dequantisation x^ = code * scale + min, exact in double;
 *   - single-query softmax attention over the dequantised rows, in double,
 *     and the KL divergence between two attention distributions
 *     (VLM_KV_Quantization section 3, D_KL(P_FP16 || P_Q)).
 *
 * Arithmetic is IEEE-754 binary32 where the quantiser fixes it (built with
 * -ffp-contract=off, no fast-math) and binary64 elsewhere.  The fp16/bf16
 * conversions are written from the IEEE-754 encoding definitions.
 */
#ifndef KVQ_ORACLE_H
#define KVQ_ORACLE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct {
  int32_t num_layers, batch, num_q_heads, num_kv_heads, head_dim, group_size;
  const int32_t *capacity;  /* [batch] rows reserved per sequence */
  const int32_t *vis_begin; /* [batch] visual span [vis_begin, vis_end) */
  const int32_t *vis_end;
  const uint8_t *k_bits; /* [num_layers*num_kv_heads] in {2,4,8,16} */
  const uint8_t *v_bits;
  int32_t rotate_k;      /* nonzero: K rows stored as codes are rotated first
                            (orc_hadamard_rotate); every other row is not */
  int32_t k_per_channel; /* nonzero: K codes are grouped per channel over
                            blocks of group_size consecutive visual tokens
                            (see orc_store_rows); V stays per token */
  /* Optional (NULL: none).  Ranges of positions inside a sequence's visual
   * span that are stored bf16 like text: sequence s owns ranges
   * [bf16_range_begin[k], bf16_range_end[k]) for k in
   * [bf16_range_offsets[s], bf16_range_offsets[s + 1]), each non-empty,
   * inside [vis_begin, vis_end), sorted and disjoint.  A one-token range
   * protects that token; a range between two images splits the span into
   * two visual spans.  Not combinable with k_per_channel. */
  const int32_t *bf16_range_offsets; /* [batch + 1] */
  const int32_t *bf16_range_begin;
  const int32_t *bf16_range_end;
} orc_config;

typedef struct {
  uint64_t total_bytes, payload_bytes, code_bytes, meta_bytes;
  uint64_t bf16_visual_bytes, bf16_text_bytes, quantized_values, stored_values;
} orc_cache_info;

/* ---- IEEE-754 conversions -------------------------------------------- */
uint16_t orc_f16_round_down(float x); /* largest binary16 <= x; zero -> +0 */
uint16_t orc_f16_round_up(float x);   /* smallest binary16 >= x; zero -> +0 */
double orc_f16_value(uint16_t h);
uint16_t orc_bf16_round_nearest_even(float x);
double orc_bf16_value(uint16_t b);

/* ---- rotation ------------------------------------------------------------ */
/* Weight-free stand-in for the outlier-removing rotation that gist.science
 * 2604.02570 (WSVD, section 2-C) places before quantisation: the normalised
 * Walsh-Hadamard matrix in Sylvester order, H[i][j] = (-1)^popcount(i & j).
 * Forward, in binary32: for s = 1, 2, 4, ..., D/2 every pair (i, i + s) with
 * bit s of i clear becomes (x_i + x_(i+s), x_i - x_(i+s)); then every value is
 * scaled by 2^-ceil(log2(D)/2) (exact).  The matching scale on the query side
 * is 2^-floor(log2(D)/2), so the two scales times D are exactly 1 and
 * <rot_q(q), rot_k(k)> = <q, k> in exact arithmetic.  D a power of two. */
void orc_hadamard_rotate(float *x, int D);
/* Inverse of the forward rotation in binary64: x = 2^-floor(log2(D)/2) H y. */
void orc_hadamard_unrotate(double *y, int D);

/* ---- quantiser ---------------------------------------------------------- */
/* One group of g values -> g codes plus fp16 (scale, min) bit patterns. */
void orc_quantize_group(const float *x, int g, int bits, uint8_t *codes,
                        uint16_t *scale16, uint16_t *min16);
/* Round half to even, from the definition (no libm call). */
double orc_round_half_even(double v);

/* ---- layout --------------------------------------------------------------- */
int orc_validate(const orc_config *c);
int orc_cache_bytes(const orc_config *c, orc_cache_info *info);
/* Byte offsets of the three planes of (layer, head, X), X = 0 for K, 1 for V.
 * A plane that has no rows gets its offset anyway (size 0). */
int orc_plane_offsets(const orc_config *c, int layer, int head, int X,
                      uint64_t *vis, uint64_t *meta, uint64_t *txt);
/* End of the coded part of sequence s's visual span.  Per-token grouping
 * codes the whole span [vis_begin, vis_end).  With k_per_channel the span is
 * coded in whole blocks of group_size tokens from vis_begin; the tail that
 * does not fill a block (the newest visual tokens, a residual window of
 * fewer than group_size tokens) is stored bf16 like text, for K and V.     */
int orc_coded_end(const orc_config *c, int seq);
/* Is position t of sequence s coded (a VIS row when its head's width is
 * below 16)?  Coded: vis_begin <= t < orc_coded_end and t in no bf16 range. */
int orc_is_coded(const orc_config *c, int seq, int t);
/* Where the row of position t of sequence s lives: plane 0 = VIS, 2 = TXT;
 * row index within that plane.  Coded positions take VIS rows in order,
 * sequence after sequence; every other position takes TXT rows in order:
 * VIS row = (coded positions of earlier sequences) + (coded positions of
 * this sequence before t), TXT row likewise over the other positions. */
int orc_row_of(const orc_config *c, int seq, int t, int *plane, int64_t *row);

/* ---- store / load ---------------------------------------------------------- */
/* Store rows t0..t1-1 of (layer, seq, head, X) from float32 src [(t1-t0), D].
 * Per-token groups (V always, K unless k_per_channel): each coded row's D
 * values form D/g groups along the head dimension, one (scale, min) pair per
 * group in the row's META row.  Per-channel K (k_per_channel, coded K rows):
 * block j of a sequence is its coded positions [vis_begin + j g,
 * vis_begin + (j + 1) g); for each channel d the g values of the block form
 * one group, quantised exactly as a per-token group; codes sit in each
 * token's VIS row as usual, and the block's META row holds D (scale, min)
 * pairs in channel order (VIS row r belongs to block row r / g).  Such a
 * store must cover every block it touches entirely (return 5 otherwise). */
int orc_store_rows(const orc_config *c, uint8_t *cache, int layer, int seq,
                   int head, int X, int t0, int t1, const float *src);
/* Dequantised row of position t as exact doubles [D]. */
/* The row's stored values, dequantised, in the stored (for rotated K rows,
 * rotated) domain; orc_load_row returns the reconstruction in the original
 * domain (the rotation undone in binary64). */
int orc_load_row_stored(const orc_config *c, const uint8_t *cache, int layer, int seq,
                        int head, int X, int t, double *out);
int orc_load_row(const orc_config *c, const uint8_t *cache, int layer, int seq,
                 int head, int X, int t, double *out);

/* ---- attention ------------------------------------------------------------- */
/* out[D] = softmax(scale * K q) V over T rows (row-major [T, D]); lse gets
 * log(sum exp(scale * K q)) in natural log.  All double. */
void orc_attention(const double *q, const double *K, const double *V, int T,
                   int D, double scale, double *out, double *lse);
/* Full decode for one (layer, seq, q-head): dequantise rows [0, len) of the
 * KV head this query head reads, then attention. q_bf16 is the query's bf16
 * bits [D]. scores (optional, [len]) receive the scaled logits. */
int orc_decode_one(const orc_config *c, const uint8_t *cache, int layer,
                   int seq, int qhead, int len, const uint16_t *q_bf16,
                   float sm_scale, double *out, double *lse, double *scores);
/* All (layer in [l0, l0+nl), seq, q-head): q/out laid out [nl, batch, Hq, D].
 * lens [batch].  Returns 0 on success. */
int orc_decode_all(const orc_config *c, const uint8_t *cache, int l0, int nl,
                   const int32_t *lens, const uint16_t *q_bf16, float sm_scale,
                   double *out);
/* KL(P || Q) for two logit vectors of length T (natural log). */
double orc_kl_logits(const double *s_p, const double *s_q, int T);

#ifdef __cplusplus
}
#endif
#endif
