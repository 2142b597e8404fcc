/*
 * kvq_oracle.c -- plain CPU oracle (TEST INFRASTRUCTURE ONLY; see the header).
 *
 * Build: gcc -std=c11 -O2 -ffp-contract=off -fno-fast-math -fPIC -shared
 * (no FMA contraction: every binary32 operation below is one IEEE operation
 * rounded to nearest even, as the quantiser definition requires).
 *
 * Method sources:
 *   [P4] nuiw.github.io "VLM_KV_Quantization": the historical K/V cache of a
 *        VLM stored at FP16 / INT8 / INT4 / INT2, Visual vs Text tokens and K vs
 *        V treated separately, same group size for every setting (sections
 *        1, 2 and 4); the KL divergence of section 3.
 *   [P1] jiinsi.com HeadGuard briefing: selected physical KV heads keep image
 *        Key (and optionally Value) at bf16 on top of any low-bit quantiser.
 * The quantiser form the pages leave open is read as group-wise asymmetric
 * min-max: min rounded down and scale rounded up to binary16 so the stored
 * pair still covers the group, codes rounded half to even.
 */
#include "kvq_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------------ */
/* IEEE-754 binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits.
 * Normal values (1 + f/2^10) 2^(e-15) for e = 1..30, subnormals f 2^-24,
 * largest finite 65504.  The spacing of binary16 numbers around a positive
 * magnitude a is 2^-24 below 2^-14, else 2^(floor(log2 a) - 10).           */

static double f16_spacing(double a) {
  int e;
  if (a < 0x1p-14) return 0x1p-24;
  frexp(a, &e); /* a = m 2^e with m in [0.5, 1): floor(log2 a) = e - 1 */
  return ldexp(1.0, e - 1 - 10);
}

static uint16_t f16_encode_magnitude(double v) {
  int e;
  double m;
  if (v == 0.0) return 0;
  if (isinf(v) || v > 65504.0) return 0x7C00;
  if (v < 0x1p-14) return (uint16_t)(v / 0x1p-24); /* exact integer */
  m = frexp(v, &e);                                 /* v = (2m) 2^(e-1) */
  return (uint16_t)(((e - 1 + 15) << 10) | (uint16_t)((2.0 * m - 1.0) * 1024.0));
}

/* Magnitudes of the two binary16 neighbours of a > 0: toward zero and away. */
static void f16_neighbours(double a, double *toward, double *away, int *exact) {
  double q, t;
  if (a > 65504.0) { *toward = 65504.0; *away = INFINITY; *exact = 0; return; }
  q = f16_spacing(a);
  t = floor(a / q) * q; /* exact: q is a power of two */
  *toward = t;
  *exact = (t == a);
  *away = *exact ? t : t + q;
}

uint16_t orc_f16_round_down(float x) {
  double a, tw, aw, v;
  int ex;
  if (x == 0.0f) return 0; /* zero is stored as +0 */
  a = fabs((double)x);
  f16_neighbours(a, &tw, &aw, &ex);
  v = (x > 0.0f) ? tw : aw;
  if (v == 0.0) return 0;
  return (uint16_t)((x < 0.0f ? 0x8000u : 0u) | f16_encode_magnitude(v));
}

uint16_t orc_f16_round_up(float x) {
  double a, tw, aw, v;
  int ex;
  if (x == 0.0f) return 0;
  a = fabs((double)x);
  f16_neighbours(a, &tw, &aw, &ex);
  v = (x > 0.0f) ? aw : tw;
  if (v == 0.0) return 0;
  return (uint16_t)((x < 0.0f ? 0x8000u : 0u) | f16_encode_magnitude(v));
}

double orc_f16_value(uint16_t h) {
  int s = h >> 15, e = (h >> 10) & 31, f = h & 1023;
  double v;
  if (e == 0) v = f * 0x1p-24;
  else if (e == 31) v = f ? NAN : INFINITY;
  else v = ldexp(1.0 + f / 1024.0, e - 15);
  return s ? -v : v;
}

/* IEEE-754 bfloat16: 1 sign, 8 exponent (bias 127), 7 fraction bits.  The
 * spacing around a is 2^-133 below 2^-126, else 2^(floor(log2 a) - 7).     */
uint16_t orc_bf16_round_nearest_even(float x) {
  double a = fabs((double)x), q, v, f, r;
  int e;
  uint16_t sign = (x < 0.0f || (x == 0.0f && signbit(x))) ? 0x8000u : 0u, mag;
  if (isnan(x)) return 0x7FC0;
  if (isinf(x)) return (uint16_t)(sign | 0x7F80);
  if (a == 0.0) return sign;
  if (a < 0x1p-126) q = 0x1p-133;
  else { frexp(a, &e); q = ldexp(1.0, e - 1 - 7); }
  v = a / q;
  f = floor(v);
  r = v - f;
  if (r > 0.5 || (r == 0.5 && fmod(f, 2.0) != 0.0)) f += 1.0;
  v = f * q; /* may be the next binade's first value: still exact */
  if (v >= 0x1p128) return (uint16_t)(sign | 0x7F80);
  if (v < 0x1p-126) mag = (uint16_t)(v / 0x1p-133);
  else {
    double m = frexp(v, &e);
    mag = (uint16_t)(((e - 1 + 127) << 7) | (uint16_t)((2.0 * m - 1.0) * 128.0));
  }
  return (uint16_t)(sign | mag);
}

double orc_bf16_value(uint16_t b) {
  int s = b >> 15, e = (b >> 7) & 255, f = b & 127;
  double v;
  if (e == 0) v = f * 0x1p-133;
  else if (e == 255) v = f ? NAN : INFINITY;
  else v = ldexp(1.0 + f / 128.0, e - 127);
  return s ? -v : v;
}

/* ------------------------------------------------------------------------ */
/* Quantiser                                                                */

double orc_round_half_even(double v) {
  double f = floor(v), r = v - f;
  if (r > 0.5) return f + 1.0;
  if (r < 0.5) return f;
  return (fmod(f, 2.0) == 0.0) ? f : f + 1.0;
}

/* Group-wise asymmetric min-max code of g values (one token, one group):
 *   mn16 = binary16 round-down of the group minimum
 *   sc16 = binary16 round-up of fl32(fl32(max - mn16) / (2^b - 1)),
 *          or 0 when fl32(max - mn16) is 0 (then every code is 0)
 *   code = clamp(round_half_even(fl32(fl32(x - mn16) / sc16)), 0, 2^b - 1)
 * so that code * sc16 + mn16 is within sc16/2 (plus binary32 rounding) of x. */
void orc_quantize_group(const float *x, int g, int bits, uint8_t *codes,
                        uint16_t *scale16, uint16_t *min16) {
  float lo = x[0], hi = x[0], mnf, range, step, scf;
  int i, n = (1 << bits) - 1;
  uint16_t mn, sc;
  for (i = 1; i < g; i++) {
    if (x[i] < lo) lo = x[i];
    if (x[i] > hi) hi = x[i];
  }
  mn = orc_f16_round_down(lo);
  mnf = (float)orc_f16_value(mn);
  range = hi - mnf;
  *min16 = mn;
  if (range == 0.0f) {
    *scale16 = 0;
    for (i = 0; i < g; i++) codes[i] = 0;
    return;
  }
  step = range / (float)n;
  sc = orc_f16_round_up(step);
  scf = (float)orc_f16_value(sc);
  *scale16 = sc;
  for (i = 0; i < g; i++) {
    float d = x[i] - mnf;
    float qv = d / scf;
    double r = orc_round_half_even((double)qv);
    if (r < 0.0) r = 0.0;
    if (r > (double)n) r = (double)n;
    codes[i] = (uint8_t)r;
  }
}

/* ------------------------------------------------------------------------ */
/* Layout: per (layer l, KV head h, X in {K, V}) three planes in this order:
 *   VIS  : one row per visual position, D*b/8 code bytes (2D bf16 bytes if b=16)
 *   META : one row per visual position when b < 16: for each group j of g
 *          values, fp16 scale then fp16 min, little-endian (4 bytes per group)
 *   TXT  : one bf16 row (2D bytes) per text position
 * Sequences are concatenated inside each plane in batch order.  Every plane
 * starts on a 256-byte boundary.  Code element d sits at bit d*b of the row's
 * little-endian byte string.                                               */

static uint64_t align256(uint64_t x) { return (x + 255u) & ~(uint64_t)255u; }

static int bits_ok(int b) { return b == 2 || b == 4 || b == 8 || b == 16; }

int orc_validate(const orc_config *c) {
  int s, i;
  if (!c || !c->capacity || !c->vis_begin || !c->vis_end || !c->k_bits || !c->v_bits)
    return 1;
  if (c->num_layers < 1 || c->batch < 1 || c->num_kv_heads < 1 || c->num_q_heads < 1)
    return 2;
  if (c->num_q_heads % c->num_kv_heads) return 2;
  if (c->head_dim < 1 || c->group_size < 1 || c->head_dim % c->group_size) return 3;
  if (c->rotate_k && (c->head_dim & (c->head_dim - 1))) return 3; /* rotation: D = 2^k */
  if (c->rotate_k && c->k_per_channel) return 3; /* one grouping of rotated rows only */
  if (c->bf16_range_offsets) {
    const int32_t *o = c->bf16_range_offsets;
    if (!c->bf16_range_begin || !c->bf16_range_end || o[0] != 0) return 5;
    for (s = 0; s < c->batch; s++) {
      int k, prev = c->vis_begin[s];
      if (o[s + 1] < o[s]) return 5;
      if (o[s + 1] > o[s] && c->k_per_channel) return 5; /* blocks must be contiguous */
      for (k = o[s]; k < o[s + 1]; k++) {
        if (c->bf16_range_begin[k] < prev || c->bf16_range_end[k] <= c->bf16_range_begin[k] ||
            c->bf16_range_end[k] > c->vis_end[s])
          return 5;
        prev = c->bf16_range_end[k];
      }
    }
  }
  for (i = 0; i < c->num_layers * c->num_kv_heads; i++) {
    if (!bits_ok(c->k_bits[i]) || !bits_ok(c->v_bits[i])) return 3;
    if ((c->head_dim * c->k_bits[i]) % 8 || (c->head_dim * c->v_bits[i]) % 8) return 3;
  }
  for (s = 0; s < c->batch; s++) {
    if (c->vis_begin[s] < 0 || c->vis_begin[s] > c->vis_end[s] ||
        c->vis_end[s] > c->capacity[s])
      return 4;
  }
  return 0;
}

int orc_coded_end(const orc_config *c, int seq) {
  int vb = c->vis_begin[seq], ve = c->vis_end[seq], g = c->group_size;
  return c->k_per_channel ? vb + (ve - vb) / g * g : ve;
}

/* Coded positions of sequence seq before position t: those of
 * [vis_begin, min(t, coded end)) minus the parts of its bf16 ranges there. */
static int64_t coded_before(const orc_config *c, int seq, int t) {
  int vb = c->vis_begin[seq], qe = orc_coded_end(c, seq), k;
  int hi = t < qe ? t : qe;
  int64_t n = hi > vb ? hi - vb : 0;
  if (c->bf16_range_offsets)
    for (k = c->bf16_range_offsets[seq]; k < c->bf16_range_offsets[seq + 1]; k++) {
      int b = c->bf16_range_begin[k], e = c->bf16_range_end[k] < hi ? c->bf16_range_end[k] : hi;
      if (e > b) n -= e - b;
    }
  return n;
}

int orc_is_coded(const orc_config *c, int seq, int t) {
  return coded_before(c, seq, t + 1) > coded_before(c, seq, t);
}

static void row_totals(const orc_config *c, uint64_t *rvis, uint64_t *rtxt) {
  uint64_t v = 0, all = 0;
  int s;
  for (s = 0; s < c->batch; s++) {
    v += (uint64_t)coded_before(c, s, c->capacity[s]);
    all += (uint64_t)c->capacity[s];
  }
  *rvis = v;
  *rtxt = all - v;
}

static uint64_t vis_row_bytes(int D, int b) {
  return b == 16 ? (uint64_t)2 * D : (uint64_t)D * b / 8;
}

int orc_cache_bytes(const orc_config *c, orc_cache_info *info) {
  uint64_t rvis, rtxt, D, G;
  int l, h, X, rc = orc_validate(c);
  if (rc) return rc;
  if (!info) return 1;
  memset(info, 0, sizeof(*info));
  row_totals(c, &rvis, &rtxt);
  D = (uint64_t)c->head_dim;
  G = D / (uint64_t)c->group_size;
  for (l = 0; l < c->num_layers; l++)
    for (h = 0; h < c->num_kv_heads; h++)
      for (X = 0; X < 2; X++) {
        int b = X ? c->v_bits[l * c->num_kv_heads + h] : c->k_bits[l * c->num_kv_heads + h];
        uint64_t vis = rvis * vis_row_bytes((int)D, b);
        uint64_t meta = b < 16 ? rvis * G * 4u : 0;
        uint64_t txt = rtxt * 2u * D;
        info->payload_bytes += vis + meta + txt;
        info->total_bytes += align256(vis) + align256(meta) + align256(txt);
        if (b < 16) {
          info->code_bytes += vis;
          info->meta_bytes += meta;
          info->quantized_values += rvis * D;
        } else {
          info->bf16_visual_bytes += vis;
        }
        info->bf16_text_bytes += txt;
        info->stored_values += (rvis + rtxt) * D;
      }
  return 0;
}

int orc_plane_offsets(const orc_config *c, int layer, int head, int X,
                      uint64_t *vis, uint64_t *meta, uint64_t *txt) {
  uint64_t rvis, rtxt, D, G, off = 0;
  int l, h, x;
  if (orc_validate(c)) return 1;
  if (layer < 0 || layer >= c->num_layers || head < 0 || head >= c->num_kv_heads ||
      X < 0 || X > 1)
    return 2;
  row_totals(c, &rvis, &rtxt);
  D = (uint64_t)c->head_dim;
  G = D / (uint64_t)c->group_size;
  for (l = 0; l < c->num_layers; l++)
    for (h = 0; h < c->num_kv_heads; h++)
      for (x = 0; x < 2; x++) {
        int b = x ? c->v_bits[l * c->num_kv_heads + h] : c->k_bits[l * c->num_kv_heads + h];
        uint64_t v = rvis * vis_row_bytes((int)D, b);
        uint64_t m = b < 16 ? rvis * G * 4u : 0;
        uint64_t t = rtxt * 2u * D;
        if (l == layer && h == head && x == X) {
          *vis = off;
          *meta = off + align256(v);
          *txt = off + align256(v) + align256(m);
          return 0;
        }
        off += align256(v) + align256(m) + align256(t);
      }
  return 3;
}

int orc_row_of(const orc_config *c, int seq, int t, int *plane, int64_t *row) {
  int64_t vbase = 0, tbase = 0, nc;
  int s;
  if (seq < 0 || seq >= c->batch || t < 0 || t >= c->capacity[seq]) return 1;
  for (s = 0; s < seq; s++) {
    int64_t nv = coded_before(c, s, c->capacity[s]);
    vbase += nv;
    tbase += c->capacity[s] - nv;
  }
  nc = coded_before(c, seq, t);
  if (orc_is_coded(c, seq, t)) {
    *plane = 0;
    *row = vbase + nc;
  } else {
    *plane = 2;
    *row = tbase + (t - nc);
  }
  return 0;
}

static void put_u16(uint8_t *p, uint16_t v) {
  p[0] = (uint8_t)(v & 255u);
  p[1] = (uint8_t)(v >> 8);
}

static uint16_t get_u16(const uint8_t *p) { return (uint16_t)(p[0] | (p[1] << 8)); }

/* ---- rotation (WSVD section 2-C, weight-free Walsh-Hadamard form) ------- */

static int log2_int(int D) {
  int k = 0;
  while ((1 << k) < D) k++;
  return k;
}

void orc_hadamard_rotate(float *x, int D) {
  int s, i;
  const float scale = ldexpf(1.0f, -((log2_int(D) + 1) / 2));
  for (s = 1; s < D; s <<= 1)
    for (i = 0; i < D; i++)
      if (!(i & s)) {
        const float a = x[i], b = x[i + s];
        x[i] = a + b;
        x[i + s] = a - b;
      }
  for (i = 0; i < D; i++) x[i] = x[i] * scale;
}

void orc_hadamard_unrotate(double *y, int D) {
  int s, i;
  const double scale = ldexp(1.0, -(log2_int(D) / 2));
  for (s = 1; s < D; s <<= 1)
    for (i = 0; i < D; i++)
      if (!(i & s)) {
        const double a = y[i], b = y[i + s];
        y[i] = a + b;
        y[i + s] = a - b;
      }
  for (i = 0; i < D; i++) y[i] *= scale;
}

/* Per-channel K (k_per_channel, b < 16): coded positions in whole blocks of
 * g tokens, one group per (block, channel); everything else bf16. */
static int store_k_blocks(const orc_config *c, uint8_t *cache, uint64_t vis, uint64_t meta,
                          uint64_t txt, int b, int seq, int t0, int t1, const float *src) {
  int D = c->head_dim, g = c->group_size, t, d, i;
  int vb = c->vis_begin[seq], qe = orc_coded_end(c, seq);
  int lo = t0 > vb ? t0 : vb, hi = t1 < qe ? t1 : qe; /* coded positions stored */
  uint64_t rb = (uint64_t)D * b / 8;
  float col[128];
  uint8_t codes[128];
  if (g > 128) return 2;
  if (lo < hi && ((lo - vb) % g || (hi - vb) % g)) return 5; /* a block cut apart */
  for (t = t0; t < t1; t++) { /* bf16 rows: text, and the residual window */
    int plane;
    int64_t row;
    if (orc_row_of(c, seq, t, &plane, &row)) return 3;
    if (plane == 2) {
      uint8_t *r = cache + txt + (uint64_t)row * 2u * D;
      for (d = 0; d < D; d++) put_u16(r + 2 * d, orc_bf16_round_nearest_even(src[(size_t)(t - t0) * D + d]));
    }
  }
  for (t = lo; t < hi; t += g) { /* block [t, t + g) */
    int plane;
    int64_t row;
    orc_row_of(c, seq, t, &plane, &row); /* the block's first VIS row */
    uint8_t *m = cache + meta + (uint64_t)(row / g) * (uint64_t)D * 4u;
    for (i = 0; i < g; i++) memset(cache + vis + (uint64_t)(row + i) * rb, 0, rb);
    for (d = 0; d < D; d++) {
      uint16_t s16, m16;
      for (i = 0; i < g; i++) col[i] = src[(size_t)(t + i - t0) * D + d];
      orc_quantize_group(col, g, b, codes, &s16, &m16);
      put_u16(m + 4 * d, s16);
      put_u16(m + 4 * d + 2, m16);
      for (i = 0; i < g; i++) {
        uint8_t *r = cache + vis + (uint64_t)(row + i) * rb;
        int bit = d * b;
        r[bit / 8] = (uint8_t)(r[bit / 8] | (codes[i] << (bit % 8)));
      }
    }
  }
  return 0;
}

int orc_store_rows(const orc_config *c, uint8_t *cache, int layer, int seq,
                   int head, int X, int t0, int t1, const float *src) {
  uint64_t vis, meta, txt;
  int D = c->head_dim, g = c->group_size, t, d, j;
  int b;
  uint8_t codes[1024];
  float rot[1024];
  if (orc_plane_offsets(c, layer, head, X, &vis, &meta, &txt)) return 1;
  if (D > 1024 || t0 < 0 || t1 > c->capacity[seq] || t0 > t1) return 2;
  b = X ? c->v_bits[layer * c->num_kv_heads + head] : c->k_bits[layer * c->num_kv_heads + head];
  if (X == 0 && c->k_per_channel && b < 16)
    return store_k_blocks(c, cache, vis, meta, txt, b, seq, t0, t1, src);
  for (t = t0; t < t1; t++) {
    const float *x = src + (size_t)(t - t0) * D;
    int plane;
    int64_t row;
    if (orc_row_of(c, seq, t, &plane, &row)) return 3;
    if (plane == 0 && b < 16) {
      uint64_t rb = (uint64_t)D * b / 8;
      uint8_t *r = cache + vis + (uint64_t)row * rb;
      uint8_t *m = cache + meta + (uint64_t)row * (uint64_t)(D / g) * 4u;
      if (X == 0 && c->rotate_k) {  /* coded K rows are rotated first */
        memcpy(rot, x, sizeof(float) * (size_t)D);
        orc_hadamard_rotate(rot, D);
        x = rot;
      }
      memset(r, 0, rb);
      for (j = 0; j < D / g; j++) {
        uint16_t s16, m16;
        orc_quantize_group(x + j * g, g, b, codes + j * g, &s16, &m16);
        put_u16(m + 4 * j, s16);
        put_u16(m + 4 * j + 2, m16);
      }
      for (d = 0; d < D; d++) {
        int bit = d * b;
        r[bit / 8] = (uint8_t)(r[bit / 8] | (codes[d] << (bit % 8)));
      }
    } else {
      uint8_t *r = cache + (plane == 0 ? vis : txt) + (uint64_t)row * 2u * D;
      for (d = 0; d < D; d++) put_u16(r + 2 * d, orc_bf16_round_nearest_even(x[d]));
    }
  }
  return 0;
}

/* Dequantise the row at (plane, row) of a (layer, head, X) whose planes start
 * at vis/meta/txt and whose visual rows use b bits. */
static void load_row_at(const orc_config *c, const uint8_t *cache, uint64_t vis,
                        uint64_t meta, uint64_t txt, int b, int plane, int64_t row,
                        int per_channel, double *out) {
  int D = c->head_dim, g = c->group_size, d;
  if (plane == 0 && b < 16) {
    uint64_t rb = (uint64_t)D * b / 8;
    const uint8_t *r = cache + vis + (uint64_t)row * rb;
    /* per token: D/g pairs in the row's META row; per channel: D pairs in
     * the META row of block row / g, pair d for channel d */
    const uint8_t *m = per_channel ? cache + meta + (uint64_t)(row / g) * (uint64_t)D * 4u
                                   : cache + meta + (uint64_t)row * (uint64_t)(D / g) * 4u;
    for (d = 0; d < D; d++) {
      int bit = d * b, j = per_channel ? d : d / g;
      int code = (r[bit / 8] >> (bit % 8)) & ((1 << b) - 1);
      double sc = orc_f16_value(get_u16(m + 4 * j));
      double mn = orc_f16_value(get_u16(m + 4 * j + 2));
      out[d] = (double)code * sc + mn; /* exact in binary64 */
    }
  } else {
    const uint8_t *r = cache + (plane == 0 ? vis : txt) + (uint64_t)row * 2u * D;
    for (d = 0; d < D; d++) out[d] = orc_bf16_value(get_u16(r + 2 * d));
  }
}

int orc_load_row_stored(const orc_config *c, const uint8_t *cache, int layer, int seq,
                        int head, int X, int t, double *out) {
  uint64_t vis, meta, txt;
  int b, plane;
  int64_t row;
  if (orc_plane_offsets(c, layer, head, X, &vis, &meta, &txt)) return 1;
  if (orc_row_of(c, seq, t, &plane, &row)) return 2;
  b = X ? c->v_bits[layer * c->num_kv_heads + head] : c->k_bits[layer * c->num_kv_heads + head];
  load_row_at(c, cache, vis, meta, txt, b, plane, row, X == 0 && c->k_per_channel, out);
  return 0;
}

int orc_load_row(const orc_config *c, const uint8_t *cache, int layer, int seq,
                 int head, int X, int t, double *out) {
  int plane, b, rc;
  int64_t row;
  rc = orc_load_row_stored(c, cache, layer, seq, head, X, t, out);
  if (rc) return rc;
  orc_row_of(c, seq, t, &plane, &row);
  b = X ? c->v_bits[layer * c->num_kv_heads + head] : c->k_bits[layer * c->num_kv_heads + head];
  if (X == 0 && c->rotate_k && plane == 0 && b < 16) orc_hadamard_unrotate(out, c->head_dim);
  return 0;
}

/* ------------------------------------------------------------------------ */
/* Attention (double): s_t = scale * <q, K_t>, p = softmax(s), out = sum p_t V_t */

void orc_attention(const double *q, const double *K, const double *V, int T,
                   int D, double scale, double *out, double *lse) {
  double *s = (double *)malloc(sizeof(double) * (size_t)(T > 0 ? T : 1));
  double M = -INFINITY, sum = 0.0;
  int t, d;
  for (t = 0; t < T; t++) {
    double dot = 0.0;
    for (d = 0; d < D; d++) dot += q[d] * K[(size_t)t * D + d];
    s[t] = scale * dot;
    if (s[t] > M) M = s[t];
  }
  for (d = 0; d < D; d++) out[d] = 0.0;
  for (t = 0; t < T; t++) {
    double p = exp(s[t] - M);
    sum += p;
    for (d = 0; d < D; d++) out[d] += p * V[(size_t)t * D + d];
  }
  for (d = 0; d < D; d++) out[d] /= sum;
  if (lse) *lse = M + log(sum);
  free(s);
}

int orc_decode_one(const orc_config *c, const uint8_t *cache, int layer,
                   int seq, int qhead, int len, const uint16_t *q_bf16,
                   float sm_scale, double *out, double *lse, double *scores) {
  int D = c->head_dim, t, d, kv, X, kb, vbits;
  uint64_t off[2][3];
  double *K, *V, *q;
  if (orc_validate(c) || seq < 0 || seq >= c->batch) return 1;
  if (len < 1 || len > c->capacity[seq]) return 1;
  kv = (int)((int64_t)qhead * c->num_kv_heads / c->num_q_heads);
  for (X = 0; X < 2; X++)
    if (orc_plane_offsets(c, layer, kv, X, &off[X][0], &off[X][1], &off[X][2])) return 2;
  kb = c->k_bits[layer * c->num_kv_heads + kv];
  vbits = c->v_bits[layer * c->num_kv_heads + kv];
  K = (double *)malloc(sizeof(double) * (size_t)len * D);
  V = (double *)malloc(sizeof(double) * (size_t)len * D);
  q = (double *)malloc(sizeof(double) * (size_t)D);
  for (d = 0; d < D; d++) q[d] = orc_bf16_value(q_bf16[d]);
  for (t = 0; t < len; t++) {
    int plane;
    int64_t row;
    orc_row_of(c, seq, t, &plane, &row); /* t < len <= capacity: in range */
    load_row_at(c, cache, off[0][0], off[0][1], off[0][2], kb, plane, row, c->k_per_channel,
                K + (size_t)t * D);
    if (c->rotate_k && plane == 0 && kb < 16) orc_hadamard_unrotate(K + (size_t)t * D, D);
    load_row_at(c, cache, off[1][0], off[1][1], off[1][2], vbits, plane, row, 0,
                V + (size_t)t * D);
  }
  orc_attention(q, K, V, len, D, (double)sm_scale, out, lse);
  if (scores) {
    for (t = 0; t < len; t++) {
      double dot = 0.0;
      for (d = 0; d < D; d++) dot += q[d] * K[(size_t)t * D + d];
      scores[t] = (double)sm_scale * dot;
    }
  }
  free(K); free(V); free(q);
  return 0;
}

int orc_decode_all(const orc_config *c, const uint8_t *cache, int l0, int nl,
                   const int32_t *lens, const uint16_t *q_bf16, float sm_scale,
                   double *out) {
  int l, s, h, D = c->head_dim, Hq = c->num_q_heads;
  for (l = 0; l < nl; l++)
    for (s = 0; s < c->batch; s++)
      for (h = 0; h < Hq; h++) {
        size_t o = (((size_t)l * c->batch + s) * Hq + h) * D;
        if (orc_decode_one(c, cache, l0 + l, s, h, lens[s], q_bf16 + o, sm_scale,
                           out + o, NULL, NULL))
          return 1;
      }
  return 0;
}

double orc_kl_logits(const double *s_p, const double *s_q, int T) {
  double mp = -INFINITY, mq = -INFINITY, zp = 0.0, zq = 0.0, kl = 0.0;
  int t;
  for (t = 0; t < T; t++) {
    if (s_p[t] > mp) mp = s_p[t];
    if (s_q[t] > mq) mq = s_q[t];
  }
  for (t = 0; t < T; t++) {
    zp += exp(s_p[t] - mp);
    zq += exp(s_q[t] - mq);
  }
  for (t = 0; t < T; t++) {
    double lp = s_p[t] - mp - log(zp);
    double lq = s_q[t] - mq - log(zq);
    kl += exp(lp) * (lp - lq);
  }
  return kl;
}
