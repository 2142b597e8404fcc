/*
 * kvq.h -- C ABI of libkvq: decode-step attention over a compressed VLM KV
 * cache on AMD Instinct MI355X (gfx950).
 *
 * What the library computes
 * -------------------------
 * A vision-language model's historical K/V cache, per layer [B, H_kv, T, D],
 * is stored compressed: inside each sequence's visual span the rows are
 * group-wise INT8/INT4/INT2 codes, everything else (system text, question
 * and generated tokens) stays at full precision, and K and V may use
 * different widths.  Sources: nuiw.github.io "VLM_KV_Quantization"
 * (section 1: the same historical cache at FP16/INT8/INT4/INT2 with the
 * Visual/Text and K/V axes separated; section 2: prompt = [system text]
 * [visual tokens] [question], cache [1, 4, T, 128] per layer with GQA 28:4;
 * section 4: K and V differ in sensitivity).  Selected physical KV heads can
 * keep their visual K, and optionally V, in bf16 on top of the low-bit
 * quantiser (jiinsi.com HeadGuard briefing, core bullets).  Decoding reads
 * the compressed rows and reconstructs them on chip inside a split-K
 * flash-decoding kernel, never writing reconstructed K/V back to memory
 * (gist.science 2604.02570, section 2-D: fused kernel, on-chip
 * reconstruction, no intermediate tensors in VRAM).
 *
 * Quantiser (one group of g values along D of one token, b bits, n = 2^b-1):
 *   mn16 = largest binary16 <= min(x)           (a zero is stored as +0)
 *   r    = fl32(max(x) - mn16)
 *   sc16 = 0 if r == 0, else smallest binary16 >= fl32(r / n)
 *   code = clamp(rint_half_even(fl32(fl32(x - mn16) / sc16)), 0, n)
 *          (0 when sc16 == 0); reconstruction x^ = code * sc16 + mn16.
 * Every fl32 is one IEEE binary32 operation, rounded to nearest even.
 * Rows stored at full precision are bf16 (round to nearest even).
 *
 * Cache layout (all integers little-endian)
 * -----------------------------------------
 * For every layer l, KV head h and X in (K, V), in that nesting order, three
 * planes, each starting on a 256-byte boundary of the cache buffer:
 *   VIS  rows for every visual position: D*b/8 bytes of codes, element d at
 *        bit d*b of the row (byte d*b/8, bit (d*b)%8); or 2*D bf16 bytes when
 *        b == 16.
 *   META rows for every visual position when b < 16: for group j = 0..D/g-1
 *        the fp16 scale then the fp16 min (4 bytes per group).
 *   TXT  one bf16 row (2*D bytes) per non-visual position.
 * Inside each plane the sequences follow each other in batch order; sequence
 * s owns vis_end[s]-vis_begin[s] VIS/META rows and capacity[s] minus that
 * many TXT rows.  Position t of sequence s is visual when
 * vis_begin[s] <= t < vis_end[s]; a text position t maps to TXT row t if
 * t < vis_begin[s], else t - (vis_end[s] - vis_begin[s]).  Padding bytes
 * between planes are unspecified.
 *
 * Ownership, streams, errors
 * --------------------------
 * Every device pointer is owned by the caller (typically torch tensors);
 * libkvq never allocates, frees or retains device memory.  Host-side global
 * state is limited to two memo tables that never change a result: the
 * compute-unit count of each device, read once, and the last four decode
 * split plans, keyed by everything a plan depends on (call shape, cache
 * configuration, device CU count) and guarded by a mutex, so a decode call
 * repeated step after step skips about 2 us of host planning.  Host arrays
 * are read only during the call.
 * kvq_quantize and kvq_decode_attention only enqueue work on `stream`
 * (a hipStream_t; NULL = the default stream) and never synchronise; faults
 * inside kernels surface at the caller's next synchronisation.  Every entry
 * point validates all arguments on the host before any HIP call: when it
 * returns an error nothing has been launched.  No C++ exception crosses the
 * ABI.  Calls are re-entrant for distinct buffers.
 *
 * Supported shapes: head_dim D in {64, 128}; group_size g in {32, 64, 128}
 * with g dividing D; bits in {2, 4, 8, 16}; num_q_heads a multiple of
 * num_kv_heads (KVQ_ERR_UNSUPPORTED otherwise); kvq_decode_attention also
 * needs num_q_heads / num_kv_heads <= 16 (KVQ_ERR_UNSUPPORTED otherwise).
 * Values whose stored fp16 scale/min would overflow binary16 (|x| > 65504)
 * are outside the supported range.
 */
#ifndef KVQ_H
#define KVQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define KVQ_ABI_VERSION 3

typedef enum {
  KVQ_OK = 0,
  KVQ_ERR_NULL = 1,        /* a required pointer is NULL                       */
  KVQ_ERR_SHAPE = 2,       /* inconsistent sizes or spans                      */
  KVQ_ERR_UNSUPPORTED = 3, /* well-formed but outside the supported shapes     */
  KVQ_ERR_RANGE = 4,       /* layer / sequence / position index out of range   */
  KVQ_ERR_WORKSPACE = 5,   /* workspace smaller than required                  */
  KVQ_ERR_ALIGN = 6,       /* device pointer misaligned                        */
  KVQ_ERR_HIP = 7,         /* a HIP runtime call or kernel launch failed       */
  KVQ_ERR_INTERNAL = 8     /* unexpected internal failure                      */
} kvq_status;

typedef enum { KVQ_SRC_F32 = 0, KVQ_SRC_BF16 = 1 } kvq_src_dtype;

/* Describes one cache.  All pointers are HOST arrays. */
typedef struct {
  int32_t num_layers;   /* L  >= 1                                             */
  int32_t batch;        /* B  >= 1 sequences                                   */
  int32_t num_q_heads;  /* Hq >= 1, multiple of num_kv_heads                   */
  int32_t num_kv_heads; /* Hkv >= 1                                            */
  int32_t head_dim;     /* D                                                   */
  int32_t group_size;   /* g, quantisation group along D                       */
  const int32_t *capacity;  /* [B] rows reserved per sequence (>= 1)          */
  const int32_t *vis_begin; /* [B] 0 <= vis_begin <= vis_end <= capacity      */
  const int32_t *vis_end;   /* [B]                                              */
  const uint8_t *k_bits;    /* [L*Hkv] K width per (layer, KV head), 16 = bf16 */
  const uint8_t *v_bits;    /* [L*Hkv] V width per (layer, KV head)            */
  int32_t rotate_k;         /* nonzero: K rows stored as codes are rotated     */
                            /* before quantisation (see below); 0: none        */
  int32_t k_per_channel;    /* nonzero: K codes grouped per channel over token */
                            /* blocks, with a bf16 residual window (below)     */
  /* Optional bf16 ranges inside the visual spans (NULL: none; see below). */
  const int32_t *bf16_range_offsets; /* [B + 1]                                */
  const int32_t *bf16_range_begin;   /* [bf16_range_offsets[B]]                */
  const int32_t *bf16_range_end;     /* [bf16_range_offsets[B]]                */
} kvq_config;

/* bf16 ranges (bf16_range_offsets != NULL).  nuiw.github.io
 * "VLM_KV_Quantization" section 1 names keeping important tokens at full
 * precision as a policy outside its study, and section 2 lays the prompt out
 * as text and visual blocks.  Sequence s may list ranges
 * [bf16_range_begin[k], bf16_range_end[k]) for k in [bf16_range_offsets[s],
 * bf16_range_offsets[s + 1]): non-empty, inside [vis_begin[s], vis_end[s]),
 * sorted and disjoint (bf16_range_offsets[0] == 0, non-decreasing).  Their
 * positions are stored bf16 exactly like text.  A one-token range protects
 * that token (a sink or a selected token); a range between two images makes
 * one sequence hold two visual spans.  The layout generalises by counting:
 * a position is coded when it lies in the visual span and in no range;
 * coded positions take VIS (and META) rows in order and every other
 * position takes TXT rows in order, sequence after sequence.  A sequence
 * may have at most 36 ranges.  Sequences with ranges are decoded with a
 * static split.  Malformed ranges return KVQ_ERR_SHAPE; ranges together
 * with k_per_channel, or more than 36 in one sequence, KVQ_ERR_UNSUPPORTED. */

/* Per-channel K groups (k_per_channel != 0).  nuiw.github.io
 * "VLM_KV_Quantization" section 4: K is stored after RoPE, its error reaches
 * every query head of the group, and it is the more sensitive side; its
 * structure runs along channels.  With this flag each channel's K values
 * over a block of group_size consecutive visual tokens form one quantisation
 * group (the same quantiser as above); V stays grouped per token along D.
 * Sequence s's visual span is coded in whole blocks from vis_begin[s]: the
 * coded span is [vis_begin, vis_begin + floor((vis_end - vis_begin) / g) g).
 * The tail that does not fill a block (the newest visual tokens, fewer than
 * g) is a residual window stored bf16 as text, for K and V alike: every rule
 * of the layout that names vis_end uses the end of the coded span instead.
 * A K META row then belongs to a block, not a token: VIS row r's (scale,
 * min) pairs are META row r / g, which holds D pairs, pair d for channel d.
 * The plane sizes are the same as with per-token groups.  kvq_quantize must
 * store whole blocks: a call whose positions cut a block of the coded span
 * apart returns KVQ_ERR_SHAPE.  Not combinable with rotate_k; the decode
 * takes fixed chunks only in multiples of 256 tokens and no (layer, head)
 * with coded K but bf16 V (KVQ_ERR_UNSUPPORTED otherwise). */

/* K rotation (rotate_k != 0).  gist.science 2604.02570 (WSVD, section 2-C)
 * rotates vectors ahead of quantisation to remove per-channel outliers; the
 * library uses the weight-free normalised Walsh-Hadamard matrix (Sylvester
 * order, H[i][j] = (-1)^popcount(i & j)).  Every K row that is stored as
 * codes (visual position, k_bits < 16) is transformed before its groups are
 * quantised, in binary32: for s = 1, 2, 4, ..., D/2 every pair (i, i + s)
 * with bit s of i clear becomes (x_i + x_(i+s), x_i - x_(i+s)), then every
 * value is multiplied by 2^-ceil(log2(D)/2).  Text rows, V rows and bf16
 * rows are never rotated.  kvq_decode_attention applies the matching
 * transform, scaled by 2^-floor(log2(D)/2), to the query for those rows, so
 * scores are q.k in exact arithmetic.  The stored bytes of a rotated cache
 * differ from an unrotated one only in those K code and meta rows; the
 * cache's size does not change.  A cache must be decoded with the rotate_k
 * it was stored with. */

typedef struct {
  uint64_t total_bytes;       /* bytes to allocate: payload + plane padding    */
  uint64_t payload_bytes;     /* exact stored bytes, no padding                */
  uint64_t code_bytes;        /* packed codes of visual rows                   */
  uint64_t meta_bytes;        /* fp16 (scale, min) pairs                       */
  uint64_t bf16_visual_bytes; /* visual rows of 16-bit (protected) heads       */
  uint64_t bf16_text_bytes;   /* text rows (every head, K and V)               */
  uint64_t quantized_values;  /* K/V scalars stored as codes                   */
  uint64_t stored_values;     /* all K/V scalars: 2*L*Hkv*D*sum(capacity)      */
} kvq_cache_info;

/* Storage size of the cache `cfg` describes, split so that the true cost of
 * a width can be read off: code and meta bytes against the values stored as
 * codes give bits per value including the fp16 (scale, min) overhead (the
 * opening checklist of nuiw.github.io "VLM_KV_Quantization" asks whether a
 * nominal INT2 cache really costs 2 bits per value, and whether the count
 * of quantised tokens is non-zero: quantized_values answers that).
 *   cfg    HOST, validated as described above
 *   info   HOST, written on success
 * Host only, pure, synchronous, touches no device.
 * Errors: KVQ_ERR_NULL (cfg/info/arrays), KVQ_ERR_SHAPE, KVQ_ERR_UNSUPPORTED. */
kvq_status kvq_cache_bytes(const kvq_config *cfg, kvq_cache_info *info);

/* Store positions [tok_begin, tok_end) of the sequences seq_ids[0..num_seqs)
 * for layers [layer_begin, layer_begin + num_layers) into `cache`.
 * Passages: nuiw.github.io "VLM_KV_Quantization" section 1 (only the
 * historical cache is compressed, with the Visual/Text and K/V axes handled
 * separately) and section 2 (K is stored after RoPE; the visual block sits
 * between the system text and the question); the HeadGuard briefing (a few
 * physical KV heads keep visual K, optionally V, at high precision).
 *
 * Each row's format follows from its position and head: a visual position in
 * a head whose width is < 16 is quantised (codes + meta); every other row
 * (text, question, generated tokens; protected heads) is stored as bf16.
 * Prefill of a whole sequence is one call over [0, capacity); appending a
 * decoded token is a call over [T, T+1).
 *
 *   cache   device, kvq_cache_info.total_bytes, 256-byte aligned, written
 *   seq_ids HOST [num_seqs], distinct, each in [0, batch)
 *   k_src,
 *   v_src   device, 16-byte aligned, contiguous
 *           [num_layers, num_seqs, num_kv_heads, tok_end - tok_begin, D]
 *           of float32 (KVQ_SRC_F32) or bf16 (KVQ_SRC_BF16)
 * Errors: KVQ_ERR_NULL, KVQ_ERR_SHAPE, KVQ_ERR_UNSUPPORTED, KVQ_ERR_ALIGN,
 * KVQ_ERR_RANGE (layer range, seq id, or a position outside [0, capacity)),
 * KVQ_ERR_HIP.  An empty token range is a no-op returning KVQ_OK. */
kvq_status kvq_quantize(const kvq_config *cfg, void *cache, int32_t layer_begin,
                        int32_t num_layers, int32_t num_seqs, const int32_t *seq_ids,
                        int32_t tok_begin, int32_t tok_end, const void *k_src,
                        const void *v_src, kvq_src_dtype src_dtype, void *stream);

/* kvq_quantize with a start position per sequence: sequence seq_ids[i]
 * stores positions [tok_begin[i], tok_begin[i] + num_tokens), one launch for
 * the whole batch.  It is the decode-time append of a ragged batch, where each
 * sequence's next token sits at its own length (nuiw.github.io
 * "VLM_KV_Quantization" section 1: generated tokens join the cache in full
 * precision; they are text positions, so they are stored bf16).  Rows are
 * stored exactly as kvq_quantize stores them.
 *
 *   tok_begin  HOST int32 [num_seqs], each >= 0 and tok_begin[i] + num_tokens
 *              <= capacity[seq_ids[i]]
 *   k_src,
 *   v_src      device, 16-byte aligned, contiguous
 *              [num_layers, num_seqs, num_kv_heads, num_tokens, D]
 * Other arguments and errors as kvq_quantize; num_tokens == 0 is a no-op. */
kvq_status kvq_quantize_ragged(const kvq_config *cfg, void *cache, int32_t layer_begin,
                               int32_t num_layers, int32_t num_seqs, const int32_t *seq_ids,
                               const int32_t *tok_begin, int32_t num_tokens,
                               const void *k_src, const void *v_src, kvq_src_dtype src_dtype,
                               void *stream);

/* One decode step of attention for layers [layer_begin, layer_begin +
 * num_layers).  Passages: gist.science 2604.02570 section 2-D (rows are
 * rebuilt on chip inside a fused flash-decoding kernel and never written back
 * to memory); nuiw.github.io "VLM_KV_Quantization" section 2 (GQA: the
 * stored KV heads serve several query heads each).  For every layer l,
 * sequence s and query head i,
 *   out[l,s,i,:] = softmax(sm_scale * K^ q) V^   over positions [0, seq_lens[s])
 * of KV head floor(i * Hkv / Hq), with K^, V^ the stored rows reconstructed
 * on chip (codes * scale + min, or bf16).  Split-K over token chunks with a
 * log-sum-exp merge; fp32 accumulation; out rounded to bf16 (nearest even).
 * A KV head whose Hq / Hkv query heads times D / g groups exceed 16 columns
 * is decoded in ceil(Hq / Hkv * (D / g) / 16) launches, one per subgroup of
 * its query heads, each reading the head's rows again.
 *
 *   cache      device, as written by kvq_quantize (read only)
 *   seq_lens   DEVICE int32 [batch], 1 <= seq_lens[s] <= capacity[s]
 *              (values outside that range are clamped into it)
 *   q          device bf16 [num_layers, batch, Hq, D], 16-byte aligned
 *   out        device bf16 [num_layers, batch, Hq, D], 16-byte aligned; must
 *              not alias q, cache or workspace
 *   sm_scale   softmax scale applied to q.k (e.g. 1/sqrt(D)), fp32
 *   chunk_tokens  0 = library choice.  A call with at least one 32-token step
 *              per wave slot of the device splits each (layer, seq, KV head)
 *              into workgroups in proportion to its capacity and per-token
 *              cost, so that all waves of the call fit the device at once, and
 *              hands its steps to those waves as they finish (the summation
 *              order, hence the output's last bits, can differ between
 *              calls); a smaller call (latency-bound) takes fixed 512-token
 *              chunks.  Otherwise a positive multiple of 32 = tokens per
 *              split-K workgroup.  Fixed chunks are assigned statically:
 *              repeated calls give identical bytes.
 *   workspace  device scratch for split partials and the merge's arrival
 *              counters, 256-byte aligned.  If workspace == NULL the call only
 *              writes the required size to *workspace_bytes and launches
 *              nothing.  Otherwise *workspace_bytes is the size provided.  The
 *              required size depends on cfg, the layer range and chunk_tokens
 *              (and, for chunk_tokens == 0, on the current device's
 *              compute-unit count).  The workspace must be zero-filled before
 *              its first use; every call leaves it ready for the next one, so a
 *              workspace can be reused across calls of any shape that fits it
 *              on caches of the same kvq_config shape (layers, batch, KV
 *              heads); zero-fill it again before using it with another.
 *              Calls that may overlap in time must use distinct workspaces.
 * Errors: KVQ_ERR_NULL, KVQ_ERR_SHAPE, KVQ_ERR_UNSUPPORTED, KVQ_ERR_ALIGN,
 * KVQ_ERR_RANGE (layer range), KVQ_ERR_WORKSPACE, KVQ_ERR_HIP. */
kvq_status kvq_decode_attention(const kvq_config *cfg, const void *cache,
                                int32_t layer_begin, int32_t num_layers,
                                const int32_t *seq_lens, const void *q, void *out,
                                float sm_scale, int32_t chunk_tokens, void *workspace,
                                size_t *workspace_bytes, void *stream);

/* The decode-time append and kvq_decode_attention in one launch: for every
 * layer l of the call, sequence s and KV head h, the token at position
 * seq_lens[s] - 1 (after clamping) is stored from k_new / v_new exactly as
 * kvq_quantize_ragged stores it, and then attended like every other
 * position.  nuiw.github.io "VLM_KV_Quantization" section 1: each generated
 * token joins the cache in full precision and is attended at the step that
 * produced it; section 2: it is a text position, so its rows are bf16.
 * The workgroup that attends the position writes its rows first (write-
 * through stores, completed before its own loads), so nothing else orders
 * the store and the read, and the append costs no launch of its own.
 *
 *   cache      device, as for kvq_decode_attention; written at the appended
 *              rows only
 *   k_new,
 *   v_new      device, 16-byte aligned, contiguous [num_layers, batch,
 *              num_kv_heads, D] of float32 (KVQ_SRC_F32) or bf16
 *              (KVQ_SRC_BF16): the rows of position seq_lens[s] - 1
 * The appended position must be a text position of its sequence: before
 * vis_begin, at or after the coded span's end, or inside a bf16 range.  A
 * position the cache stores coded (or bf16 in a protected head's visual rows)
 * is not written, and the call then attends whatever the cache held there.
 * Other arguments, the workspace contract and errors as kvq_decode_attention
 * (KVQ_ERR_NULL also for k_new / v_new, KVQ_ERR_ALIGN for their alignment,
 * KVQ_ERR_UNSUPPORTED for another src_dtype). */
kvq_status kvq_decode_attention_append(const kvq_config *cfg, void *cache, int32_t layer_begin,
                                       int32_t num_layers, const int32_t *seq_lens,
                                       const void *k_new, const void *v_new,
                                       kvq_src_dtype src_dtype, const void *q, void *out,
                                       float sm_scale, int32_t chunk_tokens, void *workspace,
                                       size_t *workspace_bytes, void *stream);

/* kvq_decode_attention without a caller workspace, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  Same arguments, semantics and kernels as
 * kvq_decode_attention minus workspace/workspace_bytes: the split partials
 * and the merge's arrival counters live in a fixed 16 MiB device array inside
 * the library, one per device, held until the process ends.  The call itself
 * allocates nothing.  The first call on a device looks the array up and
 * clears its counter area with a kernel on `stream`.
 *
 * Limits: the cache's num_layers * batch * num_kv_heads must be <= 16384, and
 * the call's partials must fit the remaining 16 MiB - 64 KiB (the default
 * split of every shape this header supports at up to 64 sequences of 16K
 * tokens fits; kvq_decode_attention's size query on the same call reports
 * what it needs, minus the counter area).  A call beyond either limit returns
 * KVQ_ERR_WORKSPACE and launches nothing.
 *
 * All calls on one device share the array: calls that may overlap in time on
 * one device (different streams without ordering between them) race and
 * give wrong results.  Calls ordered on one stream, or otherwise serialised,
 * are safe, whatever their shapes.
 * Errors: as kvq_decode_attention, with KVQ_ERR_WORKSPACE for the limits
 * above and KVQ_ERR_HIP if the array cannot be found on the current device. */
kvq_status kvq_decode_attention_noalloc(const kvq_config *cfg, const void *cache,
                                        int32_t layer_begin, int32_t num_layers,
                                        const int32_t *seq_lens, const void *q, void *out,
                                        float sm_scale, int32_t chunk_tokens, void *stream);

/* ---- Low-rank latent cache --------------------------------------------
 * gist.science 2604.02570 (WSVD), section 2-A: every attention head has its
 * own low-rank factorisation, so the cache of one (layer, KV head) holds
 * latent rows c_t of width r (the rank) instead of K/V rows of width D, and
 * K_t = c^K_t B_K, V_t = c^V_t B_V with per-head r x D up-projections;
 * section 2-D: K and V are reconstructed on chip inside flash decoding and
 * never written to memory.  The latents come from the model (the down
 * projection of the hidden state); this library stores and attends over
 * them.
 *
 * Layout (bf16, little-endian): sequence s owns rows [row0_s, row0_s +
 * capacity[s]) of every plane, row0_s = the sum of the earlier capacities
 * each rounded up to 32.  For every layer l and KV head h, in that nesting
 * order, a K plane then a V plane, each align256(R * rank * 2) bytes with R
 * = row0 of a sequence past the last; element j of row t of a plane at
 * byte (t * rank + j) * 2.  Padding rows and bytes are never read as data.
 *
 * Supported: head_dim in {64, 128}; rank in {32, 64, 96, 128} and <= head_dim;
 * num_q_heads a multiple of num_kv_heads with a ratio <= 16; a plane below
 * 2 GiB (KVQ_ERR_UNSUPPORTED otherwise). */
typedef struct {
  int32_t num_layers;       /* L                                                */
  int32_t batch;            /* B                                                */
  int32_t num_q_heads;      /* Hq                                               */
  int32_t num_kv_heads;     /* Hkv                                              */
  int32_t head_dim;         /* D                                                */
  int32_t rank;             /* r                                                */
  const int32_t *capacity;  /* HOST [B] rows reserved per sequence (>= 1)      */
} kvq_latent_config;

/* Bytes of the latent cache `cfg` describes (the layout above).
 *   cfg    HOST; bytes HOST, written on success.
 * Host only, pure, synchronous.  Errors: KVQ_ERR_NULL, KVQ_ERR_SHAPE,
 * KVQ_ERR_UNSUPPORTED. */
kvq_status kvq_latent_cache_bytes(const kvq_latent_config *cfg, uint64_t *bytes);

/* Store latent rows of positions [tok_begin, tok_end) of the sequences
 * seq_ids[0..num_seqs) for layers [layer_begin, layer_begin + num_layers)
 * (the cached per-head latents of WSVD section 2-A), bit for bit.
 *   cache      device, kvq_latent_cache_bytes bytes, 256-byte aligned
 *   seq_ids    HOST [num_seqs], distinct, each in [0, batch)
 *   k_latent,
 *   v_latent   device bf16, 16-byte aligned, contiguous
 *              [num_layers, num_seqs, Hkv, tok_end - tok_begin, rank]
 * Enqueues on `stream` only.  Errors: KVQ_ERR_NULL, KVQ_ERR_SHAPE (seq ids
 * repeated, tok_end < tok_begin), KVQ_ERR_UNSUPPORTED, KVQ_ERR_ALIGN,
 * KVQ_ERR_RANGE (layers, seq ids, positions outside [0, capacity)),
 * KVQ_ERR_HIP.  An empty range is a no-op. */
kvq_status kvq_latent_store(const kvq_latent_config *cfg, void *cache, int32_t layer_begin,
                            int32_t num_layers, int32_t num_seqs, const int32_t *seq_ids,
                            int32_t tok_begin, int32_t tok_end, const void *k_latent,
                            const void *v_latent, void *stream);

/* One decode step over the latent cache (WSVD section 2-D): for every layer
 * l, sequence s and query head i, with h = floor(i * Hkv / Hq),
 *   out[l,s,i,:] = softmax(sm_scale * K q) V   over positions [0, seq_lens[s])
 * where K = C_K B_K and V = C_V B_V are the latents of (l, h) times its
 * up-projections.  K and V are never formed: the query is projected once
 * (q' = B_K q) and attends over the latents, and B_V is applied to the
 * merged latent output (the same result up to rounding order).  Split-K over
 * token chunks with a log-sum-exp merge, done by the last workgroup of a
 * (layer, sequence, KV head) to finish; fp32 accumulation, bf16 output
 * (nearest even).
 *   cache      device, as written by kvq_latent_store (read only)
 *   seq_lens   DEVICE int32 [batch], clamped into [1, capacity[s]]
 *   up_k,
 *   up_v       device bf16 [L, Hkv, rank, D] (all layers of the cache),
 *              16-byte aligned: B_K and B_V of every (layer, KV head)
 *   q, out     device bf16 [num_layers, batch, Hq, D], 16-byte aligned; out
 *              must not alias any input or the workspace
 *   chunk_tokens  0 = library choice (about one workgroup per compute unit
 *              over the call; its waves take the chunk's steps as they
 *              finish, so the summation order, hence the output's last bits,
 *              can differ between calls), else a positive multiple of 32 =
 *              tokens per workgroup, steps assigned statically: repeated
 *              calls give identical bytes.
 *   workspace  device, 256-byte aligned: arrival counters for every (layer,
 *              sequence, KV head) of the cache, then the split partials;
 *              NULL = only write the required size to *workspace_bytes.
 *              Must be zero-filled before its first use; every call leaves
 *              the counters at zero again.  Calls that may overlap in time
 *              must use distinct workspaces.
 * One kernel launch per 64 sequences, enqueued on `stream`.
 * Errors: KVQ_ERR_NULL, KVQ_ERR_SHAPE, KVQ_ERR_UNSUPPORTED (also more than
 * 4096 chunks per sequence), KVQ_ERR_ALIGN, KVQ_ERR_RANGE, KVQ_ERR_WORKSPACE,
 * KVQ_ERR_HIP. */
kvq_status kvq_latent_decode(const kvq_latent_config *cfg, const void *cache,
                             int32_t layer_begin, int32_t num_layers, const int32_t *seq_lens,
                             const void *up_k, const void *up_v, const void *q, void *out,
                             float sm_scale, int32_t chunk_tokens, void *workspace,
                             size_t *workspace_bytes, void *stream);

/* Static description of a status code (never NULL; unknown codes get a
 * generic string).  A utility of the ABI, not a step of the method. */
const char *kvq_status_string(kvq_status s);

#ifdef __cplusplus
}
#endif
#endif /* KVQ_H */
