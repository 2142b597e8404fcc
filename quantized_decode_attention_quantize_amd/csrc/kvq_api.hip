// kvq_api.hip -- host side of libkvq: argument validation, cache layout,
// split planning and the extern "C" entry points declared in include/kvq.h.
//
// Every entry point validates all of its arguments before the first HIP
// call, so an error return means nothing was launched.  No exception leaves
// this file.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <new>
#include <vector>

#include "../../include/kvq.h"
#include "kvq_internal.h"

namespace kvq {
namespace {

bool bits_ok(int b) { return b == 2 || b == 4 || b == 8 || b == 16; }

// Validates everything kvq_config carries.
kvq_status check_config(const kvq_config* c) {
  if (!c || !c->capacity || !c->vis_begin || !c->vis_end || !c->k_bits || !c->v_bits)
    return KVQ_ERR_NULL;
  if (c->num_layers < 1 || c->batch < 1 || c->num_q_heads < 1 || c->num_kv_heads < 1 ||
      c->head_dim < 1 || c->group_size < 1)
    return KVQ_ERR_SHAPE;
  if (c->num_q_heads % c->num_kv_heads) return KVQ_ERR_SHAPE;
  if (c->head_dim != 64 && c->head_dim != 128) return KVQ_ERR_UNSUPPORTED;
  if (c->group_size != 32 && c->group_size != 64 && c->group_size != 128)
    return KVQ_ERR_UNSUPPORTED;
  if (c->group_size > c->head_dim || c->head_dim % c->group_size) return KVQ_ERR_UNSUPPORTED;
  const int64_t nlh = int64_t(c->num_layers) * c->num_kv_heads;
  for (int64_t i = 0; i < nlh; ++i)
    if (!bits_ok(c->k_bits[i]) || !bits_ok(c->v_bits[i])) return KVQ_ERR_UNSUPPORTED;
  int64_t total = 0;
  for (int s = 0; s < c->batch; ++s) {
    if (c->capacity[s] < 1 || c->vis_begin[s] < 0 || c->vis_begin[s] > c->vis_end[s] ||
        c->vis_end[s] > c->capacity[s])
      return KVQ_ERR_SHAPE;
    total += c->capacity[s];
  }
  if (total >= (int64_t(1) << 31)) return KVQ_ERR_UNSUPPORTED;  // row indices are 32-bit
  return KVQ_OK;
}

// Plane geometry of a validated config.
struct Layout {
  int L, B, Hq, Hkv, D, g, G;
  int64_t Rvis = 0, Rtxt = 0;
  std::vector<int64_t> vrow0, trow0;  // first VIS / TXT row of each sequence
  std::vector<uint64_t> vis_off;      // [L*Hkv*2] VIS plane byte offset
  kvq_cache_info info{};

  explicit Layout(const kvq_config* c)
      : L(c->num_layers), B(c->batch), Hq(c->num_q_heads), Hkv(c->num_kv_heads),
        D(c->head_dim), g(c->group_size), G(c->num_q_heads / c->num_kv_heads),
        vrow0(c->batch), trow0(c->batch), vis_off(size_t(c->num_layers) * c->num_kv_heads * 2) {
    for (int s = 0; s < B; ++s) {
      const int64_t nv = c->vis_end[s] - c->vis_begin[s];
      vrow0[s] = Rvis;
      trow0[s] = Rtxt;
      Rvis += nv;
      Rtxt += c->capacity[s] - nv;
    }
    uint64_t off = 0;
    for (int l = 0; l < L; ++l)
      for (int h = 0; h < Hkv; ++h)
        for (int X = 0; X < 2; ++X) {
          const int b = X ? c->v_bits[l * Hkv + h] : c->k_bits[l * Hkv + h];
          const uint64_t vis = uint64_t(Rvis) * vis_row_bytes(D, b);
          const uint64_t meta = b < 16 ? uint64_t(Rvis) * (D / g) * 4 : 0;
          const uint64_t txt = uint64_t(Rtxt) * 2 * D;
          vis_off[(size_t(l) * Hkv + h) * 2 + X] = off;
          off += align256(vis) + align256(meta) + align256(txt);
          info.payload_bytes += vis + meta + txt;
          if (b < 16) {
            info.code_bytes += vis;
            info.meta_bytes += meta;
            info.quantized_values += uint64_t(Rvis) * D;
          } else {
            info.bf16_visual_bytes += vis;
          }
          info.bf16_text_bytes += txt;
          info.stored_values += uint64_t(Rvis + Rtxt) * D;
        }
    info.total_bytes = off;
  }
};

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

int bits_of(const kvq_config* c, int l, int h, int X) {
  return X ? c->v_bits[l * c->num_kv_heads + h] : c->k_bits[l * c->num_kv_heads + h];
}

// Library choice of the split chunk: aim for about `target` workgroups over
// the whole call, in multiples of `quantum` tokens.
int default_chunk(const kvq_config* c, int nl, int quantum, int64_t target) {
  int64_t rows = 0;
  for (int s = 0; s < c->batch; ++s) rows += c->capacity[s];
  const int64_t work = rows * nl * c->num_kv_heads;
  int64_t ch = (work + target - 1) / target;
  ch = ((ch + quantum - 1) / quantum) * quantum;
  return int(std::max<int64_t>(ch, quantum));
}

// Compute units of the current device (256 on MI355X); 256 when no device
// can be queried (host-only use such as workspace size queries in tests).
// The count is read once per device and cached.
int device_cus() {
  constexpr int kMaxDevices = 64;
  static std::atomic<int> cached[kMaxDevices];
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  if (dev >= 0 && dev < kMaxDevices && (n = cached[dev].load(std::memory_order_relaxed)) > 0)
    return n;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      n < 1)
    return 256;
  if (dev >= 0 && dev < kMaxDevices) cached[dev].store(n, std::memory_order_relaxed);
  return n;
}

static_assert(sizeof(DecodeArgs) <= 4096, "decode kernel arguments exceed 4 KB");
static_assert(sizeof(QuantizeArgs) <= 4096, "quantize kernel arguments exceed 4 KB");

struct DecodePlan {
  int chunk;                  // tokens per workgroup; 0 = balanced split
  std::vector<int> nx;        // [batch] workgroups per (layer, head) before mult
  std::vector<uint8_t> mult;  // [num_layers * Hkv] of the call: heavy-head multiplier
  int max_chunks;
  int64_t entries;
  size_t o_bytes, ml_bytes, cnt_bytes, arrive_bytes, total;
};

// Split planning.  With chunk_tokens > 0 (or on the general kernel) every
// workgroup takes a fixed token chunk.  Otherwise (matrix-core kernel) the
// split is balanced: each (layer, seq, head) gets workgroups in proportion to
// its capacity and cost so that all waves fit the device in one round
// (8 waves per CU: the kernel runs at two waves per SIMD); all-bf16 heads move
// ~4.6x the bytes per token of INT4/INT2 heads and take about twice as long
// per step, so they get twice the workgroups.
DecodePlan plan_decode(const kvq_config* c, int layer_begin, int nl, int chunk_tokens,
                       bool use_mfma) {
  DecodePlan p;
  const int B = c->batch, Hkv = c->num_kv_heads;
  p.nx.assign(B, 1);
  p.mult.assign(size_t(nl) * Hkv, 1);
  if (chunk_tokens > 0 || !use_mfma) {
    p.chunk = chunk_tokens > 0 ? chunk_tokens : default_chunk(c, nl, 256, 1024);
    for (int s = 0; s < B; ++s) p.nx[s] = (c->capacity[s] + p.chunk - 1) / p.chunk;
  } else {
    p.chunk = 0;
    int64_t msum = 0;
    for (int i = 0; i < nl * Hkv; ++i) {
      const int l = layer_begin + i / Hkv, h = i % Hkv;
      p.mult[i] = (bits_of(c, l, h, 0) == 16 && bits_of(c, l, h, 1) == 16) ? 2 : 1;
      msum += p.mult[i];
    }
    int64_t caps = 0;
    for (int s = 0; s < B; ++s) caps += c->capacity[s];
    // Budget: one 8-wave workgroup per CU (the kernel runs two waves per
    // SIMD), so every CU carries the same load and all waves run in one round.
    const int64_t budget = int64_t(device_cus());
    constexpr int kMinWaveTokens = 128;  // keep >= 4 steps per wave
    std::vector<double> frac(B);
    int64_t used = 0;
    for (int s = 0; s < B; ++s) {
      const double want = double(budget) * double(c->capacity[s]) / double(caps * msum);
      const int nmax = (c->capacity[s] + kMfmaWaves * kMinWaveTokens - 1) /
                       (kMfmaWaves * kMinWaveTokens);
      p.nx[s] = std::max(1, std::min(int(want), nmax));
      frac[s] = p.nx[s] < nmax ? want - std::floor(want) : -1.0;
      used += int64_t(p.nx[s]) * msum;
    }
    // largest remainders take what is left of the budget
    while (used + msum <= budget) {
      int best = -1;
      for (int s = 0; s < B; ++s)
        if (frac[s] > 0.0 && (best < 0 || frac[s] > frac[best])) best = s;
      if (best < 0) break;
      ++p.nx[best];
      frac[best] = -1.0;
      used += msum;
    }
  }
  int mx = 1;
  for (int s = 0; s < B; ++s) mx = std::max(mx, p.nx[s]);
  int mm = 1;
  for (uint8_t m : p.mult) mm = std::max<int>(mm, m);
  p.max_chunks = mx * mm;
  const int G = c->num_q_heads / c->num_kv_heads;
  p.entries = int64_t(nl) * B * Hkv * p.max_chunks;
  p.o_bytes = size_t(align256(p.entries * G * c->head_dim * 4));
  p.ml_bytes = size_t(align256(p.entries * G * 2 * 4));
  p.cnt_bytes = size_t(align256(int64_t(nl) * B * Hkv * 4));
  p.arrive_bytes = size_t(align256(int64_t(nl) * B * Hkv * 4));
  p.total = p.o_bytes + p.ml_bytes + p.cnt_bytes + p.arrive_bytes;
  return p;
}

}  // namespace
}  // namespace kvq

using namespace kvq;

extern "C" const char* kvq_status_string(kvq_status s) {
  switch (s) {
    case KVQ_OK: return "ok";
    case KVQ_ERR_NULL: return "required pointer is NULL";
    case KVQ_ERR_SHAPE: return "inconsistent sizes or spans";
    case KVQ_ERR_UNSUPPORTED: return "unsupported shape, width or dtype";
    case KVQ_ERR_RANGE: return "index out of range";
    case KVQ_ERR_WORKSPACE: return "workspace too small";
    case KVQ_ERR_ALIGN: return "device pointer misaligned";
    case KVQ_ERR_HIP: return "HIP runtime error";
    case KVQ_ERR_INTERNAL: return "internal error";
  }
  return "unknown status";
}

extern "C" kvq_status kvq_cache_bytes(const kvq_config* cfg, kvq_cache_info* info) {
  try {
    if (!info) return KVQ_ERR_NULL;
    const kvq_status st = check_config(cfg);
    if (st != KVQ_OK) return st;
    Layout lay(cfg);
    *info = lay.info;
    return KVQ_OK;
  } catch (...) {
    return KVQ_ERR_INTERNAL;
  }
}

extern "C" kvq_status kvq_quantize(const kvq_config* cfg, void* cache, int32_t layer_begin,
                                   int32_t num_layers, int32_t num_seqs, const int32_t* seq_ids,
                                   int32_t tok_begin, int32_t tok_end, const void* k_src,
                                   const void* v_src, kvq_src_dtype src_dtype, void* stream) {
  try {
    kvq_status st = check_config(cfg);
    if (st != KVQ_OK) return st;
    if (src_dtype != KVQ_SRC_F32 && src_dtype != KVQ_SRC_BF16) return KVQ_ERR_UNSUPPORTED;
    if (num_layers < 1 || num_seqs < 0 || tok_begin < 0 || tok_end < tok_begin)
      return KVQ_ERR_SHAPE;
    if (layer_begin < 0 || layer_begin > cfg->num_layers - num_layers) return KVQ_ERR_RANGE;
    if (num_seqs == 0 || tok_end == tok_begin) return KVQ_OK;
    if (!cache || !k_src || !v_src || !seq_ids) return KVQ_ERR_NULL;
    if (!aligned(cache, 256) || !aligned(k_src, 16) || !aligned(v_src, 16)) return KVQ_ERR_ALIGN;
    std::vector<char> seen(cfg->batch, 0);
    for (int i = 0; i < num_seqs; ++i) {
      const int s = seq_ids[i];
      if (s < 0 || s >= cfg->batch) return KVQ_ERR_RANGE;
      if (seen[s]) return KVQ_ERR_SHAPE;
      seen[s] = 1;
      if (tok_end > cfg->capacity[s]) return KVQ_ERR_RANGE;
    }
    Layout lay(cfg);
    if (lay.info.total_bytes / 256 >= (uint64_t(1) << 32)) return KVQ_ERR_UNSUPPORTED;

    const int nlh = num_layers * cfg->num_kv_heads;
    for (int lh0 = 0; lh0 < nlh; lh0 += kMaxLH) {
      const int nlh_l = std::min(kMaxLH, nlh - lh0);
      for (int s0 = 0; s0 < num_seqs; s0 += kMaxSeq) {
        const int ns_l = std::min(kMaxSeq, num_seqs - s0);
        QuantizeArgs a;
        std::memset(&a, 0, sizeof(a));
        a.cache = static_cast<uint8_t*>(cache);
        a.k_src = k_src;
        a.v_src = v_src;
        a.Rvis = lay.Rvis;
        a.D = lay.D;
        a.g = lay.g;
        a.src_bf16 = src_dtype == KVQ_SRC_BF16;
        a.tok_begin = tok_begin;
        a.n_tok = tok_end - tok_begin;
        a.num_seqs_total = num_seqs;
        a.seq_off = s0;
        a.Hkv = cfg->num_kv_heads;
        a.lh_off = lh0;
        for (int i = 0; i < nlh_l; ++i) {
          const int glh = lh0 + i;
          const int l = layer_begin + glh / cfg->num_kv_heads, h = glh % cfg->num_kv_heads;
          for (int X = 0; X < 2; ++X) {
            a.base256[i][X] = uint32_t(lay.vis_off[(size_t(l) * cfg->num_kv_heads + h) * 2 + X] / 256);
            a.bits[i][X] = uint8_t(bits_of(cfg, l, h, X));
          }
        }
        for (int i = 0; i < ns_l; ++i) {
          const int s = seq_ids[s0 + i];
          a.vb[i] = cfg->vis_begin[s];
          a.ve[i] = cfg->vis_end[s];
          a.vrow0[i] = int32_t(lay.vrow0[s]);
          a.trow0[i] = int32_t(lay.trow0[s]);
        }
        if (launch_quantize(a, nlh_l, ns_l, static_cast<hipStream_t>(stream)) != hipSuccess)
          return KVQ_ERR_HIP;
      }
    }
    return KVQ_OK;
  } catch (const std::bad_alloc&) {
    return KVQ_ERR_INTERNAL;
  } catch (...) {
    return KVQ_ERR_INTERNAL;
  }
}

extern "C" kvq_status kvq_decode_attention(const kvq_config* cfg, const void* cache,
                                           int32_t layer_begin, int32_t num_layers,
                                           const int32_t* seq_lens, const void* q, void* out,
                                           float sm_scale, int32_t chunk_tokens,
                                           void* workspace, size_t* workspace_bytes,
                                           void* stream) {
  try {
    kvq_status st = check_config(cfg);
    if (st != KVQ_OK) return st;
    if (!workspace_bytes) return KVQ_ERR_NULL;
    if (num_layers < 1) return KVQ_ERR_SHAPE;
    if (layer_begin < 0 || layer_begin > cfg->num_layers - num_layers) return KVQ_ERR_RANGE;
    if (chunk_tokens < 0 || chunk_tokens % 32) return KVQ_ERR_SHAPE;
    const int G = cfg->num_q_heads / cfg->num_kv_heads;
    if (G > kMaxGroupRatio) return KVQ_ERR_UNSUPPORTED;
    const bool use_mfma = mfma_supported(cfg->head_dim, cfg->group_size, G);
    const DecodePlan plan = plan_decode(cfg, layer_begin, num_layers, chunk_tokens, use_mfma);
    if (!workspace) {
      *workspace_bytes = plan.total;
      return KVQ_OK;
    }
    if (!cache || !seq_lens || !q || !out) return KVQ_ERR_NULL;
    if (*workspace_bytes < plan.total) return KVQ_ERR_WORKSPACE;
    if (!aligned(cache, 256) || !aligned(workspace, 256) || !aligned(q, 16) || !aligned(out, 16) ||
        !aligned(seq_lens, 4))
      return KVQ_ERR_ALIGN;
    Layout lay(cfg);
    if (lay.info.total_bytes / 256 >= (uint64_t(1) << 32)) return KVQ_ERR_UNSUPPORTED;

    const int Hkv = cfg->num_kv_heads;
    const int nlh = num_layers * Hkv;
    // Heavier (layer, head) pairs first so long workgroups start early.
    std::vector<int> order(nlh);
    for (int i = 0; i < nlh; ++i) order[i] = i;
    std::stable_sort(order.begin(), order.end(), [&](int x, int y) {
      const int lx = layer_begin + x / Hkv, hx = x % Hkv, ly = layer_begin + y / Hkv, hy = y % Hkv;
      const int bx = vis_row_bytes(lay.D, bits_of(cfg, lx, hx, 0)) + vis_row_bytes(lay.D, bits_of(cfg, lx, hx, 1));
      const int by = vis_row_bytes(lay.D, bits_of(cfg, ly, hy, 0)) + vis_row_bytes(lay.D, bits_of(cfg, ly, hy, 1));
      return bx > by;
    });

    // Matrix-core launches are per visual format: each launch takes the pairs
    // whose visual K/V widths are one (kb, vb) combination, and the all-bf16
    // (protected) pairs ride along with the first such group.
    std::vector<int> fkey(nlh);
    std::vector<int> groups;  // distinct keys kb * 32 + vb, in slot order
    for (int i = 0; i < nlh; ++i) {
      const int glh = order[i], l = layer_begin + glh / Hkv, h = glh % Hkv;
      fkey[i] = bits_of(cfg, l, h, 0) * 32 + bits_of(cfg, l, h, 1);
    }
    for (int i = 0; i < nlh; ++i)
      if (fkey[i] != 16 * 32 + 16 && std::find(groups.begin(), groups.end(), fkey[i]) == groups.end())
        groups.push_back(fkey[i]);
    if (groups.empty()) groups.push_back(16 * 32 + 16);
    if (!use_mfma) groups.assign(1, -1);  // the general kernel takes every format

    uint8_t* ws = static_cast<uint8_t*>(workspace);
    const hipStream_t hs = static_cast<hipStream_t>(stream);
    std::vector<int> sel;
    sel.reserve(nlh);
    for (int s0 = 0; s0 < cfg->batch; s0 += kMaxSeq) {
      const int ns_l = std::min(kMaxSeq, cfg->batch - s0);
      DecodeArgs a;
      std::memset(&a, 0, sizeof(a));
      a.cache = static_cast<const uint8_t*>(cache);
      a.seq_lens = seq_lens;
      a.q = static_cast<const uint16_t*>(q);
      a.out = static_cast<uint16_t*>(out);
      a.ws_o = reinterpret_cast<float*>(ws);
      a.ws_ml = reinterpret_cast<float*>(ws + plan.o_bytes);
      a.ws_cnt = reinterpret_cast<int32_t*>(ws + plan.o_bytes + plan.ml_bytes);
      a.ws_arrive = reinterpret_cast<int32_t*>(ws + plan.o_bytes + plan.ml_bytes + plan.cnt_bytes);
      a.qscale = sm_scale * 1.4426950408889634f;
      a.Rvis = lay.Rvis;
      a.D = lay.D;
      a.g = lay.g;
      a.G = G;
      a.Hkv = Hkv;
      a.Hq = cfg->num_q_heads;
      a.B = cfg->batch;
      a.chunk = plan.chunk;
      a.max_chunks = plan.max_chunks;
      a.seq_off = s0;
      for (int i = 0; i < ns_l; ++i) {
        const int s = s0 + i;
        a.vb[i] = cfg->vis_begin[s];
        a.ve[i] = cfg->vis_end[s];
        a.cap[i] = cfg->capacity[s];
        a.vrow0[i] = int32_t(lay.vrow0[s]);
        a.trow0[i] = int32_t(lay.trow0[s]);
        a.nx[i] = plan.nx[s];
        a.nxcum[i + 1] = a.nxcum[i] + plan.nx[s];
      }
      a.n_seq = ns_l;
      for (size_t gi = 0; gi < groups.size(); ++gi) {
        const int key = groups[gi];
        sel.clear();
        for (int i = 0; i < nlh; ++i)
          if (key < 0 || fkey[i] == key || (gi == 0 && fkey[i] == 16 * 32 + 16)) sel.push_back(i);
        for (size_t k0 = 0; k0 < sel.size(); k0 += kMaxLH) {
          const int nlh_l = int(std::min<size_t>(kMaxLH, sel.size() - k0));
          a.n_lh = nlh_l;
          for (int i = 0; i < nlh_l; ++i) {
            const int glh = order[sel[k0 + i]];  // layer-local * Hkv + head
            const int l = layer_begin + glh / Hkv, h = glh % Hkv;
            for (int X = 0; X < 2; ++X) {
              a.base256[i][X] = uint32_t(lay.vis_off[(size_t(l) * Hkv + h) * 2 + X] / 256);
              a.bits[i][X] = uint8_t(bits_of(cfg, l, h, X));
            }
            a.lh_glob[i] = uint16_t(glh);
            a.mult[i] = plan.mult[glh];
            a.mcum[i + 1] = uint16_t(a.mcum[i] + a.mult[i]);
          }
          const hipError_t e = use_mfma ? launch_decode_mfma(a, key / 32, key % 32, hs)
                                        : launch_decode_simple(a, ns_l, hs);
          if (e != hipSuccess) return KVQ_ERR_HIP;
        }
      }
      // the general kernel leaves split partials for a separate merge; the
      // matrix-core kernel merges them itself
      if (!use_mfma && plan.max_chunks > 1 &&
          launch_decode_merge(a, num_layers, ns_l, hs) != hipSuccess)
        return KVQ_ERR_HIP;
    }
    return KVQ_OK;
  } catch (...) {
    return KVQ_ERR_INTERNAL;
  }
}
