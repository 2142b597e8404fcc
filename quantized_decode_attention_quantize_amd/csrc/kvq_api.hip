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
#include <memory>
#include <mutex>
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
  if (c->num_q_heads % c->num_kv_heads) return KVQ_ERR_UNSUPPORTED;
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
  if (c->k_per_channel && c->rotate_k) return KVQ_ERR_UNSUPPORTED;
  if (c->bf16_range_offsets) {
    const int32_t* o = c->bf16_range_offsets;
    if (!c->bf16_range_begin || !c->bf16_range_end) return KVQ_ERR_NULL;
    if (o[0] != 0) return KVQ_ERR_SHAPE;
    for (int s = 0; s < c->batch; ++s) {
      if (o[s + 1] < o[s]) return KVQ_ERR_SHAPE;
      int prev = c->vis_begin[s];
      for (int k = o[s]; k < o[s + 1]; ++k) {
        const int b = c->bf16_range_begin[k], e = c->bf16_range_end[k];
        if (b < prev || e <= b || e > c->vis_end[s]) return KVQ_ERR_SHAPE;
        prev = e;
      }
      if (o[s + 1] > o[s] && c->k_per_channel) return KVQ_ERR_UNSUPPORTED;
      if (o[s + 1] - o[s] > kMaxRangesD) return KVQ_ERR_UNSUPPORTED;
    }
  }
  return KVQ_OK;
}

// bf16 ranges of sequence s: [first, last) indices into the range arrays.
int ranges_first(const kvq_config* c, int s) {
  return c->bf16_range_offsets ? c->bf16_range_offsets[s] : 0;
}
int ranges_count(const kvq_config* c, int s) {
  return c->bf16_range_offsets ? c->bf16_range_offsets[s + 1] - c->bf16_range_offsets[s] : 0;
}

// End of the coded part of sequence s's visual span: all of it with per-token
// groups; whole g-token blocks from vis_begin with per-channel K (the tail is
// the bf16 residual window).
int coded_end(const kvq_config* c, int s) {
  const int vb = c->vis_begin[s], ve = c->vis_end[s], g = c->group_size;
  return c->k_per_channel ? vb + (ve - vb) / g * g : ve;
}

// Coded positions of sequence s: its coded span minus its bf16 ranges.
int64_t coded_count(const kvq_config* c, int s) {
  int64_t n = coded_end(c, s) - c->vis_begin[s];
  for (int k = ranges_first(c, s); k < ranges_first(c, s) + ranges_count(c, s); ++k)
    n -= c->bf16_range_end[k] - c->bf16_range_begin[k];
  return n;
}

// Consecutive sequence groups [s0, s0 + n) of at most kMaxSeq sequences
// whose bf16 ranges fit a launch's table of `max_ranges`.
std::vector<std::pair<int, int>> sequence_groups(const kvq_config* c, const int32_t* ids,
                                                 int count, int max_ranges) {
  std::vector<std::pair<int, int>> out;
  int s0 = 0;
  while (s0 < count) {
    int n = 0, nr = 0;
    while (s0 + n < count && n < kMaxSeq) {
      const int r = ranges_count(c, ids ? ids[s0 + n] : s0 + n);
      if (n > 0 && nr + r > max_ranges) break;
      nr += r;
      ++n;
    }
    out.emplace_back(s0, n);
    s0 += n;
  }
  return out;
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
      const int64_t nv = coded_count(c, s);
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

}  // namespace

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

namespace {

static_assert(sizeof(DecodeArgs) <= 4096, "decode kernel arguments exceed 4 KB");
static_assert(sizeof(QuantizeArgs) <= 4096, "quantize kernel arguments exceed 4 KB");

// One kernel launch of a decode call: up to kMaxLH (layer, head) slots of
// one visual format over up to kMaxSeq sequences.  Work is laid out in units
// (waves): slot i and sequence s get mult[i] * nx[s] consecutive units,
// slot-major.
struct LaunchPlan {
  int key;                  // format key kb * 32 + vb
  int s0, ns;               // sequences [s0, s0 + ns) of the call
  std::vector<int> glh;     // per slot: layer-local * Hkv + head
  std::vector<int> mult;    // per slot
  std::vector<int> nx;      // per sequence of the launch
};

struct DecodePlan {
  int chunk;                // tokens per split; 0 = balanced split
  int nsub, gsub;           // query-head subgroups of every launch, heads in each (<=)
  std::vector<LaunchPlan> launches;
  int max_chunks;           // partial slots per (layer, seq, head)
  int64_t entries;
  size_t o_bytes, ml_bytes, cnt_bytes, arrive_bytes, total;
};

// Relative time of one row of a (layer, head) pair on the matrix-core
// kernel: the bytes its visual row moves plus a fixed share for the per-row
// arithmetic (waves of INT4/INT2 and of bf16 heads at D = 128 running side by
// side take about 1 : 3.5 per row, which this reproduces).
constexpr double kPerChannelCost = 1.8;  // per-channel coded rows vs per-token, measured

double row_cost(int D, int g, int kb, int vb) {
  double bytes = vis_row_bytes(D, kb) + vis_row_bytes(D, vb);
  if (kb < 16) bytes += (D / g) * 4;
  if (vb < 16) bytes += (D / g) * 4;
  return 0.38 * D + bytes;
}

// Smallest-maximum split of `budget` units over items of weight w[k], each
// item at least one unit: n[k] = max(1, ceil(w[k] / T)) for the least T (to
// bisection precision) with sum n <= budget.  Needs budget >= w.size().
void minmax_split(const std::vector<double>& w, int64_t budget, std::vector<int>& n) {
  const int64_t K = int64_t(w.size());
  double wmax = 0.0, wsum = 0.0;
  for (double x : w) {
    wmax = std::max(wmax, x);
    wsum += x;
  }
  if (wmax <= 0.0) wmax = wsum = 1.0;
  auto units = [](double x, double T) {
    return std::max<int64_t>(1, int64_t(std::ceil(x / T)));
  };
  auto need = [&](double T) {
    int64_t t = 0;
    for (double x : w) t += units(x, T);
    return t;
  };
  // sum ceil(w / T) lies in [wsum / T, wsum / T + K], so the optimum lies in
  // [wsum / budget, wsum / (budget - K)] (and T = wmax always fits)
  double lo = wsum / double(budget), hi = wmax;
  if (budget > K) hi = std::min(hi, wsum / double(budget - K));
  if (need(hi) > budget) hi = wmax;
  for (int it = 0; it < 24; ++it) {
    const double mid = 0.5 * (lo + hi);
    if (need(mid) <= budget) hi = mid; else lo = mid;
  }
  n.resize(w.size());
  for (size_t k = 0; k < w.size(); ++k) n[k] = int(units(w[k], hi));
}

// Balanced split of one matrix-core launch over `waves` units.  Per
// (slot i, seq s) the work is cost[i] * cap[s]; the layout gives it
// mult[i] * nx[s] units, so the slowest unit takes
// max_i(cost_i / mult_i) * max_s(cap_s / nx_s), which is returned.  For each
// candidate total X of nx, nx is the smallest-maximum split of X by capacity
// and mult that of waves / X by cost; the best candidate wins.
double balance_units(const std::vector<double>& cost, const std::vector<double>& cap,
                     int64_t waves, std::vector<int>& mult, std::vector<int>& nx) {
  const int64_t S = int64_t(cost.size()), B = int64_t(cap.size());
  const int64_t xmax = std::max<int64_t>(B, waves / S);
  const int64_t span = xmax - B + 1;
  const int64_t ncand = std::min<int64_t>(span, 32);
  double best = -1.0;
  int64_t best_units = 0;
  std::vector<int> m, x;
  for (int64_t k = 0; k < ncand; ++k) {
    const int64_t X = ncand == 1 ? B : B + (span - 1) * k / (ncand - 1);
    minmax_split(cap, X, x);
    int64_t xs = 0;
    for (int v : x) xs += v;
    minmax_split(cost, std::max<int64_t>(S, waves / xs), m);
    double tm = 0.0, tx = 0.0;
    int64_t ms = 0;
    for (int64_t i = 0; i < S; ++i) {
      tm = std::max(tm, cost[i] / m[i]);
      ms += m[i];
    }
    for (int64_t s = 0; s < B; ++s) tx = std::max(tx, cap[s] / x[s]);
    const double t = tm * tx;
    if (best < 0.0 || t < best * (1.0 - 1e-9) || (t <= best * (1.0 + 1e-9) && ms * xs < best_units)) {
      best = t;
      best_units = ms * xs;
      mult = m;
      nx = x;
    }
  }
  return best;
}

// Balanced split of one matrix-core launch over `waves` wave slots, in
// waves.  A split in whole workgroups (every entry a multiple of 8 waves)
// keeps each (layer, seq, head) of a workgroup on one claim counter and
// leaves fewer partials to merge; it is taken unless the wave-granular split
// is clearly faster (the loop often runs near the memory bound, where extra
// balance buys less than the model says).
void balance_launch(const std::vector<double>& cost, const std::vector<double>& cap,
                    int64_t waves, std::vector<int>& mult, std::vector<int>& nx) {
  std::vector<int> mw, xw, mg, xg;
  const double tw = balance_units(cost, cap, waves, mw, xw);
  const int64_t groups = waves / kMfmaWaves;
  if (groups >= int64_t(cost.size()) * int64_t(cap.size())) {
    const double tg = balance_units(cost, cap, groups, mg, xg) / kMfmaWaves;
    if (tg <= 1.15 * tw) {
      for (int& m : mg) m *= kMfmaWaves;
      mult = mg;
      nx = xg;
      return;
    }
  }
  mult = mw;
  nx = xw;
}

// Pieces (workgroups touched) of the unit range [w0, w0 + n) at `per` units
// per workgroup.
int64_t pieces(int64_t w0, int64_t n, int per) { return (w0 + n - 1) / per - w0 / per + 1; }

// Split planning.  With chunk_tokens > 0 every (layer, seq, head) is cut into
// fixed token chunks, one workgroup each.  Otherwise each launch spreads its
// work over all the device's wave slots (8 waves per CU, two per SIMD) with
// the balanced split above; a workgroup may then hold waves of several
// (layer, seq, head) entries.  A KV head whose query heads need more than
// one 16-column tile ((D / g) * G > 16) is decoded in nsub launches, one per
// subgroup of its query heads: each reads the K/V rows again, which still
// runs far ahead of any vector-ALU path.
constexpr int kSmallCallChunk = 512;  // tokens per workgroup for small calls (see below)

DecodePlan plan_decode(const kvq_config* c, int layer_begin, int nl, int chunk_tokens) {
  DecodePlan p;
  const int B = c->batch, Hkv = c->num_kv_heads, D = c->head_dim, g = c->group_size;
  const int nlh = nl * Hkv;
  const int Gfull = c->num_q_heads / Hkv;
  p.nsub = mfma_subgroups(D, g, Gfull);
  p.gsub = (Gfull + p.nsub - 1) / p.nsub;
  p.chunk = chunk_tokens > 0 ? chunk_tokens : 0;
  // A small call (fewer rows than one 32-token step per wave slot, e.g. one
  // layer of a 6K-token sequence) is bound by latency, not bandwidth: fixed
  // 512-token chunks (static, 2 steps per wave, at most 16 partials for a
  // 6K-token sequence, which the wave-parallel merge takes) beat spreading
  // it over every wave slot, and 1024-token ones (one-layer launches of the
  // 28-layer HeadGuard step: 15.45 against 17.8 us).
  if (p.chunk == 0) {
    int64_t rows = 0;
    for (int s = 0; s < B; ++s) rows += int64_t(c->capacity[s]) * nlh;
    if (rows < int64_t(32) * kMfmaWaves * device_cus()) p.chunk = kSmallCallChunk;
  }

  // Heavier (layer, head) pairs first.  Matrix-core launches are per visual
  // format: each takes the pairs whose visual K/V widths are one (kb, vb)
  // combination, and the all-bf16 (protected) pairs ride along with the
  // first such group.
  std::vector<int> order(nlh);
  for (int i = 0; i < nlh; ++i) order[i] = i;
  auto row_bytes = [&](int glh) {
    const int l = layer_begin + glh / Hkv, h = glh % Hkv;
    return vis_row_bytes(D, bits_of(c, l, h, 0)) + vis_row_bytes(D, bits_of(c, l, h, 1));
  };
  std::stable_sort(order.begin(), order.end(),
                   [&](int x, int y) { return row_bytes(x) > row_bytes(y); });
  std::vector<int> fkey(nlh);
  std::vector<int> groups;  // distinct keys kb * 32 + vb, in slot order
  for (int i = 0; i < nlh; ++i) {
    const int glh = order[i], l = layer_begin + glh / Hkv, h = glh % Hkv;
    fkey[i] = bits_of(c, l, h, 0) * 32 + bits_of(c, l, h, 1);
  }
  for (int i = 0; i < nlh; ++i)
    if (fkey[i] != 16 * 32 + 16 && std::find(groups.begin(), groups.end(), fkey[i]) == groups.end())
      groups.push_back(fkey[i]);
  if (groups.empty()) groups.push_back(16 * 32 + 16);

  const int64_t wave_slots = int64_t(kMfmaWaves) * device_cus();
  constexpr int kMinWaveRows = 64;  // fewer rows per wave only add merge work
  int64_t max_pieces = 1;
  for (const auto& grp : sequence_groups(c, nullptr, B, kMaxRangesD)) {
    const int s0 = grp.first, ns = grp.second;
    for (size_t gi = 0; gi < groups.size(); ++gi) {
      std::vector<int> sel;
      for (int i = 0; i < nlh; ++i)
        if (groups[gi] < 0 || fkey[i] == groups[gi] || (gi == 0 && fkey[i] == 16 * 32 + 16))
          sel.push_back(order[i]);
      for (size_t k0 = 0; k0 < sel.size(); k0 += kMaxLH) {
        LaunchPlan L;
        L.key = groups[gi];
        L.s0 = s0;
        L.ns = ns;
        L.glh.assign(sel.begin() + k0, sel.begin() + std::min(sel.size(), k0 + kMaxLH));
        const int S = int(L.glh.size());
        if (p.chunk > 0) {
          // fixed chunks: one workgroup (8 waves on the matrix-core kernel) each
          L.mult.assign(S, kMfmaWaves);
          L.nx.resize(ns);
          for (int i = 0; i < ns; ++i) L.nx[i] = (c->capacity[s0 + i] + p.chunk - 1) / p.chunk;
        } else {
          std::vector<double> cost(S), cap(ns);
          double rows = 0.0;
          for (int i = 0; i < S; ++i) {
            const int l = layer_begin + L.glh[i] / Hkv, h = L.glh[i] % Hkv;
            const int kb = bits_of(c, l, h, 0);
            cost[i] = row_cost(D, g, kb, bits_of(c, l, h, 1));
            // coded per-channel K takes a second MFMA per k-step and a META
            // stage per block: its steps measured 1.8x the per-token ones
            if (c->k_per_channel && kb < 16) cost[i] *= kPerChannelCost;
          }
          for (int i = 0; i < ns; ++i) {
            cap[i] = c->capacity[s0 + i];
            rows += cap[i] * S;
          }
          const int64_t waves = std::max<int64_t>(
              1, std::min<int64_t>(wave_slots, int64_t(rows / kMinWaveRows)));
          balance_launch(cost, cap, waves, L.mult, L.nx);
        }
        // partials per (layer, seq, head): workgroups its unit range touches
        const int per = kMfmaWaves;
        int64_t xs = 0, mc = 0;
        for (int v : L.nx) xs += v;
        for (int i = 0; i < S; ++i) {
          int64_t xc = 0;
          for (int s = 0; s < ns; ++s) {
            const int64_t w0 = xs * mc + int64_t(L.mult[i]) * xc;
            max_pieces = std::max(max_pieces, pieces(w0, int64_t(L.mult[i]) * L.nx[s], per));
            xc += L.nx[s];
          }
          mc += L.mult[i];
        }
        p.launches.push_back(std::move(L));
      }
    }
  }
  p.max_chunks = int(max_pieces);
  const int G = p.gsub;  // partials hold one subgroup's heads at a time
  p.entries = int64_t(nl) * B * Hkv * p.max_chunks;
  // The arrival counters come first and are sized by the cache configuration
  // (every layer, sequence and KV head), not by this call: every call on one
  // cache finds them at the same offsets, and no call's partials ever land on
  // them, so a workspace zero-filled once stays valid for calls of any shape.
  p.arrive_bytes = size_t(align256(int64_t(c->num_layers) * B * Hkv * 4));
  p.o_bytes = size_t(align256(p.entries * G * c->head_dim * 4));
  p.ml_bytes = size_t(align256(p.entries * G * 2 * 4));
  p.cnt_bytes = size_t(align256(int64_t(nl) * B * Hkv * 4));
  p.total = p.arrive_bytes + p.o_bytes + p.ml_bytes + p.cnt_bytes;
  return p;
}

// Plans depend only on the call's shape (not on the sequence lengths, which
// stay on the device), and decoding repeats one shape step after step, so the
// last few plans are kept, keyed by everything plan_decode reads: the layer
// count of the cache sizes the arrival counters, so it is part of the key.
std::shared_ptr<const DecodePlan> cached_plan(const kvq_config* c, int layer_begin, int nl,
                                              int chunk_tokens) {
  constexpr size_t kKeep = 4;
  static std::mutex mu;
  static std::vector<std::pair<std::vector<int32_t>, std::shared_ptr<const DecodePlan>>> kept;
  const int Hkv = c->num_kv_heads;
  std::vector<int32_t> key = {layer_begin, nl, chunk_tokens, device_cus(),
                              c->num_layers, c->batch, c->num_q_heads, Hkv, c->head_dim,
                              c->group_size, c->k_per_channel != 0};
  key.reserve(key.size() + c->batch + size_t(nl) * Hkv);
  for (int s = 0; s < c->batch; ++s) key.push_back(c->capacity[s]);
  for (int s = 0; s < c->batch; ++s) key.push_back(ranges_count(c, s));  // launch grouping
  for (int i = layer_begin * Hkv; i < (layer_begin + nl) * Hkv; ++i)
    key.push_back(c->k_bits[i] * 32 + c->v_bits[i]);
  std::lock_guard<std::mutex> lock(mu);
  for (size_t i = 0; i < kept.size(); ++i)
    if (kept[i].first == key) {
      std::rotate(kept.begin(), kept.begin() + i, kept.begin() + i + 1);  // most recent first
      return kept.front().second;
    }
  auto plan = std::make_shared<const DecodePlan>(
      plan_decode(c, layer_begin, nl, chunk_tokens));
  kept.insert(kept.begin(), {std::move(key), plan});
  if (kept.size() > kKeep) kept.pop_back();
  return plan;
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

// Shared body of the two store calls: sequence seq_ids[i] stores positions
// [tok0[i], tok0[i] + n_tok).
kvq_status quantize_rows(const kvq_config* cfg, void* cache, int32_t layer_begin,
                         int32_t num_layers, int32_t num_seqs, const int32_t* seq_ids,
                         const int32_t* tok0, int32_t n_tok, const void* k_src,
                         const void* v_src, kvq_src_dtype src_dtype, void* stream) {
  kvq_status st = check_config(cfg);
  if (st != KVQ_OK) return st;
  if (src_dtype != KVQ_SRC_F32 && src_dtype != KVQ_SRC_BF16) return KVQ_ERR_UNSUPPORTED;
  if (num_layers < 1 || num_seqs < 0 || n_tok < 0) return KVQ_ERR_SHAPE;
  if (layer_begin < 0 || layer_begin > cfg->num_layers - num_layers) return KVQ_ERR_RANGE;
  if (num_seqs == 0 || n_tok == 0) return KVQ_OK;
  if (!cache || !k_src || !v_src || !seq_ids || !tok0) return KVQ_ERR_NULL;
  if (!aligned(cache, 256) || !aligned(k_src, 16) || !aligned(v_src, 16)) return KVQ_ERR_ALIGN;
  std::vector<char> seen(cfg->batch, 0);
  for (int i = 0; i < num_seqs; ++i) {
    const int s = seq_ids[i];
    if (s < 0 || s >= cfg->batch) return KVQ_ERR_RANGE;
    if (seen[s]) return KVQ_ERR_SHAPE;
    seen[s] = 1;
    if (tok0[i] < 0) return KVQ_ERR_SHAPE;
    if (int64_t(tok0[i]) + n_tok > cfg->capacity[s]) return KVQ_ERR_RANGE;
  }
  // per-channel K: the stored positions must not cut a block of the coded span
  std::vector<int> kb0(num_seqs, 0), kbn(num_seqs, 0);
  if (cfg->k_per_channel) {
    const int g = cfg->group_size;
    for (int i = 0; i < num_seqs; ++i) {
      const int s = seq_ids[i], vb = cfg->vis_begin[s], qe = coded_end(cfg, s);
      const int lo = std::max(tok0[i], vb), hi = std::min(tok0[i] + n_tok, qe);
      if (lo < hi) {
        if ((lo - vb) % g || (hi - vb) % g) return KVQ_ERR_SHAPE;
        kb0[i] = (lo - vb) / g;
        kbn[i] = (hi - lo) / g;
      }
    }
  }
  Layout lay(cfg);
  if (lay.info.total_bytes / 256 >= (uint64_t(1) << 32)) return KVQ_ERR_UNSUPPORTED;

  const int nlh = num_layers * cfg->num_kv_heads;
  const auto groups = sequence_groups(cfg, seq_ids, num_seqs, kMaxRangesQ);
  for (int lh0 = 0; lh0 < nlh; lh0 += kMaxLH) {
    const int nlh_l = std::min(kMaxLH, nlh - lh0);
    for (const auto& grp : groups) {
      const int s0 = grp.first, ns_l = grp.second;
      QuantizeArgs a;
      std::memset(&a, 0, sizeof(a));
      a.cache = static_cast<uint8_t*>(cache);
      a.k_src = k_src;
      a.v_src = v_src;
      a.Rvis = lay.Rvis;
      a.D = lay.D;
      a.g = lay.g;
      a.src_bf16 = src_dtype == KVQ_SRC_BF16;
      a.rotate_k = cfg->rotate_k != 0;
      a.n_tok = n_tok;
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
      a.k_per_channel = cfg->k_per_channel != 0;
      int max_blocks = 0;
      for (int i = 0; i < ns_l; ++i) {
        const int s = seq_ids[s0 + i];
        a.rng_first[i + 1] = a.rng_first[i] + ranges_count(cfg, s);
        for (int k = 0; k < ranges_count(cfg, s); ++k) {
          a.rng_b[a.rng_first[i] + k] = cfg->bf16_range_begin[ranges_first(cfg, s) + k];
          a.rng_e[a.rng_first[i] + k] = cfg->bf16_range_end[ranges_first(cfg, s) + k];
        }
        a.vb[i] = cfg->vis_begin[s];
        a.ve[i] = coded_end(cfg, s);
        a.vrow0[i] = int32_t(lay.vrow0[s]);
        a.trow0[i] = int32_t(lay.trow0[s]);
        a.tok0[i] = tok0[s0 + i];
        a.kblk0[i] = kb0[s0 + i];
        a.kblkn[i] = kbn[s0 + i];
        max_blocks = std::max(max_blocks, kbn[s0 + i]);
      }
      if (launch_quantize(a, nlh_l, ns_l, static_cast<hipStream_t>(stream)) != hipSuccess)
        return KVQ_ERR_HIP;
      if (a.k_per_channel &&
          launch_quantize_kblocks(a, nlh_l, ns_l, max_blocks, static_cast<hipStream_t>(stream)) !=
              hipSuccess)
        return KVQ_ERR_HIP;
    }
  }
  return KVQ_OK;
}

extern "C" kvq_status kvq_quantize(const kvq_config* cfg, void* cache, int32_t layer_begin,
                                   int32_t num_layers, int32_t num_seqs, const int32_t* seq_ids,
                                   int32_t tok_begin, int32_t tok_end, const void* k_src,
                                   const void* v_src, kvq_src_dtype src_dtype, void* stream) {
  try {
    if (tok_begin < 0 || tok_end < tok_begin) {
      const kvq_status st = check_config(cfg);
      return st != KVQ_OK ? st : KVQ_ERR_SHAPE;
    }
    const std::vector<int32_t> tok0(size_t(std::max(num_seqs, 0)), tok_begin);
    return quantize_rows(cfg, cache, layer_begin, num_layers, num_seqs, seq_ids, tok0.data(),
                         tok_end - tok_begin, k_src, v_src, src_dtype, stream);
  } catch (const std::bad_alloc&) {
    return KVQ_ERR_INTERNAL;
  } catch (...) {
    return KVQ_ERR_INTERNAL;
  }
}

extern "C" kvq_status kvq_quantize_ragged(const kvq_config* cfg, void* cache,
                                          int32_t layer_begin, int32_t num_layers,
                                          int32_t num_seqs, const int32_t* seq_ids,
                                          const int32_t* tok_begin, int32_t num_tokens,
                                          const void* k_src, const void* v_src,
                                          kvq_src_dtype src_dtype, void* stream) {
  try {
    return quantize_rows(cfg, cache, layer_begin, num_layers, num_seqs, seq_ids, tok_begin,
                         num_tokens, k_src, v_src, src_dtype, stream);
  } catch (const std::bad_alloc&) {
    return KVQ_ERR_INTERNAL;
  } catch (...) {
    return KVQ_ERR_INTERNAL;
  }
}

// Workspace regions of one decode call: the merge's arrival counters, the
// partial rows, their (m, l) pairs and the per-entry partial counts.
struct WsRegions {
  uint8_t* arrive;
  uint8_t* rest;  // partials, (m, l) pairs and counts follow here, as planned
};

// Checks shared by both decode entry points; on success *plan holds the call's
// split plan.
static kvq_status decode_prologue(const kvq_config* cfg, int32_t layer_begin, int32_t num_layers,
                           int32_t chunk_tokens, std::shared_ptr<const DecodePlan>* plan) {
  kvq_status st = check_config(cfg);
  if (st != KVQ_OK) return st;
  if (num_layers < 1) return KVQ_ERR_SHAPE;
  if (layer_begin < 0 || layer_begin > cfg->num_layers - num_layers) return KVQ_ERR_RANGE;
  if (chunk_tokens < 0 || chunk_tokens % 32) return KVQ_ERR_SHAPE;
  const int G = cfg->num_q_heads / cfg->num_kv_heads;
  if (G > kMaxGroupRatio) return KVQ_ERR_UNSUPPORTED;
  if (mfma_subgroups(cfg->head_dim, cfg->group_size, G) < 1) return KVQ_ERR_UNSUPPORTED;
  if (cfg->k_per_channel) {
    // per-channel K runs on the staged path (coded K with coded V), and its
    // 32-token steps must fall on the block grid: fixed chunks in multiples
    // of 256 tokens (eight waves of whole steps)
    if (chunk_tokens % 256) return KVQ_ERR_UNSUPPORTED;
    for (int i = layer_begin * cfg->num_kv_heads; i < (layer_begin + num_layers) * cfg->num_kv_heads; ++i)
      if (cfg->k_bits[i] < 16 && cfg->v_bits[i] == 16) return KVQ_ERR_UNSUPPORTED;
  }
  *plan = cached_plan(cfg, layer_begin, num_layers, chunk_tokens);
  return KVQ_OK;
}

// Launches of one validated decode call over workspace regions `wr`.
// Sources of a decode-time append (kvq_decode_attention_append); mode 0: none.
struct AppendSrc {
  const void* k = nullptr;
  const void* v = nullptr;
  int mode = 0;  // 1 bf16, 2 fp32
};

static kvq_status decode_launch(const kvq_config* cfg, const void* cache, int32_t layer_begin,
                         int32_t num_layers, const int32_t* seq_lens, const void* q, void* out,
                         float sm_scale, const DecodePlan& plan, WsRegions wr,
                         void* stream, AppendSrc app = AppendSrc()) {
  if (!cache || !seq_lens || !q || !out) return KVQ_ERR_NULL;
  if (!aligned(cache, 256) || !aligned(q, 16) || !aligned(out, 16) || !aligned(seq_lens, 4))
    return KVQ_ERR_ALIGN;
  Layout lay(cfg);
  if (lay.info.total_bytes / 256 >= (uint64_t(1) << 32)) return KVQ_ERR_UNSUPPORTED;

  const int Hkv = cfg->num_kv_heads;
  const int G = cfg->num_q_heads / Hkv;
  // unit counts of every launch fit the kernels' 32-bit block arithmetic
  for (const LaunchPlan& L : plan.launches) {
    int64_t xs = 0, ms = 0;
    for (int v : L.nx) xs += v;
    for (int v : L.mult) ms += v;
    if (xs * ms >= (int64_t(1) << 31) || ms > 0xFFFF) return KVQ_ERR_UNSUPPORTED;
  }
  const hipStream_t hs = static_cast<hipStream_t>(stream);
  // every launch once per query-head subgroup (stream order keeps a
  // subgroup's use of the workspace after the previous one's)
  for (int sg = 0; sg < plan.nsub; ++sg)
  for (const LaunchPlan& L : plan.launches) {
    const int g0 = sg * plan.gsub;  // first query head of the subgroup
    DecodeArgs a;
    std::memset(&a, 0, sizeof(a));
    a.cache = static_cast<const uint8_t*>(cache);
    a.seq_lens = seq_lens;
    a.q = static_cast<const uint16_t*>(q) + int64_t(g0) * cfg->head_dim;
    a.out = static_cast<uint16_t*>(out) + int64_t(g0) * cfg->head_dim;
    a.ws_arrive = reinterpret_cast<int32_t*>(wr.arrive);
    a.ws_o = reinterpret_cast<float*>(wr.rest);
    a.ws_ml = reinterpret_cast<float*>(wr.rest + plan.o_bytes);
    a.ws_cnt = reinterpret_cast<int32_t*>(wr.rest + plan.o_bytes + plan.ml_bytes);
    a.qscale = sm_scale * 1.4426950408889634f;
    a.Rvis = lay.Rvis;
    a.D = lay.D;
    a.g = lay.g;
    a.G = std::min(plan.gsub, G - g0);
    a.g_stride = uint8_t(G);
    a.Hkv = Hkv;
    a.Hq = cfg->num_q_heads;
    a.B = cfg->batch;
    a.chunk = plan.chunk;
    a.rotate_k = cfg->rotate_k != 0;
    a.k_per_channel = cfg->k_per_channel != 0;
    a.max_chunks = plan.max_chunks;
    a.app_mode = uint8_t(app.mode);
    a.app_k = app.k;
    a.app_v = app.v;
    a.seq_off = L.s0;
    a.n_seq = L.ns;
    for (int i = 0; i < L.ns; ++i) {
      const int s = L.s0 + i;
      a.vb[i] = cfg->vis_begin[s];
      a.ve[i] = coded_end(cfg, s);
      a.cap[i] = cfg->capacity[s];
      a.vrow0[i] = int32_t(lay.vrow0[s]);
      a.trow0[i] = int32_t(lay.trow0[s]);
      a.nxcum[i + 1] = a.nxcum[i] + L.nx[i];
      a.rng_first[i + 1] = uint8_t(a.rng_first[i] + ranges_count(cfg, s));
      for (int k = 0; k < ranges_count(cfg, s); ++k) {
        a.rng_b[a.rng_first[i] + k] = cfg->bf16_range_begin[ranges_first(cfg, s) + k];
        a.rng_e[a.rng_first[i] + k] = cfg->bf16_range_end[ranges_first(cfg, s) + k];
      }
    }
    a.n_lh = int(L.glh.size());
    for (int i = 0; i < a.n_lh; ++i) {
      const int glh = L.glh[i];  // layer-local * Hkv + head
      const int l = layer_begin + glh / Hkv, h = glh % Hkv;
      for (int X = 0; X < 2; ++X) {
        a.base256[i][X] = uint32_t(lay.vis_off[(size_t(l) * Hkv + h) * 2 + X] / 256);
        a.bits[i][X] = uint8_t(bits_of(cfg, l, h, X));
      }
      a.lh_glob[i] = uint16_t(glh);
      a.mult[i] = uint16_t(L.mult[i]);
      a.mcum[i + 1] = uint16_t(a.mcum[i] + a.mult[i]);
    }
    if (launch_decode_mfma(a, L.key / 32, L.key % 32, hs) != hipSuccess) return KVQ_ERR_HIP;
  }
  return KVQ_OK;
}

extern "C" kvq_status kvq_decode_attention(const kvq_config* cfg, const void* cache,
                                           int32_t layer_begin, int32_t num_layers,
                                           const int32_t* seq_lens, const void* q, void* out,
                                           float sm_scale, int32_t chunk_tokens,
                                           void* workspace, size_t* workspace_bytes,
                                           void* stream) {
  try {
    std::shared_ptr<const DecodePlan> plan;
    kvq_status st = decode_prologue(cfg, layer_begin, num_layers, chunk_tokens, &plan);
    if (st != KVQ_OK) return st;
    if (!workspace_bytes) return KVQ_ERR_NULL;
    if (!workspace) {
      *workspace_bytes = plan->total;
      return KVQ_OK;
    }
    if (!cache || !seq_lens || !q || !out) return KVQ_ERR_NULL;
    if (*workspace_bytes < plan->total) return KVQ_ERR_WORKSPACE;
    if (!aligned(workspace, 256)) return KVQ_ERR_ALIGN;
    uint8_t* ws = static_cast<uint8_t*>(workspace);
    return decode_launch(cfg, cache, layer_begin, num_layers, seq_lens, q, out, sm_scale, *plan,
                         WsRegions{ws, ws + plan->arrive_bytes}, stream);
  } catch (...) {
    return KVQ_ERR_INTERNAL;
  }
}

extern "C" kvq_status kvq_decode_attention_append(
    const kvq_config* cfg, void* cache, int32_t layer_begin, int32_t num_layers,
    const int32_t* seq_lens, const void* k_new, const void* v_new, kvq_src_dtype src_dtype,
    const void* q, void* out, float sm_scale, int32_t chunk_tokens, void* workspace,
    size_t* workspace_bytes, void* stream) {
  try {
    std::shared_ptr<const DecodePlan> plan;
    kvq_status st = decode_prologue(cfg, layer_begin, num_layers, chunk_tokens, &plan);
    if (st != KVQ_OK) return st;
    if (!workspace_bytes) return KVQ_ERR_NULL;
    if (!workspace) {
      *workspace_bytes = plan->total;
      return KVQ_OK;
    }
    if (!cache || !seq_lens || !q || !out || !k_new || !v_new) return KVQ_ERR_NULL;
    if (src_dtype != KVQ_SRC_BF16 && src_dtype != KVQ_SRC_F32) return KVQ_ERR_UNSUPPORTED;
    if (*workspace_bytes < plan->total) return KVQ_ERR_WORKSPACE;
    if (!aligned(workspace, 256) || !aligned(k_new, 16) || !aligned(v_new, 16))
      return KVQ_ERR_ALIGN;
    uint8_t* ws = static_cast<uint8_t*>(workspace);
    AppendSrc app;
    app.k = k_new;
    app.v = v_new;
    app.mode = src_dtype == KVQ_SRC_BF16 ? 1 : 2;
    return decode_launch(cfg, cache, layer_begin, num_layers, seq_lens, q, out, sm_scale, *plan,
                         WsRegions{ws, ws + plan->arrive_bytes}, stream, app);
  } catch (...) {
    return KVQ_ERR_INTERNAL;
  }
}

// ---------------------------------------------------------------------------
// Decode without a caller workspace.  The split partials and arrival counters
// live in `scratch`, one copy per device (each GPU the library runs on holds
// it until the process ends).  Its first kScratchCounterBytes hold the arrival
// counters of every cache shape (indexed by (layer, seq, KV head), at most
// kScratchCounterBytes / 4 of them); the partials follow, so no call's
// partials ever land on another shape's counters.  Every call leaves the
// counters it used at zero, so the counter area stays zero between calls.
constexpr size_t kScratchBytes = size_t(16) << 20;
constexpr size_t kScratchCounterBytes = size_t(64) << 10;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

static __global__ void zero_words_kernel(uint32_t* p, int n) {
  const int i = int(blockIdx.x * blockDim.x + threadIdx.x);
  if (i < n) p[i] = 0u;
}

// Device address of this device's `scratch` (the array's name is only a
// host-side stand-in).  Looked up once per device, with that device current;
// the first call on a device also clears the counter area with a kernel on
// the caller's stream (a kernel, not a memset, so a graph may capture it).
static kvq_status scratch_for_device(hipStream_t stream, uint8_t** out) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static uint8_t* ptrs[kMaxDevices] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return KVQ_ERR_HIP;
  std::lock_guard<std::mutex> lock(mu);
  if (!ptrs[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return KVQ_ERR_HIP;
    constexpr int n = int(kScratchCounterBytes / 4);
    hipLaunchKernelGGL(zero_words_kernel, dim3((n + 255) / 256), dim3(256), 0, stream,
                       static_cast<uint32_t*>(p), n);
    if (hipGetLastError() != hipSuccess) return KVQ_ERR_HIP;
    ptrs[dev] = static_cast<uint8_t*>(p);
  }
  *out = ptrs[dev];
  return KVQ_OK;
}

extern "C" kvq_status kvq_decode_attention_noalloc(const kvq_config* cfg, const void* cache,
                                                   int32_t layer_begin, int32_t num_layers,
                                                   const int32_t* seq_lens, const void* q,
                                                   void* out, float sm_scale,
                                                   int32_t chunk_tokens, void* stream) {
  try {
    std::shared_ptr<const DecodePlan> plan;
    kvq_status st = decode_prologue(cfg, layer_begin, num_layers, chunk_tokens, &plan);
    if (st != KVQ_OK) return st;
    if (!cache || !seq_lens || !q || !out) return KVQ_ERR_NULL;
    // counters of this cache shape, then the call's partials, must fit
    const int64_t counters = int64_t(cfg->num_layers) * cfg->batch * cfg->num_kv_heads;
    if (counters * 4 > int64_t(kScratchCounterBytes) ||
        plan->total - plan->arrive_bytes > kScratchBytes - kScratchCounterBytes)
      return KVQ_ERR_WORKSPACE;
    uint8_t* base = nullptr;
    st = scratch_for_device(static_cast<hipStream_t>(stream), &base);
    if (st != KVQ_OK) return st;
    return decode_launch(cfg, cache, layer_begin, num_layers, seq_lens, q, out, sm_scale, *plan,
                         WsRegions{base, base + kScratchCounterBytes}, stream);
  } catch (...) {
    return KVQ_ERR_INTERNAL;
  }
}
