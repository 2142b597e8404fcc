// Host replay of the matrix-core decode split.  Compiles the library's host
// side (planning and argument packing) with the kernel launchers replaced by
// recorders, then walks every wave of every recorded launch the way the
// kernel assigns work: unit -> (slot, sequence, index), the wave's static
// token range, and its piece's claimed visual range.  Checks that every
// token of every (layer, seq, head) is processed exactly once, that partial
// indices stay below the workspace's partial count, and that an entry's
// pieces are numbered 0 .. pieces - 1.  Prints one line per case and "ok".
#include "../quantized_decode_attention_quantize_amd/csrc/kvq_api.hip"

#include <cstdio>
#include <map>
#include <set>

namespace kvq {
static std::vector<DecodeArgs> g_mfma;
hipError_t launch_quantize(const QuantizeArgs&, int, int, hipStream_t) { return hipSuccess; }
hipError_t launch_quantize_kblocks(const QuantizeArgs&, int, int, int, hipStream_t) {
  return hipSuccess;
}
hipError_t launch_decode_mfma(const DecodeArgs& a, int, int, hipStream_t) {
  g_mfma.push_back(a);
  return hipSuccess;
}
bool mfma_supported(int D, int g, int G) { return (D == 64 || D == 128) && G * (D / g) <= 16; }
int mfma_subgroups(int D, int g, int G) {
  if (!(D == 64 || D == 128) || g < 32 || D % g) return 0;
  return (G * (D / g) + 15) / 16;
}
}  // namespace kvq
using namespace kvq;

// unit b -> slot, sequence index, index within the entry (linear search: the
// plain definition of the layout, independent of the kernel's ballots)
static void unit_of(const DecodeArgs& a, int b, int& slot, int& sl, int& x) {
  const int per = a.nxcum[a.n_seq];
  slot = 0;
  while (slot + 1 < a.n_lh && per * int(a.mcum[slot + 1]) <= b) ++slot;
  const int r = b - per * int(a.mcum[slot]), m = a.mult[slot];
  sl = 0;
  while (sl + 1 < a.n_seq && m * a.nxcum[sl + 1] <= r) ++sl;
  x = r - m * a.nxcum[sl];
}

static int run_case(const char* name, int L, int B, int Hq, int Hkv, int D, int g,
                    std::vector<int> cap, std::vector<int> vb, std::vector<int> ve,
                    std::vector<uint8_t> kb, std::vector<uint8_t> vbits, int chunk,
                    int per_channel = 0,
                    const std::vector<std::vector<std::pair<int, int>>>& ranges = {}) {
  kvq_config c{};
  c.k_per_channel = per_channel;
  std::vector<int32_t> r_off(1, 0), r_b, r_e;
  for (const auto& seq : ranges) {
    for (const auto& r : seq) { r_b.push_back(r.first); r_e.push_back(r.second); }
    r_off.push_back(int32_t(r_b.size()));
  }
  r_b.push_back(0); r_e.push_back(0);
  if (!ranges.empty()) {
    c.bf16_range_offsets = r_off.data(); c.bf16_range_begin = r_b.data();
    c.bf16_range_end = r_e.data();
  }
  // rows of every position by counting: coded positions (in the coded span
  // and no range) take VIS rows in order, the rest TXT rows, sequence after
  // sequence; -1 marks a position of the other plane
  std::vector<std::pair<std::vector<long>, std::vector<long>>> row_of(B);
  {
    long vr = 0, tr = 0;
    for (int s = 0; s < B; ++s) {
      int cend = ve[s];
      if (per_channel) cend = vb[s] + (ve[s] - vb[s]) / g * g;
      row_of[s].first.assign(cap[s], -1);
      row_of[s].second.assign(cap[s], -1);
      for (int t = 0; t < cap[s]; ++t) {
        bool coded = t >= vb[s] && t < cend;
        if (!ranges.empty())
          for (const auto& r : ranges[s]) coded = coded && !(t >= r.first && t < r.second);
        if (coded) row_of[s].first[t] = vr++;
        else row_of[s].second[t] = tr++;
      }
    }
  }
  c.num_layers = L; c.batch = B; c.num_q_heads = Hq; c.num_kv_heads = Hkv;
  c.head_dim = D; c.group_size = g;
  c.capacity = cap.data(); c.vis_begin = vb.data(); c.vis_end = ve.data();
  c.k_bits = kb.data(); c.v_bits = vbits.data();
  size_t need = 0;
  if (kvq_decode_attention(&c, nullptr, 0, L, nullptr, nullptr, nullptr, 0.1f, chunk, nullptr,
                           &need, nullptr) != KVQ_OK) {
    printf("%s: size query failed\n", name);
    return 1;
  }
  g_mfma.clear();
  size_t n = need;
  // pointers are only packed into the arguments, never dereferenced here
  if (kvq_decode_attention(&c, (void*)0x100000, 0, L, (const int32_t*)0x1000, (void*)0x2000,
                           (void*)0x3000, 0.1f, chunk, (void*)0x100000, &n, nullptr) != KVQ_OK) {
    printf("%s: call failed\n", name);
    return 1;
  }
  int bad = 0;
  std::map<long, std::vector<int>> cov;
  std::map<long, std::set<int>> seen_px;
  std::map<long, int> npieces;
  std::map<long, std::set<long>> heads_seen;  // per entry: its subgroups (first head, count)
  // per entry: waves that would store the appended row (kvq_decode_attention_append),
  // and whether the last position is stored as a text row
  std::map<long, int> app_owners;
  std::map<long, bool> app_text;
  long waves = 0;
  for (const DecodeArgs& a : g_mfma) {
    const long total = long(a.nxcum[a.n_seq]) * a.mcum[a.n_lh];
    waves += total;
    for (long b = 0; b * kMfmaWaves < total; ++b) {
      const int b8 = int(b) * kMfmaWaves;
      for (int pos = 0; pos < kMfmaWaves && b8 + pos < total; ++pos) {
        int slot, sl, u;
        unit_of(a, b8 + pos, slot, sl, u);
        const int ne = (a.nxcum[sl + 1] - a.nxcum[sl]) * int(a.mult[slot]), w0 = b8 + pos - u;
        const int p_lo = std::max(w0, b8) - b8, p_hi = std::min(w0 + ne, b8 + kMfmaWaves) - b8;
        const int px = int(b) - w0 / kMfmaWaves;
        const int pn = (w0 + ne - 1) / kMfmaWaves - w0 / kMfmaWaves + 1;
        if (px < 0 || px >= pn || pn > a.max_chunks) {
          printf("%s: piece %d of %d, %d partial slots\n", name, px, pn, a.max_chunks);
          ++bad;
        }
        const int lh = a.lh_glob[slot], l = lh / Hkv, h = lh % Hkv, s = a.seq_off + sl;
        const int len = a.cap[sl];  // seq_lens = capacity
        // query-head subgroup of this launch: q points at its first head
        const long g0 = long(reinterpret_cast<const char*>(a.q) - reinterpret_cast<const char*>(0x2000)) /
                        (2 * D);
        const long key = ((g0 * L + l) * B + s) * Hkv + h;
        if (a.g_stride != Hq / Hkv || (g0 % a.G != 0 && g0 + a.G != Hq / Hkv)) {
          if (bad < 8) printf("%s: subgroup at head %ld of %d heads, stride %d\n", name, g0, a.G,
                              a.g_stride);
          ++bad;
        }
        heads_seen[(long(l) * B + s) * Hkv + h].insert(g0 * 100 + a.G);
        std::vector<int>& cv = cov[key];
        if (cv.empty()) cv.assign(len, 0);
        seen_px[key].insert(px);
        npieces[key] = pn;
        const int vbeg = a.vb[sl], vend = a.ve[sl];  // vend: end of the coded span
        const int phase = a.k_per_channel ? (32 - vbeg % 32) % 32 : 0;
        int wa, wb, ga, gb, gt;
        if (a.chunk > 0)
          wave_range(u / kMfmaWaves, u % kMfmaWaves, ne / kMfmaWaves, len, a.chunk, kMfmaWaves,
                     wa, wb, phase);
        else
          wave_range(u, 0, ne, len, 0, 1, wa, wb, phase);
        wave_range(p_lo + b8 - w0, 0, ne, len, 0, 1, ga, gt, phase);
        wave_range(p_hi - 1 + b8 - w0, 0, ne, len, 0, 1, gt, gb, phase);
        // the kernel's segments: text prefix, text suffix, then the coded
        // pieces and bf16 ranges of the span in turn
        const int r_lo = a.rng_first[sl], nr = a.rng_first[sl + 1] - r_lo;
        int range_total = 0;
        for (int k = 0; k < nr; ++k) range_total += a.rng_e[r_lo + k] - a.rng_b[r_lo + k];
        const bool dyn = a.chunk == 0 && nr == 0;
        int skipped = 0;
        for (int seg = 0; seg < 3 + 2 * nr; ++seg) {
          const bool vis = seg >= 2 && ((seg - 2) & 1) == 0;
          int f0, f1;
          long frow;
          if (seg == 0) {
            f0 = 0; f1 = vbeg; frow = a.trow0[sl];
          } else if (seg == 1) {
            f0 = vend; f1 = a.cap[sl]; frow = a.trow0[sl] + vbeg + range_total;
          } else {
            const int k = (seg - 2) >> 1;
            if (vis) {
              f0 = k == 0 ? vbeg : a.rng_e[r_lo + k - 1];
              f1 = k < nr ? a.rng_b[r_lo + k] : vend;
              frow = a.vrow0[sl] + (f0 - vbeg) - skipped;
            } else {
              f0 = a.rng_b[r_lo + k]; f1 = a.rng_e[r_lo + k];
              frow = a.trow0[sl] + vbeg + skipped;
              skipped += f1 - f0;
            }
          }
          int x0, x1;
          if (vis && dyn) {
            if (pos != p_lo) continue;  // the piece's claimed range, once per piece
            x0 = std::max(ga, f0);
            x1 = std::min(gb, f1);
          } else if (dyn) {  // text rows: all on the entry's text unit
            const bool mine = u == text_unit(w0, ne, kMfmaWaves);
            x0 = mine ? std::min(f0, len) : 0;
            x1 = mine ? std::min(f1, len) : 0;
          } else {
            x0 = std::max(wa, f0);
            x1 = std::min(wb, f1);
          }
          // per-channel K: a visual segment's 32-token steps start on the
          // block grid, so none straddles two blocks of g tokens
          if (vis && a.k_per_channel && x0 < x1 && (x0 - vbeg) % 32) {
            if (bad < 8) printf("%s: visual segment at %d off the step grid\n", name, x0 - vbeg);
            ++bad;
          }
          // every row against the layout's plain definition (by counting)
          for (int tk = x0; tk < x1; ++tk) {
            const long want = vis ? row_of[s].first[tk] : row_of[s].second[tk];
            if (want < 0 || frow + (tk - f0) != want) {
              if (bad < 8)
                printf("%s: seq %d token %d (%s) row %ld, layout row %ld\n", name, s, tk,
                       vis ? "coded" : "bf16", frow + (tk - f0), want);
              ++bad;
            }
          }
          for (int tk = x0; tk < x1; ++tk) cv[tk]++;
          // the append's owner: the kernel's test on the same segment range
          if (!vis && x0 <= len - 1 && len - 1 < x1) app_owners[key]++;
        }
        app_text[key] = row_of[s].second[len - 1] >= 0;
      }
    }
  }
  for (auto& kv : cov) {
    for (size_t tk = 0; tk < kv.second.size(); ++tk)
      if (kv.second[tk] != 1) {
        if (bad < 8) printf("%s: entry %ld token %zu processed %d times\n", name, kv.first, tk, kv.second[tk]);
        ++bad;
      }
    if (int(seen_px[kv.first].size()) != npieces[kv.first]) {
      printf("%s: entry %ld has %zu of %d pieces\n", name, kv.first, seen_px[kv.first].size(),
             npieces[kv.first]);
      ++bad;
    }
  }
  // the appended position (seq_lens - 1): exactly one wave of each entry and
  // subgroup stores it when it is a text row, none otherwise
  for (auto& kv : app_text) {
    const int want = kv.second ? 1 : 0, got = app_owners.count(kv.first) ? app_owners[kv.first] : 0;
    if (got != want) {
      if (bad < 8) printf("%s: entry %ld appended row owned by %d waves, want %d\n", name, kv.first,
                          got, want);
      ++bad;
    }
  }
  // every query head of every entry in exactly one subgroup
  for (auto& kv : heads_seen) {
    int covered = 0;
    for (long x : kv.second) covered += int(x % 100);
    if (covered != Hq / Hkv) {
      if (bad < 8) printf("%s: entry %ld has %d of %d query heads\n", name, kv.first, covered, Hq / Hkv);
      ++bad;
    }
  }
  const long nsub = heads_seen.empty() ? 1 : long(heads_seen.begin()->second.size());
  if (!g_mfma.empty() && long(cov.size()) != long(L) * B * Hkv * nsub) {
    printf("%s: %zu entries covered of %ld\n", name, cov.size(), long(L) * B * Hkv * nsub);
    ++bad;
  }
  printf("%-16s chunk %5d launches %zu waves %ld workspace %zu %s\n", name, chunk, g_mfma.size(),
         waves, need, bad ? "FAIL" : "ok");
  return bad;
}

int main() {
  int bad = 0;
  // 28 layers x 4 KV heads, one 6288-row sequence; 0, 14 or all heads bf16
  for (int prot : {0, 14, 112}) {
    std::vector<uint8_t> kb(112, 4), vb(112, 2);
    for (int i = 0; i < prot; ++i) kb[(i * 37) % 112] = vb[(i * 37) % 112] = 16;
    for (int ch : {0, 1024}) bad += run_case("28x4 6288", 28, 1, 28, 4, 128, 64, {6288}, {14}, {6287}, kb, vb, ch);
  }
  bad += run_case("4 x 32769", 1, 4, 32, 8, 128, 64, {32769, 32769, 32769, 32769},
                  {14, 14, 14, 14}, {32768, 32768, 32768, 32768}, std::vector<uint8_t>(8, 4),
                  std::vector<uint8_t>(8, 2), 0);
  {  // 70 ragged sequences (two launches of the sequence table)
    std::vector<int> cap, vbg, ve;
    uint32_t x = 12345;
    for (int s = 0; s < 70; ++s) {
      x = x * 1664525u + 1013904223u;
      const int l = 1024 + int(x % 15360u);
      cap.push_back(l); vbg.push_back(14); ve.push_back(l - 1);
    }
    bad += run_case("70 ragged", 1, 70, 28, 4, 128, 64, cap, vbg, ve, std::vector<uint8_t>(4, 4),
                    std::vector<uint8_t>(4, 2), 0);
  }
  bad += run_case("mixed widths", 2, 3, 8, 2, 64, 32, {40, 1, 97}, {3, 0, 10}, {35, 1, 97},
                  {4, 16, 8, 2}, {2, 16, 8, 4}, 0);
  bad += run_case("320 pairs", 40, 1, 32, 8, 128, 64, {2000}, {5}, {1990},
                  std::vector<uint8_t>(320, 4), std::vector<uint8_t>(320, 4), 0);
  for (int len : {1, 31, 33, 200})
    bad += run_case("short", 2, 2, 8, 2, 128, 64, {len, len}, {0, 0}, {len, len}, {4, 4, 4, 16},
                    {2, 2, 2, 16}, 0);
  // per-channel K (coded spans in whole blocks, steps on the block grid)
  for (int ch : {0, 256, 1024})
    bad += run_case("pc 28x4 6288", 28, 1, 28, 4, 128, 64, {6288}, {14}, {6287},
                    std::vector<uint8_t>(112, 4), std::vector<uint8_t>(112, 2), ch, 1);
  bad += run_case("pc 4 x 32769", 1, 4, 32, 8, 128, 64, {32769, 32769, 32769, 32769},
                  {64, 7, 100, 0}, {32768, 32000, 30000, 31999}, std::vector<uint8_t>(8, 4),
                  std::vector<uint8_t>(8, 2), 0, 1);
  bad += run_case("pc mixed", 2, 3, 8, 2, 64, 32, {400, 1, 970}, {3, 0, 10}, {350, 1, 970},
                  {4, 8, 8, 2}, {2, 4, 8, 4}, 0, 1);
  // one layer (a small call: library-chosen 1024-token chunks), plain and
  // per-channel
  bad += run_case("1x4 6288", 1, 1, 28, 4, 128, 64, {6288}, {14}, {6287},
                  std::vector<uint8_t>(4, 4), std::vector<uint8_t>(4, 2), 0);
  bad += run_case("pc 1x4 6288", 1, 1, 28, 4, 128, 64, {6288}, {14}, {6287},
                  std::vector<uint8_t>(4, 4), std::vector<uint8_t>(4, 2), 0, 1);
  // more than one 16-column tile per KV head: query-head subgroups
  bad += run_case("sub 28/4 g32", 2, 2, 28, 4, 128, 32, {700, 300}, {14, 0}, {690, 300},
                  std::vector<uint8_t>(8, 4), std::vector<uint8_t>(8, 2), 0);
  bad += run_case("sub 16/1 g32", 1, 1, 16, 1, 128, 32, {6288}, {14}, {6287},
                  std::vector<uint8_t>(1, 4), std::vector<uint8_t>(1, 2), 256);
  // bf16 ranges inside the visual spans (static split for those sequences)
  using R = std::vector<std::vector<std::pair<int, int>>>;
  for (int ch : {0, 1024}) {
    std::vector<uint8_t> kb(112, 4), vb(112, 2);
    for (int i = 0; i < 14; ++i) kb[(i * 37) % 112] = vb[(i * 37) % 112] = 16;
    bad += run_case("rng 28x4 6288", 28, 1, 28, 4, 128, 64, {6288}, {14}, {6287}, kb, vb, ch, 0,
                    R{{{14, 15}, {600, 601}, {3000, 3100}, {6000, 6287}}});
  }
  {  // 36 one-token ranges in one sequence, none in the other two
    std::vector<std::pair<int, int>> many;
    for (int i = 0; i < 36; ++i) many.push_back({20 + 97 * i, 21 + 97 * i + (i % 3)});
    for (int ch : {0, 256})
      bad += run_case("rng 36", 2, 3, 32, 8, 128, 64, {4000, 3600, 129}, {10, 10, 0},
                      {3990, 3600, 129}, std::vector<uint8_t>(16, 4), std::vector<uint8_t>(16, 2),
                      ch, 0, R{{}, many, {}});
  }
  {  // 70 ragged sequences with 0-3 ranges each (several range tables)
    std::vector<int> cap, vbg, ve;
    R rng;
    uint32_t x = 777;
    for (int s = 0; s < 70; ++s) {
      x = x * 1664525u + 1013904223u;
      const int l = 512 + int(x % 8000u);
      cap.push_back(l); vbg.push_back(5); ve.push_back(l - 3);
      std::vector<std::pair<int, int>> r;
      const int k = s % 4;
      for (int i = 0; i < k; ++i) {
        const int b = 5 + (l - 8) * i / k + 1;
        r.push_back({b, std::min(b + 1 + int(x % 200u), l - 3)});
      }
      rng.push_back(r);
    }
    bad += run_case("rng 70 ragged", 1, 70, 28, 4, 128, 64, cap, vbg, ve,
                    std::vector<uint8_t>(4, 4), std::vector<uint8_t>(4, 2), 0, 0, rng);
  }
  bad += run_case("rng mixed", 2, 3, 8, 2, 64, 32, {40, 1, 97}, {3, 0, 10}, {35, 1, 97},
                  {4, 16, 8, 2}, {2, 16, 8, 4}, 0, 0, R{{{3, 4}, {30, 35}}, {}, {{10, 97}}});
  printf(bad ? "FAIL\n" : "ok\n");
  return bad != 0;
}
