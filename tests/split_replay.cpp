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
hipError_t launch_decode_simple(const DecodeArgs&, int, hipStream_t) { return hipSuccess; }
hipError_t launch_decode_merge(const DecodeArgs&, int, int, hipStream_t) { return hipSuccess; }
hipError_t launch_decode_mfma(const DecodeArgs& a, int, int, hipStream_t) {
  g_mfma.push_back(a);
  return hipSuccess;
}
bool mfma_supported(int D, int g, int G) { return (D == 64 || D == 128) && G * (D / g) <= 16; }
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
                    int per_channel = 0) {
  kvq_config c{};
  c.k_per_channel = per_channel;
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
  long waves = 0;
  for (const DecodeArgs& a : g_mfma) {
    const long total = long(a.nxcum[a.n_seq]) * a.mcum[a.n_lh];
    waves += total;
    for (long b = 0; b * kMfmaWaves < total; ++b) {
      const int b8 = int(b) * kMfmaWaves;
      for (int pos = 0; pos < kMfmaWaves && b8 + pos < total; ++pos) {
        int slot, sl, u;
        unit_of(a, b8 + pos, slot, sl, u);
        const int ne = a.nx[sl] * int(a.mult[slot]), w0 = b8 + pos - u;
        const int p_lo = std::max(w0, b8) - b8, p_hi = std::min(w0 + ne, b8 + kMfmaWaves) - b8;
        const int px = int(b) - w0 / kMfmaWaves;
        const int pn = (w0 + ne - 1) / kMfmaWaves - w0 / kMfmaWaves + 1;
        if (px < 0 || px >= pn || pn > a.max_chunks) {
          printf("%s: piece %d of %d, %d partial slots\n", name, px, pn, a.max_chunks);
          ++bad;
        }
        const int lh = a.lh_glob[slot], l = lh / Hkv, h = lh % Hkv, s = a.seq_off + sl;
        const int len = a.cap[sl];  // seq_lens = capacity
        const long key = (long(l) * B + s) * Hkv + h;
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
        for (int seg = 0; seg < 3; ++seg) {
          const bool vis = seg == 2;
          int x0, x1;
          if (vis && a.chunk == 0) {
            if (pos != p_lo) continue;  // the piece's claimed range, once per piece
            x0 = std::max(ga, vbeg);
            x1 = std::min(gb, vend);
          } else {
            x0 = seg == 0 ? wa : vis ? std::max(wa, vbeg) : std::max(wa, vend);
            x1 = seg == 0 ? std::min(wb, vbeg) : vis ? std::min(wb, vend) : wb;
          }
          // per-channel K: a visual segment's 32-token steps start on the
          // block grid, so none straddles two blocks of g tokens
          if (vis && a.k_per_channel && x0 < x1 && (x0 - vbeg) % 32) {
            if (bad < 8) printf("%s: visual segment at %d off the step grid\n", name, x0 - vbeg);
            ++bad;
          }
          for (int tk = x0; tk < x1; ++tk) cv[tk]++;
        }
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
  if (!g_mfma.empty() && long(cov.size()) != long(L) * B * Hkv) {
    printf("%s: %zu entries covered of %d\n", name, cov.size(), L * B * Hkv);
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
  printf(bad ? "FAIL\n" : "ok\n");
  return bad != 0;
}
