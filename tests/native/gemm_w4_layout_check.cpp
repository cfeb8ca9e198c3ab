// CPU check of the four-wave GEMM's LDS layouts (linear_layers_amd/csrc/
// gemm_w4_layout.hpp), over every wave, lane, fragment block and substep:
//   * the DMA placement (lane -> LDS slot, slot -> operand chunk through the
//     swizzle) puts every chunk of the tile in LDS exactly once;
//   * each fragment read (ds_read_b128, or two ds_read_b64_tr_b16 whose
//     4x4 transpose across 16 lanes is modelled here) hands every lane the 8
//     operand values the 16x16x32 MFMA expects: row (column) w0 + 16 f +
//     (lane & 15), K values 32 s + 8 (lane >> 4) .. + 7;
//   * the offsets the kernel forms (one base register per fragment group plus
//     an immediate) equal the direct formulas;
//   * every access stays inside the tile;
//   * no LDS bank conflicts under the bank model stated in the layout header
//     (64 banks of 4 bytes; ds_read_b128 serves lanes 8..23, then 0..7 with
//     24..31, then the same groups of lanes 32..63; ds_read_b64_tr_b16 serves
//     lanes 0..31, then 32..63), fitted to the conflict counts rocprofv3
//     measured for probe patterns on the GPU.
// Exit status 0 and "OK" on success; the first failure is printed.
#include <cstdio>
#include <cstdlib>
#include <map>
#include <set>
#include <utility>
#include <vector>

#include "../../linear_layers_amd/csrc/gemm_w4_layout.hpp"

using namespace tpmlp::w4;

static int fails = 0;
#define CHECK(cond, ...)                                   \
  do {                                                     \
    if (!(cond)) {                                         \
      if (fails++ < 10) {                                  \
        std::printf("FAIL %s:%d: ", __FILE__, __LINE__);   \
        std::printf(__VA_ARGS__);                          \
        std::printf("\n");                                 \
      }                                                    \
    }                                                      \
  } while (0)

typedef std::pair<int, int> Elem;  // (row or K-row, K or column) of the operand

// rows: tile rows (M or N); kmaj: K-contiguous; nw: waves staging it (K step 64).
static void check_tile(int rows, bool kmaj, int nw, int wave_rows) {
  const int bkt = 64, cpr = 8, qpr = rows / 8;
  const int bytes = rows * bkt * 2, slots = rows * cpr;
  const int instr = slots / (64 * nw);
  CHECK(slots % (64 * nw) == 0, "slots");
  // LDS byte -> operand element (kmaj: (row, k); else (k, col))
  std::vector<Elem> lds(bytes / 2, Elem(-1, -1));
  std::set<Elem> seen;
  for (int w = 0; w < nw; ++w)
    for (int j = 0; j < instr; ++j)
      for (int l = 0; l < 64; ++l) {
        const int s = (w * instr + j) * 64 + l;   // DMA: lane l of load j writes LDS bytes M0 + 16 l
        const int base = (w * instr + j) * 1024 + 16 * l;
        CHECK(base == s * 16, "slot order");
        for (int e = 0; e < 8; ++e) {
          Elem el;
          if (kmaj) {
            const int row = s / cpr, c = pos_k(row, s % cpr);
            el = Elem(row, c * 8 + e);
          } else {
            const int k = s / qpr, q = pos_t(qpr, k, s % qpr);
            CHECK(q >= 0 && q < qpr, "pos_t leaves the row");
            el = Elem(k, q * 8 + e);
          }
          CHECK(lds[base / 2 + e].first < 0, "LDS byte written twice");
          lds[base / 2 + e] = el;
          CHECK(seen.insert(el).second, "chunk loaded twice");
        }
      }
  CHECK((int)seen.size() == rows * bkt, "tile not covered");
  const int nsub = bkt / 32;
  for (int w0 = 0; w0 < rows; w0 += wave_rows) {
    const int nf = wave_rows / 16;
    for (int f = 0; f < nf; ++f)
      for (int s = 0; s < nsub; ++s) {
        if (kmaj) {
          // one ds_read_b128 per lane
          std::vector<int> addr(64);
          for (int l = 0; l < 64; ++l) {
            const uint32_t a = frag_k(w0, l, f, s);
            CHECK(a == frag_k_fast(w0, l, f, s), "frag_k_fast w0 %d l %d f %d s %d", w0, l, f, s);
            CHECK(a + 16 <= (uint32_t)bytes && a % 16 == 0, "frag_k bounds");
            addr[l] = (int)a;
            for (int e = 0; e < 8; ++e) {
              const Elem got = lds[a / 2 + e];
              const Elem want(w0 + 16 * f + (l & 15), 32 * s + 8 * (l >> 4) + e);
              CHECK(got == want, "K-major fragment rows %d f %d s %d lane %d e %d: (%d,%d) want (%d,%d)", rows, f, s,
                    l, e, got.first, got.second, want.first, want.second);
            }
          }
          for (int h = 0; h < 2; ++h)       // lanes 8..23, then 0..7 with 24..31 (+32 h)
            for (int t = 0; t < 2; ++t) {
              std::map<int, int> bank;
              for (int u = 0; u < 16; ++u) {
                const int l = 32 * h + (t == 0 ? 8 + u : (u < 8 ? u : 16 + u));
                for (int b = 0; b < 4; ++b) bank[((addr[l] / 4) + b) % 64]++;
              }
              for (auto& kv : bank) CHECK(kv.second == 1, "b128 bank conflict rows %d f %d s %d", rows, f, s);
            }
        } else {
          for (int r = 0; r < 2; ++r) {
            std::vector<int> addr(64);
            for (int l = 0; l < 64; ++l) {
              const uint32_t a = frag_t(qpr, w0, l, f, s, r);
              CHECK(a == frag_t_fast(qpr, w0, l, f, s, r), "frag_t_fast");
              CHECK(a + 8 <= (uint32_t)bytes && a % 8 == 0, "frag_t bounds");
              addr[l] = (int)a;
            }
            // transposing read: within each 16-lane group, lane j receives
            // element j % 4 of lane 4 e + j / 4's 4 values, for e = 0..3
            for (int l = 0; l < 64; ++l) {
              const int g = l >> 4, j = l & 15;
              for (int e = 0; e < 4; ++e) {
                const int src = 16 * g + 4 * e + j / 4;
                const Elem got = lds[addr[src] / 2 + (j % 4)];
                const Elem want(32 * s + 8 * g + 4 * r + e, w0 + 16 * f + j);
                CHECK(got == want, "MN fragment rows %d f %d s %d r %d lane %d e %d: (%d,%d) want (%d,%d)", rows, f,
                      s, r, l, e, got.first, got.second, want.first, want.second);
              }
            }
            for (int h = 0; h < 2; ++h) {   // 32 lanes per cycle
              std::map<int, int> bank;
              for (int l = 32 * h; l < 32 * h + 32; ++l)
                for (int b = 0; b < 2; ++b) bank[((addr[l] / 4) + b) % 64]++;
              for (auto& kv : bank) CHECK(kv.second == 1, "tr bank conflict rows %d f %d s %d r %d", rows, f, s, r);
            }
          }
        }
      }
  }
}

int main() {
  for (bool kmaj : {true, false}) {
    check_tile(256, kmaj, 4, 128);
    check_tile(128, kmaj, 4, 64);
    check_tile(192, kmaj, 4, 96);
  }
  if (fails) {
    std::printf("%d failures\n", fails);
    return 1;
  }
  std::printf("OK\n");
  return 0;
}
