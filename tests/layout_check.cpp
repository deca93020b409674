// Host-side check of the LDS tile layout and MFMA operand addressing in
// attn_layout.h: simulates the direct loads that fill a tile, then every lane
// of every row-fragment and transposed-fragment read, and checks (1) each lane
// gets exactly the elements the MFMA operand needs and (2) no access pattern
// has LDS bank conflicts.  The transposed read is modelled from the measured
// behaviour of ds_read_b64_tr_b16: in each group of 16 lanes, slot j of lane i
// is element (i & 3) of the 4 values addressed by lane 4j + (i >> 2).
#include <cstdio>
#include <set>
#include <vector>

#include "attn_layout.h"

using namespace attn::layout;

static int failures = 0;
#define EXPECT(c, ...) do { if (!(c)) { if (failures++ < 20) { std::printf(__VA_ARGS__); std::printf("\n"); } } } while (0)

template <int D>
void check(int rows) {
  std::vector<int> lds(rows * D, -1);  // one entry per bf16 slot; value = global row*D + col
  for (int b = 0; b < rows * 2 * D; b += 16) {
    int r, c;
    direct_src<D>(b, r, c);
    EXPECT(r >= 0 && r < rows && c >= 0 && c < D / 8, "D%d direct_src(%d) -> r %d c %d", D, b, r, c);
    for (int e = 0; e < 8; ++e) lds[b / 2 + e] = r * D + c * 8 + e;
  }
  std::set<int> seen(lds.begin(), lds.end());
  EXPECT((int)seen.size() == rows * D && !seen.count(-1), "D%d tile not a permutation", D);
  for (int r = 0; r < rows; ++r)
    for (int col = 0; col < D; ++col)
      EXPECT(lds[elem_off<D>(r, col) / 2] == r * D + col, "D%d elem_off(%d,%d)", D, r, col);

  // row fragments and their banks (ds_read_b128 is served 16 lanes at a time)
  for (int row0 = 0; row0 + 32 <= rows; row0 += 32)
    for (int slab = 0; slab < D / 16; ++slab) {
      for (int lane = 0; lane < 64; ++lane) {
        const int off = row_frag_off<D>(lane, row0, slab);
        EXPECT(off % 16 == 0, "D%d row frag misaligned", D);
        for (int e = 0; e < 8; ++e)
          EXPECT(lds[off / 2 + e] == (row0 + lane % 32) * D + 16 * slab + 8 * (lane / 32) + e,
                 "D%d row frag row0 %d slab %d lane %d e %d", D, row0, slab, lane, e);
      }
      for (int g = 0; g < 4; ++g) {
        std::set<int> banks;
        for (int lane = 16 * g; lane < 16 * g + 16; ++lane)
          for (int w = 0; w < 4; ++w) banks.insert((row_frag_off<D>(lane, row0, slab) / 4 + w) % 64);
        EXPECT(banks.size() == 64, "D%d row frag bank conflict row0 %d slab %d group %d (%zu banks)", D,
               row0, slab, g, banks.size());
      }
    }

  // transposed fragments and their banks (ds_read_b64 is served 32 lanes at a time)
  for (int row0 = 0; row0 + 16 <= rows; row0 += 16)
    for (int col0 = 0; col0 < D; col0 += 32)
      for (int half = 0; half < 2; ++half) {
        int src[64][4];
        for (int lane = 0; lane < 64; ++lane) {
          const int off = tr_frag_off<D>(lane, row0, col0, half);
          EXPECT(off % 8 == 0, "D%d tr address misaligned", D);
          for (int k = 0; k < 4; ++k) src[lane][k] = lds[off / 2 + k];
        }
        for (int lane = 0; lane < 64; ++lane) {
          const int i = lane & 15, base = lane & ~15;
          for (int j = 0; j < 4; ++j) {
            const int got = src[base + 4 * j + (i >> 2)][i & 3];
            const int want = (row0 + 4 * (lane >> 5) + 8 * half + j) * D + col0 + (lane & 31);
            EXPECT(got == want, "D%d tr row0 %d col0 %d half %d lane %d slot %d: got %d want %d", D, row0,
                   col0, half, lane, j, got, want);
          }
        }
        for (int h = 0; h < 2; ++h) {
          std::set<int> banks;
          for (int lane = 32 * h; lane < 32 * h + 32; ++lane)
            for (int w = 0; w < 2; ++w) banks.insert((tr_frag_off<D>(lane, row0, col0, half) / 4 + w) % 64);
          EXPECT(banks.size() == 64, "D%d tr bank conflict row0 %d col0 %d half %d (%zu banks)", D, row0,
                 col0, half, banks.size());
        }
      }
}

int main() {
  check<128>(64);
  check<128>(128);
  check<64>(64);
  check<64>(128);
  std::printf("%s (%d failures)\n", failures ? "FAIL" : "OK", failures);
  return failures ? 1 : 0;
}
