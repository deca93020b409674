// Host-side check of the LDS tile layout and MFMA operand addressing in
// attn_layout.h: simulates the direct loads that fill a tile, then every lane
// of every row-fragment and transposed-fragment read, and checks (1) each lane
// gets exactly the elements the MFMA operand needs and (2) no access pattern
// has LDS bank conflicts.  The transposed read is modelled from the measured
// behaviour of ds_read_b64_tr_b16: in each group of 16 lanes, slot j of lane i
// is element (i & 3) of the 4 values addressed by lane 4j + (i >> 2); and of
// ds_read_b64_tr_b8 for the 8-bit tiles: byte j of lane i is byte (i & 7) of
// the 8 bytes addressed by lane 2j + (i >> 3).
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

// 8-bit tiles (d = 128 bytes per row): rows x 128 bytes.
void check_f8(int rows) {
  std::vector<int> lds(rows * 128, -1);   // one entry per byte; value = global row*128 + col
  for (int b = 0; b < rows * 128; b += 16) {
    int r, c;
    direct_src<64>(b, r, c);
    for (int e = 0; e < 16; ++e) lds[b + e] = r * 128 + c * 16 + e;
  }
  for (int r = 0; r < rows; ++r)
    for (int col = 0; col < 128; ++col)
      EXPECT(lds[f8_off(r, col)] == r * 128 + col, "f8_off(%d,%d)", r, col);
  // row fragments: lane l gets row row0 + l%32, bytes 64m + 32(l/32) + 16e .. +15
  for (int row0 = 0; row0 + 32 <= rows; row0 += 32)
    for (int m = 0; m < 2; ++m)
      for (int e = 0; e < 2; ++e) {
        for (int lane = 0; lane < 64; ++lane) {
          const int off = f8_row_frag_off(lane, row0, m, e);
          EXPECT(off % 16 == 0, "f8 row frag misaligned");
          for (int k = 0; k < 16; ++k)
            EXPECT(lds[off + k] == (row0 + lane % 32) * 128 + 64 * m + 32 * (lane / 32) + 16 * e + k,
                   "f8 row frag lane %d m %d e %d byte %d", lane, m, e, k);
        }
        for (int g = 0; g < 4; ++g) {
          std::set<int> banks;
          for (int lane = 16 * g; lane < 16 * g + 16; ++lane)
            for (int w = 0; w < 4; ++w) banks.insert((f8_row_frag_off(lane, row0, m, e) / 4 + w) % 64);
          EXPECT(banks.size() == 64, "f8 row frag bank conflict row0 %d m %d e %d group %d", row0, m, e, g);
        }
      }
  // transposed fragments: lane l, byte 8t + j = V[k0 + key(hi, 8t + j)][32db + l%32]
  for (int k0 = 0; k0 + 64 <= rows; k0 += 64)
    for (int db = 0; db < 4; ++db)
      for (int t = 0; t < 4; ++t) {
        int addr[64];
        for (int lane = 0; lane < 64; ++lane) {
          addr[lane] = f8_tr_off(lane, k0, db, t);
          EXPECT(addr[lane] % 8 == 0, "f8 tr misaligned");
        }
        for (int lane = 0; lane < 64; ++lane) {
          const int g = lane >> 4, i = lane & 15, hi = lane >> 5;
          for (int j = 0; j < 8; ++j) {
            const int src = addr[16 * g + 2 * j + (i >> 3)] + (i & 7);
            const int want = (k0 + f8_pair_key(hi, 8 * t + j)) * 128 + 32 * db + lane % 32;
            EXPECT(lds[src] == want, "f8 tr k0 %d db %d t %d lane %d byte %d", k0, db, t, lane, j);
          }
        }
        for (int half = 0; half < 2; ++half) {   // served 32 lanes (256 bytes) at a time
          std::set<int> banks;
          for (int lane = 32 * half; lane < 32 * half + 32; ++lane)
            for (int w = 0; w < 2; ++w) banks.insert((addr[lane] / 4 + w) % 64);
          EXPECT(banks.size() == 64, "f8 tr bank conflict k0 %d db %d t %d half %d (%zu banks)", k0, db, t,
                 half, banks.size());
        }
      }
  // the pair's keys: each lane-half sees every key of 64 exactly... once per
  // pair of lane-halves: hi = 0 and hi = 1 together cover keys 0..63
  std::set<int> keys;
  for (int hi = 0; hi < 2; ++hi)
    for (int b = 0; b < 32; ++b) keys.insert(f8_pair_key(hi, b));
  EXPECT(keys.size() == 64 && *keys.begin() == 0 && *keys.rbegin() == 63, "f8 pair keys");
}

int main() {
  check_f8(128);
  check<128>(64);
  check<128>(128);
  check<64>(64);
  check<64>(128);
  std::printf("%s (%d failures)\n", failures ? "FAIL" : "OK", failures);
  return failures ? 1 : 0;
}
