// Host check of packed_grid (attn_launch.h), the grid size of packed launches:
// for every valid boundary table (rising, from 0 to T, lengths <= max_seqlen)
// it must cover every real block -- heads * sum_b ceil(len_b / BS) workgroups --
// never exceed the plain (sequence, head, block) grid, and equal that grid
// for unpacked calls and for batches beyond kMaxPackedSeqs sequences.  Tables
// come from a fixed-seed generator; prints one line and exits 0 on success.
#include "attn_launch.h"

#include <algorithm>
#include <cstdint>
#include <cstdio>
#include <vector>

namespace {

uint64_t state = 0x9E3779B97F4A7C15ull;
uint64_t next() {   // SplitMix64
  uint64_t z = (state += 0x9E3779B97F4A7C15ull);
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

}  // namespace

int main() {
  const int block_sizes[] = {64, 128, 256};
  int failures = 0, cases = 0;
  for (int trial = 0; trial < 4000; ++trial) {
    const int B = 1 + (int)(next() % 700);
    const int longest_cap = 1 + (int)(next() % 5000);
    std::vector<int> cu(B + 1, 0);
    int Nmax = 0;
    for (int b = 0; b < B; ++b) {
      const int len = (next() % 7 == 0) ? 0 : (int)(next() % (uint64_t)(longest_cap + 1));
      cu[b + 1] = cu[b] + len;
      Nmax = std::max(Nmax, len);
    }
    const int T = cu[B];
    if (T == 0 || Nmax == 0) continue;   // empty batches never launch
    attn::Packing p;
    p.cu = cu.data();
    p.T = T;
    for (int BS : block_sizes) {
      const int heads = 1 + (int)(next() % 64);
      long long real = 0;
      for (int b = 0; b < B; ++b) real += (cu[b + 1] - cu[b] + BS - 1) / BS;
      real *= heads;
      const long long plain = (long long)B * heads * ((Nmax + BS - 1) / BS);
      const long long g = attn::packed_grid(p, B, heads, BS, plain);
      ++cases;
      bool ok = g >= real && g <= plain;
      if (B > attn::kMaxPackedSeqs) ok = ok && g == plain;
      attn::Packing none;
      ok = ok && attn::packed_grid(none, B, heads, BS, plain) == plain;
      if (!ok) {
        if (++failures <= 5)
          std::printf("FAIL B=%d T=%d Nmax=%d BS=%d heads=%d: grid %lld, real %lld, plain %lld\n", B, T,
                      Nmax, BS, heads, g, real, plain);
      }
    }
  }
  std::printf("%s: %d cases, %d failures\n", failures ? "FAIL" : "ok", cases, failures);
  return failures ? 1 : 0;
}
