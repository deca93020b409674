// attn_fwd.hip -- tiled exact attention forward for gfx950 (MI355X).
//
// Method (page "从“算力黑洞”到“效率革命”：大模型Attention的演进之路", §4, and page
// "6.1 … 長上下文擴展技術：FlashAttention、RoPE 與稀疏注意力", §2.2): Q, K and V
// are cut into blocks along the sequence; a block of query rows is held on
// chip while K/V tiles stream past it.  Each tile's scores are formed, the
// row maxima raised where the tile holds larger scores, the exponential sums
// carried forward under the new maxima, and the tile's values added with
// their weights -- all on chip, so the N x N scores never reach device memory.
// Only O and the per-row log-sum-exp are written.
//
// gfx950 mapping
//   * one workgroup = NW waves x 32 query rows of one (batch, head); each wave
//     keeps its 32 Q rows as MFMA B operands in registers for the whole loop;
//   * S^T = K Q^T is computed (keys are the MFMA rows), so the 32x32 C layout
//     gives each lane one query column: the row max and row sum are in-register
//     over 16 values plus one exchange with lane l^32;
//   * the same accumulators, rounded to bf16, are directly the B operand of
//     O^T = V^T P^T (the k-slot order inside one MFMA is free as long as A and
//     B agree), so P never goes through LDS;
//   * K and V tiles are copied global -> LDS by 16-byte direct loads (no
//     staging registers) into row-major, XOR-swizzled tiles: K is read as
//     row fragments, V^T with the transposing LDS read, both free of bank
//     conflicts; tiles are double-buffered, the next tile's loads are in
//     flight while the current one is computed, one barrier per tile;
//   * two waves per SIMD, so one wave's softmax VALU work runs under the
//     other's MFMAs;
//   * causal: key tiles past a workgroup's last row are never loaded, a wave
//     skips tiles past its own last row, and only tiles that cross the
//     diagonal (or the ragged end of the sequence) evaluate the mask;
//   * sliding window (page "6.1 … 長上下文擴展技術", §4): with LOCAL a query
//     sees keys |i - j| <= window (and j <= i under the causal mask); key
//     tiles outside the band of a workgroup are never loaded, a wave skips
//     tiles outside its rows' bands, and only tiles that cross a band edge
//     evaluate the mask;
//   * exp is 2^x with scale*log2(e) folded into one FMA; the LSE is converted
//     back to natural-log units of the scaled scores before it is stored;
//   * workgroups run heaviest causal block first, and when B*Hq is a multiple
//     of 8 the workgroup -> (head, block) map keeps each head on one XCD so its
//     K/V stay in that XCD's L2.
#include "attn_device.h"
#include "attn_launch.h"

namespace attn {
namespace {

template <int D, int BC, int NW>
struct FwdCfg {
  static constexpr int kThreads = NW * 64;
  static constexpr int kBR = NW * 32;               // query rows per workgroup
  static constexpr int kTile = BC * 2 * D;          // bytes of one K or V tile
  static constexpr int kLdsBytes = 2 * 2 * kTile;   // double-buffered K and V
  static_assert(BC % 32 == 0 && D % 32 == 0, "tile shape");
};

// Rescaling of the running output.  The reference maximum a row's
// exponentials are taken against moves when a tile's maximum exceeds it by
// more than LAG (log2 units); the multiply of the accumulator is skipped
// whenever no row of the wave moved.  LAG = 0 keeps the exact running max, so
// the largest probability of a row is exactly 1 and rounds to bf16 without
// error (this matters for peaked rows).  LAG > 0 gives the same quotient
// sum 2^(s-m) v / sum 2^(s-m) with factors bounded by 2^LAG, and skips most
// rescales, at the cost of rounding that largest term too.
template <int D, int BC, int NW, int WPE, bool CAUSAL, bool LOCAL, int LAG = 0>
__global__ __attribute__((amdgpu_flat_work_group_size(NW * 64, NW * 64),
                          amdgpu_waves_per_eu(WPE, WPE))) void attn_fwd_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
    const uint16_t* __restrict__ V, uint16_t* __restrict__ O, float* __restrict__ LSE,
    int Nmax, int BH, int Hq, int Hkv, int G, int n_qb, float scale_log2, int xcd_remap,
    int window, Packing pk) {
  using C = FwdCfg<D, BC, NW>;
  constexpr int kPrefetch = 6; // K fragments in flight ahead of their MFMA
  constexpr int DS = D / 16;   // k-slabs of the QK^T contraction
  constexpr int KB = BC / 32;  // 32-key blocks per tile
  constexpr int DB = D / 32;   // 32-wide d blocks of O^T

  extern __shared__ __attribute__((aligned(1024))) unsigned char smem[];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l32 = lane & 31;
  const int hi = lane >> 5;

  // ---- workgroup -> (batch*head, query block) ----
  int b, h, qb;
  const int w = blockIdx.x;
  if (pk.cu && BH / Hq <= kMaxPackedSeqs) {
    // packed: real blocks only, heaviest (most key tiles) first
    PackedUnits pu;
    pu.init(pk, BH / Hq, Nmax, C::kBR);
    if (!pu.unit(w, Hq, b, h, qb)) return;
  } else {
    int bh, qrank;
    if (xcd_remap) {
      const int hx = BH >> 3;
      const int i = w >> 3;
      bh = (w & 7) * hx + (i % hx);
      qrank = i / hx;
    } else {
      bh = w % BH;
      qrank = w / BH;
    }
    qb = CAUSAL ? (n_qb - 1 - qrank) : qrank;
    b = bh / Hq;
    h = bh - b * Hq;
  }
  const int hk = h / G;
  // this pair's sequence: N rows of queries and keys (packed: its own length)
  const SeqSpan sp = seq_span(pk, Nmax, b);
  const int N = sp.len;
  const int q0 = qb * C::kBR;
  if (q0 >= N) return;   // a block past a shorter packed sequence (uniform)
  const size_t q_row0 = sp.row0(pk, Nmax, b, h, Hq);
  const size_t kv_row0 = sp.row0(pk, Nmax, b, hk, Hkv);
  const uint16_t* Qp = Q + q_row0 * D;
  const uint16_t* Kp = K + kv_row0 * D;
  const uint16_t* Vp = V + kv_row0 * D;

  const int qw0 = q0 + wave * 32;  // first query row of this wave
  const int qw1 = qw0 + 31;        // last query row of this wave
  const bool wave_live = qw0 < N;

  // ---- Q^T fragments (B operand), kept in registers for the whole loop ----
  u32x4 qf[DS];
  {
    const int row = qw0 + l32;
#pragma unroll
    for (int s = 0; s < DS; ++s)
      qf[s] = row < N ? *(const u32x4*)(Qp + (size_t)row * D + s * 16 + 8 * hi) : zero4();
  }

  // keys this workgroup's rows can see: [kv_begin, kv_end)
  const int kv_begin = LOCAL ? max(0, q0 - window) : 0;
  const int kv_end = CAUSAL ? min(N, q0 + C::kBR) : (LOCAL ? min(N, q0 + C::kBR + window) : N);
  const int j_first = kv_begin / BC;
  const int n_tiles = (kv_end + BC - 1) / BC;

  TileLoader<D, BC, NW> ldr;
  ldr.init(wave, lane);
  auto issue_tile = [&](int j, int buf) {
    unsigned char* kt = smem + buf * 2 * C::kTile;
    ldr.load(Kp, j * BC, N, kt, wave);
    ldr.load(Vp, j * BC, N, kt + C::kTile, wave);
  };

  // ---- running statistics and the O^T accumulator ----
  f32x16 acc[DB];
  float m_run = -INFINITY, l_run = 0.f;
#pragma unroll
  for (int db = 0; db < DB; ++db) acc[db] = f32x16{};

  issue_tile(j_first, j_first & 1);
  wait_all_memory();
  __syncthreads();

  for (int j = j_first; j < n_tiles; ++j) {
    const int buf = j & 1;
    const int kstart = j * BC;
    if (j + 1 < n_tiles) issue_tile(j + 1, buf ^ 1);

    // the tile meets this wave's band: some key in [qw0 - w, qw1 (+ w)]
    const bool in_band = !LOCAL || (kstart + BC - 1 >= qw0 - window && (CAUSAL || kstart <= qw1 + window));
    if (wave_live && (!CAUSAL || kstart <= qw1) && in_band) {
      const unsigned char* kt = smem + buf * 2 * C::kTile;
      const unsigned char* vt = kt + C::kTile;

      // S^T[x] = K_tile Q^T  (32 keys x 32 queries per accumulator).  The K
      // fragments go through a ring of kPrefetch registers, each read issued
      // kPrefetch MFMAs before its use, and the scheduling groups keep the
      // compiler to one read per MFMA so the LDS latency hides under them.
      f32x16 s[KB];
#pragma unroll
      for (int x = 0; x < KB; ++x) s[x] = f32x16{};
      {
        constexpr int NSI = DS * KB;   // step i: key block i % KB, slab i / KB
        u32x4 kr[kPrefetch];
#pragma unroll
        for (int i = 0; i < kPrefetch; ++i) kr[i] = row_frag<D>(kt, lane, (i % KB) * 32, i / KB);
#pragma unroll
        for (int i = 0; i < NSI; ++i) {
          const u32x4 a = kr[i % kPrefetch];
          const int n = i + kPrefetch;
          if (n < NSI) kr[i % kPrefetch] = row_frag<D>(kt, lane, (n % KB) * 32, n / KB);
          s[i % KB] = mfma_32x32x16(a, qf[i / KB], s[i % KB]);
        }
        __builtin_amdgcn_sched_group_barrier(kSchedDsRead, kPrefetch, 0);
#pragma unroll
        for (int i = 0; i < NSI - kPrefetch; ++i) {
          __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
          __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 1, 0);
        }
        __builtin_amdgcn_sched_group_barrier(kSchedMfma, kPrefetch, 0);
      }

      // mask: only tiles that cross the diagonal, a band edge or the ragged end
      const bool need_mask = (kstart + BC > N) || (CAUSAL && kstart + BC - 1 > qw0) ||
                             (LOCAL && (kstart < qw1 - window || (!CAUSAL && kstart + BC - 1 > qw0 + window)));
      // Slot i of block x holds key kb0 + c with kb0 = kstart + 32x + 4hi and
      // c = 8(i/4) + i%4, so with t = q - kb0 each test compares the constant
      // c: key >= N <=> c > N - kb0 - 1, key > q <=> c > t, key > q + w <=>
      // c > t + w, key < q - w <=> c < t - w.
      if (need_mask) {
        const int q = qw0 + l32;
#pragma unroll
        for (int x = 0; x < KB; ++x) {
          const int kb0 = kstart + x * 32 + 4 * hi;
          const int t = q - kb0;
          int lim = N - kb0 - 1;
          if (CAUSAL) lim = min(lim, t);
          if (LOCAL && !CAUSAL) lim = min(lim, t + window);
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int c = 8 * (i >> 2) + (i & 3);
            if (c > lim || (LOCAL && c < t - window)) s[x][i] = -INFINITY;
          }
        }
      }

      // online softmax: running max, rescale, exp, running sum, P -> bf16
      float mx = -INFINITY;
#pragma unroll
      for (int x = 0; x < KB; ++x)
#pragma unroll
        for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[x][i]);
      mx = pair_max(mx) * scale_log2;
      const bool move = mx > m_run + (float)LAG;
      if (__any(move)) {
        const float m_new = move ? mx : m_run;
        // 0 on a row's first visible tile.  With a window, rows of one wave can
        // reach their band in different tiles; a row still at m_run = -inf
        // that does not move keeps alpha = 1 (exp2(-inf - -inf) would be NaN).
        const float alpha = (LOCAL && !move) ? 1.f : exp2_fast(m_run - m_new);
        m_run = m_new;
        l_run *= alpha;
#pragma unroll
        for (int db = 0; db < DB; ++db) acc[db] *= alpha;
      }
      // Without a window m_run is finite from the first visited tile on (key 0
      // is visible to every row).  With one, a row can meet a tile that is all
      // outside its band before its first visible key; its m_run is still
      // -inf and its exponentials are taken against 0 instead (all are 0).
      const float m_ref = LOCAL && m_run == -INFINITY ? 0.f : m_run;
      u32x4 pf[KB][2];
      float lsum = 0.f;
#pragma unroll
      for (int x = 0; x < KB; ++x) {
        float p[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          p[i] = exp2_fast(__builtin_fmaf(s[x][i], scale_log2, -m_ref));
          lsum += p[i];
        }
        pf[x][0] = pack8(p);
        pf[x][1] = pack8(p + 8);
      }
      l_run += lsum;

      // O^T[db] += V^T P^T: slab h2 of key block x holds keys
      // x*32 + 16*h2 + {4*hi..4*hi+3, 8+4*hi..8+4*hi+3} in this lane's k slots
#pragma unroll
      for (int x = 0; x < KB; ++x)
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
          for (int db = 0; db < DB; ++db)
            acc[db] = mfma_32x32x16(tr_frag<D>(vt, lane, x * 32 + 16 * h2, db * 32), pf[x][h2], acc[db]);
    }

    wait_all_memory();
    __syncthreads();
  }

  if (!wave_live) return;
  // ---- epilogue: O = acc / l, LSE = (m + log2 l) * ln 2 ----
  const float lt = pair_sum(l_run);
  const float inv = 1.f / lt;
  const int q = qw0 + l32;
  if (q < N) {
    uint16_t* orow = O + (q_row0 + q) * D;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int d0 = db * 32 + 8 * r + 4 * hi;
        const f32x16& a = acc[db];
        *(u32x2*)(orow + d0) = u32x2{pack_bf16x2(a[4 * r + 0] * inv, a[4 * r + 1] * inv),
                                     pack_bf16x2(a[4 * r + 2] * inv, a[4 * r + 3] * inv)};
      }
    if (hi == 0) LSE[q_row0 + q] = (m_run + log2_fast(lt)) * kLn2;
  }
}

template <int D, int BC, int NW, int WPE, bool CAUSAL, bool LOCAL, int LAG = 0>
hipError_t launch_fwd_t(const FwdArgs& a, hipStream_t stream) {
  using C = FwdCfg<D, BC, NW>;
  const int n_qb = (a.N + C::kBR - 1) / C::kBR;
  const int BH = a.B * a.Hq;
  const long long grid = packed_grid(a.pack, a.B, a.Hq, C::kBR, (long long)BH * n_qb);
  if (grid > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  if (grid == 0) return hipSuccess;
  auto kern = attn_fwd_kernel<D, BC, NW, WPE, CAUSAL, LOCAL, LAG>;
  // more than 64 KB of dynamic LDS has to be allowed per kernel instance and device
  static std::atomic<uint64_t> lds_set{0};
  const hipError_t attr = allow_lds_on_device((const void*)kern, C::kLdsBytes, lds_set);
  if (attr != hipSuccess) return attr;
  const int remap = xcd_remap(BH, a.pack);
  hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(C::kThreads), C::kLdsBytes, stream,
                     (const uint16_t*)a.q, (const uint16_t*)a.k, (const uint16_t*)a.v,
                     (uint16_t*)a.o, a.lse, a.N, BH, a.Hq, a.Hkv, a.Hq / a.Hkv, n_qb,
                     a.scale * kLog2e, remap, a.window, a.pack);
  return hipGetLastError();
}

template <int NW>
hipError_t launch_fwd_nw(const FwdArgs& a, bool local, hipStream_t stream) {
  constexpr int BC = 128, WPE = 2;
  if (a.d == 128) {
    if (local)
      return a.causal ? launch_fwd_t<128, BC, NW, WPE, true, true>(a, stream)
                      : launch_fwd_t<128, BC, NW, WPE, false, true>(a, stream);
    return a.causal ? launch_fwd_t<128, BC, NW, WPE, true, false>(a, stream)
                    : launch_fwd_t<128, BC, NW, WPE, false, false>(a, stream);
  }
  if (local)
    return a.causal ? launch_fwd_t<64, BC, NW, WPE, true, true>(a, stream)
                    : launch_fwd_t<64, BC, NW, WPE, false, true>(a, stream);
  return a.causal ? launch_fwd_t<64, BC, NW, WPE, true, false>(a, stream)
                  : launch_fwd_t<64, BC, NW, WPE, false, false>(a, stream);
}

constexpr int kCUs = 256;   // compute units of the chip

}  // namespace

hipError_t launch_fwd(const FwdArgs& a, hipStream_t stream) {
  // 8 waves x 32 rows = 256 query rows per workgroup, 128-key tiles (128 KB
  // of double-buffered LDS: one workgroup per CU), two waves per SIMD.  A
  // grid of fewer than 256 such workgroups leaves CUs idle, and one of
  // exactly 256 under the causal mask (blocks of unequal length) leaves them
  // unbalanced; there 4-wave workgroups of 128 rows (one wave per SIMD) share
  // the rows out over twice as many CUs.  At d = 64 two 4-wave workgroups
  // (64 KB of LDS each) share a CU, keeping two waves per SIMD, and the finer
  // blocks also win for short sequences (N <= 2048: 1.07-1.14x at 512-1024
  // eight-wave blocks) while longer ones tie or lose up to 5 %.  A row's
  // arithmetic does not depend on the workgroup size, so both give bitwise
  // the same O and LSE.  A window that covers every key changes nothing and
  // takes the plain kernel.
  const bool local = a.window >= 0 && a.window < a.N - 1;
  const long long grid8 =
      packed_grid(a.pack, a.B, a.Hq, 256, (long long)a.B * a.Hq * ((a.N + 255) / 256));
  const bool small = grid8 < kCUs || (a.causal && !local && grid8 <= kCUs) ||
                     (a.d == 64 && a.N <= 2048);
  return small ? launch_fwd_nw<4>(a, local, stream) : launch_fwd_nw<8>(a, local, stream);
}

}  // namespace attn
