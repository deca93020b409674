// attn_bwd.hip -- backward pass with recomputation from the log-sum-exp, gfx950.
//
// Method (page "6.1 … 長上下文擴展技術：FlashAttention、RoPE 與稀疏注意力", §2.2;
// page "从“算力黑洞”到“效率革命”：大模型Attention的演进之路", §4): the forward kept
// only O and the per-row log-sum-exp; the backward recomputes each block of
// probabilities from Q, K and that statistic instead of reading an N x N
// matrix back, trading one extra multiply for a full HBM round trip.
//
// With P_ij = exp(tau q_i.k_j - LSE_i) on visible keys:
//   dV_j = sum_i P_ij dO_i,   dP_ij = dO_i . v_j,
//   dS_ij = P_ij (dP_ij - D_i) with D_i = dO_i . O_i (= sum_k P_ik dP_ik),
//   dQ_i = tau sum_j dS_ij k_j,   dK_j = tau sum_i dS_ij q_i.
//
// Kernels, no atomics (bitwise deterministic):
//   bwd_pre   D_i = rowsum(dO_i * O_i)                          (memory bound)
//   bwd_dkdv  one workgroup per (batch, K/V head, 32*NWK keys): the key block's
//             K and V stay in LDS; 2*NWK waves = NWK key groups of 32 x two
//             halves of each 64-row query tile, each wave with dK^T and dV^T
//             in fp32 registers; the loop runs over the query tiles of every
//             query head of the group, so grouped heads are summed without
//             atomics; the two halves' partial sums are added through LDS at
//             the end;
//   bwd_dq    one workgroup per (batch, query head, 32*NW queries); each wave
//             owns 32 queries with dQ^T in registers and loops over key tiles;
//   bwd_grads the dK/dV and the dQ workgroups in one launch (what attn_bwd
//             runs after bwd_pre; the two separate kernels serve the
//             attn_bwd_dkdv and attn_bwd_dq calls, bitwise the same gradients).
// Causal and window masks are evaluated only on tiles that cross the
// diagonal, a band edge or the ragged end, as one branch per tile.
// All tiles move global -> LDS by 16-byte direct loads into the swizzled
// layout of attn_layout.h; operands are row fragments or transposing LDS
// reads.  The C layout of one product goes straight back as the B operand of
// the next (see the forward).  Both main kernels run two waves per SIMD.
#include "attn_device.h"
#include "attn_launch.h"

namespace attn {
namespace {

// ---------------------------------------------------------------------------
// D_i = sum_t dO[i,t] * O[i,t]   (fp32, one value per query row)
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void bwd_pre_kernel(const uint16_t* __restrict__ O,
                                                      const uint16_t* __restrict__ dO,
                                                      float* __restrict__ Dl, int rows) {
  constexpr int TPR = D / 8;        // threads per row, 16 bytes each
  constexpr int RPB = 256 / TPR;    // rows per block
  const int row = blockIdx.x * RPB + threadIdx.x / TPR;
  const int c = threadIdx.x % TPR;
  float acc = 0.f;
  if (row < rows) {
    const u32x4 a = *(const u32x4*)(O + (size_t)row * D + c * 8);
    const u32x4 b = *(const u32x4*)(dO + (size_t)row * D + c * 8);
#pragma unroll
    for (int w = 0; w < 4; ++w) acc += bf16_lo(a[w]) * bf16_lo(b[w]) + bf16_hi(a[w]) * bf16_hi(b[w]);
  }
#pragma unroll
  for (int off = TPR / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off, 64);
  if (row < rows && c == 0) Dl[row] = acc;
}

// ---------------------------------------------------------------------------
// dK, dV
// ---------------------------------------------------------------------------
template <int D, int NWK>
struct DkdvCfg {
  static constexpr int kNW = 2 * NWK;             // waves: NWK key groups x 2 query halves
  static constexpr int kThreads = kNW * 64;
  static constexpr int kBKV = NWK * 32;           // keys per workgroup
  static constexpr int kBQ = 64;                  // query rows per tile
  static constexpr int kKVTile = kBKV * 2 * D;    // bytes of the K (or V) block
  static constexpr int kQTile = kBQ * 2 * D;      // bytes of a Q (or dO) tile
  // LDS: K | V | (Q, dO) buffer 0 | (Q, dO) buffer 1 | (lse, delta) x 2
  static constexpr int kK = 0;
  static constexpr int kV = kKVTile;
  static constexpr int kQBuf = 2 * kKVTile;
  static constexpr int kStats = kQBuf + 2 * 2 * kQTile;
  static constexpr int kLdsBytes = kStats + 2 * 2 * kBQ * 4;
  // the second query half's dK^T, dV^T, parked for the final reduction
  static constexpr int kRedBytes = NWK * 2 * (D / 32) * 16 * 64 * 4;
  static_assert(kRedBytes <= kLdsBytes, "reduction fits in the tile memory");
};

// One dK/dV workgroup: w is its index in the dK/dV grid, smem its LDS.  With
// LOCAL, query i sees key j only when |i - j| <= window.  With S > 1 the G
// query heads of each K/V head are shared out over S workgroups of G/S heads
// each, which write fp32 partial sums to `part` instead of dK and dV.
template <int D, int NWK, bool CAUSAL, bool LOCAL>
__device__ __forceinline__ void dkdv_block(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    const uint16_t* __restrict__ dO, const float* __restrict__ LSE, const float* __restrict__ Dl,
    uint16_t* __restrict__ dK, uint16_t* __restrict__ dV, int Nmax, int BHkv, int Hq, int Hkv, int G,
    float scale, float scale_log2, int xcd_remap, int window, const Packing& pk, int w, int S,
    float* __restrict__ part, unsigned char* smem) {
  using C = DkdvCfg<D, NWK>;
  constexpr int kPrefetch = 3;   // (A, B) fragment pairs in flight ahead of their MFMA
  constexpr int NW = C::kNW;
  constexpr int BQ = C::kBQ;
  constexpr int DS = D / 16;
  constexpr int DB = D / 32;

  const int tid = threadIdx.x, lane = tid & 63, l32 = lane & 31, hi = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: scalar tile tests
  const int kg = wave % NWK;      // key group: keys kw0 .. kw0+31
  const int qh = wave / NWK;      // query half: rows 32*qh .. 32*qh+31 of each tile

  // heaviest key blocks (the first ones under the causal mask) first; when
  // B*Hkv*S is a multiple of 8 all key blocks of one (K/V head, split) share
  // an XCD, so the Q/dO tiles they all read stay in that XCD's L2
  int b, hk, kb, split = 0;
  if (pk.cu && BHkv / Hkv <= kMaxPackedSeqs) {
    // packed: real key blocks only, heaviest (most query tiles after them) first
    // (K/V head, split) pairs take the place of heads
    PackedUnits pu;
    pu.init(pk, BHkv / Hkv, Nmax, C::kBKV);
    int level, hks;
    if (!pu.unit(w, Hkv * S, b, hks, level)) return;
    hk = hks / S;
    split = hks - hk * S;
    const int len = seq_span(pk, Nmax, b).len;
    kb = (len + C::kBKV - 1) / C::kBKV - 1 - level;
  } else {
    const int BHS = BHkv * S;   // (K/V head, split) pairs
    int bhs;
    if (xcd_remap) {
      const int hx = BHS >> 3;
      const int i = w >> 3;
      bhs = (w & 7) * hx + (i % hx);
      kb = i / hx;
    } else {
      bhs = w % BHS;
      kb = w / BHS;
    }
    const int bhk = bhs / S;
    split = bhs - bhk * S;
    b = bhk / Hkv;
    hk = bhk - b * Hkv;
  }
  const int Gs = G / S;                  // query heads of this workgroup
  const SeqSpan sp = seq_span(pk, Nmax, b);
  const int N = sp.len;                  // rows of this sequence
  const int k0 = kb * C::kBKV;
  if (k0 >= N) return;                   // a block past a shorter packed sequence (uniform)
  const int kw0 = k0 + kg * 32;
  const size_t kv_off = sp.row0(pk, Nmax, b, hk, Hkv) * D;
  // rows of query head hk*G + split*Gs + hh start at q_row0 + hh * q_hstride
  const size_t q_row0 = sp.row0(pk, Nmax, b, hk * G + split * Gs, Hq);
  const size_t q_hstride = head_stride(pk, Nmax);

  unsigned char* Kt = smem + C::kK;
  unsigned char* Vt = smem + C::kV;
  auto qtile = [&](int buf) { return smem + C::kQBuf + buf * 2 * C::kQTile; };
  auto stats = [&](int buf) { return (float*)(smem + C::kStats + buf * 2 * BQ * 4); };

  const int n_qt = (N + BQ - 1) / BQ;
  // query tiles [qt0, qt_end) hold every query that sees one of these keys
  const int q_first = CAUSAL ? k0 : (LOCAL ? max(0, k0 - window) : 0);
  const int qt0 = q_first / BQ;
  const int qt_end = LOCAL ? min(n_qt, (k0 + C::kBKV + window + BQ - 1) / BQ) : n_qt;
  const int per_head = qt_end - qt0;
  const int n_iter = per_head * Gs;

  // the query tile of iteration it is (head hk*G + split*Gs + it / per_head, tile
  // qt0 + it % per_head); both are stepped incrementally instead of divided
  TileLoader<D, BQ, NW> ldq;
  ldq.init(wave, lane);
  auto issue = [&](int hh, int qt, int buf) {
    const size_t qh_off = (q_row0 + hh * q_hstride) * D;
    ldq.load(Q + qh_off, qt * BQ, N, qtile(buf), wave);
    ldq.load(dO + qh_off, qt * BQ, N, qtile(buf) + C::kQTile, wave);
  };
  // Threads 0..63 fetch the LSE of one row of the tile, threads 64..127 its D.
  // The raw value stays in a register until store_stats, after the tile's
  // math, so the load's latency hides under that math; rows past N become
  // LSE = +inf (P = 0) and D = 0.
  float stat_raw = 0.f;
  bool stat_valid = false;
  auto load_stats = [&](int hh, int qt) {
    const int row = qt * BQ + (tid & (BQ - 1));
    stat_valid = tid < 2 * BQ && row < N;
    if (stat_valid) {
      const size_t idx = q_row0 + hh * q_hstride + row;
      stat_raw = (tid < BQ ? LSE : Dl)[idx];
    }
  };
  auto store_stats = [&](int buf) {
    if (tid < BQ) stats(buf)[tid] = stat_valid ? stat_raw * kLog2e : INFINITY;
    else if (tid < 2 * BQ) stats(buf)[tid] = stat_valid ? stat_raw : 0.f;
  };

  {
    TileLoader<D, C::kBKV, NW> ldk;
    ldk.init(wave, lane);
    ldk.load(K + kv_off, k0, N, Kt, wave);
    ldk.load(V + kv_off, k0, N, Vt, wave);
  }
  int hh_n = 0, qt_n = qt0;     // the tile most recently issued
  issue(hh_n, qt_n, 0);
  load_stats(hh_n, qt_n);
  store_stats(0);
  wait_all_memory();
  __syncthreads();

  f32x16 dkT[DB], dvT[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) {
    dkT[db] = f32x16{};
    dvT[db] = f32x16{};
  }

  for (int it = 0; it < n_iter; ++it) {
    const int buf = it & 1;
    const int qs = qt_n * BQ + 32 * qh;   // first query row of this wave in tile it
    if (it + 1 < n_iter) {
      if (++qt_n == qt_end) {
        qt_n = qt0;
        ++hh_n;
      }
      issue(hh_n, qt_n, buf ^ 1);
      load_stats(hh_n, qt_n);
    }
    // the wave's 32 queries and 32 keys share at least one visible pair
    const bool in_band = !LOCAL || (qs <= kw0 + 31 + window && (CAUSAL || qs + 31 >= kw0 - window));
    if (kw0 < N && !(CAUSAL && qs + 31 < kw0) && in_band) {
      const unsigned char* Qt = qtile(buf);
      const unsigned char* dOt = Qt + C::kQTile;
      const float* lse_l = stats(buf);
      const float* del_l = lse_l + BQ;

      // S = Q K^T and dP = dO V^T: 32 queries x 32 keys, lane holds key column l%32
      // Step i uses slab i/2 of (Q, K) for S (even i) or of (dO, V) for dP
      // (odd i); both operands go through a ring of kPrefetch register pairs.
      f32x16 s = f32x16{}, dp = f32x16{};
      {
        constexpr int NSI = 2 * DS;
        auto fa = [&](int i) { return row_frag<D>((i & 1) ? dOt : Qt, lane, 32 * qh, i >> 1); };
        auto fb = [&](int i) { return row_frag<D>((i & 1) ? Vt : Kt, lane, 32 * kg, i >> 1); };
        u32x4 ra[kPrefetch], rb[kPrefetch];
#pragma unroll
        for (int i = 0; i < kPrefetch; ++i) {
          ra[i] = fa(i);
          rb[i] = fb(i);
        }
#pragma unroll
        for (int i = 0; i < NSI; ++i) {
          const u32x4 a = ra[i % kPrefetch], bb = rb[i % kPrefetch];
          if (i + kPrefetch < NSI) {
            ra[i % kPrefetch] = fa(i + kPrefetch);
            rb[i % kPrefetch] = fb(i + kPrefetch);
          }
          if (i & 1) dp = mfma_32x32x16(a, bb, dp);
          else s = mfma_32x32x16(a, bb, s);
        }
        __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 2 * kPrefetch, 0);
#pragma unroll
        for (int i = 0; i < NSI - kPrefetch; ++i) {
          __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
          __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 2, 0);
        }
        __builtin_amdgcn_sched_group_barrier(kSchedMfma, kPrefetch, 0);
      }

      // P = 2^(s*tau*log2e - LSE*log2e), dS = P (dP - D); rows 8r + 4hi + 0..3
      const bool need_mask = (CAUSAL && qs < kw0 + 31) ||
                             (LOCAL && (qs + 31 > kw0 + window || (!CAUSAL && qs < kw0 + 31 - window)));
      float p[16], ds[16];
      f32x4 dv[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const f32x4 lv = *(const f32x4*)(lse_l + 32 * qh + 8 * r + 4 * hi);
        dv[r] = *(const f32x4*)(del_l + 32 * qh + 8 * r + 4 * hi);
#pragma unroll
        for (int e = 0; e < 4; ++e) p[4 * r + e] = exp2_fast(__builtin_fmaf(s[4 * r + e], scale_log2, -lv[e]));
      }
      // The mask, as one branch for the tile so that unmasked tiles skip it:
      // slot 4r + e holds query qs + 4hi + c with c = 8r + e and this lane's
      // key is kw0 + l32, so with t = kw0 + l32 - qs - 4hi each test is a
      // compare of the constant c -- key > q <=> c < t, key < q - window <=>
      // c > t + window, key > q + window <=> c < t - window.
      if (need_mask) {
        const int t = kw0 + l32 - qs - 4 * hi;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int c = 8 * (i >> 2) + (i & 3);
          if ((CAUSAL && c < t) || (LOCAL && (c > t + window || (!CAUSAL && c < t - window)))) p[i] = 0.f;
        }
      }
#pragma unroll
      for (int i = 0; i < 16; ++i) ds[i] = p[i] * (dp[i] - dv[i >> 2][i & 3]);

      // dV^T += dO^T P and dK^T += Q^T dS: k slots of slab h2 are query rows
      // 16*h2 + {4hi..4hi+3, 8+4hi..8+4hi+3} of this wave's 32 rows
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2) {
        const u32x4 pb = pack8(p + 8 * h2);
        const u32x4 dsb = pack8(ds + 8 * h2);
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          dvT[db] = mfma_32x32x16(tr_frag<D>(dOt, lane, 32 * qh + 16 * h2, db * 32), pb, dvT[db]);
          dkT[db] = mfma_32x32x16(tr_frag<D>(Qt, lane, 32 * qh + 16 * h2, db * 32), dsb, dkT[db]);
        }
      }
    }

    if (it + 1 < n_iter) store_stats(buf ^ 1);
    wait_all_memory();
    __syncthreads();
  }

  // add the second query half's partial sums to the first half's
  float* red = (float*)smem;
  auto red_at = [&](int t, int db, int i) { return red + ((((kg * 2 + t) * DB + db) * 16 + i) * 64 + lane); };
  if (qh == 1) {
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        *red_at(0, db, i) = dkT[db][i];
        *red_at(1, db, i) = dvT[db][i];
      }
  }
  __syncthreads();
  if (qh == 1) return;

  // epilogue: lane holds key kw0 + l%32, d rows db*32 + 8r + 4hi + 0..3
  const int key = kw0 + l32;
  if (key < N && part) {
    // this split's fp32 sums, dK still unscaled
    const size_t plane = pk.cu ? (size_t)Hkv * pk.T * D : (size_t)BHkv * Nmax * D;
    float* pkr = part + 2 * split * plane + kv_off + (size_t)key * D;
    float* pvr = pkr + plane;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int d0 = db * 32 + 8 * r + 4 * hi;
        f32x4 a, v;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          a[e] = dkT[db][4 * r + e] + *red_at(0, db, 4 * r + e);
          v[e] = dvT[db][4 * r + e] + *red_at(1, db, 4 * r + e);
        }
        *(f32x4*)(pkr + d0) = a;
        *(f32x4*)(pvr + d0) = v;
      }
  } else if (key < N) {
    uint16_t* dkr = dK + kv_off + (size_t)key * D;
    uint16_t* dvr = dV + kv_off + (size_t)key * D;
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      f32x16 a = dkT[db], v = dvT[db];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        a[i] = (a[i] + *red_at(0, db, i)) * scale;
        v[i] += *red_at(1, db, i);
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int d0 = db * 32 + 8 * r + 4 * hi;
        *(u32x2*)(dkr + d0) = u32x2{pack_bf16x2(a[4 * r], a[4 * r + 1]), pack_bf16x2(a[4 * r + 2], a[4 * r + 3])};
        *(u32x2*)(dvr + d0) = u32x2{pack_bf16x2(v[4 * r], v[4 * r + 1]), pack_bf16x2(v[4 * r + 2], v[4 * r + 3])};
      }
    }
  }
}

template <int D, int NWK, int WPE, bool CAUSAL, bool LOCAL>
__global__ __attribute__((amdgpu_flat_work_group_size(2 * NWK * 64, 2 * NWK * 64),
                          amdgpu_waves_per_eu(WPE, WPE))) void bwd_dkdv_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    const uint16_t* __restrict__ dO, const float* __restrict__ LSE, const float* __restrict__ Dl,
    uint16_t* __restrict__ dK, uint16_t* __restrict__ dV, int N, int BHkv, int Hq, int Hkv, int G,
    float scale, float scale_log2, int xcd_remap, int window, Packing pk) {
  extern __shared__ __attribute__((aligned(1024))) unsigned char smem[];
  dkdv_block<D, NWK, CAUSAL, LOCAL>(Q, K, V, dO, LSE, Dl, dK, dV, N, BHkv, Hq, Hkv, G, scale,
                                    scale_log2, xcd_remap, window, pk, blockIdx.x, 1, nullptr,
                                    smem);
}

// ---------------------------------------------------------------------------
// dQ
// ---------------------------------------------------------------------------
template <int D, int BC, int NW>
struct DqCfg {
  static constexpr int kThreads = NW * 64;
  static constexpr int kBQ = NW * 32;               // query rows per workgroup
  static constexpr int kTile = BC * 2 * D;          // bytes of one K or V tile
  static constexpr int kLdsBytes = 2 * 2 * kTile;   // double-buffered K and V
};

// One dQ workgroup: w is its index in the dQ grid, smem its LDS.  With LOCAL,
// query i sees key j only when |i - j| <= window.
template <int D, int BC, int NW, bool CAUSAL, bool LOCAL>
__device__ __forceinline__ void dq_block(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    const uint16_t* __restrict__ dO, const float* __restrict__ LSE, const float* __restrict__ Dl,
    uint16_t* __restrict__ dQ, int Nmax, int BH, int Hq, int Hkv, int G, int n_qb, float scale,
    float scale_log2, int xcd_remap, int window, const Packing& pk, int w, unsigned char* smem) {
  using C = DqCfg<D, BC, NW>;
  constexpr int kPrefetch = 6;   // K/V fragments in flight ahead of their MFMA
  constexpr int DS = D / 16;
  constexpr int DB = D / 32;
  constexpr int KB = BC / 32;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, l32 = lane & 31, hi = lane >> 5;

  int b, h, qb;
  if (pk.cu && BH / Hq <= kMaxPackedSeqs) {
    // packed: real query blocks only, heaviest (most key tiles) first
    PackedUnits pu;
    pu.init(pk, BH / Hq, Nmax, C::kBQ);
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
  const SeqSpan sp = seq_span(pk, Nmax, b);
  const int N = sp.len;                  // rows of this sequence
  const int q0 = qb * C::kBQ;
  if (q0 >= N) return;                   // a block past a shorter packed sequence (uniform)
  const size_t q_row0 = sp.row0(pk, Nmax, b, h, Hq);
  const size_t q_off = q_row0 * D;
  const size_t kv_off = sp.row0(pk, Nmax, b, hk, Hkv) * D;
  const int qw0 = q0 + wave * 32;
  const int q = qw0 + l32;              // this lane's query row
  const bool wave_live = qw0 < N;

  u32x4 qf[DS], dof[DS];
#pragma unroll
  for (int s = 0; s < DS; ++s) {
    qf[s] = q < N ? *(const u32x4*)(Q + q_off + (size_t)q * D + s * 16 + 8 * hi) : zero4();
    dof[s] = q < N ? *(const u32x4*)(dO + q_off + (size_t)q * D + s * 16 + 8 * hi) : zero4();
  }
  const float lse_l2 = q < N ? LSE[q_row0 + q] * kLog2e : INFINITY;
  const float del = q < N ? Dl[q_row0 + q] : 0.f;

  f32x16 dqT[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) dqT[db] = f32x16{};

  // keys this workgroup's queries can see: [kv_begin, kv_end)
  const int kv_begin = LOCAL ? max(0, q0 - window) : 0;
  const int kv_end = CAUSAL ? min(N, q0 + C::kBQ) : (LOCAL ? min(N, q0 + C::kBQ + window) : N);
  const int j_first = kv_begin / BC;
  const int n_tiles = (kv_end + BC - 1) / BC;
  TileLoader<D, BC, NW> ldk;
  ldk.init(wave, lane);
  auto issue_tile = [&](int j, int buf) {
    unsigned char* kt = smem + buf * 2 * C::kTile;
    ldk.load(K + kv_off, j * BC, N, kt, wave);
    ldk.load(V + kv_off, j * BC, N, kt + C::kTile, wave);
  };
  issue_tile(j_first, j_first & 1);
  wait_all_memory();
  __syncthreads();

  // a key range [k_lo, k_hi] meets the band of this wave's 32 queries
  auto meets_band = [&](int k_lo, int k_hi) {
    return !LOCAL || (k_hi >= qw0 - window && (CAUSAL || k_lo <= qw0 + 31 + window));
  };
  for (int j = j_first; j < n_tiles; ++j) {
    const int buf = j & 1;
    const int kstart = j * BC;
    if (j + 1 < n_tiles) issue_tile(j + 1, buf ^ 1);
    if (wave_live && (!CAUSAL || kstart <= qw0 + 31) && meets_band(kstart, kstart + BC - 1)) {
      const unsigned char* kt = smem + buf * 2 * C::kTile;
      const unsigned char* vt = kt + C::kTile;
      const bool need_mask = (kstart + BC > N) || (CAUSAL && kstart + BC - 1 > qw0) ||
                             (LOCAL && (kstart < qw0 + 31 - window ||
                                        (!CAUSAL && kstart + BC - 1 > qw0 + window)));
#pragma unroll
      for (int x = 0; x < KB; ++x) {
        // 32-key blocks outside every row's band are skipped (wave-uniform)
        if (LOCAL && !meets_band(kstart + x * 32, kstart + x * 32 + 31)) continue;
        // S^T and dP^T: 32 keys x 32 queries, lane holds query column l%32
        // Step i reads slab i/2 of K (even i) or V (odd i); the fragments go
        // through a ring of kPrefetch registers, one LDS read per MFMA.
        f32x16 s = f32x16{}, dp = f32x16{};
        {
          constexpr int NSI = 2 * DS;
          auto frag = [&](int i) { return row_frag<D>((i & 1) ? vt : kt, lane, x * 32, i >> 1); };
          u32x4 fr[kPrefetch];
#pragma unroll
          for (int i = 0; i < kPrefetch; ++i) fr[i] = frag(i);
#pragma unroll
          for (int i = 0; i < NSI; ++i) {
            const u32x4 a = fr[i % kPrefetch];
            if (i + kPrefetch < NSI) fr[i % kPrefetch] = frag(i + kPrefetch);
            if (i & 1) dp = mfma_32x32x16(a, dof[i >> 1], dp);
            else s = mfma_32x32x16(a, qf[i >> 1], s);
          }
          __builtin_amdgcn_sched_group_barrier(kSchedDsRead, kPrefetch, 0);
#pragma unroll
          for (int i = 0; i < NSI - kPrefetch; ++i) {
            __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
            __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 1, 0);
          }
          __builtin_amdgcn_sched_group_barrier(kSchedMfma, kPrefetch, 0);
        }
        float p[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) p[i] = exp2_fast(__builtin_fmaf(s[i], scale_log2, -lse_l2));
        // The mask, as one branch for the block: slot i holds key kb0 + c with
        // kb0 = kstart + 32x + 4hi and c = 8(i/4) + i%4, so with t = q - kb0
        // each test is a compare of the constant c:
        //   key >= N <=> c > N - kb0 - 1,   key > q <=> c > t,
        //   key > q + window <=> c > t + window,   key < q - window <=> c < t - window.
        if (need_mask) {
          const int kb0 = kstart + x * 32 + 4 * hi;
          const int t = q - kb0;
          int lim = N - kb0 - 1;
          if (CAUSAL) lim = min(lim, t);
          if (LOCAL && !CAUSAL) lim = min(lim, t + window);
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int c = 8 * (i >> 2) + (i & 3);
            if (c > lim || (LOCAL && c < t - window)) p[i] = 0.f;
          }
        }
        float ds[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) ds[i] = p[i] * (dp[i] - del);
        // dQ^T += K^T dS^T: k slots of slab h2 are keys 16*h2 + {4hi.., 8+4hi..}
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2) {
          const u32x4 dsb = pack8(ds + 8 * h2);
#pragma unroll
          for (int db = 0; db < DB; ++db)
            dqT[db] = mfma_32x32x16(tr_frag<D>(kt, lane, x * 32 + 16 * h2, db * 32), dsb, dqT[db]);
        }
      }
    }
    wait_all_memory();
    __syncthreads();
  }

  if (q < N) {
    uint16_t* dqr = dQ + q_off + (size_t)q * D;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int d0 = db * 32 + 8 * r + 4 * hi;
        *(u32x2*)(dqr + d0) = u32x2{pack_bf16x2(dqT[db][4 * r] * scale, dqT[db][4 * r + 1] * scale),
                                    pack_bf16x2(dqT[db][4 * r + 2] * scale, dqT[db][4 * r + 3] * scale)};
      }
  }
}

template <int D, int BC, int NW, int WPE, bool CAUSAL, bool LOCAL>
__global__ __attribute__((amdgpu_flat_work_group_size(NW * 64, NW * 64),
                          amdgpu_waves_per_eu(WPE, WPE))) void bwd_dq_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    const uint16_t* __restrict__ dO, const float* __restrict__ LSE, const float* __restrict__ Dl,
    uint16_t* __restrict__ dQ, int N, int BH, int Hq, int Hkv, int G, int n_qb, float scale,
    float scale_log2, int xcd_remap, int window, Packing pk) {
  extern __shared__ __attribute__((aligned(1024))) unsigned char smem[];
  dq_block<D, BC, NW, CAUSAL, LOCAL>(Q, K, V, dO, LSE, Dl, dQ, N, BH, Hq, Hkv, G, n_qb, scale,
                                     scale_log2, xcd_remap, window, pk, blockIdx.x, smem);
}

// dK/dV and dQ in one launch: workgroups [0, n_dkdv) are dK/dV blocks and the
// rest dQ blocks (a packed batch of up to kMaxPackedSeqs sequences: its real
// dK/dV units, then its real dQ units, then empty workgroups).  The two
// halves are independent (both read only the inputs, LSE and D), so dQ blocks
// fill the CUs that dK/dV blocks release instead of waiting for the whole
// dK/dV grid to drain.  Both halves use NW waves.  With S > 1 the dK/dV blocks
// write partial sums to `part` (see dkdv_block) for bwd_dkdv_reduce_kernel.
template <int D, int NWK, int BC, int NW, int WPE, bool CAUSAL, bool LOCAL>
__global__ __attribute__((amdgpu_flat_work_group_size(NW * 64, NW * 64),
                          amdgpu_waves_per_eu(WPE, WPE))) void bwd_grads_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    const uint16_t* __restrict__ dO, const float* __restrict__ LSE, const float* __restrict__ Dl,
    uint16_t* __restrict__ dQ, uint16_t* __restrict__ dK, uint16_t* __restrict__ dV, int N,
    int BHkv, int BH, int Hq, int Hkv, int G, int n_dkdv, int n_qb, float scale, float scale_log2,
    int xcd_kv, int xcd_q, int window, Packing pk, int S, float* __restrict__ part) {
  static_assert(2 * NWK == NW, "both halves run the same number of waves");
  extern __shared__ __attribute__((aligned(1024))) unsigned char smem[];
  const int w = blockIdx.x;
  int split = n_dkdv;
  if (pk.cu && BHkv / Hkv <= kMaxPackedSeqs) {
    // packed: the real dK/dV units come first, then the real dQ units; the
    // rest of the grid (sized for the longest sequence) is empty
    PackedUnits pu;
    pu.init(pk, BHkv / Hkv, N, DkdvCfg<D, NWK>::kBKV);
    split = (int)pu.at_or_above(0, Hkv * S);
  }
  if (w < split)
    dkdv_block<D, NWK, CAUSAL, LOCAL>(Q, K, V, dO, LSE, Dl, dK, dV, N, BHkv, Hq, Hkv, G, scale,
                                      scale_log2, xcd_kv, window, pk, w, S, part, smem);
  else
    dq_block<D, BC, NW, CAUSAL, LOCAL>(Q, K, V, dO, LSE, Dl, dQ, N, BH, Hq, Hkv, G, n_qb, scale,
                                       scale_log2, xcd_q, window, pk, w - split, smem);
}

// dK = scale * sum_s part[s][0], dV = sum_s part[s][1], added in split order
// (so the result is the same on every run), rounded to bf16.  Thread i takes
// elements 4i .. 4i+3 of the n4 * 4 in each plane.
__global__ __launch_bounds__(256) void bwd_dkdv_reduce_kernel(const float* __restrict__ part,
                                                              uint16_t* __restrict__ dK,
                                                              uint16_t* __restrict__ dV,
                                                              size_t n4, int S, float scale) {
  const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n4) return;
  const f32x4* p = (const f32x4*)part + i;
  f32x4 k = p[0], v = p[n4];
  for (int s = 1; s < S; ++s) {
    k += p[2 * s * n4];
    v += p[(2 * s + 1) * n4];
  }
  *(u32x2*)(dK + 4 * i) = u32x2{pack_bf16x2(k[0] * scale, k[1] * scale),
                                pack_bf16x2(k[2] * scale, k[3] * scale)};
  *(u32x2*)(dV + 4 * i) = u32x2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
}

// Dynamic LDS beyond 64 KB, allowed once per kernel instance and device.
template <typename KernelT>
hipError_t allow_lds(KernelT kern, int bytes, std::atomic<uint64_t>& done) {
  return allow_lds_on_device((const void*)kern, bytes, done);
}

template <int D>
hipError_t launch_pre_t(const BwdArgs& a, hipStream_t stream) {
  const int rows = (int)a.rows();   // the host checks that it fits
  constexpr int RPB = 256 / (D / 8);
  hipLaunchKernelGGL(bwd_pre_kernel<D>, dim3((rows + RPB - 1) / RPB), dim3(256), 0, stream,
                     (const uint16_t*)a.o, (const uint16_t*)a.dout, a.delta, rows);
  return hipGetLastError();
}

// Workgroup shapes, per head dimension.  d = 128: dK/dV blocks of 4 key
// groups x 2 query halves = 8 waves, 128 keys; dQ blocks of 8 waves x 32
// queries over 128-key tiles (128 KB of double-buffered LDS: one workgroup
// per CU); the d = 64 shape below on grids too short to fill the chip
// (LaunchGrads).  d = 64: half of each -- 2 key groups (64 keys) and 4 dQ waves
// (128 queries) -- whose LDS (64 KB) lets two workgroups share a CU, so the
// CU still runs two waves per SIMD over finer blocks (measured 1.00-1.20x
// the 8-wave launch on every d = 64 shape tried).  A wave's work is the same
// in both shapes, so the gradients are bitwise equal.
template <int D>
struct BwdShape {
  static constexpr int kNWK = D == 64 ? 2 : 4;    // dK/dV key groups
  static constexpr int kDqNW = 2 * kNWK;          // dQ waves (= the dK/dV block's waves)
};
constexpr int kDkdvWPE = 2;
constexpr int kDqBC = 128, kDqWPE = 2;
constexpr int kBwdCUs = 256;   // compute units of the chip
static_assert(BwdShape<128>::kNWK * 32 == kBwdKeysPerBlock, "the host's split rule counts these blocks");
inline int kv_splits_of(const BwdArgs& a) { return a.kv_splits; }

template <int D, bool CAUSAL, bool LOCAL>
struct LaunchDkdv {
  static hipError_t run(const BwdArgs& a, hipStream_t stream) {
    using CK = DkdvCfg<D, BwdShape<D>::kNWK>;
    auto kern = bwd_dkdv_kernel<D, BwdShape<D>::kNWK, kDkdvWPE, CAUSAL, LOCAL>;
    static std::atomic<uint64_t> lds_set{0};
    const hipError_t attr = allow_lds(kern, CK::kLdsBytes, lds_set);
    if (attr != hipSuccess) return attr;
    const int n_kb = (a.N + CK::kBKV - 1) / CK::kBKV;
    const int BHkv = a.B * a.Hkv;
    const long long grid = packed_grid(a.pack, a.B, a.Hkv, CK::kBKV, (long long)BHkv * n_kb);
    if (grid > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    if (grid == 0) return hipSuccess;
    hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(CK::kThreads), CK::kLdsBytes, stream,
                       (const uint16_t*)a.q, (const uint16_t*)a.k, (const uint16_t*)a.v,
                       (const uint16_t*)a.dout, a.lse, a.delta, (uint16_t*)a.dk, (uint16_t*)a.dv,
                       a.N, BHkv, a.Hq, a.Hkv, a.Hq / a.Hkv, a.scale, a.scale * kLog2e,
                       xcd_remap(BHkv, a.pack), a.window, a.pack);
    return hipGetLastError();
  }
};

template <int D, bool CAUSAL, bool LOCAL>
struct LaunchDq {
  static hipError_t run(const BwdArgs& a, hipStream_t stream) {
    using CQ = DqCfg<D, kDqBC, BwdShape<D>::kDqNW>;
    auto kern = bwd_dq_kernel<D, kDqBC, BwdShape<D>::kDqNW, kDqWPE, CAUSAL, LOCAL>;
    static std::atomic<uint64_t> lds_set{0};
    const hipError_t attr = allow_lds(kern, CQ::kLdsBytes, lds_set);
    if (attr != hipSuccess) return attr;
    const int n_qb = (a.N + CQ::kBQ - 1) / CQ::kBQ;
    const int BH = a.B * a.Hq;
    const long long grid = packed_grid(a.pack, a.B, a.Hq, CQ::kBQ, (long long)BH * n_qb);
    if (grid > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    if (grid == 0) return hipSuccess;
    hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(CQ::kThreads), CQ::kLdsBytes, stream,
                       (const uint16_t*)a.q, (const uint16_t*)a.k, (const uint16_t*)a.v,
                       (const uint16_t*)a.dout, a.lse, a.delta, (uint16_t*)a.dq, a.N, BH, a.Hq,
                       a.Hkv, a.Hq / a.Hkv, n_qb, a.scale, a.scale * kLog2e, xcd_remap(BH, a.pack),
                       a.window, a.pack);
    return hipGetLastError();
  }
};

template <int D, bool CAUSAL, bool LOCAL>
struct LaunchGrads {
  // One launch with NWK key groups per dK/dV block and 2*NWK dQ waves.
  template <int NWK>
  static hipError_t run_shape(const BwdArgs& a, hipStream_t stream) {
    using CK = DkdvCfg<D, NWK>;
    using CQ = DqCfg<D, kDqBC, 2 * NWK>;
    static_assert(CK::kThreads == CQ::kThreads, "one workgroup size for both halves");
    constexpr int lds = CK::kLdsBytes > CQ::kLdsBytes ? CK::kLdsBytes : CQ::kLdsBytes;
    auto kern = bwd_grads_kernel<D, NWK, kDqBC, 2 * NWK, kDqWPE, CAUSAL, LOCAL>;
    static std::atomic<uint64_t> lds_set{0};
    const hipError_t attr = allow_lds(kern, lds, lds_set);
    if (attr != hipSuccess) return attr;
    const int BHkv = a.B * a.Hkv, BH = a.B * a.Hq;
    const int n_kb = (a.N + CK::kBKV - 1) / CK::kBKV;
    const int n_qb = (a.N + CQ::kBQ - 1) / CQ::kBQ;
    const int S = kv_splits_of(a);
    const long long n_dkdv = (long long)BHkv * n_kb * S;
    const long long grid = packed_grid(a.pack, a.B, a.Hkv * S, CK::kBKV, n_dkdv) +
                           packed_grid(a.pack, a.B, a.Hq, CQ::kBQ, (long long)BH * n_qb);
    if (grid > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    if (grid == 0) return hipSuccess;
    hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(CK::kThreads), lds, stream,
                       (const uint16_t*)a.q, (const uint16_t*)a.k, (const uint16_t*)a.v,
                       (const uint16_t*)a.dout, a.lse, a.delta, (uint16_t*)a.dq, (uint16_t*)a.dk,
                       (uint16_t*)a.dv, a.N, BHkv, BH, a.Hq, a.Hkv, a.Hq / a.Hkv, (int)n_dkdv,
                       n_qb, a.scale, a.scale * kLog2e, xcd_remap(BHkv * S, a.pack),
                       xcd_remap(BH, a.pack), a.window, a.pack, S, S > 1 ? a.part : nullptr);
    return hipGetLastError();
  }

  // d = 128 takes 4-wave blocks too when the 8-wave grid would not fill the
  // chip: at one 4-wave workgroup per CU (128 KB of LDS) twice as many CUs
  // then work (1.15-1.28x measured at 96-192 eight-wave blocks, 15-23 %
  // slower from 384 up); the gradients are bitwise the same.
  static hipError_t run(const BwdArgs& a, hipStream_t stream) {
    if (D == 128) {
      using CK = DkdvCfg<D, BwdShape<D>::kNWK>;
      using CQ = DqCfg<D, kDqBC, BwdShape<D>::kDqNW>;
      const long long n_kb = (a.N + CK::kBKV - 1) / CK::kBKV;
      const long long n_qb = (a.N + CQ::kBQ - 1) / CQ::kBQ;
      const int S = kv_splits_of(a);
      const long long grid8 =
          packed_grid(a.pack, a.B, a.Hkv * S, CK::kBKV, (long long)a.B * a.Hkv * n_kb * S) +
          packed_grid(a.pack, a.B, a.Hq, CQ::kBQ, (long long)a.B * a.Hq * n_qb);
      if (grid8 < kBwdCUs) return run_shape<BwdShape<64>::kNWK>(a, stream);
    }
    return run_shape<BwdShape<D>::kNWK>(a, stream);
  }
};

// (d, causal, window) -> kernel instance.  A window that covers every key
// changes nothing and takes the plain kernels.
template <template <int, bool, bool> class L>
hipError_t dispatch(const BwdArgs& a, hipStream_t stream) {
  const bool local = a.window >= 0 && a.window < a.N - 1;
  if (a.d == 128) {
    if (local) return a.causal ? L<128, true, true>::run(a, stream) : L<128, false, true>::run(a, stream);
    return a.causal ? L<128, true, false>::run(a, stream) : L<128, false, false>::run(a, stream);
  }
  if (local) return a.causal ? L<64, true, true>::run(a, stream) : L<64, false, true>::run(a, stream);
  return a.causal ? L<64, true, false>::run(a, stream) : L<64, false, false>::run(a, stream);
}

}  // namespace

hipError_t launch_bwd_grads(const BwdArgs& a, hipStream_t stream) {
  const int S = kv_splits_of(a);
  if (S < 1 || (a.Hq / a.Hkv) % S != 0 || (S > 1 && !a.part)) return hipErrorInvalidValue;
  hipError_t e = dispatch<LaunchGrads>(a, stream);
  if (e != hipSuccess || S == 1) return e;
  // one plane of dK (or dV): B*Hkv*N rows, packed Hkv*T
  const size_t n4 = (a.pack.cu ? (size_t)a.Hkv * a.pack.T : (size_t)a.B * a.Hkv * a.N) * a.d / 4;
  hipLaunchKernelGGL(bwd_dkdv_reduce_kernel, dim3((unsigned)((n4 + 255) / 256)), dim3(256), 0,
                     stream, a.part, (uint16_t*)a.dk, (uint16_t*)a.dv, n4, S, a.scale);
  return hipGetLastError();
}

hipError_t launch_bwd_pre(const BwdArgs& a, hipStream_t stream) {
  return a.d == 128 ? launch_pre_t<128>(a, stream) : launch_pre_t<64>(a, stream);
}

hipError_t launch_bwd_dkdv(const BwdArgs& a, hipStream_t stream) {
  return dispatch<LaunchDkdv>(a, stream);
}

hipError_t launch_bwd_dq(const BwdArgs& a, hipStream_t stream) {
  return dispatch<LaunchDq>(a, stream);
}

hipError_t launch_bwd(const BwdArgs& a, hipStream_t stream) {
  hipError_t e = launch_bwd_pre(a, stream);
  return e == hipSuccess ? launch_bwd_grads(a, stream) : e;
}

}  // namespace attn
