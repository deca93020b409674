// attn_fwd_fp8.hip -- forward of exact attention over 8-bit (OCP E4M3) inputs
// on gfx950's 8-bit matrix unit (v_mfma_scale_f32_32x32x64_f8f6f4, unit
// block scales).
//
// Page "6.1 2023 年代：長上下文擴展技術：FlashAttention、RoPE 與稀疏注意力", §2.3:
// FlashAttention-3 adds a low-bit path, and the method stays exact.  Here Q, K
// and V arrive as E4M3 codes, each (batch, head) with an fp32 descale factor;
// the result is softmax attention of the dequantized values, O in bf16 and
// LSE in fp32 as in the bf16 forward (page "6.1 …", §2.2).
//
// gfx950 mapping (d = 128; the structure of the bf16 forward in attn_fwd.hip):
//   * one workgroup = 8 (or, on small grids, 4) waves x 32 query rows of one
//     (b, h), heaviest causal blocks first; 128-key K and V tiles of 16 KB
//     each, double-buffered through direct 16-byte global -> LDS loads (an
//     8-bit row of 128 bytes has the layout of a d = 64 bf16 row, see
//     attn_layout.h);
//   * S^T = K Q^T per 32-key block: two 32x32x64 8-bit MFMAs (d 0..63 and
//     64..127), Q^T held in registers, K row fragments from LDS;
//   * online softmax in fp32 exactly as the bf16 forward; the probabilities
//     are taken against the running maximum *times 2^8* (p' = 2^(s - m + 8),
//     so 0 <= p' <= 256) and rounded to E4M3 -- the 8-bit format's largest
//     value is 448 and its relative spacing 2^-3, so the rounding error is at
//     most 2^-4 p' (2^-10 below 2^-6, the subnormal range); the running sum
//     takes the unrounded p', so O = sum q(p') v / sum p' and the LSE is exact
//     up to fp32 rounding;
//   * O^T += V^T P^T per 64 keys and 32-wide d block: one 32x32x64 MFMA whose
//     B operand packs the two score blocks' p' (C layout) and whose A operand
//     comes from four 8-bit transposing LDS reads in the same key order;
//   * epilogue: O = acc * v_descale / l (bf16), LSE = (m + log2 l - 8) ln 2.
#include "attn_device.h"
#include "attn_launch.h"

#include <type_traits>

namespace attn {
namespace {

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x2 __attribute__((ext_vector_type(2)));

constexpr int kF8D = 128;       // head dim (bytes per 8-bit row)
constexpr int kF8BC = 128;      // keys per tile
// Workgroups of 8 waves (256 query rows), or of 4 (128 rows) when 8-wave
// blocks would leave CUs idle; two waves per SIMD either way (4-wave
// workgroups run two to a CU).  A wave's work -- its 32 rows against the
// same 128-key tiles -- is the same in both, so are its outputs, bitwise.
constexpr int kF8CUs = 256;     // MI355X
constexpr int kF8Tile = kF8BC * kF8D;           // bytes of one K or V tile
constexpr int kF8Lds = 2 * 2 * kF8Tile;         // double-buffered K and V (64 KB)
constexpr int kE8M0One = 127;                   // block scale exponent 0 (x1.0)

// D = A B + C with 32x64 (A) and 64x32 (B) E4M3 operands, fp32 accumulate.
__device__ __forceinline__ f32x16 mfma_f8(i32x8 a, i32x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, kE8M0One, 0, kE8M0One);
}

__device__ __forceinline__ i32x8 join(i32x4 a, i32x4 b) {
  return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}

// K row fragment of MFMA m: this lane's row, bytes 64m + 32*(lane/32) .. +31.
__device__ __forceinline__ i32x8 k_frag(const unsigned char* tile, int lane, int row0, int m) {
  return join(*(const i32x4*)(tile + layout::f8_row_frag_off(lane, row0, m, 0)),
              *(const i32x4*)(tile + layout::f8_row_frag_off(lane, row0, m, 1)));
}

// V^T fragment for d block db and the 64 keys k0 .. k0+63 (four transposing reads).
__device__ __forceinline__ i32x8 vt_frag(const unsigned char* tile, int lane, int k0, int db) {
  typedef __attribute__((address_space(3))) i32x2 lds_i32x2;
  i32x2 r[4];
#pragma unroll
  for (int t = 0; t < 4; ++t)
    r[t] = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
        (lds_i32x2*)(tile + layout::f8_tr_off(lane, k0, db, t)));
  return i32x8{r[0][0], r[0][1], r[1][0], r[1][1], r[2][0], r[2][1], r[3][0], r[3][1]};
}

// Four probabilities -> four E4M3 bytes (round to nearest even; 0 <= p <= 256).
__device__ __forceinline__ int pack4_f8(float a, float b, float c, float d) {
  // the two converts write the low and the high half of w; the bits passed
  // in as the untouched half (a's) are overwritten by the second, and reusing
  // a's register saves materialising a constant there
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, __builtin_bit_cast(int, a), false);
  return __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
}

template <bool CAUSAL, int NW>
__global__ __attribute__((amdgpu_flat_work_group_size(NW * 64, NW * 64),
                          amdgpu_waves_per_eu(2, 2))) void attn_fwd_fp8_kernel(
    const uint8_t* __restrict__ Q, const uint8_t* __restrict__ K, const uint8_t* __restrict__ V,
    const float* __restrict__ q_descale, const float* __restrict__ k_descale,
    const float* __restrict__ v_descale, uint16_t* __restrict__ O, float* __restrict__ LSE,
    int N, int BH, int Hq, int Hkv, int G, int n_qb, float tau_log2e, int xcd_remap) {
  constexpr int KB = kF8BC / 32;   // 32-key score blocks per tile
  constexpr int DB = kF8D / 32;    // 32-wide d blocks of O^T
  constexpr int kPrefK = 3;        // K fragments in flight ahead of their MFMA
  constexpr int kPrefV = 2;        // V^T fragments in flight ahead of their MFMA
  extern __shared__ __attribute__((aligned(1024))) unsigned char smem[];

  const int tid = threadIdx.x, lane = tid & 63, l32 = lane & 31, hi = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

  int bh, qrank;
  const int w = blockIdx.x;
  if (xcd_remap) {
    const int hx = BH >> 3;
    const int i = w >> 3;
    bh = (w & 7) * hx + (i % hx);
    qrank = i / hx;
  } else {
    bh = w % BH;
    qrank = w / BH;
  }
  const int qb = CAUSAL ? (n_qb - 1 - qrank) : qrank;
  const int b = bh / Hq, h = bh - b * Hq, hk = h / G;
  const size_t kv_row0 = ((size_t)b * Hkv + hk) * N;
  const uint8_t* Qp = Q + (size_t)bh * N * kF8D;
  const uint8_t* Kp = K + kv_row0 * kF8D;
  const uint8_t* Vp = V + kv_row0 * kF8D;
  // scores in log2 units: tau * log2(e) * q_descale * k_descale.  The running
  // maximum is taken over the unscaled scores and multiplied afterwards, which
  // needs a positive factor.  A zero descale stands for an all-zero head: every
  // score is 0 and the attention is uniform over the visible keys; the smallest
  // normal factor gives exactly that to within 2^-100 of a score (|raw score| <
  // 448^2 * 128 < 2^25) and keeps masked keys at -inf (a zero factor would turn
  // them into NaN).  A negative product or a non-finite factor has no
  // meaningful maximum here: the head's O and LSE become NaN.
  const float qk = q_descale[bh] * k_descale[b * Hkv + hk];
  float scale_log2 = tau_log2e * qk;
  if (qk == 0.f) scale_log2 = __FLT_MIN__;
  else if (!(qk > 0.f) || !(scale_log2 < INFINITY)) scale_log2 = __builtin_nanf("");
  const float vds = v_descale[b * Hkv + hk];

  const int q0 = qb * NW * 32;
  const int qw0 = q0 + wave * 32, qw1 = qw0 + 31;
  const bool wave_live = qw0 < N;

  // Q^T (B operand) of both MFMAs: this lane's query, bytes 64m + 32hi .. +31
  i32x8 qf[2];
  {
    const int row = qw0 + l32;
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      const uint8_t* src = Qp + (size_t)row * kF8D + 64 * m + 32 * hi;
      qf[m] = row < N ? join(*(const i32x4*)src, *(const i32x4*)(src + 16)) : i32x8{};
    }
  }
  // the Q loads' wait, once, before the tile loads start
#pragma unroll
  for (int m = 0; m < 2; ++m) asm volatile("" ::"v"(qf[m]));

  const int kv_end = CAUSAL ? min(N, q0 + NW * 32) : N;
  const int n_tiles = (kv_end + kF8BC - 1) / kF8BC;

  // an 8-bit row of 128 bytes is loaded exactly like a d = 64 bf16 row
  TileLoader<64, kF8BC, NW> ldr;
  ldr.init(wave, lane);
  auto stage = [&](int j) { return smem + (j & 1) * 2 * kF8Tile; };
  auto issue_tile = [&](int j) {
    unsigned char* kt = stage(j);
    ldr.load((const uint16_t*)Kp, j * kF8BC, N, kt, wave);
    ldr.load((const uint16_t*)Vp, j * kF8BC, N, kt + kF8Tile, wave);
  };

  f32x16 acc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) acc[db] = f32x16{};
  float m_run = -INFINITY, l_run = 0.f;

  issue_tile(0);
  wait_all_memory();
  __syncthreads();
  // A wave works on tiles [0, n_act): under the causal mask those that start
  // at or before its last row.  Tiles from n_mask on cross the diagonal or the
  // ragged end and take the mask.  The unmasked, the masked and the idle tiles
  // run as three loops -- every wave still issues every tile's loads and meets
  // every barrier -- so no idle or masked path merges into the accumulators
  // of the main loop (with such a merge the compiler copies all 64
  // accumulator registers on every tile).
  const int n_act = !wave_live ? 0 : (CAUSAL ? min(n_tiles, qw1 / kF8BC + 1) : n_tiles);
  const int n_mask = CAUSAL ? min(N / kF8BC, (qw0 + 1) / kF8BC) : N / kF8BC;
  const int n_plain = min(n_act, n_mask);
  auto tile = [&](int j, auto masked) {
    constexpr bool MASK = decltype(masked)::value;
    const int kstart = j * kF8BC;
    const unsigned char* kt = stage(j);
    const unsigned char* vt = kt + kF8Tile;

    // S^T[x] = K_x Q^T: 32 keys x 32 queries, lane holds query column l%32.
    // Step i is key block i % KB, d half i / KB; the K fragments go through
    // a ring of kPrefK registers, each read issued kPrefK MFMAs ahead.
    f32x16 s[KB];
#pragma unroll
    for (int x = 0; x < KB; ++x) s[x] = f32x16{};
    {
      constexpr int NS = 2 * KB;
      i32x8 kr[kPrefK];
#pragma unroll
      for (int i = 0; i < kPrefK; ++i) kr[i] = k_frag(kt, lane, 32 * (i % KB), i / KB);
#pragma unroll
      for (int i = 0; i < NS; ++i) {
        const i32x8 a = kr[i % kPrefK];
        if (i + kPrefK < NS) kr[i % kPrefK] = k_frag(kt, lane, 32 * ((i + kPrefK) % KB), (i + kPrefK) / KB);
        s[i % KB] = mfma_f8(a, qf[i / KB], s[i % KB]);
      }
      __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 2 * kPrefK, 0);
#pragma unroll
      for (int i = 0; i < NS - kPrefK; ++i) {
        __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
        __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 2, 0);
      }
      __builtin_amdgcn_sched_group_barrier(kSchedMfma, kPrefK, 0);
    }

    // slot i of block x holds key kb0 + 8(i/4) + i%4 (kb0 = kstart + 32x + 4hi):
    // key >= N or key > q is a compare of that constant offset against lim
    if (MASK) {
      const int q = qw0 + l32;
#pragma unroll
      for (int x = 0; x < KB; ++x) {
        const int kb0 = kstart + 32 * x + 4 * hi;
        const int lim = CAUSAL ? min(N - kb0 - 1, q - kb0) : N - kb0 - 1;
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if (8 * (i >> 2) + (i & 3) > lim) s[x][i] = -INFINITY;
      }
    }

    // online softmax (exact running max; key 0 is visible to every row, so
    // m_run is finite from the first visited tile on)
    float mx = -INFINITY;
#pragma unroll
    for (int x = 0; x < KB; ++x)
#pragma unroll
      for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[x][i]);
    mx = pair_max(mx) * scale_log2;
    const bool move = mx > m_run;
    if (__any(move)) {
      const float m_new = move ? mx : m_run;
      const float alpha = exp2_fast(m_run - m_new);
      m_run = m_new;
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < DB; ++db) acc[db] *= alpha;
    }
    // p' = 2^(s - m + 8) in [0, 256]; the sum takes p' before rounding
    const float shift = 8.f - m_run;
    i32x8 pf[KB / 2];
    float lsum = 0.f;
#pragma unroll
    for (int y = 0; y < KB / 2; ++y) {
      int wv[8];
#pragma unroll
      for (int xx = 0; xx < 2; ++xx)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          float p[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            p[e] = exp2_fast(__builtin_fmaf(s[2 * y + xx][4 * r + e], scale_log2, shift));
            lsum += p[e];
          }
          wv[4 * xx + r] = pack4_f8(p[0], p[1], p[2], p[3]);
        }
      pf[y] = i32x8{wv[0], wv[1], wv[2], wv[3], wv[4], wv[5], wv[6], wv[7]};
    }
    l_run += lsum;

    // O^T[db] += V^T P^T over the tile's two 64-key pairs; step i is pair
    // i / DB, d block i % DB, with the V^T fragments kPrefV steps ahead
    {
      constexpr int NP = (KB / 2) * DB;
      i32x8 vr[kPrefV];
#pragma unroll
      for (int i = 0; i < kPrefV; ++i) vr[i] = vt_frag(vt, lane, 64 * (i / DB), i % DB);
#pragma unroll
      for (int i = 0; i < NP; ++i) {
        const i32x8 a = vr[i % kPrefV];
        if (i + kPrefV < NP) vr[i % kPrefV] = vt_frag(vt, lane, 64 * ((i + kPrefV) / DB), (i + kPrefV) % DB);
        acc[i % DB] = mfma_f8(a, pf[i / DB], acc[i % DB]);
      }
      __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 4 * kPrefV, 0);
#pragma unroll
      for (int i = 0; i < NP - kPrefV; ++i) {
        __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
        __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 4, 0);
      }
      __builtin_amdgcn_sched_group_barrier(kSchedMfma, kPrefV, 0);
    }
  };
  int j = 0;
  for (; j < n_plain; ++j) {
    if (j + 1 < n_tiles) issue_tile(j + 1);
    tile(j, std::false_type{});
    wait_all_memory();
    __syncthreads();
  }
  for (; j < n_act; ++j) {
    if (j + 1 < n_tiles) issue_tile(j + 1);
    tile(j, std::true_type{});
    wait_all_memory();
    __syncthreads();
  }
  for (; j < n_tiles; ++j) {
    if (j + 1 < n_tiles) issue_tile(j + 1);
    wait_all_memory();
    __syncthreads();
  }

  if (!wave_live) return;
  const float lt = pair_sum(l_run);
  const float inv = vds / lt;
  const int q = qw0 + l32;
  if (q < N) {
    uint16_t* orow = O + ((size_t)bh * N + q) * kF8D;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int d0 = db * 32 + 8 * r + 4 * hi;
        const f32x16& a = acc[db];
        *(u32x2*)(orow + d0) = u32x2{pack_bf16x2(a[4 * r + 0] * inv, a[4 * r + 1] * inv),
                                     pack_bf16x2(a[4 * r + 2] * inv, a[4 * r + 3] * inv)};
      }
    if (hi == 0) LSE[(size_t)bh * N + q] = (m_run + log2_fast(lt) - 8.f) * kLn2;
  }
}

template <bool CAUSAL, int NW>
hipError_t launch_fp8_nw(const Fp8FwdArgs& a, hipStream_t stream) {
  const int n_qb = (a.N + NW * 32 - 1) / (NW * 32);
  const int BH = a.B * a.Hq;
  const long long grid = (long long)BH * n_qb;
  if (grid > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  auto kern = attn_fwd_fp8_kernel<CAUSAL, NW>;
  static std::atomic<uint64_t> lds_set{0};
  const hipError_t attr = allow_lds_on_device((const void*)kern, kF8Lds, lds_set);
  if (attr != hipSuccess) return attr;
  hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(NW * 64), kF8Lds, stream,
                     (const uint8_t*)a.q, (const uint8_t*)a.k, (const uint8_t*)a.v, a.q_descale,
                     a.k_descale, a.v_descale, (uint16_t*)a.o, a.lse, a.N, BH, a.Hq, a.Hkv,
                     a.Hq / a.Hkv, n_qb, a.scale * kLog2e, xcd_remap(BH, Packing{}));
  return hipGetLastError();
}

// 4-wave workgroups when the 8-wave grid has fewer workgroups than CUs, or,
// under the causal mask, no more than one per CU (the heaviest block then
// sets the time, and halving the blocks halves it): measured same-process,
// 25-42 % faster there, while from two 8-wave blocks per CU on the two
// forms are within a few percent and the 8-wave one is kept.
template <bool CAUSAL>
hipError_t launch_fp8_t(const Fp8FwdArgs& a, hipStream_t stream) {
  const long long grid8 = (long long)a.B * a.Hq * ((a.N + 255) / 256);
  const bool small = grid8 < kF8CUs || (CAUSAL && grid8 <= kF8CUs);
  return small ? launch_fp8_nw<CAUSAL, 4>(a, stream) : launch_fp8_nw<CAUSAL, 8>(a, stream);
}

}  // namespace

hipError_t launch_fwd_fp8(const Fp8FwdArgs& a, hipStream_t stream) {
  return a.causal ? launch_fp8_t<true>(a, stream) : launch_fp8_t<false>(a, stream);
}

}  // namespace attn
