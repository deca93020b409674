// attn_fwd.hip -- tiled exact attention forward for gfx950 (MI355X).
//
// Method (page "从“算力黑洞”到“效率革命”：大模型Attention的演进之路", §4, and page
// "6.1 … 長上下文擴展技術：FlashAttention、RoPE 與稀疏注意力", §2.2): Q, K and V
// are cut into blocks along the sequence; a block of query rows is held on
// chip while K/V tiles stream past it, and for each tile the four steps
// "score -> update the row max -> accumulate the exp-sum -> accumulate the
// weighted V" run without the N x N scores ever leaving the chip.  Only O and
// the per-row log-sum-exp are written.
//
// gfx950 mapping
//   * one workgroup = NW waves = NW*QG*32 query rows of one (batch, head);
//     each wave owns QG groups of 32 query rows for the whole key loop;
//   * S^T = K Q^T is computed (keys are the MFMA rows), so the 32x32 C
//     layout gives each lane one query column: the row max and row sum are
//     in-register over 16 values plus one exchange with lane l^32;
//   * the same accumulators, rounded to bf16, are directly the B operand of
//     O^T = V^T P^T (the k-slot order inside one MFMA is free as long as A and
//     B agree), so P never goes through LDS;
//   * K tiles sit in LDS row-major (rows padded by 16 bytes: conflict-free
//     16-byte reads), V tiles "4 keys per d" so the transposed V operand is
//     two 8-byte reads; both are double-buffered, the next tile's global loads
//     are in flight while the current tile is computed, one barrier per tile;
//   * causal: key tiles past a workgroup's last row are never loaded, a wave
//     skips tiles past its own last row, and only tiles that cross the
//     diagonal (or the ragged end of the sequence) evaluate the mask;
//   * exp is 2^x with scale*log2(e) folded into one FMA; the LSE is converted
//     back to natural log units of the scaled scores before it is stored;
//   * workgroups run heaviest causal block first, and when B*Hq is a multiple
//     of 8 the workgroup -> (head, block) map keeps each head on one XCD so its
//     K/V stay in that XCD's L2.
#include "attn_device.h"
#include "attn_launch.h"

namespace attn {
namespace {

template <int D, int QG, int BC, int NW>
struct FwdCfg {
  static constexpr int kThreads = NW * 64;
  static constexpr int kBR = NW * QG * 32;            // query rows per workgroup
  static constexpr int kKStride = D * 2 + 16;         // bytes per K row in LDS (padded)
  static constexpr int kKTileBytes = BC * kKStride;
  static constexpr int kVGroupBytes = D * 8;          // 4 keys x D, "4 keys per d"
  static constexpr int kVTileBytes = (BC / 4) * kVGroupBytes;
  static constexpr int kKChunks = BC * D / 8;         // 16-byte chunks in a K tile
  static constexpr int kVUnits = (BC / 4) * (D / 8);  // 4 keys x 8 d units in a V tile
  static constexpr int kKPer = (kKChunks + kThreads - 1) / kThreads;
  static constexpr int kVPer = (kVUnits + kThreads - 1) / kThreads;
  static constexpr int kLdsBytes = 2 * (kKTileBytes + kVTileBytes);
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
template <int D, int QG, int BC, int NW, int WPE, bool CAUSAL, int LAG = 0>
__global__ __attribute__((amdgpu_flat_work_group_size(NW * 64, NW * 64),
                          amdgpu_waves_per_eu(WPE, WPE))) void attn_fwd_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
    const uint16_t* __restrict__ V, uint16_t* __restrict__ O, float* __restrict__ LSE,
    int N, int BH, int Hq, int Hkv, int G, int n_qb, float scale_log2, int xcd_remap) {
  using C = FwdCfg<D, QG, BC, NW>;
  constexpr int NT = C::kThreads;
  constexpr int DS = D / 16;   // k-slabs of the QK^T contraction
  constexpr int KB = BC / 32;  // 32-key blocks per tile
  constexpr int DB = D / 32;   // 32-wide d blocks of O^T

  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  unsigned char* lds_k = smem;
  unsigned char* lds_v = smem + 2 * C::kKTileBytes;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l32 = lane & 31;
  const int hi = lane >> 5;

  // ---- workgroup -> (batch*head, query block) ----
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
  const int b = bh / Hq;
  const int h = bh - b * Hq;
  const int hk = h / G;
  const uint16_t* Qp = Q + (size_t)bh * N * D;
  const uint16_t* Kp = K + ((size_t)b * Hkv + hk) * N * D;
  const uint16_t* Vp = V + ((size_t)b * Hkv + hk) * N * D;

  const int q0 = qb * C::kBR;
  const int qw0 = q0 + wave * QG * 32;  // first query row of this wave
  const int qw1 = qw0 + QG * 32 - 1;    // last query row of this wave
  const bool wave_live = qw0 < N;

  // ---- Q^T fragments (B operand), kept in registers for the whole loop ----
  u32x4 qf[QG][DS];
#pragma unroll
  for (int g = 0; g < QG; ++g) {
    const int row = qw0 + g * 32 + l32;
#pragma unroll
    for (int s = 0; s < DS; ++s)
      qf[g][s] = row < N ? *(const u32x4*)(Qp + (size_t)row * D + s * 16 + 8 * hi) : zero4();
  }

  const int kv_end = CAUSAL ? min(N, q0 + C::kBR) : N;
  const int n_tiles = (kv_end + BC - 1) / BC;

  // ---- global -> register staging of one K/V tile ----
  u32x4 kreg[C::kKPer];
  u32x4 vreg[C::kVPer][4];
  auto load_tile = [&](int kstart) {
#pragma unroll
    for (int it = 0; it < C::kKPer; ++it) {
      const int c = it * NT + tid;
      if (C::kKChunks % NT == 0 || c < C::kKChunks) {
        const int row = c / (D / 8), col = c % (D / 8);
        const int key = kstart + row;
        kreg[it] = key < N ? *(const u32x4*)(Kp + (size_t)key * D + col * 8) : zero4();
      }
    }
#pragma unroll
    for (int it = 0; it < C::kVPer; ++it) {
      const int u = it * NT + tid;
      if (C::kVUnits % NT == 0 || u < C::kVUnits) {
        const int g = u / (D / 8), col = u % (D / 8);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int key = kstart + 4 * g + r;
          vreg[it][r] = key < N ? *(const u32x4*)(Vp + (size_t)key * D + col * 8) : zero4();
        }
      }
    }
  };
  auto store_tile = [&](int buf) {
    unsigned char* kb = lds_k + buf * C::kKTileBytes;
    unsigned char* vb = lds_v + buf * C::kVTileBytes;
#pragma unroll
    for (int it = 0; it < C::kKPer; ++it) {
      const int c = it * NT + tid;
      if (C::kKChunks % NT == 0 || c < C::kKChunks) {
        const int row = c / (D / 8), col = c % (D / 8);
        *(u32x4*)(kb + row * C::kKStride + col * 16) = kreg[it];
      }
    }
#pragma unroll
    for (int it = 0; it < C::kVPer; ++it) {
      const int u = it * NT + tid;
      if (C::kVUnits % NT == 0 || u < C::kVUnits) {
        const int g = u / (D / 8), col = u % (D / 8);
        u32x2 t[8];
        interleave4x8(vreg[it], t);
        unsigned char* dst = vb + g * C::kVGroupBytes + col * 8 * 8;
#pragma unroll
        for (int j = 0; j < 4; ++j)
          *(u32x4*)(dst + 16 * j) = u32x4{t[2 * j][0], t[2 * j][1], t[2 * j + 1][0], t[2 * j + 1][1]};
      }
    }
  };

  // ---- running statistics and the O^T accumulator ----
  f32x16 acc[DB][QG];
  float m_run[QG], l_run[QG];
#pragma unroll
  for (int g = 0; g < QG; ++g) {
    m_run[g] = -INFINITY;
    l_run[g] = 0.f;
#pragma unroll
    for (int db = 0; db < DB; ++db) acc[db][g] = f32x16{};
  }

  load_tile(0);
  store_tile(0);
  __syncthreads();

  for (int j = 0; j < n_tiles; ++j) {
    const int buf = j & 1;
    const int kstart = j * BC;
    if (j + 1 < n_tiles) load_tile(kstart + BC);

    const bool wave_has_keys = wave_live && (!CAUSAL || kstart <= qw1);
    if (wave_has_keys) {
      const unsigned char* kb = lds_k + buf * C::kKTileBytes;
      const unsigned char* vb = lds_v + buf * C::kVTileBytes;

      // S^T[kb][g] = K_tile Q^T  (32 keys x 32 queries per accumulator)
      f32x16 s[KB][QG];
#pragma unroll
      for (int x = 0; x < KB; ++x)
#pragma unroll
        for (int g = 0; g < QG; ++g) s[x][g] = f32x16{};
#pragma unroll
      for (int sl = 0; sl < DS; ++sl) {
#pragma unroll
        for (int x = 0; x < KB; ++x) {
          const u32x4 a = *(const u32x4*)(kb + (x * 32 + l32) * C::kKStride + (sl * 16 + 8 * hi) * 2);
#pragma unroll
          for (int g = 0; g < QG; ++g) s[x][g] = mfma_32x32x16(a, qf[g][sl], s[x][g]);
        }
      }

      // mask: only tiles that cross the diagonal or the ragged end
      const bool need_mask = (kstart + BC > N) || (CAUSAL && kstart + BC - 1 > qw0);
      if (need_mask) {
#pragma unroll
        for (int x = 0; x < KB; ++x)
#pragma unroll
          for (int g = 0; g < QG; ++g) {
            const int q = qw0 + g * 32 + l32;
#pragma unroll
            for (int i = 0; i < 16; ++i) {
              const int key = kstart + x * 32 + 8 * (i >> 2) + 4 * hi + (i & 3);
              if (key >= N || (CAUSAL && key > q)) s[x][g][i] = -INFINITY;
            }
          }
      }

      // online softmax: running max, rescale, exp, running sum, P -> bf16
      u32x4 pf[QG][KB][2];
#pragma unroll
      for (int g = 0; g < QG; ++g) {
        float mx = -INFINITY;
#pragma unroll
        for (int x = 0; x < KB; ++x)
#pragma unroll
          for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[x][g][i]);
        mx = fmaxf(mx, swap_halves(mx)) * scale_log2;
        // move the reference maximum only when it falls more than LAG behind
        const bool move = mx > m_run[g] + (float)LAG;
        if (__any(move)) {
          const float m_new = move ? mx : m_run[g];
          const float alpha = exp2_fast(m_run[g] - m_new);   // 0 on the first tile
          m_run[g] = m_new;
          l_run[g] *= alpha;
#pragma unroll
          for (int db = 0; db < DB; ++db) acc[db][g] *= alpha;
        }
        // m_run is finite from the first visited tile on: key 0 is visible to every row
        const float m_use = m_run[g];
        float lsum = 0.f;
#pragma unroll
        for (int x = 0; x < KB; ++x) {
          float p[16];
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            p[i] = exp2_fast(__builtin_fmaf(s[x][g][i], scale_log2, -m_use));
            lsum += p[i];
          }
#pragma unroll
          for (int h2 = 0; h2 < 2; ++h2)
            pf[g][x][h2] = u32x4{pack_bf16x2(p[8 * h2 + 0], p[8 * h2 + 1]),
                                 pack_bf16x2(p[8 * h2 + 2], p[8 * h2 + 3]),
                                 pack_bf16x2(p[8 * h2 + 4], p[8 * h2 + 5]),
                                 pack_bf16x2(p[8 * h2 + 6], p[8 * h2 + 7])};
        }
        l_run[g] += lsum;
      }

      // O^T[db][g] += V^T P^T: slab h2 of key block x holds keys
      // x*32 + 16*h2 + {4*hi..4*hi+3, 8+4*hi..8+4*hi+3} in this lane's k slots
#pragma unroll
      for (int x = 0; x < KB; ++x)
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2) {
          const int g0 = x * 8 + h2 * 4 + hi;  // 4-key group of k slots 0..3
#pragma unroll
          for (int db = 0; db < DB; ++db) {
            const int dcol = db * 32 + l32;
            const u32x2 lo = *(const u32x2*)(vb + g0 * C::kVGroupBytes + dcol * 8);
            const u32x2 up = *(const u32x2*)(vb + (g0 + 2) * C::kVGroupBytes + dcol * 8);
            const u32x4 a = u32x4{lo[0], lo[1], up[0], up[1]};
#pragma unroll
            for (int g = 0; g < QG; ++g) acc[db][g] = mfma_32x32x16(a, pf[g][x][h2], acc[db][g]);
          }
        }
    }

    if (j + 1 < n_tiles) store_tile(buf ^ 1);
    __syncthreads();
  }

  if (!wave_live) return;
  // ---- epilogue: O = acc / l, LSE = (m + log2 l) * ln 2 ----
#pragma unroll
  for (int g = 0; g < QG; ++g) {
    const float lt = l_run[g] + swap_halves(l_run[g]);
    const float inv = 1.f / lt;
    const int q = qw0 + g * 32 + l32;
    if (q < N) {
      uint16_t* orow = O + ((size_t)bh * N + q) * D;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int d0 = db * 32 + 8 * r + 4 * hi;
          const f32x16& a = acc[db][g];
          *(u32x2*)(orow + d0) = u32x2{pack_bf16x2(a[4 * r + 0] * inv, a[4 * r + 1] * inv),
                                       pack_bf16x2(a[4 * r + 2] * inv, a[4 * r + 3] * inv)};
        }
      if (hi == 0) LSE[(size_t)bh * N + q] = (m_run[g] + log2_fast(lt)) * kLn2;
    }
  }
}

template <int D, int QG, int BC, int NW, int WPE, bool CAUSAL, int LAG = 0>
hipError_t launch_fwd_t(const FwdArgs& a, hipStream_t stream) {
  using C = FwdCfg<D, QG, BC, NW>;
  const int n_qb = (a.N + C::kBR - 1) / C::kBR;
  const int BH = a.B * a.Hq;
  const long long grid = (long long)BH * n_qb;
  if (grid > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  auto kern = attn_fwd_kernel<D, QG, BC, NW, WPE, CAUSAL, LAG>;
  // more than 64 KB of dynamic LDS has to be allowed once per kernel instance
  static const hipError_t attr = hipFuncSetAttribute(
      (const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, C::kLdsBytes);
  if (attr != hipSuccess) return attr;
  const int xcd_remap = (BH % 8 == 0) ? 1 : 0;
  hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(C::kThreads), C::kLdsBytes, stream,
                     (const uint16_t*)a.q, (const uint16_t*)a.k, (const uint16_t*)a.v,
                     (uint16_t*)a.o, a.lse, a.N, BH, a.Hq, a.Hkv, a.Hq / a.Hkv, n_qb,
                     a.scale * kLog2e, xcd_remap);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd(const FwdArgs& a, hipStream_t stream) {
  // 8 waves x 32 rows = 256 query rows per workgroup, 128-key tiles (135 KB
  // of double-buffered LDS: one workgroup per CU), two waves per SIMD (<= 256
  // registers each) so one wave's softmax VALU work overlaps the other's MFMAs.
  constexpr int QG = 1, BC = 128, NW = 8, WPE = 2;
  if (a.d == 128)
    return a.causal ? launch_fwd_t<128, QG, BC, NW, WPE, true>(a, stream)
                    : launch_fwd_t<128, QG, BC, NW, WPE, false>(a, stream);
  return a.causal ? launch_fwd_t<64, QG, BC, NW, WPE, true>(a, stream)
                  : launch_fwd_t<64, QG, BC, NW, WPE, false>(a, stream);
}

}  // namespace attn
