// attn_decode.hip -- forward for decoding against a KV cache (N_q << N_k) on
// gfx950: the key axis is split across workgroups and the partial results are
// merged by their log-sum-exp.
//
// Setting (page "从“算力黑洞”到“效率革命”：大模型Attention的演进之路", §1 and §3,
// and page "6.1 … 長上下文擴展技術", §1.5): each generated token's queries
// attend to the whole cached K/V history, whose size grows with the context,
// so the work is a streaming read of K and V with very few query rows.  The
// queries are the last N_q positions of the sequence (query i at position
// i + N_k - N_q; the causal mask and the window are taken between positions).
// Splitting the keys into chunks and merging per-chunk (O, LSE) pairs is the
// identity of the online softmax (page "6.1 …", §2.2): with LSE_c the
// log-sum-exp of chunk c, LSE = ln sum_c exp(LSE_c) and
// O = sum_c exp(LSE_c - LSE) O_c.
//
// gfx950 mapping
//   * one workgroup = one (batch, K/V head, block of 32 query rows, key chunk);
//     the rows are the G query heads of the group times the N_q queries, so a
//     K/V byte is read once per group, not once per query head (the work is
//     HBM-bound: 4 d FLOP per (row, key) against 4 d bytes of K and V per key);
//   * four waves hold the same 32 rows (Q^T as MFMA B operands in registers)
//     and split every 128-key tile into four 32-key blocks: S^T = K Q^T and
//     O^T += V^T P^T on v_mfma_f32_32x32x16_bf16 with the same tile layout,
//     direct loads and fragment reads as the main forward; each wave keeps its
//     own running max, sum and accumulator;
//   * the tiles stream through an LDS ring of up to 128 KB (two 64 KB stages
//     for d = 128, four 32 KB stages for d = 64): the next tiles' loads are in
//     flight while one tile is computed, and each wave waits only for the
//     oldest (vmcnt counts the newer tiles' loads).  Measured on d = 128:
//     deeper rings of smaller tiles, or two workgroups per CU, read no faster;
//     the kernel streams K and V at the rate a plain read kernel reaches;
//   * at the end the waves' partials meet in LDS and are merged, and the
//     chunk's normalised O (fp32) and LSE are written to the workspace;
//   * a second kernel merges the chunks of every row into O (bf16) and LSE.
#include "attn_device.h"
#include "attn_launch.h"

#include <mutex>

namespace attn {

// The per-chunk partials of attn_fwd_decode_static, for callers that cannot
// allocate: a fixed array in device memory that the library holds for the
// life of the process, one copy per GPU (each GPU's copy has its own address,
// looked up once per device by decode_static_scratch below).  Host code never
// passes this name to a kernel -- on the host it is only a stand-in for the
// symbol -- but the device address that lookup returns.
static __device__ __align__(256) float scratch[kDecodeStaticScratchBytes / sizeof(float)];

namespace {

// The shared tile loader (attn_device.h) with non-temporal loads: each K/V
// byte of a decode launch is read exactly once, by one workgroup, so the
// loads need not stay in the caches.  Measured on the chip: a read-only
// probe over 2 GiB reaches 6.99 TB/s with contiguous per-workgroup chunks and
// non-temporal loads against 6.0-6.2 TB/s with cached ones, and this kernel
// 7.04 against 5.89 TB/s at decode-32K (outputs bitwise unchanged).
template <int D, int ROWS, int NW>
struct StreamLoader : TileLoader<D, ROWS, NW> {
  using Base = TileLoader<D, ROWS, NW>;
  __device__ __forceinline__ void load(const uint16_t* g, int row0, int N, unsigned char* tile,
                                       int wave) const {
#pragma unroll
    for (int k = 0; k < Base::kPer; ++k) {
      const int seg = k * NW + wave;
      if (Base::kSegs % NW == 0 || seg < Base::kSegs) {
        const unsigned row = min((unsigned)row0 + (this->rc[k] >> Base::kRowShift), (unsigned)(N - 1));
        const unsigned voff = (row << Base::kRowShift) | (this->rc[k] & (Base::kRowBytes - 1));
        const unsigned lds = (unsigned)(uintptr_t)(tile + seg * 1024);
        asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2 nt"
                     :
                     : "s"(__builtin_amdgcn_readfirstlane(lds)), "v"(voff), "s"(g)
                     : "memory", "m0");
      }
    }
  }
};

constexpr int kDecNW = 4;            // waves per workgroup, 32 keys of each tile each
constexpr int kDecBC = 32 * kDecNW;  // keys per tile
constexpr int kDecRows = 32;         // query rows per workgroup
constexpr int kDecLdsBudget = 128 * 1024;
constexpr int kDecMaxStages = 4;

template <int D>
struct DecCfg {
  static constexpr int kTile = kDecBC * 2 * D;      // bytes of one K or V tile
  // tiles resident in the LDS ring
  static constexpr int kStages = kDecLdsBudget / (2 * kTile) < kDecMaxStages
                                     ? kDecLdsBudget / (2 * kTile) : kDecMaxStages;
  static constexpr int kLdsBytes = kStages * 2 * kTile;
  // direct loads one wave issues per tile (K and V)
  static constexpr int kLoadsPerTile = 2 * TileLoader<D, kDecBC, kDecNW>::kPer;
  static_assert(kStages >= 2, "at least double buffering");
  static_assert(TileLoader<D, kDecBC, kDecNW>::kSegs % kDecNW == 0, "every wave issues kPer loads");
  static_assert((kStages - 2) * kLoadsPerTile < 64, "vmcnt range");
  // the merge reuses the tile memory: per wave m and l (32 rows each) and the
  // O^T accumulator (D x 32 fp32)
  static constexpr int kMergeBytes = kDecNW * (2 * kDecRows + D * kDecRows) * 4;
  static_assert(kMergeBytes <= kLdsBytes, "merge fits in the tile memory");
};

// Barrier once this wave has at most `later` tiles' loads outstanding
// (PER loads per tile, later <= MAXL).
template <int PER, int MAXL>
__device__ __forceinline__ void barrier_tiles_at_most(int later) {
  if constexpr (MAXL > 0) {
    if (later >= MAXL) {
      barrier_vmem_at_most<MAXL * PER>();
      return;
    }
    barrier_tiles_at_most<PER, MAXL - 1>(later);
  } else {
    barrier_vmem_at_most<0>();
  }
}

// Workspace layout: o_part [splits][B*Hq*Nq][D] fp32, then lse_part
// [splits][B*Hq*Nq] fp32.
template <int D, bool CAUSAL, bool LOCAL>
__global__ __attribute__((amdgpu_flat_work_group_size(kDecNW * 64, kDecNW * 64),
                          amdgpu_waves_per_eu(2, 2))) void attn_decode_split_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
    const uint16_t* __restrict__ V, float* __restrict__ o_part, float* __restrict__ lse_part,
    int Hq, int Hkv, int G, int Nq, int Nk, int n_rb, int n_bhk, int chunk, int rows_total,
    float scale_log2, int window) {
  using C = DecCfg<D>;
  constexpr int DS = D / 16;
  constexpr int DB = D / 32;

  extern __shared__ __attribute__((aligned(1024))) unsigned char smem[];
  const int tid = threadIdx.x, lane = tid & 63, l32 = lane & 31, hi = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

  // workgroup -> (split, batch*K/V head, row block); row blocks of one chunk
  // are adjacent so they share the chunk's K/V in L2
  int w = blockIdx.x;
  const int rb = w % n_rb;
  w /= n_rb;
  const int bhk = w % n_bhk;
  const int split = w / n_bhk;
  const int b = bhk / Hkv, hk = bhk - b * Hkv;
  (void)Hkv;
  const uint16_t* Kp = K + ((size_t)b * Hkv + hk) * Nk * D;
  const uint16_t* Vp = V + ((size_t)b * Hkv + hk) * Nk * D;

  // this lane's query row: r = rb*32 + l%32 -> (head hk*G + r / Nq, query r % Nq)
  const int R = G * Nq;
  const int r = rb * kDecRows + l32;
  const bool row_ok = r < R;
  const int g = row_ok ? r / Nq : 0;
  const int qi = row_ok ? r - g * Nq : 0;
  const int h = hk * G + g;
  const int pos = qi + Nk - Nq;                      // sequence position of the query
  const size_t row_id = ((size_t)b * Hq + h) * Nq + qi;

  u32x4 qf[DS];
#pragma unroll
  for (int sl = 0; sl < DS; ++sl)
    qf[sl] = row_ok ? *(const u32x4*)(Q + row_id * D + sl * 16 + 8 * hi) : zero4();
  // Take the Q loads' wait here, once: left to the compiler it lands at the
  // first MFMA inside the key loop as a full vmcnt(0), which would also drain
  // the K/V tiles in flight on every iteration.
#pragma unroll
  for (int sl = 0; sl < DS; ++sl) asm volatile("" ::"v"(qf[sl]));

  // key range of the chunk, narrowed with a window to what the earliest query
  // (position N_k - N_q) can see
  int k_begin = split * chunk;
  const int k_end = min(Nk, k_begin + chunk);
  if (LOCAL) k_begin = max(k_begin, Nk - Nq - window);
  const int j_first = k_begin / kDecBC;
  const int n_tiles = k_end > k_begin ? (k_end + kDecBC - 1) / kDecBC : j_first;

  StreamLoader<D, kDecBC, kDecNW> ldr;
  ldr.init(wave, lane);
  auto stage = [&](int j) { return smem + (j % C::kStages) * 2 * C::kTile; };
  auto issue_tile = [&](int j) {
    unsigned char* kt = stage(j);
    ldr.load(Kp, j * kDecBC, Nk, kt, wave);
    ldr.load(Vp, j * kDecBC, Nk, kt + C::kTile, wave);
  };

  f32x16 acc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) acc[db] = f32x16{};
  float m_run = -INFINITY, l_run = 0.f;

  for (int j = j_first; j < min(n_tiles, j_first + C::kStages - 1); ++j) issue_tile(j);
  for (int j = j_first; j < n_tiles; ++j) {
    // tile j has landed once at most the loads of the tiles issued after it
    // are outstanding; the barrier then also orders the last reads of stage
    // (j - 1) before its reuse by tile j + kStages - 1
    barrier_tiles_at_most<C::kLoadsPerTile, C::kStages - 2>(min(n_tiles - 1 - j, C::kStages - 2));
    if (j + C::kStages - 1 < n_tiles) issue_tile(j + C::kStages - 1);
    const int kw = j * kDecBC + wave * 32;         // this wave's 32 keys
    if (kw < k_end && kw + 31 >= k_begin) {
      const unsigned char* kt = stage(j);
      const unsigned char* vt = kt + C::kTile;
      f32x16 s = f32x16{};
#pragma unroll
      for (int sl = 0; sl < DS; ++sl) s = mfma_32x32x16(row_frag<D>(kt, lane, wave * 32, sl), qf[sl], s);
      // mask: keys outside the chunk or past N_k, past the row's position
      // (causal), outside its window, and padding rows
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int key = kw + 8 * (i >> 2) + 4 * hi + (i & 3);
        const bool out = !row_ok || key < k_begin || key >= k_end || (CAUSAL && key > pos) ||
                         (LOCAL && (key < pos - window || (!CAUSAL && key > pos + window)));
        if (out) s[i] = -INFINITY;
      }
      float mx = -INFINITY;
#pragma unroll
      for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[i]);
      mx = pair_max(mx) * scale_log2;
      const bool move = mx > m_run;
      if (__any(move)) {
        const float m_new = move ? mx : m_run;
        const float alpha = move ? exp2_fast(m_run - m_new) : 1.f;
        m_run = m_new;
        l_run *= alpha;
#pragma unroll
        for (int db = 0; db < DB; ++db) acc[db] *= alpha;
      }
      const float m_ref = m_run == -INFINITY ? 0.f : m_run;
      float p[16];
      float lsum = 0.f;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        p[i] = exp2_fast(__builtin_fmaf(s[i], scale_log2, -m_ref));
        lsum += p[i];
      }
      l_run += lsum;
      const u32x4 pb0 = pack8(p), pb1 = pack8(p + 8);
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        acc[db] = mfma_32x32x16(tr_frag<D>(vt, lane, wave * 32, db * 32), pb0, acc[db]);
        acc[db] = mfma_32x32x16(tr_frag<D>(vt, lane, wave * 32 + 16, db * 32), pb1, acc[db]);
      }
    }
  }
  wait_all_memory();
  __syncthreads();

  // ---- merge the waves' partials in LDS ----
  const float l_tot = pair_sum(l_run);
  float* m_l = (float*)smem;                        // [wave][32] running max (log2 units)
  float* l_l = m_l + kDecNW * kDecRows;             // [wave][32] sums
  float* a_l = l_l + kDecNW * kDecRows;             // [wave][db][i][lane] accumulators
  if (hi == 0) {
    m_l[wave * kDecRows + l32] = m_run;
    l_l[wave * kDecRows + l32] = l_tot;
  }
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) a_l[((wave * DB + db) * 16 + i) * 64 + lane] = acc[db][i];
  __syncthreads();

  // wave w combines d blocks w, w + kDecNW, ...
  float M = -INFINITY;
#pragma unroll
  for (int v = 0; v < kDecNW; ++v) M = fmaxf(M, m_l[v * kDecRows + l32]);
  float wt[kDecNW];
  float L = 0.f;
#pragma unroll
  for (int v = 0; v < kDecNW; ++v) {
    const float mv = m_l[v * kDecRows + l32];
    wt[v] = mv == -INFINITY ? 0.f : exp2_fast(mv - M);
    L += wt[v] * l_l[v * kDecRows + l32];
  }
  const float inv = L > 0.f ? 1.f / L : 0.f;
  const size_t out_row = (size_t)split * rows_total + row_id;
  for (int db = wave; db < DB; db += kDecNW) {
    f32x16 o = f32x16{};
#pragma unroll
    for (int v = 0; v < kDecNW; ++v)
#pragma unroll
      for (int i = 0; i < 16; ++i) o[i] += wt[v] * a_l[((v * DB + db) * 16 + i) * 64 + lane];
    if (row_ok) {
      float* orow = o_part + out_row * D;
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const int d0 = db * 32 + 8 * rr + 4 * hi;
        *(f32x4*)(orow + d0) = f32x4{o[4 * rr] * inv, o[4 * rr + 1] * inv, o[4 * rr + 2] * inv,
                                     o[4 * rr + 3] * inv};
      }
    }
  }
  if (row_ok && wave == 0 && hi == 0)
    lse_part[out_row] = L > 0.f ? (M + log2_fast(L)) * kLn2 : -INFINITY;
}

// One wave per query row: LSE = ln sum_c exp(LSE_c), O = sum_c exp(LSE_c - LSE) O_c.
template <int D>
__global__ __launch_bounds__(256) void attn_decode_merge_kernel(
    const float* __restrict__ o_part, const float* __restrict__ lse_part, uint16_t* __restrict__ O,
    float* __restrict__ LSE, int rows_total, int n_splits) {
  constexpr int PER = D / 64;   // elements of the row per lane
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= rows_total) return;
  float mx = -INFINITY;
  for (int c = 0; c < n_splits; ++c) mx = fmaxf(mx, lse_part[(size_t)c * rows_total + row]);
  float sum = 0.f;
  float o[PER];
#pragma unroll
  for (int e = 0; e < PER; ++e) o[e] = 0.f;
  for (int c = 0; c < n_splits; ++c) {
    const float lc = lse_part[(size_t)c * rows_total + row];
    if (lc == -INFINITY) continue;
    const float wgt = __expf(lc - mx);
    sum += wgt;
    const float* src = o_part + ((size_t)c * rows_total + row) * D + lane * PER;
#pragma unroll
    for (int e = 0; e < PER; ++e) o[e] += wgt * src[e];
  }
  const float inv = 1.f / sum;   // every row sees at least its own position's key
  uint16_t* dst = O + (size_t)row * D + lane * PER;
  if (PER == 1) {
    dst[0] = (uint16_t)(pack_bf16x2(o[0] * inv, 0.f) & 0xFFFFu);
  } else {
#pragma unroll
    for (int e = 0; e + 1 < PER; e += 2) *(uint32_t*)(dst + e) = pack_bf16x2(o[e] * inv, o[e + 1] * inv);
  }
  if (lane == 0) LSE[row] = mx + __logf(sum);
}

template <int D, bool CAUSAL, bool LOCAL>
hipError_t launch_decode_t(const DecodeArgs& a, hipStream_t stream) {
  using C = DecCfg<D>;
  const int G = a.Hq / a.Hkv;
  const int n_rb = (G * a.Nq + kDecRows - 1) / kDecRows;
  const int rows_total = a.B * a.Hq * a.Nq;
  const int n_bhk = a.B * a.Hkv;
  const long long grid = (long long)n_bhk * n_rb * a.n_splits;
  if (grid > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  auto kern = attn_decode_split_kernel<D, CAUSAL, LOCAL>;
  static std::atomic<uint64_t> lds_set{0};
  const hipError_t attr = allow_lds_on_device((const void*)kern, C::kLdsBytes, lds_set);
  if (attr != hipSuccess) return attr;
  float* o_part = a.workspace;
  float* lse_part = o_part + (size_t)a.n_splits * rows_total * D;
  hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(kDecNW * 64), C::kLdsBytes, stream,
                     (const uint16_t*)a.q, (const uint16_t*)a.k, (const uint16_t*)a.v, o_part,
                     lse_part, a.Hq, a.Hkv, G, a.Nq, a.Nk, n_rb, n_bhk, a.chunk, rows_total,
                     a.scale * kLog2e, a.window);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(attn_decode_merge_kernel<D>, dim3((rows_total + 3) / 4), dim3(256), 0, stream,
                     o_part, lse_part, (uint16_t*)a.o, a.lse, rows_total, a.n_splits);
  return hipGetLastError();
}

}  // namespace

int decode_splits(int B, int Hq, int Hkv, int Nq, int Nk, int requested, int* chunk) {
  const int G = Hq / Hkv;
  const int n_rb = (G * Nq + kDecRows - 1) / kDecRows;
  const int n_tiles = (Nk + kDecBC - 1) / kDecBC;
  int s = requested;
  if (s <= 0) {
    // about two rounds of workgroups over the 256 CUs (one resident per CU:
    // 128 KB of LDS), at least one tile each
    const long long base = (long long)B * Hkv * n_rb;
    s = (int)((512 + base - 1) / base);
  }
  s = max(1, min(s, n_tiles));
  const int tiles_per = (n_tiles + s - 1) / s;
  s = (n_tiles + tiles_per - 1) / tiles_per;        // no empty chunk
  *chunk = tiles_per * kDecBC;
  return s;
}

hipError_t decode_static_scratch(float** out) {
  constexpr int kMaxDev = 64;
  static std::atomic<float*> addr[kMaxDev];
  static std::mutex lookup;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDev) return hipErrorInvalidDevice;
  float* p = addr[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> g(lookup);
    p = addr[dev].load(std::memory_order_acquire);
    if (!p) {
      void* a = nullptr;
      e = hipGetSymbolAddress(&a, HIP_SYMBOL(scratch));   // with this device current
      if (e != hipSuccess) return e;
      if (!a) return hipErrorInvalidSymbol;
      p = (float*)a;
      addr[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return hipSuccess;
}

hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream) {
  const bool local = a.window >= 0 && a.window < a.Nk - 1;
  if (a.d == 128) {
    if (local) return a.causal ? launch_decode_t<128, true, true>(a, stream) : launch_decode_t<128, false, true>(a, stream);
    return a.causal ? launch_decode_t<128, true, false>(a, stream) : launch_decode_t<128, false, false>(a, stream);
  }
  if (local) return a.causal ? launch_decode_t<64, true, true>(a, stream) : launch_decode_t<64, false, true>(a, stream);
  return a.causal ? launch_decode_t<64, true, false>(a, stream) : launch_decode_t<64, false, false>(a, stream);
}

}  // namespace attn
