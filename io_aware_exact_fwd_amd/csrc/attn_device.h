// attn_device.h -- gfx950 (CDNA4) device helpers shared by the attention kernels.
//
// Everything here is written for one target: wave64, bf16 MFMA
// v_mfma_f32_32x32x16_bf16, 160 KB of LDS per CU.  No other architecture is
// compiled or supported.
//
// MFMA 32x32x16 lane layout (D = A*B + C, A is 32x16, B is 16x32):
//   A: lane l holds A[l%32][8*(l/32) .. 8*(l/32)+7]   (8 bf16, one 16-byte value)
//   B: lane l holds B[8*(l/32) .. +7][l%32]
//   C: lane l, accumulator i holds C[8*(i/4) + 4*(l/32) + (i%4)][l%32]
// The kernels only rely on A and B sharing one k<->(lane,slot) map, and on
// the C layout above; the C layout is checked on the device by the test suite.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attn {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// One 32x32x16 bf16 MFMA with fp32 accumulation.
__device__ __forceinline__ f32x16 mfma_32x32x16(u32x4 a, u32x4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// Two fp32 -> packed bf16 pair, round to nearest even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2 v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

// 2^x on the transcendental unit (v_exp_f32); 2^-inf = 0.
__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ float log2_fast(float x) { return __builtin_amdgcn_logf(x); }

// max / sum of x over the lane pair (l, l^32) -- the two halves of a column
// in the 32x32 C layout.  v_permlane32_swap exchanges the upper half of its
// first operand with the lower half of its second; with x in both, one of the
// two results holds the partner's value and the other x itself, so the
// symmetric op of the two results is the pair's max / sum in every lane.
__device__ __forceinline__ float pair_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ u32x4 zero4() { return u32x4{0u, 0u, 0u, 0u}; }

}  // namespace attn

namespace attn {

// Eight fp32 values -> one bf16x8 MFMA operand (round to nearest even).
__device__ __forceinline__ u32x4 pack8(const float* p) {
  return u32x4{pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3]), pack_bf16x2(p[4], p[5]),
               pack_bf16x2(p[6], p[7])};
}

__device__ __forceinline__ float bf16_lo(uint32_t x) { return __uint_as_float(x << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t x) { return __uint_as_float(x & 0xFFFF0000u); }

}  // namespace attn

#include "attn_launch.h"
#include "attn_layout.h"

namespace attn {

// The rows one (batch, head) pair owns.  Fixed length ([B, H, N, d]): rows
// (b H + h) N .. + N - 1.  Packed ([H, T, d], see Packing): rows h T + cu[b]
// .. h T + cu[b+1] - 1.  Boundaries are clamped to [0, T] and lengths to N,
// so a malformed table cannot move an access outside the tensors (its rows
// are then simply not all computed).  b is uniform, so the two boundary reads
// are scalar loads.
struct SeqSpan {
  int start;  // first row of the sequence within each head's rows (0: fixed length)
  int len;    // rows (queries and keys) of the sequence
  // first row of head h (of H) for batch b
  __device__ __forceinline__ size_t row0(const Packing& p, int N, int b, int h, int H) const {
    return p.cu ? (size_t)h * p.T + start : ((size_t)b * H + h) * N;
  }
};

__device__ __forceinline__ SeqSpan seq_span(const Packing& p, int N, int b) {
  if (!p.cu) return SeqSpan{0, N};
  const int c0 = min(max(p.cu[b], 0), p.T);
  const int c1 = min(max(p.cu[b + 1], c0), p.T);
  return SeqSpan{c0, min(c1 - c0, N)};
}

// Row distance between consecutive heads of one batch (N, or T when packed).
__device__ __forceinline__ size_t head_stride(const Packing& p, int N) {
  return p.cu ? (size_t)p.T : (size_t)N;
}

// ---------------------------------------------------------------------------
// Work units of a packed batch, heaviest first.
//
// A grid sized for B sequences of the longest length holds many workgroups
// whose block lies past the end of a shorter sequence.  Instead of mapping
// the workgroup index to (sequence, head, block) arithmetically and returning
// from those, a packed launch enumerates only the real units: sequence b owns
// n_b = ceil(len_b / BS) blocks of BS rows, and block k of it gets a level L
// (0 <= L < n_b) that grows with its cost (the caller picks L = k or
// L = n_b - 1 - k).  Units are ordered by level, highest first, then by
// sequence, then by head (Hn per sequence); with
//     C(L) = Hn * sum_b max(0, n_b - L)
// units at levels >= L, unit w sits at the largest level L with C(L) > w, and
// its rank among that level's units is w - C(L+1).  Every workgroup index past
// C(0) is empty and comes after all real ones.  Each wave evaluates this
// itself, with the block counts of up to kMaxPackedSeqs sequences held in its
// lanes (b = lane + 64 j); the lengths are clamped exactly as seq_span does.
// ---------------------------------------------------------------------------
static_assert(kMaxPackedSeqs % 64 == 0, "whole waves of sequences");

// Sum / max of v over the 64 lanes of a wave (every lane active), returned in
// a scalar register: four DPP steps give every lane its 16-lane row's result
// (swap neighbours, swap pairs, mirror each half row, mirror the row), and the
// four rows are combined through readlane.
__device__ __forceinline__ int wave_sum_i32(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0xB1, 0xF, 0xF, true);    // quad_perm [1,0,3,2]
  v += __builtin_amdgcn_update_dpp(0, v, 0x4E, 0xF, 0xF, true);    // quad_perm [2,3,0,1]
  v += __builtin_amdgcn_update_dpp(0, v, 0x141, 0xF, 0xF, true);   // row_half_mirror
  v += __builtin_amdgcn_update_dpp(0, v, 0x140, 0xF, 0xF, true);   // row_mirror
  return __builtin_amdgcn_readlane(v, 0) + __builtin_amdgcn_readlane(v, 16) +
         __builtin_amdgcn_readlane(v, 32) + __builtin_amdgcn_readlane(v, 48);
}
__device__ __forceinline__ int wave_max_i32(int v) {
  v = max(v, __builtin_amdgcn_update_dpp(0, v, 0xB1, 0xF, 0xF, true));
  v = max(v, __builtin_amdgcn_update_dpp(0, v, 0x4E, 0xF, 0xF, true));
  v = max(v, __builtin_amdgcn_update_dpp(0, v, 0x141, 0xF, 0xF, true));
  v = max(v, __builtin_amdgcn_update_dpp(0, v, 0x140, 0xF, 0xF, true));
  return max(max(__builtin_amdgcn_readlane(v, 0), __builtin_amdgcn_readlane(v, 16)),
             max(__builtin_amdgcn_readlane(v, 32), __builtin_amdgcn_readlane(v, 48)));
}

struct PackedUnits {
  int n[kMaxPackedSeqs / 64];   // blocks of sequence lane + 64 j (0 past B)
  int nmax;                     // most blocks of any sequence (wave-uniform)

  // All boundary loads are issued before any is used (indices past B are
  // clamped to B, a valid entry, and their counts zeroed), so the table costs
  // one memory round trip.
  __device__ __forceinline__ void init(const Packing& p, int B, int Nmax, int BS) {
    const int lane = threadIdx.x & 63;
    int lo[kMaxPackedSeqs / 64], hi[kMaxPackedSeqs / 64];
#pragma unroll
    for (int j = 0; j < kMaxPackedSeqs / 64; ++j) {
      const int b = min(lane + 64 * j, B);
      lo[j] = p.cu[b];
      hi[j] = p.cu[min(b + 1, B)];
    }
    int m = 0;
#pragma unroll
    for (int j = 0; j < kMaxPackedSeqs / 64; ++j) {
      const int c0 = min(max(lo[j], 0), p.T);
      const int c1 = min(max(hi[j], c0), p.T);
      const int len = min(c1 - c0, Nmax);
      n[j] = lane + 64 * j < B ? (len + BS - 1) / BS : 0;
      m = max(m, n[j]);
    }
    nmax = wave_max_i32(m);
  }
  // units at levels >= L (wave-uniform)
  __device__ __forceinline__ long long at_or_above(int L, int Hn) const {
    int s = 0;
#pragma unroll
    for (int j = 0; j < kMaxPackedSeqs / 64; ++j) s += max(0, n[j] - L);
    return (long long)wave_sum_i32(s) * Hn;
  }
  // Unit w: false when w is past the last unit; else its sequence, head and level.
  __device__ __forceinline__ bool unit(long long w, int Hn, int& b, int& h, int& level) const {
    if (w >= at_or_above(0, Hn)) return false;
    int lo = 0, hi = nmax - 1;   // at_or_above(lo) > w throughout
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (at_or_above(mid, Hn) > w) lo = mid;
      else hi = mid - 1;
    }
    const long long r = w - at_or_above(lo + 1, Hn);
    const int rank = (int)(r / Hn);
    h = (int)(r - (long long)rank * Hn);
    level = lo;
    // the rank-th sequence (in index order) with more than lo blocks
    int seen = 0;
    b = -1;
#pragma unroll
    for (int j = 0; j < kMaxPackedSeqs / 64; ++j) {
      const unsigned long long m = __ballot(n[j] > lo);
      const int c = __popcll(m);
      if (b < 0 && rank < seen + c) {
        unsigned long long mm = m;
        for (int t = seen; t < rank; ++t) mm &= mm - 1;   // drop the lower set bits
        b = 64 * j + __builtin_ctzll(mm);
      }
      seen += c;
    }
    b = __builtin_amdgcn_readfirstlane(b);
    h = __builtin_amdgcn_readfirstlane(h);
    level = __builtin_amdgcn_readfirstlane(level);
    return true;
  }
};

// Instruction classes for __builtin_amdgcn_sched_group_barrier.
constexpr int kSchedMfma = 0x008;
constexpr int kSchedDsRead = 0x100;

// Wait for every outstanding memory operation of this wave (global loads,
// including the direct-to-LDS ones, and LDS reads).
__device__ __forceinline__ void wait_all_memory() { __builtin_amdgcn_s_waitcnt(0); }

// Workgroup barrier for tiles filled by direct loads.  Each wave first waits
// until at most N of its vector-memory operations are outstanding (they
// complete in issue order, so every direct load but the N most recent has
// written LDS) and all its LDS operations are done; then s_barrier.  Unlike
// __syncthreads() this does not wait for *every* outstanding load, so a
// prefetch issued before the barrier stays in flight across it.  The empty
// asm statements keep the compiler from moving memory accesses across.
// s_waitcnt immediate on gfx9: vmcnt[3:0] in bits 3:0, vmcnt[5:4] in bits
// 15:14, expcnt in bits 6:4 (7 = no wait), lgkmcnt in bits 11:8.
template <int N>
__device__ __forceinline__ void barrier_vmem_at_most() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (0 << 8));
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Direct 16-byte global -> LDS loads of a ROWS x D tile (swizzled layout of
// attn_layout.h): one global_load_lds_dwordx4 moves 1 KB (lane i's 16 bytes
// land at LDS base + 16 i), and the NW waves of the workgroup split the tile's
// segments.  Rows at or past N repeat row N-1 (finite data; every kernel masks
// those rows or keys out).
//
// The loads are issued from inline asm with a wave-uniform SGPR base and a
// 32-bit VGPR byte offset.  Two reasons: the per-lane part of each segment's
// offset is a single loop-invariant VGPR (not a 64-bit address per segment),
// and the compiler's wait-count pass does not see an LDS DMA in flight --
// when it does, it drains every outstanding LDS read (lgkmcnt(0)) before each
// MFMA that consumes one, which serialises the LDS latency.  The asm has no
// register outputs (the data goes to LDS), so nothing in flight can land in a
// reused register; the one consequence is that the compiler never waits for
// these loads, so every kernel waits for them itself (wait_all_memory() or
// barrier_vmem_at_most<N>()) before the barrier that publishes the tile.
// Byte offsets stay below 2^32 because N * D < 2^31 is checked on the host.
template <int D, int ROWS, int NW>
struct TileLoader {
  static constexpr int kSegs = ROWS * 2 * D / 1024;
  static constexpr int kPer = (kSegs + NW - 1) / NW;   // segments per wave
  static constexpr int kRowBytes = 2 * D;
  static constexpr int kRowShift = D == 128 ? 8 : 7;
  static_assert(kSegs * 1024 == ROWS * 2 * D, "tile is a whole number of 1 KB segments");
  static_assert((1 << kRowShift) == kRowBytes, "row size");
  unsigned rc[kPer];   // this lane's (row << kRowShift) | (chunk * 16) in each segment

  __device__ __forceinline__ void init(int wave, int lane) {
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
      int r, c;
      layout::direct_src<D>((k * NW + wave) * 1024 + lane * 16, r, c);
      rc[k] = ((unsigned)r << kRowShift) | (unsigned)(c * 16);
    }
  }
  // Rows row0 .. row0+ROWS-1 of the [N, D] matrix at g into `tile`.
  __device__ __forceinline__ void load(const uint16_t* g, int row0, int N, unsigned char* tile,
                                       int wave) const {
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
      const int seg = k * NW + wave;
      if (kSegs % NW == 0 || seg < kSegs) {
        const unsigned row = min((unsigned)row0 + (rc[k] >> kRowShift), (unsigned)(N - 1));
        const unsigned voff = (row << kRowShift) | (rc[k] & (kRowBytes - 1));
        const unsigned lds = (unsigned)(uintptr_t)(tile + seg * 1024);
        asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2"
                     :
                     : "s"(__builtin_amdgcn_readfirstlane(lds)), "v"(voff), "s"(g)
                     : "memory", "m0");
      }
    }
  }
};

// Row fragment (A or B operand): lane l gets row row0 + l%32, columns
// 16*slab + 8*(l/32) .. +7 of a swizzled tile.
template <int D>
__device__ __forceinline__ u32x4 row_frag(const unsigned char* tile, int lane, int row0, int slab) {
  return *(const u32x4*)(tile + layout::row_frag_off<D>(lane, row0, slab));
}

// Transposed A operand from a swizzled tile (two ds_read_b64_tr_b16): lane l
// gets column col0 + l%32; slots 0..3 = rows row0 + 4*(l/32) + 0..3, slots
// 4..7 = rows row0 + 8 + 4*(l/32) + 0..3.  row0 is a multiple of 16, col0 of 32.
template <int D>
__device__ __forceinline__ u32x4 tr_frag(const unsigned char* tile, int lane, int row0, int col0) {
  typedef short i16x4 __attribute__((ext_vector_type(4)));
  typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
  const i16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_i16x4*)(tile + layout::tr_frag_off<D>(lane, row0, col0, 0)));
  const i16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_i16x4*)(tile + layout::tr_frag_off<D>(lane, row0, col0, 1)));
  const u32x2 ua = __builtin_bit_cast(u32x2, a), ub = __builtin_bit_cast(u32x2, b);
  return u32x4{ua[0], ua[1], ub[0], ub[1]};
}

}  // namespace attn
