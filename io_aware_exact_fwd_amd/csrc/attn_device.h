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

// Value held by lane (l ^ 32): the partner that holds the other half of a
// row in the 32x32 C layout.
__device__ __forceinline__ float swap_halves(float x) {
  return __shfl_xor(x, 32, 64);
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

#include "attn_layout.h"

namespace attn {

// Wait for every outstanding memory operation of this wave (global loads,
// including the direct-to-LDS ones, and LDS reads).
__device__ __forceinline__ void wait_all_memory() { __builtin_amdgcn_s_waitcnt(0); }

// Direct 16-byte global -> LDS loads of a ROWS x D tile (swizzled layout of
// attn_layout.h) starting at global row row0 of `g` ([N, D] rows).  One
// instruction moves 1 KB; the NW waves of the workgroup split the tile's
// segments.  Rows at or past N repeat row N-1 (finite data; every kernel
// masks those rows or keys out).
template <int D, int ROWS, int NW>
__device__ __forceinline__ void direct_tile_load(const uint16_t* __restrict__ g, int row0, int N,
                                                 unsigned char* tile, int wave, int lane) {
  constexpr int kSegs = ROWS * 2 * D / 1024;
  static_assert(kSegs * 1024 == ROWS * 2 * D, "tile is a whole number of 1 KB segments");
#pragma unroll
  for (int k = 0; k < (kSegs + NW - 1) / NW; ++k) {
    const int seg = k * NW + wave;
    if (kSegs % NW == 0 || seg < kSegs) {
      int r, c;
      layout::direct_src<D>(seg * 1024 + lane * 16, r, c);
      const int gr = min(row0 + r, N - 1);
      const uint16_t* src = g + (size_t)gr * D + c * 8;
      __builtin_amdgcn_global_load_lds((const void __attribute__((address_space(1)))*)src,
                                       (void __attribute__((address_space(3)))*)(tile + seg * 1024),
                                       16, 0, 0);
    }
  }
}

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
