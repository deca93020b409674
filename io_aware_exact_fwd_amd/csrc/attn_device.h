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

// Interleave 4 rows of 8 bf16 (one 16-byte value each) into 8 columns of
// 4 bf16: out[j] = {r0[j], r1[j], r2[j], r3[j]} packed in 8 bytes.  Used to
// store a K/V tile "4 keys per d" so that a transposed MFMA operand is two
// 8-byte LDS reads.
__device__ __forceinline__ void interleave4x8(const u32x4 (&r)[4], u32x2 (&out)[8]) {
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const uint32_t a = r[0][w], b = r[1][w], c = r[2][w], d = r[3][w];
    // even column 2w: low halves; odd column 2w+1: high halves
    out[2 * w][0] = (a & 0xFFFFu) | (b << 16);
    out[2 * w][1] = (c & 0xFFFFu) | (d << 16);
    out[2 * w + 1][0] = (a >> 16) | (b & 0xFFFF0000u);
    out[2 * w + 1][1] = (c >> 16) | (d & 0xFFFF0000u);
  }
}

}  // namespace attn

namespace attn {

// Stages an R x D bf16 tile (rows row0.., rows >= N read as zero) from global
// memory through registers into LDS, in units of 4 rows x 8 columns per
// thread.  store() can write two LDS copies from one load:
//   row-major, rows `stride` bytes apart (16 bytes of padding per row keep
//   16-byte reads of 32 consecutive rows free of bank conflicts), and
//   "4 rows per column": for each group of 4 rows, D entries of 8 bytes
//   holding rows 4g..4g+3 of one column, so a transposed MFMA operand is two
//   8-byte reads.
template <int D, int R, int NT>
struct TileStager {
  static constexpr int kUnits = (R / 4) * (D / 8);
  static constexpr int kPer = (kUnits + NT - 1) / NT;
  static constexpr int kRowStride = D * 2 + 16;   // bytes, row-major copy
  static constexpr int kGroupBytes = D * 8;       // bytes, one 4-row group
  static constexpr int kRowMajorBytes = R * kRowStride;
  static constexpr int kInterleavedBytes = (R / 4) * kGroupBytes;
  u32x4 reg[kPer][4];

  __device__ __forceinline__ void load(const uint16_t* __restrict__ base, int row0, int N, int tid) {
#pragma unroll
    for (int it = 0; it < kPer; ++it) {
      const int u = it * NT + tid;
      if (kUnits % NT == 0 || u < kUnits) {
        const int g = u / (D / 8), c = u % (D / 8);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int row = row0 + 4 * g + r;
          reg[it][r] = row < N ? *(const u32x4*)(base + (size_t)row * D + c * 8) : zero4();
        }
      }
    }
  }

  template <bool ROWMAJOR, bool INTERLEAVED>
  __device__ __forceinline__ void store(unsigned char* rm, unsigned char* il, int tid) const {
#pragma unroll
    for (int it = 0; it < kPer; ++it) {
      const int u = it * NT + tid;
      if (kUnits % NT == 0 || u < kUnits) {
        const int g = u / (D / 8), c = u % (D / 8);
        if (ROWMAJOR) {
#pragma unroll
          for (int r = 0; r < 4; ++r) *(u32x4*)(rm + (4 * g + r) * kRowStride + c * 16) = reg[it][r];
        }
        if (INTERLEAVED) {
          u32x2 t[8];
          interleave4x8(reg[it], t);
          unsigned char* dst = il + g * kGroupBytes + c * 64;
#pragma unroll
          for (int j = 0; j < 4; ++j)
            *(u32x4*)(dst + 16 * j) = u32x4{t[2 * j][0], t[2 * j][1], t[2 * j + 1][0], t[2 * j + 1][1]};
        }
      }
    }
  }
};

// A operand (lane: row l%32, 8 consecutive columns) read from a row-major
// LDS copy: rows row0 + l%32, columns 16*slab + 8*(l/32) .. +7.
template <int STRIDE>
__device__ __forceinline__ u32x4 lds_row_frag(const unsigned char* rm, int row0, int slab, int l32, int hi) {
  return *(const u32x4*)(rm + (row0 + l32) * STRIDE + (slab * 16 + 8 * hi) * 2);
}

// Transposed A operand from a "4 rows per column" LDS copy: column `col`,
// k slots 0..3 = rows 4*g0 .. 4*g0+3, k slots 4..7 = rows 4*(g0+2) .. +3.
template <int GROUP_BYTES>
__device__ __forceinline__ u32x4 lds_tr_frag(const unsigned char* il, int g0, int col) {
  const u32x2 lo = *(const u32x2*)(il + g0 * GROUP_BYTES + col * 8);
  const u32x2 up = *(const u32x2*)(il + (g0 + 2) * GROUP_BYTES + col * 8);
  return u32x4{lo[0], lo[1], up[0], up[1]};
}

// Eight fp32 values -> one bf16x8 MFMA operand (round to nearest even).
__device__ __forceinline__ u32x4 pack8(const float* p) {
  return u32x4{pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3]), pack_bf16x2(p[4], p[5]),
               pack_bf16x2(p[6], p[7])};
}

__device__ __forceinline__ float bf16_lo(uint32_t x) { return __uint_as_float(x << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t x) { return __uint_as_float(x & 0xFFFF0000u); }

}  // namespace attn
