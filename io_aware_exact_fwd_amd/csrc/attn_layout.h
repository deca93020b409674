// attn_layout.h -- LDS tile layout and MFMA operand addressing (index math only).
//
// No HIP dependency: the same functions compile for the gfx950 kernels and for
// a host-side checker that simulates every lane of every access pattern.
//
// Tile layout.  A tile holds `rows` rows of D bf16 values (2*D bytes per row,
// no padding), each row cut into D/8 chunks of 16 bytes.  Chunk c of row r is
// stored at position c ^ swz(r) inside the row.  The XOR swizzle is chosen so
// that both access patterns the kernels use are free of LDS bank conflicts
// (64 banks of 4 bytes):
//   * row fragments: 16 lanes read one chunk from each of 16 consecutive rows
//     (ds_read_b128) -- the 16 rows land on 16 distinct chunk positions;
//   * transposed fragments: 32 lanes read 8 bytes each from 4 consecutive rows
//     (4-row aligned) x 32 consecutive columns (ds_read_b64_tr_b16) -- the 4
//     rows land on disjoint 64-byte blocks.
// Rows are filled by 16-byte direct loads (global_load_lds): one instruction
// writes 1 KB of consecutive LDS bytes, lane i writing bytes 16i..16i+15, so
// each lane loads the global chunk that belongs at its LDS position.
//
// Transposed read (ds_read_b64_tr_b16), per group of 16 lanes: every lane
// supplies the address of 4 consecutive bf16; result slot j of lane i is
// element (i & 3) of the 4 values addressed by lane 4j + (i >> 2).
#pragma once

#if defined(__HIPCC__)
#define ATTN_HD __host__ __device__ __forceinline__
#else
#define ATTN_HD inline
#endif

namespace attn {
namespace layout {

// Chunk-position swizzle of row r (value < D/8).
template <int D>
ATTN_HD int swz(int r) {
  static_assert(D == 64 || D == 128, "head dim");
  return D == 128 ? (((r & 3) << 2) | ((r >> 2) & 3))
                  : ((((r >> 1) & 1) << 2) | ((r >> 2) & 3));
}

// Byte offset of chunk c (columns 8c..8c+7) of row r.
template <int D>
ATTN_HD int chunk_off(int r, int c) {
  return r * 2 * D + ((c ^ swz<D>(r)) << 4);
}

// Byte offset of column `col` (any column) of row r.
template <int D>
ATTN_HD int elem_off(int r, int col) {
  return chunk_off<D>(r, col >> 3) + ((col & 7) << 1);
}

// Direct load: the 16 LDS bytes at tile byte b (a multiple of 16) hold global
// row `row` (tile-relative), chunk `chunk`.
template <int D>
ATTN_HD void direct_src(int b, int& row, int& chunk) {
  row = b / (2 * D);
  const int pos = (b % (2 * D)) >> 4;
  chunk = pos ^ swz<D>(row);
}

// Row fragment of a 32x32x16 MFMA operand (A or B: lane l holds row
// row0 + l%32, columns 16*slab + 8*(l/32) .. +7): its byte offset.
template <int D>
ATTN_HD int row_frag_off(int lane, int row0, int slab) {
  return chunk_off<D>(row0 + (lane & 31), 2 * slab + (lane >> 5));
}

// Transposed fragment of a 32x32x16 MFMA A operand whose rows (m) are tile
// columns and whose k index runs over tile rows: lane l receives column
// col0 + l%32, and in slots 0..3 the tile rows row0 + 4*(l/32) + 0..3, in
// slots 4..7 the rows row0 + 8 + 4*(l/32) + 0..3 (half = 0 / 1 selects the
// read for slots 0..3 / 4..7).  Returns the address this lane supplies.
template <int D>
ATTN_HD int tr_frag_off(int lane, int row0, int col0, int half) {
  const int g = lane >> 4, s = lane & 15;
  const int row = row0 + 4 * (g >> 1) + 8 * half + (s >> 2);
  const int col = col0 + 16 * (g & 1) + 4 * (s & 3);
  return elem_off<D>(row, col);
}

}  // namespace layout
}  // namespace attn
