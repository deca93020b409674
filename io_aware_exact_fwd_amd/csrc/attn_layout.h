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

// ---------------------------------------------------------------------------
// 8-bit (E4M3) tiles, d = 128.  A row of 128 bytes is exactly a D = 64 bf16
// row, and the tile uses that layout: 16-byte chunks, swz<64>, filled by the
// same direct loads (direct_src<64>).  Its two access patterns are conflict
// free as well:
//   * row fragments of the 32x32x64 8-bit MFMA: lane l reads row row0 + l%32,
//     bytes 64m + 32*(l/32) .. +31 (two chunks, two ds_read_b128);
//   * transposed fragments (ds_read_b64_tr_b8; per group of 16 lanes, byte j
//     of lane i is byte (i & 7) of the 8 bytes addressed by lane
//     2j + (i >> 3)): a lane receives 8 keys of one d column per read.
// ---------------------------------------------------------------------------

// Byte offset of byte column `col` of row r in an 8-bit tile.
ATTN_HD int f8_off(int r, int col) { return chunk_off<64>(r, col >> 4) + (col & 15); }

// Row fragment, MFMA m (d bytes 64m .. 64m+63), half e of this lane's 32
// bytes: the 16-byte read's offset.
ATTN_HD int f8_row_frag_off(int lane, int row0, int m, int e) {
  return chunk_off<64>(row0 + (lane & 31), 4 * m + 2 * (lane >> 5) + e);
}

// Key (relative to the 64-key pair) that byte b of a lane in lane-half hi
// holds, in both operands of O^T += V^T P^T: bytes 16x + i come from
// accumulator i of the score block x of the pair, whose C-layout row is
// 8(i/4) + 4hi + (i%4).
ATTN_HD int f8_pair_key(int hi, int b) {
  const int x = b >> 4, i = b & 15;
  return 32 * x + 8 * (i >> 2) + 4 * hi + (i & 3);
}

// Transposed fragment of V^T for d block db (columns 32db .. 32db+31) and the
// 64 keys k0 .. k0+63, read t (bytes 8t .. 8t+7 of the lane's operand): the
// address this lane supplies.  In each group of 16 lanes, lane 2j + s points
// at the 8 bytes of row f8_pair_key(hi, 8t + j) starting at column
// 32db + 16(g & 1) + 8s, so lane i of the group receives column
// 32db + 16(g & 1) + i with byte j holding that key.
ATTN_HD int f8_tr_off(int lane, int k0, int db, int t) {
  const int g = lane >> 4, q = lane & 15, j = q >> 1, s = q & 1, hi = g >> 1;
  const int row = k0 + f8_pair_key(hi, 8 * t + j);
  return f8_off(row, 32 * db + 16 * (g & 1) + 8 * s);
}

}  // namespace layout
}  // namespace attn
