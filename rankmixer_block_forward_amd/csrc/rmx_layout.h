// Index maps of the operand layouts and of the Sparse-MoE tile table.  Plain integer
// arithmetic, compiled for the kernels (RMX_HD = __host__ __device__) and by a host-only
// check (RMX_HD defined empty) that runs every map over whole buffers under
// AddressSanitizer.
#pragma once
#include <stddef.h>
#include <stdint.h>

#ifndef RMX_HD
#define RMX_HD __host__ __device__
#endif

namespace rmx {

// Rows of one group of a matrix in the packed operand layout (blocks of 256 rows).
RMX_HD inline int64_t pk_rows(int64_t rows) { return (rows + 255) / 256 * 256; }

// ---- Packed operand layout of a bf16 matrix [rows, K], K % 32 == 0: blocks of 256 rows x
// 32 columns (16 KB), ordered [row block][K step]; inside a block row r holds its four
// 16-byte chunks, chunk c at position c ^ pk_swz(r).  A K step of a 256-row block is then
// one contiguous 16 KB that lands in LDS as is, already swizzled for conflict-free 16-byte
// fragment reads.  Rows are padded to a multiple of 256 (pk_rows).
RMX_HD inline int pk_swz(int r) { return ((r >> 1) ^ (r >> 2)) & 3; }
// element offset of (row, col) with col % 8 == 0: the start of a 16-byte chunk
RMX_HD inline size_t pk_off(int row, int col, int K) {
  const int rb = row >> 8, r = row & 255, kt = col >> 5, c = (col >> 3) & 3;
  return ((size_t(rb) * size_t(K >> 5) + size_t(kt)) << 13) + size_t(r << 5) + size_t((c ^ pk_swz(r)) << 3);
}
// Byte offset, inside one 16 KB K step of a 256-row block, of row r's 16-byte chunk c: where
// the matrix-core loops read their fragments (bf16: k = 8 c .. 8 c + 7 of the step; MXFP8:
// k = 16 c .. 16 c + 15).
RMX_HD inline uint32_t pk_lds_off(int r, int c) { return uint32_t(r * 64 + ((c ^ pk_swz(r)) << 4)); }
// Loads that gather row-major rows into that layout: K step piece p (0..15, 16 rows of
// 64 bytes) is filled by one wave, lane l writing 16 bytes at p * 1024 + 16 l, which is
// slot l % 4 of tile row 16 p + l / 4 and so takes chunk (l % 4) ^ pk_swz(row) of the row.
RMX_HD inline int pk_gather_row(int piece, int lane) { return 16 * piece + (lane >> 2); }
RMX_HD inline int pk_gather_chunk(int row, int lane) { return (lane & 3) ^ pk_swz(row); }

// ---- MXFP8 operands (OCP Microscaling Formats (MX) Specification v1.0, FP8 E4M3 elements,
// one E8M0 power-of-two scale per 32 consecutive values along K).  A matrix [rows, K]
// (K % 64 == 0, rows padded to a multiple of 256) is stored as blocks of 256 rows x 64 K
// (16 KB), ordered [row block][K step]; inside a block row r holds four 16-byte chunks of
// 16 consecutive k, chunk c at position c ^ pk_swz(r).  Its scales are 512 bytes per block,
// laid out so that lane l of the wave that owns rows 128 h .. 128 h + 127 of the block finds
// the scales of rows 128 h + 32 i + (l % 32), i = 0..3, for the 32-value half l / 32 of the
// K step in one 32-bit word, byte i: the scale operand of the MFMA.
// byte offset of (row, k), k % 16 == 0 (the start of a chunk; + 8 for its second half)
RMX_HD inline size_t mx_off(int row, int k, int K) {
  const int rb = row >> 8, r = row & 255, kt = k >> 6, c = (k >> 4) & 3;
  return ((size_t(rb) * size_t(K >> 6) + size_t(kt)) << 14) + size_t(r << 6) + size_t((c ^ pk_swz(r)) << 4);
}
// byte offset of the scale of (row, 32-value block kb)
RMX_HD inline size_t mx_scale_off(int row, int kb, int K) {
  const int rb = row >> 8, r = row & 255;
  return ((size_t(rb) * size_t(K >> 6) + size_t(kb >> 1)) << 9) + size_t((r >> 7) << 8) +
         size_t((((kb & 1) << 5) | (r & 31)) << 2) + size_t((r >> 5) & 3);
}

// ---- Tile order of the dense products.
constexpr int NUM_XCD = 8;    // MI355X: 8 accelerator complex dies, each with its own L2
constexpr int TILE_BAND = 8;  // row tiles per band of the dense tile order
// Workgroups are dealt to the XCDs round-robin.  Remap so that each XCD receives a
// contiguous range of tile indices (a bijection of [0, nblocks)), so that the tiles
// resident on one XCD at a time share their weight panels and A rows in its L2.
RMX_HD inline int xcd_remap(int bid, int nblocks) {
  const int xcd = bid % NUM_XCD, pos = bid / NUM_XCD;
  const int base = nblocks / NUM_XCD, extra = nblocks % NUM_XCD;
  return xcd * base + (xcd < extra ? xcd : extra) + pos;
}
// Tile rem (0 <= rem < nMt * nNt) of one group: bands of TILE_BAND row tiles (the last band
// may be shorter), N tiles in order inside a band, row tiles fastest.
RMX_HD inline void band_tile(int rem, int nMt, int nNt, int& mt, int& nt) {
  const int band = rem / (TILE_BAND * nNt);
  const int in_band = rem - band * TILE_BAND * nNt;
  const int left = nMt - band * TILE_BAND;
  const int bm = TILE_BAND < left ? TILE_BAND : left;
  nt = in_band / bm;
  mt = band * TILE_BAND + (in_band - nt * bm);
}

// ---- Sparse-MoE tile table.  Group g (token t, expert e) holds tile_start[g + 1] -
// tile_start[g] row tiles (its active rows rounded up to whole tiles; none for an empty
// group).  The grouped products number their tiles group by group, inside a group N tile
// nt outer and row tile mt inner:
//   tile = tile_start[g] * nNt + nt * (tile_start[g + 1] - tile_start[g]) + mt.
// moe_tile_locate inverts that map for 0 <= tile < tile_start[G] * nNt: g is the one group
// with tile_start[g] * nNt <= tile < tile_start[g + 1] * nNt (binary search; empty groups,
// whose range is empty, are never chosen).
RMX_HD inline void moe_tile_locate(const int* tile_start, int G, int nNt, int tile, int& g, int& mt, int& nt) {
  int glo = 0, ghi = G;  // invariant: tile_start[glo] * nNt <= tile < tile_start[ghi] * nNt
  while (ghi - glo > 1) {
    const int mid = (glo + ghi) >> 1;
    if (tile_start[mid] * nNt <= tile) glo = mid; else ghi = mid;
  }
  g = glo;
  const int mtiles = tile_start[g + 1] - tile_start[g];
  const int local = tile - tile_start[g] * nNt;
  nt = local / mtiles;
  mt = local - nt * mtiles;
}
// The persistent grouped products give XCD x the contiguous tiles [lo, hi) (consecutive
// tiles share a group's weights, which then stay in that XCD's L2); its workgroups stride
// through them.
RMX_HD inline void moe_xcd_span(int total, int xcd, int num_xcd, int& lo, int& hi) {
  const int chunk = (total + num_xcd - 1) / num_xcd;
  lo = xcd * chunk;
  hi = lo + chunk < total ? lo + chunk : total;
}

}  // namespace rmx
