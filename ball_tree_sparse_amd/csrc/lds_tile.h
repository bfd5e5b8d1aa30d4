// Row-major bf16 tiles in LDS that serve both row reads and gfx950's
// transposed reads, for the backward passes:
//  * row reads (ds_read_b128): a lane reads 8 consecutive columns of one row;
//  * transposed reads (ds_read_b64_tr_b16): in each 16-lane group, lane l
//    receives element l%4 of the 8-byte runs addressed by lanes l/4, l/4+4,
//    l/4+8, l/4+12, so four rows x 16 columns become 4 rows for each of 16
//    columns.
// Rows inside a 16-row slice come out in the order in which an MFMA C tile
// feeds a B operand (bits 2 and 3 of the row position swapped).
#pragma once
#include "common.h"

namespace bt {

// Element offset of 16-byte piece p of row r in a row-major LDS tile of D
// columns.  Sixteen consecutive rows put piece p in sixteen different bank
// groups, and four consecutive rows starting at a multiple of four cover
// every bank once per 32-column span.
template <int D>
BT_DEV int tile_off(int r, int p) {
  int f;
  if constexpr (D == 32) f = (r >> 2) & 3;
  else f = (((r >> 1) & 1) << 2) | ((r >> 2) & 3);
  return r * D + ((p ^ f) << 3);
}

// Four bf16 of a 16-lane transposed read; p points at this lane's 8-byte
// run in LDS.
BT_DEV s16x4 lds_read_tr16(const uint16_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((BT_LDS_AS s16x4*)p);
}

// A operand X^T[d][rows] of a 16-row slice (rows sl*16 ...) and the 32-column
// block db of a tile: lane L holds d = db*32 + L%32 and the rows 8t + 4*(L/32)
// + e (t = 0, 1; e = 0..3) of the slice, in that element order.
template <int D>
BT_DEV bf16x8 tr_operand(const uint16_t* tile, int sl, int db) {
  const int lane = threadIdx.x & 63, grp = lane >> 4, s = lane & 15;
  const int col = db * 32 + 16 * (grp & 1) + 4 * (s & 3);     // this lane's 4 columns
  const int r0 = sl * 16 + 4 * (grp >> 1) + (s >> 2);
  const s16x4 a = lds_read_tr16(tile + tile_off<D>(r0, col >> 3) + (col & 4));
  const s16x4 b = lds_read_tr16(tile + tile_off<D>(r0 + 8, col >> 3) + (col & 4));
  const s16x8 x = __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8, x);
}

}  // namespace bt
