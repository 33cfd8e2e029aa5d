// Element order of the fp32 split-K partial tiles written by the matmuls of
// the dense-row paths (forward fallback, backward dense rows).
#pragma once

namespace twell {

// Partial tiles are stored in the accumulators' own order: register i of
// block (bm, bn) of wave w is 64 consecutive floats, one per lane, so every
// store is one contiguous 256-byte write.  These map a tile element
// (row, col) to that position.
// gate / up tiles (8 waves, 128 x 64 wave tiles, NWM = 4, NWN = 2):
__device__ __forceinline__ int gate_up_part_index(int row, int col) {
  const int w = (row >> 7) * 4 + (col >> 6), bm = (row & 127) >> 5, bn = (col & 63) >> 5;
  const int rr = row & 31, i = 4 * (rr >> 3) + (rr & 3), lane = ((rr & 7) >> 2) * 32 + (col & 31);
  return (((w * 4 + bm) * 2 + bn) * 16 + i) * 64 + lane;
}
// down tiles of BN columns (4 waves of 64 rows, 2 x BN/32 blocks):
template <int BN>
__device__ __forceinline__ int down_part_index(int row, int col) {
  constexpr int NB = BN / 32;
  const int w = row >> 6, bm = (row & 63) >> 5, bn = col >> 5;
  const int rr = row & 31, i = 4 * (rr >> 3) + (rr & 3), lane = ((rr & 7) >> 2) * 32 + (col & 31);
  return (((w * 2 + bm) * NB + bn) * 16 + i) * 64 + lane;
}

}  // namespace twell
