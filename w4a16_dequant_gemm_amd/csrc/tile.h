// Tile order of the MFMA GEMM kernels (W4A16 prefill, W8A8 product).
#pragma once

namespace w4a16 {

// Output tile of hardware block `bid` for a TM x TN tile grid.  Block b runs on XCD b % 8;
// the blocks of one XCD take a contiguous range of tile numbers (the grid is padded to a
// multiple of 8), and tile numbers run down kTileGroup tile rows before moving one tile
// column, so the tiles an XCD holds at once form a compact block that shares activation
// and weight panels in that XCD's L2.  Returns false for the padding blocks.
constexpr int kTileGroup = 4;

__device__ __forceinline__ bool xcd_tile(int bid, int TM, int TN, int& mt, int& nt) {
    const int tiles = TM * TN;
    const int per_xcd = (tiles + 7) / 8;
    const int t = (bid % 8) * per_xcd + bid / 8;
    if (t >= tiles) return false;
    const int group = t / (kTileGroup * TN);
    const int first = group * kTileGroup;
    const int gm = TM - first < kTileGroup ? TM - first : kTileGroup;   // rows in this (last) group
    const int r = t - first * TN;
    mt = first + r % gm;
    nt = r / gm;
    return true;
}

}  // namespace w4a16
