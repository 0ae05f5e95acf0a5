// Layout-table formats shared by the host layout compiler and the kernels.
#pragma once

#include <cstdint>

namespace bsmm {

// Output-block groups (32x32 blocks): kGroupOut consecutive output blocks per group;
// each group-table entry is kGroupInts int32 (contraction block, presence mask, the
// kGroupOut ids, two zeros).
constexpr int kGroupOut = 8;
constexpr int kGroupInts = 12;
constexpr int kGroupMaxSteps = 1024;   // longest group walk the group kernels take

// Weight-gradient tiles (32x32 blocks): kTileSide x kTileSide blocks of the layout;
// a tile holding at least kTileMin blocks is computed as one unit, the other blocks
// go to row groups.
constexpr int kTileSide = 8;
constexpr int kTileMin = 16;
constexpr int kTileWaves = 8;   // a tile's blocks are split over 8 waves, in order
// Tiles are processed in super-blocks of kSuperRows x kSuperCols tiles (layout.cpp).
constexpr int kSuperRows = 4;
constexpr int kSuperCols = 8;

// Weight-gradient tiles of small blocks (8x8 and 16x16): 256 x 256 features of the
// layout, cut into 16 x 16 quads of 16 x 16 features (one 16x16 block, or 2 x 2 blocks
// of 8x8).  Per tile with any block: (first x feature, first dy feature, index of its
// first id, 0); per tile 16 quad-row masks (bit j: quad column j holds a block); per
// tile 256 quads x (1 or 4) ids, row-major quads, blocks within a quad row-major, -1
// where absent.
constexpr int kSmallTileFeat = 256;
constexpr int kSmallQuads = 16;

}  // namespace bsmm
