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
// Blocks outside the dense tiles: row groups of at most this many ids.
constexpr int kRestGroup = 2;
constexpr int kSuperRows = 4;
constexpr int kSuperCols = 8;

// Weight-gradient tiles of small blocks (8x8 and 16x16): 256 x 256 features of the
// layout, cut into 16 x 16 quads of 16 x 16 features (one 16x16 block, or 2 x 2 blocks
// of 8x8).  Per tile with any block: (first x feature, first dy feature, index of its
// first id, 0); per tile and wave (16 waves) kSmallPlanInts ints: the number of quads
// of the wave's quad row that hold a block, their quad columns in ascending order (one
// byte each, four to an int from the low byte, zero past the end), the quad row, then
// zeros (rows are dealt to waves so that waves w, w + 4, w + 8, w + 12 together hold
// about a quarter of the tile's quads); per tile 256 quads x (1 or 4) ids, row-major
// quads, blocks within a quad row-major, -1 where absent.
constexpr int kSmallTileFeat = 256;
constexpr int kSmallQuads = 16;
constexpr int kSmallPlanInts = 8;

}  // namespace bsmm
