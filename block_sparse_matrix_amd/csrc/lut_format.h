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

}  // namespace bsmm
