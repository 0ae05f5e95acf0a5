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

}  // namespace bsmm
