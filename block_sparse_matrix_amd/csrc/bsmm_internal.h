// Internal declarations shared by the host-side layout compiler, the C ABI and the
// kernel launchers of libbsmm.  Not installed; the public interface is include/bsmm.h.
#pragma once

#include <cstdint>
#include <map>
#include <mutex>
#include <string>
#include <vector>

#include "bsmm.h"
#include "lut_format.h"

namespace bsmm {

constexpr int32_t kRecCap = 1024;   // entries kept inline in a list record

// Host look-up tables compiled from a 0/1 block layout.
//
// Block ids number the layout's nonzeros in row-major order (the reading of
// BlocksparseMatMul.w_shape / block_coord in the kiteco/blocksparse README, "API
// Documentation" › blocksparse.matmul).  Every table below is derived from that
// numbering:
//   coords   (c, k) of each id, id order.
//   colptr / colent   fprop lists: for output block k, entries (c, id) with L[c][k]=1,
//                     ascending c.  colptr has S+1 offsets into colent (pairs).
//   rowptr / rowent   bprop lists: for input block c, entries (k, id), ascending k.
//   colorder / roworder  list indices by descending length (ties: ascending index);
//                     kernels hand the longest lists out first for load balance.
struct HostLut {
    int64_t R = 0, S = 0, nnz = 0;
    int b = 0, fa = 1;
    std::vector<int32_t> coords;
    std::vector<int32_t> colptr, colent;
    std::vector<int32_t> rowptr, rowent;
    std::vector<int32_t> colorder, roworder;
    // Per list in processing order (colorder / roworder): (list, start, length, 0);
    // one 16-byte scalar load gives a workgroup everything it needs to find its list.
    std::vector<int32_t> colwork, rowwork;
    // Per list in processing order a fixed-stride record: the work descriptor (list,
    // start, length, 0), then the first min(length, kRecCap) entries (blk, id).  A workgroup fetches its header and
    // first entries with one load instead of a descriptor load followed by a list load.
    std::vector<int32_t> colrec, rowrec;
    int32_t col_rsi = 0, row_rsi = 0;   // record stride in int32
    // Weight-gradient groups: runs of up to 8 consecutive ids within one layout row,
    // in id order: (first id, count, row, 0).
    std::vector<int32_t> ugroups;
    int32_t max_col = 0, max_row = 0;   // longest fprop / bprop list
    // Output-block groups (32x32 blocks only): kGroupOut consecutive output blocks
    // share one walk over the contraction blocks.  fprop: groups of block columns k,
    // walking c ascending; bprop: groups of block rows c, walking k ascending.  Entry
    // (kGroupInts int32): contraction block, mask of the group's blocks present there
    // (bit j: output block kGroupOut*g + j), the ids of those blocks (0 where absent),
    // 0, 0.  gptr holds groups+1 entry offsets.
    std::vector<int32_t> cgptr, cgent, rgptr, rgent;
    // Weight-gradient tiles (32x32 blocks only): utiles (r0, c0, blocks, first) per
    // tile with at least kTileMin blocks, in super-block order (kSuperRows x kSuperCols
    // tiles, row-major within and between super-blocks); utblk holds, per such
    // tile from index first, the ids of its 8x8 positions row-major (-1 where absent);
    // the other blocks in urest row groups (first, count, row, 1), whose ids are
    // urids[first .. first+count-1].
    std::vector<int32_t> utiles, utblk, urest, urids;
    // Small-block weight-gradient tiles (8x8 and 16x16 blocks; format in lut_format.h):
    // stiles (4 per tile), stplan (16 x 8 per tile), stids (256 or 1024 per tile).
    std::vector<int32_t> stiles, stplan, stids;
};

// Builds every table above.  Pure host code: never touches HIP.  Returns false with a
// message on invalid input (checked before anything is built).
bool compile_layout(const uint8_t* layout, int64_t R, int64_t S, int b, int fa, HostLut& out,
                    std::string& err);

// Device copy of the tables: one allocation, the arrays laid out back to back.
struct DeviceLut {
    void* base = nullptr;
    const int32_t* coords = nullptr;   // int2 per id
    const int32_t* colptr = nullptr;
    const int32_t* colent = nullptr;   // int2 per entry
    const int32_t* rowptr = nullptr;
    const int32_t* rowent = nullptr;
    const int32_t* colorder = nullptr;
    const int32_t* roworder = nullptr;
    const int32_t* colwork = nullptr;
    const int32_t* rowwork = nullptr;
    const int32_t* ugroups = nullptr;
    int32_t nugroups = 0;
    const int32_t* colrec = nullptr;
    const int32_t* rowrec = nullptr;
    const int32_t* cgptr = nullptr;
    const int32_t* cgent = nullptr;
    const int32_t* rgptr = nullptr;
    const int32_t* rgent = nullptr;
    const int32_t* utiles = nullptr;
    const int32_t* utblk = nullptr;
    const int32_t* urest = nullptr;
    const int32_t* urids = nullptr;
    int32_t nutiles = 0, nurest = 0;
    const int32_t* stiles = nullptr;
    const int32_t* stplan = nullptr;
    const int32_t* stids = nullptr;
    int32_t nstiles = 0;
};

}  // namespace bsmm

struct bsmm_plan {
    bsmm::HostLut lut;
    int force[3] = {0, 0, 0};   // forced kernel kind per pass (fprop, bprop, updat), 0 = automatic
    std::mutex mu;
    std::vector<char> image;              // the tables packed as on the device (source of the uploads)
    std::map<int, bsmm::DeviceLut> dev;   // per HIP device ordinal
};

// SparseProj: a one-to-one map of nproj projected features into nhidden dense ones
// (kiteco/blocksparse README, "API Documentation" › blocksparse.matmul › SparseProj).
// lut[p] is the dense feature of projected feature p; inv[h] the projected feature of
// dense feature h, or -1.  Immutable after create; the device copy (lut then inv, one
// allocation) is made per device on first use.
struct bsmm_proj_plan {
    int64_t nhidden = 0, nproj = 0;
    std::vector<int32_t> lut, inv;
    std::mutex mu;
    std::vector<int32_t> image;    // lut followed by inv (source of the uploads)
    std::map<int, int32_t*> dev;   // per HIP device ordinal: lut (nproj) followed by inv (nhidden)
};

// BlocksparseConv: channel-list blocks and the convolution geometry (kiteco/blocksparse
// README, "API Documentation" › blocksparse.conv › BlocksparseConv).  cidx / kidx hold
// each block's Bc input and Bk output channels; kptr/kent list, per output channel, its
// (block, position in the block's output list) pairs in block order (fprop), cptr/cent
// the same per input channel (bprop).  Immutable after create; one device copy of the
// tables per device, made on first use.
struct bsmm_conv_plan {
    int64_t C = 0, K = 0;
    int nb = 0, Bc = 0, Bk = 0;
    int TRS[3] = {1, 1, 1}, DHW[3] = {1, 1, 1}, MPQ[3] = {1, 1, 1};
    int st[3] = {1, 1, 1}, dl[3] = {1, 1, 1}, pad[3] = {0, 0, 0};
    std::vector<int32_t> cidx, kidx, kptr, kent, cptr, cent;
    // Matrix-core grouping per pass (0 fprop: blocks by output channel list; 1 bprop: by
    // input channel list): group offsets, block ids, and the channels no block writes.
    // gok[p] is false when two groups share a channel (the direct kernels run then).
    std::vector<int32_t> gptr[2], gblk[2], zch[2];
    bool gok[2] = {false, false};
    std::mutex mu;
    std::vector<int32_t> image;    // all the arrays above back to back (source of the uploads)
    std::map<int, int32_t*> dev;   // per HIP device: the same, on the device
};
