// Kernel argument blocks and host launchers (implemented in kernels.hip).
#pragma once

#include <hip/hip_runtime_api.h>

#include <cstdint>

#include "lut_format.h"

namespace bsmm {

// fprop / bprop: out[:, o-block] = sum over list(o) of in[:, blk-block] . Wop.
struct MMArgs {
    const void* in;        // x (fprop) or dy (bprop), storage dtype
    const void* w;         // (nnz, b, b)
    void* out;             // y (fprop) or dx (bprop)
    const int32_t* work;   // per list, longest first: (output block, start, length, 0)
    const int32_t* ptr;    // nout+1 list offsets (natural order)
    const int32_t* rec;    // per list (processing order): (list, start, len, 0) + first entries
    int32_t rsi;           // record stride, int32
    const int32_t* ent;    // (blk, id) pairs
    int64_t N;             // minibatch
    int32_t fin, fout;     // feature counts of in and out
    int32_t nout;          // number of lists (output blocks)
    int32_t ntiles;        // minibatch tiles (set by the launcher)
    uint32_t in_bytes;     // size of `in`, bytes (< 2^31)
    uint32_t w_bytes;      // size of `w`, bytes (< 2^31)
    const int32_t* gptr;   // output-block groups (32x32 blocks): ngroups+1 offsets
    const int32_t* gent;   // group entries, kGroupInts int32 each
    int32_t ngroups;       // 0: no group table
    int32_t gfill;         // blocks per group entry, percent of kGroupOut
    int32_t gmax;          // most entries in one group
    int32_t force;         // MMKind to use (0: automatic)
    uint32_t rec_bytes;    // size of the record array (`rec`), bytes
    int32_t maxlen;        // longest list
};

// The small-minibatch kernel (rows.hip) takes lists of at most this many entries.
constexpr int kRowsMaxLen = 256;

// Largest tensor the kernels address with 32-bit buffer offsets.
constexpr uint64_t kMaxTensorBytes = 0x7fff0000ull;

constexpr int kMaxGroup = 8;

struct UpArgs {
    uint32_t x_bytes, dy_bytes;   // size of each x_t / dy_t, bytes (< 2^31)
    const void* xs[kMaxGroup];
    const void* dys[kMaxGroup];
    void* dw;
    const int32_t* coords;  // (c, k) per id
    int64_t N;
    int32_t C, K;
    int32_t nnz;
    int32_t G;
    int32_t dwdt;
    int32_t bpw;            // blocks per wave (set by the launcher)
    const int32_t* groups;  // row groups of <= 8 consecutive ids: (first id, count, row, 0)
    int32_t ngroups;
    // 32x32 blocks: dense tiles (r0, c0, blocks, first) with their blocks (row, column in
    // the tile, id, 0), and the remaining blocks in row groups (first, count, row, 1)
    // whose ids are rids[first ..]
    const int32_t* tiles;
    const int32_t* tblk;
    int32_t ntiles;
    const int32_t* rest;
    const int32_t* rids;
    int32_t nrest;
    int32_t force;          // UpKind to use (0: automatic)
    int32_t split;          // tiles: contraction split in this many parts (1: none)
    float* ws;              // tiles with split > 1: fp32 partial sums, split*ntiles*64 blocks
    int32_t nrids;          // blocks outside the tiles (entries of rids)
    int32_t rsplit;         // those blocks' contraction split (1: none, written to dw directly)
    float* rws;             // rsplit > 1: fp32 partial sums, rsplit*nrids blocks, part-major
    int32_t acc;            // 1: add the sum to what dw holds (dW += ...); 0: overwrite
    // 8x8 and 16x16 blocks: small-block tiles (lut_format.h)
    const int32_t* stiles;
    const int32_t* stplan;
    const int32_t* stids;
    int32_t nstiles;
};

// Contraction split of the weight-gradient tiles: enough parts to give ~256 workgroups,
// at most kMaxSplit.  Splits need split*ntiles*64*b*b*4 bytes of workspace.
constexpr int kMaxSplit = 8;
inline int tile_split(int ntiles) {
    if (ntiles <= 0) return 1;
    const int p = 256 / ntiles;
    return p < 1 ? 1 : p > kMaxSplit ? kMaxSplit : p;
}
// Contraction split of the blocks outside the tiles (their row groups are few, a few
// hundred 4-wave workgroups): eight parts, each summed over the step groups in order,
// then the parts in order.  Needs kRestSplit*nrids*b*b*4 more bytes of workspace.
constexpr int kRestSplit = 8;

// Kernel choice of a pass for its arguments (the launchers use the same choice).  A
// forced kind that cannot serve the arguments gives -1.
enum MMKind { MM_N16 = 1, MM_N64, MM_MID, MM_STACK, MM_GROUPS, MM_V_W16, MM_V_STACK1, MM_V_STACK2, MM_N64_W8, MM_ROWS };
enum UpKind { UP_D2B1 = 1, UP_D1B2, UP_ROWS, UP_D4B1, UP_D2B2, UP_D2B4, UP_D2B8, UP_D1B4, UP_TILES, UP_RUNS, UP_STILES };
int mm_kind(const MMArgs& a, int dt, int b, int fa);
const char* mm_kind_name(int kind);
int updat_kind(const UpArgs& a, int dt, int b, int fa);
const char* updat_kind_name(int kind);
int mm_kind_of_name(const char* name);      // 0 if unknown
int updat_kind_of_name(const char* name);

hipError_t launch_mm(const MMArgs& a, int dt, int b, int fa, bool transw, void* stream, int pass);
// 32x32 blocks, 16-bit storage: output-block groups (a.gptr / a.gent / a.ngroups)
hipError_t launch_mm_groups(const MMArgs& a, int dt, int fa, bool transw, void* stream, int pass);
// 32x32 blocks, N <= 64, feature_axis 1, lists of at most kRowsMaxLen entries
hipError_t launch_mm_rows(const MMArgs& a, int dt, bool transw, void* stream, int pass);
hipError_t launch_updat(const UpArgs& a, int dt, int b, int fa, void* stream);
hipError_t launch_identity(void* w, const int32_t* coords, int64_t nnz, int b, int dt, void* stream);

// Layer norm over the feature axis (norm.hip).  Axis 1: x, y (N, C); axis 0: (C, N).
struct LnArgs {
    const void* x;
    void* y;
    const void* dy;
    void* dx;
    const float* g;
    const float* b;
    float* mean;    // forward: written (may be NULL); gradient: read
    float* rstd;
    float* dg;
    float* db;
    float* ws;      // workspace (ln_workspace_bytes)
    int64_t N, C;
    int axis, dt, relu;
    float eps;
    // set by ln_plan
    int vw;         // storage values per load: 16 bytes' worth, or 1
    int nv;         // axis 1: loads per thread per row
    int64_t rpb;    // axis 1 gradient: rows per workgroup
    int nparts;     // gradient: partial dg/db sets in the workspace
    int nchunks;    // axis 0: 128-row chunks
    void *e0, *e1;  // timing events around the launches (or NULL)
};
// Fills the plan fields; -1 if a row (axis 1) is too long for the register-resident
// kernels.  `aligned`: every tensor base is 16-byte aligned.
int ln_plan(LnArgs& a, bool grad, bool aligned);
size_t ln_workspace_bytes(int64_t N, int64_t C, int axis, bool grad);   // any plan fits
hipError_t launch_layer_norm(const LnArgs& a, bool grad, void* stream);
hipError_t launch_ln_zero_params(float* dg, float* db, int64_t C, void* stream);   // dg = db = 0

// Weight normalisation per output feature over the stored blocks (wnorm.hip).
struct WnArgs {
    const void* w;          // (nnz, b, b), w_dt
    const void* dy;         // gradient: upstream gradient of the output, dy_dt
    void* out;              // forward: normalised weights (out_dt); gradient: dW (float32)
    const float* gain;      // K = S*b, or NULL (gain 1)
    float* norms;           // forward: K column norms, or NULL
    float* dgain;           // gradient: K, or NULL
    const int32_t* colptr;  // fprop column lists (device layout tables)
    const int32_t* colent;
    int64_t S;
    int b, w_dt, out_dt, dy_dt;
    float eps;
    void *e0, *e1;
};
hipError_t launch_l2_normalize(const WnArgs& a, bool grad, void* stream);

// SparseProj (proj.hip): out[., j] = combine(base[., j], src[., map[j]]) over the output
// features j, for activations (N, features) (fa 1) or (features, N) (fa 0).
enum ProjMode {
    PROJ_GATHER = 0,    // out = src[map]                        (map: lut, out width nproj)
    PROJ_SCATTER,       // out = map >= 0 ? src[map] : 0         (map: inv, out width nhidden)
    PROJ_ADD,           // out = map >= 0 ? base + src[map] : base
    PROJ_MUL,           // out = map >= 0 ? base * src[map] : base
    PROJ_GATHER_MUL     // out = base[map] * src[map]            (map: lut; base and src both dense)
};
struct ProjArgs {
    const void* base;      // ADD, MUL: dense (width wout); GATHER_MUL: dense (width wsrc)
    const void* src;
    void* out;
    const int32_t* map;    // wout entries
    int64_t N, wout, wsrc;
    int mode, fa, dt;
};
hipError_t launch_proj(const ProjArgs& a, void* stream);

// BlocksparseConv (conv.hip).  Activations (N, channels, D, H, W); filter
// (nblocks, Bc, T, R, S, Bk); channel lists and per-channel block lists on the device.
struct ConvArgs {
    const void* a;        // fprop: I; bprop: dO; updat: I
    const void* b;        // fprop / bprop: F; updat: dO
    void* out;            // O, dI (storage dtype) or dF (float32)
    const int32_t* cidx;  // nblocks * Bc input channels
    const int32_t* kidx;  // nblocks * Bk output channels
    const int32_t* lptr;  // fprop: K+1 offsets of kent; bprop: C+1 offsets of cent
    const int32_t* lent;  // (block, position in the block's list) pairs
    int64_t N, C, K;
    int nb, Bc, Bk;
    int T, R, S, D, H, W, M, P, Q;
    int st[3], dl[3], pad[3];
    int dt;
    // Matrix-core path (2-D, stride 1, dilation 1, 16-bit; fprop, and bprop as the
    // transposed convolution): blocks grouped by their output channel list (the
    // pass's output role), the groups' lists disjoint.
    int mfma;             // 1: the matrix-core kernel; 2: the gathering matrix-core kernel
    const int32_t* gptr;  // ngroups+1 offsets into gblk
    const int32_t* gblk;  // block ids of each group, ascending
    int ngroups;
    const int32_t* zch;   // output channels in no block (written as zero), nz of them
    int nz;
    int TH;               // output rows per workgroup
    int cpitch;           // LDS elements per staged channel
    int lds_bytes;
    uint32_t a_bytes;     // size of `a` in bytes when below 2^31 (32-bit buffer offsets), else 0
    uint32_t b_bytes;     // the same for `b` (set for the filter gradient, where it is dO)
    // matrix-core filter gradient: contraction split in nparts parts (fp32 partials in
    // ws, nparts * nblocks*Bc*T*R*S*Bk floats, then their sum in part order); 1: none
    int nparts;
    float* ws;
};
// Parts of the matrix-core filter gradient's contraction for N images (about 16
// workgroups per compute unit, at least 4 steps each, at most 16).
int conv_updat_parts(const ConvArgs& a);
hipError_t launch_conv(const ConvArgs& a, int pass, void* stream);   // pass: 0 fprop, 1 bprop, 2 updat
// LDS layout of the matrix-core conv kernel: fills a.TH, a.cpitch, a.lds_bytes; false
// when the shape does not fit it (the direct kernels run instead).
bool conv_mfma_plan(ConvArgs& a, int pass);
// The gathering matrix-core fprop / bprop applies (any geometry and dtype; output
// channels per block 16, 32 or 64; bprop: Bk a multiple of 16 bytes' worth of values;
// the pass's input below 2 GiB); it needs the block groups and a 16-byte aligned filter.
bool conv_gather_ok(const ConvArgs& a, int pass);
// The gathering matrix-core filter gradient applies: every shape the matrix-core filter
// gradient above does not take, with Bc and Bk of 16, 32 or 64 and I and dO below 2 GiB.
bool conv_gather_updat_ok(const ConvArgs& a);
// The filter gradient's matrix-core kernel applies (2-D / 1-D, stride 1, dilation 1,
// 16-bit, Bc and Bk multiples of 16 up to 64); no grouping needed.
bool conv_mfma_updat_ok(const ConvArgs& a);

// Kernel timing hook (api.hip): when profiling is active on this thread, hands out a
// pair of HIP events to record around the next launch of `pass`; else sets both NULL.
void prof_events(int pass, void** start, void** stop);

}  // namespace bsmm
