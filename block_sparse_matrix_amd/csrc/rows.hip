// fprop and bprop for small minibatches (N <= 64) with 32x32 blocks and feature_axis 1.
//
//   fprop  y[:, k-block]  = sum over c with L[c][k]=1 of x[:, c-block]  . W[id(c,k)]
//   bprop  dx[:, c-block] = sum over k with L[c][k]=1 of dy[:, k-block] . W[id(c,k)]^T
// (kiteco/blocksparse README, "API Documentation" › blocksparse.matmul ›
// BlocksparseMatMul.__call__; the README's usage example is hidden 4096, block 32 and
// a minibatch of 64.)
//
// At this size the weight stream is the work.  A workgroup (4 waves, one per SIMD)
// owns one output block's list and one 32-row minibatch tile; its waves take the list's
// entries w, w + 4, w + 8, ... (all of a wave's entries come from the list's record in
// one load per lane, so the weight and activation loads depend on one load level only)
// and add their partial tiles in wave order through LDS, so results are
// bit-reproducible.  The two minibatch tiles of a list run on one XCD: the second
// tile's weight reads hit that XCD's L2, and each weight block crosses HBM once.  Each
// wave keeps two list entries of loads in flight: deeper rings were measured slower
// (the loads in flight across an XCD's 128 waves then outgrow its 4 MB L2).
//
// Operand fragments (matrix-core steps on 16x16 tiles, D[m][n] = sum_k A[m][k] B[k][n],
// lane l = 16 g + r holding A[m = r][k = g..], B[k = g..][n = r] and D[4 g + v][r]):
//   A  the activations, m = minibatch row (16 per tile), k = the block's contraction
//      index; with feature_axis 1 the contraction index is contiguous, so one 16-byte
//      load per fragment.
//   B  the weight block, n = output feature of the block.  bprop contracts over W's
//      fast index: 16-byte loads.  fprop contracts over W's rows: fp32 takes 8-byte
//      loads of two adjacent outputs (n = r stands for output 2 r + t in tile t), 16-bit
//      storage stages the block in a wave-private LDS tile and reads it back with the
//      transposing LDS read.
//   fp32 uses four 16x16x4 steps per 16 contraction values: lane group g's four values
//   in step u are contraction indices 16 u + 4 g .. 16 u + 4 g + 3, the same map for
//   both operands.  bprop (every dtype) loads the dy rows and the weight rows in row
//   order, four consecutive lanes covering one row's 64 bytes, which the memory path
//   serves several times faster than the fragment order (consecutive lanes on different
//   rows); a lane permutation in registers (ds_bpermute) then forms the fragments (fp32
//   bprop 11 % faster, 16-bit bprop ~5 %; fprop gained nothing from it).
#include <cstdio>
#include <cstdlib>
#include <type_traits>

#include "common.h"

namespace bsmm {

__device__ __forceinline__ u32x2 bload64(rsrc_t r, uint32_t voff, uint32_t soff) {
    return __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, 0));
}

// 16 rows x 64 bytes loaded in row order (lane l: row l / 4, 16-byte chunk l % 4) to the
// fragment order (lane l: row l % 16, chunk l / 16): lane l takes lane 4 (l % 16) + l / 16.
__device__ __forceinline__ u32x4 rows_to_frag(const u32x4& v, int lane) {
    const int src = (4 * (lane & 15) + (lane >> 4)) * 4;
    return u32x4{(uint32_t)__builtin_amdgcn_ds_bpermute(src, (int)v.x), (uint32_t)__builtin_amdgcn_ds_bpermute(src, (int)v.y),
                 (uint32_t)__builtin_amdgcn_ds_bpermute(src, (int)v.z), (uint32_t)__builtin_amdgcn_ds_bpermute(src, (int)v.w)};
}

template <int DT, bool TW> struct RowsCfgT {
    static constexpr bool F32 = DT == BSMM_F32;
    static constexpr int S = F32 ? 4 : 2;
    static constexpr bool WTR = !TW && !F32;     // 16-bit fprop: weight through LDS
    static constexpr bool W8 = F32 && !TW;       // fp32 fprop: 8-byte weight loads
    static constexpr int U = F32 ? 2 : 1;        // activation loads per tile and block
    static constexpr int WR = F32 ? (TW ? 4 : 8) : 2;
    static constexpr int WPITCH = 40;            // staged weight row pitch, 16-bit elements
    static constexpr bool XROW = TW;             // bprop: activation rows loaded in row order
    static constexpr bool WROW = !F32 && TW;             // 16-bit bprop weight rows too
    // output feature (within the block) of lane row r in output tile t
    static __device__ __forceinline__ int qmap(int t, int r) { return W8 ? 2 * r + t : 16 * t + r; }
};

template <int DT, bool TW, int MT> struct RowsSlot;
template <int DT, bool TW, int MT> struct RowsSlot {
    using C = RowsCfgT<DT, TW>;
    u32x4 x[MT * C::U];
    typename std::conditional<C::W8, u32x2, u32x4>::type w[C::WR];
};

// One list entry's contribution: acc[mt][t] += the activation tile mt . the weight
// block's output tile t (fragment maps at the top of the file).
template <int DT, bool TW, int MT>
__device__ __forceinline__ void rows_compute(f32x4 (&acc)[MT][2], const RowsSlot<DT, TW, MT>& sl,
                                              BSMM_LDS uint16_t* wt, int lane) {
    using C = RowsCfgT<DT, TW>;
    if constexpr (C::F32) {
        u32x4 xf[MT * 2];   // activation fragments
#pragma unroll
        for (int i = 0; i < MT * 2; i++) xf[i] = C::XROW ? rows_to_frag(sl.x[i], lane) : sl.x[i];
        typename std::conditional<C::W8, u32x2, u32x4>::type wf[C::WR];
#pragma unroll
        for (int i = 0; i < C::WR; i++) {
            if constexpr (C::W8)
                wf[i] = sl.w[i];
            else
                wf[i] = rows_to_frag(sl.w[i], lane);   // bprop weight rows, loaded in row order
        }
#pragma unroll
        for (int u = 0; u < 2; u++)
#pragma unroll
            for (int v = 0; v < 4; v++)
#pragma unroll
                for (int mt = 0; mt < MT; mt++)
#pragma unroll
                    for (int t = 0; t < 2; t++) {
                        const uint32_t av = xf[mt * 2 + u][v];
                        uint32_t bv;
                        if constexpr (C::W8)
                            bv = wf[u * 4 + v][t];
                        else
                            bv = wf[t * 2 + u][v];
                        acc[mt][t] = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(av), __uint_as_float(bv),
                                                                          acc[mt][t], 0, 0, 0);
                    }
    } else {
        u32x4 wf[2];
        if constexpr (C::WTR) {
#pragma unroll
            for (int i = 0; i < 2; i++) {
                const int c = lane + 64 * i;
                lds_store16(wt + (c >> 2) * C::WPITCH + 8 * (c & 3), sl.w[i]);
            }
            wave_lds_order();
            wf[0] = frag_tr16(wt, C::WPITCH, 0, lane);
            wf[1] = frag_tr16(wt, C::WPITCH, 16, lane);
            wave_lds_order();
        } else {
            wf[0] = C::WROW ? rows_to_frag(sl.w[0], lane) : sl.w[0];
            wf[1] = C::WROW ? rows_to_frag(sl.w[1], lane) : sl.w[1];
        }
        u32x4 xf[MT];
#pragma unroll
        for (int mt = 0; mt < MT; mt++) xf[mt] = C::XROW ? rows_to_frag(sl.x[mt], lane) : sl.x[mt];
#pragma unroll
        for (int mt = 0; mt < MT; mt++)
#pragma unroll
            for (int t = 0; t < 2; t++) mma<DT>(acc[mt][t], xf[mt], wf[t]);
    }
}

// rows_kernel: MT 16-row minibatch tiles per workgroup, WAVES waves splitting the
// list, a ring of D list entries per wave.
template <int DT, bool TW, int MT, int WAVES, int D>
__global__ __launch_bounds__(64 * WAVES) void rows_kernel(MMArgs a) {
    using C = RowsCfgT<DT, TW>;
    using Slot = RowsSlot<DT, TW, MT>;
    constexpr int B = 32, S = C::S, U = C::U, WR = C::WR;
    constexpr int TILE = MT * 2 * 64;   // f32x4 per partial tile
    __shared__ __attribute__((aligned(16))) f32x4 red[WAVES > 1 ? WAVES * TILE : 1];
    __shared__ __attribute__((aligned(16))) uint16_t wtl[C::WTR ? WAVES * 32 * C::WPITCH : 8];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int r16 = lane & 15, g = lane >> 4;
    int li, nt;
    wg_decode(blockIdx.x, a.nout, a.ntiles, li, nt);
    if (li < 0) return;   // the whole workgroup leaves together
    // record: header (list, start, length, 0), then the entries (blk, id); this wave's
    // entries (w + WAVES j, lane j) in one 8-byte load per lane, issued with the header
    // load (entries past the list's length read the next record or zeros: never used)
    const rsrc_t rrec = make_rsrc(a.rec, a.rec_bytes);
    const uint32_t rbase = (uint32_t)li * (uint32_t)a.rsi * 4u;
    const u32x2 en = bload64(rrec, (uint32_t)(4 + 2 * (wave + WAVES * lane)) * 4u, rbase);
    const int ex = (int)en.x, ey = (int)en.y;
    const int4 hdr = *reinterpret_cast<const int4*>(a.rec + (int64_t)li * a.rsi);
    const int o = hdr.x, len = hdr.z;
    const int nmine = len > wave ? (len - wave + WAVES - 1) / WAVES : 0;   // <= 64 (launcher)
    const int N = (int)a.N;
    const int n0 = nt * 16 * MT;
    const rsrc_t rin = make_rsrc(a.in, a.in_bytes);
    const rsrc_t rw = make_rsrc(a.w, a.w_bytes);
    BSMM_LDS uint16_t* wt = (BSMM_LDS uint16_t*)wtl + wave * 32 * C::WPITCH;

    uint32_t xo[MT * U];
#pragma unroll
    for (int mt = 0; mt < MT; mt++)
#pragma unroll
        for (int u = 0; u < U; u++) {
            // bprop: row order (lane l: row l / 4, values 16 u + 4 (l % 4) .. or 8 (l % 4) ..);
            // else fragment order (lane l: row l % 16, values 16 u + 4 (l / 16) .. or 8 (l / 16) ..)
            const int n = n0 + 16 * mt + (C::XROW ? lane >> 2 : r16);
            const int k0 = C::F32 ? 16 * u + 4 * (C::XROW ? lane & 3 : g) : 8 * (C::XROW ? lane & 3 : g);
            xo[mt * U + u] = n < N ? ((uint32_t)n * (uint32_t)a.fin + k0) * S : kOffLane;
        }
    uint32_t wo[WR];
#pragma unroll
    for (int i = 0; i < WR; i++) {
        if constexpr (C::W8)
            wo[i] = (uint32_t)(((16 * (i / 4) + 4 * g + i % 4) * B + 2 * r16) * S);
        else if constexpr (C::F32)   // row order, as the activations
            wo[i] = (uint32_t)(((16 * (i / 2) + (lane >> 2)) * B + 16 * (i % 2) + 4 * (lane & 3)) * S);
        else if constexpr (C::WTR)
            wo[i] = (uint32_t)((((lane + 64 * i) >> 2) * B + 8 * ((lane + 64 * i) & 3)) * S);
        else if constexpr (C::WROW)
            wo[i] = (uint32_t)(((16 * i + (lane >> 2)) * B + 8 * (lane & 3)) * S);
        else
            wo[i] = (uint32_t)(((16 * i + r16) * B + 8 * g) * S);
    }

    auto load_slot = [&](Slot& sl, int j) {
        const bool ok = j < nmine;   // wave-uniform
        const int jj = ok ? j : 0;
        const int blk = __builtin_amdgcn_readlane(ex, jj), id = __builtin_amdgcn_readlane(ey, jj);
        const uint32_t xs = ok ? (uint32_t)blk * (B * S) : kOffOff;
        const uint32_t ws = ok ? (uint32_t)id * (B * B * S) : kOffOff;
#pragma unroll
        for (int i = 0; i < MT * U; i++) sl.x[i] = bload128(rin, xo[i], xs);
#pragma unroll
        for (int i = 0; i < WR; i++) {
            if constexpr (C::W8)
                sl.w[i] = bload64(rw, wo[i], ws);
            else
                sl.w[i] = bload128(rw, wo[i], ws);
        }
    };

    f32x4 acc[MT][2];
#pragma unroll
    for (int mt = 0; mt < MT; mt++) acc[mt][0] = acc[mt][1] = f32x4{0.f, 0.f, 0.f, 0.f};
    auto compute = [&](const Slot& sl) { rows_compute<DT, TW, MT>(acc, sl, wt, lane); };

    {
        Slot ring[D];
#pragma unroll
        for (int i = 0; i < D; i++) {
            load_slot(ring[i], i);
            // issue the slots oldest first: the wait at the loop's top then covers one slot
            __builtin_amdgcn_sched_barrier(0);
        }
        for (int j = 0; j < nmine; j += D) {
#pragma unroll
            for (int i = 0; i < D; i++) {
                if (j + i < nmine) compute(ring[i]);
                load_slot(ring[i], j + i + D);
            }
        }
    }

    auto store = [&](int mt, int l, const f32x4& s0, const f32x4& s1) {
        const int lr = l & 15, lg = l >> 4;
        const int64_t c0 = (int64_t)o * 32 + C::qmap(0, lr), c1 = (int64_t)o * 32 + C::qmap(1, lr);
#pragma unroll
        for (int v = 0; v < 4; v++) {
            const int64_t n = n0 + 16 * mt + 4 * lg + v;
            if (n < N) {
                if constexpr (C::W8) {   // outputs 2 lr, 2 lr + 1: one 8-byte store
                    *reinterpret_cast<u32x2*>((float*)a.out + n * a.fout + c0) =
                        u32x2{__float_as_uint(s0[v]), __float_as_uint(s1[v])};
                } else {
                    store_elt(a.out, n * a.fout + c0, s0[v], DT);
                    store_elt(a.out, n * a.fout + c1, s1[v], DT);
                }
            }
        }
    };
    if constexpr (WAVES == 1) {
#pragma unroll
        for (int mt = 0; mt < MT; mt++) store(mt, lane, acc[mt][0], acc[mt][1]);
    } else {
#pragma unroll
        for (int mt = 0; mt < MT; mt++)
#pragma unroll
            for (int t = 0; t < 2; t++) red[wave * TILE + (mt * 2 + t) * 64 + lane] = acc[mt][t];
        __syncthreads();
        for (int i = threadIdx.x; i < MT * 64; i += 64 * WAVES) {   // (mt, lane), both output tiles
            const int mt = i >> 6, l = i & 63;
            f32x4 s0 = red[(mt * 2) * 64 + l], s1 = red[(mt * 2 + 1) * 64 + l];
#pragma unroll
            for (int w = 1; w < WAVES; w++) {
                s0 += red[w * TILE + (mt * 2) * 64 + l];
                s1 += red[w * TILE + (mt * 2 + 1) * 64 + l];
            }
            store(mt, l, s0, s1);
        }
    }
}

template <int DT, bool TW, int MT, int WAVES, int D>
static hipError_t launch_rows_t(MMArgs a, hipStream_t st, int pass) {
    a.ntiles = (int)((a.N + 16 * MT - 1) / (16 * MT));
    const int64_t grid = (int64_t)mm_grid(a.nout, a.ntiles);
    if (grid > INT32_MAX) return hipErrorInvalidConfiguration;
    return launch(pass, rows_kernel<DT, TW, MT, WAVES, D>, dim3((unsigned)grid), dim3(64 * WAVES), st, a);
}

// Shape: 2 minibatch tiles of 16 rows, 4 waves, 2 list entries in flight per wave
// (measured fastest on the 4096-wide, N = 64 workload among 1/2/4 tiles, 4/8 waves and
// rings of 2/4/8/16 entries).  BSMM_ROWS_CFG=<tiles>,<waves>,<depth> (read once)
// selects one of the other instantiated shapes for A/B measurements.
static int rows_cfg() {
    static const int key = [] {
        int mt = 2, waves = 4, depth = 2;
        if (const char* e = getenv("BSMM_ROWS_CFG")) sscanf(e, "%d,%d,%d", &mt, &waves, &depth);
        return mt * 100 + waves * 10 + depth;
    }();
    return key;
}

template <int DT, bool TW>
static hipError_t launch_rows_dt(const MMArgs& a, hipStream_t st, int pass) {
    switch (rows_cfg()) {
    case 244: return launch_rows_t<DT, TW, 2, 4, 4>(a, st, pass);
    case 282: return launch_rows_t<DT, TW, 2, 8, 2>(a, st, pass);
    case 142: return launch_rows_t<DT, TW, 1, 4, 2>(a, st, pass);
    default: return launch_rows_t<DT, TW, 2, 4, 2>(a, st, pass);
    }
}

hipError_t launch_mm_rows(const MMArgs& a, int dt, bool transw, void* stream, int pass) {
    hipStream_t st = (hipStream_t)stream;
    switch (dt * 2 + (transw ? 1 : 0)) {
    case 0: return launch_rows_dt<BSMM_F32, false>(a, st, pass);
    case 1: return launch_rows_dt<BSMM_F32, true>(a, st, pass);
    case 2: return launch_rows_dt<BSMM_BF16, false>(a, st, pass);
    case 3: return launch_rows_dt<BSMM_BF16, true>(a, st, pass);
    case 4: return launch_rows_dt<BSMM_F16, false>(a, st, pass);
    case 5: return launch_rows_dt<BSMM_F16, true>(a, st, pass);
    }
    return hipErrorInvalidValue;
}

}  // namespace bsmm
