// fprop and bprop of the block-sparse product on gfx950.
//
//   fprop  y[:, k-block]  = sum over c with L[c][k]=1 of x[:, c-block]  . W[id(c,k)]
//   bprop  dx[:, c-block] = sum over k with L[c][k]=1 of dy[:, k-block] . W[id(c,k)]^T
// (kiteco/blocksparse README, "API Documentation" › blocksparse.matmul ›
// BlocksparseMatMul.__call__ and its input gradient.)
//
// One kernel serves both: an output block o owns a list of entries (in-block, id)
// (the layout column for fprop, the row for bprop); out[:, o] = sum over the list of
// in[:, blk] . Wop with Wop[p][q] = W[id][p][q] (fprop) or W[id][q][p] (bprop).
//
// A workgroup (4 waves) computes an NT x b tile of one output block.  Waves split the
// NT minibatch rows (WM) and/or the list (WK); WK partial tiles are added in wave
// order through LDS, so results are bit-reproducible.  The contraction runs in steps
// of 32 (16-bit) or 16 (fp32) values, i.e. 32/b entries per step for b < 32.  Each
// wave keeps D steps of global loads in flight in a register ring.
//
// Operands reach the matrix cores in one of three ways:
//   direct   the contraction index is contiguous in memory (activations with
//            feature_axis 1, the weight in bprop): one 16-byte load per fragment.
//   tr       the contraction index is the slow one (activations with feature_axis 0,
//            the weight in fprop), 16-bit types: rows are loaded with 16-byte loads,
//            stored to a wave-private LDS tile and read back with the transposing
//            LDS read (frag_tr16).
//   strided  the same case for fp32: four 4-byte loads per fragment (16 lanes read
//            64 contiguous bytes per row).
// The output tile is oriented so that each lane holds four consecutive outputs of
// one row of the stored layout and writes them with one vector store.
#include <cstdlib>

#include <cstring>

#include "common.h"

namespace bsmm {

template <int DT, int B, int FA, bool TW, int MT, int WM, int WK, int D>
struct MMCfg {
    static constexpr int VEC = Elt<DT>::VEC, KS = 4 * VEC;
    static constexpr int QT = (B + 15) / 16;
    static constexpr int NTW = 16 * MT, NT = NTW * WM;
    static constexpr bool S16 = DT != BSMM_F32;
    static constexpr bool W_TR = !TW && S16;
    static constexpr bool X_TR = FA == 0 && S16;
    static constexpr int WCH = B / 8;                        // 16-byte chunks per weight row
    static constexpr int WR = W_TR ? (4 * B + 63) / 64 : QT;  // weight registers per lane and step
    static constexpr int WPITCH = QT * 16 + 8;               // LDS row pitch, elements
    static constexpr int XPITCH = NTW + 8;
    static constexpr int WTILE = W_TR ? 32 * WPITCH : 0;     // elements per wave
    static constexpr int XTILE = X_TR ? 32 * XPITCH : 0;
    static constexpr int WAVES = WM * WK, THREADS = 64 * WAVES;
    static constexpr int TILE_BYTES = WAVES * (WTILE + XTILE) * 2;
    static constexpr int RED_BYTES = WK > 1 ? WAVES * MT * QT * 64 * 16 : 0;   // partial tiles
    static constexpr int SMEM = TILE_BYTES > RED_BYTES ? TILE_BYTES : RED_BYTES;
    // List entries staged in LDS at a time.  16-bit 8x8 blocks with features first and
    // whole-list waves stage 128: their lists are short (about 100 entries at 10 %
    // density over 1024 block rows) and the smaller stage lets 6 instead of 4 waves per
    // SIMD fit (hidden 8192, N = 1024: fprop and bprop about 11 % faster).  Elsewhere
    // 1024 (16x16 fp16 with features first measured slower with 256).
    static constexpr int LCAP = (B == 8 && FA == 0 && S16 && WK == 1) ? 128 : 1024;
};

template <int WR, int XR> struct Slot {
    u32x4 w[WR];
    u32x4 x[XR];
};

template <int DT, int B, int FA, bool TW, int MT, int WM, int WK, int D>
__global__ __launch_bounds__(64 * WM * WK) void mm_kernel(MMArgs a) {
    using Cfg = MMCfg<DT, B, FA, TW, MT, WM, WK, D>;
    using T = typename Elt<DT>::T;
    constexpr int S = (int)sizeof(T);
    constexpr int VEC = Cfg::VEC, KS = Cfg::KS, QT = Cfg::QT, NT = Cfg::NT, NTW = Cfg::NTW;
    constexpr int WR = Cfg::WR;
    // UNI: a contraction step never spans two list entries, so the entry of a step is
    // the same for the whole wave and its addresses are scalar offsets.
    constexpr bool UNI = B >= KS;
    constexpr int EPS = UNI ? 1 : KS / B;   // entries per step
    // wave-private transpose tiles during the walk; the WK partial tiles afterwards
    __shared__ __attribute__((aligned(16))) char smem[Cfg::SMEM > 0 ? Cfg::SMEM : 16];
    // The list is staged in LDS (chunks of Cfg::LCAP entries): the ring's loads then depend
    // on LDS reads only, never on another global load, which would make the wave wait
    // for every load in flight.
    constexpr int LCAP = Cfg::LCAP;
    __shared__ int2 lst[LCAP];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wm = wave % WM, wk = wave / WM;
    const int r16 = lane & 15, g = lane >> 4;

    int li, nt;
    wg_decode(blockIdx.x, a.nout, a.ntiles, li, nt);
    if (li < 0) return;   // the whole workgroup leaves together
    // the list's record: header (length, start) and its first entries, one load level
    const int* rec = a.rec + (int64_t)li * a.rsi;
    const int4 hdr = *reinterpret_cast<const int4*>(rec);
    const int o = hdr.x, beg = hdr.y, len = hdr.z;
    const int2* __restrict__ rent = reinterpret_cast<const int2*>(rec + 4);
    const int rs = (a.rsi - 4) / 2;
    const int N = (int)a.N;
    const int n0w = nt * NT + wm * NTW;
    const int2* __restrict__ gent = reinterpret_cast<const int2*>(a.ent) + beg;
    const rsrc_t rin = make_rsrc(a.in, a.in_bytes);
    const rsrc_t rw = make_rsrc(a.w, a.w_bytes);
    const bool xvec = (N % 8) == 0;

    BSMM_LDS uint16_t* wt = (BSMM_LDS uint16_t*)smem + wave * (Cfg::WTILE + Cfg::XTILE);
    BSMM_LDS uint16_t* xt = wt + Cfg::WTILE;
    if constexpr (Cfg::W_TR && B == 8) {
        // columns 8..15 of the weight tile stay zero (b = 8 uses half a 16-wide tile)
        for (int i = lane; i < 32 * Cfg::WPITCH; i += 64) wt[i] = 0;
    }

    // ---- per-lane constants: byte offsets inside a weight block / activation tile and
    // the lane's entry within a step (0 when UNI); kOffLane for lanes with no data ----
    uint32_t wc[WR];
    int wel[WR];
#pragma unroll
    for (int i = 0; i < WR; i++) {
        if constexpr (Cfg::W_TR) {
            const int c = lane + 64 * i;
            const bool cv = c < 4 * B;
            const int r = cv ? c / Cfg::WCH : 0, cc = c % Cfg::WCH;
            wel[i] = UNI ? 0 : r / B;
            const int p = UNI ? r : r % B;
            wc[i] = cv ? (uint32_t)((p * B + cc * 8) * S) : kOffLane;
        } else {
            const int q = 16 * i + r16;
            const int pl = UNI ? g * VEC : (g * VEC) % B;
            wel[i] = UNI ? 0 : (g * VEC) / B;
            wc[i] = q < B ? (uint32_t)((TW ? q * B + pl : pl * B + q) * S) : kOffLane;
        }
    }
    uint32_t xc[MT];
    int xel[MT], xn[MT];
#pragma unroll
    for (int i = 0; i < MT; i++) {
        if constexpr (Cfg::X_TR) {
            const int c = lane + 64 * i;
            const int r = c / (2 * MT), cc = c % (2 * MT);
            const int n = n0w + cc * 8;
            xel[i] = UNI ? 0 : r / B;
            const int p = UNI ? r : r % B;
            xn[i] = n;
            xc[i] = n < N ? (uint32_t)p * (uint32_t)N * S + (uint32_t)n * S : kOffLane;
        } else {
            const int n = n0w + 16 * i + r16;
            const int pl = UNI ? g * VEC : (g * VEC) % B;
            xel[i] = UNI ? 0 : (g * VEC) / B;
            xn[i] = n;
            if constexpr (FA == 1)
                xc[i] = n < N ? ((uint32_t)n * a.fin + pl) * S : kOffLane;
            else
                xc[i] = n < N ? ((uint32_t)pl * N + n) * S : kOffLane;
        }
    }

    int clen = 0;     // entries of the current chunk
    int csteps = 0;   // contraction steps of the current chunk
    auto load_slot = [&](Slot<WR, MT>& sl, int s) {
        const bool sv = s < csteps;   // wave-uniform
        const int eu = UNI ? (s * KS) / B : s * EPS;
        const int pu = UNI ? (s * KS) % B : 0;
        if constexpr (UNI) {
            const bool ev = sv && eu < clen;
            const int2 en = lst[ev ? eu : 0];
            const int blk = __builtin_amdgcn_readfirstlane(en.x), id = __builtin_amdgcn_readfirstlane(en.y);
            // ---- weight ----
            const uint32_t ws = (uint32_t)id * (B * B * S) + (TW ? pu * S : (Cfg::W_TR ? 0 : pu * B * S));
#pragma unroll
            for (int i = 0; i < WR; i++) {
                if constexpr (Cfg::W_TR || TW) {
                    sl.w[i] = bload128(rw, wc[i], ev ? ws : kOffOff);
                } else {   // fp32, contraction index is the weight row
#pragma unroll
                    for (int v = 0; v < 4; v++) sl.w[i][v] = bload32(rw, wc[i] + v * B * S, ev ? ws : kOffOff);
                }
            }
            // ---- activations ----
#pragma unroll
            for (int i = 0; i < MT; i++) {
                if constexpr (Cfg::X_TR) {
                    const uint32_t xs = (uint32_t)blk * B * (uint32_t)N * S;
                    if (xvec) {
                        sl.x[i] = bload128(rin, xc[i], ev ? xs : kOffOff);
                    } else {   // rows not 16-byte aligned: element loads, tail masked
                        uint32_t h[8];
#pragma unroll
                        for (int v = 0; v < 8; v++)
                            h[v] = bload16(rin, xn[i] + v < N ? xc[i] + v * S : kOffLane, ev ? xs : kOffOff);
                        sl.x[i] = u32x4{h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16),
                                        h[6] | (h[7] << 16)};
                    }
                } else if constexpr (FA == 1) {
                    sl.x[i] = bload128(rin, xc[i], ev ? (uint32_t)(blk * B + pu) * S : kOffOff);
                } else {   // fp32, feature-major activations: four rows per fragment
#pragma unroll
                    for (int v = 0; v < 4; v++)
                        sl.x[i][v] = bload32(rin, xc[i], ev ? ((uint32_t)(blk * B + pu + v) * N) * S : kOffOff);
                }
            }
        } else {
            // ---- weight: the entry differs between lane groups ----
#pragma unroll
            for (int i = 0; i < WR; i++) {
                const int e = eu + wel[i];
                const bool ok = sv && e < clen;
                const int id = lst[ok ? e : 0].y;
                const uint32_t vo = ok ? wc[i] + (uint32_t)id * (B * B * S) : kOffLane;
                if constexpr (Cfg::W_TR || TW) {
                    sl.w[i] = bload128(rw, vo, 0);
                } else {
#pragma unroll
                    for (int v = 0; v < 4; v++) sl.w[i][v] = bload32(rw, vo + v * B * S, 0);
                }
            }
            // ---- activations ----
#pragma unroll
            for (int i = 0; i < MT; i++) {
                const int e = eu + xel[i];
                const bool ok = sv && e < clen;
                const int blk = lst[ok ? e : 0].x;
                if constexpr (Cfg::X_TR) {
                    const uint32_t vo = ok ? xc[i] + (uint32_t)blk * B * (uint32_t)N * S : kOffLane;
                    if (xvec) {
                        sl.x[i] = bload128(rin, vo, 0);
                    } else {
                        uint32_t h[8];
#pragma unroll
                        for (int v = 0; v < 8; v++) h[v] = bload16(rin, xn[i] + v < N ? vo + v * S : kOffLane, 0);
                        sl.x[i] = u32x4{h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16),
                                        h[6] | (h[7] << 16)};
                    }
                } else if constexpr (FA == 1) {
                    sl.x[i] = bload128(rin, ok ? xc[i] + (uint32_t)blk * B * S : kOffLane, 0);
                } else {
                    const uint32_t vo = ok ? xc[i] + (uint32_t)blk * B * (uint32_t)N * S : kOffLane;
#pragma unroll
                    for (int v = 0; v < 4; v++) sl.x[i][v] = bload32(rin, vo, (uint32_t)v * N * S);
                }
            }
        }
    };

    f32x4 acc[MT][QT];
#pragma unroll
    for (int i = 0; i < MT; i++)
#pragma unroll
        for (int j = 0; j < QT; j++) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    auto compute_slot = [&](const Slot<WR, MT>& sl) {
        if constexpr (Cfg::W_TR) {
#pragma unroll
            for (int i = 0; i < WR; i++) {
                const int c = lane + 64 * i;
                if (c < 4 * B) lds_store16(wt + (c / Cfg::WCH) * Cfg::WPITCH + (c % Cfg::WCH) * 8, sl.w[i]);
            }
        }
        if constexpr (Cfg::X_TR) {
#pragma unroll
            for (int i = 0; i < MT; i++) {
                const int c = lane + 64 * i;
                lds_store16(xt + (c / (2 * MT)) * Cfg::XPITCH + (c % (2 * MT)) * 8, sl.x[i]);
            }
        }
        wave_lds_order();
        u32x4 wf[QT], xf[MT];
#pragma unroll
        for (int qt = 0; qt < QT; qt++) {
            if constexpr (Cfg::W_TR)
                wf[qt] = frag_tr16(wt, Cfg::WPITCH, 16 * qt, lane);
            else
                wf[qt] = sl.w[qt];
        }
#pragma unroll
        for (int mt = 0; mt < MT; mt++) {
            if constexpr (Cfg::X_TR)
                xf[mt] = frag_tr16(xt, Cfg::XPITCH, 16 * mt, lane);
            else
                xf[mt] = sl.x[mt];
        }
        wave_lds_order();
#pragma unroll
        for (int mt = 0; mt < MT; mt++)
#pragma unroll
            for (int qt = 0; qt < QT; qt++) {
                if constexpr (FA == 1)
                    mma<DT>(acc[mt][qt], wf[qt], xf[mt]);   // D[q][n]
                else
                    mma<DT>(acc[mt][qt], xf[mt], wf[qt]);   // D[n][q]
            }
    };

    {   // first chunk straight from the record (entries past the length are unused)
        const int first = rs < LCAP ? rs : LCAP;
        for (int i = threadIdx.x; i < first; i += Cfg::THREADS) lst[i] = rent[i];
    }
    for (int cbeg = 0; cbeg < len; cbeg += LCAP) {
        clen = len - cbeg < LCAP ? len - cbeg : LCAP;
        if (cbeg > 0) {
            __syncthreads();   // the previous chunk is no longer read
            for (int i = threadIdx.x; i < clen; i += Cfg::THREADS) lst[i] = gent[cbeg + i];
        }
        __syncthreads();
        csteps = (clen * B + KS - 1) / KS;
        const int mysteps = csteps > wk ? (csteps - wk + WK - 1) / WK : 0;
        Slot<WR, MT> ring[D];
#pragma unroll
        for (int i = 0; i < D; i++) {
            load_slot(ring[i], wk + WK * i);
            // issue the slots oldest first, as the loop does: the wait at the loop's top
            // then covers only the slot it consumes, not every load in flight
            __builtin_amdgcn_sched_barrier(0);
        }
        // steps past the end compute on zeros; the trip count stays a multiple of D
        for (int j = 0; j < mysteps; j += D) {
#pragma unroll
            for (int i = 0; i < D; i++) {
                compute_slot(ring[i]);
                load_slot(ring[i], wk + WK * (j + i + D));
            }
        }
    }

    const bool ovec = (N % 4) == 0;
    // lane `l` of a wave holds, for tile (mt, qt), four consecutive outputs of one row of
    // the stored layout; write them (vector store when aligned and in range)
    auto store_tile = [&](int mt, int qt, int l, const f32x4& v4) {
        const int lr16 = l & 15, lg = l >> 4;
        if constexpr (FA == 1) {
            const int64_t n = n0w + mt * 16 + lr16;   // out[n][q .. q+3]
            const int q = qt * 16 + 4 * lg;
            if (n < N && q < B) store4<DT>(a.out, n * a.fout + (int64_t)o * B + q, v4);
        } else {
            const int q = qt * 16 + lr16;              // out[q][n .. n+3]
            const int64_t n = n0w + mt * 16 + 4 * lg;
            if (q < B && n < N) {
                const int64_t base = ((int64_t)o * B + q) * N + n;
                if (ovec && n + 4 <= N) {
                    store4<DT>(a.out, base, v4);
                } else {
#pragma unroll
                    for (int v = 0; v < 4; v++)
                        if (n + v < N) store_elt(a.out, base + v, v4[v], DT);
                }
            }
        }
    };

    if constexpr (WK > 1) {
        // WK partial tiles: every wave parks its tile in LDS, then each wave adds up a
        // share of the tile's elements over the WK partials in wave order.
        __syncthreads();   // transpose tiles are dead; reuse the space
        f32x4* red = reinterpret_cast<f32x4*>(smem);   // [wm][wk][tile][lane]
        constexpr int TL = MT * QT * 64;
#pragma unroll
        for (int i = 0; i < MT; i++)
#pragma unroll
            for (int j = 0; j < QT; j++) red[(wm * WK + wk) * TL + (i * QT + j) * 64 + lane] = acc[i][j];
        __syncthreads();
        for (int sidx = wk * 64 + lane; sidx < TL; sidx += WK * 64) {
            f32x4 sum = red[(wm * WK) * TL + sidx];
#pragma unroll
            for (int r = 1; r < WK; r++) sum += red[(wm * WK + r) * TL + sidx];
            const int tile = sidx / 64;
            store_tile(tile / QT, tile % QT, sidx % 64, sum);
        }
    } else {
#pragma unroll
        for (int mt = 0; mt < MT; mt++)
#pragma unroll
            for (int qt = 0; qt < QT; qt++) store_tile(mt, qt, lane, acc[mt][qt]);
    }
}

// ---------------------------------------------------------------------------------
// Large minibatch.  A workgroup (4 waves) computes a 64*MTW-row x b tile of one output
// block; each wave owns 16*MTW rows and walks the whole list.  The list's weight blocks
// are staged in LDS once (in chunks) and shared by the waves: block rows are stacked
// in list order, so for fprop the stack is the K-major tile the transposing read
// expects, and for bprop each row holds one q with p contiguous.  Only activations
// stream from global memory, through a ring of D steps per wave.  Workgroups are
// dealt so that each XCD works on one minibatch tile at a time, columns in natural
// order: the activation rows of that tile stay in the XCD's L2 while every list that
// uses them runs.
constexpr int WSTACK_BYTES = 48 * 1024;

template <int DT, int B, int FA, bool TW, int MTW, int D>
struct MMLCfg {
    static constexpr int VEC = Elt<DT>::VEC, KS = 4 * VEC;
    static constexpr int S = DT == BSMM_F32 ? 4 : 2;
    static constexpr int QT = (B + 15) / 16;
    static constexpr int NTW = 16 * MTW, NT = 4 * NTW;
    static constexpr bool S16 = DT != BSMM_F32;
    static constexpr bool X_TR = FA == 0 && S16;
    static constexpr int EPS = B >= KS ? 1 : KS / B;          // entries per step
    static constexpr int PW = (TW ? B : QT * 16) + 8;         // stack row pitch, elements
    // entries per chunk: a multiple of EPS; stack rows padded to whole steps + one zero row
    static constexpr int ECAP = ((WSTACK_BYTES / (PW * S) - KS - 1) / B) / EPS * EPS;
    static constexpr int ROWS = ((ECAP * B + KS - 1) / KS) * KS;   // stack rows
    static constexpr int ZROW = ROWS;                           // an all-zero row
    static constexpr int STACK = (ROWS + 1) * PW;               // elements
    static constexpr int XPITCH = NTW + 8;
    static constexpr int XTILE = X_TR ? 32 * XPITCH : 0;        // elements per wave
    static_assert(ECAP >= EPS, "stack too small");
};

template <int DT, int B, int FA, bool TW, int MTW, int D>
__global__ __launch_bounds__(256) void mml_kernel(MMArgs a) {
    using Cfg = MMLCfg<DT, B, FA, TW, MTW, D>;
    using T = typename Elt<DT>::T;
    constexpr int S = Cfg::S, VEC = Cfg::VEC, KS = Cfg::KS, QT = Cfg::QT, NT = Cfg::NT, NTW = Cfg::NTW;
    constexpr int PW = Cfg::PW, ECAP = Cfg::ECAP;
    constexpr bool UNI = B >= KS;
    constexpr int EPS = Cfg::EPS;
    constexpr int CH = 16 / S;   // elements per 16-byte chunk
    __shared__ __attribute__((aligned(16))) T wst[Cfg::STACK];
    __shared__ __attribute__((aligned(16))) uint16_t xtl[Cfg::X_TR ? 4 * Cfg::XTILE : 8];
    __shared__ int2 lst[ECAP];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int r16 = lane & 15, g = lane >> 4;

    // workgroup -> (list, minibatch tile)
    int li, nt;
    {
        const int bid = blockIdx.x, xcd = bid & 7, slot = bid >> 3;
        if (a.ntiles >= 8) {   // each XCD walks the lists of one tile at a time
            li = slot % a.nout;
            nt = (slot / a.nout) * 8 + xcd;
            if (nt >= a.ntiles) return;
        } else {
            li = (slot / a.ntiles) * 8 + xcd;
            nt = slot % a.ntiles;
            if (li >= a.nout) return;
        }
    }
    const int* rec = a.rec + (int64_t)li * a.rsi;
    const int4 hdr = *reinterpret_cast<const int4*>(rec);
    const int o = hdr.x, beg = hdr.y, len = hdr.z;
    const int2* __restrict__ rent = reinterpret_cast<const int2*>(rec + 4);
    const int rs = (a.rsi - 4) / 2;
    const int N = (int)a.N;
    const int n0w = nt * NT + wave * NTW;
    const int2* __restrict__ gent = reinterpret_cast<const int2*>(a.ent) + beg;
    const rsrc_t rin = make_rsrc(a.in, a.in_bytes);
    const rsrc_t rw = make_rsrc(a.w, a.w_bytes);
    const bool xvec = (N % 8) == 0;
    BSMM_LDS uint16_t* xt = (BSMM_LDS uint16_t*)xtl + wave * Cfg::XTILE;
    BSMM_LDS T* stk = (BSMM_LDS T*)wst;

    // zero the stack once: padding columns, the zero row and rows past a short list
    // are never written afterwards except by the staging of real block rows
    for (int i = threadIdx.x; i < Cfg::STACK; i += 256) stk[i] = (T)0;

    // ---- activation fragments: per-lane constants (as in mm_kernel) ----
    uint32_t xc[MTW];
    int xel[MTW], xn[MTW];
#pragma unroll
    for (int i = 0; i < MTW; i++) {
        if constexpr (Cfg::X_TR) {
            const int c = lane + 64 * i;
            const int r = c / (2 * MTW), cc = c % (2 * MTW);
            const int n = n0w + cc * 8;
            xel[i] = UNI ? 0 : r / B;
            const int p = UNI ? r : r % B;
            xn[i] = n;
            xc[i] = n < N ? (uint32_t)p * (uint32_t)N * S + (uint32_t)n * S : kOffLane;
        } else {
            const int n = n0w + 16 * i + r16;
            const int pl = UNI ? g * VEC : (g * VEC) % B;
            xel[i] = UNI ? 0 : (g * VEC) / B;
            xn[i] = n;
            if constexpr (FA == 1)
                xc[i] = n < N ? ((uint32_t)n * a.fin + pl) * S : kOffLane;
            else
                xc[i] = n < N ? ((uint32_t)pl * N + n) * S : kOffLane;
        }
    }

    int clen = 0, csteps = 0;
    auto load_x = [&](u32x4* xr, int s) {
        const bool sv = s < csteps;
        const int eu = UNI ? (s * KS) / B : s * EPS;
        const int pu = UNI ? (s * KS) % B : 0;
#pragma unroll
        for (int i = 0; i < MTW; i++) {
            const int e = eu + xel[i];
            const bool ok = sv && e < clen;
            const int blk = UNI ? __builtin_amdgcn_readfirstlane(lst[ok ? e : 0].x) : lst[ok ? e : 0].x;
            if constexpr (Cfg::X_TR) {
                const uint32_t vo = ok ? xc[i] + (uint32_t)blk * B * (uint32_t)N * S : kOffLane;
                if (xvec) {
                    xr[i] = bload128(rin, vo, 0);
                } else {
                    uint32_t h[8];
#pragma unroll
                    for (int v = 0; v < 8; v++) h[v] = bload16(rin, xn[i] + v < N ? vo + v * S : kOffLane, 0);
                    xr[i] = u32x4{h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16), h[6] | (h[7] << 16)};
                }
            } else if constexpr (FA == 1) {
                xr[i] = bload128(rin, ok ? xc[i] : kOffLane, (uint32_t)(blk * B + pu) * S);
            } else {
                const uint32_t vo = ok ? xc[i] : kOffLane;
#pragma unroll
                for (int v = 0; v < 4; v++) xr[i][v] = bload32(rin, vo, ((uint32_t)(blk * B + pu + v) * N) * S);
            }
        }
    };

    f32x4 acc[MTW][QT];
#pragma unroll
    for (int i = 0; i < MTW; i++)
#pragma unroll
        for (int j = 0; j < QT; j++) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    auto compute = [&](const u32x4* xr, int s) {
        const int K0 = s * KS + g * VEC;   // this lane group's first contraction index
        u32x4 wf[QT], xf[MTW];
#pragma unroll
        for (int qt = 0; qt < QT; qt++) {
            const int q = 16 * qt + r16;
            if constexpr (!TW && Cfg::S16) {
                wf[qt] = frag_tr16((const BSMM_LDS uint16_t*)stk + s * KS * PW, PW, 16 * qt, lane);
            } else if constexpr (!TW) {   // fp32: rows K0 + v, column q (zero columns past b)
#pragma unroll
                for (int v = 0; v < 4; v++) wf[qt][v] = __float_as_uint(stk[(K0 + v) * PW + q]);
            } else {   // bprop: row e*B + q holds W[id][q][.]; p contiguous
                const int e = K0 / B, p0 = K0 % B;
                const int row = q < B ? e * B + q : Cfg::ZROW;
                wf[qt] = *reinterpret_cast<const BSMM_LDS u32x4*>(stk + row * PW + (q < B ? p0 : 0));
            }
        }
        if constexpr (Cfg::X_TR) {
#pragma unroll
            for (int i = 0; i < MTW; i++) {
                const int c = lane + 64 * i;
                lds_store16(xt + (c / (2 * MTW)) * Cfg::XPITCH + (c % (2 * MTW)) * 8, xr[i]);
            }
            wave_lds_order();
#pragma unroll
            for (int mt = 0; mt < MTW; mt++) xf[mt] = frag_tr16(xt, Cfg::XPITCH, 16 * mt, lane);
            wave_lds_order();
        } else {
#pragma unroll
            for (int mt = 0; mt < MTW; mt++) xf[mt] = xr[mt];
        }
#pragma unroll
        for (int mt = 0; mt < MTW; mt++)
#pragma unroll
            for (int qt = 0; qt < QT; qt++) {
                if constexpr (FA == 1)
                    mma<DT>(acc[mt][qt], wf[qt], xf[mt]);   // D[q][n]
                else
                    mma<DT>(acc[mt][qt], xf[mt], wf[qt]);   // D[n][q]
            }
    };

    {   // first chunk straight from the record
        const int first = rs < ECAP ? rs : ECAP;
        for (int i = threadIdx.x; i < first; i += 256) lst[i] = rent[i];
    }
    for (int cbeg = 0; cbeg < len; cbeg += ECAP) {
        clen = len - cbeg < ECAP ? len - cbeg : ECAP;
        csteps = (clen * B + KS - 1) / KS;
        __syncthreads();   // previous chunk fully consumed (and the stack zeroed)
        if (cbeg > 0) {
            for (int i = threadIdx.x; i < clen; i += 256) lst[i] = gent[cbeg + i];
            __syncthreads();
        }
        // stage the chunk's weight blocks: block e's row r -> stack row e*B + r
        {
            constexpr int CPB = B * B / CH;   // chunks per block
            for (int t = threadIdx.x; t < clen * CPB; t += 256) {
                const int e = t / CPB, rc = t % CPB;
                const int r = rc / (B / CH), cc = rc % (B / CH);
                const uint32_t off = (uint32_t)lst[e].y * (B * B * S) + (uint32_t)(r * B + cc * CH) * S;
                const u32x4 v = bload128(rw, off, 0);
                *reinterpret_cast<BSMM_LDS u32x4*>(stk + (e * B + r) * PW + cc * CH) = v;
            }
            // rows of a partial last step beyond the list must read as zero
            for (int i = clen * B * PW + threadIdx.x; i < csteps * KS * PW; i += 256) stk[i] = (T)0;
        }
        u32x4 ring[D][MTW];
#pragma unroll
        for (int i = 0; i < D; i++) load_x(ring[i], i);
        __syncthreads();   // stack ready
        for (int j = 0; j < csteps; j += D) {
#pragma unroll
            for (int i = 0; i < D; i++) {
                if (j + i < csteps) compute(ring[i], j + i);   // no loads inside: branch is harmless
                load_x(ring[i], j + i + D);
            }
        }
    }

    const bool ovec = (N % 4) == 0;
#pragma unroll
    for (int mt = 0; mt < MTW; mt++)
#pragma unroll
        for (int qt = 0; qt < QT; qt++) {
            if constexpr (FA == 1) {
                const int n = n0w + mt * 16 + r16;   // out[n][q .. q+3]
                const int q = qt * 16 + 4 * g;
                if (n < N && q < B) store4<DT>(a.out, (int64_t)n * a.fout + (int64_t)o * B + q, acc[mt][qt]);
            } else {
                const int q = qt * 16 + r16;          // out[q][n .. n+3]
                const int n = n0w + mt * 16 + 4 * g;
                if (q < B && n < N) {
                    const int64_t base = ((int64_t)o * B + q) * N + n;
                    if (ovec && n + 4 <= N) {
                        store4<DT>(a.out, base, acc[mt][qt]);
                    } else {
#pragma unroll
                        for (int v = 0; v < 4; v++)
                            if (n + v < N) store_elt(a.out, base + v, acc[mt][qt][v], DT);
                    }
                }
            }
        }
}

template <int DT, int B, int FA, bool TW, int MTW, int D>
static hipError_t launch_large(MMArgs a, hipStream_t st, int pass) {
    constexpr int NT = 64 * MTW;
    a.ntiles = (int)((a.N + NT - 1) / NT);
    int64_t grid;
    if (a.ntiles >= 8)
        grid = (int64_t)a.nout * ((a.ntiles + 7) / 8) * 8;
    else
        grid = (int64_t)((a.nout + 7) / 8) * 8 * a.ntiles;
    if (grid > INT32_MAX) return hipErrorInvalidConfiguration;
    return launch(pass, mml_kernel<DT, B, FA, TW, MTW, D>, dim3((unsigned)grid), dim3(256), st, a);
}

// ---------------------------------------------------------------------------------

template <int DT, int B, int FA, bool TW, int MT, int WM, int WK, int D>
static hipError_t launch_cfg(MMArgs a, hipStream_t st, int pass) {
    constexpr int NT = 16 * MT * WM;
    a.ntiles = (int)((a.N + NT - 1) / NT);
    const int64_t grid = (int64_t)mm_grid(a.nout, a.ntiles);
    if (grid > INT32_MAX) return hipErrorInvalidConfiguration;
    return launch(pass, mm_kernel<DT, B, FA, TW, MT, WM, WK, D>, dim3((unsigned)grid), dim3(64 * WM * WK), st, a);
}

// BSMM_MM_VARIANT=<n> (read once) forces one of the launch shapes below for A/B
// measurements; every variant computes the same result.  0 or unset: automatic.
static int mm_variant() {
    static const int v = [] {
        const char* e = getenv("BSMM_MM_VARIANT");
        return e ? atoi(e) : 0;
    }();
    return v;
}

template <int DT, int B, int FA, bool TW>
static hipError_t launch_mm_t(const MMArgs& a, int kind, hipStream_t st, int pass) {
    constexpr int DS = DT == BSMM_F32 ? 2 : 4;   // fp32 fragments take four loads each
    // 128-row tiles: a 4-step ring pays off for 16-bit 16x16 blocks (bprop 29.9 -> 27.3 us
    // at 4096 features, N = 512); 8x8 blocks run slower with it (fprop 149 -> 167 us)
    constexpr int DM = DT != BSMM_F32 && B == 16 ? 4 : 2;
    switch (kind) {
    case MM_N16: return launch_cfg<DT, B, FA, TW, 1, 1, 4, DS>(a, st, pass);
    case MM_N64: return launch_cfg<DT, B, FA, TW, 2, 1, 4, DS>(a, st, pass);
    case MM_MID:
        // 8x8 blocks, 16-bit, features first: 2 waves x 64 rows, so each activation row
        // piece is a whole 128-byte line (4 waves x 32 rows read half lines): b = 8,
        // N = 1024 fprop 156.6 -> 139-140 us, bprop 141.6 -> 121.6 us; 16x16 blocks
        // run slower that way (hidden 4096, N = 512 fprop 32.2 -> 35.3 us)
        if constexpr (B == 8 && FA == 0 && DT != BSMM_F32) return launch_cfg<DT, B, FA, TW, 4, 2, 1, DM>(a, st, pass);
        return launch_cfg<DT, B, FA, TW, 2, 4, 1, DM>(a, st, pass);
    case MM_STACK: return launch_large<DT, B, FA, TW, 4, DS>(a, st, pass);
    case MM_V_W16: return launch_cfg<DT, B, FA, TW, 2, 1, 16, DS>(a, st, pass);
    case MM_N64_W8: return launch_cfg<DT, B, FA, TW, 2, 1, 8, DS>(a, st, pass);
    case MM_V_STACK1: return launch_large<DT, B, FA, TW, 1, 4>(a, st, pass);
    case MM_V_STACK2: return launch_large<DT, B, FA, TW, 2, 4>(a, st, pass);
    }
    return hipErrorInvalidValue;
}

template <int DT, bool TW>
static hipError_t launch_mm_dt(const MMArgs& a, int kind, int b, int fa, hipStream_t st, int pass) {
    switch (b * 2 + fa) {
    case 16: return launch_mm_t<DT, 8, 0, TW>(a, kind, st, pass);
    case 17: return launch_mm_t<DT, 8, 1, TW>(a, kind, st, pass);
    case 32: return launch_mm_t<DT, 16, 0, TW>(a, kind, st, pass);
    case 33: return launch_mm_t<DT, 16, 1, TW>(a, kind, st, pass);
    case 64: return launch_mm_t<DT, 32, 0, TW>(a, kind, st, pass);
    case 65: return launch_mm_t<DT, 32, 1, TW>(a, kind, st, pass);
    }
    return hipErrorInvalidValue;
}

int mm_kind(const MMArgs& a, int dt, int b, int fa) {
    // Output-block groups: 32x32 blocks, 16-bit storage, long minibatches (whole
    // 8-row chunks when features lead), and groups dense enough that one activation
    // slab feeds several blocks.
    const bool groups_ok = b == 32 && dt != BSMM_F32 && a.ngroups > 0 && a.gmax <= kGroupMaxSteps &&
                           (fa == 1 || a.N % 8 == 0);
    // Small minibatch, 32x32 blocks, features last (rows.hip): lists of at most 256
    // entries (64 per wave)
    const bool rows_ok = b == 32 && fa == 1 && a.N > 0 && a.N <= 64 && a.maxlen <= kRowsMaxLen;
    if (a.force > 0) {
        if (a.force == MM_GROUPS && !groups_ok) return -1;
        if (a.force == MM_ROWS && !rows_ok) return -1;
        return a.force;
    }
    switch (mm_variant()) {
    case 1: return MM_N64;
    case 2: return MM_V_W16;
    case 3: return MM_MID;
    case 4: return MM_V_STACK1;
    case 5: return MM_V_STACK2;
    case 6: return MM_STACK;
    case 7:
        if (groups_ok) return MM_GROUPS;
        break;
    default: break;
    }
    // Sparser groups still win once they fill the chip twice over (>= 512 workgroups of
    // 256 rows): measured on 256x256 layouts at N = 4096, from about 17 % fill (a
    // Bernoulli(0.1) layout; band + 3 % random at 24 %) against the weight-stack kernel.
    const int64_t gwgs = (int64_t)((a.N + 255) / 256) * a.ngroups;
    if (groups_ok && a.N >= 1024 && (a.gfill >= 25 || (a.gfill >= 17 && gwgs >= 512))) return MM_GROUPS;
    if (rows_ok) return MM_ROWS;
    // Small minibatch: the weight stream dominates and there are few output tiles, so
    // the 4 waves of a workgroup split each block list (measured fastest at N = 64).
    if (a.N <= 16) return MM_N16;
    // fp32 fragments take four loads each: 8 waves per list (each walking an eighth of
    // it) keep more of them in flight (measured 25 -> 19 us fprop at 4096 features,
    // N = 64); 16-bit storage stays at 4 waves (8 were no faster)
    if (a.N <= 64) return dt == BSMM_F32 ? MM_N64_W8 : MM_N64;
    // Large minibatch (N >= 2048): weights staged once per workgroup, activations
    // streamed, one minibatch tile per XCD at a time.  In between, 4 waves split 128
    // rows and each walks the list (measured faster there).
    if (a.N >= 2048) return MM_STACK;
    return MM_MID;
}

const char* mm_kind_name(int kind) {
    switch (kind) {
    case MM_N16: return "list_n16";
    case MM_N64: return "list_n64";
    case MM_MID: return "list_rows128";
    case MM_STACK: return "list_weight_stack";
    case MM_GROUPS: return "output_groups";
    case MM_V_W16: return "list_n64_16waves";
    case MM_N64_W8: return "list_n64_8waves";
    case MM_ROWS: return "rows_n64";
    case MM_V_STACK1: return "list_weight_stack_64";
    case MM_V_STACK2: return "list_weight_stack_128";
    }
    return "none";
}

int mm_kind_of_name(const char* name) {
    for (int k = MM_N16; k <= MM_ROWS; k++)
        if (std::strcmp(name, mm_kind_name(k)) == 0) return k;
    return 0;
}

hipError_t launch_mm(const MMArgs& a, int dt, int b, int fa, bool transw, void* stream, int pass) {
    hipStream_t st = (hipStream_t)stream;
    if (a.nout == 0) return hipSuccess;
    const int kind = mm_kind(a, dt, b, fa);
    if (kind < 0) return hipErrorNotSupported;
    if (kind == MM_GROUPS) return launch_mm_groups(a, dt, fa, transw, stream, pass);
    if (kind == MM_ROWS) return launch_mm_rows(a, dt, transw, stream, pass);
    switch (dt * 2 + (transw ? 1 : 0)) {
    case 0: return launch_mm_dt<BSMM_F32, false>(a, kind, b, fa, st, pass);
    case 1: return launch_mm_dt<BSMM_F32, true>(a, kind, b, fa, st, pass);
    case 2: return launch_mm_dt<BSMM_BF16, false>(a, kind, b, fa, st, pass);
    case 3: return launch_mm_dt<BSMM_BF16, true>(a, kind, b, fa, st, pass);
    case 4: return launch_mm_dt<BSMM_F16, false>(a, kind, b, fa, st, pass);
    case 5: return launch_mm_dt<BSMM_F16, true>(a, kind, b, fa, st, pass);
    }
    return hipErrorInvalidValue;
}

}  // namespace bsmm
