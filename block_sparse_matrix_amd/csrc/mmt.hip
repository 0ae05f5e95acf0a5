// fprop / bprop for 32x32 blocks over long minibatches, by output-block groups.
//
// fprop (kiteco/blocksparse README, "API Documentation" › BlocksparseMatMul.__call__)
// computes y = x · W̃ with W̃ the C x K matrix whose b x b blocks are the stored
// weights where the layout is 1 and zero elsewhere; bprop computes dx = dy · W̃ᵀ.
//
// Here a workgroup owns 256 minibatch rows of 8 consecutive output blocks (256
// output features) and walks the contraction blocks that hold any of them (the
// layout compiler's group table, ascending).  Each step loads one activation slab
// (256 rows x 32 features) and the step's present weight blocks; the weights are
// staged in LDS, where all 4 waves read them.  The 4 waves each take 64 rows and all
// 8 output blocks, so the slab is read from global memory once for up to 8 blocks
// and every wave does the same matrix-core work at every step.  The 8 x 2 x 4 accumulator tiles of a wave (256 fp32 per lane) stay in
// registers for the whole walk and are written once at the end.
//
// Pipeline: PD register stages of global loads in flight, two LDS buffers, one
// barrier per step.  Workgroups are dealt so that an XCD works through whole
// minibatch tiles: the groups running together on one XCD read the same activation
// rows, which then come from that XCD's L2.
#include "common.h"

namespace bsmm {

template <int DT, int FA, int WAVES>
struct MTCfg {
    static constexpr int B = 32, OG = kGroupOut;
    static constexpr int NT = 256, NTW = NT / WAVES;   // minibatch rows per workgroup / wave
    static constexpr int QT = NTW / 16;                // 16-row tiles per wave
    static constexpr int THREADS = 64 * WAVES;
    static constexpr int CPT = 16 / WAVES;             // 16-byte chunks per thread: slab or weights
    // Features-last activations are read straight into operand fragments; features-
    // first ones are staged in LDS (rows of 256 minibatch values) and read transposed.
    static constexpr bool XL = FA == 0;
    static constexpr int XP = NT + 8;
    static constexpr int XTILE = XL ? B * XP : 0;
    static constexpr int WTILE = OG * B * B;   // weight blocks, unpadded, swizzled
    static constexpr int STAGE = XTILE + WTILE;   // elements per LDS buffer
    static constexpr int ECAP = kGroupMaxSteps;   // group entries held in LDS
};

// Weight tiles in LDS: 32 rows of 64 bytes, the four 16-byte chunks of row r permuted
// by chunk ^ wswz(r).  With this permutation the staging stores, the transposing
// fragment reads (fprop) and the row fragment reads (bprop) each touch every LDS bank
// at most once per pass, for 32 or 64 banks.
__device__ __forceinline__ int wswz(int r) { return (((r >> 1) ^ (r >> 2)) & 1) | ((((r >> 1) ^ (r >> 3)) & 1) << 1); }
__device__ __forceinline__ int widx(int r, int col) { return r * 32 + ((((col >> 3) ^ wswz(r)) << 3) | (col & 7)); }

template <int DT, int FA, bool TW, int WAVES, bool XF, int RD>
__global__ __launch_bounds__(64 * WAVES) void mmt_kernel(MMArgs a) {
    using Cfg = MTCfg<DT, FA, WAVES>;
    constexpr int B = Cfg::B, OG = Cfg::OG, NT = Cfg::NT, NTW = Cfg::NTW;
    constexpr int QT = Cfg::QT, THREADS = Cfg::THREADS, CPT = Cfg::CPT;
    constexpr int XP = Cfg::XP, STAGE = Cfg::STAGE, XTILE = Cfg::XTILE;
    constexpr bool XL = Cfg::XL;
    constexpr int S = 2;
    constexpr int SNT = 4, SG = 8;
    __shared__ __attribute__((aligned(16))) uint16_t smem[3 * STAGE];
    __shared__ __attribute__((aligned(16))) int lent[Cfg::ECAP * kGroupInts];

    // workgroup -> (minibatch tile, group).  The (tile, group) grid is cut into
    // super-tiles of SNT tiles x SG groups, one per XCD at a time (32 workgroups, one
    // per CU), dealt round-robin over the XCDs: the groups of a super-tile share each
    // activation slab and its tiles share each weight block through the XCD's L2.
    const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
    const int sgs = (a.ngroups + SG - 1) / SG;
    const int k = (slot / (SNT * SG)) * 8 + xcd, idx = slot % (SNT * SG);
    const int nt = (k / sgs) * SNT + idx / SG, gi = (k % sgs) * SG + idx % SG;
    if (nt >= a.ntiles || gi >= a.ngroups) return;   // whole workgroup
    const int n0 = nt * NT;
    const int N = (int)a.N;
    const int gbeg = a.gptr[gi], nsteps = a.gptr[gi + 1] - gbeg;
    const int* __restrict__ gent = a.gent + (int64_t)gbeg * kGroupInts;

    const int t = threadIdx.x, lane = t & 63;
    const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
    const int m16 = lane & 15, g4 = lane >> 4;
    const int nw0 = wave * NTW;
    const rsrc_t rin = make_rsrc(a.in, a.in_bytes);
    const rsrc_t rw = make_rsrc(a.w, a.w_bytes);

    // Activation offsets (the step adds a scalar part).  XL: 16-byte chunk i of the
    // slab (32 rows of 256 values), 32 lanes per row.  Otherwise: fragment q of this
    // wave, lane (m16, g4) -> row nw0 + 16q + m16, features 8*g4 .. +7.
    constexpr int XN = XL ? CPT : QT;
    uint32_t xo[XN];
    int xl[XN];
#pragma unroll
    for (int i = 0; i < XN; i++) {
        if constexpr (XL) {
            const int q = t + THREADS * i, r = q >> 5, ch = q & 31;
            const int n = n0 + 8 * ch;
            xo[i] = n < N ? ((uint32_t)r * N + n) * S : kOffLane;
            xl[i] = r * XP + 8 * ch;
        } else {
            const int n = n0 + nw0 + 16 * i + m16;
            xo[i] = n < N ? ((uint32_t)n * a.fin + 8 * g4) * S : kOffLane;
            xl[i] = 0;
        }
    }
    // weights: instruction i of wave w stages half (w & 1) of block slot
    // i*WAVES/2 + (w >> 1), 1 KB contiguous per instruction; the block's id is a scalar
    // offset
    const int wh = (t >> 6) & 1, wsl = __builtin_amdgcn_readfirstlane(t >> 7);
    const int wrow = 16 * wh + (lane >> 2);
    const uint32_t wo = (uint32_t)(wrow * B + 8 * (t & 3)) * S;
    const int wl = widx(wrow, 8 * (t & 3));

    // The group's entries are copied to LDS once; an entry is read there (before the
    // barrier that precedes its loads) so no global load sits between two steps.
    for (int i = t; i < nsteps * kGroupInts; i += THREADS) lent[i] = gent[i];

    struct Stage {
        u32x4 x[XL ? XN : 1], w[CPT];   // x: staged activations (features first)
        int mask, c;   // of the step whose loads the slot holds (or will hold)
    };
    struct XFrag {     // directly loaded activation fragments (features last)
        u32x4 x[XL ? 1 : XN];
    };
    struct Ent {
        int c, mask, id[CPT];
    };
    // one entry: three broadcast LDS reads, then scalars (index clamped, mask cleared
    // past the end, so nothing here branches)
    auto read_ent = [&](int s) -> Ent {
        const bool sv = s < nsteps;   // workgroup-uniform
        typedef int i32x4 __attribute__((ext_vector_type(4)));
        const BSMM_LDS i32x4* e = (const BSMM_LDS i32x4*)(lent + (sv ? s : 0) * kGroupInts);
        const i32x4 e0 = e[0], e1 = e[1], e2 = e[2];
        const int ids[8] = {e0.z, e0.w, e1.x, e1.y, e1.z, e1.w, e2.x, e2.y};
        Ent r;
        r.c = __builtin_amdgcn_readfirstlane(e0.x);
        const int mk = __builtin_amdgcn_readfirstlane(e0.y);
        r.mask = sv ? mk : 0;
#pragma unroll
        for (int i = 0; i < CPT; i++) {
            int v = __builtin_amdgcn_readfirstlane(ids[i * (WAVES / 2)]);
#pragma unroll
            for (int k = 1; k < WAVES / 2; k++)
                if (wsl == k) v = __builtin_amdgcn_readfirstlane(ids[i * (WAVES / 2) + k]);
            r.id[i] = v;
        }
        return r;
    };
    auto issue_x = [&](u32x4* dst, const Stage& st) {   // activations of the step recorded in st
        uint32_t xs;
        if constexpr (XL)
            xs = st.mask ? (uint32_t)st.c * B * N * S : kOffOff;
        else
            xs = st.mask ? (uint32_t)st.c * B * S : kOffOff;
#pragma unroll
        for (int i = 0; i < XN; i++) dst[i] = bload128(rin, xo[i], xs);
    };
    auto issue_w = [&](Stage& st, const Ent& e) {
        st.mask = e.mask;
        st.c = e.c;
#pragma unroll
        for (int i = 0; i < CPT; i++) {
            const bool wv = (e.mask >> (i * (WAVES / 2) + wsl)) & 1;   // wave-uniform
            st.w[i] = bload128(rw, wo, wv ? (uint32_t)e.id[i] * B * B * S : kOffOff);
        }
    };
    auto stage_lds = [&](const Stage& st, BSMM_LDS uint16_t* buf) {
        if constexpr (XL) {
#pragma unroll
            for (int i = 0; i < XN; i++) lds_store16(buf + xl[i], st.x[i]);
        }
#pragma unroll
        for (int i = 0; i < CPT; i++) lds_store16(buf + XTILE + (i * (WAVES / 2) + wsl) * B * B + wl, st.w[i]);
    };

    f32x4 acc[OG][2][QT];
#pragma unroll
    for (int j = 0; j < OG; j++)
#pragma unroll
        for (int kt = 0; kt < 2; kt++)
#pragma unroll
            for (int q = 0; q < QT; q++) acc[j][kt][q] = f32x4{0.f, 0.f, 0.f, 0.f};

    // Lane offsets (elements, within a block) of the weight fragment reads, computed
    // once: the block and buffer then only add a uniform offset.
    int wfo[2][2];
#pragma unroll
    for (int kt = 0; kt < 2; kt++) {
        if constexpr (TW) {   // bprop: output index = block row, contraction along the row
            wfo[kt][0] = widx(16 * kt + m16, 8 * g4);
            wfo[kt][1] = 0;
        } else {              // fprop: output index = block column, contraction down it
            const int r0 = 8 * g4 + (m16 >> 2), c = 16 * kt + 4 * (m16 & 3);
            wfo[kt][0] = widx(r0, c);
            wfo[kt][1] = widx(r0 + 4, c);
        }
    }
    auto wfrag = [&](const BSMM_LDS uint16_t* wt, int j, int kt) -> u32x4 {
        const BSMM_LDS uint16_t* blk = wt + j * B * B;
        if constexpr (TW) {
            return *reinterpret_cast<const BSMM_LDS u32x4*>(blk + wfo[kt][0]);
        } else {   // the transposing read of wfrag_tr
            const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((BSMM_LDS i16x4*)(blk + wfo[kt][0]));
            const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((BSMM_LDS i16x4*)(blk + wfo[kt][1]));
            const u32x2 ul = __builtin_bit_cast(u32x2, lo), uh = __builtin_bit_cast(u32x2, hi);
            return u32x4{ul.x, ul.y, uh.x, uh.y};
        }
    };
    // Operand fragments of one step, in registers: the present weight blocks (and, for
    // features-first activations, this wave's activation rows) read from an LDS buffer.
    struct Frags {
        u32x4 w[OG][2];
        u32x4 x[XL ? QT : 1];
    };
    // blocks [j0, j1) of a step
    auto read_frags = [&](Frags& f, const BSMM_LDS uint16_t* buf, int mask, int j0 = 0, int j1 = kGroupOut) {
        if constexpr (XL) {
            if (j0 == 0) {
#pragma unroll
                for (int q = 0; q < QT; q++) f.x[q] = frag_tr16(buf, XP, nw0 + 16 * q, lane);
            }
        }
#pragma unroll
        for (int j = j0; j < j1; j++)
            if ((mask >> j) & 1) {   // workgroup-uniform
                f.w[j][0] = wfrag(buf + XTILE, j, 0);
                f.w[j][1] = wfrag(buf + XTILE, j, 1);
            }
    };
    auto compute = [&](const Frags& f, const XFrag& st, int mask, int j0 = 0, int j1 = kGroupOut) {
#pragma unroll
        for (int j = j0; j < j1; j++)
            if ((mask >> j) & 1) {   // workgroup-uniform
#pragma unroll
                for (int q = 0; q < QT; q++) {
                    const u32x4 xf = XL ? f.x[q] : st.x[q];
                    if constexpr (FA == 1) {
                        mma<DT>(acc[j][0][q], f.w[j][0], xf);
                        mma<DT>(acc[j][1][q], f.w[j][1], xf);
                    } else {
                        mma<DT>(acc[j][0][q], xf, f.w[j][0]);
                        mma<DT>(acc[j][1][q], xf, f.w[j][1]);
                    }
                }
            }
    };

    // Software pipeline, one barrier per step, three LDS buffers (step s in buffer
    // s % 3), RD register slots of weight loads.  At step s: weights (and staged
    // activations) of step s+1, loaded RD steps earlier, go to LDS; after the barrier
    // the loads for step s+1+RD refill the freed slot, and the products of step s run;
    // directly loaded activation fragments are loaded two steps ahead.  With XF the fragments of step s+1 are read into a second
    // register set during step s (their LDS latency hides behind step s's products);
    // otherwise step s reads its own fragments, and the other wave on the SIMD covers
    // the wait.  A buffer is rewritten two barriers after its last read, and every
    // barrier waits for the LDS reads before it.  No branch surrounds a global load, so
    // the compiler waits only for the data each instruction consumes.  Steps past the
    // end carry mask 0 and no-op loads.
    Stage ring[RD];
    XFrag xr[2];   // features last: activation fragments of steps s, s+1 (by parity)
    Frags fr[XF ? 2 : 1];
    int fmask[2];
    BSMM_LDS uint16_t* lds = (BSMM_LDS uint16_t*)smem;
    __syncthreads();   // entries in LDS
    {
        int m0 = 0;
#pragma unroll
        for (int k = 0; k < RD; k++) {
            const Ent e = read_ent(k);
            if (k == 0) m0 = e.mask;
            issue_w(ring[k], e);
            if constexpr (XL)
                issue_x(ring[k].x, ring[k]);   // staged with step k's weights
            else if (k < 2)
                issue_x(xr[k].x, ring[k]);     // step k's fragments
        }
        stage_lds(ring[0], lds);
        fmask[0] = m0;
        fmask[1] = 0;
        issue_w(ring[0], read_ent(RD));
        if constexpr (XL) issue_x(ring[0].x, ring[0]);
        __syncthreads();
        if constexpr (XF) read_frags(fr[0], lds, fmask[0]);
    }
    for (int s0 = 0; s0 < nsteps; s0 += RD) {
        const int b0 = s0 % 3;
#pragma unroll
        for (int r = 0; r < RD; r++) {
            const int s = s0 + r, rn = (r + 1) % RD, p = r & 1;
            const int bc = (b0 + r) % 3, bn = (b0 + r + 1) % 3;   // buffers of steps s, s+1
            stage_lds(ring[rn], lds + bn * STAGE);
            const int m1 = ring[rn].mask;
            const Ent en = read_ent(s + 1 + RD);
            __syncthreads();
            issue_w(ring[rn], en);
            if constexpr (XL) issue_x(ring[rn].x, ring[rn]);
            if constexpr (XF) {
                read_frags(fr[p ^ 1], lds + bn * STAGE, m1);
                compute(fr[p], xr[p], fmask[p]);
            } else {   // two halves: fewer fragment registers live at once
#pragma unroll
                for (int h = 0; h < OG; h += OG / 2) {
                    read_frags(fr[0], lds + bc * STAGE, fmask[p], h, h + OG / 2);
                    compute(fr[0], xr[p], fmask[p], h, h + OG / 2);
                }
            }
            fmask[p ^ 1] = m1;
            if constexpr (!XL) issue_x(xr[p].x, ring[(r + 2) % RD]);   // step s+2
        }
    }

    // epilogue: FA 1 holds D[out][n] (4 consecutive outputs of one row per lane),
    // FA 0 holds D[n][out] (4 consecutive rows of one output)
#pragma unroll
    for (int j = 0; j < OG; j++) {
        const int ob = gi * OG + j;
        if (ob >= a.nout) break;
#pragma unroll
        for (int kt = 0; kt < 2; kt++)
#pragma unroll
            for (int q = 0; q < QT; q++) {
                if constexpr (FA == 1) {
                    const int n = n0 + nw0 + 16 * q + m16;
                    const int o = ob * B + 16 * kt + 4 * g4;
                    if (n < N) store4<DT>(a.out, (int64_t)n * a.fout + o, acc[j][kt][q]);
                } else {
                    const int n = n0 + nw0 + 16 * q + 4 * g4;
                    const int o = ob * B + 16 * kt + m16;
                    if (n < N) store4<DT>(a.out, (int64_t)o * N + n, acc[j][kt][q]);
                }
            }
    }
}

template <int DT, int FA, bool TW, int WAVES, bool XF, int RD>
static hipError_t launch_mmt(MMArgs a, hipStream_t st, int pass) {
    a.ntiles = (int)((a.N + 255) / 256);
    // super-tiles of 4 minibatch tiles x 8 groups, 32 workgroups each
    const int64_t supers = (int64_t)((a.ntiles + 3) / 4) * ((a.ngroups + 7) / 8);
    const int64_t grid = ((supers + 7) / 8) * 8 * 32;
    if (grid > INT32_MAX / 2) return hipErrorInvalidConfiguration;
    return launch(pass, mmt_kernel<DT, FA, TW, WAVES, XF, RD>, dim3((unsigned)grid), dim3(64 * WAVES), st, a);
}

hipError_t launch_mm_groups(const MMArgs& a, int dt, int fa, bool transw, void* stream, int pass) {
    hipStream_t st = (hipStream_t)stream;
    // Features-last: 8 waves (two per SIMD), each step reads its own fragments.
    // Features-first (activations staged in LDS too): 4 waves with a second fragment
    // set, read one step ahead (the extra staging registers leave no room for 8).
    switch ((dt == BSMM_F16 ? 4 : 0) + fa * 2 + (transw ? 1 : 0)) {
    case 0: return launch_mmt<BSMM_BF16, 0, false, 4, true, 2>(a, st, pass);
    case 1: return launch_mmt<BSMM_BF16, 0, true, 4, true, 2>(a, st, pass);
    case 2: return launch_mmt<BSMM_BF16, 1, false, 8, false, 2>(a, st, pass);
    case 3: return launch_mmt<BSMM_BF16, 1, true, 8, false, 2>(a, st, pass);
    case 4: return launch_mmt<BSMM_F16, 0, false, 4, true, 2>(a, st, pass);
    case 5: return launch_mmt<BSMM_F16, 0, true, 4, true, 2>(a, st, pass);
    case 6: return launch_mmt<BSMM_F16, 1, false, 8, false, 2>(a, st, pass);
    case 7: return launch_mmt<BSMM_F16, 1, true, 8, false, 2>(a, st, pass);
    }
    return hipErrorInvalidValue;
}

}  // namespace bsmm
