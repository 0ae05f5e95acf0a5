// fprop / bprop for 32x32 blocks over long minibatches, by output-block groups.
//
// fprop (kiteco/blocksparse README, "API Documentation" › BlocksparseMatMul.__call__)
// computes y = x · W̃ with W̃ the C x K matrix whose b x b blocks are the stored
// weights where the layout is 1 and zero elsewhere; bprop computes dx = dy · W̃ᵀ.
//
// Here a workgroup owns 256 minibatch rows of 8 consecutive output blocks (256
// output features) and walks the contraction blocks that hold any of them (the
// layout compiler's group table, ascending).  Each step stages one activation slab
// (256 rows x 32 features) and the step's present weight blocks in LDS; the 4 waves
// each take 64 rows and all 8 output blocks, so the slab is read from global memory
// once for up to 8 blocks and every wave does the same matrix-core work at every
// step.  The 8 x 2 x 4 accumulator tiles of a wave (256 fp32 per lane) stay in
// registers for the whole walk and are written once at the end.
//
// Pipeline: PD register stages of global loads in flight, two LDS buffers, one
// barrier per step.  Workgroups are dealt so that an XCD works through whole
// minibatch tiles: the groups running together on one XCD read the same activation
// rows, which then come from that XCD's L2.
#include "common.h"

namespace bsmm {

template <int DT, int FA>
struct MTCfg {
    static constexpr int B = 32, OG = kGroupOut;
    static constexpr int NT = 256, NTW = 64;              // minibatch rows per workgroup / wave
    static constexpr int XP = FA == 1 ? B + 8 : NT + 8;   // activation tile pitch, elements
    static constexpr int XTILE = (FA == 1 ? NT : B) * XP;
    static constexpr int WP = B + 8;                      // weight tile pitch
    static constexpr int WTILE = OG * B * WP;
    static constexpr int STAGE = XTILE + WTILE;           // elements per LDS buffer
    static constexpr int ECAP = kGroupMaxSteps;           // group entries held in LDS
};

template <int DT, int FA, bool TW, int PD>
__global__ __launch_bounds__(256) void mmt_kernel(MMArgs a) {
    using Cfg = MTCfg<DT, FA>;
    constexpr int B = Cfg::B, OG = Cfg::OG, NT = Cfg::NT, NTW = Cfg::NTW;
    constexpr int XP = Cfg::XP, WP = Cfg::WP, STAGE = Cfg::STAGE, XTILE = Cfg::XTILE;
    constexpr int S = 2;
    __shared__ __attribute__((aligned(16))) uint16_t smem[2 * STAGE];
    __shared__ __attribute__((aligned(16))) int lent[Cfg::ECAP * kGroupInts];

    // workgroup -> (minibatch tile, group): XCD x takes the x-th contiguous range
    const int total = a.ntiles * a.ngroups;
    const int per = (total + 7) / 8;
    const int u = (blockIdx.x & 7) * per + (blockIdx.x >> 3);
    if (u >= total) return;   // whole workgroup
    const int nt = u / a.ngroups, gi = u % a.ngroups;
    const int n0 = nt * NT;
    const int N = (int)a.N;
    const int gbeg = a.gptr[gi], nsteps = a.gptr[gi + 1] - gbeg;
    const int* __restrict__ gent = a.gent + (int64_t)gbeg * kGroupInts;

    const int t = threadIdx.x, lane = t & 63;
    const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
    const rsrc_t rin = make_rsrc(a.in, a.in_bytes);
    const rsrc_t rw = make_rsrc(a.w, a.w_bytes);

    // per-lane parts of the load offsets (the step adds a scalar part)
    uint32_t xo[4];
    int xl[4];   // LDS element offset of each 16-byte chunk of the activation slab
#pragma unroll
    for (int i = 0; i < 4; i++) {
        if constexpr (FA == 1) {
            const int n = n0 + t;
            xo[i] = n < N ? (uint32_t)n * a.fin * S + 16 * i : kOffLane;
            xl[i] = t * XP + 8 * i;
        } else {
            const int q = t + 256 * i, r = q >> 5, ch = q & 31;
            const int n = n0 + 8 * ch;
            xo[i] = n < N ? ((uint32_t)r * N + n) * S : kOffLane;
            xl[i] = r * XP + 8 * ch;
        }
    }
    const int wj = t >> 5, wr = t & 31;   // weight block slot and row this thread stages

    // The group's entries are copied to LDS once; an entry is read there (before the
    // barrier that precedes its loads) so no global load sits between two steps.
    for (int i = t; i < nsteps * kGroupInts; i += 256) lent[i] = gent[i];

    struct Stage {
        u32x4 x[4], w[4];
        int mask;
    };
    struct Ent {
        int c, mask, id;
    };
    auto read_ent = [&](int s) -> Ent {
        const bool sv = s < nsteps;   // workgroup-uniform
        const int* e = lent + (sv ? s : 0) * kGroupInts;
        Ent r;
        r.c = __builtin_amdgcn_readfirstlane(e[0]);
        r.mask = sv ? __builtin_amdgcn_readfirstlane(e[1]) : 0;
        r.id = e[2 + wj];
        return r;
    };
    auto issue = [&](Stage& st, const Ent& e) {
        st.mask = e.mask;
        uint32_t xs;
        if constexpr (FA == 1)
            xs = e.mask ? (uint32_t)e.c * B * S : kOffOff;
        else
            xs = e.mask ? (uint32_t)e.c * B * N * S : kOffOff;
#pragma unroll
        for (int i = 0; i < 4; i++) st.x[i] = bload128(rin, xo[i], xs);
        const bool wv = (e.mask >> wj) & 1;
        const uint32_t wo = wv ? ((uint32_t)e.id * B * B + wr * B) * S : kOffLane;
#pragma unroll
        for (int i = 0; i < 4; i++) st.w[i] = bload128(rw, wo, 16 * i);
    };
    auto stage_lds = [&](const Stage& st, BSMM_LDS uint16_t* buf) {
#pragma unroll
        for (int i = 0; i < 4; i++) lds_store16(buf + xl[i], st.x[i]);
#pragma unroll
        for (int i = 0; i < 4; i++) lds_store16(buf + XTILE + (wj * B + wr) * WP + 8 * i, st.w[i]);
    };

    f32x4 acc[OG][2][4];
#pragma unroll
    for (int j = 0; j < OG; j++)
#pragma unroll
        for (int kt = 0; kt < 2; kt++)
#pragma unroll
            for (int q = 0; q < 4; q++) acc[j][kt][q] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int m16 = lane & 15, g4 = lane >> 4;
    const int nw0 = wave * NTW;
    auto wfrag = [&](const BSMM_LDS uint16_t* wt, int j, int kt) -> u32x4 {
        if constexpr (TW)   // bprop: output index = block row, contraction along the row
            return *reinterpret_cast<const BSMM_LDS u32x4*>(wt + (j * B + 16 * kt + m16) * WP + 8 * g4);
        else                // fprop: output index = block column, contraction down it
            return frag_tr16(wt + j * B * WP, WP, 16 * kt, lane);
    };
    auto compute = [&](const BSMM_LDS uint16_t* buf, int mask) {
        const BSMM_LDS uint16_t* xt = buf;
        const BSMM_LDS uint16_t* wt = buf + XTILE;
        u32x4 xf[4];
#pragma unroll
        for (int q = 0; q < 4; q++) {
            if constexpr (FA == 1)
                xf[q] = *reinterpret_cast<const BSMM_LDS u32x4*>(xt + (nw0 + 16 * q + m16) * XP + 8 * g4);
            else
                xf[q] = frag_tr16(xt, XP, nw0 + 16 * q, lane);
        }
        if (mask == 0) return;
        // the next present block's fragments are read while this block's products run
        int j0 = __builtin_ctz(mask);
        u32x4 cur0 = wfrag(wt, j0, 0), cur1 = wfrag(wt, j0, 1);
#pragma unroll
        for (int j = 0; j < OG; j++) {
            if ((mask >> j) & 1) {   // workgroup-uniform
                const int rest = mask & ~((2 << j) - 1);
                const int jn = rest ? __builtin_ctz(rest) : j;
                const u32x4 nxt0 = wfrag(wt, jn, 0), nxt1 = wfrag(wt, jn, 1);
#pragma unroll
                for (int q = 0; q < 4; q++) {
                    if constexpr (FA == 1) {
                        mma<DT>(acc[j][0][q], cur0, xf[q]);
                        mma<DT>(acc[j][1][q], cur1, xf[q]);
                    } else {
                        mma<DT>(acc[j][0][q], xf[q], cur0);
                        mma<DT>(acc[j][1][q], xf[q], cur1);
                    }
                }
                cur0 = nxt0;
                cur1 = nxt1;
            }
        }
    };

    Stage ring[PD];
    BSMM_LDS uint16_t* lds = (BSMM_LDS uint16_t*)smem;
    __syncthreads();   // entries in LDS
    if (nsteps > 0) {
#pragma unroll
        for (int i = 0; i < PD; i++) issue(ring[i], read_ent(i));
    }
    for (int s0 = 0; s0 < nsteps; s0 += PD) {
#pragma unroll
        for (int i = 0; i < PD; i++) {
            const int s = s0 + i;
            if (s < nsteps) {   // workgroup-uniform
                BSMM_LDS uint16_t* buf = lds + (s & 1) * STAGE;
                stage_lds(ring[i], buf);
                const int mask = ring[i].mask;
                const Ent en = read_ent(s + PD);
                __syncthreads();
                issue(ring[i], en);
                compute(buf, mask);
            }
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
            for (int q = 0; q < 4; q++) {
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

template <int DT, int FA, bool TW, int PD>
static hipError_t launch_mmt(MMArgs a, hipStream_t st, int pass) {
    a.ntiles = (int)((a.N + 255) / 256);
    const int64_t total = (int64_t)a.ntiles * a.ngroups;
    if (total > INT32_MAX / 2) return hipErrorInvalidConfiguration;
    const int64_t grid = ((total + 7) / 8) * 8;
    return launch(pass, mmt_kernel<DT, FA, TW, PD>, dim3((unsigned)grid), dim3(256), st, a);
}

hipError_t launch_mm_groups(const MMArgs& a, int dt, int fa, bool transw, void* stream, int pass) {
    hipStream_t st = (hipStream_t)stream;
    constexpr int PD = 2;
    switch ((dt == BSMM_F16 ? 4 : 0) + fa * 2 + (transw ? 1 : 0)) {
    case 0: return launch_mmt<BSMM_BF16, 0, false, PD>(a, st, pass);
    case 1: return launch_mmt<BSMM_BF16, 0, true, PD>(a, st, pass);
    case 2: return launch_mmt<BSMM_BF16, 1, false, PD>(a, st, pass);
    case 3: return launch_mmt<BSMM_BF16, 1, true, PD>(a, st, pass);
    case 4: return launch_mmt<BSMM_F16, 0, false, PD>(a, st, pass);
    case 5: return launch_mmt<BSMM_F16, 0, true, PD>(a, st, pass);
    case 6: return launch_mmt<BSMM_F16, 1, false, PD>(a, st, pass);
    case 7: return launch_mmt<BSMM_F16, 1, true, PD>(a, st, pass);
    }
    return hipErrorInvalidValue;
}

}  // namespace bsmm
