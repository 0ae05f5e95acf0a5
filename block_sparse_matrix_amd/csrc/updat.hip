// Weight gradient (updat) of the block-sparse product on gfx950.
//
//   dW[id(c,k)][p][q] = sum over steps t < G, minibatch rows n of  x_t[n, c*b+p] . dy_t[n, k*b+q]
// for the present blocks only (kiteco/blocksparse README, "API Documentation" ›
// blocksparse.matmul › __call__ with dw_dtype; group_param_grads sums up to 8 steps
// that share W into one product).  feature_axis 0 reads x_t[c*b+p, n], dy_t[k*b+q, n].
//
// Each block has exactly one writer, so there are no atomics and the result does not
// depend on scheduling.  A wave walks a run of blocks; for each it contracts over the
// G*N minibatch rows in steps of 32 (16-bit) or 16 (fp32) rows, with D steps of
// global loads in flight in a register ring that runs across block boundaries.  The
// contraction index (the minibatch row) is the slow index of both operands when
// feature_axis = 1: 16-bit rows are staged through a wave-private LDS tile and read
// back transposed; fp32 uses 4-byte loads.  With feature_axis = 0 both operands are
// read directly with 16-byte loads.  The 16x16 result tiles are computed as
// D[q][p] so that each lane stores four consecutive dW values of one row.
#include <cstdlib>

#include "common.h"

namespace bsmm {

template <int DT, int B, int FA, int D>
__global__ __launch_bounds__(256) void updat_kernel(UpArgs a) {
    using T = typename Elt<DT>::T;
    constexpr int VEC = Elt<DT>::VEC, KS = 4 * VEC;
    constexpr int PT = (B + 15) / 16;
    constexpr bool TR = FA == 1 && DT != BSMM_F32;
    constexpr int WCH = B / 8;
    constexpr int RR = TR ? (4 * B + 63) / 64 : PT;
    constexpr int PITCH = PT * 16 + 8;
    constexpr int TILE = 32 * PITCH;
    __shared__ __attribute__((aligned(16))) uint16_t lds[TR ? 4 * 2 * TILE : 8];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int r16 = lane & 15, g = lane >> 4;
    const int64_t N = a.N;
    const int spt = (int)((N + KS - 1) / KS);
    const int nsb = a.G * spt;   // steps per block
    const int64_t b0 = ((int64_t)blockIdx.x * 4 + wave) * a.bpw;
    if (b0 >= a.nnz) return;   // no workgroup barrier in this kernel
    const int nblk = (int)((a.nnz - b0) < a.bpw ? (a.nnz - b0) : a.bpw);
    const int items = nsb > 0 ? nblk * nsb : 0;
    const bool xvec = (N % VEC) == 0;
    // Coordinates of this wave's blocks, one block per lane, read back with readlane:
    // the ring's loads then depend on no other global load.
    int cl = 0, kl = 0;
    if (lane < nblk) {
        cl = a.coords[2 * (b0 + lane)];
        kl = a.coords[2 * (b0 + lane) + 1];
    }

    BSMM_LDS uint16_t* xt = (BSMM_LDS uint16_t*)lds + wave * 2 * TILE;
    BSMM_LDS uint16_t* dt = xt + TILE;
    if constexpr (TR && B == 8) {
        for (int i = lane; i < 2 * TILE; i += 64) xt[i] = 0;
    }

    struct SlotU {
        u32x4 x[RR];
        u32x4 d[RR];
    };

    // Loads are issued unconditionally (clamped address, value masked afterwards) so
    // the count of loads in flight does not depend on the path taken.
    auto load_slot = [&](SlotU& sl, int it0) {
        const bool iv = it0 < items;   // wave-uniform
        const int it = iv ? it0 : 0;
        const int j = it / nsb, st = it % nsb;
        const int t = st / spt;
        const int64_t nb = (int64_t)(st % spt) * KS;
        const int c = __builtin_amdgcn_readlane(cl, j), k = __builtin_amdgcn_readlane(kl, j);
        const T* __restrict__ x = (const T*)a.xs[t];
        const T* __restrict__ dy = (const T*)a.dys[t];
        if constexpr (TR) {
#pragma unroll
            for (int ri = 0; ri < RR; ri++) {
                const int ch0 = lane + 64 * ri;
                const bool chv = ch0 < 4 * B;
                const int ch = chv ? ch0 : 0;
                const int r = ch / WCH, cc = ch % WCH;
                const int64_t n = nb + r;
                const bool ok = iv && chv && n < N;
                sl.x[ri] = load_vec<DT>(or_zero(ok, x + n * a.C + (int64_t)c * B + cc * 8));
                sl.d[ri] = load_vec<DT>(or_zero(ok, dy + n * a.K + (int64_t)k * B + cc * 8));
            }
        } else if constexpr (FA == 1) {   // fp32, minibatch-major: four rows per fragment
            const int64_t n = nb + 4 * g;
            const int nval = iv ? (int)(N - n >= 4 ? 4 : (N - n > 0 ? N - n : 0)) : 0;
#pragma unroll
            for (int pt = 0; pt < PT; pt++) {
                const int p = pt * 16 + r16;
                const int nv = p < B ? nval : 0;
                sl.x[pt] = load_strided<DT>(x + n * a.C + (int64_t)c * B + p, a.C, nv);
                sl.d[pt] = load_strided<DT>(dy + n * a.K + (int64_t)k * B + p, a.K, nv);
            }
        } else {   // feature-major: contraction index contiguous
            const int64_t n = nb + g * VEC;
#pragma unroll
            for (int pt = 0; pt < PT; pt++) {
                const int p = pt * 16 + r16;
                const T* xp = x + ((int64_t)c * B + p) * N + n;
                const T* dp = dy + ((int64_t)k * B + p) * N + n;
                const bool ok = iv && p < B && n < N;
                if (xvec) {
                    sl.x[pt] = load_vec<DT>(or_zero(ok, xp));
                    sl.d[pt] = load_vec<DT>(or_zero(ok, dp));
                } else {
                    const int nval = ok ? (int)(N - n >= VEC ? VEC : N - n) : 0;
                    sl.x[pt] = load_strided<DT>(or_zero(ok, xp), 1, nval);
                    sl.d[pt] = load_strided<DT>(or_zero(ok, dp), 1, nval);
                }
            }
        }
    };

    f32x4 acc[PT][PT];
#pragma unroll
    for (int i = 0; i < PT; i++)
#pragma unroll
        for (int j = 0; j < PT; j++) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    auto compute_slot = [&](const SlotU& sl, int it) {
        u32x4 xf[PT], df[PT];
        if constexpr (TR) {
#pragma unroll
            for (int ri = 0; ri < RR; ri++) {
                const int ch = lane + 64 * ri;
                if (ch < 4 * B) {
                    const int off = (ch / WCH) * PITCH + (ch % WCH) * 8;
                    lds_store16(xt + off, sl.x[ri]);
                    lds_store16(dt + off, sl.d[ri]);
                }
            }
            wave_lds_order();
#pragma unroll
            for (int pt = 0; pt < PT; pt++) {
                xf[pt] = frag_tr16(xt, PITCH, 16 * pt, lane);
                df[pt] = frag_tr16(dt, PITCH, 16 * pt, lane);
            }
            wave_lds_order();
        } else {
#pragma unroll
            for (int pt = 0; pt < PT; pt++) {
                xf[pt] = sl.x[pt];
                df[pt] = sl.d[pt];
            }
        }
#pragma unroll
        for (int qt = 0; qt < PT; qt++)
#pragma unroll
            for (int pt = 0; pt < PT; pt++) mma<DT>(acc[qt][pt], df[qt], xf[pt]);   // D[q][p]
        if (it < items && (it % nsb) == nsb - 1) {   // last step of a block: store, restart
            const int64_t id = b0 + it / nsb;
            const int64_t base = id * B * B;
#pragma unroll
            for (int qt = 0; qt < PT; qt++)
#pragma unroll
                for (int pt = 0; pt < PT; pt++) {
                    const int p = pt * 16 + r16, q = qt * 16 + 4 * g;
                    if (p < B && q < B) {
                        const int64_t idx = base + p * B + q;
                        if (a.dwdt == BSMM_F32)
                            store4<BSMM_F32>(a.dw, idx, acc[qt][pt]);
                        else if (a.dwdt == BSMM_BF16)
                            store4<BSMM_BF16>(a.dw, idx, acc[qt][pt]);
                        else
                            store4<BSMM_F16>(a.dw, idx, acc[qt][pt]);
                    }
                    acc[qt][pt] = f32x4{0.f, 0.f, 0.f, 0.f};
                }
        }
    };

    if (items == 0) {
        // N = 0: every block of this wave is the empty sum
        for (int j = 0; j < nblk; j++) {
            const int64_t base = (b0 + j) * B * B;
            for (int e = lane; e < B * B; e += 64) store_elt(a.dw, base + e, 0.f, a.dwdt);
        }
        return;
    }

    SlotU ring[D];
#pragma unroll
    for (int i = 0; i < D; i++) load_slot(ring[i], i);
    for (int j = 0; j < items; j += D) {
#pragma unroll
        for (int i = 0; i < D; i++) {
            compute_slot(ring[i], j + i);   // items past the end add zeros and store nothing
            load_slot(ring[i], j + i + D);
        }
    }
}

// BSMM_UPDAT_VARIANT=<n> (read once) forces a ring depth / blocks-per-wave pair for
// A/B measurements; 0 or unset: automatic.
static int updat_variant() {
    static const int v = [] {
        const char* e = getenv("BSMM_UPDAT_VARIANT");
        return e ? atoi(e) : 0;
    }();
    return v;
}

template <int DT, int B, int FA, int D>
static hipError_t launch_updat_cfg(UpArgs a, int bpw, hipStream_t st) {
    a.bpw = bpw;
    const int64_t waves = ((int64_t)a.nnz + bpw - 1) / bpw;
    const int64_t grid = (waves + 3) / 4;
    return launch(BSMM_PASS_UPDAT, updat_kernel<DT, B, FA, D>, dim3((unsigned)grid), dim3(256), st, a);
}

template <int DT, int B, int FA>
static hipError_t launch_updat_t(const UpArgs& a, hipStream_t st) {
    switch (updat_variant()) {
    case 1: return launch_updat_cfg<DT, B, FA, 2>(a, 1, st);
    case 2: return launch_updat_cfg<DT, B, FA, 4>(a, 1, st);
    case 3: return launch_updat_cfg<DT, B, FA, 2>(a, 2, st);
    case 4: return launch_updat_cfg<DT, B, FA, 4>(a, 2, st);
    case 5: return launch_updat_cfg<DT, B, FA, 4>(a, 4, st);
    case 6: return launch_updat_cfg<DT, B, FA, 8>(a, 4, st);
    default: break;
    }
    // One block per wave: a wave loads, contracts, stores its block and exits, so no
    // wave ever waits on its own stores (stores count in the same counter as loads).
    return launch_updat_cfg<DT, B, FA, 4>(a, 1, st);
}

template <int DT>
static hipError_t launch_updat_dt(const UpArgs& a, int b, int fa, hipStream_t st) {
    switch (b * 2 + fa) {
    case 16: return launch_updat_t<DT, 8, 0>(a, st);
    case 17: return launch_updat_t<DT, 8, 1>(a, st);
    case 32: return launch_updat_t<DT, 16, 0>(a, st);
    case 33: return launch_updat_t<DT, 16, 1>(a, st);
    case 64: return launch_updat_t<DT, 32, 0>(a, st);
    case 65: return launch_updat_t<DT, 32, 1>(a, st);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_updat(const UpArgs& a, int dt, int b, int fa, void* stream) {
    hipStream_t st = (hipStream_t)stream;
    if (a.nnz == 0) return hipSuccess;
    switch (dt) {
    case BSMM_F32: return launch_updat_dt<BSMM_F32>(a, b, fa, st);
    case BSMM_BF16: return launch_updat_dt<BSMM_BF16>(a, b, fa, st);
    case BSMM_F16: return launch_updat_dt<BSMM_F16>(a, b, fa, st);
    }
    return hipErrorInvalidValue;
}

}  // namespace bsmm
