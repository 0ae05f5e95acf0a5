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
#include <cstring>

#include "common.h"

namespace bsmm {

// Four consecutive dW values at element idx, in the weight-gradient dtype.  With a.acc
// the fp32 sum is first added to the value dW holds (decoded exactly), and the total
// is rounded once (RNE) to the storage type: dW += sum.  The stores are non-temporal:
// the gradient is written once and not read back by this pass, so it streams to memory
// instead of displacing the activations the other blocks read from L2 (measured 12.3 ->
// 10.8 us for the 32 MiB fp32 gradient of the 4096-wide, N = 64 workload).
__device__ __forceinline__ void store_dw4(const UpArgs& a, int64_t idx, f32x4 v) {
    if (a.acc) {
        if (a.dwdt == BSMM_F32) {
            v += *reinterpret_cast<const f32x4*>((const float*)a.dw + idx);
        } else {
            const u32x2 o = *reinterpret_cast<const u32x2*>((const uint16_t*)a.dw + idx);
            const uint32_t h[4] = {o.x & 0xffffu, o.x >> 16, o.y & 0xffffu, o.y >> 16};
#pragma unroll
            for (int i = 0; i < 4; i++)
                v[i] += a.dwdt == BSMM_BF16 ? __uint_as_float(h[i] << 16)
                                            : (float)__builtin_bit_cast(_Float16, (uint16_t)h[i]);
        }
    }
    if (a.dwdt == BSMM_F32) {
        __builtin_nontemporal_store(v, reinterpret_cast<f32x4*>((float*)a.dw + idx));
    } else {
        u32x2 w;
        if (a.dwdt == BSMM_BF16) {
            w.x = to_storage16<BSMM_BF16>(v.x) | (to_storage16<BSMM_BF16>(v.y) << 16);
            w.y = to_storage16<BSMM_BF16>(v.z) | (to_storage16<BSMM_BF16>(v.w) << 16);
        } else {
            w.x = to_storage16<BSMM_F16>(v.x) | (to_storage16<BSMM_F16>(v.y) << 16);
            w.y = to_storage16<BSMM_F16>(v.z) | (to_storage16<BSMM_F16>(v.w) << 16);
        }
        __builtin_nontemporal_store(w, reinterpret_cast<u32x2*>((uint16_t*)a.dw + idx));
    }
}

// Descriptors of the tensors of step group t.  With one group (the common case) they are
// built once, before the loops: selecting a group pointer from the argument block inside
// a loop puts a scalar load and its wait in every step.
struct PickOne {
    rsrc_t rx, ry;
    __device__ void operator()(const UpArgs&, int, rsrc_t& x, rsrc_t& y) const {
        x = rx;
        y = ry;
    }
};
// Several groups: the descriptors of the last group asked for are kept, and rebuilt
// (a scalar load from the argument block) only when a step of another group comes.
struct PickMany {
    int t = -1;
    rsrc_t rx, ry;
    __device__ void operator()(const UpArgs& a, int tt, rsrc_t& x, rsrc_t& y) {
        if (tt != t) {   // uniform; once per group and pipeline position
            const void* xp = a.xs[0];
            const void* dp = a.dys[0];
#pragma unroll
            for (int u = 1; u < kMaxGroup; u++)
                if (tt == u) {
                    xp = a.xs[u];
                    dp = a.dys[u];
                }
            rx = make_rsrc(xp, a.x_bytes);
            ry = make_rsrc(dp, a.dy_bytes);
            t = tt;
        }
        x = rx;
        y = ry;
    }
};
__device__ inline PickOne pick_one(const UpArgs& a) {
    return PickOne{make_rsrc(a.xs[0], a.x_bytes), make_rsrc(a.dys[0], a.dy_bytes)};
}

template <int DT, int B, int FA, int D>
__global__ __launch_bounds__(256) void updat_kernel(UpArgs a) {
    using T = typename Elt<DT>::T;
    constexpr int S = (int)sizeof(T);
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
    const int N = (int)a.N;
    const int spt = (N + KS - 1) / KS;
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

    // Per-lane byte offsets relative to the step's first row (minibatch-major) or to the
    // block's first feature row (feature-major).  With minibatch-major activations a row
    // past the minibatch lies past the end of the tensor, so it reads as zero by itself.
    uint32_t xc[RR], dc[RR];
#pragma unroll
    for (int i = 0; i < RR; i++) {
        if constexpr (TR) {
            const int ch = lane + 64 * i;
            const bool chv = ch < 4 * B;
            const int r = chv ? ch / WCH : 0, cc = ch % WCH;
            xc[i] = chv ? (uint32_t)(r * a.C + cc * 8) * S : kOffLane;
            dc[i] = chv ? (uint32_t)(r * a.K + cc * 8) * S : kOffLane;
        } else if constexpr (FA == 1) {   // fp32: rows 4g + v of the step
            const int p = 16 * i + r16;
            xc[i] = p < B ? (uint32_t)(4 * g * a.C + p) * S : kOffLane;
            dc[i] = p < B ? (uint32_t)(4 * g * a.K + p) * S : kOffLane;
        } else {
            const int p = 16 * i + r16;
            xc[i] = p < B ? ((uint32_t)p * N + g * VEC) * S : kOffLane;
            dc[i] = xc[i];
        }
    }

    struct SlotU {
        u32x4 x[RR];
        u32x4 d[RR];
    };

    auto load_slot = [&](SlotU& sl, int it0, auto& pick) {
        const bool iv = it0 < items;   // wave-uniform
        const int it = iv ? it0 : 0;
        const int j = it / nsb, st = it % nsb;
        const int t = st / spt;
        const int nb = (st % spt) * KS;
        const int c = __builtin_amdgcn_readlane(cl, j), k = __builtin_amdgcn_readlane(kl, j);
        rsrc_t rx, rd;
        pick(a, t, rx, rd);
        if constexpr (TR) {
            const uint32_t xs = iv ? (uint32_t)(nb * a.C + c * B) * S : kOffOff;
            const uint32_t ds = iv ? (uint32_t)(nb * a.K + k * B) * S : kOffOff;
#pragma unroll
            for (int i = 0; i < RR; i++) {
                sl.x[i] = bload128(rx, xc[i], xs);
                sl.d[i] = bload128(rd, dc[i], ds);
            }
        } else if constexpr (FA == 1) {   // fp32, minibatch-major: four rows per fragment
#pragma unroll
            for (int i = 0; i < RR; i++)
#pragma unroll
                for (int v = 0; v < 4; v++) {
                    sl.x[i][v] = bload32(rx, xc[i], iv ? (uint32_t)((nb + v) * a.C + c * B) * S : kOffOff);
                    sl.d[i][v] = bload32(rd, dc[i], iv ? (uint32_t)((nb + v) * a.K + k * B) * S : kOffOff);
                }
        } else {   // feature-major: the contraction index is contiguous
            const uint32_t xs = iv ? ((uint32_t)c * B * N + nb) * S : kOffOff;
            const uint32_t ds = iv ? ((uint32_t)k * B * N + nb) * S : kOffOff;
            const int nl = nb + g * VEC;   // the lane group's first minibatch row
#pragma unroll
            for (int i = 0; i < RR; i++) {
                if (xvec) {
                    const bool ok = nl < N;
                    sl.x[i] = bload128(rx, ok ? xc[i] : kOffLane, xs);
                    sl.d[i] = bload128(rd, ok ? dc[i] : kOffLane, ds);
                } else {   // rows not 16-byte aligned: element loads, tail masked
                    uint32_t hx[VEC], hd[VEC];
#pragma unroll
                    for (int v = 0; v < VEC; v++) {
                        const uint32_t vo = nl + v < N ? xc[i] + v * S : kOffLane;
                        if constexpr (DT == BSMM_F32) {
                            hx[v] = bload32(rx, vo, xs);
                            hd[v] = bload32(rd, vo, ds);
                        } else {
                            hx[v] = bload16(rx, vo, xs);
                            hd[v] = bload16(rd, vo, ds);
                        }
                    }
                    if constexpr (DT == BSMM_F32) {
                        sl.x[i] = u32x4{hx[0], hx[1], hx[2], hx[3]};
                        sl.d[i] = u32x4{hd[0], hd[1], hd[2], hd[3]};
                    } else {
                        sl.x[i] = u32x4{hx[0] | (hx[1] << 16), hx[2] | (hx[3] << 16), hx[4] | (hx[5] << 16),
                                        hx[6] | (hx[7] << 16)};
                        sl.d[i] = u32x4{hd[0] | (hd[1] << 16), hd[2] | (hd[3] << 16), hd[4] | (hd[5] << 16),
                                        hd[6] | (hd[7] << 16)};
                    }
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
                        store_dw4(a, idx, acc[qt][pt]);
                    }
                    acc[qt][pt] = f32x4{0.f, 0.f, 0.f, 0.f};
                }
        }
    };

    if (items == 0) {
        // N = 0: every block of this wave is the empty sum (nothing to add when
        // accumulating)
        for (int j = 0; j < (a.acc ? 0 : nblk); j++) {
            const int64_t base = (b0 + j) * B * B;
            for (int e = lane; e < B * B; e += 64) store_elt(a.dw, base + e, 0.f, a.dwdt);
        }
        return;
    }

    auto run = [&](auto&& pick) {
        SlotU ring[D];
#pragma unroll
        for (int i = 0; i < D; i++) load_slot(ring[i], i, pick);
        for (int j = 0; j < items; j += D) {
#pragma unroll
            for (int i = 0; i < D; i++) {
                compute_slot(ring[i], j + i);   // items past the end add zeros and store nothing
                load_slot(ring[i], j + i + D, pick);
            }
        }
    };
    if (a.G == 1) {
        PickOne p1 = pick_one(a);
        run(p1);
    } else {
        PickMany pm;
        run(pm);
    }
}

// ---------------------------------------------------------------------------------
// Grouped weight gradient for long contractions (many minibatch steps per block).
// A workgroup owns a group of up to GM blocks of one layout row c (consecutive ids):
// every step loads the x_t slab of row c once and the dy_t slab of each block's
// column, so the x slab is shared by the group.  The 4 waves split the contraction
// steps; their partial tiles are added in wave order through LDS and each block is
// written once.  Groups are dealt to XCDs in contiguous row ranges, so neighbouring
// rows (which share columns, e.g. in a banded layout) reuse dy slabs from one L2.
// With nparts > 1 the contraction is also cut into nparts consecutive step ranges, one
// workgroup each (an XCD runs part 0 of each of its groups, then part 1, ...), and part
// p of the group's j-th block goes to pws[(p * nrids + first + j) * b * b ...] instead
// of dw: written when addp is 0, added to what is there otherwise (one writer per
// element, launches in stream order).  Only listed groups (ids in rids) take parts.
template <int DT, int B, int FA, int GM, int D>
struct UGCfg {
    static constexpr int VEC = Elt<DT>::VEC, KS = 4 * VEC;
    static constexpr int PT = (B + 15) / 16;
    static constexpr bool TR = FA == 1 && DT != BSMM_F32;
    static constexpr int WCH = B / 8;
    static constexpr int RR = TR ? (4 * B + 63) / 64 : PT;
    static constexpr int NS = 1 + GM;   // slab 0: x, slabs 1..GM: dy of each block
    static constexpr int PITCH = PT * 16 + 8;
    static constexpr int TILE = 32 * PITCH;
    static constexpr int TILE_BYTES = TR ? 4 * NS * TILE * 2 : 0;
    static constexpr int RED_BYTES = 4 * GM * PT * PT * 64 * 16;
    static constexpr int SMEM = TILE_BYTES > RED_BYTES ? TILE_BYTES : RED_BYTES;
};

template <int DT, int B, int FA, int GM, int D>
__global__ __launch_bounds__(256) void updg_kernel(UpArgs a, const int4* __restrict__ groups, int ngroups,
                                                   int nparts, float* __restrict__ pws, int addp) {
    using Cfg = UGCfg<DT, B, FA, GM, D>;
    using T = typename Elt<DT>::T;
    constexpr int S = (int)sizeof(T);
    constexpr int VEC = Cfg::VEC, KS = Cfg::KS, PT = Cfg::PT, RR = Cfg::RR, NS = Cfg::NS;
    constexpr int PITCH = Cfg::PITCH, TILE = Cfg::TILE, WCH = Cfg::WCH;
    constexpr bool TR = Cfg::TR;
    __shared__ __attribute__((aligned(16))) char smem[Cfg::SMEM];

    const int lane = threadIdx.x & 63;
    const int wk = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int r16 = lane & 15, g = lane >> 4;
    // group index: XCD x takes the x-th contiguous range of groups (rows)
    const int gpx = (ngroups + 7) / 8;
    const int slot = blockIdx.x >> 3, part = slot / gpx;
    const int gi = (blockIdx.x & 7) * gpx + slot % gpx;
    if (gi >= ngroups || part >= nparts) return;   // whole workgroup
    const int4 gr = groups[gi];   // (first, count, row, 0: ids first.. / 1: ids rids[first..])
    const int id0 = gr.x, cnt = gr.y, c = gr.z;
    const bool listed = gr.w != 0;
    const int N = (int)a.N;
    const int spt = (N + KS - 1) / KS;
    const int nsb = a.G * spt;
    const bool xvec = (N % VEC) == 0;
    int kl = 0;
    if (lane < cnt) kl = a.coords[2 * (listed ? a.rids[id0 + lane] : id0 + lane) + 1];

    BSMM_LDS uint16_t* tiles = (BSMM_LDS uint16_t*)smem + wk * NS * TILE;
    if constexpr (TR && B == 8) {
        for (int i = lane; i < NS * TILE; i += 64) tiles[i] = 0;
    }

    uint32_t xc[RR], dc[RR];
#pragma unroll
    for (int i = 0; i < RR; i++) {
        if constexpr (TR) {
            const int ch = lane + 64 * i;
            const bool chv = ch < 4 * B;
            const int r = chv ? ch / WCH : 0, cc = ch % WCH;
            xc[i] = chv ? (uint32_t)(r * a.C + cc * 8) * S : kOffLane;
            dc[i] = chv ? (uint32_t)(r * a.K + cc * 8) * S : kOffLane;
        } else if constexpr (FA == 1) {
            const int p = 16 * i + r16;
            xc[i] = p < B ? (uint32_t)(4 * g * a.C + p) * S : kOffLane;
            dc[i] = p < B ? (uint32_t)(4 * g * a.K + p) * S : kOffLane;
        } else {
            const int p = 16 * i + r16;
            xc[i] = p < B ? ((uint32_t)p * N + g * VEC) * S : kOffLane;
            dc[i] = xc[i];
        }
    }

    struct Slot {
        u32x4 v[NS][RR];
    };

    // one slab (rows nb.. of x_t at feature block fb, or of dy_t) into registers
    auto load_slab = [&](u32x4* out, rsrc_t r, const uint32_t* lc, int F, int fb, int nb, bool ok) {
        if constexpr (TR) {
            const uint32_t so = ok ? (uint32_t)(nb * F + fb * B) * S : kOffOff;
#pragma unroll
            for (int i = 0; i < RR; i++) out[i] = bload128(r, lc[i], so);
        } else if constexpr (FA == 1) {
#pragma unroll
            for (int i = 0; i < RR; i++)
#pragma unroll
                for (int v = 0; v < 4; v++) out[i][v] = bload32(r, lc[i], ok ? (uint32_t)((nb + v) * F + fb * B) * S : kOffOff);
        } else {
            const uint32_t so = ok ? ((uint32_t)fb * B * N + nb) * S : kOffOff;
            const int nl = nb + g * VEC;
#pragma unroll
            for (int i = 0; i < RR; i++) {
                if (xvec) {
                    out[i] = bload128(r, nl < N ? lc[i] : kOffLane, so);
                } else {
                    uint32_t h[VEC];
#pragma unroll
                    for (int v = 0; v < VEC; v++) {
                        const uint32_t vo = nl + v < N ? lc[i] + v * S : kOffLane;
                        h[v] = DT == BSMM_F32 ? bload32(r, vo, so) : bload16(r, vo, so);
                    }
                    if constexpr (DT == BSMM_F32)
                        out[i] = u32x4{h[0], h[1], h[2], h[3]};
                    else
                        out[i] = u32x4{h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16),
                                       h[6] | (h[7] << 16)};
                }
            }
        }
    };

    // this part's steps [sbeg, send)
    const int sbeg = (int)((int64_t)nsb * part / nparts), send = (int)((int64_t)nsb * (part + 1) / nparts);
    auto load_slot = [&](Slot& sl, int sr, auto& pick) {   // sr: step within the part
        const int st0 = sbeg + sr;
        const bool sv = st0 < send;   // wave-uniform
        const int st = sv ? st0 : 0;
        const int t = st / spt;
        const int nb = (st % spt) * KS;
        rsrc_t rx, rd;
        pick(a, t, rx, rd);
        load_slab(sl.v[0], rx, xc, a.C, c, nb, sv);
#pragma unroll
        for (int j = 0; j < GM; j++) {
            const int k = __builtin_amdgcn_readlane(kl, j);
            load_slab(sl.v[1 + j], rd, dc, a.K, k, nb, sv && j < cnt);
        }
    };

    f32x4 acc[GM][PT][PT];
#pragma unroll
    for (int j = 0; j < GM; j++)
#pragma unroll
        for (int q = 0; q < PT; q++)
#pragma unroll
            for (int p = 0; p < PT; p++) acc[j][q][p] = f32x4{0.f, 0.f, 0.f, 0.f};

    auto compute = [&](const Slot& sl) {
        u32x4 fr[NS][PT];
        if constexpr (TR) {   // only the slabs of the group's blocks (slab 0 = x, 1..cnt = dy)
#pragma unroll
            for (int sidx = 0; sidx < NS; sidx++)
                if (sidx <= cnt) {   // wave-uniform
#pragma unroll
                    for (int i = 0; i < RR; i++) {
                        const int ch = lane + 64 * i;
                        if (ch < 4 * B) lds_store16(tiles + sidx * TILE + (ch / WCH) * PITCH + (ch % WCH) * 8, sl.v[sidx][i]);
                    }
                }
            wave_lds_order();
#pragma unroll
            for (int sidx = 0; sidx < NS; sidx++)
                if (sidx <= cnt) {
#pragma unroll
                    for (int pt = 0; pt < PT; pt++) fr[sidx][pt] = frag_tr16(tiles + sidx * TILE, PITCH, 16 * pt, lane);
                }
            wave_lds_order();
        } else {
#pragma unroll
            for (int sidx = 0; sidx < NS; sidx++)
#pragma unroll
                for (int pt = 0; pt < PT; pt++) fr[sidx][pt] = sl.v[sidx][pt];
        }
#pragma unroll
        for (int j = 0; j < GM; j++)
            if (j < cnt)
#pragma unroll
                for (int qt = 0; qt < PT; qt++)
#pragma unroll
                    for (int pt = 0; pt < PT; pt++) mma<DT>(acc[j][qt][pt], fr[1 + j][qt], fr[0][pt]);   // D[q][p]
    };

    const int nps = send - sbeg;
    const int mysteps = nps > wk ? (nps - wk + 3) / 4 : 0;
    auto run = [&](auto&& pick) {
        Slot ring[D];
#pragma unroll
        for (int i = 0; i < D; i++) load_slot(ring[i], wk + 4 * i, pick);
        for (int j = 0; j < mysteps; j += D) {
#pragma unroll
            for (int i = 0; i < D; i++) {
                if (j + i < mysteps) compute(ring[i]);   // no loads inside
                load_slot(ring[i], wk + 4 * (j + i + D), pick);
            }
        }
    };
    if (a.G == 1) {
        PickOne p1 = pick_one(a);
        run(p1);
    } else {
        PickMany pm;
        run(pm);
    }

    // partial tiles of the 4 waves, added in wave order
    __syncthreads();
    f32x4* red = reinterpret_cast<f32x4*>(smem);   // [wave][block][qt][pt][lane]
    constexpr int PER = GM * PT * PT * 64;
#pragma unroll
    for (int j = 0; j < GM; j++)
#pragma unroll
        for (int qt = 0; qt < PT; qt++)
#pragma unroll
            for (int pt = 0; pt < PT; pt++) red[wk * PER + ((j * PT + qt) * PT + pt) * 64 + lane] = acc[j][qt][pt];
    __syncthreads();
    for (int sidx = threadIdx.x; sidx < PER; sidx += 256) {
        const int j = sidx / (PT * PT * 64);
        if (j >= cnt) continue;
        f32x4 sum = red[sidx];
#pragma unroll
        for (int w = 1; w < 4; w++) sum += red[w * PER + sidx];
        const int rem = sidx % (PT * PT * 64);
        const int qt = rem / (PT * 64), pt = (rem / 64) % PT, l = rem % 64;
        const int p = pt * 16 + (l & 15), q = qt * 16 + 4 * (l >> 4);
        if (p < B && q < B) {
            if (pws) {   // listed groups only: id0 + j is the block's entry of rids
                f32x4* dst = reinterpret_cast<f32x4*>(pws + ((int64_t)part * a.nrids + id0 + j) * B * B + p * B + q);
                if (addp) sum += *dst;
                *dst = sum;
            } else {
                const int64_t idx = (int64_t)(listed ? a.rids[id0 + j] : id0 + j) * B * B + p * B + q;
                store_dw4(a, idx, sum);
            }
        }
    }
}

// ---------------------------------------------------------------------------------
// Weight gradient of dense tiles (32x32 blocks, 16-bit activations, long contractions).
// A workgroup owns one tile of 8x8 layout blocks holding at least kTileMin blocks.
// Every step of 32 minibatch rows stages the tile's 256 input features of x_t and its
// 256 output features of dy_t in LDS once; wave w takes tile row w: its x fragments
// are read once per step and feed every present block of the row, whose 32x32
// products accumulate in registers over the whole contraction (register slots by
// tile column, so every LDS offset is a lane constant plus a fixed part).
// Pipeline as in the output-group fprop: RD register stages of loads, three LDS
// buffers, one barrier per step, no branch around a global load.  Features-last
// activations sit in LDS as [row][feature] rows of 512 bytes (chunk-permuted so the
// transposing reads hit each bank once per pass); features-first as [feature][row]
// rows of 64 bytes read straight into fragments.
// 16-byte chunk permutation of 512-byte rows; independent of row bit 2, so the two
// transposing reads of a fragment (rows r and r + 4) differ by a fixed offset
__device__ __forceinline__ int aswz(int r) {
    return (((r ^ (r >> 1)) & 1) << 1) | (((r ^ (r >> 3)) & 1) << 2) | (((r ^ (r >> 4)) & 1) << 3);
}
__device__ __forceinline__ int bswz(int r) {   // the same for 64-byte rows
    return (((r >> 1) ^ (r >> 2)) & 1) | ((((r >> 1) ^ (r >> 3)) & 1) << 1);
}

template <int DT, int FA, int RD>
__global__ __launch_bounds__(512) void updt_kernel(UpArgs a) {
    constexpr int B = 32, T = kTileSide, TF = T * B, KS = 32, S = 2;
    constexpr int TILE = KS * TF;      // elements of one operand tile
    constexpr int STAGE = 2 * TILE;    // x tile, then dy tile
    static_assert(T == 8 && kTileWaves == 8, "one wave per tile row");
    __shared__ __attribute__((aligned(16))) uint16_t smem[3 * STAGE];

    const int t = threadIdx.x, lane = t & 63;
    const int wave = __builtin_amdgcn_readfirstlane(t >> 6);   // = tile row
    const int m16 = lane & 15, g4 = lane >> 4;
    // tiles in row-major order, XCD x taking the x-th contiguous range (neighbouring
    // tiles share x rows or dy columns in that XCD's L2)
    // With a contraction split, workgroup (tile, part) sums steps [part*nsb/split, ..).
    const int units = a.ntiles * a.split;
    const int per = (units + 7) / 8;
    const int un = (blockIdx.x & 7) * per + (blockIdx.x >> 3);
    if (un >= units) return;   // whole workgroup
    const int ti = un / a.split, part = un % a.split;
    const int4 tl = reinterpret_cast<const int4*>(a.tiles)[ti];
    const int r0 = tl.x, c0 = tl.y;
    // ids of this wave's row (scalar loads), -1 where absent
    const int* rowids = a.tblk + tl.w + wave * T;
    int ids[T], mask = 0;
#pragma unroll
    for (int c = 0; c < T; c++) {
        ids[c] = __builtin_amdgcn_readfirstlane(rowids[c]);
        mask |= (ids[c] >= 0 ? 1 : 0) << c;
    }
    mask = __builtin_amdgcn_readfirstlane(mask);   // keeps the presence tests scalar
    const int N = (int)a.N;
    const int spt = (N + KS - 1) / KS;
    const int nall = a.G * spt;
    const int sbeg = (int)((int64_t)part * nall / a.split);
    const int nsb = (int)((int64_t)(part + 1) * nall / a.split) - sbeg;   // this part's steps

    // staging: chunk q = t + 512 i of each operand tile
    uint32_t xo[2], yo[2];
    int ql[2];
#pragma unroll
    for (int i = 0; i < 2; i++) {
        const int q = t + 512 * i;
        if constexpr (FA == 1) {   // row n = q / 32, features 8 (q % 32) ..
            const int r = q >> 5, ch = q & 31;
            xo[i] = r0 * B + 8 * ch < a.C ? (uint32_t)(r * a.C + r0 * B + 8 * ch) * S : kOffLane;
            yo[i] = c0 * B + 8 * ch < a.K ? (uint32_t)(r * a.K + c0 * B + 8 * ch) * S : kOffLane;
            ql[i] = r * TF + ((ch ^ aswz(r)) << 3);
        } else {                   // feature row q / 4, minibatch values 8 (q % 4) ..
            const int r = q >> 2, ch = q & 3;
            xo[i] = r0 * B + r < a.C ? ((uint32_t)(r0 * B + r) * N + 8 * ch) * S : kOffLane;
            yo[i] = c0 * B + r < a.K ? ((uint32_t)(c0 * B + r) * N + 8 * ch) * S : kOffLane;
            ql[i] = r * KS + ((ch ^ bswz(r)) << 3);
        }
    }

    struct Stage {
        u32x4 x[2], y[2];
    };
    auto issue = [&](Stage& st, int s, auto& pick) {
        const bool sv = s < nsb;   // workgroup-uniform
        const int ss = sbeg + (sv ? s : 0);
        const int tt = ss / spt, nb0 = (ss % spt) * KS;
        rsrc_t rx, ry;
        pick(a, tt, rx, ry);
        const uint32_t so = !sv ? kOffOff : FA == 1 ? (uint32_t)nb0 * a.C * S : (uint32_t)nb0 * S;
        const uint32_t sy = !sv ? kOffOff : FA == 1 ? (uint32_t)nb0 * a.K * S : (uint32_t)nb0 * S;
#pragma unroll
        for (int i = 0; i < 2; i++) {
            // Features last: rows past N lie past the tensor's end and read zero by the
            // range check.  Features first: a chunk past N is switched off with the top
            // offset bit (arithmetic, so no branch appears around the load).
            uint32_t off = 0;
            if constexpr (FA == 0) off = ((uint32_t)(N - 1 - nb0 - 8 * ((t + 512 * i) & 3)) >> 31) << 31;
            st.x[i] = bload128(rx, xo[i] | off, so);
            st.y[i] = bload128(ry, yo[i] | off, sy);
        }
    };
    auto stage_lds = [&](const Stage& st, BSMM_LDS uint16_t* buf) {
#pragma unroll
        for (int i = 0; i < 2; i++) {
            lds_store16(buf + ql[i], st.x[i]);
            lds_store16(buf + TILE + ql[i], st.y[i]);
        }
    };

    // LDS element offsets of the fragment reads (within an operand tile), per lane:
    // fragment of features [32 blk + 16 kt, +16), contraction = rows n.  Features last:
    // two transposing reads (rows 8 g4 + m16/4, +4) whose permuted chunk index is a lane
    // constant plus 32 (blk ^ key); tile columns blk = 4 hi + lo give one lane constant
    // per (lo, kt) and a fixed 128 hi (the read of row r + 4 is 4 rows further on).
    int boff[4][2];   // [blk & 3][kt]
    int aoff[2];      // this wave's row, [kt]
    {
        const int r = 8 * g4 + (m16 >> 2), sw = aswz(r), key = sw >> 2;   // rows r, r + 4
#pragma unroll
        for (int kt = 0; kt < 2; kt++) {
            const int base = FA == 1 ? r * TF + 4 * (m16 & 1) + 8 * ((m16 & 3) >> 1) + 16 * (kt ^ ((sw >> 1) & 1))
                                     : (16 * kt + m16) * KS + ((g4 ^ bswz(16 * kt + m16)) << 3);
#pragma unroll
            for (int lo = 0; lo < 4; lo++) boff[lo][kt] = FA == 1 ? base + 32 * (lo ^ key) : base + lo * B * KS;
            aoff[kt] = FA == 1 ? base + 32 * (wave ^ key) : base + wave * B * KS;
        }
    }
    auto frag_at = [&](const BSMM_LDS uint16_t* tile, int o) -> u32x4 {
        if constexpr (FA == 1) {
            const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((BSMM_LDS i16x4*)(tile + o));
            const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((BSMM_LDS i16x4*)(tile + o + 4 * TF));
            const u32x2 ul = __builtin_bit_cast(u32x2, lo), uh = __builtin_bit_cast(u32x2, hi);
            return u32x4{ul.x, ul.y, uh.x, uh.y};
        } else {
            return *reinterpret_cast<const BSMM_LDS u32x4*>(tile + o);
        }
    };
    // column blk's fragment kt: FA 1 tile columns 4..7 sit 128 elements on (the XOR
    // leaves bit 2 of blk alone); FA 0 rows of 32 elements, blk*32 rows on
    auto bfrag = [&](const BSMM_LDS uint16_t* tile, int blk, int kt) -> u32x4 {
        return frag_at(tile + (blk >> 2) * (FA == 1 ? 128 : 4 * B * KS), boff[blk & 3][kt]);
    };

    f32x4 acc[T][2][2];
#pragma unroll
    for (int c = 0; c < T; c++)
#pragma unroll
        for (int kt = 0; kt < 2; kt++)
#pragma unroll
            for (int ct = 0; ct < 2; ct++) acc[c][kt][ct] = f32x4{0.f, 0.f, 0.f, 0.f};

    auto compute = [&](const BSMM_LDS uint16_t* buf) {
        if (mask == 0) return;
        u32x4 af[2];
#pragma unroll
        for (int ct = 0; ct < 2; ct++) af[ct] = frag_at(buf, aoff[ct]);
        constexpr int BB = 2;   // blocks per batch of reads
#pragma unroll
        for (int h0 = 0; h0 < T; h0 += BB) {
            u32x4 bf[BB][2];
#pragma unroll
            for (int c = 0; c < BB; c++)
                if ((mask >> (h0 + c)) & 1) {   // wave-uniform
                    bf[c][0] = bfrag(buf + TILE, h0 + c, 0);
                    bf[c][1] = bfrag(buf + TILE, h0 + c, 1);
                }
#pragma unroll
            for (int c = 0; c < BB; c++)
                if ((mask >> (h0 + c)) & 1) {
#pragma unroll
                    for (int ct = 0; ct < 2; ct++) {
                        mma<DT>(acc[h0 + c][0][ct], bf[c][0], af[ct]);   // D[k][c]
                        mma<DT>(acc[h0 + c][1][ct], bf[c][1], af[ct]);
                    }
                }
        }
    };

    BSMM_LDS uint16_t* lds = (BSMM_LDS uint16_t*)smem;
    auto run = [&](auto&& pick) {
        Stage ring[RD];
#pragma unroll
        for (int k = 0; k < RD; k++) issue(ring[k], k, pick);
        stage_lds(ring[0], lds);
        issue(ring[0], RD, pick);
        __syncthreads();
        for (int s0 = 0; s0 < nsb; s0 += RD) {
            const int b0 = s0 % 3;
#pragma unroll
            for (int r = 0; r < RD; r++) {
                const int s = s0 + r, rn = (r + 1) % RD;
                const int bc = (b0 + r) % 3, bn = (b0 + r + 1) % 3;
                stage_lds(ring[rn], lds + bn * STAGE);   // step s+1
                __syncthreads();
                issue(ring[rn], s + 1 + RD, pick);
                compute(lds + bc * STAGE);
            }
        }
    };
    if (a.G == 1) {
        PickOne p1 = pick_one(a);
        run(p1);
    } else {
        PickMany pm;
        run(pm);
    }

    // D[k][c]: lane holds k = 16kt + 4 g4 + v, c = 16ct + m16 -> 4 consecutive dW values;
    // with a split, fp32 partials go to workspace slot (part, tile, position)
#pragma unroll
    for (int c = 0; c < T; c++) {
        if (!((mask >> c) & 1)) continue;
        const int id = ids[c];
        const int64_t pslot = ((int64_t)part * a.ntiles + ti) * (T * T) + wave * T + c;
#pragma unroll
        for (int kt = 0; kt < 2; kt++)
#pragma unroll
            for (int ct = 0; ct < 2; ct++) {
                const int e = (16 * ct + m16) * B + 16 * kt + 4 * g4;
                const int64_t idx = (int64_t)id * B * B + e;
                if (a.split > 1)
                    store4<BSMM_F32>(a.ws, pslot * B * B + e, acc[c][kt][ct]);
                else
                    store_dw4(a, idx, acc[c][kt][ct]);
            }
    }
}

template <int DT, int B, int FA, int GM = 8>
static hipError_t launch_updat_grouped(const UpArgs& a, const int4* groups, int ngroups, hipStream_t st,
                                       void* e0 = nullptr, void* e1 = nullptr, bool own_events = true,
                                       int nparts = 1, float* pws = nullptr, int addp = 0) {
    const int grid = ((ngroups + 7) / 8) * 8 * nparts;
    if (own_events)
        return launch(BSMM_PASS_UPDAT, updg_kernel<DT, B, FA, GM, 2>, dim3((unsigned)grid), dim3(256), st, a, groups,
                      ngroups, nparts, pws, addp);
    return launch_ev(updg_kernel<DT, B, FA, GM, 2>, dim3((unsigned)grid), dim3(256), st, e0, e1, a, groups, ngroups,
                     nparts, pws, addp);
}

// Sum of the contraction parts of every block outside the tiles, in part order, to dW:
// one workgroup per block.
template <int B>
__global__ __launch_bounds__(256) void updg_reduce(UpArgs a) {
    const int r = blockIdx.x;
    const int id = a.rids[r];
    for (int e = 4 * threadIdx.x; e < B * B; e += 4 * 256) {
        f32x4 s = *reinterpret_cast<const f32x4*>(a.rws + (int64_t)r * B * B + e);
        for (int p = 1; p < a.rsplit; p++)
            s += *reinterpret_cast<const f32x4*>(a.rws + ((int64_t)p * a.nrids + r) * B * B + e);
        store_dw4(a, (int64_t)id * B * B + e, s);
    }
}

// Sum of the split parts of every tile block, in part order (deterministic), to dW: one
// workgroup per (tile, block position), so all the blocks' part reads are in flight at
// once (absent positions leave at once).
template <int B>
__global__ __launch_bounds__(256) void updt_reduce(UpArgs a) {
    constexpr int TT = kTileSide * kTileSide;
    const int ti = blockIdx.x / TT, pos = blockIdx.x % TT;
    const int4 tl = reinterpret_cast<const int4*>(a.tiles)[ti];
    const int id = a.tblk[tl.w + pos];
    if (id < 0) return;   // whole workgroup
    for (int e = 4 * threadIdx.x; e < B * B; e += 4 * 256) {
        f32x4 s = f32x4{0.f, 0.f, 0.f, 0.f};
        for (int p = 0; p < a.split; p++)
            s += *reinterpret_cast<const f32x4*>(a.ws + (((int64_t)p * a.ntiles + ti) * TT + pos) * B * B + e);
        const int64_t idx = (int64_t)id * B * B + e;
        store_dw4(a, idx, s);
    }
}

// Dense tiles (with a contraction split: partials, then their sum), then the remaining
// blocks in row groups; one timing record spans the launches.
template <int DT, int B, int FA>
static hipError_t launch_updat_tiles(const UpArgs& a, hipStream_t st) {
    if constexpr (B != 32 || DT == BSMM_F32) {
        return hipErrorInvalidValue;
    } else {
        void *e0 = nullptr, *e1 = nullptr;
        prof_events(BSMM_PASS_UPDAT, &e0, &e1);
        const bool more = a.split > 1 || a.nrest > 0;
        const int grid = ((a.ntiles * a.split + 7) / 8) * 8;
        hipError_t e = launch_ev(updt_kernel<DT, FA, 2>, dim3((unsigned)grid), dim3(512), st, e0, more ? nullptr : e1, a);
        if (e != hipSuccess) return e;
        if (a.split > 1) {
            e = launch_ev(updt_reduce<B>, dim3((unsigned)(a.ntiles * kTileSide * kTileSide)), dim3(256), st, nullptr,
                          a.nrest > 0 ? nullptr : e1, a);
            if (e != hipSuccess) return e;
        }
        if (a.nrest == 0) return hipSuccess;
        if (a.rsplit > 1) {
            // Remaining blocks with a contraction split: fp32 parts in rws (one launch per
            // step group, each adding its group to the parts, so a launch reads one group's
            // activations only), then the parts' sum to dW.
            for (int t = 0; t < a.G; t++) {
                UpArgs at = a;
                at.G = 1;
                at.xs[0] = a.xs[t];
                at.dys[0] = a.dys[t];
                e = launch_updat_grouped<DT, B, FA, kRestGroup>(at, (const int4*)a.rest, a.nrest, st, nullptr, nullptr,
                                                                false, a.rsplit, a.rws, t > 0);
                if (e != hipSuccess) return e;
            }
            return launch_ev(updg_reduce<B>, dim3((unsigned)a.nrids), dim3(256), st, nullptr, e1, a);
        }
        if (a.G > 1 && a.dwdt == BSMM_F32) {
            // Remaining blocks of several step groups, fp32 dW: one launch per group, each
            // adding its group to dW (the first overwrites unless the call accumulates).
            // A launch then reads one group's activations only, which stay in the
            // memory-side cache while every row group reads the dy slabs of its blocks;
            // one launch over all groups streams them all at once and misses it.
            for (int t = 0; t < a.G; t++) {
                UpArgs at = a;
                at.G = 1;
                at.xs[0] = a.xs[t];
                at.dys[0] = a.dys[t];
                at.acc = a.acc || t > 0;
                e = launch_updat_grouped<DT, B, FA, kRestGroup>(at, (const int4*)a.rest, a.nrest, st, nullptr,
                                                                t == a.G - 1 ? e1 : nullptr, false);
                if (e != hipSuccess) return e;
            }
            return hipSuccess;
        }
        return launch_updat_grouped<DT, B, FA, kRestGroup>(a, (const int4*)a.rest, a.nrest, st, nullptr, e1, false);
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

// ---------------------------------------------------------------------------------
// Short contractions (one step group of N <= 64 rows) with 32x32 blocks and
// feature_axis 1.  A wave takes a run of RL consecutive ids of one layout row c (a part
// of a row group): it loads the x slab of row c once, then for each block the dy slab
// of its column, contracts over the N rows and writes the block.  Stores write whole 128-byte
// dW rows: fp32 pairs output columns 2r, 2r+1 in lane r (the operand map of rows.hip),
// 16-bit storage (operands through the transposing LDS read) passes the finished
// block through a wave-private LDS tile.
// Two consecutive dW values (as store_dw4: accumulate when asked, round once, stream).
__device__ __forceinline__ void store_dw2(const UpArgs& a, int64_t idx, float v0, float v1) {
    if (a.dwdt == BSMM_F32) {
        if (a.acc) {
            const float2 o = *reinterpret_cast<const float2*>((const float*)a.dw + idx);
            v0 += o.x;
            v1 += o.y;
        }
        __builtin_nontemporal_store(u32x2{__float_as_uint(v0), __float_as_uint(v1)},
                                    reinterpret_cast<u32x2*>((float*)a.dw + idx));
        return;
    }
    const bool bf = a.dwdt == BSMM_BF16;
    if (a.acc) {
        const uint32_t o = *reinterpret_cast<const uint32_t*>((const uint16_t*)a.dw + idx);
        const uint32_t h0 = o & 0xffffu, h1 = o >> 16;
        v0 += bf ? __uint_as_float(h0 << 16) : (float)__builtin_bit_cast(_Float16, (uint16_t)h0);
        v1 += bf ? __uint_as_float(h1 << 16) : (float)__builtin_bit_cast(_Float16, (uint16_t)h1);
    }
    const uint32_t w = bf ? to_storage16<BSMM_BF16>(v0) | (to_storage16<BSMM_BF16>(v1) << 16)
                          : to_storage16<BSMM_F16>(v0) | (to_storage16<BSMM_F16>(v1) << 16);
    __builtin_nontemporal_store(w, reinterpret_cast<uint32_t*>((uint16_t*)a.dw + idx));
}

__device__ __forceinline__ u32x2 bload64u(rsrc_t r, uint32_t voff, uint32_t soff) {
    return __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, 0));
}

template <int DT, int D, int RL>
__global__ __launch_bounds__(256) void updr_kernel(UpArgs a) {
    constexpr int B = 32;
    constexpr bool F32 = DT == BSMM_F32;
    // fp32: 4 chunks of 16 rows, 4 matrix-core steps of 4 rows each; 16-bit: 2 chunks
    // of 32 rows, one step each
    constexpr int NCH = F32 ? 4 : 2;
    constexpr int PITCH = 40;            // staged 32-row chunk, 16-bit elements per row
    constexpr int OPITCH = 36;           // finished block, floats per row
    __shared__ __attribute__((aligned(16))) uint16_t stg[F32 ? 8 : 4 * 32 * PITCH];
    __shared__ __attribute__((aligned(16))) float otl[F32 ? 4 : 4 * 32 * OPITCH];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int r16 = lane & 15, g = lane >> 4;
    // wave -> (row group, run of RL of its blocks)
    constexpr int RPG = (8 + RL - 1) / RL;   // runs per row group
    const int wid = blockIdx.x * 4 + wave, gi = wid / RPG, ri = wid % RPG;
    if (gi >= a.ngroups) return;   // no workgroup barrier in this kernel
    const int4 grp = reinterpret_cast<const int4*>(a.groups)[gi];
    const int first = grp.x + ri * RL, crow = grp.z;
    const int cnt = grp.y - ri * RL < RL ? grp.y - ri * RL : RL;
    if (cnt <= 0) return;
    int kl = 0;
    if (lane < cnt) kl = a.coords[2 * (first + lane) + 1];
    const int N = (int)a.N;
    const rsrc_t rx = make_rsrc(a.xs[0], a.x_bytes);
    const rsrc_t ry = make_rsrc(a.dys[0], a.dy_bytes);
    BSMM_LDS uint16_t* st = (BSMM_LDS uint16_t*)stg + wave * 32 * PITCH;
    BSMM_LDS float* ot = (BSMM_LDS float*)otl + wave * 32 * OPITCH;

    if constexpr (F32) {
        // lane (r16, g), chunk ch, step v: row 16 ch + 4 v + g, columns 2 r16, 2 r16 + 1
        uint32_t xo[NCH * 4], yo[NCH * 4];
#pragma unroll
        for (int i = 0; i < NCH * 4; i++) {
            const int n = 4 * i + g;
            xo[i] = n < N ? ((uint32_t)n * a.C + 2 * r16) * 4u : kOffLane;
            yo[i] = n < N ? ((uint32_t)n * a.K + 2 * r16) * 4u : kOffLane;
        }
        u32x2 xf[NCH * 4];
#pragma unroll
        for (int i = 0; i < NCH * 4; i++) xf[i] = bload64u(rx, xo[i], (uint32_t)crow * (B * 4));
        struct Slot {
            u32x2 y[NCH * 4];
        };
        auto load = [&](Slot& sl, int j) {
            const bool ok = j < cnt;
            const int k = __builtin_amdgcn_readlane(kl, ok ? j : 0);
            const uint32_t so = ok ? (uint32_t)k * (B * 4) : kOffOff;
#pragma unroll
            for (int i = 0; i < NCH * 4; i++) sl.y[i] = bload64u(ry, yo[i], so);
        };
        Slot ring[D];
#pragma unroll
        for (int i = 0; i < D; i++) {
            load(ring[i], i);
            __builtin_amdgcn_sched_barrier(0);
        }
        for (int j = 0; j < cnt; j += D) {
#pragma unroll
            for (int i = 0; i < D; i++) {
                if (j + i < cnt) {
                    f32x4 acc[2][2];
#pragma unroll
                    for (int pt = 0; pt < 2; pt++) acc[pt][0] = acc[pt][1] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int s = 0; s < NCH * 4; s++)
#pragma unroll
                        for (int pt = 0; pt < 2; pt++)
#pragma unroll
                            for (int qt = 0; qt < 2; qt++)
                                acc[pt][qt] = __builtin_amdgcn_mfma_f32_16x16x4f32(
                                    __uint_as_float(xf[s][pt]), __uint_as_float(ring[i].y[s][qt]), acc[pt][qt], 0, 0, 0);
                    // lane holds dW[p = 8 g + 2 v + pt][q = 2 r16 + qt]
                    const int64_t base = (int64_t)(first + j + i) * B * B;
#pragma unroll
                    for (int pt = 0; pt < 2; pt++)
#pragma unroll
                        for (int v = 0; v < 4; v++)
                            store_dw2(a, base + (8 * g + 2 * v + pt) * B + 2 * r16, acc[pt][0][v], acc[pt][1][v]);
                }
                load(ring[i], j + i + D);
            }
        }
    } else {
        // 16-byte chunk c = lane + 64 h of a 32-row chunk: row c / 4, columns 8 (c % 4) ..
        uint32_t xo[NCH * 2], yo[NCH * 2];
#pragma unroll
        for (int i = 0; i < NCH * 2; i++) {
            const int ch = i / 2, c = lane + 64 * (i % 2);
            const int n = 32 * ch + (c >> 2);
            xo[i] = n < N ? ((uint32_t)n * a.C + 8 * (c & 3)) * 2u : kOffLane;
            yo[i] = n < N ? ((uint32_t)n * a.K + 8 * (c & 3)) * 2u : kOffLane;
        }
        auto frags = [&](const u32x4* v, u32x4* f) {   // two 32x32 tiles -> 2 chunks x 2 fragments
#pragma unroll
            for (int ch = 0; ch < NCH; ch++) {
#pragma unroll
                for (int h = 0; h < 2; h++) {
                    const int c = lane + 64 * h;
                    lds_store16(st + (c >> 2) * PITCH + 8 * (c & 3), v[ch * 2 + h]);
                }
                wave_lds_order();
                f[ch * 2] = frag_tr16(st, PITCH, 0, lane);
                f[ch * 2 + 1] = frag_tr16(st, PITCH, 16, lane);
                wave_lds_order();
            }
        };
        u32x4 xf[NCH * 2];
        {
            u32x4 xv[NCH * 2];
#pragma unroll
            for (int i = 0; i < NCH * 2; i++) xv[i] = bload128(rx, xo[i], (uint32_t)crow * (B * 2));
            frags(xv, xf);
        }
        struct Slot {
            u32x4 y[NCH * 2];
        };
        auto load = [&](Slot& sl, int j) {
            const bool ok = j < cnt;
            const int k = __builtin_amdgcn_readlane(kl, ok ? j : 0);
            const uint32_t so = ok ? (uint32_t)k * (B * 2) : kOffOff;
#pragma unroll
            for (int i = 0; i < NCH * 2; i++) sl.y[i] = bload128(ry, yo[i], so);
        };
        Slot ring[D];
#pragma unroll
        for (int i = 0; i < D; i++) {
            load(ring[i], i);
            __builtin_amdgcn_sched_barrier(0);
        }
        for (int j = 0; j < cnt; j += D) {
#pragma unroll
            for (int i = 0; i < D; i++) {
                if (j + i < cnt) {
                    u32x4 yf[NCH * 2];
                    frags(ring[i].y, yf);
                    f32x4 acc[2][2];
#pragma unroll
                    for (int pt = 0; pt < 2; pt++) acc[pt][0] = acc[pt][1] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int ch = 0; ch < NCH; ch++)
#pragma unroll
                        for (int pt = 0; pt < 2; pt++)
#pragma unroll
                            for (int qt = 0; qt < 2; qt++) mma<DT>(acc[pt][qt], xf[ch * 2 + pt], yf[ch * 2 + qt]);
                    // lane holds D[p = 16 pt + 4 g + v][q = 16 qt + r16]: through LDS so that
                    // 8 lanes store one whole row
#pragma unroll
                    for (int pt = 0; pt < 2; pt++)
#pragma unroll
                        for (int qt = 0; qt < 2; qt++)
#pragma unroll
                            for (int v = 0; v < 4; v++) ot[(16 * pt + 4 * g + v) * OPITCH + 16 * qt + r16] = acc[pt][qt][v];
                    wave_lds_order();
                    const int64_t base = (int64_t)(first + j + i) * B * B;
#pragma unroll
                    for (int h = 0; h < 4; h++) {
                        const int row = 8 * h + (lane >> 3), col = 4 * (lane & 7);
                        const f32x4 v = *reinterpret_cast<const BSMM_LDS f32x4*>(ot + row * OPITCH + col);
                        store_dw4(a, base + row * B + col, v);
                    }
                    wave_lds_order();
                }
                load(ring[i], j + i + D);
            }
        }
    }
}

// fp32, one block per wave: the same products in two halves of 32 rows, each half's
// x and dy loads (16 rows x 32 columns x 4 bytes each) into 32 registers with the row
// step in the scalar offset.  At under 64 registers all of a launch's waves are
// resident at once (8 per SIMD), so the waves leave the matrix cores one after another
// and each one's dW stores overlap the others' products, instead of whole rounds of
// waves loading, multiplying and storing in step.
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(8, 8))) void updr1_f32_kernel(UpArgs a) {
    constexpr int B = 32;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int r16 = lane & 15, g = lane >> 4;
    const int wid = blockIdx.x * 4 + wave, gi = wid / 8, ri = wid % 8;
    if (gi >= a.ngroups) return;   // no workgroup barrier in this kernel
    const int4 grp = reinterpret_cast<const int4*>(a.groups)[gi];
    if (ri >= grp.y) return;
    const int id = grp.x + ri, crow = grp.z;
    const int k = __builtin_amdgcn_readfirstlane(a.coords[2 * id + 1]);
    const int N = (int)a.N;
    const rsrc_t rx = make_rsrc(a.xs[0], a.x_bytes);
    const rsrc_t ry = make_rsrc(a.dys[0], a.dy_bytes);
    // load i of half h reads row 32 h + 4 i + g, columns 2 r16 and 2 r16 + 1
    const uint32_t xb = ((uint32_t)g * a.C + 2 * r16) * 4u, yb = ((uint32_t)g * a.K + 2 * r16) * 4u;
    const uint32_t xs0 = (uint32_t)crow * (B * 4), ys0 = (uint32_t)k * (B * 4);
    f32x4 acc[2][2];
#pragma unroll
    for (int pt = 0; pt < 2; pt++) acc[pt][0] = acc[pt][1] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int h = 0; h < 2; h++) {
        u32x2 xf[8], yf[8];
#pragma unroll
        for (int i = 0; i < 8; i++) {
            const int r = 32 * h + 4 * i;
            const bool ok = r + g < N;
            xf[i] = bload64u(rx, ok ? xb : kOffLane, (uint32_t)r * a.C * 4u + xs0);
            yf[i] = bload64u(ry, ok ? yb : kOffLane, (uint32_t)r * a.K * 4u + ys0);
        }
#pragma unroll
        for (int i = 0; i < 8; i++)
#pragma unroll
            for (int pt = 0; pt < 2; pt++)
#pragma unroll
                for (int qt = 0; qt < 2; qt++)
                    acc[pt][qt] = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(xf[i][pt]),
                                                                      __uint_as_float(yf[i][qt]), acc[pt][qt], 0, 0, 0);
    }
    // lane holds dW[p = 8 g + 2 v + pt][q = 2 r16 + qt]: 4 whole 128-byte rows per store
    const int64_t base = (int64_t)id * B * B;
#pragma unroll
    for (int pt = 0; pt < 2; pt++)
#pragma unroll
        for (int v = 0; v < 4; v++) store_dw2(a, base + (8 * g + 2 * v + pt) * B + 2 * r16, acc[pt][0][v], acc[pt][1][v]);
}

template <int DT, int RL>
static hipError_t launch_updat_runs_t(const UpArgs& a, hipStream_t st) {
    const int64_t waves = (int64_t)a.ngroups * ((8 + RL - 1) / RL);
    const int64_t grid = (waves + 3) / 4;
    if (grid == 0) return hipSuccess;
    return launch(BSMM_PASS_UPDAT, updr_kernel<DT, 2, RL>, dim3((unsigned)grid), dim3(256), st, a);
}

// Blocks per wave: 1 (more waves hide more latency; measured on the 4096-wide N = 64
// workload among 1, 2, 4 and 8: fp32 20.4 / 21.2 / 27.4 / 30.2 us; bf16 in alternating
// runs on one box 9.3-9.9 us with 1 against 10.1-10.6 with 2, 10.3-10.4 with 4).
// BSMM_UPDAT_RUN=<1|2|4|8> (read once) overrides it for A/B measurements.
static int updat_run_len(int) {
    static const int forced = [] {
        const char* e = getenv("BSMM_UPDAT_RUN");
        return e ? atoi(e) : 0;
    }();
    if (forced == 1 || forced == 2 || forced == 4 || forced == 8) return forced;
    return 1;
}

template <int DT>
static hipError_t launch_updat_runs(const UpArgs& a, hipStream_t st) {
    // fp32, one block per wave: the two-half kernel (4096 features, N = 64: 20.2-21.9 ->
    // 16.9-18.8 us in alternating runs on one box)
    if (DT == BSMM_F32 && updat_run_len(DT) == 1) {
        const int64_t grid = ((int64_t)a.ngroups * 8 + 3) / 4;
        if (grid == 0) return hipSuccess;
        return launch(BSMM_PASS_UPDAT, updr1_f32_kernel, dim3((unsigned)grid), dim3(256), st, a);
    }
    switch (updat_run_len(DT)) {
    case 1: return launch_updat_runs_t<DT, 1>(a, st);
    case 2: return launch_updat_runs_t<DT, 2>(a, st);
    case 8: return launch_updat_runs_t<DT, 8>(a, st);
    default: return launch_updat_runs_t<DT, 4>(a, st);
    }
}

// ---------------------------------------------------------------------------------
// Small blocks (8x8, 16x16), features first (x, dy stored (features, N)), 16-bit, long
// contractions.  A workgroup (16 waves) owns one tile of 256 x 256 features of the
// layout; per step of 32 minibatch columns it stages the tile's 256 dy feature rows in
// LDS once (16 KB, every thread one 16-byte load) and each wave loads the 16 x feature
// rows of its quad row straight into a fragment (features first: the contraction index
// is contiguous).  The wave then runs one 16x16x32 matrix-core step per present quad of
// its row (a quad is one 16x16 block, or 2 x 2 blocks of 8x8), the dy fragment read from
// LDS.  The row's present quads come as a list (layout compiler), walked four entries
// at a time: the group's fragment reads are issued together, so the waves meeting at
// the step's barrier each wait for about one LDS round trip per four quads, not one per
// quad.  The layout compiler also picks which quad row each wave takes, so that the
// four SIMDs of the compute unit (wave w runs on SIMD w % 4) get about the same number
// of quads: their matrix cores, not the waves, set the pace of a step.  The quads'
// fp32 sums stay in registers (slot = list position) for the whole contraction.  Loads run RD steps ahead in registers, the LDS
// stage is double buffered: one barrier per step.  Each block has one writer; no
// atomics.
template <int DT, int B, int RD>
__global__ __launch_bounds__(1024) void upds_kernel(UpArgs a) {
    constexpr int TF = kSmallTileFeat, Q = kSmallQuads, KS = 32, IPQ = B == 8 ? 4 : 1;
    constexpr int PITCH = KS + 8;   // staged row: 32 values + 16 bytes (fragment reads hit every bank once)
    __shared__ __attribute__((aligned(16))) uint16_t stg[2][TF * PITCH];          // dy rows of the tile
    __shared__ __attribute__((aligned(16))) uint16_t xst[2][16 * 16 * PITCH];     // x rows, 16 per wave
    const int t = threadIdx.x, lane = t & 63;
    const int w = __builtin_amdgcn_readfirstlane(t >> 6);   // quad row
    const int r16 = lane & 15, g = lane >> 4;
    // tiles in super-block order, XCD x taking the x-th contiguous range
    const int per = (a.nstiles + 7) / 8;
    const int ti = (blockIdx.x & 7) * per + (blockIdx.x >> 3);
    if (ti >= a.nstiles) return;   // whole workgroup
    const int4 tl = reinterpret_cast<const int4*>(a.stiles)[ti];
    const int fx0 = tl.x, fy0 = tl.y, first = tl.z;
    // the wave's quad row and its list: length, then the row's quad columns, one byte
    // each, four to an int
    const int* pl = a.stplan + (ti * Q + w) * kSmallPlanInts;
    const int cnt = __builtin_amdgcn_readfirstlane(pl[0]);
    const int qr = __builtin_amdgcn_readfirstlane(pl[5]);
    uint32_t ent[Q / 4];
#pragma unroll
    for (int k = 0; k < Q / 4; k++) ent[k] = (uint32_t)__builtin_amdgcn_readfirstlane(pl[1 + k]);
    const int ngr = (cnt + 3) >> 2;
    const int N = (int)a.N;
    const int spt = N / KS + (N % KS ? 1 : 0);
    const int nsteps = a.G * spt;

    // Loads go row by row: lane l takes row l / 4 of the wave's 16 feature rows, columns
    // n0 + 8 (l % 4) .. (four consecutive lanes read one row's 64 bytes, which the memory
    // path serves several times faster than the matrix-core fragment order, where
    // consecutive lanes hold different rows).  Wave w loads the 16 x rows of its quad
    // row (features fx0 + 16 qr ..) and the 16 dy rows of quad column w (fy0 + 16 w ..);
    // both go to LDS as rows, and the fragments are read back from there.  (N % 8 == 0:
    // an 8-column chunk is all in or all out.)
    const int lr = lane >> 2, lc = lane & 3;
    const int fx = fx0 + 16 * qr + lr, fy = fy0 + 16 * w + lr;
    const uint32_t xo = fx < a.C ? (uint32_t)fx * N * 2u + 16u * lc : kOffLane;
    const uint32_t yo = fy < a.K ? (uint32_t)fy * N * 2u + 16u * lc : kOffLane;
    const int ql = (16 * w + lr) * PITCH + 8 * lc;   // this lane's stage slot (dy row 16 w + l / 4)
    const int xl = w * 16 * PITCH + lr * PITCH + 8 * lc;   // and its x slot
    struct Slot {
        u32x4 x, y;
    };
    auto issue = [&](Slot& sl, int s, auto& pick) {
        const bool sv = s < nsteps;   // uniform
        const int ss = sv ? s : 0;
        const int tt = ss / spt, n0 = (ss % spt) * KS;
        rsrc_t rx, ry;
        pick(a, tt, rx, ry);
        const uint32_t so = sv ? (uint32_t)n0 * 2u : kOffOff;
        // a chunk past N is switched off with the top offset bit (no branch)
        const uint32_t off = ((uint32_t)(N - 1 - n0 - 8 * lc) >> 31) << 31;
        sl.x = bload128(rx, xo | off, so);
        sl.y = bload128(ry, yo | off, so);
    };
    // fragments: lane l holds row l % 16, columns 8 (l / 16) ..; dy of quad column j at
    // stage row 16 j + l % 16, x at this wave's row l % 16
    const int boff = r16 * PITCH + 8 * g;
    const int xf = w * 16 * PITCH + r16 * PITCH + 8 * g;
    f32x4 acc[Q];
#pragma unroll
    for (int j = 0; j < Q; j++) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};

    auto run = [&](auto&& pick) {
        Slot ring[RD];
#pragma unroll
        for (int i = 0; i < RD; i++) {
            issue(ring[i], i, pick);
            __builtin_amdgcn_sched_barrier(0);
        }
        lds_store16((BSMM_LDS uint16_t*)stg[0] + ql, ring[0].y);
        lds_store16((BSMM_LDS uint16_t*)xst[0] + xl, ring[0].x);
        __syncthreads();
        for (int s0 = 0; s0 < nsteps; s0 += RD) {
#pragma unroll
            for (int i = 0; i < RD; i++) {
                const int s = s0 + i;
                const BSMM_LDS uint16_t* cur = (const BSMM_LDS uint16_t*)stg[s & 1] + boff;
                if (s < nsteps) {
                    const u32x4 xfr = *reinterpret_cast<const BSMM_LDS u32x4*>((const BSMM_LDS uint16_t*)xst[s & 1] + xf);
#pragma unroll
                    for (int k = 0; k < Q / 4; k++) {
                        if (k < ngr) {   // uniform
                            // the group's columns are decoded again every step (a few
                            // scalar instructions) rather than held across the loop
                            uint32_t ek = ent[k];
                            asm volatile("" : "+s"(ek));
                            u32x4 bf[4];
#pragma unroll
                            for (int q = 0; q < 4; q++)
                                if (4 * k + q < cnt) bf[q] = *reinterpret_cast<const BSMM_LDS u32x4*>(cur + ((ek >> (8 * q)) & 15u) * 16 * PITCH);
                            __builtin_amdgcn_sched_barrier(0);   // the group's reads in flight first
#pragma unroll
                            for (int q = 0; q < 4; q++)
                                if (4 * k + q < cnt) mma<DT>(acc[4 * k + q], xfr, bf[q]);   // D[x f][dy f]
                        }
                    }
                }
                // stage step s + 1 (loaded RD - 1 steps ago), then refill this slot
                BSMM_LDS uint16_t* nxt = (BSMM_LDS uint16_t*)stg[(s + 1) & 1];
                lds_store16(nxt + ql, ring[(i + 1) % RD].y);
                lds_store16((BSMM_LDS uint16_t*)xst[(s + 1) & 1] + xl, ring[(i + 1) % RD].x);
                issue(ring[i], s + RD, pick);
                __syncthreads();
            }
        }
    };
    if (a.G == 1) {
        PickOne p1 = pick_one(a);
        run(p1);
    } else {
        PickMany pm;
        run(pm);
    }

    // lane holds D[4 g + v][r16] of each listed quad: x feature 4 g + v, dy feature r16.
    // Those four elements lie in one block (8x8 blocks: block row g / 2, column r16 / 8
    // of the quad), so a lane needs one id per quad; all of them are loaded together
    // (entries past the list's end load quad column 0's and are not used) before any
    // store, one memory round trip rather than one per quad.
    const int* ids = a.stids + first + qr * Q * IPQ;
    const int sub = B == 16 ? 0 : (g >> 1) * 2 + (r16 >> 3);
    int idv[Q];
#pragma unroll
    for (int jj = 0; jj < Q; jj++) {
        const int j = (int)((ent[jj >> 2] >> (8 * (jj & 3))) & 15u);   // quad column
        idv[jj] = ids[j * IPQ + sub];
    }
    const int64_t e0 = B == 16 ? (int64_t)(4 * g) * 16 + r16 : (int64_t)((4 * g) & 7) * 8 + (r16 & 7);
#pragma unroll
    for (int jj = 0; jj < Q; jj++) {
        if (jj >= cnt) continue;   // uniform (no break: the loop unrolls, acc stays in registers)
        if (idv[jj] < 0) continue;
        const int64_t base = (int64_t)idv[jj] * B * B + e0;   // element (4 g, r16); v adds v rows
        if (a.acc) {
            float o[4];
#pragma unroll
            for (int v = 0; v < 4; v++) {
                const int64_t idx = base + v * B;
                if (a.dwdt == BSMM_F32) o[v] = ((const float*)a.dw)[idx];
                else {
                    const uint32_t h = ((const uint16_t*)a.dw)[idx];
                    o[v] = a.dwdt == BSMM_BF16 ? __uint_as_float(h << 16) : (float)__builtin_bit_cast(_Float16, (uint16_t)h);
                }
            }
#pragma unroll
            for (int v = 0; v < 4; v++) store_elt(a.dw, base + v * B, acc[jj][v] + o[v], a.dwdt);
        } else {
#pragma unroll
            for (int v = 0; v < 4; v++) store_elt(a.dw, base + v * B, acc[jj][v], a.dwdt);
        }
    }
}

template <int DT, int B>
static hipError_t launch_updat_small_tiles(const UpArgs& a, hipStream_t st) {
    if constexpr (DT == BSMM_F32 || (B != 8 && B != 16)) {
        return hipErrorInvalidValue;
    } else {
        const int grid = ((a.nstiles + 7) / 8) * 8;
        if (grid == 0) return hipSuccess;
        return launch(BSMM_PASS_UPDAT, upds_kernel<DT, B, 3>, dim3((unsigned)grid), dim3(1024), st, a);
    }
}

template <int DT, int B, int FA>
static hipError_t launch_updat_t(const UpArgs& a, int kind, hipStream_t st) {
    switch (kind) {
    case UP_D2B1: return launch_updat_cfg<DT, B, FA, 2>(a, 1, st);
    case UP_D4B1: return launch_updat_cfg<DT, B, FA, 4>(a, 1, st);
    case UP_D2B2: return launch_updat_cfg<DT, B, FA, 2>(a, 2, st);
    case UP_ROWS: return launch_updat_grouped<DT, B, FA>(a, (const int4*)a.groups, a.ngroups, st);
    case UP_D2B4: return launch_updat_cfg<DT, B, FA, 2>(a, 4, st);
    case UP_D1B2: return launch_updat_cfg<DT, B, FA, 1>(a, 2, st);
    case UP_D2B8: return launch_updat_cfg<DT, B, FA, 2>(a, 8, st);
    case UP_D1B4: return launch_updat_cfg<DT, B, FA, 1>(a, 4, st);
    case UP_TILES: return launch_updat_tiles<DT, B, FA>(a, st);
    case UP_RUNS:
        if constexpr (B == 32 && FA == 1) return launch_updat_runs<DT>(a, st);
        break;
    case UP_STILES:
        if constexpr (B < 32 && FA == 0) return launch_updat_small_tiles<DT, B>(a, st);
        break;
    }
    return hipErrorInvalidValue;
}

int updat_kind(const UpArgs& a, int dt, int b, int fa) {
    const int KS0 = dt == BSMM_F32 ? 16 : 32;
    const int64_t steps0 = (int64_t)a.G * ((a.N + KS0 - 1) / KS0);
    // dense 8x8-block tiles: 32x32 blocks, 16-bit, long contractions (whole 8-row
    // chunks when features lead)
    const bool tiles_ok = b == 32 && dt != BSMM_F32 && a.ntiles > 0 && steps0 >= 16 && (fa == 1 || a.N % 8 == 0);
    // enough workgroups (tiles x contraction parts) to occupy at least half the CUs
    const bool tiles_wide = a.ntiles * a.split >= 128;
    // one step group of at most 64 rows, 32x32 blocks, features last: row runs
    const bool runs_ok = b == 32 && fa == 1 && a.G == 1 && a.N > 0 && a.N <= 64 && a.ngroups > 0;
    // small blocks, features first, 16-bit, whole 8-column chunks, >= 8 steps of 32
    const bool stiles_ok = b < 32 && fa == 0 && dt != BSMM_F32 && a.nstiles > 0 && a.N % 8 == 0 &&
                           (int64_t)a.G * ((a.N + 31) / 32) >= 8;
    if (a.force > 0) {
        if (a.force == UP_TILES && !tiles_ok) return -1;
        if (a.force == UP_RUNS && !runs_ok) return -1;
        if (a.force == UP_STILES && !stiles_ok) return -1;
        return a.force;
    }
    switch (updat_variant()) {
    case 1: return UP_D2B1;
    case 2: return UP_D4B1;
    case 3: return UP_D2B2;
    case 4: return UP_ROWS;
    case 5: return UP_D2B4;
    case 6: return UP_D1B2;
    case 7: return UP_D2B8;
    case 8: return UP_D1B4;
    case 9:
        if (tiles_ok) return UP_TILES;
        break;
    default: break;
    }
    if (tiles_ok && tiles_wide) return UP_TILES;
    if (runs_ok) return UP_RUNS;
    if (stiles_ok) return UP_STILES;
    const int KS = dt == BSMM_F32 ? 16 : 32;
    const int64_t steps = (int64_t)a.G * ((a.N + KS - 1) / KS);
    // Long contractions: row groups, 4 waves per block group.
    if (steps >= 16) return UP_ROWS;
    // Short ones: a wave takes one or two blocks (two once there are enough blocks for
    // >= 2 waves per SIMD), loads, contracts, stores and exits; with two blocks a wave
    // keeps no ring (measured best: waves, not the ring, hide the latency here).
    if ((int64_t)a.nnz / 2 >= 2048) return UP_D1B2;
    return UP_D2B1;
}

int updat_kind_of_name(const char* name) {
    for (int k = UP_D2B1; k <= UP_STILES; k++)
        if (std::strcmp(name, updat_kind_name(k)) == 0) return k;
    return 0;
}

const char* updat_kind_name(int kind) {
    switch (kind) {
    case UP_D2B1: return "blocks_1perwave";
    case UP_D1B2: return "blocks_2perwave";
    case UP_ROWS: return "row_groups";
    case UP_D4B1: return "blocks_1perwave_ring4";
    case UP_D2B2: return "blocks_2perwave_ring2";
    case UP_D2B4: return "blocks_4perwave";
    case UP_D2B8: return "blocks_8perwave";
    case UP_D1B4: return "blocks_4perwave_noring";
    case UP_TILES: return "dense_tiles";
    case UP_RUNS: return "row_runs";
    case UP_STILES: return "small_tiles";
    }
    return "none";
}

template <int DT>
static hipError_t launch_updat_dt(const UpArgs& a, int kind, int b, int fa, hipStream_t st) {
    switch (b * 2 + fa) {
    case 16: return launch_updat_t<DT, 8, 0>(a, kind, st);
    case 17: return launch_updat_t<DT, 8, 1>(a, kind, st);
    case 32: return launch_updat_t<DT, 16, 0>(a, kind, st);
    case 33: return launch_updat_t<DT, 16, 1>(a, kind, st);
    case 64: return launch_updat_t<DT, 32, 0>(a, kind, st);
    case 65: return launch_updat_t<DT, 32, 1>(a, kind, st);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_updat(const UpArgs& a, int dt, int b, int fa, void* stream) {
    hipStream_t st = (hipStream_t)stream;
    if (a.nnz == 0) return hipSuccess;
    const int kind = updat_kind(a, dt, b, fa);
    if (kind < 0) return hipErrorNotSupported;
    switch (dt) {
    case BSMM_F32: return launch_updat_dt<BSMM_F32>(a, kind, b, fa, st);
    case BSMM_BF16: return launch_updat_dt<BSMM_BF16>(a, kind, b, fa, st);
    case BSMM_F16: return launch_updat_dt<BSMM_F16>(a, kind, b, fa, st);
    }
    return hipErrorInvalidValue;
}

}  // namespace bsmm
