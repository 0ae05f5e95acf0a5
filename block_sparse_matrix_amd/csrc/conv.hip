// BlocksparseConv: a convolution whose filter exists only for blocks of channels
// (kiteco/blocksparse README, "API Documentation" › blocksparse.conv ›
// BlocksparseConv(BCK, TRS, DHW, MPQ, strides, dilates, padding)).  Block b couples the
// input channels C_b[0..Bc) to the output channels K_b[0..Bk) through its filter
// F[b] (Bc, T, R, S, Bk); blocks may share channels, and their contributions add.
//
//   fprop  O[n, K_b[j], m, p, q] += sum_{i,t,r,s} I[n, C_b[i], m*st-pad+t*dl, ...] * F[b,i,t,r,s,j]
//   bprop  dI = the input gradient of fprop for dO
//   updat  dF[b,i,t,r,s,j] = sum_{n,m,p,q} I[n, C_b[i], ...] * dO[n, K_b[j], m, p, q]
//
// Activations are (N, channels, D, H, W), 1-D and 2-D images being 3-D ones with
// leading sizes of 1; input positions outside the image read as zero.
//
// fprop and bprop: one thread per output element, the spatial innermost index fastest,
// so a wave shares one channel's block list (uniform loops, broadcast filter loads) and
// reads neighbouring activations.  Each walks its channel's (block, position) list
// from the host-built tables, in list order, accumulating in fp32: deterministic.
// updat: one workgroup per filter row (b, i, t, r, s): the threads stride over the
// (n, m, p, q) positions, each input value is loaded once and multiplied into all Bk
// outputs in registers, and the partial sums are added in a fixed order (wave
// butterflies, then the waves in order).
#include "common.h"

namespace bsmm {

template <int DT> __device__ __forceinline__ float cv_load(const void* p, int64_t i) {
    if constexpr (DT == BSMM_F32) {
        return ((const float*)p)[i];
    } else {
        const uint16_t h = ((const uint16_t*)p)[i];
        if constexpr (DT == BSMM_BF16)
            return __uint_as_float((uint32_t)h << 16);
        else
            return (float)__builtin_bit_cast(_Float16, h);
    }
}

template <int DT>
__global__ __launch_bounds__(256) void conv_fprop_kernel(ConvArgs a) {
    const int64_t MPQ = (int64_t)a.M * a.P * a.Q, total = a.N * a.K * MPQ;
    const int64_t DHW = (int64_t)a.D * a.H * a.W;
    const int TRS = a.T * a.R * a.S;
    for (int64_t o = (int64_t)blockIdx.x * 256 + threadIdx.x; o < total; o += (int64_t)gridDim.x * 256) {
        const int q = (int)(o % a.Q), p = (int)((o / a.Q) % a.P), m = (int)((o / ((int64_t)a.P * a.Q)) % a.M);
        const int64_t nk = o / MPQ;
        const int k = (int)(nk % a.K);
        const int64_t n = nk / a.K;
        float acc = 0.f;
        for (int e = a.lptr[k]; e < a.lptr[k + 1]; e++) {
            const int b = a.lent[2 * e], j = a.lent[2 * e + 1];
            for (int t = 0; t < a.T; t++) {
                const int d = m * a.st[0] - a.pad[0] + t * a.dl[0];
                if (d < 0 || d >= a.D) continue;
                for (int r = 0; r < a.R; r++) {
                    const int h = p * a.st[1] - a.pad[1] + r * a.dl[1];
                    if (h < 0 || h >= a.H) continue;
                    for (int s = 0; s < a.S; s++) {
                        const int w = q * a.st[2] - a.pad[2] + s * a.dl[2];
                        if (w < 0 || w >= a.W) continue;
                        const int64_t sp = ((int64_t)d * a.H + h) * a.W + w;
                        const int tap = (t * a.R + r) * a.S + s;
                        for (int i = 0; i < a.Bc; i++) {
                            const int c = a.cidx[b * a.Bc + i];
                            acc += cv_load<DT>(a.a, (n * a.C + c) * DHW + sp) *
                                   cv_load<DT>(a.b, (((int64_t)b * a.Bc + i) * TRS + tap) * a.Bk + j);
                        }
                    }
                }
            }
        }
        store_elt(a.out, o, acc, DT);
    }
}

template <int DT>
__global__ __launch_bounds__(256) void conv_bprop_kernel(ConvArgs a) {
    const int64_t DHW = (int64_t)a.D * a.H * a.W, total = a.N * a.C * DHW;
    const int64_t MPQ = (int64_t)a.M * a.P * a.Q;
    const int TRS = a.T * a.R * a.S;
    for (int64_t o = (int64_t)blockIdx.x * 256 + threadIdx.x; o < total; o += (int64_t)gridDim.x * 256) {
        const int w = (int)(o % a.W), h = (int)((o / a.W) % a.H), d = (int)((o / ((int64_t)a.H * a.W)) % a.D);
        const int64_t nc = o / DHW;
        const int c = (int)(nc % a.C);
        const int64_t n = nc / a.C;
        float acc = 0.f;
        for (int e = a.lptr[c]; e < a.lptr[c + 1]; e++) {
            const int b = a.lent[2 * e], i = a.lent[2 * e + 1];
            for (int t = 0; t < a.T; t++) {
                const int md = d + a.pad[0] - t * a.dl[0];
                if (md < 0 || md % a.st[0]) continue;
                const int m = md / a.st[0];
                if (m >= a.M) continue;
                for (int r = 0; r < a.R; r++) {
                    const int pd = h + a.pad[1] - r * a.dl[1];
                    if (pd < 0 || pd % a.st[1]) continue;
                    const int p = pd / a.st[1];
                    if (p >= a.P) continue;
                    for (int s = 0; s < a.S; s++) {
                        const int qd = w + a.pad[2] - s * a.dl[2];
                        if (qd < 0 || qd % a.st[2]) continue;
                        const int q = qd / a.st[2];
                        if (q >= a.Q) continue;
                        const int64_t sp = ((int64_t)m * a.P + p) * a.Q + q;
                        const int tap = (t * a.R + r) * a.S + s;
                        const int64_t fb = (((int64_t)b * a.Bc + i) * TRS + tap) * a.Bk;
                        for (int j = 0; j < a.Bk; j++) {
                            const int k = a.kidx[b * a.Bk + j];
                            acc += cv_load<DT>(a.a, (n * a.K + k) * MPQ + sp) * cv_load<DT>(a.b, fb + j);
                        }
                    }
                }
            }
        }
        store_elt(a.out, o, acc, DT);
    }
}

constexpr int kConvMaxBk = 64;

template <int DT>
__global__ __launch_bounds__(256) void conv_updat_kernel(ConvArgs a) {
    // filter row (b, i, t, r, s)
    const int TRS = a.T * a.R * a.S;
    const int row = blockIdx.x;
    const int tap = row % TRS, bi = row / TRS;
    const int b = bi / a.Bc, i = bi % a.Bc;
    const int s = tap % a.S, r = (tap / a.S) % a.R, t = tap / (a.S * a.R);
    const int c = a.cidx[b * a.Bc + i];
    const int64_t MPQ = (int64_t)a.M * a.P * a.Q, DHW = (int64_t)a.D * a.H * a.W;
    const int64_t total = a.N * MPQ;
    int kk[kConvMaxBk];
    float acc[kConvMaxBk];
#pragma unroll
    for (int j = 0; j < kConvMaxBk; j++) {
        kk[j] = j < a.Bk ? a.kidx[b * a.Bk + j] : 0;
        acc[j] = 0.f;
    }
    for (int64_t u = threadIdx.x; u < total; u += 256) {
        const int q = (int)(u % a.Q), p = (int)((u / a.Q) % a.P), m = (int)((u / ((int64_t)a.P * a.Q)) % a.M);
        const int64_t n = u / MPQ;
        const int d = m * a.st[0] - a.pad[0] + t * a.dl[0];
        const int h = p * a.st[1] - a.pad[1] + r * a.dl[1];
        const int w = q * a.st[2] - a.pad[2] + s * a.dl[2];
        if (d < 0 || d >= a.D || h < 0 || h >= a.H || w < 0 || w >= a.W) continue;
        const float x = cv_load<DT>(a.a, (n * a.C + c) * DHW + ((int64_t)d * a.H + h) * a.W + w);
        const int64_t sp = ((int64_t)m * a.P + p) * a.Q + q;
#pragma unroll
        for (int j = 0; j < kConvMaxBk; j++)
            if (j < a.Bk) acc[j] += x * cv_load<DT>(a.b, (n * a.K + kk[j]) * MPQ + sp);
    }
    // fixed-order reduction: butterfly within each wave, then the 4 waves in order
    __shared__ float part[4][kConvMaxBk];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
    for (int j = 0; j < kConvMaxBk; j++) {
        if (j < a.Bk) {   // workgroup-uniform
            float v = acc[j];
#pragma unroll
            for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
            if (lane == 0) part[wave][j] = v;
        }
    }
    __syncthreads();
    if ((int)threadIdx.x < a.Bk) {
        const int j = threadIdx.x;
        const float v = ((part[0][j] + part[1][j]) + part[2][j]) + part[3][j];
        ((float*)a.out)[(int64_t)row * a.Bk + j] = v;
    }
}

// Eight 16-bit values starting D elements past the start of the middle chunk of
// c[0..11] (three consecutive 8-element chunks), |D| <= 3: whole dwords for even D, a
// 16-bit funnel of neighbouring dwords for odd D.
template <int D>
__device__ __forceinline__ u32x4 conv_shifted(const uint32_t (&c)[12]) {
    if constexpr ((D & 1) == 0) {
        constexpr int o = 4 + D / 2;
        return u32x4{c[o], c[o + 1], c[o + 2], c[o + 3]};
    } else {
        constexpr int m = (7 + D) / 2;
        return u32x4{__builtin_amdgcn_alignbyte(c[m + 1], c[m], 2), __builtin_amdgcn_alignbyte(c[m + 2], c[m + 1], 2),
                     __builtin_amdgcn_alignbyte(c[m + 3], c[m + 2], 2), __builtin_amdgcn_alignbyte(c[m + 4], c[m + 3], 2)};
    }
}

// ---------------------------------------------------------------------------------
// Matrix-core path: 2-D images, stride 1, dilation 1, 16-bit storage.  A workgroup (4
// waves) owns one group of blocks that share an output channel list (CO = 16*OT
// channels), one image and TH output rows.  For each block of the group and each slab
// of 32 contraction channels it stages in LDS the slab's input rows (TH + R - 1 rows with
// the halo, zero outside the image) once per column shift s of the filter, so that tap
// (r, s) reads its operand at an aligned column: copy s holds column x + s - pad at x.
// The filter slab is staged as [tap][output channel][32 contraction channels].  Each
// tap is then one 32-deep v_mfma_f32_16x16x32 step per (16-position tile, 16-channel
// tile): the position operand comes from the staged rows with the transposing LDS read
// ([channel][position] tile), the filter operand with one 16-byte read.  Wave w takes
// position tiles w, w+4, ... and all output tiles, accumulating in registers over the
// group's blocks, taps and slabs in a fixed order.
//
// bprop runs the same kernel as the convolution of dO with the flipped, transposed
// filter: contraction over each block's output channels, outputs its input channels,
// pads F - 1 - pad.
template <int DT, int OT, bool TR>
__global__ __launch_bounds__(256) void conv_mfma_kernel(ConvArgs a) {
    extern __shared__ __attribute__((aligned(16))) uint16_t dsm[];
    constexpr int CO = 16 * OT;
    const int CI = TR ? a.Bk : a.Bc;                       // contraction channels per block
    const int32_t* in_idx = TR ? a.kidx : a.cidx;
    const int32_t* out_idx = TR ? a.cidx : a.kidx;
    const int Hi = TR ? a.P : a.H, Wi = TR ? a.Q : a.W;    // this pass's input image
    const int Ho = TR ? a.H : a.P, Wo = TR ? a.W : a.Q;    // and output image
    const int R = a.R, S = a.S, RS = R * S;
    const int ph = TR ? R - 1 - a.pad[1] : a.pad[1], pw = TR ? S - 1 - a.pad[2] : a.pad[2];
    const int64_t Cin = TR ? a.K : a.C, Cout = TR ? a.C : a.K;
    const int PT = (Wo + 15) / 16, COLS = PT * 16;
    const int TH = a.TH, ROWS = TH + R - 1, CP = a.cpitch;
    BSMM_LDS uint16_t* xs = (BSMM_LDS uint16_t*)dsm;              // [s][32 channels][CP]
    BSMM_LDS uint16_t* fs = xs + S * 32 * CP;                       // [tap][CO][40]
    __shared__ int chs[32];                                         // the slab's input channels

    const int nyt = (Ho + TH - 1) / TH;
    const int yt = blockIdx.x % nyt;
    const int64_t rest = blockIdx.x / nyt;
    const int64_t n = rest % a.N;
    const int g = (int)(rest / a.N);
    const int y0 = yt * TH;
    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    const int m16 = lane & 15, g4 = lane >> 4;
    const int npt = TH * PT;

    f32x4 acc[4][OT];
#pragma unroll
    for (int u = 0; u < 4; u++)
#pragma unroll
        for (int o = 0; o < OT; o++) acc[u][o] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int gb = a.gptr[g], ge = a.gptr[g + 1];
    const rsrc_t rin = make_rsrc(a.a, a.a_bytes);
    for (int e = gb; e < ge; e++) {
        const int b = a.gblk[e];
        for (int slab = 0; slab < CI / 32; slab++) {
            __syncthreads();   // the previous slab's LDS is no longer read
            if (t < 32) chs[t] = in_idx[b * CI + slab * 32 + t];
            __syncthreads();
            // input rows: a thread copies whole staged rows (channel c, row rr), each source
            // element read once for every shift s it serves.  Buffer loads: positions
            // outside the image get an out-of-range offset and read as zero, so every load
            // is issued unconditionally.
            const int XW = COLS + S - 1;
            // Rows of a multiple of 8 elements start 16-byte aligned: read them in aligned
            // 8-element chunks (each wholly inside or outside the row) and write each copy
            // s as 16-byte chunks, staged columns col .. col+7 holding source columns
            // col + s - pw ..; shifts of at most 3 either way.
            const bool vec = Wi % 8 == 0 && pw <= 3 && S - 1 - pw <= 3;
            for (int q = t; q < 32 * ROWS; q += 256) {
                const int rr = q % ROWS, c = q / ROWS;
                const int y = y0 + rr - ph;
                const bool yok = y >= 0 && y < Hi;
                const uint32_t row = yok ? (uint32_t)(((n * Cin + chs[c]) * Hi + y) * Wi) * 2u : 0u;
                BSMM_LDS uint16_t* dst = xs + c * CP + rr * COLS;
                if (vec) {
                    auto chunk = [&](int x0) {
                        return bload128(rin, yok && x0 >= 0 && x0 < Wi ? row + 2u * x0 : kOffLane, 0);
                    };
                    u32x4 ca = chunk(-8), cb = chunk(0), cc = chunk(8);
                    for (int col = 0; col < COLS; col += 8) {
                        const uint32_t w[12] = {ca.x, ca.y, ca.z, ca.w, cb.x, cb.y, cb.z, cb.w, cc.x, cc.y, cc.z, cc.w};
                        for (int sh = 0; sh < S; sh++) {
                            u32x4 v;
                            switch (sh - pw) {
                            case -3: v = conv_shifted<-3>(w); break;
                            case -2: v = conv_shifted<-2>(w); break;
                            case -1: v = conv_shifted<-1>(w); break;
                            case 0: v = conv_shifted<0>(w); break;
                            case 1: v = conv_shifted<1>(w); break;
                            case 2: v = conv_shifted<2>(w); break;
                            default: v = conv_shifted<3>(w); break;
                            }
                            lds_store16(dst + sh * 32 * CP + col, v);
                        }
                        ca = cb;
                        cb = cc;
                        cc = chunk(col + 16);
                    }
                    continue;
                }
                for (int x0 = 0; x0 < XW; x0 += 8) {
                    uint32_t v[8];
#pragma unroll
                    for (int h = 0; h < 8; h++) {
                        const int x = x0 + h - pw;
                        v[h] = bload16(rin, yok && x >= 0 && x < Wi ? row + 2u * x : kOffLane, 0);
                    }
#pragma unroll
                    for (int h = 0; h < 8; h++) {
                        for (int s = 0; s < S; s++) {
                            const int col = x0 + h - s;
                            if (col >= 0 && col < COLS) dst[s * 32 * CP + col] = (uint16_t)v[h];
                        }
                    }
                }
            }
            // filter slab: fs[tap][o][ci] (o: this pass's output channel in the block, ci:
            // contraction channel in the slab), read in 16-byte runs of the stored layout
            if constexpr (TR) {
                // stored F[b, i = o, tap', j = slab*32 + ci]: 32 consecutive j per (o, tap');
                // the transposed convolution takes the flipped tap
                for (int q = t; q < CO * RS * 4; q += 256) {
                    const int part = q % 4, tp = (q / 4) % RS, o = q / (4 * RS);
                    const int tap = (R - 1 - tp / S) * S + (S - 1 - tp % S);
                    const u32x4 v = *reinterpret_cast<const u32x4*>(
                        (const uint16_t*)a.b + (((int64_t)b * a.Bc + o) * RS + tp) * a.Bk + slab * 32 + part * 8);
                    *reinterpret_cast<BSMM_LDS u32x4*>(fs + (tap * CO + o) * 40 + part * 8) = v;
                }
            } else {
                // stored F[b, i = slab*32 + ci, tap, j = o]: CO consecutive o per (ci, tap);
                // adjacent lanes take adjacent ci, so their LDS writes are consecutive
                for (int q = t; q < 32 * RS * (CO / 8); q += 256) {
                    const int ci = q % 32, part = (q / 32) % (CO / 8), tap = q / (32 * (CO / 8));
                    const u32x4 v = *reinterpret_cast<const u32x4*>(
                        (const uint16_t*)a.b + (((int64_t)b * a.Bc + slab * 32 + ci) * RS + tap) * a.Bk + part * 8);
                    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
                    for (int h = 0; h < 8; h++)
                        fs[(tap * CO + part * 8 + h) * 40 + ci] = (uint16_t)(h & 1 ? w[h >> 1] >> 16 : w[h >> 1] & 0xffffu);
                }
            }
            __syncthreads();
            for (int tap = 0; tap < RS; tap++) {
                const int r = tap / S, s = tap % S;
                u32x4 bf[OT];
#pragma unroll
                for (int o = 0; o < OT; o++)
                    bf[o] = *reinterpret_cast<const BSMM_LDS u32x4*>(fs + (tap * CO + o * 16 + m16) * 40 + 8 * g4);
#pragma unroll
                for (int u = 0; u < 4; u++) {
                    const int pt = wave + 4 * u;
                    if (pt < npt) {   // wave-uniform
                        const int ty = pt / PT, px = pt % PT;
                        const u32x4 af = frag_tr16(xs + s * 32 * CP + (ty + r) * COLS + px * 16, CP, 0, lane);
#pragma unroll
                        for (int o = 0; o < OT; o++) mma<DT>(acc[u][o], af, bf[o]);
                    }
                }
            }
        }
    }
    // lane holds D[position 4*g4 + v][channel m16] of each tile
    const int b0 = a.gblk[gb];
#pragma unroll
    for (int u = 0; u < 4; u++) {
        const int pt = wave + 4 * u;
        if (pt >= npt) continue;
        const int ty = pt / PT, px = pt % PT;
        const int y = y0 + ty;
        if (y >= Ho) continue;
#pragma unroll
        for (int o = 0; o < OT; o++) {
            const int oc = out_idx[b0 * CO + o * 16 + m16];
#pragma unroll
            for (int v = 0; v < 4; v++) {
                const int x = px * 16 + 4 * g4 + v;
                if (x < Wo) store_elt(a.out, ((n * Cout + oc) * Ho + y) * Wo + x, acc[u][o][v], DT);
            }
        }
    }
}

// Filter gradient on the matrix cores (2-D / 1-D, stride 1, dilation 1, 16-bit; Bc and
// Bk multiples of 16, at most 64): one workgroup (8 waves) per (block, filter tap) owns
// dF[b, :, tap, :] and contracts over every (image, output position) in steps of 256
// positions, taken in the flattened (row, column) order of the output image:
// dF[b, i, tap, j] = sum over positions of I[n, C_b[i], y + r - ph, x + s - pw] *
// dO[n, K_b[j], y, x].  Each step stages the block's shifted input values (zero outside
// the image or past the last position) and its output-gradient values in LDS as
// [channel][128 positions]; a lane's operand is then 8 consecutive positions of one
// channel (one 16-byte LDS read), eight 32-deep steps per 16x16 tile, wave w taking
// tiles w and w + 8.  The next step's
// values are loaded into registers while the current one computes.  Every output has
// one writer and a fixed summation order.
template <int DT>
__global__ __launch_bounds__(512) void conv_mfma_updat_kernel(ConvArgs a) {
    constexpr int SP = 256, XP = SP + 8;          // positions per step, LDS row pitch
    constexpr int NTH = 512;
    // LDS sized to the block (conv_updat_lds_bytes): two buffers of the input values
    // [Bc][XP], then two of the output-gradient values [Bk][XP]
    extern __shared__ __attribute__((aligned(16))) uint16_t dsm[];
    const int RS = a.R * a.S;
    const int part = blockIdx.x % a.nparts, bt = blockIdx.x / a.nparts;
    const int b = bt / RS, tap = bt % RS;
    const int r = tap / a.S, s = tap % a.S;
    const int Bc = a.Bc, Bk = a.Bk;
    const int H = a.H, W = a.W, P = a.P, Q = a.Q;
    const int64_t PQ = (int64_t)P * Q, HW = (int64_t)H * W;
    const int64_t nsteps_img = (PQ + SP - 1) / SP, nsteps = a.N * nsteps_img;
    // this workgroup's share of the contraction steps
    const int64_t st0 = nsteps * part / a.nparts, st1 = nsteps * (part + 1) / a.nparts;
    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    const int m16 = lane & 15, g4 = lane >> 4;
    const rsrc_t rin = make_rsrc(a.a, a.a_bytes);
    const uint16_t* dO = (const uint16_t*)a.b;
    // staging work per thread: input values (channel, position) and output-gradient
    // 8-position pieces; at most 64 x 128 of each
    const int nd = Bk * SP / 8;
    constexpr int MI = 64 * SP / NTH, MD = 64 * SP / 8 / NTH;   // 32 and 4
    uint16_t vi[MI];
    u32x4 vd[MD];
    const bool dvec = (PQ % 8) == 0;
    __shared__ int sch[128];   // the block's input channels, then its output channels
    if (t < Bc) sch[t] = a.cidx[b * Bc + t];
    if (t < Bk) sch[64 + t] = a.kidx[b * Bk + t];
    __syncthreads();
    // a thread stages one position of the step (t % SP) for channels t / SP + (NTH/SP)*u
    const int tpp = t % SP, tc = t / SP;
    auto load = [&](int64_t st) {
        const int64_t n = st / nsteps_img;
        const int p0 = (int)(st % nsteps_img) * SP;
        const int p = p0 + tpp;
        const int y = p / Q + r - a.pad[1], x = p % Q + s - a.pad[2];
        const bool ok = st < nsteps && p < PQ && y >= 0 && y < H && x >= 0 && x < W;
        const uint32_t base = ok ? (uint32_t)(n * a.C * HW + (int64_t)y * W + x) * 2u : 0u;
#pragma unroll
        for (int u = 0; u < MI; u++) {   // unconditional buffer loads; misses read zero
            const int c = tc + (NTH / SP) * u;
            vi[u] = (uint16_t)bload16(rin, ok && c < Bc ? base + (uint32_t)(sch[c] * HW) * 2u : kOffLane, 0);
        }
#pragma unroll
        for (int u = 0; u < MD; u++) {
            const int q = t + NTH * u;
            u32x4 v = u32x4{0u, 0u, 0u, 0u};
            if (q < nd && st < nsteps) {
                const int k = q / (SP / 8), pc = q % (SP / 8);
                const int p = p0 + 8 * pc;
                const uint16_t* row = dO + (n * a.K + sch[64 + k]) * PQ;
                if (dvec && p + 8 <= PQ) {
                    v = *reinterpret_cast<const u32x4*>(row + p);
                } else {
                    uint32_t h[8];
#pragma unroll
                    for (int e = 0; e < 8; e++) h[e] = p + e < PQ ? row[p + e] : 0u;
                    v = u32x4{h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16), h[6] | (h[7] << 16)};
                }
            }
            vd[u] = v;
        }
    };
    BSMM_LDS uint16_t* smi = (BSMM_LDS uint16_t*)dsm;
    BSMM_LDS uint16_t* smd = smi + 2 * Bc * XP;
    auto stage = [&](int buf) {
        BSMM_LDS uint16_t* li = smi + buf * Bc * XP;
        BSMM_LDS uint16_t* ld = smd + buf * Bk * XP;
#pragma unroll
        for (int u = 0; u < MI; u++) {
            const int c = tc + (NTH / SP) * u;
            if (c < Bc) li[c * XP + tpp] = vi[u];
        }
#pragma unroll
        for (int u = 0; u < MD; u++) {
            const int q = t + NTH * u;
            if (q < nd) *reinterpret_cast<BSMM_LDS u32x4*>(ld + (q / (SP / 8)) * XP + 8 * (q % (SP / 8))) = vd[u];
        }
    };
    // wave w: tiles (it, jt) = w, w+8 of the (Bc/16) x (Bk/16) grid
    const int ti = Bc / 16, tj = Bk / 16, ntile = ti * tj;
    f32x4 acc[2];
#pragma unroll
    for (int u = 0; u < 2; u++) acc[u] = f32x4{0.f, 0.f, 0.f, 0.f};
    load(st0);
    for (int64_t st = st0; st < st1; st++) {
        const int buf = (int)((st - st0) & 1);
        stage(buf);
        __syncthreads();
        load(st + 1);   // in flight during this step's products
        const BSMM_LDS uint16_t* li = smi + buf * Bc * XP;
        const BSMM_LDS uint16_t* ld = smd + buf * Bk * XP;
#pragma unroll
        for (int u = 0; u < 2; u++) {
            const int tile = wave + 8 * u;
            if (tile < ntile) {   // wave-uniform
                const int it = tile / tj, jt = tile % tj;
#pragma unroll
                for (int kk = 0; kk < SP / 32; kk++) {
                    const u32x4 fa = *reinterpret_cast<const BSMM_LDS u32x4*>(li + (it * 16 + m16) * XP + kk * 32 + 8 * g4);
                    const u32x4 fb = *reinterpret_cast<const BSMM_LDS u32x4*>(ld + (jt * 16 + m16) * XP + kk * 32 + 8 * g4);
                    mma<DT>(acc[u], fb, fa);   // D[j][i]: lane holds j = 4*g4 + v, i = m16
                }
            }
        }
        // the other buffer is rewritten next step: no barrier needed here, the barrier
        // after the next stage orders it (two buffers)
    }
    const int RSn = RS;
#pragma unroll
    for (int u = 0; u < 2; u++) {
        const int tile = wave + 8 * u;
        if (tile >= ntile) continue;
        const int it = tile / tj, jt = tile % tj;
        const int i = it * 16 + m16;
#pragma unroll
        for (int v = 0; v < 4; v++) {
            const int j = jt * 16 + 4 * g4 + v;
            const int64_t e = (((int64_t)b * Bc + i) * RSn + tap) * Bk + j;
            if (a.nparts > 1)
                a.ws[(int64_t)part * a.nb * Bc * RSn * Bk + e] = acc[u][v];
            else
                ((float*)a.out)[e] = acc[u][v];
        }
    }
}

// Filter gradient, row form (2-D / 1-D, stride 1, dilation 1, 16-bit; Bc and Bk of 16,
// 32 or 64; input and output widths multiples of 8; column shifts s - pad of at most 3
// either way).  One workgroup (8 waves) per (block, filter row r, part) owns
// dF[b, :, (r, s), :] for every column tap s: each step of SP output positions (whole
// 8-position pieces of output rows, flattened row-major) stages the dO values once and
// the input row pieces once per shift s (aligned 16-byte loads of the three 8-element
// chunks around each piece, shifted in registers: conv_shifted), so the step's dO
// fragment feeds all S taps.  Against one workgroup per tap this reads each input and
// dO value once per filter row instead of once per tap, with 16-byte loads instead of
// per-element gathers.  Waves take 16x16 (j, i) tiles; with fewer than 8 tiles the
// waves of a tile split the step's 32-deep chunks and their partial tiles are added in
// wave order at the end.  One writer per output, fixed summation order.
template <int DT, int SP, int TPW>
__global__ __launch_bounds__(512) void conv_updat_rows_kernel(ConvArgs a) {
    constexpr int XP = SP + 8, NTH = 512, NCH = SP / 8, KK = SP / 32;
    constexpr int MI = (64 * NCH + NTH - 1) / NTH;   // staging items per thread (<= 64 channels)
    constexpr int SMAX = 7;
    extern __shared__ __attribute__((aligned(16))) uint16_t dsm[];
    const int S = a.S, R = a.R, RS = R * S;
    const int part = blockIdx.x % a.nparts, br = blockIdx.x / a.nparts;
    const int b = br / R, r = br % R;
    const int Bc = a.Bc, Bk = a.Bk;
    const int H = a.H, W = a.W, P = a.P, Q = a.Q;
    const int64_t PQ = (int64_t)P * Q, HW = (int64_t)H * W;
    const int64_t nsteps_img = (PQ + SP - 1) / SP, nsteps = a.N * nsteps_img;
    const int64_t st0 = nsteps * part / a.nparts, st1 = nsteps * (part + 1) / a.nparts;
    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    const int m16 = lane & 15, g4 = lane >> 4;
    const int ph = a.pad[1], pw = a.pad[2];
    const rsrc_t rin = make_rsrc(a.a, a.a_bytes);
    const uint16_t* dO = (const uint16_t*)a.b;
    __shared__ int sch[128];   // the block's input channels, then its output channels
    if (t < Bc) sch[t] = a.cidx[b * Bc + t];
    if (t < Bk) sch[64 + t] = a.kidx[b * Bk + t];
    __syncthreads();

    u32x4 vin[MI][3], vd[MI];
    auto load = [&](int64_t st) {
        const bool sv = st < nsteps;
        const int64_t n = sv ? st / nsteps_img : 0;
        const int p0 = sv ? (int)(st % nsteps_img) * SP : 0;
#pragma unroll
        for (int u = 0; u < MI; u++) {
            const int item = t + NTH * u, c = item / NCH, ch = item % NCH;
            const int p = p0 + 8 * ch;
            const int y = p / Q, x0 = p % Q, yi = y + r - ph;
            const bool ok = sv && c < Bc && p < PQ && yi >= 0 && yi < H;
            const int64_t row = ok ? ((n * a.C + sch[c]) * HW + (int64_t)yi * W) : 0;
            auto chunk = [&](int xx) {   // an aligned 8-element chunk, wholly inside or outside the row
                return bload128(rin, ok && xx >= 0 && xx < W ? (uint32_t)((row + xx) * 2) : kOffLane, 0);
            };
            vin[u][0] = chunk(x0 - 8);
            vin[u][1] = chunk(x0);
            vin[u][2] = chunk(x0 + 8);
            const int k = item / NCH;
            u32x4 v = u32x4{0u, 0u, 0u, 0u};
            if (sv && k < Bk && p < PQ) v = *reinterpret_cast<const u32x4*>(dO + (n * a.K + sch[64 + k]) * PQ + p);
            vd[u] = v;
        }
    };
    BSMM_LDS uint16_t* smi = (BSMM_LDS uint16_t*)dsm;          // [buf][s][c][XP]
    BSMM_LDS uint16_t* smd = smi + 2 * S * Bc * XP;             // [buf][k][XP]
    auto stage = [&](int buf) {
        BSMM_LDS uint16_t* li = smi + buf * S * Bc * XP;
        BSMM_LDS uint16_t* ld = smd + buf * Bk * XP;
#pragma unroll
        for (int u = 0; u < MI; u++) {
            const int item = t + NTH * u, c = item / NCH, ch = item % NCH;
            if (c < Bc) {
                const uint32_t w12[12] = {vin[u][0].x, vin[u][0].y, vin[u][0].z, vin[u][0].w, vin[u][1].x, vin[u][1].y,
                                          vin[u][1].z, vin[u][1].w, vin[u][2].x, vin[u][2].y, vin[u][2].z, vin[u][2].w};
                for (int sh = 0; sh < S; sh++) {
                    u32x4 v;
                    switch (sh - pw) {
                    case -3: v = conv_shifted<-3>(w12); break;
                    case -2: v = conv_shifted<-2>(w12); break;
                    case -1: v = conv_shifted<-1>(w12); break;
                    case 0: v = conv_shifted<0>(w12); break;
                    case 1: v = conv_shifted<1>(w12); break;
                    case 2: v = conv_shifted<2>(w12); break;
                    default: v = conv_shifted<3>(w12); break;
                    }
                    lds_store16(li + (sh * Bc + c) * XP + 8 * ch, v);
                }
            }
            if (item / NCH < Bk) lds_store16(ld + (item / NCH) * XP + 8 * ch, vd[u]);
        }
    };
    // tiles of the (Bk/16) x (Bc/16) grid: wave w takes tiles w, w+8 (TPW of them) over the
    // whole step, or, with fewer than 8 tiles, tile w % ntile and part w / ntile of the
    // step's 32-deep chunks
    const int tj = Bk / 16, ntile = tj * (Bc / 16);
    const int nh = ntile >= 8 ? 1 : 8 / ntile, half = ntile >= 8 ? 0 : wave / ntile;
    const int kk0 = half * KK / nh, kk1 = (half + 1) * KK / nh;
    f32x4 acc[TPW][SMAX];
#pragma unroll
    for (int u = 0; u < TPW; u++)
#pragma unroll
        for (int sh = 0; sh < SMAX; sh++) acc[u][sh] = f32x4{0.f, 0.f, 0.f, 0.f};
    load(st0);
    for (int64_t st = st0; st < st1; st++) {
        const int buf = (int)((st - st0) & 1);
        stage(buf);
        __syncthreads();
        load(st + 1);   // in flight during this step's products
        const BSMM_LDS uint16_t* li = smi + buf * S * Bc * XP;
        const BSMM_LDS uint16_t* ld = smd + buf * Bk * XP;
#pragma unroll
        for (int u = 0; u < TPW; u++) {
            const int tile = ntile >= 8 ? wave + 8 * u : wave % ntile;
            const int jt = tile % tj, it = tile / tj;
            for (int kk = kk0; kk < kk1; kk++) {
                const u32x4 fb = *reinterpret_cast<const BSMM_LDS u32x4*>(ld + (jt * 16 + m16) * XP + kk * 32 + 8 * g4);
#pragma unroll
                for (int sh = 0; sh < SMAX; sh++)
                    if (sh < S) {
                        const u32x4 fa = *reinterpret_cast<const BSMM_LDS u32x4*>(
                            li + (sh * Bc + it * 16 + m16) * XP + kk * 32 + 8 * g4);
                        mma<DT>(acc[u][sh], fb, fa);   // D[j][i]: lane holds j = 4*g4 + v, i = m16
                    }
            }
        }
        // the other buffer is rewritten next step, after the barrier that follows its stage
    }
    // partial tiles of a tile's waves (ntile < 8), added in wave order
    f32x4* red = reinterpret_cast<f32x4*>(dsm);   // [wave][tap][lane]
    if (nh > 1) {
        __syncthreads();   // the step buffers are no longer read
        if (half > 0)
#pragma unroll
            for (int sh = 0; sh < SMAX; sh++)
                if (sh < S) red[(wave * SMAX + sh) * 64 + lane] = acc[0][sh];
        __syncthreads();
        if (half == 0)
            for (int hh = 1; hh < nh; hh++)
#pragma unroll
                for (int sh = 0; sh < SMAX; sh++)
                    if (sh < S) acc[0][sh] += red[((wave + hh * ntile) * SMAX + sh) * 64 + lane];
    }
    if (half > 0) return;
#pragma unroll
    for (int u = 0; u < TPW; u++) {
        const int tile = ntile >= 8 ? wave + 8 * u : wave % ntile;
        if (tile >= ntile) continue;
        const int jt = tile % tj, it = tile / tj;
        const int i = it * 16 + m16;
#pragma unroll
        for (int sh = 0; sh < SMAX; sh++) {
            if (sh >= S) continue;
            const int tap = r * S + sh;
#pragma unroll
            for (int v = 0; v < 4; v++) {
                const int j = jt * 16 + 4 * g4 + v;
                const int64_t e = (((int64_t)b * Bc + i) * RS + tap) * Bk + j;
                if (a.nparts > 1)
                    a.ws[(int64_t)part * a.nb * Bc * RS * Bk + e] = acc[u][sh][v];
                else
                    ((float*)a.out)[e] = acc[u][sh][v];
            }
        }
    }
}

// Positions per step of the row-form filter gradient (its LDS: two buffers of S input
// copies and the dO values), or 0 when the shape does not fit it.
static int conv_updat_rows_sp(const ConvArgs& a) {
    if (!conv_mfma_updat_ok(a)) return 0;
    if ((a.Bc != 16 && a.Bc != 32 && a.Bc != 64) || (a.Bk != 16 && a.Bk != 32 && a.Bk != 64)) return 0;
    if (a.W % 8 != 0 || a.Q % 8 != 0 || a.S > 7 || a.pad[2] > 3 || a.S - 1 - a.pad[2] > 3) return 0;
    for (int sp : {256, 128}) {
        const int64_t lds = 2LL * (a.S * a.Bc + a.Bk) * (sp + 8) * 2;
        if (lds <= 160 * 1024) return sp;
    }
    return 0;
}

// Sum of the filter gradient's parts in part order (deterministic).
__global__ __launch_bounds__(256) void conv_updat_reduce(ConvArgs a, int64_t E) {
    for (int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x; e < E; e += (int64_t)gridDim.x * 256) {
        float v = 0.f;
        for (int p = 0; p < a.nparts; p++) v += a.ws[p * E + e];
        ((float*)a.out)[e] = v;
    }
}

bool conv_gather_updat_ok(const ConvArgs& a) {
    if (conv_mfma_updat_ok(a) || a.a_bytes == 0 || a.b_bytes == 0) return false;
    return (a.Bc == 16 || a.Bc == 32 || a.Bc == 64) && (a.Bk == 16 || a.Bk == 32 || a.Bk == 64);
}

int conv_updat_parts(const ConvArgs& a) {
    const bool gather = conv_gather_updat_ok(a);
    const int64_t wgs = gather ? (int64_t)a.nb * a.T * a.R * a.S
                               : (int64_t)a.nb * a.R * (conv_updat_rows_sp(a) ? 1 : a.S);
    const int64_t mpq = (int64_t)a.M * a.P * a.Q, np = gather ? 128 : 256;
    const int64_t steps = a.N * ((mpq + np - 1) / np);
    int64_t p = wgs > 0 ? (4096 + wgs - 1) / wgs : 1;   // ~16 workgroups per compute unit
    if (p > 16) p = 16;
    if (p > steps / 4) p = steps / 4;
    return p < 1 ? 1 : (int)p;
}

bool conv_mfma_updat_ok(const ConvArgs& a) {
    if (a.dt == BSMM_F32 || a.T != 1 || a.D != 1 || a.a_bytes == 0) return false;
    for (int i = 0; i < 3; i++)
        if (a.st[i] != 1 || a.dl[i] != 1) return false;
    return a.Bc % 16 == 0 && a.Bk % 16 == 0 && a.Bc <= 64 && a.Bk <= 64;
}

// ---------------------------------------------------------------------------------
// Gathering matrix-core path (fprop and bprop for any geometry: 1-, 2- or 3-D images,
// strides, dilations, every padding; fp32 and 16-bit storage).  It is the implicit
// product of each filter tap with the input values that tap reads:
//
//   out[n, o, pos] = sum over the group's blocks b, taps tau, contraction channels c of
//                    Wop[b, tau][o][c] * In[n, in(b, c), src(pos, tau)]
//
// fprop: src = pos*stride - pad + tau*dilation per dimension (zero outside the image),
// Wop[o][c] = F[b, c, tau, o].  bprop (the input gradient): src = (pos + pad -
// tau*dilation) / stride where that divides exactly and lands inside dO, else zero,
// Wop[o][c] = F[b, o, tau, c]; this is the transposed convolution with no flipped
// filter copy.  A workgroup (4 waves) owns one block group (blocks sharing one output
// channel list, CO = 16*OT channels), one image and 256 consecutive output positions,
// one per thread.  Per step (block, tap, KC contraction channels) each thread gathers
// its position's KC input values (one buffer load per channel: the channel offset is
// scalar, the position offset per lane, out-of-image positions read zero) and writes
// them as one LDS row [position][channel]; the filter tile is staged as [output
// channel][channel].  Both operand fragments are then plain 16-byte LDS reads (lane l:
// row l % 16, channels 16 bytes' worth from (l / 16)); wave w runs position tiles 4w ..
// 4w+3 against every output tile.  The next step's loads are in flight during the
// current step's products (double-buffered LDS, one barrier per step); the sum runs in
// a fixed order (blocks, taps, channels): deterministic.
// Positions of the largest residue class (residue 0 in every dimension) of a D x H x W
// image under strides st.
__host__ __device__ inline int64_t conv_class_max(int D, int H, int W, const int* st) {
    return (int64_t)((D + st[0] - 1) / st[0]) * ((H + st[1] - 1) / st[1]) * ((W + st[2] - 1) / st[2]);
}

template <int DT, int OT, bool TR, int NP>
__global__ __launch_bounds__(256) void conv_gather_kernel(ConvArgs a) {
    constexpr bool F32 = DT == BSMM_F32;
    constexpr int ES = F32 ? 4 : 2;          // bytes per value
    constexpr int VEC = 16 / ES;             // values per 16 bytes
    constexpr int KC = 4 * VEC;              // contraction channels per step
    constexpr int CO = 16 * OT;
    // NP output positions per workgroup (256 or 64): TPP threads per position, each
    // gathering CPT of the step's channels; TPW 16-position tiles per wave
    constexpr int TPP = 256 / NP, CPT = KC / TPP, TPW = NP / 64;
    constexpr int PITCH = 80;                // LDS row: KC values (64 bytes) + 16
    constexpr int WCH = KC * CO / VEC;       // 16-byte filter chunks per step (<= 256)
    __shared__ __attribute__((aligned(16))) char gsm[2][NP * PITCH];
    __shared__ __attribute__((aligned(16))) char wsm[2][CO * PITCH];

    const int CI = TR ? a.Bk : a.Bc;
    const int32_t* in_idx = TR ? a.kidx : a.cidx;
    const int32_t* out_idx = TR ? a.cidx : a.kidx;
    const int Di = TR ? a.M : a.D, Hi = TR ? a.P : a.H, Wi = TR ? a.Q : a.W;   // gathered tensor
    const int Ho = TR ? a.H : a.P, Wo = TR ? a.W : a.Q;                         // this pass's output
    const int64_t HWi = (int64_t)Di * Hi * Wi;
    const int64_t HWo = (int64_t)(TR ? a.D : a.M) * Ho * Wo;
    const int64_t Cin = TR ? a.K : a.C, Cout = TR ? a.C : a.K;
    const int TRS = a.T * a.R * a.S;
    const int nch = (CI + KC - 1) / KC;

    // The input gradient with a stride above 1 takes its output positions one residue
    // class (position mod stride in every dimension) at a time: inside a class the taps
    // that divide exactly are the same for every position, so the others are skipped
    // whole.  Otherwise one class holds every position.  Class positions: x_d = cr[d] +
    // k*cs[d], k < cn[d].
    const bool cls = TR && (a.st[0] > 1 || a.st[1] > 1 || a.st[2] > 1);
    const int Do = TR ? a.D : a.M;
    int cr[3] = {0, 0, 0}, cs[3] = {1, 1, 1}, cn[3] = {Do, Ho, Wo};
    int64_t tile, rest;
    if (cls) {
        const int nclass = a.st[0] * a.st[1] * a.st[2];
        const int64_t tpc = (conv_class_max(Do, Ho, Wo, a.st) + NP - 1) / NP;
        const int64_t ct = blockIdx.x % (nclass * tpc);
        rest = blockIdx.x / (nclass * tpc);
        const int cl = (int)(ct / tpc);
        tile = ct % tpc;
        cr[2] = cl % a.st[2];
        cr[1] = (cl / a.st[2]) % a.st[1];
        cr[0] = cl / (a.st[2] * a.st[1]);
#pragma unroll
        for (int d = 0; d < 3; d++) {
            cs[d] = a.st[d];
            cn[d] = cr[d] < cn[d] ? (cn[d] - cr[d] + a.st[d] - 1) / a.st[d] : 0;
        }
    } else {
        const int64_t tpc = (HWo + NP - 1) / NP;
        tile = blockIdx.x % tpc;
        rest = blockIdx.x / tpc;
    }
    const int64_t ccount = (int64_t)cn[0] * cn[1] * cn[2];
    const int64_t n = rest % a.N;
    const int g = (int)(rest / a.N);
    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    // this thread's position and channel part (the part is the wave's: a scalar)
    const int tp = t % NP, cq = TPP == 1 ? 0 : __builtin_amdgcn_readfirstlane(t / NP);
    const int gb = a.gptr[g], ge = a.gptr[g + 1];
    const int nsteps = ccount > 0 ? (ge - gb) * TRS * nch : 0;   // an empty class writes nothing
    const rsrc_t rin = make_rsrc(a.a, a.a_bytes);
    // position i of the class -> its element offset in the output image
    auto coords = [&](int64_t i, int& x0, int& x1, int& x2) {
        x2 = cr[2] + (int)(i % cn[2]) * cs[2];
        x1 = cr[1] + (int)((i / cn[2]) % cn[1]) * cs[1];
        x0 = cr[0] + (int)(i / ((int64_t)cn[2] * cn[1])) * cs[0];
    };

    // this thread's output position
    const int64_t pidx = tile * NP + tp;
    const bool pok = pidx < ccount;
    int od = 0, oh = 0, ow = 0;
    if (pok) coords(pidx, od, oh, ow);
    // steps whose tap has no exactly dividing position in this class are skipped
    auto tap_ok = [&](int tap) -> bool {
        if (!cls) return true;
        const int t3[3] = {tap / (a.S * a.R), (tap / a.S) % a.R, tap % a.S};
#pragma unroll
        for (int d = 0; d < 3; d++) {
            const int u = cr[d] + a.pad[d] - t3[d] * a.dl[d];
            if (((u % a.st[d]) + a.st[d]) % a.st[d] != 0) return false;
        }
        return true;
    };
    auto next_step = [&](int st) {
        while (st < nsteps && !tap_ok((st / nch) % TRS)) st++;
        return st;
    };

    // per-lane element offset of the gathered value for tap (tt, r, s), or -1
    auto src_of = [&](int tt, int r, int s) -> int64_t {
        int c3[3];
        const int o3[3] = {od, oh, ow}, t3[3] = {tt, r, s}, n3[3] = {Di, Hi, Wi};
#pragma unroll
        for (int d = 0; d < 3; d++) {
            if constexpr (TR) {
                const int u = o3[d] + a.pad[d] - t3[d] * a.dl[d];
                if (u < 0 || u % a.st[d] != 0) return -1;
                c3[d] = u / a.st[d];
            } else {
                c3[d] = o3[d] * a.st[d] - a.pad[d] + t3[d] * a.dl[d];
            }
            if (c3[d] < 0 || c3[d] >= n3[d]) return -1;
        }
        return ((int64_t)c3[0] * Hi + c3[1]) * Wi + c3[2];
    };

    uint32_t gv[CPT];   // the next step's gathered values (16-bit: low half)
    u32x4 wv;          // and one 16-byte filter chunk (threads < WCH)
    const int wc = t / (CO / VEC), wp = t % (CO / VEC);   // fprop chunk: channel, output part
    const int bo = t / (KC / VEC), bq = t % (KC / VEC);   // bprop chunk: output, channel part
    auto issue = [&](int step) {
        const int chunk = step % nch, tap = (step / nch) % TRS, e = step / (nch * TRS);
        const int b = __builtin_amdgcn_readfirstlane(a.gblk[gb + e]);
        const int s = tap % a.S, r = (tap / a.S) % a.R, tt = tap / (a.S * a.R);
        const int64_t so = pok ? src_of(tt, r, s) : -1;
        const uint32_t voff = so >= 0 ? (uint32_t)(so * ES) : kOffLane;
        const int c0 = chunk * KC, cc0 = c0 + cq * CPT;
#pragma unroll
        for (int c = 0; c < CPT; c++) {
            const bool cv = cc0 + c < CI;   // uniform per wave
            const int ch = cv ? in_idx[b * CI + cc0 + c] : 0;
            const uint32_t soff = cv ? (uint32_t)(((n * Cin + ch) * HWi) * ES) : kOffOff;
            gv[c] = F32 ? bload32(rin, voff, soff) : bload16(rin, voff, soff);
        }
        const void* fp = kZero16;
        if constexpr (TR) {
            if (t < WCH && c0 + bq * VEC < CI)
                fp = (const char*)a.b + ((((int64_t)b * a.Bc + bo) * TRS + tap) * a.Bk + c0 + bq * VEC) * ES;
        } else {
            if (t < WCH && c0 + wc < CI)
                fp = (const char*)a.b + ((((int64_t)b * a.Bc + c0 + wc) * TRS + tap) * a.Bk + wp * VEC) * ES;
        }
        wv = *reinterpret_cast<const u32x4*>(fp);
    };
    auto stage = [&](int buf) {
        char* grow = gsm[buf] + tp * PITCH + cq * (64 / TPP);
#pragma unroll
        for (int j = 0; j < CPT / VEC; j++) {
            u32x4 v;
            if constexpr (F32) {
                v = u32x4{gv[4 * j], gv[4 * j + 1], gv[4 * j + 2], gv[4 * j + 3]};
            } else {
                v = u32x4{gv[8 * j] | (gv[8 * j + 1] << 16), gv[8 * j + 2] | (gv[8 * j + 3] << 16),
                          gv[8 * j + 4] | (gv[8 * j + 5] << 16), gv[8 * j + 6] | (gv[8 * j + 7] << 16)};
            }
            *reinterpret_cast<u32x4*>(grow + 16 * j) = v;
        }
        if (t < WCH) {
            if constexpr (TR) {
                *reinterpret_cast<u32x4*>(wsm[buf] + bo * PITCH + bq * 16) = wv;
            } else {
                const uint32_t w[4] = {wv.x, wv.y, wv.z, wv.w};
#pragma unroll
                for (int h = 0; h < VEC; h++) {
                    char* dst = wsm[buf] + (wp * VEC + h) * PITCH + wc * ES;
                    if constexpr (F32)
                        *reinterpret_cast<uint32_t*>(dst) = w[h];
                    else
                        *reinterpret_cast<uint16_t*>(dst) = (uint16_t)(h & 1 ? w[h >> 1] >> 16 : w[h >> 1]);
                }
            }
        }
    };

    f32x4 acc[TPW][OT];
#pragma unroll
    for (int u = 0; u < TPW; u++)
#pragma unroll
        for (int o = 0; o < OT; o++) acc[u][o] = f32x4{0.f, 0.f, 0.f, 0.f};
    const int m16 = lane & 15, q16 = (lane >> 4) * 16;
    int step = next_step(0), buf = 0;
    if (step < nsteps) {
        issue(step);
        stage(0);
    }
    __syncthreads();
    while (step < nsteps) {
        const int nxt = next_step(step + 1);
        if (nxt < nsteps) issue(nxt);
        u32x4 bf[OT];
#pragma unroll
        for (int o = 0; o < OT; o++) bf[o] = *reinterpret_cast<const u32x4*>(wsm[buf] + (o * 16 + m16) * PITCH + q16);
#pragma unroll
        for (int u = 0; u < TPW; u++) {
            const u32x4 af = *reinterpret_cast<const u32x4*>(gsm[buf] + ((wave * TPW + u) * 16 + m16) * PITCH + q16);
#pragma unroll
            for (int o = 0; o < OT; o++) mma<DT>(acc[u][o], af, bf[o]);
        }
        if (nxt < nsteps) stage(buf ^ 1);
        __syncthreads();
        buf ^= 1;
        step = nxt;
    }
    // lane: class positions 4*(lane/16) .. +3 of each of its tiles, output channel
    // o*16 + lane%16 (consecutive in memory unless positions go by residue class)
    const int b0 = a.gblk[gb];
    const bool vec = !cls && HWo % 4 == 0;
#pragma unroll
    for (int o = 0; o < OT; o++) {
        const int64_t ch = out_idx[b0 * CO + o * 16 + m16];
        const int64_t base = (n * Cout + ch) * HWo;
#pragma unroll
        for (int u = 0; u < TPW; u++) {
            const int64_t p0 = tile * NP + (wave * TPW + u) * 16 + 4 * (lane >> 4);
            if (vec && p0 + 4 <= HWo) {
                store4<DT>(a.out, base + p0, acc[u][o]);
            } else {
#pragma unroll
                for (int v = 0; v < 4; v++)
                    if (p0 + v < ccount) {
                        int x0, x1, x2;
                        coords(p0 + v, x0, x1, x2);
                        store_elt(a.out, base + ((int64_t)x0 * Ho + x1) * Wo + x2, acc[u][o][v], DT);
                    }
            }
        }
    }
}

// Gathering matrix-core filter gradient (any geometry and dtype; Bc and Bk of 16, 32 or
// 64): dF[b, :, tau, :] = G^T . dO over the (image, position) pairs, where G[p][c] =
// In[n, C_b[c], src(p, tau)] (the fprop gather, zero outside the image).  One workgroup
// per (block, tap, part) walks its part of the (image, 128-position tile) steps: two
// threads per position load half of its Bc gathered input values and half of its Bk dO
// values (channel offsets scalar, position offsets per lane) into registers during the
// previous step's products, then write them as [channel][position] rows; each wave
// contracts 32 of the step's positions for every (16 x 16) tile of dF (both fragments
// plain 16-byte LDS reads).  The waves' partial tiles are added in wave order, and parts
// (with a workspace) are summed in part order by conv_updat_reduce: deterministic.
template <int DT, int BCT, int BKT>
__global__ __launch_bounds__(256) void conv_gather_updat_kernel(ConvArgs a) {
    extern __shared__ __attribute__((aligned(16))) uint16_t dsm[];
    constexpr bool F32 = DT == BSMM_F32;
    constexpr int ES = F32 ? 4 : 2;
    constexpr int BC = 16 * BCT, BK = 16 * BKT, HC = BC / 2, HK = BK / 2;
    constexpr int NP = 128;                   // positions per step
    constexpr int PP = NP * ES + 16;          // LDS row pitch, bytes
    char* gs = reinterpret_cast<char*>(dsm);  // [BC][PP]
    char* ds = gs + BC * PP;                  // [BK][PP]

    const int TRS = a.T * a.R * a.S;
    const int part = blockIdx.x % a.nparts;
    const int bt = blockIdx.x / a.nparts;
    const int tap = bt % TRS, b = bt / TRS;
    const int s = tap % a.S, r = (tap / a.S) % a.R, tt = tap / (a.S * a.R);
    const int64_t MPQ = (int64_t)a.M * a.P * a.Q, DHW = (int64_t)a.D * a.H * a.W;
    const int64_t npt = (MPQ + NP - 1) / NP, nst = a.N * npt;
    const int64_t s0 = nst * part / a.nparts, s1 = nst * (part + 1) / a.nparts;
    const rsrc_t rin = make_rsrc(a.a, a.a_bytes), rdo = make_rsrc(a.b, a.b_bytes);
    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    const int p = t % NP, hh = t / NP;

    uint32_t gv[HC], dv[HK];
    auto issue = [&](int64_t step) {
        const int64_t n = step / npt, pos = (step % npt) * NP + p;
        uint32_t vi = kOffLane, vo = kOffLane;
        if (pos < MPQ) {
            vo = (uint32_t)(pos * ES);
            const int ow = (int)(pos % a.Q), oh = (int)((pos / a.Q) % a.P), od = (int)(pos / ((int64_t)a.Q * a.P));
            const int id = od * a.st[0] - a.pad[0] + tt * a.dl[0];
            const int ih = oh * a.st[1] - a.pad[1] + r * a.dl[1];
            const int iw = ow * a.st[2] - a.pad[2] + s * a.dl[2];
            if (id >= 0 && id < a.D && ih >= 0 && ih < a.H && iw >= 0 && iw < a.W)
                vi = (uint32_t)((((int64_t)id * a.H + ih) * a.W + iw) * ES);
        }
#pragma unroll
        for (int c = 0; c < HC; c++) {
            const int ch = a.cidx[b * BC + hh * HC + c];
            const uint32_t so = (uint32_t)((n * a.C + ch) * DHW * ES);
            gv[c] = F32 ? bload32(rin, vi, so) : bload16(rin, vi, so);
        }
#pragma unroll
        for (int j = 0; j < HK; j++) {
            const int kc = a.kidx[b * BK + hh * HK + j];
            const uint32_t so = (uint32_t)((n * a.K + kc) * MPQ * ES);
            dv[j] = F32 ? bload32(rdo, vo, so) : bload16(rdo, vo, so);
        }
    };
    auto stage = [&]() {
#pragma unroll
        for (int c = 0; c < HC; c++) {
            char* dst = gs + (hh * HC + c) * PP + p * ES;
            if constexpr (F32)
                *reinterpret_cast<uint32_t*>(dst) = gv[c];
            else
                *reinterpret_cast<uint16_t*>(dst) = (uint16_t)gv[c];
        }
#pragma unroll
        for (int j = 0; j < HK; j++) {
            char* dst = ds + (hh * HK + j) * PP + p * ES;
            if constexpr (F32)
                *reinterpret_cast<uint32_t*>(dst) = dv[j];
            else
                *reinterpret_cast<uint16_t*>(dst) = (uint16_t)dv[j];
        }
    };

    f32x4 acc[BCT][BKT];
#pragma unroll
    for (int i = 0; i < BCT; i++)
#pragma unroll
        for (int j = 0; j < BKT; j++) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    const int m16 = lane & 15, g4 = lane >> 4;
    if (s0 < s1) issue(s0);
    for (int64_t step = s0; step < s1; step++) {
        __syncthreads();   // the previous step's fragments are read
        stage();
        __syncthreads();
        if (step + 1 < s1) issue(step + 1);
        // wave w: positions 32w .. 32w+31 of the step (16-bit: one 32-deep fragment; fp32:
        // two of 16)
#pragma unroll
        for (int f = 0; f < (F32 ? 2 : 1); f++) {
            const int off = (F32 ? (32 * wave + 16 * f + 4 * g4) : (32 * wave + 8 * g4)) * ES;
            u32x4 bf[BKT];
#pragma unroll
            for (int j = 0; j < BKT; j++) bf[j] = *reinterpret_cast<const u32x4*>(ds + (16 * j + m16) * PP + off);
#pragma unroll
            for (int i = 0; i < BCT; i++) {
                const u32x4 af = *reinterpret_cast<const u32x4*>(gs + (16 * i + m16) * PP + off);
#pragma unroll
                for (int j = 0; j < BKT; j++) mma<DT>(acc[i][j], af, bf[j]);
            }
        }
    }
    // the four waves' partial tiles, added in wave order
    __syncthreads();
    f32x4* red = reinterpret_cast<f32x4*>(dsm);   // [wave][tile][lane]
    constexpr int NT = BCT * BKT;
#pragma unroll
    for (int i = 0; i < BCT; i++)
#pragma unroll
        for (int j = 0; j < BKT; j++) red[(wave * NT + i * BKT + j) * 64 + lane] = acc[i][j];
    __syncthreads();
    float* out = a.nparts > 1 ? a.ws + (int64_t)part * a.nb * BC * TRS * BK : (float*)a.out;
    for (int q = t; q < NT * 64; q += 256) {
        const int tile = q / 64, l = q % 64;
        const f32x4 v = ((red[tile * 64 + l] + red[(NT + tile) * 64 + l]) + red[(2 * NT + tile) * 64 + l]) +
                        red[(3 * NT + tile) * 64 + l];
        const int i0 = (tile / BKT) * 16 + 4 * (l >> 4), j = (tile % BKT) * 16 + (l & 15);
#pragma unroll
        for (int v4 = 0; v4 < 4; v4++) out[(((int64_t)b * BC + i0 + v4) * TRS + tap) * BK + j] = v[v4];
    }
}

// Output channels that no block writes: zero.
template <int DT>
__global__ __launch_bounds__(256) void conv_zero_kernel(ConvArgs a, int64_t Cout, int64_t HWo) {
    const int64_t total = a.N * a.nz * HWo;
    for (int64_t o = (int64_t)blockIdx.x * 256 + threadIdx.x; o < total; o += (int64_t)gridDim.x * 256) {
        const int64_t sp = o % HWo, zc = (o / HWo) % a.nz, n = o / (HWo * a.nz);
        store_elt(a.out, (n * Cout + a.zch[zc]) * HWo + sp, 0.f, DT);
    }
}

bool conv_mfma_plan(ConvArgs& a, int pass) {
    if (pass > 1 || a.dt == BSMM_F32 || a.T != 1 || a.D != 1 || a.a_bytes == 0) return false;
    for (int i = 0; i < 3; i++)
        if (a.st[i] != 1 || a.dl[i] != 1) return false;
    const int CI = pass == 1 ? a.Bk : a.Bc, CO = pass == 1 ? a.Bc : a.Bk;
    if (CI % 32 != 0 || (CO != 16 && CO != 32 && CO != 64)) return false;
    if (pass == 1 && (a.pad[1] > a.R - 1 || a.pad[2] > a.S - 1)) return false;   // transposed pads >= 0
    const int Wo = pass == 1 ? a.W : a.Q;
    const int PT = (Wo + 15) / 16;
    if (PT > 16) return false;
    const int Ho = pass == 1 ? a.H : a.P;
    a.TH = PT >= 8 ? 1 : 8 / PT;
    if (a.TH > Ho) a.TH = Ho;
    const int ROWS = a.TH + a.R - 1;
    a.cpitch = ROWS * PT * 16 + 8;
    a.lds_bytes = (a.S * 32 * a.cpitch + a.R * a.S * CO * 40) * 2;
    return a.lds_bytes <= 80 * 1024;   // two workgroups per compute unit
}

template <int DT, int OT, bool TR>
static hipError_t launch_conv_mfma_t(const ConvArgs& a, hipStream_t st) {
    const int Ho = TR ? a.H : a.P;
    const int64_t grid = (int64_t)a.ngroups * a.N * ((Ho + a.TH - 1) / a.TH);
    if (grid > INT32_MAX) return hipErrorInvalidConfiguration;
    const int pass = TR ? BSMM_PASS_CONV_BPROP : BSMM_PASS_CONV_FPROP;
    void *e0 = nullptr, *e1 = nullptr;
    prof_events(pass, &e0, &e1);   // one timing record spans both launches
    if (a.nz > 0) {   // zero the channels no block writes
        const int64_t HWo = TR ? (int64_t)a.H * a.W : (int64_t)a.P * a.Q;
        const int64_t Cout = TR ? a.C : a.K;
        int64_t zg = (a.N * a.nz * HWo + 255) / 256;
        if (zg > (1 << 20)) zg = 1 << 20;
        hipError_t e = launch_ev(conv_zero_kernel<DT>, dim3((unsigned)zg), dim3(256), st, e0, nullptr, a, Cout, HWo);
        if (e != hipSuccess) return e;
        e0 = nullptr;
    }
    auto kern = conv_mfma_kernel<DT, OT, TR>;
    if (e0 || e1)
        hipExtLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(256), a.lds_bytes, st, (hipEvent_t)e0, (hipEvent_t)e1,
                              0, a);
    else
        hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(256), a.lds_bytes, st, a);
    return hipGetLastError();
}

bool conv_gather_ok(const ConvArgs& a, int pass) {
    if (pass > 1 || a.a_bytes == 0) return false;
    const int CO = pass == 1 ? a.Bc : a.Bk;
    if (CO != 16 && CO != 32 && CO != 64) return false;
    const int vec = a.dt == BSMM_F32 ? 4 : 8;
    return pass == 0 || a.Bk % vec == 0;   // bprop reads 16-byte runs of the contraction
}

// The channels no group writes are zeroed first; one timing record spans both launches.
template <int DT, int OT, bool TR>
static hipError_t launch_conv_gather_t(const ConvArgs& a, hipStream_t st) {
    const int64_t HWo = TR ? (int64_t)a.D * a.H * a.W : (int64_t)a.M * a.P * a.Q;
    const bool cls = TR && (a.st[0] > 1 || a.st[1] > 1 || a.st[2] > 1);   // residue classes
    auto tiles = [&](int np) {
        return cls ? (int64_t)a.st[0] * a.st[1] * a.st[2] * ((conv_class_max(a.D, a.H, a.W, a.st) + np - 1) / np)
                   : (HWo + np - 1) / np;
    };
    // 256-position tiles while they give at least two workgroups per CU, else 64
    const bool big = (int64_t)a.ngroups * a.N * tiles(256) >= 512;
    const int64_t grid = (int64_t)a.ngroups * a.N * tiles(big ? 256 : 64);
    if (grid > INT32_MAX) return hipErrorInvalidConfiguration;
    const int pass = TR ? BSMM_PASS_CONV_BPROP : BSMM_PASS_CONV_FPROP;
    void *e0 = nullptr, *e1 = nullptr;
    prof_events(pass, &e0, &e1);
    if (a.nz > 0) {
        const int64_t Cout = TR ? a.C : a.K;
        int64_t zg = (a.N * a.nz * HWo + 255) / 256;
        if (zg > (1 << 20)) zg = 1 << 20;
        hipError_t e = launch_ev(conv_zero_kernel<DT>, dim3((unsigned)zg), dim3(256), st, e0, nullptr, a, Cout, HWo);
        if (e != hipSuccess) return e;
        e0 = nullptr;
    }
    if (grid == 0) return hipSuccess;
    if (big) return launch_ev(conv_gather_kernel<DT, OT, TR, 256>, dim3((unsigned)grid), dim3(256), st, e0, e1, a);
    return launch_ev(conv_gather_kernel<DT, OT, TR, 64>, dim3((unsigned)grid), dim3(256), st, e0, e1, a);
}

template <int DT, bool TR>
static hipError_t launch_conv_gather(const ConvArgs& a, hipStream_t st) {
    switch (TR ? a.Bc : a.Bk) {
    case 16: return launch_conv_gather_t<DT, 1, TR>(a, st);
    case 32: return launch_conv_gather_t<DT, 2, TR>(a, st);
    case 64: return launch_conv_gather_t<DT, 4, TR>(a, st);
    }
    return hipErrorInvalidValue;
}

template <int DT, bool TR>
static hipError_t launch_conv_mfma(const ConvArgs& a, hipStream_t st) {
    switch (TR ? a.Bc : a.Bk) {
    case 16: return launch_conv_mfma_t<DT, 1, TR>(a, st);
    case 32: return launch_conv_mfma_t<DT, 2, TR>(a, st);
    case 64: return launch_conv_mfma_t<DT, 4, TR>(a, st);
    }
    return hipErrorInvalidValue;
}

template <int DT, int BCT, int BKT>
static hipError_t launch_conv_gather_updat_t(const ConvArgs& a, hipStream_t st) {
    const int64_t wgs = (int64_t)a.nb * a.T * a.R * a.S * a.nparts;
    if (wgs == 0) return hipSuccess;
    if (wgs > INT32_MAX) return hipErrorInvalidConfiguration;
    constexpr int ES = DT == BSMM_F32 ? 4 : 2;
    const int stage = 16 * (BCT + BKT) * (128 * ES + 16), red = 4 * BCT * BKT * 64 * 16;
    const int lds = stage > red ? stage : red;
    void *e0 = nullptr, *e1 = nullptr;   // one timing record spans the parts and their sum
    prof_events(BSMM_PASS_CONV_UPDAT, &e0, &e1);
    auto kern = conv_gather_updat_kernel<DT, BCT, BKT>;
    if (e0 || e1)
        hipExtLaunchKernelGGL(kern, dim3((unsigned)wgs), dim3(256), lds, st, (hipEvent_t)e0,
                              (hipEvent_t)(a.nparts == 1 ? e1 : nullptr), 0, a);
    else
        hipLaunchKernelGGL(kern, dim3((unsigned)wgs), dim3(256), lds, st, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || a.nparts == 1) return e;
    const int64_t E = (int64_t)a.nb * a.Bc * a.T * a.R * a.S * a.Bk;
    int64_t rg = (E + 255) / 256;
    if (rg > 4096) rg = 4096;
    return launch_ev(conv_updat_reduce, dim3((unsigned)rg), dim3(256), st, nullptr, e1, a, E);
}

template <int DT, int BCT>
static hipError_t launch_conv_gather_updat_c(const ConvArgs& a, hipStream_t st) {
    switch (a.Bk) {
    case 16: return launch_conv_gather_updat_t<DT, BCT, 1>(a, st);
    case 32: return launch_conv_gather_updat_t<DT, BCT, 2>(a, st);
    case 64: return launch_conv_gather_updat_t<DT, BCT, 4>(a, st);
    }
    return hipErrorInvalidValue;
}

template <int DT>
static hipError_t launch_conv_gather_updat(const ConvArgs& a, hipStream_t st) {
    switch (a.Bc) {
    case 16: return launch_conv_gather_updat_c<DT, 1>(a, st);
    case 32: return launch_conv_gather_updat_c<DT, 2>(a, st);
    case 64: return launch_conv_gather_updat_c<DT, 4>(a, st);
    }
    return hipErrorInvalidValue;
}

template <int DT>
static hipError_t launch_conv_dt(const ConvArgs& a, int pass, hipStream_t st) {
    if constexpr (DT != BSMM_F32) {
        if (a.mfma == 1 && pass == 0) return launch_conv_mfma<DT, false>(a, st);
        if (a.mfma == 1 && pass == 1) return launch_conv_mfma<DT, true>(a, st);
    }
    if (a.mfma == 2 && pass == 0) return launch_conv_gather<DT, false>(a, st);
    if (a.mfma == 2 && pass == 1) return launch_conv_gather<DT, true>(a, st);
    if (pass == 2 && DT != BSMM_F32 && conv_updat_rows_sp(a)) {
        const int sp = conv_updat_rows_sp(a);
        const int64_t wgs = (int64_t)a.nb * a.R * a.nparts;
        if (wgs == 0) return hipSuccess;
        if (wgs > INT32_MAX) return hipErrorInvalidConfiguration;
        const int ntile = (a.Bc / 16) * (a.Bk / 16);
        const int64_t lds = std::max<int64_t>(2LL * (a.S * a.Bc + a.Bk) * (sp + 8) * 2, 8LL * 7 * 64 * 16);
        void *e0 = nullptr, *e1 = nullptr;
        prof_events(BSMM_PASS_CONV_UPDAT, &e0, &e1);
        auto kern = sp == 256 ? (ntile > 8 ? conv_updat_rows_kernel<DT, 256, 2> : conv_updat_rows_kernel<DT, 256, 1>)
                              : (ntile > 8 ? conv_updat_rows_kernel<DT, 128, 2> : conv_updat_rows_kernel<DT, 128, 1>);
        if (e0 || e1)
            hipExtLaunchKernelGGL(kern, dim3((unsigned)wgs), dim3(512), (uint32_t)lds, st, (hipEvent_t)e0,
                                  (hipEvent_t)(a.nparts == 1 ? e1 : nullptr), 0, a);
        else
            hipLaunchKernelGGL(kern, dim3((unsigned)wgs), dim3(512), (uint32_t)lds, st, a);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess || a.nparts == 1) return e;
        const int64_t E = (int64_t)a.nb * a.Bc * a.R * a.S * a.Bk;
        int64_t rg = (E + 255) / 256;
        if (rg > 4096) rg = 4096;
        return launch_ev(conv_updat_reduce, dim3((unsigned)rg), dim3(256), st, nullptr, e1, a, E);
    }
    if (pass == 2 && DT != BSMM_F32 && conv_mfma_updat_ok(a)) {
        const int64_t wgs = (int64_t)a.nb * a.R * a.S * a.nparts;
        if (wgs == 0) return hipSuccess;
        if (wgs > INT32_MAX) return hipErrorInvalidConfiguration;
        const int lds = 2 * (a.Bc + a.Bk) * (256 + 8) * 2;
        // one timing record spans the partial sums and their reduction
        void *e0 = nullptr, *e1 = nullptr;
        prof_events(BSMM_PASS_CONV_UPDAT, &e0, &e1);
        auto kern = conv_mfma_updat_kernel<DT>;
        if (e0 || e1)
            hipExtLaunchKernelGGL(kern, dim3((unsigned)wgs), dim3(512), lds, st, (hipEvent_t)e0,
                                  (hipEvent_t)(a.nparts == 1 ? e1 : nullptr), 0, a);
        else
            hipLaunchKernelGGL(kern, dim3((unsigned)wgs), dim3(512), lds, st, a);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess || a.nparts == 1) return e;
        const int64_t E = (int64_t)a.nb * a.Bc * a.R * a.S * a.Bk;
        int64_t rg = (E + 255) / 256;
        if (rg > 4096) rg = 4096;
        return launch_ev(conv_updat_reduce, dim3((unsigned)rg), dim3(256), st, nullptr, e1, a, E);
    }
    if (pass == 2 && conv_gather_updat_ok(a)) return launch_conv_gather_updat<DT>(a, st);
    if (pass == 2) {
        const int64_t rows = (int64_t)a.nb * a.Bc * a.T * a.R * a.S;
        if (rows == 0) return hipSuccess;
        if (rows > INT32_MAX) return hipErrorInvalidConfiguration;
        return launch(BSMM_PASS_CONV_UPDAT, conv_updat_kernel<DT>, dim3((unsigned)rows), dim3(256), st, a);
    }
    const int64_t total = pass == 0 ? a.N * a.K * a.M * a.P * a.Q : a.N * a.C * a.D * a.H * a.W;
    if (total == 0) return hipSuccess;
    int64_t grid = (total + 255) / 256;
    if (grid > (1 << 20)) grid = 1 << 20;   // grid-stride beyond that
    if (pass == 0) return launch(BSMM_PASS_CONV_FPROP, conv_fprop_kernel<DT>, dim3((unsigned)grid), dim3(256), st, a);
    return launch(BSMM_PASS_CONV_BPROP, conv_bprop_kernel<DT>, dim3((unsigned)grid), dim3(256), st, a);
}

hipError_t launch_conv(const ConvArgs& a, int pass, void* stream) {
    hipStream_t st = (hipStream_t)stream;
    switch (a.dt) {
    case BSMM_F32: return launch_conv_dt<BSMM_F32>(a, pass, st);
    case BSMM_BF16: return launch_conv_dt<BSMM_BF16>(a, pass, st);
    case BSMM_F16: return launch_conv_dt<BSMM_F16>(a, pass, st);
    }
    return hipErrorInvalidValue;
}

}  // namespace bsmm
