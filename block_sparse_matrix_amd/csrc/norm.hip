// Layer norm over the feature axis of either activation layout, with the optional
// ReLU at the end, and its gradient (kiteco/blocksparse README, "API Documentation" ›
// blocksparse.norms › layer_norm(x, g, b, axis=1, epsilon=1e-6, relu=False)).
//
// Per normalised vector (a row of an (N, C) array for axis 1, a column of a (C, N)
// array for axis 0): mean and biased variance over its C features, xhat =
// (x - mean) * rstd with rstd = 1/sqrt(var + epsilon), y = xhat * g + b per feature,
// then max(y, 0) when relu.  Gradient, with dyr = dy masked by y > 0 when relu:
// dg = sum over vectors of dyr * xhat, db = sum of dyr,
// dx = rstd * (dyr*g - mean(dyr*g) - xhat * mean(dyr*g * xhat)).
// Statistics and sums are fp32; every sum has a fixed order (deterministic).
//
// Axis 1: one workgroup per row holds the row in registers (one HBM read of x, one
// write of y); the gradient (512 threads) takes a run of rows per workgroup with the
// next rows in flight and leaves per-run partial dg/db in the workspace, added in run
// order by a second kernel.
// Axis 0: a workgroup owns 32 16-byte column vectors x a chunk of 128 rows held in
// registers, so every load is a coalesced row segment.  The chunks' column statistics
// (mean and squared deviations, or plain sums for the gradient) go through the
// workspace and are merged once per column in a fixed order (ln_cols_merge).
// Bound: HBM (|x| + |y| forward, |x| + |dy| + |dx| backward, plus the small partials).
#include "common.h"

// No fused multiply-adds from contraction in this file: the gradient subtracts the mean
// of the rounded products dy*g from those same rounded products, so a product must not
// be rounded in one place and kept exact (fused) in another.
#pragma clang fp contract(off)

namespace bsmm {

constexpr int kLnThreads = 256;
constexpr int kLnChunk = 128;   // rows per workgroup, axis 0

// ---- element access: VW consecutive values at element index idx (VW = 16 bytes' worth
// of storage, or 1 for rows/columns that are not 16-byte aligned) ----
template <int DT> __device__ __forceinline__ float ln_elt(const void* base, int64_t idx) {
    if constexpr (DT == BSMM_F32) {
        return ((const float*)base)[idx];
    } else {
        const uint32_t h = ((const uint16_t*)base)[idx];
        if constexpr (DT == BSMM_BF16)
            return __uint_as_float(h << 16);
        else
            return (float)__builtin_bit_cast(_Float16, (uint16_t)h);
    }
}
template <int DT, int VW> __device__ __forceinline__ void ln_load(const void* base, int64_t idx, float* v) {
    if constexpr (VW == 1) {
        v[0] = ln_elt<DT>(base, idx);
    } else {
        constexpr int S = DT == BSMM_F32 ? 4 : 2;
        const u32x4 w = *reinterpret_cast<const u32x4*>((const char*)base + idx * S);
        const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
        if constexpr (DT == BSMM_F32) {
#pragma unroll
            for (int i = 0; i < 4; i++) v[i] = __uint_as_float(ws[i]);
        } else if constexpr (DT == BSMM_BF16) {
#pragma unroll
            for (int i = 0; i < 4; i++) {
                v[2 * i] = __uint_as_float(ws[i] << 16);
                v[2 * i + 1] = __uint_as_float(ws[i] & 0xffff0000u);
            }
        } else {
#pragma unroll
            for (int i = 0; i < 4; i++) {
                v[2 * i] = (float)__builtin_bit_cast(_Float16, (uint16_t)(ws[i] & 0xffffu));
                v[2 * i + 1] = (float)__builtin_bit_cast(_Float16, (uint16_t)(ws[i] >> 16));
            }
        }
    }
}
template <int DT, int VW> __device__ __forceinline__ void ln_store(void* base, int64_t idx, const float* v) {
    if constexpr (VW == 1) {
        store_elt(base, idx, v[0], DT);
    } else if constexpr (DT == BSMM_F32) {
        *reinterpret_cast<f32x4*>((float*)base + idx) = f32x4{v[0], v[1], v[2], v[3]};
    } else {
        u32x4 w;
        w.x = to_storage16<DT>(v[0]) | (to_storage16<DT>(v[1]) << 16);
        w.y = to_storage16<DT>(v[2]) | (to_storage16<DT>(v[3]) << 16);
        w.z = to_storage16<DT>(v[4]) | (to_storage16<DT>(v[5]) << 16);
        w.w = to_storage16<DT>(v[6]) | (to_storage16<DT>(v[7]) << 16);
        *reinterpret_cast<u32x4*>((uint16_t*)base + idx) = w;
    }
}
// VW consecutive fp32 parameters (16-byte aligned when VW > 1)
template <int VW> __device__ __forceinline__ void ln_param(const float* p, int64_t idx, float* v) {
    if constexpr (VW == 1) {
        v[0] = p[idx];
    } else {
#pragma unroll
        for (int i = 0; i < VW; i += 4) {
            const f32x4 q = *reinterpret_cast<const f32x4*>(p + idx + i);
            v[i] = q.x;
            v[i + 1] = q.y;
            v[i + 2] = q.z;
            v[i + 3] = q.w;
        }
    }
}

// Factor of the upstream gradient under the ReLU: 0 where the pre-ReLU output is not
// positive, else 1.  A multiplier rather than a select of dy: hipcc (ROCm 7.2) turned
// `relu && !(pre > 0) ? 0 : dy` into a store of 0 for every lane of the ReLU branch.
__device__ __forceinline__ float ln_keep(int relu, float pre) { return (relu == 0 || pre > 0.f) ? 1.f : 0.f; }

// Sum of (a, b) over the workgroup's W waves: butterfly within each wave, then the W
// wave totals in wave order.  Every thread gets the result.
template <int W = kLnThreads / 64>
__device__ __forceinline__ void ln_sum2(float& a, float& b, float* red) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        a += __shfl_xor(a, o);
        b += __shfl_xor(b, o);
    }
    const int w = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) {
        red[2 * w] = a;
        red[2 * w + 1] = b;
    }
    __syncthreads();
    a = 0.f;
    b = 0.f;
#pragma unroll
    for (int i = 0; i < W; i++) {
        a += red[2 * i];
        b += red[2 * i + 1];
    }
    __syncthreads();   // red is reused by the next call
}

// ---------------------------------------------------------------------------------
// axis 1, forward: one row per workgroup, element e = (i*256 + t)*VW + k in registers
template <int DT, int VW, int NV>
__global__ __launch_bounds__(kLnThreads) void ln_fwd_rows(LnArgs a) {
    __shared__ float red[8];
    const int t = threadIdx.x;
    const int C = (int)a.C;
    const int64_t row = (int64_t)blockIdx.x * C;
    float v[NV][VW];
    float s = 0.f, unused = 0.f;
#pragma unroll
    for (int i = 0; i < NV; i++) {
        const int e = (i * kLnThreads + t) * VW;
        if (e < C) {
            ln_load<DT, VW>(a.x, row + e, v[i]);
#pragma unroll
            for (int k = 0; k < VW; k++) s += v[i][k];
        } else {
#pragma unroll
            for (int k = 0; k < VW; k++) v[i][k] = 0.f;
        }
    }
    ln_sum2(s, unused, red);
    const float mean = s / (float)C;
    float q = 0.f;
#pragma unroll
    for (int i = 0; i < NV; i++) {
        const int e = (i * kLnThreads + t) * VW;
        if (e < C) {
#pragma unroll
            for (int k = 0; k < VW; k++) {
                const float d = v[i][k] - mean;
                q += d * d;
            }
        }
    }
    unused = 0.f;
    ln_sum2(q, unused, red);
    const float rstd = 1.0f / sqrtf(q / (float)C + a.eps);
#pragma unroll
    for (int i = 0; i < NV; i++) {
        const int e = (i * kLnThreads + t) * VW;
        if (e < C) {
            float g[VW], b[VW], y[VW];
            ln_param<VW>(a.g, e, g);
            ln_param<VW>(a.b, e, b);
#pragma unroll
            for (int k = 0; k < VW; k++) {
                y[k] = (v[i][k] - mean) * rstd * g[k] + b[k];
                if (a.relu) y[k] = fmaxf(y[k], 0.f);
            }
            ln_store<DT, VW>(a.y, row + e, y);
        }
    }
    if (t == 0 && a.mean) {
        a.mean[blockIdx.x] = mean;
        a.rstd[blockIdx.x] = rstd;
    }
}

// axis 1, gradient: rows [blockIdx.x*RPB, +RPB); per-run partial dg, db to the
// workspace.  The next two rows' x and dy are in flight while the current row is
// reduced (always issued: past the run's end a row re-reads itself; lanes past C read
// element 0, unused).
constexpr int kLnBwdThreads = 512;   // 8 waves: two per SIMD hide each other's latency
template <int DT, int VW, int NV>
__global__ __launch_bounds__(kLnBwdThreads) void ln_bwd_rows(LnArgs a) {
    constexpr int kLnThreads = kLnBwdThreads;   // element e = (i*512 + t)*VW + k
    __shared__ float red[16];
    const int t = threadIdx.x;
    const int C = (int)a.C;
    const int64_t r0 = (int64_t)blockIdx.x * a.rpb;
    const int64_t r1 = r0 + a.rpb < a.N ? r0 + a.rpb : a.N;
    float pg[NV][VW], pb[NV][VW], g[NV][VW], b[NV][VW];
    int el[NV];
#pragma unroll
    for (int i = 0; i < NV; i++) {
        const int e = (i * kLnThreads + t) * VW;
        el[i] = e < C ? e : 0;
        ln_param<VW>(a.g, el[i], g[i]);
        ln_param<VW>(a.b, el[i], b[i]);
#pragma unroll
        for (int k = 0; k < VW; k++) pg[i][k] = pb[i][k] = 0.f;
    }
    // two rows ahead in registers (slots A = row n+1, B = row n+2 when the loop body
    // starts), for rows of up to 16 values per thread; longer rows load in the body
    constexpr bool PF = NV * VW <= 16;
    // (the row's mean and rstd travel with it: a load issued after the prefetch and
    // consumed at once would make the wave wait for the prefetch too)
    float xa[NV][VW], da[NV][VW], xb[NV][VW], db_[NV][VW];
    float ma = 0.f, ra = 0.f, mb = 0.f, rb = 0.f;
    auto load_row = [&](int64_t n, float (*xo)[VW], float (*dout)[VW], float& mo, float& ro) {
        mo = a.mean[n];
        ro = a.rstd[n];
#pragma unroll
        for (int i = 0; i < NV; i++) {
            ln_load<DT, VW>(a.x, n * C + el[i], xo[i]);
            ln_load<DT, VW>(a.dy, n * C + el[i], dout[i]);
        }
    };
    if constexpr (PF) {
        load_row(r0, xa, da, ma, ra);
        load_row(r0 + 1 < r1 ? r0 + 1 : r0, xb, db_, mb, rb);
    }
    for (int64_t n = r0; n < r1; n++) {   // workgroup-uniform
        float x[NV][VW], dy[NV][VW];
        float mean, rstd;
        if constexpr (PF) {
#pragma unroll
            for (int i = 0; i < NV; i++)
#pragma unroll
                for (int k = 0; k < VW; k++) {
                    x[i][k] = xa[i][k];
                    dy[i][k] = da[i][k];
                    xa[i][k] = xb[i][k];
                    da[i][k] = db_[i][k];
                }
            mean = ma;
            rstd = ra;
            ma = mb;
            ra = rb;
            load_row(n + 2 < r1 ? n + 2 : n, xb, db_, mb, rb);
        } else {
            load_row(n, x, dy, mean, rstd);
        }
        // xhat and dyr*g are recomputed for dx below rather than kept (registers)
        float s1 = 0.f, s2 = 0.f;
#pragma unroll
        for (int i = 0; i < NV; i++) {
            const bool ok = (i * kLnThreads + t) * VW < C;
#pragma unroll
            for (int k = 0; k < VW; k++) {
                const float xhat = (x[i][k] - mean) * rstd;
                const float dyr = ok ? dy[i][k] * ln_keep(a.relu, xhat * g[i][k] + b[i][k]) : 0.f;
                const float dh = dyr * g[i][k];
                pg[i][k] += dyr * xhat;
                pb[i][k] += dyr;
                s1 += dh;
                s2 += dh * xhat;
            }
        }
        ln_sum2<kLnBwdThreads / 64>(s1, s2, red);
        const float m1 = s1 / (float)C, m2 = s2 / (float)C;
#pragma unroll
        for (int i = 0; i < NV; i++) {
            const int e = (i * kLnThreads + t) * VW;
            if (e < C) {
                float dx[VW];
#pragma unroll
                for (int k = 0; k < VW; k++) {
                    const float xhat = (x[i][k] - mean) * rstd;
                    const float dh = dy[i][k] * ln_keep(a.relu, xhat * g[i][k] + b[i][k]) * g[i][k];
                    dx[k] = rstd * (dh - m1 - xhat * m2);
                }
                ln_store<DT, VW>(a.dx, n * C + e, dx);
            }
        }
    }
    float* wg = a.ws + (int64_t)blockIdx.x * C;
    float* wb = a.ws + (int64_t)a.nparts * C + (int64_t)blockIdx.x * C;
#pragma unroll
    for (int i = 0; i < NV; i++) {
        const int e = (i * kLnThreads + t) * VW;
        if (e < C) {
#pragma unroll
            for (int k = 0; k < VW; k++) {
                wg[e + k] = pg[i][k];
                wb[e + k] = pb[i][k];
            }
        }
    }
}

// dg[c], db[c] from the nparts partials of the workspace: a workgroup takes 32
// features; lane l of 8 adds the parts p = l, l + 8, ... in order, then the 8 lane sums
// are added in lane order (a fixed order: deterministic).
constexpr int kLnRedCols = 32;
__global__ __launch_bounds__(kLnThreads) void ln_param_reduce(LnArgs a, int64_t len, const float* wg, const float* wb) {
    __shared__ float red[2][8][kLnRedCols];
    const int cl = threadIdx.x % kLnRedCols, pl = threadIdx.x / kLnRedCols;
    const int64_t c = (int64_t)blockIdx.x * kLnRedCols + cl;
    const bool ok = c < len;
    const int64_t cc = ok ? c : 0;
    float sg = 0.f, sb = 0.f;
    int p = pl;
    for (; p + 24 < a.nparts; p += 32) {   // four parts in flight per lane
        const float g0 = wg[(int64_t)p * len + cc], g1 = wg[(int64_t)(p + 8) * len + cc];
        const float g2 = wg[(int64_t)(p + 16) * len + cc], g3 = wg[(int64_t)(p + 24) * len + cc];
        const float b0 = wb[(int64_t)p * len + cc], b1 = wb[(int64_t)(p + 8) * len + cc];
        const float b2 = wb[(int64_t)(p + 16) * len + cc], b3 = wb[(int64_t)(p + 24) * len + cc];
        sg = (((sg + g0) + g1) + g2) + g3;
        sb = (((sb + b0) + b1) + b2) + b3;
    }
    for (; p < a.nparts; p += 8) {
        sg += wg[(int64_t)p * len + cc];
        sb += wb[(int64_t)p * len + cc];
    }
    red[0][pl][cl] = sg;
    red[1][pl][cl] = sb;
    __syncthreads();
    if (pl == 0 && ok) {
        float tg = 0.f, tb = 0.f;
#pragma unroll
        for (int l = 0; l < 8; l++) {
            tg += red[0][l][cl];
            tb += red[1][l][cl];
        }
        a.dg[c] = tg;
        a.db[c] = tb;
    }
}

// axis 0: the chunks' partial statistics of each column merged once into chunk 0's
// slot of the workspace.  A workgroup takes 32 columns; lane l of 8 merges chunks
// l, l + 8, ... in order, then the 8 lane results are merged in lane order (a fixed
// order: deterministic).  Forward: (mean, rstd) from per-chunk (mean, M2) by the
// pairwise update of count, mean and squared deviations; gradient: (mean of dyr*g,
// mean of dyr*g*xhat) from plain per-chunk sums.
struct LnStat {
    double n;
    float mean, m2;
};
__device__ __forceinline__ void ln_stat_add(LnStat& a, double nb, float mb, float m2b) {
    const double tot = a.n + nb;
    if (tot == 0.0) return;
    const float d = mb - a.mean;
    a.mean += d * (float)(nb / tot);
    a.m2 += m2b + d * d * (float)(a.n * nb / tot);
    a.n = tot;
}
__global__ __launch_bounds__(kLnThreads) void ln_cols_merge(LnArgs a, int grad) {
    __shared__ float red[3][8][32];
    const int cl = threadIdx.x & 31, l = threadIdx.x >> 5;
    const int64_t n = (int64_t)blockIdx.x * 32 + cl;
    const bool ok = n < a.N;
    const int64_t nn = ok ? n : 0;
    float2* w = reinterpret_cast<float2*>(a.ws);
    LnStat st{0.0, 0.f, 0.f};
    float s1 = 0.f, s2 = 0.f;
    for (int c = l; c < a.nchunks; c += 8) {
        const float2 v = w[(int64_t)c * a.N + nn];
        if (grad) {
            s1 += v.x;
            s2 += v.y;
        } else {
            const int64_t left = a.C - (int64_t)c * kLnChunk;
            ln_stat_add(st, (double)(left < kLnChunk ? left : kLnChunk), v.x, v.y);
        }
    }
    red[0][l][cl] = grad ? s1 : st.mean;
    red[1][l][cl] = grad ? s2 : st.m2;
    red[2][l][cl] = (float)st.n;   // chunk rows: exact in float (at most C)
    __syncthreads();   // every chunk's slot has been read: slot 0 may be overwritten
    if (l != 0 || !ok) return;
    if (grad) {
        float t1 = 0.f, t2 = 0.f;
        for (int k = 0; k < 8; k++) {
            t1 += red[0][k][cl];
            t2 += red[1][k][cl];
        }
        w[n] = make_float2(t1 / (float)a.C, t2 / (float)a.C);
        return;
    }
    LnStat tot{0.0, 0.f, 0.f};
    for (int k = 0; k < 8; k++) ln_stat_add(tot, (double)red[2][k][cl], red[0][k][cl], red[1][k][cl]);
    const float rstd = 1.0f / sqrtf(tot.m2 / (float)a.C + a.eps);
    w[n] = make_float2(tot.mean, rstd);
    if (a.mean) {
        a.mean[n] = tot.mean;
        a.rstd[n] = rstd;
    }
}

// ---------------------------------------------------------------------------------
// axis 0: thread t owns column vector cv = t % 32 (columns n0 .. n0+VW-1) and row lane
// rl = t / 32 (rows chunk*128 + rl + 8j)
struct LnCols {
    int64_t n0, r0;
    int cv, rl, nrows;
    bool colok;
};
template <int VW> __device__ __forceinline__ LnCols ln_cols(const LnArgs& a) {
    LnCols p;
    p.cv = threadIdx.x & 31;
    p.rl = threadIdx.x >> 5;
    p.n0 = ((int64_t)blockIdx.x * 32 + p.cv) * VW;
    p.r0 = (int64_t)blockIdx.y * kLnChunk;
    const int64_t left = a.C - p.r0;
    p.nrows = left < kLnChunk ? (int)left : kLnChunk;
    p.colok = p.n0 < a.N;   // VW > 1: N % VW == 0, so a vector is all in or all out
    return p;
}
// Sum of VW per-thread column values over the 8 row lanes, in lane order; every row
// lane gets the result.
template <int VW> __device__ __forceinline__ void ln_sum_lanes(float* v, float* red /* [8][32][VW] */) {
    const int cv = threadIdx.x & 31, rl = threadIdx.x >> 5;
#pragma unroll
    for (int k = 0; k < VW; k++) red[(rl * 32 + cv) * VW + k] = v[k];
    __syncthreads();
#pragma unroll
    for (int k = 0; k < VW; k++) {
        float s = 0.f;
#pragma unroll
        for (int l = 0; l < 8; l++) s += red[(l * 32 + cv) * VW + k];
        v[k] = s;
    }
    __syncthreads();
}

// Rows rl + 8j, j < RJ, of this thread's chunk: every load is issued, rows past the
// chunk's end re-read its first row and are masked out of every use.
constexpr int kLnRJ = kLnChunk / 8;
template <int DT, int VW, int J>
__device__ __forceinline__ void ln_load_rows(const void* base, const LnCols& p, int64_t N, int j0, float (*v)[VW]) {
#pragma unroll
    for (int j = 0; j < J; j++) {
        const int r = p.rl + 8 * (j0 + j);
        ln_load<DT, VW>(base, (p.r0 + (r < p.nrows ? r : 0)) * N + p.n0, v[j]);
    }
}

// forward pass 1: per chunk and column, the chunk's mean and sum of squared deviations
// (the chunk's rows stay in registers between the two sums)
template <int DT, int VW>
__global__ __launch_bounds__(kLnThreads) void ln_fwd_cols_stats(LnArgs a) {
    __shared__ float red[8 * 32 * VW];
    LnCols p = ln_cols<VW>(a);
    if (!p.colok) p.n0 = 0;   // loads stay in bounds; results unused
    float x[kLnRJ][VW];
    ln_load_rows<DT, VW, kLnRJ>(a.x, p, a.N, 0, x);
    float s[VW], q[VW], m[VW];
#pragma unroll
    for (int k = 0; k < VW; k++) s[k] = q[k] = 0.f;
#pragma unroll
    for (int j = 0; j < kLnRJ; j++)
        if (p.rl + 8 * j < p.nrows)
#pragma unroll
            for (int k = 0; k < VW; k++) s[k] += x[j][k];
    ln_sum_lanes<VW>(s, red);
#pragma unroll
    for (int k = 0; k < VW; k++) m[k] = s[k] / (float)p.nrows;
#pragma unroll
    for (int j = 0; j < kLnRJ; j++)
        if (p.rl + 8 * j < p.nrows)
#pragma unroll
            for (int k = 0; k < VW; k++) {
                const float d = x[j][k] - m[k];
                q[k] += d * d;
            }
    ln_sum_lanes<VW>(q, red);
    if (p.rl == 0 && p.colok) {
        float2* w = reinterpret_cast<float2*>(a.ws) + (int64_t)blockIdx.y * a.N + p.n0;
#pragma unroll
        for (int k = 0; k < VW; k++) w[k] = make_float2(m[k], q[k]);
    }
}

// forward pass 3 (after ln_cols_merge): normalise this chunk
template <int DT, int VW>
__global__ __launch_bounds__(kLnThreads) void ln_fwd_cols_norm(LnArgs a) {
    const LnCols p = ln_cols<VW>(a);
    if (!p.colok) return;   // no barrier below
    float x[kLnRJ][VW];
    ln_load_rows<DT, VW, kLnRJ>(a.x, p, a.N, 0, x);
    float mean[VW], rstd[VW];
    const float2* w = reinterpret_cast<const float2*>(a.ws);   // merged: (mean, rstd)
#pragma unroll
    for (int k = 0; k < VW; k++) {
        const float2 st = w[p.n0 + k];
        mean[k] = st.x;
        rstd[k] = st.y;
    }
#pragma unroll
    for (int j = 0; j < kLnRJ; j++) {
        const int r = p.rl + 8 * j;
        if (r < p.nrows) {
            const int64_t c = p.r0 + r;
            const float g = a.g[c], b = a.b[c];
            float y[VW];
#pragma unroll
            for (int k = 0; k < VW; k++) {
                y[k] = (x[j][k] - mean[k]) * rstd[k] * g + b;
                if (a.relu) y[k] = fmaxf(y[k], 0.f);
            }
            ln_store<DT, VW>(a.y, c * a.N + p.n0, y);
        }
    }
}

// gradient pass 1: per chunk and column the sums of dyr*g and dyr*g*xhat (workspace
// part 1); per row and column block the sums of dyr*xhat and dyr (part 2).  The chunk
// is taken in two halves of 8 rows per thread, each half's loads issued together.
template <int DT, int VW>
__global__ __launch_bounds__(kLnThreads) void ln_bwd_cols_stats(LnArgs a) {
    __shared__ float red[8 * 32 * VW];
    LnCols p = ln_cols<VW>(a);
    const bool colok = p.colok;
    if (!colok) p.n0 = 0;   // loads stay in bounds; contributions masked
    float s1[VW], s2[VW], mean[VW], rstd[VW];
#pragma unroll
    for (int k = 0; k < VW; k++) {
        s1[k] = s2[k] = 0.f;
        mean[k] = a.mean[p.n0 + k];
        rstd[k] = a.rstd[p.n0 + k];
    }
    float* pg = a.ws + (int64_t)a.nchunks * a.N * 2 + (int64_t)blockIdx.x * a.C;
    float* pb = pg + (int64_t)a.nparts * a.C;
    constexpr int H = kLnRJ / 2;
#pragma unroll
    for (int h = 0; h < kLnRJ; h += H) {
        float x[H][VW], dy[H][VW];
        ln_load_rows<DT, VW, H>(a.x, p, a.N, h, x);
        ln_load_rows<DT, VW, H>(a.dy, p, a.N, h, dy);
#pragma unroll
        for (int j = 0; j < H; j++) {
            const int r = p.rl + 8 * (h + j);
            const bool rok = r < p.nrows;
            const int64_t c = p.r0 + (rok ? r : 0);
            const float g = a.g[c], b = a.b[c];
            float rg = 0.f, rb = 0.f;
            if (colok && rok) {
#pragma unroll
                for (int k = 0; k < VW; k++) {
                    const float xhat = (x[j][k] - mean[k]) * rstd[k];
                    const float dyr = dy[j][k] * ln_keep(a.relu, xhat * g + b);
                    const float dh = dyr * g;
                    s1[k] += dh;
                    s2[k] += dh * xhat;
                    rg += dyr * xhat;
                    rb += dyr;
                }
            }
            // the row's sums over this block's columns: the 32 column lanes of a half wave
#pragma unroll
            for (int o = 16; o > 0; o >>= 1) {
                rg += __shfl_xor(rg, o);
                rb += __shfl_xor(rb, o);
            }
            if (p.cv == 0 && rok) {
                pg[c] = rg;
                pb[c] = rb;
            }
        }
    }
    ln_sum_lanes<VW>(s1, red);
    ln_sum_lanes<VW>(s2, red);
    if (p.rl == 0 && colok) {
        float2* w = reinterpret_cast<float2*>(a.ws) + (int64_t)blockIdx.y * a.N + p.n0;
#pragma unroll
        for (int k = 0; k < VW; k++) w[k] = make_float2(s1[k], s2[k]);
    }
}

// gradient pass 3 (after ln_cols_merge): dx of this chunk
template <int DT, int VW>
__global__ __launch_bounds__(kLnThreads) void ln_bwd_cols_dx(LnArgs a) {
    const LnCols p = ln_cols<VW>(a);
    if (!p.colok) return;
    constexpr int H = kLnRJ / 2;
    float x[H][VW], dy[H][VW];
    ln_load_rows<DT, VW, H>(a.x, p, a.N, 0, x);
    ln_load_rows<DT, VW, H>(a.dy, p, a.N, 0, dy);
    float m1[VW], m2[VW], mean[VW], rstd[VW];
    const float2* w = reinterpret_cast<const float2*>(a.ws);   // merged column means
#pragma unroll
    for (int k = 0; k < VW; k++) {
        const float2 st = w[p.n0 + k];
        m1[k] = st.x;
        m2[k] = st.y;
        mean[k] = a.mean[p.n0 + k];
        rstd[k] = a.rstd[p.n0 + k];
    }
#pragma unroll
    for (int h = 0; h < kLnRJ; h += H) {
        if (h > 0) {
            ln_load_rows<DT, VW, H>(a.x, p, a.N, h, x);
            ln_load_rows<DT, VW, H>(a.dy, p, a.N, h, dy);
        }
#pragma unroll
        for (int j = 0; j < H; j++) {
            const int r = p.rl + 8 * (h + j);
            if (r < p.nrows) {
                const int64_t c = p.r0 + r;
                const float g = a.g[c], b = a.b[c];
                float dx[VW];
#pragma unroll
                for (int k = 0; k < VW; k++) {
                    const float xhat = (x[j][k] - mean[k]) * rstd[k];
                    const float dyr = dy[j][k] * ln_keep(a.relu, xhat * g + b);
                    dx[k] = rstd[k] * (dyr * g - m1[k] - xhat * m2[k]);
                }
                ln_store<DT, VW>(a.dx, c * a.N + p.n0, dx);
            }
        }
    }
}

// ---------------------------------------------------------------------------------
// host side
namespace {

template <int DT, int VW>
hipError_t ln_rows_nv(LnArgs a, int nv, bool grad, hipStream_t st) {
    const dim3 blk(kLnThreads);
#define BSMM_LN_ROWS(NVV)                                                                         \
    case NVV:                                                                                     \
        if constexpr (VW == 1 || NVV <= 8) { /* 16-byte loads: at most 8 per thread */           \
            if (!grad)                                                                            \
                return launch_ev(ln_fwd_rows<DT, VW, NVV>, dim3((unsigned)a.N), blk, st, a.e0, a.e1, a); \
            hipError_t e = launch_ev(ln_bwd_rows<DT, VW, NVV>, dim3((unsigned)a.nparts), dim3(kLnBwdThreads), st, \
                                     a.e0, nullptr, a);                                          \
            if (e != hipSuccess) return e;                                                        \
            return launch_ev(ln_param_reduce, dim3((unsigned)((a.C + kLnRedCols - 1) / kLnRedCols)), \
                             blk, st, nullptr, a.e1, a, a.C, (const float*)a.ws,                  \
                             (const float*)(a.ws + (int64_t)a.nparts * a.C));                     \
        }                                                                                         \
        return hipErrorInvalidValue;
    switch (nv) {
        BSMM_LN_ROWS(1)
        BSMM_LN_ROWS(2)
        BSMM_LN_ROWS(4)
        BSMM_LN_ROWS(8)
        BSMM_LN_ROWS(16)
        BSMM_LN_ROWS(32)
    }
#undef BSMM_LN_ROWS
    return hipErrorInvalidValue;
}

template <int DT, int VW>
hipError_t ln_cols_launch(LnArgs a, bool grad, hipStream_t st) {
    const dim3 grid((unsigned)((a.N + 32 * VW - 1) / (32 * VW)), (unsigned)a.nchunks), blk(kLnThreads);
    const dim3 mgrid((unsigned)((a.N + 31) / 32));
    hipError_t e = grad ? launch_ev(ln_bwd_cols_stats<DT, VW>, grid, blk, st, a.e0, nullptr, a)
                        : launch_ev(ln_fwd_cols_stats<DT, VW>, grid, blk, st, a.e0, nullptr, a);
    if (e != hipSuccess) return e;
    e = launch_ev(ln_cols_merge, mgrid, blk, st, nullptr, nullptr, a, grad ? 1 : 0);
    if (e != hipSuccess) return e;
    if (!grad) return launch_ev(ln_fwd_cols_norm<DT, VW>, grid, blk, st, nullptr, a.e1, a);
    e = launch_ev(ln_bwd_cols_dx<DT, VW>, grid, blk, st, nullptr, nullptr, a);
    if (e != hipSuccess) return e;
    const float* pg = a.ws + (int64_t)a.nchunks * a.N * 2;
    return launch_ev(ln_param_reduce, dim3((unsigned)((a.C + kLnRedCols - 1) / kLnRedCols)), blk, st, nullptr,
                     a.e1, a, a.C, pg, pg + (int64_t)a.nparts * a.C);
}

template <int DT>
hipError_t ln_dt(const LnArgs& a, bool grad, hipStream_t st) {
    constexpr int VEC = Elt<DT>::VEC;
    if (a.axis == 1) {
        if (a.vw > 1) return ln_rows_nv<DT, VEC>(a, a.nv, grad, st);
        return ln_rows_nv<DT, 1>(a, a.nv, grad, st);
    }
    if (a.vw > 1) return ln_cols_launch<DT, VEC>(a, grad, st);
    return ln_cols_launch<DT, 1>(a, grad, st);
}

}  // namespace

int ln_plan(LnArgs& a, bool grad, bool aligned) {
    const int vec = a.dt == BSMM_F32 ? 4 : 8;
    if (a.axis == 1) {
        a.vw = (aligned && a.C % vec == 0) ? vec : 1;
        const int64_t per = (int64_t)(grad ? kLnBwdThreads : kLnThreads) * a.vw;
        const int64_t need = (a.C + per - 1) / per;
        int nv = 1;
        while (nv < need) nv *= 2;
        if (nv > (a.vw > 1 ? 8 : 32)) return -1;   // row does not fit the registers
        a.nv = nv;
        a.rpb = (a.N + 255) / 256;
        a.nparts = grad ? (int)((a.N + a.rpb - 1) / a.rpb) : 0;
        a.nchunks = 0;
    } else {
        a.vw = (aligned && a.N % vec == 0) ? vec : 1;
        a.nv = 0;
        a.rpb = 0;
        a.nchunks = (int)((a.C + kLnChunk - 1) / kLnChunk);
        if (a.nchunks > 65535) return -1;   // grid y
        a.nparts = grad ? (int)((a.N + 32 * a.vw - 1) / (32 * a.vw)) : 0;
    }
    return 0;
}

size_t ln_workspace_bytes(int64_t N, int64_t C, int axis, bool grad) {
    // the largest any plan uses (axis 0: one-value loads give the most column blocks)
    if (N <= 0 || C <= 0) return 0;
    if (axis == 1) {
        const int64_t rpb = (N + 255) / 256, parts = (N + rpb - 1) / rpb;
        return grad ? (size_t)2 * parts * C * sizeof(float) : 0;
    }
    const int64_t chunks = (C + kLnChunk - 1) / kLnChunk, parts = (N + 31) / 32;
    size_t b = (size_t)chunks * N * 2 * sizeof(float);
    if (grad) b += (size_t)2 * parts * C * sizeof(float);
    return b;
}

hipError_t launch_ln_zero_params(float* dg, float* db, int64_t C, void* stream) {
    LnArgs a{};
    a.dg = dg;
    a.db = db;
    a.nparts = 0;
    return launch_ev(ln_param_reduce, dim3((unsigned)((C + kLnRedCols - 1) / kLnRedCols)), dim3(kLnThreads),
                     (hipStream_t)stream, nullptr, nullptr, a, C, (const float*)nullptr, (const float*)nullptr);
}

hipError_t launch_layer_norm(const LnArgs& a, bool grad, void* stream) {
    hipStream_t st = (hipStream_t)stream;
    switch (a.dt) {
    case BSMM_F32: return ln_dt<BSMM_F32>(a, grad, st);
    case BSMM_BF16: return ln_dt<BSMM_BF16>(a, grad, st);
    case BSMM_F16: return ln_dt<BSMM_F16>(a, grad, st);
    }
    return hipErrorInvalidValue;
}

}  // namespace bsmm
