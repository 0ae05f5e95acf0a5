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
// write of y); the gradient takes a run of rows per workgroup and leaves per-run
// partial dg/db in the workspace, added in run order by a second kernel.
// Axis 0: a workgroup owns 32 16-byte column vectors x a chunk of 128 rows, so every
// load is a coalesced row segment.  Column statistics are combined over the chunks
// (per-chunk mean and squared deviations, merged in chunk order) through the workspace.
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

// Sum of (a, b) over the 256 threads: butterfly within each wave, then the four wave
// totals in wave order.  Every thread gets the result.
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
    a = (red[0] + red[2]) + (red[4] + red[6]);
    b = (red[1] + red[3]) + (red[5] + red[7]);
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

// axis 1, gradient: rows [blockIdx.x*RPB, +RPB); per-run partial dg, db to the workspace
template <int DT, int VW, int NV>
__global__ __launch_bounds__(kLnThreads) void ln_bwd_rows(LnArgs a) {
    __shared__ float red[8];
    const int t = threadIdx.x;
    const int C = (int)a.C;
    const int64_t r0 = (int64_t)blockIdx.x * a.rpb;
    const int64_t r1 = r0 + a.rpb < a.N ? r0 + a.rpb : a.N;
    float pg[NV][VW], pb[NV][VW], g[NV][VW], b[NV][VW];
#pragma unroll
    for (int i = 0; i < NV; i++) {
        const int e = (i * kLnThreads + t) * VW;
#pragma unroll
        for (int k = 0; k < VW; k++) pg[i][k] = pb[i][k] = g[i][k] = b[i][k] = 0.f;
        if (e < C) {
            ln_param<VW>(a.g, e, g[i]);
            ln_param<VW>(a.b, e, b[i]);
        }
    }
    for (int64_t n = r0; n < r1; n++) {   // workgroup-uniform
        const int64_t row = n * C;
        const float mean = a.mean[n], rstd = a.rstd[n];
        float xh[NV][VW], dh[NV][VW];
        float s1 = 0.f, s2 = 0.f;
#pragma unroll
        for (int i = 0; i < NV; i++) {
            const int e = (i * kLnThreads + t) * VW;
#pragma unroll
            for (int k = 0; k < VW; k++) xh[i][k] = dh[i][k] = 0.f;
            if (e < C) {
                float x[VW], dy[VW];
                ln_load<DT, VW>(a.x, row + e, x);
                ln_load<DT, VW>(a.dy, row + e, dy);
#pragma unroll
                for (int k = 0; k < VW; k++) {
                    const float xhat = (x[k] - mean) * rstd;
                    const float dyr = dy[k] * ln_keep(a.relu, xhat * g[i][k] + b[i][k]);
                    pg[i][k] += dyr * xhat;
                    pb[i][k] += dyr;
                    xh[i][k] = xhat;
                    dh[i][k] = dyr * g[i][k];
                    s1 += dh[i][k];
                    s2 += dh[i][k] * xhat;
                }
            }
        }
        ln_sum2(s1, s2, red);
        const float m1 = s1 / (float)C, m2 = s2 / (float)C;
#pragma unroll
        for (int i = 0; i < NV; i++) {
            const int e = (i * kLnThreads + t) * VW;
            if (e < C) {
                float dx[VW];
#pragma unroll
                for (int k = 0; k < VW; k++) dx[k] = rstd * (dh[i][k] - m1 - xh[i][k] * m2);
                ln_store<DT, VW>(a.dx, row + e, dx);
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

// dg[c], db[c]: the nparts partials of the workspace added in part order
__global__ __launch_bounds__(kLnThreads) void ln_param_reduce(LnArgs a, int64_t len, const float* wg, const float* wb) {
    const int64_t c = (int64_t)blockIdx.x * kLnThreads + threadIdx.x;
    if (c >= len) return;
    float sg = 0.f, sb = 0.f;
    for (int p = 0; p < a.nparts; p++) {
        sg += wg[(int64_t)p * len + c];
        sb += wb[(int64_t)p * len + c];
    }
    a.dg[c] = sg;
    a.db[c] = sb;
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

// forward pass 1: per chunk and column, the chunk's mean and sum of squared deviations
template <int DT, int VW>
__global__ __launch_bounds__(kLnThreads) void ln_fwd_cols_stats(LnArgs a) {
    __shared__ float red[8 * 32 * VW];
    const LnCols p = ln_cols<VW>(a);
    float s[VW], q[VW];
#pragma unroll
    for (int k = 0; k < VW; k++) s[k] = q[k] = 0.f;
    if (p.colok)
        for (int r = p.rl; r < p.nrows; r += 8) {
            float x[VW];
            ln_load<DT, VW>(a.x, (p.r0 + r) * a.N + p.n0, x);
#pragma unroll
            for (int k = 0; k < VW; k++) s[k] += x[k];
        }
    ln_sum_lanes<VW>(s, red);
    float m[VW];
#pragma unroll
    for (int k = 0; k < VW; k++) m[k] = s[k] / (float)p.nrows;
    if (p.colok)
        for (int r = p.rl; r < p.nrows; r += 8) {   // second read of the chunk: from cache
            float x[VW];
            ln_load<DT, VW>(a.x, (p.r0 + r) * a.N + p.n0, x);
#pragma unroll
            for (int k = 0; k < VW; k++) {
                const float d = x[k] - m[k];
                q[k] += d * d;
            }
        }
    ln_sum_lanes<VW>(q, red);
    if (p.rl == 0 && p.colok) {
        float2* w = reinterpret_cast<float2*>(a.ws) + (int64_t)blockIdx.y * a.N + p.n0;
#pragma unroll
        for (int k = 0; k < VW; k++) w[k] = make_float2(m[k], q[k]);
    }
}

// forward pass 2: merge the chunks' statistics (chunk order), normalise this chunk
template <int DT, int VW>
__global__ __launch_bounds__(kLnThreads) void ln_fwd_cols_norm(LnArgs a) {
    const LnCols p = ln_cols<VW>(a);
    if (!p.colok) return;   // no barrier below
    float mean[VW], m2[VW];
    double cnt = 0.0;
#pragma unroll
    for (int k = 0; k < VW; k++) mean[k] = m2[k] = 0.f;
    const float2* w = reinterpret_cast<const float2*>(a.ws);
    for (int c = 0; c < a.nchunks; c++) {
        const int64_t left = a.C - (int64_t)c * kLnChunk;
        const double nb = (double)(left < kLnChunk ? left : kLnChunk);
        const double tot = cnt + nb;
        const float fa = (float)(nb / tot), fb = (float)(cnt * nb / tot);
#pragma unroll
        for (int k = 0; k < VW; k++) {
            const float2 st = w[(int64_t)c * a.N + p.n0 + k];
            const float d = st.x - mean[k];
            mean[k] += d * fa;
            m2[k] += st.y + d * d * fb;
        }
        cnt = tot;
    }
    float rstd[VW];
#pragma unroll
    for (int k = 0; k < VW; k++) rstd[k] = 1.0f / sqrtf(m2[k] / (float)a.C + a.eps);
    if (blockIdx.y == 0 && p.rl == 0 && a.mean) {
#pragma unroll
        for (int k = 0; k < VW; k++) {
            a.mean[p.n0 + k] = mean[k];
            a.rstd[p.n0 + k] = rstd[k];
        }
    }
    for (int r = p.rl; r < p.nrows; r += 8) {
        const int64_t c = p.r0 + r;
        const float g = a.g[c], b = a.b[c];
        float x[VW], y[VW];
        ln_load<DT, VW>(a.x, c * a.N + p.n0, x);
#pragma unroll
        for (int k = 0; k < VW; k++) {
            y[k] = (x[k] - mean[k]) * rstd[k] * g + b;
            if (a.relu) y[k] = fmaxf(y[k], 0.f);
        }
        ln_store<DT, VW>(a.y, c * a.N + p.n0, y);
    }
}

// gradient pass 1: per chunk and column the sums of dyr*g and dyr*g*xhat (workspace
// part 1); per row and column block the sums of dyr*xhat and dyr (part 2)
template <int DT, int VW>
__global__ __launch_bounds__(kLnThreads) void ln_bwd_cols_stats(LnArgs a) {
    __shared__ float red[8 * 32 * VW];
    const LnCols p = ln_cols<VW>(a);
    float s1[VW], s2[VW], mean[VW], rstd[VW];
#pragma unroll
    for (int k = 0; k < VW; k++) {
        s1[k] = s2[k] = 0.f;
        mean[k] = p.colok ? a.mean[p.n0 + k] : 0.f;
        rstd[k] = p.colok ? a.rstd[p.n0 + k] : 0.f;
    }
    float* pg = a.ws + (int64_t)a.nchunks * a.N * 2 + (int64_t)blockIdx.x * a.C;
    float* pb = pg + (int64_t)a.nparts * a.C;
    for (int r = p.rl; r < kLnChunk; r += 8) {   // uniform trip count: shuffles below
        const bool rok = r < p.nrows;
        const int64_t c = p.r0 + (rok ? r : 0);
        const float g = a.g[c], b = a.b[c];
        float rg = 0.f, rb = 0.f;
        if (p.colok && rok) {
            float x[VW], dy[VW];
            ln_load<DT, VW>(a.x, c * a.N + p.n0, x);
            ln_load<DT, VW>(a.dy, c * a.N + p.n0, dy);
#pragma unroll
            for (int k = 0; k < VW; k++) {
                const float xhat = (x[k] - mean[k]) * rstd[k];
                const float dyr = dy[k] * ln_keep(a.relu, xhat * g + b);
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
    ln_sum_lanes<VW>(s1, red);
    ln_sum_lanes<VW>(s2, red);
    if (p.rl == 0 && p.colok) {
        float2* w = reinterpret_cast<float2*>(a.ws) + (int64_t)blockIdx.y * a.N + p.n0;
#pragma unroll
        for (int k = 0; k < VW; k++) w[k] = make_float2(s1[k], s2[k]);
    }
}

// gradient pass 2: the chunks' column sums added in chunk order, then dx of this chunk
template <int DT, int VW>
__global__ __launch_bounds__(kLnThreads) void ln_bwd_cols_dx(LnArgs a) {
    const LnCols p = ln_cols<VW>(a);
    if (!p.colok) return;
    float m1[VW], m2[VW], mean[VW], rstd[VW];
#pragma unroll
    for (int k = 0; k < VW; k++) {
        m1[k] = m2[k] = 0.f;
        mean[k] = a.mean[p.n0 + k];
        rstd[k] = a.rstd[p.n0 + k];
    }
    const float2* w = reinterpret_cast<const float2*>(a.ws);
    for (int c = 0; c < a.nchunks; c++)
#pragma unroll
        for (int k = 0; k < VW; k++) {
            const float2 st = w[(int64_t)c * a.N + p.n0 + k];
            m1[k] += st.x;
            m2[k] += st.y;
        }
#pragma unroll
    for (int k = 0; k < VW; k++) {
        m1[k] /= (float)a.C;
        m2[k] /= (float)a.C;
    }
    for (int r = p.rl; r < p.nrows; r += 8) {
        const int64_t c = p.r0 + r;
        const float g = a.g[c], b = a.b[c];
        float x[VW], dy[VW], dx[VW];
        ln_load<DT, VW>(a.x, c * a.N + p.n0, x);
        ln_load<DT, VW>(a.dy, c * a.N + p.n0, dy);
#pragma unroll
        for (int k = 0; k < VW; k++) {
            const float xhat = (x[k] - mean[k]) * rstd[k];
            const float dyr = dy[k] * ln_keep(a.relu, xhat * g + b);
            dx[k] = rstd[k] * (dyr * g - m1[k] - xhat * m2[k]);
        }
        ln_store<DT, VW>(a.dx, c * a.N + p.n0, dx);
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
            hipError_t e = launch_ev(ln_bwd_rows<DT, VW, NVV>, dim3((unsigned)a.nparts), blk, st,   \
                                     a.e0, nullptr, a);                                          \
            if (e != hipSuccess) return e;                                                        \
            return launch_ev(ln_param_reduce, dim3((unsigned)((a.C + kLnThreads - 1) / kLnThreads)), \
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
    if (!grad) {
        hipError_t e = launch_ev(ln_fwd_cols_stats<DT, VW>, grid, blk, st, a.e0, nullptr, a);
        if (e != hipSuccess) return e;
        return launch_ev(ln_fwd_cols_norm<DT, VW>, grid, blk, st, nullptr, a.e1, a);
    }
    hipError_t e = launch_ev(ln_bwd_cols_stats<DT, VW>, grid, blk, st, a.e0, nullptr, a);
    if (e != hipSuccess) return e;
    e = launch_ev(ln_bwd_cols_dx<DT, VW>, grid, blk, st, nullptr, nullptr, a);
    if (e != hipSuccess) return e;
    const float* pg = a.ws + (int64_t)a.nchunks * a.N * 2;
    return launch_ev(ln_param_reduce, dim3((unsigned)((a.C + kLnThreads - 1) / kLnThreads)), blk, st, nullptr,
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
        const int64_t per = (int64_t)kLnThreads * a.vw;
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
    return launch_ev(ln_param_reduce, dim3((unsigned)((C + kLnThreads - 1) / kLnThreads)), dim3(kLnThreads),
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
