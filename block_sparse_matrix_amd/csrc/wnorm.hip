// Weight normalisation of the stored blocks per output feature, and its gradient
// (kiteco/blocksparse README, "API Documentation" › blocksparse.matmul ›
// BlocksparseMatMul.l2_normalize(W, gain=None, epsilon=1e-6, dtype)).
//
// Output feature o = k*b + j is column j of the blocks in block column k:
//   n[o]  = sqrt(max(sum over those blocks and rows i of W^2, epsilon)),
//   out   = W * g[o] / n[o]                       (g = 1 without a gain),
// and for an upstream dOut, with s[o] = the column's sum of dOut * W:
//   dW    = g[o]/n[o] * dOut - [sum of squares > epsilon] * g[o]*s[o]/n[o]^3 * W,
//   dg[o] = s[o] / n[o].
// A workgroup owns one block column and walks its block list (the fprop column list
// of the layout tables) twice in 16-byte vectors: the column sums (fp32, a fixed
// order: deterministic), then the elementwise pass, whose re-read hits L2.
// Bound: HBM (|W| read, |out| written; |dOut| + |W| read, |dW| written).
#include "common.h"

namespace bsmm {

constexpr int kWnThreads = 1024;   // 16 waves: a block column's loads all in flight

// VW consecutive values of storage dtype DT at element idx (VW = 4 or 8; 8- or 16-byte
// aligned), widened to float
template <int DT, int VW> __device__ __forceinline__ void wn_loadv(const void* base, int64_t idx, float* v) {
    if constexpr (DT == BSMM_F32) {
#pragma unroll
        for (int h = 0; h < VW; h += 4) {
            const f32x4 q = *reinterpret_cast<const f32x4*>((const float*)base + idx + h);
            v[h] = q.x;
            v[h + 1] = q.y;
            v[h + 2] = q.z;
            v[h + 3] = q.w;
        }
    } else {
        uint32_t w[VW / 2];
        if constexpr (VW == 8) {
            const u32x4 q = *reinterpret_cast<const u32x4*>((const uint16_t*)base + idx);
            w[0] = q.x; w[1] = q.y; w[2] = q.z; w[3] = q.w;
        } else {
            const u32x2 q = *reinterpret_cast<const u32x2*>((const uint16_t*)base + idx);
            w[0] = q.x; w[1] = q.y;
        }
#pragma unroll
        for (int i = 0; i < VW / 2; i++) {
            if constexpr (DT == BSMM_BF16) {
                v[2 * i] = __uint_as_float(w[i] << 16);
                v[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
            } else {
                v[2 * i] = (float)__builtin_bit_cast(_Float16, (uint16_t)(w[i] & 0xffffu));
                v[2 * i + 1] = (float)__builtin_bit_cast(_Float16, (uint16_t)(w[i] >> 16));
            }
        }
    }
}
template <int DT, int VW> __device__ __forceinline__ void wn_storev(void* base, int64_t idx, const float* v) {
    if constexpr (DT == BSMM_F32) {
#pragma unroll
        for (int h = 0; h < VW; h += 4)
            *reinterpret_cast<f32x4*>((float*)base + idx + h) = f32x4{v[h], v[h + 1], v[h + 2], v[h + 3]};
    } else {
        uint32_t w[VW / 2];
#pragma unroll
        for (int i = 0; i < VW / 2; i++) w[i] = to_storage16<DT>(v[2 * i]) | (to_storage16<DT>(v[2 * i + 1]) << 16);
        if constexpr (VW == 8)
            *reinterpret_cast<u32x4*>((uint16_t*)base + idx) = u32x4{w[0], w[1], w[2], w[3]};
        else
            *reinterpret_cast<u32x2*>((uint16_t*)base + idx) = u32x2{w[0], w[1]};
    }
}

// Work map: a thread owns one 16-byte vector of the weights' storage (VW values of one
// block row) per block; the workgroup covers P blocks of the list side by side, walked
// U at a time so that U loads per thread are in flight.  Thread t: block slot t / VB,
// row (t % VB) / VR, columns (t % VR)*VW .. +VW-1.
template <int B, int DTI> struct WnMap {
    static constexpr int VW = DTI == BSMM_F32 ? 4 : 8;
    static constexpr int VR = B / VW;                 // vectors per block row (>= 1)
    static constexpr int VB = B * VR;                 // vectors per block
    static constexpr int P = kWnThreads / VB;         // blocks side by side (>= 1)
    static constexpr int U = 8;
    static_assert(B % VW == 0 && kWnThreads % VB == 0, "work map");
};

// Column sums of two per-thread VW-vectors over the threads of the same column vector
// (threads t, t + VR, t + 2 VR, ...): a halving tree over the thread index (fixed
// order: deterministic); thread t < B gets column t's sums.
template <int B, int VW, int VR>
__device__ __forceinline__ void wn_colsum(const float* a, const float* b, float* ra, float* rb, float& oa, float& ob) {
    const int t = threadIdx.x;
#pragma unroll
    for (int k = 0; k < VW; k++) {
        ra[t * VW + k] = a[k];
        rb[t * VW + k] = b[k];
    }
    __syncthreads();
#pragma unroll
    for (int half = kWnThreads / 2; half >= VR; half >>= 1) {
        if (t < half)
#pragma unroll
            for (int k = 0; k < VW; k++) {
                ra[t * VW + k] += ra[(t + half) * VW + k];
                rb[t * VW + k] += rb[(t + half) * VW + k];
            }
        __syncthreads();
    }
    oa = ob = 0.f;
    if (t < B) {
        oa = ra[t];   // thread cv = t / VW's value k = t % VW: index cv*VW + k = t
        ob = rb[t];
    }
}

template <int B, int DTI, int DTO>
__global__ __launch_bounds__(kWnThreads) void wn_fwd(WnArgs a) {
    using Map = WnMap<B, DTI>;
    constexpr int VW = Map::VW, VR = Map::VR, VB = Map::VB, P = Map::P, U = Map::U;
    __shared__ float ra[kWnThreads * VW], rb[kWnThreads * VW], scale[B];
    const int k = blockIdx.x, t = threadIdx.x;
    const int beg = a.colptr[k], end = a.colptr[k + 1];
    const int slot = t / VB, e0 = (t % VB) * VW;   // element offset inside a block
    float ss[VW], zero[VW];
#pragma unroll
    for (int i = 0; i < VW; i++) ss[i] = zero[i] = 0.f;
    for (int q0 = beg + slot; q0 < end; q0 += P * U) {
        float v[U][VW];
#pragma unroll
        for (int uu = 0; uu < U; uu++) {   // loads first; blocks past the end read block q0
            const int q = q0 + P * uu;
            wn_loadv<DTI, VW>(a.w, (int64_t)a.colent[2 * (q < end ? q : q0) + 1] * B * B + e0, v[uu]);
        }
#pragma unroll
        for (int uu = 0; uu < U; uu++)
            if (q0 + P * uu < end)
#pragma unroll
                for (int i = 0; i < VW; i++) ss[i] += v[uu][i] * v[uu][i];
    }
    float s, unused;
    wn_colsum<B, VW, VR>(ss, zero, ra, rb, s, unused);
    if (t < B) {
        const int o = k * B + t;
        const float n = sqrtf(fmaxf(s, a.eps));
        if (a.norms) a.norms[o] = n;
        scale[t] = (a.gain ? a.gain[o] : 1.0f) / n;
    }
    __syncthreads();
    float sc[VW];
#pragma unroll
    for (int i = 0; i < VW; i++) sc[i] = scale[(e0 + i) % B];
    for (int q0 = beg + slot; q0 < end; q0 += P * U) {   // U loads in flight, then U stores
        float v[U][VW];
        int64_t idx[U];
#pragma unroll
        for (int uu = 0; uu < U; uu++) {
            const int q = q0 + P * uu;
            idx[uu] = (int64_t)a.colent[2 * (q < end ? q : q0) + 1] * B * B + e0;
            wn_loadv<DTI, VW>(a.w, idx[uu], v[uu]);
        }
#pragma unroll
        for (int uu = 0; uu < U; uu++)
            if (q0 + P * uu < end) {
#pragma unroll
                for (int i = 0; i < VW; i++) v[uu][i] *= sc[i];
                wn_storev<DTO, VW>(a.out, idx[uu], v[uu]);
            }
    }
}

template <int B, int DTI, int DTD>
__global__ __launch_bounds__(kWnThreads) void wn_bwd(WnArgs a) {
    using Map = WnMap<B, DTI>;
    constexpr int VW = Map::VW, VR = Map::VR, VB = Map::VB, P = Map::P, U = Map::U;
    __shared__ float ra[kWnThreads * VW], rb[kWnThreads * VW], ca[B], cb[B];
    const int k = blockIdx.x, t = threadIdx.x;
    const int beg = a.colptr[k], end = a.colptr[k + 1];
    const int slot = t / VB, e0 = (t % VB) * VW;
    float ss[VW], sd[VW];
#pragma unroll
    for (int i = 0; i < VW; i++) ss[i] = sd[i] = 0.f;
    for (int q0 = beg + slot; q0 < end; q0 += P * (U / 2)) {   // two tensors: U/2 blocks
        float w[U / 2][VW], d[U / 2][VW];
#pragma unroll
        for (int uu = 0; uu < U / 2; uu++) {
            const int q = q0 + P * uu;
            const int64_t idx = (int64_t)a.colent[2 * (q < end ? q : q0) + 1] * B * B + e0;
            wn_loadv<DTI, VW>(a.w, idx, w[uu]);
            wn_loadv<DTD, VW>(a.dy, idx, d[uu]);
        }
#pragma unroll
        for (int uu = 0; uu < U / 2; uu++)
            if (q0 + P * uu < end)
#pragma unroll
                for (int i = 0; i < VW; i++) {
                    ss[i] += w[uu][i] * w[uu][i];
                    sd[i] += d[uu][i] * w[uu][i];
                }
    }
    float s2, s1;
    wn_colsum<B, VW, VR>(ss, sd, ra, rb, s2, s1);
    if (t < B) {
        const int o = k * B + t;
        const float n = sqrtf(fmaxf(s2, a.eps));
        const float g = a.gain ? a.gain[o] : 1.0f;
        ca[t] = g / n;
        cb[t] = s2 > a.eps ? g * s1 / (n * n * n) : 0.f;
        if (a.dgain) a.dgain[o] = s1 / n;
    }
    __syncthreads();
    float c1[VW], c2[VW];
#pragma unroll
    for (int i = 0; i < VW; i++) {
        c1[i] = ca[(e0 + i) % B];
        c2[i] = cb[(e0 + i) % B];
    }
    constexpr int U2 = U / 2;
    for (int q0 = beg + slot; q0 < end; q0 += P * U2) {
        float w[U2][VW], d[U2][VW];
        int64_t idx[U2];
#pragma unroll
        for (int uu = 0; uu < U2; uu++) {
            const int q = q0 + P * uu;
            idx[uu] = (int64_t)a.colent[2 * (q < end ? q : q0) + 1] * B * B + e0;
            wn_loadv<DTI, VW>(a.w, idx[uu], w[uu]);
            wn_loadv<DTD, VW>(a.dy, idx[uu], d[uu]);
        }
#pragma unroll
        for (int uu = 0; uu < U2; uu++)
            if (q0 + P * uu < end) {
                float r[VW];
#pragma unroll
                for (int i = 0; i < VW; i++) r[i] = c1[i] * d[uu][i] - c2[i] * w[uu][i];
                wn_storev<BSMM_F32, VW>(a.out, idx[uu], r);
            }
    }
}

namespace {
template <int B, int DTI>
hipError_t wn_b(const WnArgs& a, bool grad, hipStream_t st) {
    const dim3 grid((unsigned)a.S), blk(kWnThreads);
    const int d2 = grad ? a.dy_dt : a.out_dt;
#define BSMM_WN(D2)                                                                               \
    case D2:                                                                                      \
        return grad ? launch_ev(wn_bwd<B, DTI, D2>, grid, blk, st, a.e0, a.e1, a)                 \
                    : launch_ev(wn_fwd<B, DTI, D2>, grid, blk, st, a.e0, a.e1, a);
    switch (d2) {
        BSMM_WN(BSMM_F32)
        BSMM_WN(BSMM_BF16)
        BSMM_WN(BSMM_F16)
    }
#undef BSMM_WN
    return hipErrorInvalidValue;
}
template <int B>
hipError_t wn_dt(const WnArgs& a, bool grad, hipStream_t st) {
    switch (a.w_dt) {
    case BSMM_F32: return wn_b<B, BSMM_F32>(a, grad, st);
    case BSMM_BF16: return wn_b<B, BSMM_BF16>(a, grad, st);
    case BSMM_F16: return wn_b<B, BSMM_F16>(a, grad, st);
    }
    return hipErrorInvalidValue;
}
}  // namespace

hipError_t launch_l2_normalize(const WnArgs& a, bool grad, void* stream) {
    hipStream_t st = (hipStream_t)stream;
    switch (a.b) {
    case 8: return wn_dt<8>(a, grad, st);
    case 16: return wn_dt<16>(a, grad, st);
    case 32: return wn_dt<32>(a, grad, st);
    }
    return hipErrorInvalidValue;
}

}  // namespace bsmm
