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
// of the layout tables) in 16-byte vectors: the column sums (fp32: a butterfly inside
// each wave, then the waves in order — deterministic), then the elementwise pass.  The
// first round of blocks stays in registers between the two passes; only longer
// columns read the rest again (from L2).
// Bound: HBM (|W| read, |out| written; |dOut| + |W| read, |dW| written).
#include "common.h"

namespace bsmm {

constexpr int kWnThreads = 1024;   // 16 waves: a block column's loads all in flight

// VW floats stored as dtype DT at element idx (round to nearest even for 16-bit)
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

// Raw storage of VW values of dtype DT (8, 16 or 32 bytes), kept in registers between
// the two passes.
template <int DT, int VW> struct WnRaw {
    static constexpr int NB = VW * (DT == BSMM_F32 ? 4 : 2);
    uint32_t w[NB / 4];
};
template <int DT, int VW> __device__ __forceinline__ void wn_rawload(WnRaw<DT, VW>& r, const void* base, int64_t idx) {
    const char* p = (const char*)base + idx * (DT == BSMM_F32 ? 4 : 2);
    if constexpr (WnRaw<DT, VW>::NB == 8) {
        const u32x2 q = *reinterpret_cast<const u32x2*>(p);
        r.w[0] = q.x;
        r.w[1] = q.y;
    } else {
#pragma unroll
        for (int h = 0; h < WnRaw<DT, VW>::NB / 16; h++) {
            const u32x4 q = *reinterpret_cast<const u32x4*>(p + 16 * h);
            r.w[4 * h] = q.x;
            r.w[4 * h + 1] = q.y;
            r.w[4 * h + 2] = q.z;
            r.w[4 * h + 3] = q.w;
        }
    }
}
template <int DT, int VW> __device__ __forceinline__ void wn_rawcvt(const WnRaw<DT, VW>& r, float* v) {
    if constexpr (DT == BSMM_F32) {
#pragma unroll
        for (int i = 0; i < VW; i++) v[i] = __uint_as_float(r.w[i]);
    } else {
#pragma unroll
        for (int i = 0; i < VW / 2; i++) {
            if constexpr (DT == BSMM_BF16) {
                v[2 * i] = __uint_as_float(r.w[i] << 16);
                v[2 * i + 1] = __uint_as_float(r.w[i] & 0xffff0000u);
            } else {
                v[2 * i] = (float)__builtin_bit_cast(_Float16, (uint16_t)(r.w[i] & 0xffffu));
                v[2 * i + 1] = (float)__builtin_bit_cast(_Float16, (uint16_t)(r.w[i] >> 16));
            }
        }
    }
}

// Work map: a thread owns one 16-byte vector of the weights' storage (VW values of one
// block row) per block; the workgroup covers P blocks of the list side by side, walked
// U at a time so that U loads per thread are in flight.  Thread t: block slot t / VB,
// row (t % VB) / VR, columns (t % VR)*VW .. +VW-1.  The first IT rounds of U blocks
// stay in registers from the sums to the elementwise pass (a column of up to IT*P*U
// blocks is read once); longer columns read the rest again.
template <int B, int DTI> struct WnMap {
    static constexpr int VW = DTI == BSMM_F32 ? 4 : 8;
    static constexpr int VR = B / VW;                 // vectors per block row (>= 1)
    static constexpr int VB = B * VR;                 // vectors per block
    static constexpr int P = kWnThreads / VB;         // blocks side by side (>= 1)
    static constexpr int U = 8;
    static constexpr int IT = 1;    // rounds kept (the gradient keeps one round of two tensors)
    static_assert(B % VW == 0 && kWnThreads % VB == 0, "work map");
};

// Column sums of two per-thread VW-vectors over the threads of the same column vector
// (threads t = cv mod VR): a butterfly over the lane bits above VR inside each wave,
// then the 16 waves' sums added in wave order (fixed order: deterministic); thread
// t < B gets column t's sums.
template <int B, int VW, int VR, bool TWO>
__device__ __forceinline__ void wn_colsum(const float* a, const float* b, float* ra, float* rb, float& oa, float& ob) {
    const int t = threadIdx.x, lane = t & 63, wv = t >> 6;
    float x[VW], y[VW];
#pragma unroll
    for (int k = 0; k < VW; k++) {
        x[k] = a[k];
        y[k] = TWO ? b[k] : 0.f;
    }
#pragma unroll
    for (int o = VR; o < 64; o <<= 1)
#pragma unroll
        for (int k = 0; k < VW; k++) {
            x[k] += __shfl_xor(x[k], o);
            if constexpr (TWO) y[k] += __shfl_xor(y[k], o);
        }
    if (lane < VR)   // lane = column vector cv: columns cv*VW .. +VW-1
#pragma unroll
        for (int k = 0; k < VW; k++) {
            ra[wv * B + lane * VW + k] = x[k];
            if constexpr (TWO) rb[wv * B + lane * VW + k] = y[k];
        }
    __syncthreads();
    oa = ob = 0.f;
    if (t < B) {
        for (int w = 0; w < kWnThreads / 64; w++) {
            oa += ra[w * B + t];
            if constexpr (TWO) ob += rb[w * B + t];
        }
    }
}

template <int B, int DTI, int DTO>
__global__ __launch_bounds__(kWnThreads) void wn_fwd(WnArgs a) {
    using Map = WnMap<B, DTI>;
    constexpr int VW = Map::VW, VR = Map::VR, VB = Map::VB, P = Map::P, U = Map::U, IT = Map::IT;
    __shared__ float ra[kWnThreads / 64 * B], rb[kWnThreads / 64 * B], scale[B];
    const int k = blockIdx.x, t = threadIdx.x;
    const int beg = a.colptr[k], end = a.colptr[k + 1];
    const int slot = t / VB, e0 = (t % VB) * VW;   // element offset inside a block
    float ss[VW];
#pragma unroll
    for (int i = 0; i < VW; i++) ss[i] = 0.f;
    // block q of the list -> its element offset; blocks past the end read the list's first
    auto off = [&](int q) { return (int64_t)a.colent[2 * (q < end ? q : beg) + 1] * B * B + e0; };
    WnRaw<DTI, VW> keep[IT][U];
#pragma unroll
    for (int it = 0; it < IT; it++) {
        const int q0 = beg + slot + it * P * U;
#pragma unroll
        for (int uu = 0; uu < U; uu++) wn_rawload<DTI, VW>(keep[it][uu], a.w, off(q0 + P * uu));
#pragma unroll
        for (int uu = 0; uu < U; uu++)
            if (q0 + P * uu < end) {
                float v[VW];
                wn_rawcvt<DTI, VW>(keep[it][uu], v);
#pragma unroll
                for (int i = 0; i < VW; i++) ss[i] += v[i] * v[i];
            }
    }
    for (int q0 = beg + slot + IT * P * U; q0 < end; q0 += P * U) {
        WnRaw<DTI, VW> r[U];
#pragma unroll
        for (int uu = 0; uu < U; uu++) wn_rawload<DTI, VW>(r[uu], a.w, off(q0 + P * uu));
#pragma unroll
        for (int uu = 0; uu < U; uu++)
            if (q0 + P * uu < end) {
                float v[VW];
                wn_rawcvt<DTI, VW>(r[uu], v);
#pragma unroll
                for (int i = 0; i < VW; i++) ss[i] += v[i] * v[i];
            }
    }
    float s, unused;
    wn_colsum<B, VW, VR, false>(ss, ss, ra, rb, s, unused);
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
    auto put = [&](const WnRaw<DTI, VW>& r, int q) {
        float v[VW];
        wn_rawcvt<DTI, VW>(r, v);
#pragma unroll
        for (int i = 0; i < VW; i++) v[i] *= sc[i];
        wn_storev<DTO, VW>(a.out, off(q), v);
    };
#pragma unroll
    for (int it = 0; it < IT; it++)
#pragma unroll
        for (int uu = 0; uu < U; uu++) {
            const int q = beg + slot + it * P * U + P * uu;
            if (q < end) put(keep[it][uu], q);
        }
    for (int q0 = beg + slot + IT * P * U; q0 < end; q0 += P * U) {   // U loads in flight, then U stores
        WnRaw<DTI, VW> r[U];
#pragma unroll
        for (int uu = 0; uu < U; uu++) wn_rawload<DTI, VW>(r[uu], a.w, off(q0 + P * uu));
#pragma unroll
        for (int uu = 0; uu < U; uu++)
            if (q0 + P * uu < end) put(r[uu], q0 + P * uu);
    }
}

template <int B, int DTI, int DTD>
__global__ __launch_bounds__(kWnThreads) void wn_bwd(WnArgs a) {
    using Map = WnMap<B, DTI>;
    constexpr int VW = Map::VW, VR = Map::VR, VB = Map::VB, P = Map::P, U2 = Map::U / 2, IT = 1;
    __shared__ float ra[kWnThreads / 64 * B], rb[kWnThreads / 64 * B], ca[B], cb[B];
    const int k = blockIdx.x, t = threadIdx.x;
    const int beg = a.colptr[k], end = a.colptr[k + 1];
    const int slot = t / VB, e0 = (t % VB) * VW;
    float ss[VW], sd[VW];
#pragma unroll
    for (int i = 0; i < VW; i++) ss[i] = sd[i] = 0.f;
    auto off = [&](int q) { return (int64_t)a.colent[2 * (q < end ? q : beg) + 1] * B * B + e0; };
    // two tensors: U/2 blocks per round
    WnRaw<DTI, VW> kw[IT][U2];
    WnRaw<DTD, VW> kd[IT][U2];
    auto sums = [&](const WnRaw<DTI, VW>& rw, const WnRaw<DTD, VW>& rd) {
        float w[VW], d[VW];
        wn_rawcvt<DTI, VW>(rw, w);
        wn_rawcvt<DTD, VW>(rd, d);
#pragma unroll
        for (int i = 0; i < VW; i++) {
            ss[i] += w[i] * w[i];
            sd[i] += d[i] * w[i];
        }
    };
#pragma unroll
    for (int it = 0; it < IT; it++) {
        const int q0 = beg + slot + it * P * U2;
#pragma unroll
        for (int uu = 0; uu < U2; uu++) {
            const int64_t idx = off(q0 + P * uu);
            wn_rawload<DTI, VW>(kw[it][uu], a.w, idx);
            wn_rawload<DTD, VW>(kd[it][uu], a.dy, idx);
        }
#pragma unroll
        for (int uu = 0; uu < U2; uu++)
            if (q0 + P * uu < end) sums(kw[it][uu], kd[it][uu]);
    }
    for (int q0 = beg + slot + IT * P * U2; q0 < end; q0 += P * U2) {
        WnRaw<DTI, VW> rw[U2];
        WnRaw<DTD, VW> rd[U2];
#pragma unroll
        for (int uu = 0; uu < U2; uu++) {
            const int64_t idx = off(q0 + P * uu);
            wn_rawload<DTI, VW>(rw[uu], a.w, idx);
            wn_rawload<DTD, VW>(rd[uu], a.dy, idx);
        }
#pragma unroll
        for (int uu = 0; uu < U2; uu++)
            if (q0 + P * uu < end) sums(rw[uu], rd[uu]);
    }
    float s2, s1;
    wn_colsum<B, VW, VR, true>(ss, sd, ra, rb, s2, s1);
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
    auto put = [&](const WnRaw<DTI, VW>& rw, const WnRaw<DTD, VW>& rd, int q) {
        float w[VW], d[VW], r[VW];
        wn_rawcvt<DTI, VW>(rw, w);
        wn_rawcvt<DTD, VW>(rd, d);
#pragma unroll
        for (int i = 0; i < VW; i++) r[i] = c1[i] * d[i] - c2[i] * w[i];
        wn_storev<BSMM_F32, VW>(a.out, off(q), r);
    };
#pragma unroll
    for (int it = 0; it < IT; it++)
#pragma unroll
        for (int uu = 0; uu < U2; uu++) {
            const int q = beg + slot + it * P * U2 + P * uu;
            if (q < end) put(kw[it][uu], kd[it][uu], q);
        }
    for (int q0 = beg + slot + IT * P * U2; q0 < end; q0 += P * U2) {
        WnRaw<DTI, VW> rw[U2];
        WnRaw<DTD, VW> rd[U2];
#pragma unroll
        for (int uu = 0; uu < U2; uu++) {
            const int64_t idx = off(q0 + P * uu);
            wn_rawload<DTI, VW>(rw[uu], a.w, idx);
            wn_rawload<DTD, VW>(rd[uu], a.dy, idx);
        }
#pragma unroll
        for (int uu = 0; uu < U2; uu++)
            if (q0 + P * uu < end) put(rw[uu], rd[uu], q0 + P * uu);
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
