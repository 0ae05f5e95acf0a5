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
// A workgroup owns one block column, or 1/FS of its features (the sums of different
// output features are independent, so FS workgroups split a column without any
// exchange), and walks the column's block list (the fprop column list of the layout
// tables) in 16-byte vectors: the column sums (fp32: a butterfly inside each wave, then
// the waves in order — deterministic), then the elementwise pass.  The first two
// rounds of blocks stay in registers between the two passes; only longer columns read
// the rest again (from L2).  The FS workgroups of a column run on one XCD, so the lines they
// share are fetched into one L2.
// Bound: HBM (|W| read, |out| written; |dOut| + |W| read, |dW| written).
#include <cstdlib>

#include "common.h"

namespace bsmm {

// Threads per whole block column (its loads all in flight); 8-wide blocks take half,
// which leaves them room for the table reads without spilling.
template <int B> constexpr int wn_threads() { return B == 8 ? 512 : 1024; }

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

// Work map: a workgroup of NT = wn_threads<B>()/FS threads owns features f*BP .. f*BP+BP-1
// (BP = B/FS) of its block column; a thread owns one 16-byte vector of the weights'
// storage (VW values of one block row) per block, and the workgroup covers P blocks of
// the list side by side, walked U at a time so that U loads per thread are in flight.
// Thread t: block slot t / VB, row (t % VB) / VR, columns f*BP + (t % VR)*VW .. +VW-1.
// The first IT rounds of U blocks stay in registers from the sums to the elementwise
// pass (a column of up to IT*P*U blocks is read once); longer columns read the rest
// again.
template <int B, int DTI, int FS> struct WnMap {
    static constexpr int VW = DTI == BSMM_F32 ? 4 : 8;
    static constexpr int BP = B / FS;                 // features per workgroup
    static constexpr int VR = BP / VW;                // vectors per block row (>= 1)
    static constexpr int VB = B * VR;                 // vectors per block
    static constexpr int NT = wn_threads<B>() / FS;   // threads
    static constexpr int P = NT / VB;                 // blocks side by side (>= 1)
    static constexpr int U = 8;
    static constexpr int IT = 2;    // rounds kept
    static_assert(BP % VW == 0 && NT % VB == 0 && NT >= 64, "work map");
};

// Most feature splits per block column that the vector width allows (B/FS a multiple
// of it, at most 4).
template <int B, int DTI> constexpr int wn_max_fs() {
    constexpr int VW = DTI == BSMM_F32 ? 4 : 8;
    return B / VW >= 4 ? 4 : B / VW;
}

// Column sums of two per-thread VW-vectors over the threads of the same column vector
// (threads t = cv mod VR): a butterfly over the lane bits above VR inside each wave,
// then the NT/64 waves' sums added in wave order (fixed order: deterministic); thread
// t < BP gets the sums of the workgroup's column t.
template <int BP, int VW, int VR, int NT, bool TWO>
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
            ra[wv * BP + lane * VW + k] = x[k];
            if constexpr (TWO) rb[wv * BP + lane * VW + k] = y[k];
        }
    __syncthreads();
    oa = ob = 0.f;
    if (t < BP) {
        for (int w = 0; w < NT / 64; w++) {
            oa += ra[w * BP + t];
            if constexpr (TWO) ob += rb[w * BP + t];
        }
    }
}

// Block column and feature part of this workgroup: the FS parts of a column share
// blockIdx mod 8 (one XCD); false past the last column.
template <int FS> __device__ __forceinline__ bool wn_decode(int S, int& k, int& f) {
    const int bid = blockIdx.x, r = bid % (8 * FS);
    k = (bid / (8 * FS)) * 8 + r % 8;
    f = r / 8;
    return k < S;
}

// The block list of column k (the fprop column list); positions past its end give the
// list's first block, and every position of an empty list the first block of the
// table (read, never used).
struct WnList {
    const int32_t* ent;
    int col, len;
    __device__ __forceinline__ WnList(const WnArgs& a, int k) {
        const int beg = a.colptr[k];
        len = a.colptr[k + 1] - beg;
        ent = a.colent + (len > 0 ? 2 * beg : 0);
        col = k;
    }
    __device__ __forceinline__ int id(int q) const { return ent[2 * (q < len ? q : 0) + 1]; }
};

template <int B, int DTI, int DTO, int FS>
__global__ __launch_bounds__((B == 8 ? 512 : 1024) / FS) void wn_fwd(WnArgs a) {
    using Map = WnMap<B, DTI, FS>;
    constexpr int VW = Map::VW, BP = Map::BP, VR = Map::VR, VB = Map::VB, NT = Map::NT, P = Map::P, U = Map::U,
                  IT = Map::IT;
    __shared__ float ra[NT / 64 * BP], rb[NT / 64 * BP], scale[BP];
    int k, f;
    if (!wn_decode<FS>((int)a.S, k, f)) return;
    const int t = threadIdx.x;
    const WnList L(a, k);
    const int len = L.len;
    const int slot = t / VB, cv = t % VR;
    const int e0 = ((t % VB) / VR) * B + f * BP + cv * VW;   // element offset inside a block
    float ss[VW];
#pragma unroll
    for (int i = 0; i < VW; i++) ss[i] = 0.f;
    auto off = [&](int q) { return (int64_t)L.id(q) * B * B + e0; };
    WnRaw<DTI, VW> keep[IT][U];
#pragma unroll
    for (int it = 0; it < IT; it++) {
        const int q0 = slot + it * P * U;
#pragma unroll
        for (int uu = 0; uu < U; uu++) wn_rawload<DTI, VW>(keep[it][uu], a.w, off(q0 + P * uu));
#pragma unroll
        for (int uu = 0; uu < U; uu++)
            if (q0 + P * uu < len) {
                float v[VW];
                wn_rawcvt<DTI, VW>(keep[it][uu], v);
#pragma unroll
                for (int i = 0; i < VW; i++) ss[i] += v[i] * v[i];
            }
    }
    for (int q0 = slot + IT * P * U; q0 < len; q0 += P * U) {
        WnRaw<DTI, VW> r[U];
#pragma unroll
        for (int uu = 0; uu < U; uu++) wn_rawload<DTI, VW>(r[uu], a.w, off(q0 + P * uu));
#pragma unroll
        for (int uu = 0; uu < U; uu++)
            if (q0 + P * uu < len) {
                float v[VW];
                wn_rawcvt<DTI, VW>(r[uu], v);
#pragma unroll
                for (int i = 0; i < VW; i++) ss[i] += v[i] * v[i];
            }
    }
    float s, unused;
    wn_colsum<BP, VW, VR, NT, false>(ss, ss, ra, rb, s, unused);
    if (t < BP) {
        const int o = L.col * B + f * BP + t;
        const float n = sqrtf(fmaxf(s, a.eps));
        if (a.norms) a.norms[o] = n;
        scale[t] = (a.gain ? a.gain[o] : 1.0f) / n;
    }
    __syncthreads();
    float sc[VW];
#pragma unroll
    for (int i = 0; i < VW; i++) sc[i] = scale[cv * VW + i];
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
            const int q = slot + it * P * U + P * uu;
            if (q < len) put(keep[it][uu], q);
        }
    for (int q0 = slot + IT * P * U; q0 < len; q0 += P * U) {   // U loads in flight, then U stores
        WnRaw<DTI, VW> r[U];
#pragma unroll
        for (int uu = 0; uu < U; uu++) wn_rawload<DTI, VW>(r[uu], a.w, off(q0 + P * uu));
#pragma unroll
        for (int uu = 0; uu < U; uu++)
            if (q0 + P * uu < len) put(r[uu], q0 + P * uu);
    }
}

template <int B, int DTI, int DTD, int FS>
__global__ __launch_bounds__((B == 8 ? 512 : 1024) / FS) void wn_bwd(WnArgs a) {
    using Map = WnMap<B, DTI, FS>;
    constexpr int VW = Map::VW, BP = Map::BP, VR = Map::VR, VB = Map::VB, NT = Map::NT, P = Map::P,
                  U2 = Map::U / 2, IT = Map::IT;
    __shared__ float ra[NT / 64 * BP], rb[NT / 64 * BP], ca[BP], cb[BP];
    int k, f;
    if (!wn_decode<FS>((int)a.S, k, f)) return;
    const int t = threadIdx.x;
    const WnList L(a, k);
    const int len = L.len;
    const int slot = t / VB, cv = t % VR;
    const int e0 = ((t % VB) / VR) * B + f * BP + cv * VW;
    float ss[VW], sd[VW];
#pragma unroll
    for (int i = 0; i < VW; i++) ss[i] = sd[i] = 0.f;
    auto off = [&](int q) { return (int64_t)L.id(q) * B * B + e0; };
    // two tensors: U/2 blocks per round, IT rounds kept
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
        const int q0 = slot + it * P * U2;
#pragma unroll
        for (int uu = 0; uu < U2; uu++) {
            const int64_t idx = off(q0 + P * uu);
            wn_rawload<DTI, VW>(kw[it][uu], a.w, idx);
            wn_rawload<DTD, VW>(kd[it][uu], a.dy, idx);
        }
#pragma unroll
        for (int uu = 0; uu < U2; uu++)
            if (q0 + P * uu < len) sums(kw[it][uu], kd[it][uu]);
    }
    for (int q0 = slot + IT * P * U2; q0 < len; q0 += P * U2) {
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
            if (q0 + P * uu < len) sums(rw[uu], rd[uu]);
    }
    float s2, s1;
    wn_colsum<BP, VW, VR, NT, true>(ss, sd, ra, rb, s2, s1);
    if (t < BP) {
        const int o = L.col * B + f * BP + t;
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
        c1[i] = ca[cv * VW + i];
        c2[i] = cb[cv * VW + i];
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
            const int q = slot + it * P * U2 + P * uu;
            if (q < len) put(kw[it][uu], kd[it][uu], q);
        }
    for (int q0 = slot + IT * P * U2; q0 < len; q0 += P * U2) {
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
            if (q0 + P * uu < len) put(rw[uu], rd[uu], q0 + P * uu);
    }
}

namespace {
template <int B, int DTI, int FS>
hipError_t wn_fs(const WnArgs& a, bool grad, hipStream_t st) {
    const dim3 grid((unsigned)(((a.S + 7) / 8) * 8 * FS)), blk(WnMap<B, DTI, FS>::NT);
    const int d2 = grad ? a.dy_dt : a.out_dt;
#define BSMM_WN(D2)                                                                               \
    case D2:                                                                                      \
        return grad ? launch_ev(wn_bwd<B, DTI, D2, FS>, grid, blk, st, a.e0, a.e1, a)             \
                    : launch_ev(wn_fwd<B, DTI, D2, FS>, grid, blk, st, a.e0, a.e1, a);
    switch (d2) {
        BSMM_WN(BSMM_F32)
        BSMM_WN(BSMM_BF16)
        BSMM_WN(BSMM_F16)
    }
#undef BSMM_WN
    return hipErrorInvalidValue;
}
// Feature splits: one workgroup per column for 8-wide blocks, two for wider ones (on
// the 4096-wide, 32-wide-block layout with bf16 weights, 1 / 2 / 4 splits: forward
// 16.8 / 14.7 / 16.4 us, gradient 23.3-23.7 / 20.1-20.7 / 26.1-26.2 us: four splits
// read 16 of every 64 bytes per row and lose more in request count than they gain in
// workgroups).  BSMM_WN_FS=1|2|4 (read once) overrides it where the vector width
// allows, for measurement.
template <int B, int DTI>
hipError_t wn_b(const WnArgs& a, bool grad, hipStream_t st) {
    constexpr int MF = wn_max_fs<B, DTI>();
    static const int env_fs = [] {
        const char* e = getenv("BSMM_WN_FS");
        return e ? atoi(e) : 0;
    }();
    const int fs = env_fs > 0 ? env_fs : (B == 8 ? 1 : 2);
    if constexpr (MF >= 4)
        if (fs >= 4) return wn_fs<B, DTI, 4>(a, grad, st);
    if constexpr (MF >= 2)
        if (fs >= 2 || B > 8) return wn_fs<B, DTI, 2>(a, grad, st);
    if constexpr (B == 8) return wn_fs<B, DTI, 1>(a, grad, st);
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
