// SparseProj: projections between a dense activation of nhidden features and a sparse
// one of nproj features through a one-to-one feature map (kiteco/blocksparse README,
// "API Documentation" › blocksparse.matmul › SparseProj: gather, scatter, scatter_add,
// scatter_mul; the map is one-to-one, so no output is written twice and the backward
// ops need no atomics).
//
// Every op is one pass over its output features j: out[., j] = combine(base[., j],
// src[., map[j]]), with map the projected->dense table (gather, and gather_mul, the
// y-gradient of scatter_mul) or the dense->projected table, -1 where a dense feature is
// not projected (scatter, scatter_add, scatter_mul).  Scatters therefore never write
// through the map: each output element is written once, in order, by one thread.
//
// Bound: HBM.  A thread takes 16 bytes of output.  Features last (N, W): 16 bytes of one
// row, with the source read as one 16-byte vector when its map entries are consecutive
// and aligned (the blocked default map), element by element otherwise.  Features first
// (W, N): 16 bytes of one output row, from one source row.  add / mul compute in fp32
// and round once (RNE) to the storage type; copies keep the stored bits.
#include "common.h"

namespace bsmm {

template <int DT> __device__ __forceinline__ float proj_load(const void* p, int64_t i) {
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
template <int DT> __device__ __forceinline__ uint32_t proj_bits(const void* p, int64_t i) {
    if constexpr (DT == BSMM_F32)
        return ((const uint32_t*)p)[i];
    else
        return ((const uint16_t*)p)[i];
}
template <int DT> __device__ __forceinline__ uint32_t proj_round(float v) {
    if constexpr (DT == BSMM_F32)
        return __float_as_uint(v);
    else
        return to_storage16<DT>(v);
}
template <int DT> __device__ __forceinline__ float bits_val(uint32_t b) {
    if constexpr (DT == BSMM_F32)
        return __uint_as_float(b);
    else if constexpr (DT == BSMM_BF16)
        return __uint_as_float(b << 16);
    else
        return (float)__builtin_bit_cast(_Float16, (uint16_t)b);
}

// one output element from its base bits (ADD, MUL) and source bits; m < 0: no source
template <int DT, int MODE> __device__ __forceinline__ uint32_t proj_combine(uint32_t base, uint32_t src, int m) {
    if constexpr (MODE == PROJ_GATHER) {
        return src;
    } else if constexpr (MODE == PROJ_SCATTER) {
        return m >= 0 ? src : 0u;
    } else if constexpr (MODE == PROJ_ADD) {
        return m >= 0 ? proj_round<DT>(bits_val<DT>(base) + bits_val<DT>(src)) : base;
    } else if constexpr (MODE == PROJ_MUL) {
        return m >= 0 ? proj_round<DT>(bits_val<DT>(base) * bits_val<DT>(src)) : base;
    } else {   // GATHER_MUL: base is the second gathered source
        return proj_round<DT>(bits_val<DT>(base) * bits_val<DT>(src));
    }
}

template <int DT> __device__ __forceinline__ void store_bits(void* p, int64_t i, uint32_t b) {
    if constexpr (DT == BSMM_F32)
        ((uint32_t*)p)[i] = b;
    else
        ((uint16_t*)p)[i] = (uint16_t)b;
}

template <int DT, int MODE, int FA>
__global__ __launch_bounds__(256) void proj_kernel(ProjArgs a) {
    constexpr int V = DT == BSMM_F32 ? 4 : 8;   // elements per 16 bytes
    constexpr bool BASE_OUT = MODE == PROJ_ADD || MODE == PROJ_MUL;   // base indexed like out
    constexpr bool BASE_SRC = MODE == PROJ_GATHER_MUL;                // base indexed like src
    const int64_t N = a.N, wout = a.wout, wsrc = a.wsrc;
    const int64_t stride = (int64_t)gridDim.x * 256;
    if constexpr (FA == 1) {
        // (N, W): vector v covers out[n][j0 .. j0+V-1]
        const bool vec = (wout % V) == 0, srcvec = (wsrc % V) == 0;
        const int64_t vpr = (wout + V - 1) / V, total = N * vpr;
        for (int64_t v = (int64_t)blockIdx.x * 256 + threadIdx.x; v < total; v += stride) {
            const int64_t n = v / vpr, j0 = (v % vpr) * V;
            const int64_t orow = n * wout, srow = n * wsrc;
            if (vec) {
                int m[V];
#pragma unroll
                for (int i = 0; i < V; i++) m[i] = a.map[j0 + i];
                bool run = srcvec && m[0] >= 0 && (m[0] % V) == 0;
#pragma unroll
                for (int i = 1; i < V; i++) run = run && m[i] == m[0] + i;
                uint32_t sb[V], bb[V];
                if (run) {   // consecutive aligned source features: one 16-byte load
                    const u32x4 q = *reinterpret_cast<const u32x4*>(
                        (const char*)a.src + (srow + m[0]) * (int64_t)(DT == BSMM_F32 ? 4 : 2));
                    if constexpr (DT == BSMM_F32) {
                        sb[0] = q.x; sb[1] = q.y; sb[2] = q.z; sb[3] = q.w;
                    } else {
                        const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
                        for (int i = 0; i < 4; i++) {
                            sb[2 * i] = w[i] & 0xffffu;
                            sb[2 * i + 1] = w[i] >> 16;
                        }
                    }
                    if constexpr (BASE_SRC) {
                        const u32x4 r = *reinterpret_cast<const u32x4*>(
                            (const char*)a.base + (srow + m[0]) * (int64_t)(DT == BSMM_F32 ? 4 : 2));
                        if constexpr (DT == BSMM_F32) {
                            bb[0] = r.x; bb[1] = r.y; bb[2] = r.z; bb[3] = r.w;
                        } else {
                            const uint32_t w[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
                            for (int i = 0; i < 4; i++) {
                                bb[2 * i] = w[i] & 0xffffu;
                                bb[2 * i + 1] = w[i] >> 16;
                            }
                        }
                    }
                } else {
#pragma unroll
                    for (int i = 0; i < V; i++) {
                        sb[i] = m[i] >= 0 ? proj_bits<DT>(a.src, srow + m[i]) : 0u;
                        if constexpr (BASE_SRC) bb[i] = proj_bits<DT>(a.base, srow + m[i]);
                    }
                }
                if constexpr (BASE_OUT) {
                    const u32x4 r = *reinterpret_cast<const u32x4*>(
                        (const char*)a.base + (orow + j0) * (int64_t)(DT == BSMM_F32 ? 4 : 2));
                    if constexpr (DT == BSMM_F32) {
                        bb[0] = r.x; bb[1] = r.y; bb[2] = r.z; bb[3] = r.w;
                    } else {
                        const uint32_t w[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
                        for (int i = 0; i < 4; i++) {
                            bb[2 * i] = w[i] & 0xffffu;
                            bb[2 * i + 1] = w[i] >> 16;
                        }
                    }
                }
                uint32_t ob[V];
#pragma unroll
                for (int i = 0; i < V; i++) ob[i] = proj_combine<DT, MODE>((BASE_OUT || BASE_SRC) ? bb[i] : 0u, sb[i], m[i]);
                u32x4 o;
                if constexpr (DT == BSMM_F32) {
                    o = u32x4{ob[0], ob[1], ob[2], ob[3]};
                } else {
                    o = u32x4{ob[0] | (ob[1] << 16), ob[2] | (ob[3] << 16), ob[4] | (ob[5] << 16), ob[6] | (ob[7] << 16)};
                }
                *reinterpret_cast<u32x4*>((char*)a.out + (orow + j0) * (int64_t)(DT == BSMM_F32 ? 4 : 2)) = o;
            } else {   // rows not a multiple of 16 bytes: element by element
                for (int i = 0; i < V && j0 + i < wout; i++) {
                    const int mi = a.map[j0 + i];
                    const uint32_t sb = mi >= 0 ? proj_bits<DT>(a.src, srow + mi) : 0u;
                    uint32_t bb = 0u;
                    if constexpr (BASE_OUT) bb = proj_bits<DT>(a.base, orow + j0 + i);
                    if constexpr (BASE_SRC) bb = proj_bits<DT>(a.base, srow + mi);
                    store_bits<DT>(a.out, orow + j0 + i, proj_combine<DT, MODE>(bb, sb, mi));
                }
            }
        }
    } else {
        // (W, N): vector v covers out[j][n0 .. n0+V-1], from source row map[j]
        const bool vec = (N % V) == 0;
        const int64_t vpr = (N + V - 1) / V, total = wout * vpr;
        for (int64_t v = (int64_t)blockIdx.x * 256 + threadIdx.x; v < total; v += stride) {
            const int64_t j = v / vpr, n0 = (v % vpr) * V;
            const int m = a.map[j];
            const int64_t o0 = j * N + n0, s0 = (int64_t)(m >= 0 ? m : 0) * N + n0;
            if (vec) {
                constexpr int S = DT == BSMM_F32 ? 4 : 2;
                u32x4 q = u32x4{0u, 0u, 0u, 0u}, r = u32x4{0u, 0u, 0u, 0u};
                if (m >= 0) q = *reinterpret_cast<const u32x4*>((const char*)a.src + s0 * S);
                if constexpr (BASE_OUT) r = *reinterpret_cast<const u32x4*>((const char*)a.base + o0 * S);
                if constexpr (BASE_SRC) r = *reinterpret_cast<const u32x4*>((const char*)a.base + s0 * S);
                u32x4 o;
                if constexpr (DT == BSMM_F32) {
#pragma unroll
                    for (int i = 0; i < 4; i++) o[i] = proj_combine<DT, MODE>(r[i], q[i], m);
                } else {
#pragma unroll
                    for (int i = 0; i < 4; i++) {
                        const uint32_t lo = proj_combine<DT, MODE>(r[i] & 0xffffu, q[i] & 0xffffu, m);
                        const uint32_t hi = proj_combine<DT, MODE>(r[i] >> 16, q[i] >> 16, m);
                        o[i] = (lo & 0xffffu) | (hi << 16);
                    }
                }
                *reinterpret_cast<u32x4*>((char*)a.out + o0 * S) = o;
            } else {
                for (int i = 0; i < V && n0 + i < N; i++) {
                    const uint32_t sb = m >= 0 ? proj_bits<DT>(a.src, s0 + i) : 0u;
                    uint32_t bb = 0u;
                    if constexpr (BASE_OUT) bb = proj_bits<DT>(a.base, o0 + i);
                    if constexpr (BASE_SRC) bb = proj_bits<DT>(a.base, s0 + i);
                    store_bits<DT>(a.out, o0 + i, proj_combine<DT, MODE>(bb, sb, m));
                }
            }
        }
    }
}

template <int DT, int MODE>
static hipError_t launch_proj_m(const ProjArgs& a, hipStream_t st) {
    constexpr int V = DT == BSMM_F32 ? 4 : 8;
    const int64_t per = a.fa == 1 ? (a.wout + V - 1) / V : (a.N + V - 1) / V;
    const int64_t total = (a.fa == 1 ? a.N : a.wout) * per;
    int64_t grid = (total + 255) / 256;
    if (grid > (1 << 16)) grid = 1 << 16;   // grid-stride beyond that
    if (grid < 1) return hipSuccess;
    const int pass = BSMM_PASS_PROJ_GATHER + MODE;
    if (a.fa == 1) return launch(pass, proj_kernel<DT, MODE, 1>, dim3((unsigned)grid), dim3(256), st, a);
    return launch(pass, proj_kernel<DT, MODE, 0>, dim3((unsigned)grid), dim3(256), st, a);
}

template <int DT>
static hipError_t launch_proj_dt(const ProjArgs& a, hipStream_t st) {
    switch (a.mode) {
    case PROJ_GATHER: return launch_proj_m<DT, PROJ_GATHER>(a, st);
    case PROJ_SCATTER: return launch_proj_m<DT, PROJ_SCATTER>(a, st);
    case PROJ_ADD: return launch_proj_m<DT, PROJ_ADD>(a, st);
    case PROJ_MUL: return launch_proj_m<DT, PROJ_MUL>(a, st);
    case PROJ_GATHER_MUL: return launch_proj_m<DT, PROJ_GATHER_MUL>(a, st);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_proj(const ProjArgs& a, void* stream) {
    hipStream_t st = (hipStream_t)stream;
    if (a.N == 0 || a.wout == 0) return hipSuccess;
    switch (a.dt) {
    case BSMM_F32: return launch_proj_dt<BSMM_F32>(a, st);
    case BSMM_BF16: return launch_proj_dt<BSMM_BF16>(a, st);
    case BSMM_F16: return launch_proj_dt<BSMM_F16>(a, st);
    }
    return hipErrorInvalidValue;
}

}  // namespace bsmm
