// Device helpers shared by the gfx950 kernels: storage types, the matrix-core step,
// fragment loaders (global and LDS-transposed), fp32 -> storage rounding, the
// XCD-aware workgroup mapping, and the host launch wrapper.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <cstdint>

#include "bsmm.h"
#include "kernels.h"

namespace bsmm {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));

#define BSMM_LDS __attribute__((address_space(3)))

// Storage element and the number of contraction values one lane holds per operand
// fragment (16 bytes): 4 fp32 or 8 bf16/f16.
template <int DT> struct Elt;
template <> struct Elt<BSMM_F32> { using T = float; static constexpr int VEC = 4; };
template <> struct Elt<BSMM_BF16> { using T = uint16_t; static constexpr int VEC = 8; };
template <> struct Elt<BSMM_F16> { using T = uint16_t; static constexpr int VEC = 8; };

// Matrix-core step on 16x16 tiles with fp32 accumulation.
//   Operand fragment (16 rows x 4*VEC contraction values): lane l holds row l % 16 and
//   contraction values 4*VEC/4*(l/16) .. +VEC-1 in element order.  Both operands use
//   the same lane -> contraction-index map, so the order the hardware uses inside one
//   instruction does not matter for the sum.
//   Result: lane l holds D[4*(l/16) + v][l % 16], v = 0..3, D[m][n] = sum_k A[m][k] B[n][k].
//   fp32: 4 x v_mfma_f32_16x16x4_f32, element v of each fragment in step v.
template <int DT> __device__ __forceinline__ void mma(f32x4& acc, const u32x4& a, const u32x4& b);
template <> __device__ __forceinline__ void mma<BSMM_F32>(f32x4& acc, const u32x4& a, const u32x4& b) {
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.x), __uint_as_float(b.x), acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.y), __uint_as_float(b.y), acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.z), __uint_as_float(b.z), acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.w), __uint_as_float(b.w), acc, 0, 0, 0);
}
template <> __device__ __forceinline__ void mma<BSMM_BF16>(f32x4& acc, const u32x4& a, const u32x4& b) {
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b),
                                                  acc, 0, 0, 0);
}
template <> __device__ __forceinline__ void mma<BSMM_F16>(f32x4& acc, const u32x4& a, const u32x4& b) {
    acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b),
                                                 acc, 0, 0, 0);
}

// fp32 -> bfloat16, round to nearest even (NaN stays NaN).
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
    u += 0x7fffu + ((u >> 16) & 1u);
    return u >> 16;
}
// fp32 -> IEEE binary16 with the hardware conversion (round to nearest even).
__device__ __forceinline__ uint32_t f32_to_f16(float f) {
    _Float16 h = (_Float16)f;
    return (uint32_t)__builtin_bit_cast(uint16_t, h);
}
template <int DT> __device__ __forceinline__ uint32_t to_storage16(float f) {
    if constexpr (DT == BSMM_BF16)
        return f32_to_bf16(f);
    else
        return f32_to_f16(f);
}
__device__ __forceinline__ void store_elt(void* base, int64_t idx, float v, int dt) {
    if (dt == BSMM_F32)
        ((float*)base)[idx] = v;
    else if (dt == BSMM_BF16)
        ((uint16_t*)base)[idx] = (uint16_t)f32_to_bf16(v);
    else
        ((uint16_t*)base)[idx] = (uint16_t)f32_to_f16(v);
}
// Four consecutive results of storage dtype DT at p (vector store when aligned).
template <int DT> __device__ __forceinline__ void store4(void* base, int64_t idx, const f32x4& v) {
    if constexpr (DT == BSMM_F32) {
        *reinterpret_cast<f32x4*>((float*)base + idx) = v;
    } else {
        u32x2 w;
        w.x = to_storage16<DT>(v.x) | (to_storage16<DT>(v.y) << 16);
        w.y = to_storage16<DT>(v.z) | (to_storage16<DT>(v.w) << 16);
        *reinterpret_cast<u32x2*>((uint16_t*)base + idx) = w;
    }
}

// 16 zero bytes in device memory: a load whose lane has nothing to read is pointed
// here instead of being skipped or masked afterwards.  Loads are then issued
// unconditionally and nothing touches their value before it is consumed, so the
// compiler can count exactly how many loads are in flight.
__device__ __attribute__((aligned(16))) uint32_t kZero16[4] = {0u, 0u, 0u, 0u};   // global, never written

template <typename T> __device__ __forceinline__ const T* or_zero(bool ok, const T* p) {
    return ok ? p : reinterpret_cast<const T*>(kZero16);
}

template <int DT> __device__ __forceinline__ u32x4 load_vec(const typename Elt<DT>::T* p) {
    return *reinterpret_cast<const u32x4*>(p);
}
// VEC elements p[0], p[s], ..., packed in order; elements at index >= nvalid read as 0
// (their loads are pointed at kZero16, so every element load is always issued).
template <int DT>
__device__ __forceinline__ u32x4 load_strided(const typename Elt<DT>::T* p, int64_t s, int nvalid) {
    using T = typename Elt<DT>::T;
    u32x4 r;
    if constexpr (DT == BSMM_F32) {
        r.x = __float_as_uint(*or_zero<T>(nvalid > 0, p));
        r.y = __float_as_uint(*or_zero<T>(nvalid > 1, p + s));
        r.z = __float_as_uint(*or_zero<T>(nvalid > 2, p + 2 * s));
        r.w = __float_as_uint(*or_zero<T>(nvalid > 3, p + 3 * s));
    } else {
        uint32_t h[8];
#pragma unroll
        for (int v = 0; v < 8; v++) h[v] = (uint32_t)*or_zero<T>(v < nvalid, p + v * s);
        r.x = h[0] | (h[1] << 16);
        r.y = h[2] | (h[3] << 16);
        r.z = h[4] | (h[5] << 16);
        r.w = h[6] | (h[7] << 16);
    }
    return r;
}

// Operand fragment from a K-major LDS tile of 16-bit values (tile[k][col], `pitch`
// elements per row) with the gfx950 transposing LDS read.  Within each 16-lane group
// the instruction hands lane 4i+j the j-th 16-bit value at the addresses of lanes i,
// i+4, i+8, i+12 (as measured on the device).  Pointing lane m of group g at row
// 8g+4h+m/4, columns col0+4*(m%4).., the two reads (h = 0, 1) give lane (m, g) the
// values tile[8g + v][col0 + m], v = 0..7: the fragment layout of mma().
__device__ __forceinline__ u32x4 frag_tr16(const BSMM_LDS uint16_t* tile, int pitch, int col0, int lane) {
    const int m = lane & 15, g = lane >> 4;
    const BSMM_LDS uint16_t* p0 = tile + (8 * g + (m >> 2)) * pitch + col0 + 4 * (m & 3);
    const i16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((BSMM_LDS i16x4*)p0);
    const i16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((BSMM_LDS i16x4*)(p0 + 4 * pitch));
    const u32x2 ua = __builtin_bit_cast(u32x2, a), ub = __builtin_bit_cast(u32x2, b);
    u32x4 r;
    r.x = ua.x;
    r.y = ua.y;
    r.z = ub.x;
    r.w = ub.y;
    return r;
}

// Raw buffer loads: a scalar 128-bit descriptor (base, size in bytes) plus a 32-bit
// per-lane offset and a 32-bit scalar offset.  On gfx950 every dword whose
// voffset + soffset lies at or beyond the descriptor's size reads as zero without
// touching memory (measured on the device), so a whole load is switched off with a
// scalar offset of kOffOff and a lane with voffset kOffLane; both leave
// voffset + soffset below 2^32 as long as sizes stay below 2^31 bytes.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr uint32_t kOffLane = 0x80000000u;
constexpr uint32_t kOffOff = 0x7fffffffu;
constexpr uint64_t kMaxBufferBytes = 0x7fff0000ull;

__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ u32x4 bload128(rsrc_t r, uint32_t voff, uint32_t soff) {
    return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0));
}
__device__ __forceinline__ uint32_t bload32(rsrc_t r, uint32_t voff, uint32_t soff) {
    return __builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, 0);
}
__device__ __forceinline__ uint32_t bload16(rsrc_t r, uint32_t voff, uint32_t soff) {
    return (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(r, voff, soff, 0);
}

__device__ __forceinline__ void lds_store16(BSMM_LDS uint16_t* p, const u32x4& v) {
    *reinterpret_cast<BSMM_LDS u32x4*>(p) = v;
}

// Compiler-only barrier between a wave's LDS stores and its LDS loads of the same
// tile (the hardware executes one wave's LDS instructions in order).
__device__ __forceinline__ void wave_lds_order() { __atomic_signal_fence(__ATOMIC_SEQ_CST); }

// Workgroup -> (list index, minibatch tile).  Workgroups are dealt round-robin over
// the 8 XCDs; the minibatch tiles of one list get ids equal mod 8, so they run on one
// XCD and share its L2 copy of the list's weight blocks.
// With 8 or more minibatch tiles the deal flips: XCD x takes tiles x, x+8, ... of every
// list, so each XCD's L2 holds its own slice of the activations while all lists walk it
// (measured 20-27 % faster on the b=8, N=1024 shape, where activations are re-read by
// every list).
__device__ __forceinline__ void wg_decode(int bid, int nlist, int ntiles, int& li, int& nt) {
    if (ntiles == 1) {
        li = bid;
        nt = 0;
    } else if (ntiles >= 8) {
        const int xcd = bid & 7, slot = bid >> 3, tpx = (ntiles + 7) / 8;
        nt = (slot % tpx) * 8 + xcd;
        li = slot / tpx;
        if (nt >= ntiles) li = nlist;
    } else {
        const int xcd = bid & 7, slot = bid >> 3;
        nt = slot % ntiles;
        li = (slot / ntiles) * 8 + xcd;
    }
    if (li >= nlist) li = -1;
}

// Grid size for nlist lists x ntiles minibatch tiles in the wg_decode mapping.
inline int mm_grid(int nlist, int ntiles) {
    if (ntiles == 1) return nlist;
    if (ntiles >= 8) return 8 * nlist * ((ntiles + 7) / 8);
    return ((nlist + 7) / 8) * 8 * ntiles;
}

// Launch on `st` with explicit timing events (either may be null).
template <typename K, typename... Args>
static hipError_t launch_ev(K kernel, dim3 grid, dim3 block, hipStream_t st, void* e0, void* e1, Args... args) {
    if (e0 || e1)
        hipExtLaunchKernelGGL(kernel, grid, block, 0, st, (hipEvent_t)e0, (hipEvent_t)e1, 0, args...);
    else
        hipLaunchKernelGGL(kernel, grid, block, 0, st, args...);
    return hipGetLastError();
}

// Launch on `st`; when kernel timing is active the dispatch records start/stop events.
template <typename K, typename... Args>
static hipError_t launch(int pass, K kernel, dim3 grid, dim3 block, hipStream_t st, Args... args) {
    void *e0 = nullptr, *e1 = nullptr;
    prof_events(pass, &e0, &e1);
    if (e0)
        hipExtLaunchKernelGGL(kernel, grid, block, 0, st, (hipEvent_t)e0, (hipEvent_t)e1, 0, args...);
    else
        hipLaunchKernelGGL(kernel, grid, block, 0, st, args...);
    return hipGetLastError();
}

}  // namespace bsmm
