// HIP kernels for gfx950 (MI355X) and their host launchers.
//
// The three passes of the block-sparse product (kiteco/blocksparse README, "API
// Documentation" › blocksparse.matmul › BlocksparseMatMul.__call__ and its
// gradients) and identity_init (same section, identity_init with gpu=True).
//
// Every contraction runs on the matrix cores with 16x16 output tiles:
//   fp32        v_mfma_f32_16x16x4_f32   (4 per K-step of 16)
//   bf16 / f16  v_mfma_f32_16x16x32_{bf16,f16} (1 per K-step of 32)
// accumulating in fp32.  A lane l of a wave holds, for a 16-row operand tile, row
// (l % 16) and a group of VEC consecutive contraction indices selected by (l / 16);
// both operands of one product use the same lane -> contraction-index map, so the
// order in which the hardware walks K inside an instruction does not matter.  The
// 16x16 result sits in lane l as rows 4*(l/16)+v, v < 4, of column l % 16.
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include "bsmm_internal.h"
#include "kernels.h"

namespace bsmm {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

template <int DT> struct Elt;
template <> struct Elt<BSMM_F32> { using T = float; static constexpr int VEC = 4; };
template <> struct Elt<BSMM_BF16> { using T = uint16_t; static constexpr int VEC = 8; };
template <> struct Elt<BSMM_F16> { using T = uint16_t; static constexpr int VEC = 8; };

// acc (16x16) += A (16 x 4*VEC) . B (4*VEC x 16), fragments as described above.
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

// fp32 -> storage, round to nearest even.
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);   // NaN stays NaN
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}
__device__ __forceinline__ uint16_t f32_to_f16(float f) {
    _Float16 h = (_Float16)f;   // v_cvt_f16_f32, default round-to-nearest-even mode
    return __builtin_bit_cast(uint16_t, h);
}
__device__ __forceinline__ void store_elt(void* base, int64_t idx, float v, int dt) {
    if (dt == BSMM_F32)
        ((float*)base)[idx] = v;
    else if (dt == BSMM_BF16)
        ((uint16_t*)base)[idx] = f32_to_bf16(v);
    else
        ((uint16_t*)base)[idx] = f32_to_f16(v);
}

// VEC contiguous elements (16 bytes, 16-byte aligned).
template <int DT> __device__ __forceinline__ u32x4 load_vec(const typename Elt<DT>::T* p) {
    return *reinterpret_cast<const u32x4*>(p);
}
// VEC elements p[0], p[s], p[2s], ... packed in K order; elements at index >= nvalid read as 0.
template <int DT>
__device__ __forceinline__ u32x4 load_strided(const typename Elt<DT>::T* p, int64_t s, int nvalid) {
    u32x4 r = {0u, 0u, 0u, 0u};
    if constexpr (DT == BSMM_F32) {
        if (nvalid > 0) r.x = __float_as_uint(p[0]);
        if (nvalid > 1) r.y = __float_as_uint(p[s]);
        if (nvalid > 2) r.z = __float_as_uint(p[2 * s]);
        if (nvalid > 3) r.w = __float_as_uint(p[3 * s]);
    } else {
        uint32_t h[8];
#pragma unroll
        for (int v = 0; v < 8; v++) h[v] = (v < nvalid) ? (uint32_t)p[v * s] : 0u;
        r.x = h[0] | (h[1] << 16);
        r.y = h[2] | (h[3] << 16);
        r.z = h[4] | (h[5] << 16);
        r.w = h[6] | (h[7] << 16);
    }
    return r;
}

// Workgroup -> (list index, N tile).  Workgroups are dealt round-robin over the
// 8 XCDs, so the N tiles of one output block are given ids that are equal mod 8:
// they run on one XCD and share its L2 copy of the weight blocks.
__device__ __forceinline__ void wg_decode(int bid, int nlist, int ntiles, int& li, int& nt) {
    if (ntiles == 1) {
        li = bid;
        nt = 0;
    } else {
        const int xcd = bid & 7, slot = bid >> 3;
        nt = slot % ntiles;
        li = (slot / ntiles) * 8 + xcd;
    }
    if (li >= nlist) li = -1;
}

// ---------------------------------------------------------------------------------
// fprop / bprop: out[:, o-block] = sum over the list of o of in[:, blk-block] . Wop
//   fprop: list = column o of the layout (entries (c, id)), Wop[p][q] = W[id][p][q]
//   bprop: list = row o (entries (k, id)),                  Wop[p][q] = W[id][q][p]
// A workgroup computes an NT x b tile (NT minibatch rows) of one output block.  Its
// 4 waves split the NT rows (WM) and/or the list's contraction steps (WK); WK partial
// sums are added in wave order through LDS, so results are deterministic.
template <int DT, int B, int FA, bool TW, int MT, int WM, int WK>
__global__ __launch_bounds__(256) void mm_kernel(MMArgs a) {
    using T = typename Elt<DT>::T;
    constexpr int VEC = Elt<DT>::VEC, KS = 4 * VEC;
    constexpr int QT = (B + 15) / 16;
    constexpr int NT = 16 * MT * WM;
    static_assert(WM * WK == 4, "four waves");
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int wm = wave % WM, wk = wave / WM;
    const int r16 = lane & 15, g = lane >> 4;

    int li, nt;
    wg_decode(blockIdx.x, a.nout, a.ntiles, li, nt);
    if (li < 0) return;   // whole workgroup leaves together
    const int o = a.order[li];
    const int beg = a.ptr[o], len = a.ptr[o + 1] - beg;
    const int64_t N = a.N;
    const int64_t n0 = (int64_t)nt * NT + wm * (16 * MT);
    const int nsteps = (len * B + KS - 1) / KS;
    const T* __restrict__ in = (const T*)a.in;
    const T* __restrict__ w = (const T*)a.w;

    f32x4 acc[MT][QT];
#pragma unroll
    for (int i = 0; i < MT; i++)
#pragma unroll
        for (int j = 0; j < QT; j++) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    for (int s = wk; s < nsteps; s += WK) {
        const int K0 = s * KS + g * VEC;
        const int e = K0 / B, p0 = K0 % B;
        const bool ev = e < len;
        int blk = 0, id = 0;
        if (ev) {
            blk = a.ent[2 * (beg + e)];
            id = a.ent[2 * (beg + e) + 1];
        }
        u32x4 xf[MT], wf[QT];
#pragma unroll
        for (int mt = 0; mt < MT; mt++) {
            const int64_t nr = n0 + mt * 16 + r16;
            xf[mt] = u32x4{0u, 0u, 0u, 0u};
            if (ev && nr < N) {
                if constexpr (FA == 1)
                    xf[mt] = load_vec<DT>(in + nr * a.fin + (int64_t)blk * B + p0);
                else
                    xf[mt] = load_strided<DT>(in + ((int64_t)blk * B + p0) * N + nr, N, VEC);
            }
        }
#pragma unroll
        for (int qt = 0; qt < QT; qt++) {
            const int q = qt * 16 + r16;
            wf[qt] = u32x4{0u, 0u, 0u, 0u};
            if (ev && q < B) {
                const T* wb = w + (int64_t)id * B * B;
                if constexpr (TW)
                    wf[qt] = load_vec<DT>(wb + q * B + p0);
                else
                    wf[qt] = load_strided<DT>(wb + p0 * B + q, B, VEC);
            }
        }
#pragma unroll
        for (int mt = 0; mt < MT; mt++)
#pragma unroll
            for (int qt = 0; qt < QT; qt++) {
                if constexpr (FA == 1)
                    mma<DT>(acc[mt][qt], xf[mt], wf[qt]);   // D[n][q]
                else
                    mma<DT>(acc[mt][qt], wf[qt], xf[mt]);   // D[q][n]
            }
    }

    if constexpr (WK > 1) {
        __shared__ f32x4 red[WM][WK - 1][MT * QT][64];
        if (wk > 0) {
#pragma unroll
            for (int i = 0; i < MT; i++)
#pragma unroll
                for (int j = 0; j < QT; j++) red[wm][wk - 1][i * QT + j][lane] = acc[i][j];
        }
        __syncthreads();
        if (wk != 0) return;
#pragma unroll
        for (int r = 0; r < WK - 1; r++)
#pragma unroll
            for (int i = 0; i < MT; i++)
#pragma unroll
                for (int j = 0; j < QT; j++) acc[i][j] += red[wm][r][i * QT + j][lane];
    }

#pragma unroll
    for (int mt = 0; mt < MT; mt++)
#pragma unroll
        for (int qt = 0; qt < QT; qt++)
#pragma unroll
            for (int v = 0; v < 4; v++) {
                if constexpr (FA == 1) {
                    const int64_t n = n0 + mt * 16 + 4 * g + v;
                    const int q = qt * 16 + r16;
                    if (n < N && q < B) store_elt(a.out, n * a.fout + (int64_t)o * B + q, acc[mt][qt][v], DT);
                } else {
                    const int q = qt * 16 + 4 * g + v;
                    const int64_t n = n0 + mt * 16 + r16;
                    if (n < N && q < B) store_elt(a.out, ((int64_t)o * B + q) * N + n, acc[mt][qt][v], DT);
                }
            }
}

// ---------------------------------------------------------------------------------
// updat: dW[id][p][q] = sum_t sum_n x_t[n, c*B+p] . dy_t[n, k*B+q]; one wave per block,
// the contraction runs over the minibatch.  Each block has exactly one writer.
template <int DT, int B, int FA>
__global__ __launch_bounds__(256) void updat_kernel(UpArgs a) {
    using T = typename Elt<DT>::T;
    constexpr int VEC = Elt<DT>::VEC, KS = 4 * VEC;
    constexpr int PT = (B + 15) / 16;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int r16 = lane & 15, g = lane >> 4;
    const int id = blockIdx.x * 4 + wave;
    if (id >= a.nnz) return;   // no workgroup barrier below
    const int c = a.coords[2 * id], k = a.coords[2 * id + 1];
    const int64_t N = a.N;
    const bool vec_ok = (FA == 0) && (N % VEC == 0);

    f32x4 acc[PT][PT];
#pragma unroll
    for (int i = 0; i < PT; i++)
#pragma unroll
        for (int j = 0; j < PT; j++) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    for (int t = 0; t < a.G; t++) {
        const T* __restrict__ x = (const T*)a.xs[t];
        const T* __restrict__ dy = (const T*)a.dys[t];
        for (int64_t nb = 0; nb < N; nb += KS) {
            const int64_t nk = nb + g * VEC;
            const int nval = (int)((N - nk) < VEC ? (N - nk > 0 ? N - nk : 0) : VEC);
            u32x4 af[PT], bf[PT];
#pragma unroll
            for (int pt = 0; pt < PT; pt++) {
                const int p = pt * 16 + r16;
                af[pt] = u32x4{0u, 0u, 0u, 0u};
                bf[pt] = u32x4{0u, 0u, 0u, 0u};
                if (p < B && nval > 0) {
                    if constexpr (FA == 1) {
                        af[pt] = load_strided<DT>(x + nk * a.C + (int64_t)c * B + p, a.C, nval);
                        bf[pt] = load_strided<DT>(dy + nk * a.K + (int64_t)k * B + p, a.K, nval);
                    } else {
                        const T* xp = x + ((int64_t)c * B + p) * N + nk;
                        const T* dp = dy + ((int64_t)k * B + p) * N + nk;
                        if (vec_ok && nval == VEC) {
                            af[pt] = load_vec<DT>(xp);
                            bf[pt] = load_vec<DT>(dp);
                        } else {
                            af[pt] = load_strided<DT>(xp, 1, nval);
                            bf[pt] = load_strided<DT>(dp, 1, nval);
                        }
                    }
                }
            }
#pragma unroll
            for (int pt = 0; pt < PT; pt++)
#pragma unroll
                for (int qt = 0; qt < PT; qt++) mma<DT>(acc[pt][qt], af[pt], bf[qt]);   // D[p][q]
        }
    }
    const int64_t base = (int64_t)id * B * B;
#pragma unroll
    for (int pt = 0; pt < PT; pt++)
#pragma unroll
        for (int qt = 0; qt < PT; qt++)
#pragma unroll
            for (int v = 0; v < 4; v++) {
                const int p = pt * 16 + 4 * g + v, q = qt * 16 + r16;
                if (p < B && q < B) store_elt(a.dw, base + p * B + q, acc[pt][qt][v], a.dwdt);
            }
}

// ---------------------------------------------------------------------------------
// identity_init: W[id] = I_b if the block is diagonal (c == k), else zero.
__global__ __launch_bounds__(256) void identity_kernel(void* w, const int32_t* coords, int64_t nnz, int B, int dt) {
    const int64_t total = nnz * B * B;
    for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < total;
         i += (int64_t)gridDim.x * blockDim.x) {
        const int64_t id = i / (B * B);
        const int r = (int)(i % (B * B));
        const bool one = coords[2 * id] == coords[2 * id + 1] && (r / B) == (r % B);
        store_elt(w, i, one ? 1.0f : 0.0f, dt);
    }
}

// ---------------------------------------------------------------------------------
// host launchers
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

static int mm_grid(int nlist, int ntiles) {
    if (ntiles == 1) return nlist;
    return ((nlist + 7) / 8) * 8 * ntiles;
}

template <int DT, int B, int FA, bool TW>
static hipError_t launch_mm_t(MMArgs a, hipStream_t st, int pass) {
    if (a.N <= 64) {
        constexpr int MT = 1, WM = 1, WK = 4, NT = 16 * MT * WM;
        a.ntiles = (int)((a.N + NT - 1) / NT);
        return launch(pass, mm_kernel<DT, B, FA, TW, MT, WM, WK>, dim3(mm_grid(a.nout, a.ntiles)), dim3(256), st, a);
    } else {
        constexpr int MT = 2, WM = 4, WK = 1, NT = 16 * MT * WM;
        a.ntiles = (int)((a.N + NT - 1) / NT);
        return launch(pass, mm_kernel<DT, B, FA, TW, MT, WM, WK>, dim3(mm_grid(a.nout, a.ntiles)), dim3(256), st, a);
    }
}

template <int DT, bool TW>
static hipError_t launch_mm_dt(MMArgs a, int b, int fa, hipStream_t st, int pass) {
    switch (b * 2 + fa) {
    case 16: return launch_mm_t<DT, 8, 0, TW>(a, st, pass);
    case 17: return launch_mm_t<DT, 8, 1, TW>(a, st, pass);
    case 32: return launch_mm_t<DT, 16, 0, TW>(a, st, pass);
    case 33: return launch_mm_t<DT, 16, 1, TW>(a, st, pass);
    case 64: return launch_mm_t<DT, 32, 0, TW>(a, st, pass);
    case 65: return launch_mm_t<DT, 32, 1, TW>(a, st, pass);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_mm(const MMArgs& a, int dt, int b, int fa, bool transw, void* stream, int pass) {
    hipStream_t st = (hipStream_t)stream;
    if (a.nout == 0) return hipSuccess;
    switch (dt * 2 + (transw ? 1 : 0)) {
    case 0: return launch_mm_dt<BSMM_F32, false>(a, b, fa, st, pass);
    case 1: return launch_mm_dt<BSMM_F32, true>(a, b, fa, st, pass);
    case 2: return launch_mm_dt<BSMM_BF16, false>(a, b, fa, st, pass);
    case 3: return launch_mm_dt<BSMM_BF16, true>(a, b, fa, st, pass);
    case 4: return launch_mm_dt<BSMM_F16, false>(a, b, fa, st, pass);
    case 5: return launch_mm_dt<BSMM_F16, true>(a, b, fa, st, pass);
    }
    return hipErrorInvalidValue;
}

template <int DT>
static hipError_t launch_updat_dt(const UpArgs& a, int b, int fa, hipStream_t st) {
    const dim3 grid((a.nnz + 3) / 4), block(256);
    switch (b * 2 + fa) {
    case 16: return launch(BSMM_PASS_UPDAT, updat_kernel<DT, 8, 0>, grid, block, st, a);
    case 17: return launch(BSMM_PASS_UPDAT, updat_kernel<DT, 8, 1>, grid, block, st, a);
    case 32: return launch(BSMM_PASS_UPDAT, updat_kernel<DT, 16, 0>, grid, block, st, a);
    case 33: return launch(BSMM_PASS_UPDAT, updat_kernel<DT, 16, 1>, grid, block, st, a);
    case 64: return launch(BSMM_PASS_UPDAT, updat_kernel<DT, 32, 0>, grid, block, st, a);
    case 65: return launch(BSMM_PASS_UPDAT, updat_kernel<DT, 32, 1>, grid, block, st, a);
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

hipError_t launch_identity(void* w, const int32_t* coords, int64_t nnz, int b, int dt, void* stream) {
    if (nnz == 0) return hipSuccess;
    const int64_t total = nnz * b * b;
    int64_t blocks = (total + 255) / 256;
    if (blocks > 65536) blocks = 65536;
    return launch(BSMM_PASS_IDENTITY, identity_kernel, dim3((unsigned)blocks), dim3(256), (hipStream_t)stream, w,
                  coords, nnz, b, dt);
}

}  // namespace bsmm
