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
    if (threadIdx.x < a.Bk) {
        const int j = threadIdx.x;
        const float v = ((part[0][j] + part[1][j]) + part[2][j]) + part[3][j];
        ((float*)a.out)[(int64_t)row * a.Bk + j] = v;
    }
}

template <int DT>
static hipError_t launch_conv_dt(const ConvArgs& a, int pass, hipStream_t st) {
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
