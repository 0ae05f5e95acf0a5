// identity_init on the device (kiteco/blocksparse README, "API Documentation" ›
// blocksparse.matmul › identity_init with gpu=True): every present block (c, k) with
// c == k becomes the b x b identity, every other block zero.
#include "common.h"

namespace bsmm {

// One thread per 16-byte chunk of W; a chunk never crosses a block row because a row
// holds b >= 8 elements and a chunk 4 (fp32) or 8 (16-bit).
template <int DT>
__global__ __launch_bounds__(256) void identity_kernel(u32x4* w, const int32_t* coords, int64_t nchunks,
                                                       int log2_chunks_per_block, int B) {
    constexpr int E = 16 / (DT == BSMM_F32 ? 4 : 2);   // elements per chunk
    for (int64_t ch = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; ch < nchunks;
         ch += (int64_t)gridDim.x * blockDim.x) {
        const int64_t id = ch >> log2_chunks_per_block;
        const int r = (int)(ch - (id << log2_chunks_per_block)) * E;   // element offset in the block
        const int i = r / B, j0 = r % B;
        const bool diag = coords[2 * id] == coords[2 * id + 1];
        u32x4 v = {0u, 0u, 0u, 0u};
        if (diag && i >= j0 && i < j0 + E) {
            const int e = i - j0;   // which element of the chunk is the one
            if constexpr (DT == BSMM_F32) {
                v[e] = 0x3f800000u;
            } else {
                const uint32_t one = DT == BSMM_BF16 ? 0x3f80u : 0x3c00u;
                v[e >> 1] = one << (16 * (e & 1));
            }
        }
        w[ch] = v;
    }
}

hipError_t launch_identity(void* w, const int32_t* coords, int64_t nnz, int b, int dt, void* stream) {
    if (nnz == 0) return hipSuccess;
    const int esize = dt == BSMM_F32 ? 4 : 2;
    const int cpb = b * b * esize / 16;   // power of two
    int lg = 0;
    while ((1 << lg) < cpb) lg++;
    const int64_t nchunks = nnz * cpb;
    int64_t blocks = (nchunks + 255) / 256;
    if (blocks > 8192) blocks = 8192;
    hipStream_t st = (hipStream_t)stream;
    switch (dt) {
    case BSMM_F32:
        return launch(BSMM_PASS_IDENTITY, identity_kernel<BSMM_F32>, dim3((unsigned)blocks), dim3(256), st,
                      (u32x4*)w, coords, nchunks, lg, b);
    case BSMM_BF16:
        return launch(BSMM_PASS_IDENTITY, identity_kernel<BSMM_BF16>, dim3((unsigned)blocks), dim3(256), st,
                      (u32x4*)w, coords, nchunks, lg, b);
    case BSMM_F16:
        return launch(BSMM_PASS_IDENTITY, identity_kernel<BSMM_F16>, dim3((unsigned)blocks), dim3(256), st,
                      (u32x4*)w, coords, nchunks, lg, b);
    }
    return hipErrorInvalidValue;
}

}  // namespace bsmm
