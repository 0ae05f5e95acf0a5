/*
 * bsmm.h -- C ABI of libbsmm, a block-sparse matrix multiply for AMD MI355X (gfx950).
 *
 * The operation is the one the kiteco/blocksparse README documents under
 * "API Documentation" › blocksparse.matmul › class BlocksparseMatMul:
 *
 *   layout  an R x S array of zeros and ones (BlocksparseMatMul.__init__, argument
 *           "layout").  Row c indexes the b-wide input feature blocks, column k the
 *           b-wide output feature blocks, so C = R*b inputs and K = S*b outputs.
 *   b       the block size, 8, 16 or 32 (__init__, argument "block_size").
 *   W       the weight, holding only the present blocks: shape (nnz, b, b)
 *           (w_shape), block id t being the t-th nonzero of the layout in row-major
 *           order (the (c,k) pair of an id is what block_coord returns).  Within a
 *           block, W[t][i][j] couples input feature c*b+i to output feature k*b+j.
 *   feature_axis  1: activations are (N, features), row-major; 0: (features, N)
 *           (__init__, argument "feature_axis"; N is the minibatch, as in the shape
 *           helpers i_shape(N) / o_shape(N)).
 *
 *   fprop   y  = x . W~        (BlocksparseMatMul.__call__)
 *   bprop   dx = dy . W~^T     (the gradient of __call__ with respect to its input)
 *   updat   dW[id(c,k)] = sum_t x_t[:, c-block]^T . dy_t[:, k-block], for present blocks
 *           only (the weight gradient, with dw_dtype; the sum over up to 8 steps that
 *           share W is what group_param_grads forms)
 *   identity_init  W[id(c,k)] = I_b when c == k, else 0 (identity_init with gpu=True)
 *
 * where W~ is the C x K matrix that is W's blocks on the present (c,k) and zero
 * elsewhere.  With feature_axis = 0 every activation is stored transposed; W's
 * storage does not change.
 *
 * Conventions for every call below:
 *   - Status codes are returned, never thrown; nothing aborts the process.  The
 *     text of the last failure on the calling thread is bsmm_last_error().
 *   - Device pointers are plain HIP device addresses (e.g. torch's data_ptr()).
 *     The caller owns every device buffer.  Each must be 16-byte aligned and
 *     dense in the layout stated; otherwise BSMM_ERR_ALIGNMENT / the result is
 *     undefined.
 *   - x, W, dy and their results share one storage dtype (BSMM_F32, BSMM_BF16,
 *     BSMM_F16).  Products accumulate in fp32; results are rounded to the storage
 *     dtype with round-to-nearest-even.
 *   - stream is a hipStream_t (NULL = the legacy default stream).  Kernels are
 *     enqueued asynchronously; no call synchronizes the device.
 *   - Every input activation and weight tensor must be at most 2 GiB - 64 KiB
 *     (2,147,418,112 bytes: the kernels read them with 32-bit offsets); larger ones are
 *     rejected with BSMM_ERR_UNSUPPORTED.  Outputs are written with 64-bit offsets.
 *   - N = 0: fprop and bprop do nothing and return BSMM_OK; updat writes dW = 0 (the
 *     empty sum).  Activation pointers may be NULL only when N = 0.
 *   - A handle is immutable after bsmm_create; it may be used from several host
 *     threads and streams at once.  Its look-up tables are copied to a device
 *     the first time a kernel call runs on that device: one hipMalloc and an
 *     asynchronous copy on that call's stream, from a host image the handle keeps.
 *     That first call must not be made while its stream is being captured into a
 *     HIP graph (it returns BSMM_ERR_UNSUPPORTED and enqueues nothing); later calls
 *     allocate nothing and may be captured.  (The same holds for the SparseProj
 *     and BlocksparseConv handles below.)
 */
#ifndef BSMM_H
#define BSMM_H

#include <stddef.h>
#include <stdint.h>

#if defined(__GNUC__)
#define BSMM_API __attribute__((visibility("default")))
#else
#define BSMM_API
#endif

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    BSMM_OK = 0,
    BSMM_ERR_INVALID_ARG = 1,   /* a size, enum or pointer argument is out of range */
    BSMM_ERR_UNSUPPORTED = 2,   /* a valid request this library does not implement */
    BSMM_ERR_ALIGNMENT = 3,     /* a device pointer is not 16-byte aligned */
    BSMM_ERR_DEVICE = 4,        /* a HIP runtime call failed */
    BSMM_ERR_OOM = 5            /* host or device allocation failed */
} bsmm_status;

/* BSMM_DTYPE_MAX_ENUM is not a dtype: it makes every int value a valid bsmm_dtype, so the
 * calls can reject an unknown code with BSMM_ERR_INVALID_ARG. */
typedef enum { BSMM_F32 = 0, BSMM_BF16 = 1, BSMM_F16 = 2, BSMM_DTYPE_MAX_ENUM = 0x7fffffff } bsmm_dtype;

typedef enum {
    BSMM_PASS_FPROP = 0,
    BSMM_PASS_BPROP = 1,
    BSMM_PASS_UPDAT = 2,
    BSMM_PASS_IDENTITY = 3,
    BSMM_PASS_LAYER_NORM = 4,
    BSMM_PASS_LAYER_NORM_GRAD = 5,
    BSMM_PASS_L2_NORMALIZE = 6,
    BSMM_PASS_L2_NORMALIZE_GRAD = 7,
    BSMM_PASS_PROJ_GATHER = 8,
    BSMM_PASS_PROJ_SCATTER = 9,
    BSMM_PASS_PROJ_SCATTER_ADD = 10,
    BSMM_PASS_PROJ_SCATTER_MUL = 11,
    BSMM_PASS_PROJ_GATHER_MUL = 12,
    BSMM_PASS_CONV_FPROP = 13,
    BSMM_PASS_CONV_BPROP = 14,
    BSMM_PASS_CONV_UPDAT = 15
} bsmm_pass;
#define BSMM_NUM_PASSES 16

typedef struct bsmm_plan* bsmm_handle;

/* Compile a layout into a handle (BlocksparseMatMul.__init__).
 *   layout        host array of R*S bytes, row-major, each 0 or 1; read during the call only.
 *   R, S          layout rows (input blocks) and columns (output blocks), each >= 1.
 *   block_size    8, 16 or 32.
 *   feature_axis  0 or 1.
 * An all-zero layout is valid (nnz = 0: outputs are zero).  Does not touch the GPU.
 * Errors: BSMM_ERR_INVALID_ARG for a NULL out/layout, R or S < 1, R*b or S*b above
 * 2^31-1, a block size outside {8,16,32}, feature_axis outside {0,1} or a layout
 * byte outside {0,1}; BSMM_ERR_OOM.  *out is set to NULL on failure. */
BSMM_API bsmm_status bsmm_create(bsmm_handle* out, const uint8_t* layout, int64_t R, int64_t S,
                        int block_size, int feature_axis);

/* Release a handle and its device tables.  NULL is ignored.  The caller must ensure
 * no kernel that uses the handle is still queued. */
BSMM_API void bsmm_destroy(bsmm_handle h);

/* w_shape: out = {nnz, b, b}. */
BSMM_API bsmm_status bsmm_w_shape(bsmm_handle h, int64_t out[3]);
/* i_shape(N): {N, C} for feature_axis 1, {C, N} for 0.  N >= 0. */
BSMM_API bsmm_status bsmm_i_shape(bsmm_handle h, int64_t N, int64_t out[2]);
/* o_shape(N): {N, K} for feature_axis 1, {K, N} for 0.  N >= 0. */
BSMM_API bsmm_status bsmm_o_shape(bsmm_handle h, int64_t N, int64_t out[2]);
/* block_coord: the layout coordinates (c, k) of block id `block` (0 <= block < nnz). */
BSMM_API bsmm_status bsmm_block_coord(bsmm_handle h, int64_t block, int64_t* c, int64_t* k);
/* Layout description: out = {R, S, b, feature_axis, nnz}. */
BSMM_API bsmm_status bsmm_plan_info(bsmm_handle h, int64_t out[5]);

/* Bytes of device workspace a pass needs for minibatch N and dtype.  Non-zero only for
 * updat with 32x32 blocks and 16-bit activations on layouts with dense 8x8-block tiles:
 * when the tiles are few, their contraction is split in parts whose fp32 partial sums
 * live in the workspace (parts x tiles x 64 x 4 KiB), and when there are enough tiles
 * for the tile kernel, the blocks outside the tiles have their contraction cut in eight
 * parts, also summed in fp32 in the workspace after the tiles' (8 x those blocks x
 * 4 KiB).  updat called with a smaller workspace splits only what it holds (the tiles'
 * parts first), and with a NULL one runs unsplit (correct, slower; the summation order,
 * and so the rounding, differs).  pass is a bsmm_pass value. */
BSMM_API bsmm_status bsmm_workspace_size(bsmm_handle h, int pass, int64_t N, bsmm_dtype dt, size_t* bytes);

/* fprop: y = x . W~.
 *   x  device, i_shape(N), dtype dt.    w  device, (nnz, b, b), dtype dt.
 *   y  device, o_shape(N), dtype dt; fully overwritten (columns of output blocks with
 *      no present block are written as zero).
 *   ws, ws_bytes  device workspace of at least bsmm_workspace_size bytes (may be NULL
 *      when that size is 0).
 * x and y must not overlap. */
BSMM_API bsmm_status bsmm_fprop(bsmm_handle h, const void* x, const void* w, void* y, int64_t N,
                       bsmm_dtype dt, void* ws, size_t ws_bytes, void* stream);

/* bprop: dx = dy . W~^T.
 *   dy device, o_shape(N); w device, (nnz, b, b); dx device, i_shape(N), fully
 *   overwritten.  All of dtype dt.  dy and dx must not overlap. */
BSMM_API bsmm_status bsmm_bprop(bsmm_handle h, const void* dy, const void* w, void* dx, int64_t N,
                       bsmm_dtype dt, void* ws, size_t ws_bytes, void* stream);

/* updat: dW[id] = sum over t < group of x_t[:, c-block]^T . dy_t[:, k-block], id = id(c,k).
 *   xs, dys  host arrays of `group` device pointers (1 <= group <= 8), each x_t of
 *            i_shape(N) and dy_t of o_shape(N), dtype dt; the host arrays are read
 *            during the call only.
 *   dw       device, (nnz, b, b), dtype dw_dt (BSMM_F32 is the default of the pages'
 *            dw_dtype; BSMM_BF16 / BSMM_F16 round the fp32 sum with RNE).  Overwritten,
 *            not accumulated into. */
BSMM_API bsmm_status bsmm_updat(bsmm_handle h, const void* const* xs, const void* const* dys, int group,
                       void* dw, int64_t N, bsmm_dtype dt, bsmm_dtype dw_dt,
                       void* ws, size_t ws_bytes, void* stream);

/* updat accumulating into dW: dW[id] += sum over t < group of x_t[:, c-block]^T .
 * dy_t[:, k-block].  Arguments, layouts, ownership and errors as bsmm_updat; dw is read
 * and written.  The fp32 sum of the call is added to the value dW holds (bf16 / f16
 * decoded exactly) and the total rounded once with RNE to dw_dt.  N = 0 leaves dW as it
 * is.  This is the weight gradient of a weight shared by more time steps than one
 * grouped call takes: the kiteco/blocksparse README ("API Documentation" ›
 * group_param_grads) combines the gradients of up to 8 time steps into one product, so
 * longer sequences add their groups' sums into one dW. */
BSMM_API bsmm_status bsmm_updat_accumulate(bsmm_handle h, const void* const* xs, const void* const* dys,
                                           int group, void* dw, int64_t N, bsmm_dtype dt, bsmm_dtype dw_dt,
                                           void* ws, size_t ws_bytes, void* stream);

/* updat for callers that cannot allocate device memory (code under HIP-graph capture,
 * tight serving loops, harnesses that forbid hipMalloc): the same result as bsmm_updat
 * (same kernels, bit for bit), with the split weight-gradient kernels' fp32 partial sums
 * in a fixed 128 MiB device array of the library instead of a caller workspace.  The
 * call makes no hipMalloc / hipFree and calls no allocating routine.
 *   Arguments as bsmm_updat without ws / ws_bytes.
 *   Errors as bsmm_updat, and BSMM_ERR_UNSUPPORTED when bsmm_workspace_size(h,
 *   BSMM_PASS_UPDAT, N, dt) exceeds 128 MiB, or when the handle's layout tables are not
 *   on the current device yet (they are uploaded by the first call of any other entry
 *   point on that device).
 * The array is one per GPU, held until the process ends, and shared by every call on
 * that GPU: calls that overlap in time on one GPU (other streams, other threads) race
 * on it and must be serialised by the caller.  Nothing in it needs to start at zero. */
BSMM_API bsmm_status bsmm_updat_noalloc(bsmm_handle h, const void* const* xs, const void* const* dys, int group,
                                        void* dw, int64_t N, bsmm_dtype dt, bsmm_dtype dw_dt, void* stream);

/* identity_init on the device: w (device, (nnz, b, b), dtype dt) is overwritten with
 * I_b for every present diagonal block (c == k) and zero for the other blocks. */
BSMM_API bsmm_status bsmm_identity_init(bsmm_handle h, void* w, bsmm_dtype dt, void* stream);

/* Static text for a status code. */
BSMM_API const char* bsmm_status_string(bsmm_status s);
/* Text of the last error raised on the calling thread ("" if none). */
BSMM_API const char* bsmm_last_error(void);

/* Name of the kernel family a pass would launch for these arguments (host only, no
 * GPU needed; the launch uses the same choice).  *name is a static string: "none" when
 * the call would launch nothing (N = 0, no blocks).  pass is a bsmm_pass value; group
 * is the updat group count (1..8; ignored by the other passes). */
BSMM_API bsmm_status bsmm_kernel_name(bsmm_handle h, int pass, int64_t N, int group, bsmm_dtype dt,
                                      const char** name);

/* Testing and tuning: make `pass` (fprop, bprop or updat) launch the kernel family
 * `name` (one of the names bsmm_kernel_name reports, e.g. "output_groups",
 * "dense_tiles") instead of the automatic choice.  A later call that the named family
 * cannot serve fails with BSMM_ERR_UNSUPPORTED and launches nothing.  NULL or ""
 * restores the automatic choice.  Unknown names give BSMM_ERR_INVALID_ARG.  This is a
 * set-up step: it must not race with calls on the same handle. */
BSMM_API bsmm_status bsmm_force_kernel(bsmm_handle h, int pass, const char* name);

/* Layout compiler output, for inspection and tests (host only, no GPU needed).
 *   which: 0 coords   (2*nnz:   c, k of every id, in id order)
 *          1 colptr   (S+1:     fprop segment starts, one per output block k)
 *          2 colent   (2*nnz:   fprop entries (c, id), ascending c within each k)
 *          3 rowptr   (R+1:     bprop segment starts, one per input block c)
 *          4 rowent   (2*nnz:   bprop entries (k, id), ascending k within each c)
 *          5 colorder (S:       output blocks by descending entry count, ties ascending)
 *          6 roworder (R:       input blocks by descending entry count, ties ascending)
 *          7 colwork  (4*S:     per output block in colorder: (k, start, length, 0))
 *          8 rowwork  (4*R:     per input block in roworder: (c, start, length, 0))
 *          9 ugroups  (4*groups: runs of <= 8 consecutive ids of one layout row, in id
 *                     order: (first id, count, c, 0); the weight-gradient work units)
 *         10 colrec   (S*stride: per output block in colorder, its colwork descriptor
 *                     then its first min(length, 1024) fprop entries (c, id), zero
 *                     padded; stride = 4 + 2*r, r = min(longest list, 1024) rounded
 *                     up to even, at least 2)
 *         11 rowrec   (the same for the bprop lists)
 *         12 cgptr    (block size 32 only, else empty: ceil(S/8)+1 offsets into cgent)
 *         13 cgent    (12 per entry: groups of 8 consecutive block columns; per group,
 *                     for every layout row c holding one of its blocks, ascending c:
 *                     c, mask (bit j: block (c, 8g+j) present), the 8 ids (0 where
 *                     absent), 0, 0)
 *         14 rgptr    (block size 32 only: ceil(R/8)+1 offsets into rgent)
 *         15 rgent    (the same for groups of 8 block rows, walking k ascending)
 *         16 utiles   (block size 32 only: 4 per weight-gradient tile, in super-blocks
 *                     of 4 x 8 tiles, row-major within and between super-blocks: first
 *                     block row, first block column, block count, index
 *                     of its first entry in utblk; tiles are 8x8 blocks of the layout
 *                     holding at least 16 blocks)
 *         17 utblk    (64 per tile: the ids of its 8x8 positions, row-major, -1 where
 *                     the layout is 0)
 *         18 urest    (4 per row group of the blocks outside those tiles, ascending
 *                     row then k; a row's blocks split into the fewest groups of at
 *                     most 4, sizes differing by at most 1: index of its first id in
 *                     urids, count, row, 1)
 *         19 urids    (the ids of those groups)
 *         20 stiles   (block size 8 or 16 only: 4 per weight-gradient tile of 256 x 256
 *                     features holding a block, in super-blocks of 4 x 8 tiles: first x
 *                     feature, first dy feature, index of its first entry in stids, 0)
 *         21 stplan   (8 per such tile and wave, 16 waves: the number of 16-feature
 *                     quads holding a block in the wave's quad row, their quad columns
 *                     ascending, one byte each, four per value from the low byte, zero
 *                     past the end, then the quad row, then 2 zeros; each row taken by
 *                     one wave, waves w, w+4, w+8, w+12 sharing one SIMD)
 *         22 stids    (per such tile, 256 quads row-major x the quad's blocks (1 for
 *                     16x16 blocks, 2 x 2 row-major for 8x8): block id or -1)
 * Copies min(cap, length) values into out (may be NULL when cap = 0) and the full
 * length into *len. */
BSMM_API bsmm_status bsmm_debug_lut(bsmm_handle h, int which, int64_t* out, int64_t cap, int64_t* len);

/* Layer norm over the feature axis, with an optional ReLU at the end ([README] "API
 * Documentation" › blocksparse.norms › layer_norm(x, g, b, axis=1, epsilon=1e-6,
 * relu=False): a layer norm for both activation layouts of the matmul above).
 * Per normalised vector -- a row of x (N, C) for axis = 1, a column of x (C, N) for
 * axis = 0 -- with mean and biased variance over its C features:
 *   y = (x - mean) * rstd * g + b,  rstd = 1/sqrt(var + epsilon),  then max(y, 0) if relu.
 * x, y: dense row-major in dtype dt (y may not alias x); g, b: float32[C] (gain, bias);
 * mean, rstd: float32[N] outputs for the gradient (both NULL to skip).  Statistics
 * and sums are fp32, in a fixed order (deterministic); y is rounded to nearest even.
 * ws: at least bsmm_layer_norm_workspace_size bytes (16-byte aligned; may be NULL when
 * that is 0), caller-owned scratch.  Asynchronous on hip_stream.
 * Errors: BSMM_ERR_INVALID_ARG (NULL tensor, N or C < 0, axis not 0/1, bad dtype,
 * epsilon < 0 or not finite, mean/rstd only one of them NULL, small workspace);
 * BSMM_ERR_ALIGNMENT (x or y not 16-byte aligned); BSMM_ERR_UNSUPPORTED (axis 1 with
 * C above 16384 for 16-bit or 8192 for fp32 storage, or a tensor above 2^31 elements);
 * BSMM_ERR_DEVICE.  Axis 0 also needs C <= 65535*128.  N = 0 or C = 0: no-op. */
BSMM_API bsmm_status bsmm_layer_norm_workspace_size(int64_t N, int64_t C, int axis, int grad, bsmm_dtype dt,
                                                    size_t* bytes);
BSMM_API bsmm_status bsmm_layer_norm(const void* x, const float* g, const float* b, void* y, float* mean,
                                     float* rstd, int64_t N, int64_t C, int axis, float epsilon, int relu,
                                     bsmm_dtype dt, void* ws, size_t ws_bytes, void* hip_stream);
/* Gradient of bsmm_layer_norm for upstream gradient dy (same layout and dtype as x),
 * from the forward's mean and rstd (not recomputed):
 *   dyr = dy, or dy * [xhat * g + b > 0] when relu,   xhat = (x - mean) * rstd,
 *   dx = rstd * (dyr*g - mean_C(dyr*g) - xhat * mean_C(dyr*g * xhat)),
 *   dg = sum over vectors of dyr * xhat,   db = sum over vectors of dyr   (float32[C]).
 * dx, dg, db are overwritten; ws as above (bsmm_layer_norm_workspace_size with
 * grad = 1).  Errors as for bsmm_layer_norm (dx, dy 16-byte aligned). */
BSMM_API bsmm_status bsmm_layer_norm_grad(const void* dy, const void* x, const float* g, const float* b,
                                          const float* mean, const float* rstd, void* dx, float* dg, float* db,
                                          int64_t N, int64_t C, int axis, int relu, bsmm_dtype dt, void* ws,
                                          size_t ws_bytes, void* hip_stream);

/* Weight normalisation of the stored blocks ([README] "API Documentation" ›
 * blocksparse.matmul › BlocksparseMatMul.l2_normalize(W, gain=None, epsilon=1e-6,
 * dtype): "to implement weight normalization").  Per output feature o = k*b + j
 * (column j of the blocks of block column k, i.e. one column of the masked C x K
 * weight):  n[o] = sqrt(max(sum of W^2 over that column's stored weights, epsilon)),
 * w_out = W * gain[o] / n[o] (gain 1 when gain is NULL).
 * w: (nnz, b, b) in w_dt; w_out: the same shape in out_dt (may not alias w); gain:
 * float32[K] or NULL; norms: float32[K] output or NULL.  Sums are fp32 in a fixed
 * order.  Errors: BSMM_ERR_INVALID_ARG (NULL handle / tensors, bad dtype, epsilon not
 * finite and > 0); BSMM_ERR_ALIGNMENT (w, w_out not 16-byte aligned);
 * BSMM_ERR_DEVICE.  nnz = 0: no-op. */
BSMM_API bsmm_status bsmm_l2_normalize(bsmm_handle h, const void* w, const float* gain, void* w_out, float* norms,
                                       float epsilon, bsmm_dtype w_dt, bsmm_dtype out_dt, void* hip_stream);
/* Gradient of bsmm_l2_normalize for the upstream gradient dy (same shape as w, dtype
 * dy_dt), with s[o] = the column's sum of dy * W:
 *   dw = gain[o]/n[o] * dy - [sum of squares > epsilon] * gain[o]*s[o]/n[o]^3 * W,
 *   dgain[o] = s[o] / n[o].
 * dw: float32 (nnz, b, b), overwritten; dgain: float32[K] or NULL.  Errors as above. */
BSMM_API bsmm_status bsmm_l2_normalize_grad(bsmm_handle h, const void* dy, const void* w, const float* gain,
                                            void* dw, float* dgain, float epsilon, bsmm_dtype dy_dt,
                                            bsmm_dtype w_dt, void* hip_stream);

/* ---- SparseProj (kiteco/blocksparse README, "API Documentation" › blocksparse.matmul ›
 * SparseProj(nhidden, nproj, proj_stride, block_size, gather_lut) with gather, scatter,
 * scatter_add and scatter_mul): projections between a dense activation of nhidden
 * features and a projected one of nproj features through a one-to-one feature map
 * lut[p] (the dense feature of projected feature p).  Activations are (N, features) for
 * feature_axis 1 and (features, N) for 0, dense and contiguous, 16-byte aligned device
 * buffers of one dtype.  The page gives no formulas; the readings:
 *   gather       y[n, p] = x[n, lut[p]]                                    y (N, nproj)
 *   scatter      y[n, lut[p]] = x[n, p], 0 at every dense feature not in lut  y (N, nhidden)
 *   scatter_add  z = x, then z[n, lut[p]] = x[n, lut[p]] + y[n, p]          z (N, nhidden)
 *   scatter_mul  z = x, then z[n, lut[p]] = x[n, lut[p]] * y[n, p]          z (N, nhidden)
 *   gather_mul   g[n, p] = a[n, lut[p]] * b[n, lut[p]]  (the y-gradient of scatter_mul)
 * Copies keep the stored bits; add and mul compute in fp32 and round once (RNE) to the
 * storage type.  Each output element is written once by one thread (the map is
 * one-to-one), so no op, forward or backward, uses atomics.  Calls are asynchronous on
 * `stream`; N = 0 is a no-op; errors as for the matmul calls (NULL or misaligned
 * pointers, bad dtype or feature_axis). */
typedef struct bsmm_proj_plan* bsmm_proj_handle;

/* Build the feature map.  gather_lut (host, nproj entries, read during the call): the
 * map itself; its entries must be distinct and in [0, nhidden) (BSMM_ERR_INVALID_ARG
 * otherwise); proj_stride and block_size are then ignored.  gather_lut NULL: the map is
 * nproj / block_size blocks of block_size consecutive dense features, block j starting
 * at j * proj_stride; nproj <= 0 means nhidden and proj_stride <= 0 means block_size;
 * nproj must be a multiple of block_size, proj_stride >= block_size, and the last block
 * must end within nhidden.  The handle owns the host map and its per-device copies. */
BSMM_API bsmm_status bsmm_proj_create(bsmm_proj_handle* out, int64_t nhidden, int64_t nproj, int64_t proj_stride,
                                      int64_t block_size, const int32_t* gather_lut);
/* Release the handle and its device copies (NULL-safe).  No call may be in flight. */
BSMM_API void bsmm_proj_destroy(bsmm_proj_handle h);
/* The dense and projected feature counts. */
BSMM_API bsmm_status bsmm_proj_info(bsmm_proj_handle h, int64_t* nhidden, int64_t* nproj);
/* The first min(cap, nproj) map entries into host array out. */
BSMM_API bsmm_status bsmm_proj_lut(bsmm_proj_handle h, int32_t* out, int64_t cap);
/* y = gather(x).  x and y must not overlap. */
BSMM_API bsmm_status bsmm_proj_gather(bsmm_proj_handle h, const void* x, void* y, int64_t N, int feature_axis,
                                      bsmm_dtype dt, void* stream);
/* y = scatter(x), every element of y written.  x and y must not overlap. */
BSMM_API bsmm_status bsmm_proj_scatter(bsmm_proj_handle h, const void* x, void* y, int64_t N, int feature_axis,
                                       bsmm_dtype dt, void* stream);
/* z = scatter_add(x, y).  z may be x (in place); y must not overlap z. */
BSMM_API bsmm_status bsmm_proj_scatter_add(bsmm_proj_handle h, const void* x, const void* y, void* z, int64_t N,
                                           int feature_axis, bsmm_dtype dt, void* stream);
/* z = scatter_mul(x, y).  z may be x (in place); y must not overlap z. */
BSMM_API bsmm_status bsmm_proj_scatter_mul(bsmm_proj_handle h, const void* x, const void* y, void* z, int64_t N,
                                           int feature_axis, bsmm_dtype dt, void* stream);
/* g = gather_mul(a, b): a, b (N, nhidden); g (N, nproj), not overlapping a or b. */
BSMM_API bsmm_status bsmm_proj_gather_mul(bsmm_proj_handle h, const void* a, const void* b, void* g, int64_t N,
                                          int feature_axis, bsmm_dtype dt, void* stream);

/* ---- BlocksparseConv (kiteco/blocksparse README, "API Documentation" › blocksparse.conv ›
 * BlocksparseConv(BCK, TRS, DHW, MPQ=None, strides, dilates, padding, edge_bias)): a
 * convolution whose filter exists only for blocks of channels.  Block b lists Bc input
 * channels C_b and Bk output channels K_b (the pages' BCK); its filter F[b] is
 * (Bc, T, R, S, Bk), F as a whole (nblocks, Bc, T, R, S, Bk) contiguous.  Blocks may
 * share channels; their contributions add.  The page gives no formulas; the readings:
 *   activations  I (N, C, D, H, W), O (N, K, M, P, Q), dense, contiguous, 16-byte aligned;
 *                1-D / 2-D images are 3-D with leading sizes of 1 (pass 1s).
 *   geometry     per dim with image X, filter F, stride st, dilation dl:
 *                SAME (padding 0): out = ceil(X/st), pad = max(0, (out-1)*st + (F-1)*dl + 1 - X) / 2;
 *                VALID (1): pad = 0, out = (X - (F-1)*dl - 1)/st + 1;
 *                explicit (2): pad = pads[d], out = (X + 2*pad - (F-1)*dl - 1)/st + 1.
 *   fprop        O[n, K_b[j], m, p, q] += sum over i, t, r, s of
 *                I[n, C_b[i], m*st-pad+t*dl, p*st-pad+r*dl, q*st-pad+s*dl] * F[b, i, t, r, s, j]
 *                over all blocks (positions outside the image read as 0); O fully written.
 *   bprop        dI = the gradient of fprop with respect to I for dO; dI fully written.
 *   updat        dF[b, i, t, r, s, j] = sum over n, m, p, q of I[...] * dO[n, K_b[j], m, p, q];
 *                dF float32, overwritten (N = 0 writes zeros).
 * Storage dtype dt for I, F, O, dO, dI (fp32 accumulation, RNE to 16-bit outputs).
 * edge_bias, MPQ (transposed convolution) and BlocksparseDeconv are not provided. */
typedef struct bsmm_conv_plan* bsmm_conv_handle;

/* Build a plan.  cidx (nblocks*Bc), kidx (nblocks*Bk): host channel lists, read during
 * the call; entries in [0, C) / [0, K), distinct within a block.  Bk <= 64.  TRS, DHW,
 * strides, dilates: 3 entries each, >= 1.  padding: 0 SAME, 1 VALID, 2 explicit (pads,
 * 3 entries >= 0).  BSMM_ERR_INVALID_ARG when the filter does not fit the padded image. */
BSMM_API bsmm_status bsmm_conv_create(bsmm_conv_handle* out, int64_t nblocks, int64_t Bc, int64_t Bk,
                                      const int32_t* cidx, const int32_t* kidx, int64_t C, int64_t K,
                                      const int64_t TRS[3], const int64_t DHW[3], const int64_t strides[3],
                                      const int64_t dilates[3], int padding, const int64_t pads[3]);
/* Release the plan and its device tables (NULL-safe).  No call may be in flight. */
BSMM_API void bsmm_conv_destroy(bsmm_conv_handle h);
/* Output image size (M, P, Q) and the leading pads of each dim. */
BSMM_API bsmm_status bsmm_conv_geometry(bsmm_conv_handle h, int64_t MPQ[3], int64_t pads[3]);
/* Which kernel family a conv pass (0 fprop, 1 bprop, 2 updat) launches for dtype dt
 * (host only): "matrix_core", "matrix_core_gather" or "direct".  Every matrix-core
 * fprop / bprop needs blocks with the same output channel list to form groups that
 * share no channel, the pass's output channels per block (Bk for fprop, Bc for bprop)
 * 16, 32 or 64, and the pass's input activation below 2 GiB (32-bit offsets).
 * "matrix_core" (the staged kernel) further needs 2-D or 1-D images, stride and
 * dilation 1, 16-bit storage, the contraction channels per block (Bc / Bk) a multiple
 * of 32 and (bprop) pads below the filter size.  "matrix_core_gather" takes every other
 * geometry (1-, 2- or 3-D, strides, dilations, any padding) and dtype, fp32 included;
 * its bprop needs Bk a multiple of 16 bytes' worth of values (4 fp32, 8 16-bit), and a
 * call whose filter is not 16-byte aligned takes the direct kernels.  updat:
 * "matrix_core" for 2-D or 1-D images, stride and dilation 1, 16-bit storage and Bc
 * and Bk multiples of 16 up to 64; "matrix_core_gather" for every other geometry and
 * dtype with Bc and Bk of 16, 32 or 64, and I and dO below 2 GiB.  Anything else takes
 * the direct kernels. */
BSMM_API bsmm_status bsmm_conv_kernel_name(bsmm_conv_handle h, int pass, bsmm_dtype dt, const char** name);
/* O = fprop(F, I). */
BSMM_API bsmm_status bsmm_conv_fprop(bsmm_conv_handle h, const void* F, const void* I, void* O, int64_t N,
                                     bsmm_dtype dt, void* stream);
/* dI = bprop(F, dO). */
BSMM_API bsmm_status bsmm_conv_bprop(bsmm_conv_handle h, const void* F, const void* dO, void* dI, int64_t N,
                                     bsmm_dtype dt, void* stream);
/* Device workspace bytes bsmm_conv_updat can use for N images (0: it uses none).  With
 * it either matrix-core filter gradient splits its contraction over the images into
 * parts whose fp32 partial sums live in the workspace, then adds them in part order. */
BSMM_API bsmm_status bsmm_conv_workspace_size(bsmm_conv_handle h, int64_t N, bsmm_dtype dt, size_t* bytes);
/* dF = updat(I, dO), float32.  ws, ws_bytes: device workspace of at least
 * bsmm_conv_workspace_size bytes, 16-byte aligned, or NULL / smaller (then unsplit:
 * correct, slower).  The workspace must not be in use by another call. */
BSMM_API bsmm_status bsmm_conv_updat(bsmm_conv_handle h, const void* I, const void* dO, float* dF, int64_t N,
                                     bsmm_dtype dt, void* ws, size_t ws_bytes, void* stream);

/* Kernel timing for measurement.  Between bsmm_profile_begin() and bsmm_profile_end()
 * every pass launched from the calling thread records HIP events around its kernels
 * (hipExtLaunchKernelGGL start/stop events, i.e. the dispatch's own timestamps).
 * bsmm_profile_end waits for those events and writes, per bsmm_pass index
 * 0..BSMM_NUM_PASSES-1, the summed milliseconds and the number of passes recorded
 * (arrays of BSMM_NUM_PASSES).  Errors:
 * BSMM_ERR_INVALID_ARG when not begun; BSMM_ERR_DEVICE. */
BSMM_API bsmm_status bsmm_profile_begin(void);
BSMM_API bsmm_status bsmm_profile_end(double ms[BSMM_NUM_PASSES], int64_t count[BSMM_NUM_PASSES]);

#ifdef __cplusplus
}
#endif

#endif /* BSMM_H */
