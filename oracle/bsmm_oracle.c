/*
 * CPU oracle for the block-sparse matrix multiply -- TEST INFRASTRUCTURE ONLY.
 *
 * Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
 * load this file's library.  The product path (libbsmm.so and its Python binding)
 * never calls it and shares no code, header, table or helper with it.
 *
 * What it computes (kiteco/blocksparse README, "API Documentation" ›
 * blocksparse.matmul › class BlocksparseMatMul):
 *   The layout L is an R x S array of zeros and ones (__init__, "layout"); block
 *   (c, k) is present when L[c][k] = 1, c indexing the input feature blocks and k
 *   the output feature blocks (block_coord returns "(c,k)").  The weight holds
 *   only the present blocks, each a dense b x b array, in the order of the block
 *   ids (w_shape; read here as (nnz, b, b), ids numbered by a row-major scan of
 *   the nonzeros of L).  Activations are (N, C) for feature_axis = 1 and (C, N)
 *   for feature_axis = 0 (__init__, "feature_axis"); C = R*b, K = S*b.
 *
 *   fprop  (__call__, y = I . W):
 *       y[n, k*b+j]  = sum over c with L[c][k]=1, over i < b:  x[n, c*b+i] * W[id(c,k)][i][j]
 *   bprop  (gradient of __call__ with respect to I):
 *       dx[n, c*b+i] = sum over k with L[c][k]=1, over j < b:  dy[n, k*b+j] * W[id(c,k)][i][j]
 *   updat  (gradient with respect to W, dw_dtype; group_param_grads sums steps):
 *       dW[id(c,k)][i][j] = sum over steps t < G, over n < N:   x_t[n, c*b+i] * dy_t[n, k*b+j]
 *   identity_init: W[id(c,k)] = the b x b identity when c == k, zero otherwise.
 *   With feature_axis = 0 the activation index [n, f] reads [f, n]; nothing else
 *   changes.
 *
 * Arithmetic: every stored value is decoded exactly to double (fp32, bfloat16 and
 * IEEE binary16 all embed exactly in binary64) and every sum is accumulated in
 * double in the order written above.  Results are returned in double.
 *
 * OpenMP splits the outermost loop over output blocks; no sum is split across
 * threads, so the results do not depend on the thread count.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { ORC_F32 = 0, ORC_BF16 = 1, ORC_F16 = 2 };

/* bfloat16: the upper 16 bits of an IEEE binary32. */
static double decode_bf16(uint16_t h) {
    uint32_t u = ((uint32_t)h) << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* IEEE 754 binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits. */
static double decode_f16(uint16_t h) {
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 0x1f;
    int m = h & 0x3ff;
    double v;
    if (e == 0)
        v = ldexp((double)m, -24);              /* zero and subnormals: m * 2^-24 */
    else if (e == 31)
        v = (m == 0) ? INFINITY : NAN;
    else
        v = ldexp((double)(m + 1024), e - 25);  /* (1 + m/1024) * 2^(e-15) */
    return sign ? -v : v;
}

double orc_decode(const void* base, int64_t idx, int dt) {
    switch (dt) {
    case ORC_F32: return (double)((const float*)base)[idx];
    case ORC_BF16: return decode_bf16(((const uint16_t*)base)[idx]);
    case ORC_F16: return decode_f16(((const uint16_t*)base)[idx]);
    default: return NAN;
    }
}

int orc_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Block ids: a row-major scan over L; id_of[c*S+k] = id or -1 when absent. */
static int64_t* make_ids(const uint8_t* L, int64_t R, int64_t S, int64_t* nnz_out) {
    int64_t* id_of = (int64_t*)malloc((size_t)(R * S) * sizeof(int64_t));
    if (!id_of) return NULL;
    int64_t next = 0;
    for (int64_t c = 0; c < R; c++)
        for (int64_t k = 0; k < S; k++)
            id_of[c * S + k] = L[c * S + k] ? next++ : -1;
    if (nnz_out) *nnz_out = next;
    return id_of;
}

int64_t orc_nnz(const uint8_t* L, int64_t R, int64_t S) {
    int64_t n = 0;
    for (int64_t t = 0; t < R * S; t++) n += L[t] != 0;
    return n;
}

/* Activation element [n, f] of a tensor with F features (fa=1: (N,F); fa=0: (F,N)). */
static inline int64_t act_index(int fa, int64_t N, int64_t F, int64_t n, int64_t f) {
    return fa ? n * F + f : f * N + n;
}

static int bad_args(const uint8_t* L, int64_t R, int64_t S, int b, int fa, int dt) {
    return !L || R < 1 || S < 1 || b < 1 || (fa != 0 && fa != 1) || dt < ORC_F32 || dt > ORC_F16;
}

int orc_fprop(const uint8_t* L, int64_t R, int64_t S, int b, int fa, int dt,
              const void* x, const void* w, int64_t N, double* y) {
    if (bad_args(L, R, S, b, fa, dt) || N < 0 || (N > 0 && (!x || !y))) return -1;
    const int64_t C = R * b, K = S * b;
    int64_t* id_of = make_ids(L, R, S, NULL);
    if (!id_of) return -2;
#pragma omp parallel for schedule(dynamic)
    for (int64_t k = 0; k < S; k++)
        for (int64_t n = 0; n < N; n++)
            for (int64_t j = 0; j < b; j++) {
                double acc = 0.0;
                for (int64_t c = 0; c < R; c++) {
                    int64_t id = id_of[c * S + k];
                    if (id < 0) continue;
                    for (int64_t i = 0; i < b; i++)
                        acc += orc_decode(x, act_index(fa, N, C, n, c * b + i), dt) *
                               orc_decode(w, (id * b + i) * b + j, dt);
                }
                y[act_index(fa, N, K, n, k * b + j)] = acc;
            }
    free(id_of);
    return 0;
}

int orc_bprop(const uint8_t* L, int64_t R, int64_t S, int b, int fa, int dt,
              const void* dy, const void* w, int64_t N, double* dx) {
    if (bad_args(L, R, S, b, fa, dt) || N < 0 || (N > 0 && (!dy || !dx))) return -1;
    const int64_t C = R * b, K = S * b;
    int64_t* id_of = make_ids(L, R, S, NULL);
    if (!id_of) return -2;
#pragma omp parallel for schedule(dynamic)
    for (int64_t c = 0; c < R; c++)
        for (int64_t n = 0; n < N; n++)
            for (int64_t i = 0; i < b; i++) {
                double acc = 0.0;
                for (int64_t k = 0; k < S; k++) {
                    int64_t id = id_of[c * S + k];
                    if (id < 0) continue;
                    for (int64_t j = 0; j < b; j++)
                        acc += orc_decode(dy, act_index(fa, N, K, n, k * b + j), dt) *
                               orc_decode(w, (id * b + i) * b + j, dt);
                }
                dx[act_index(fa, N, C, n, c * b + i)] = acc;
            }
    free(id_of);
    return 0;
}

/* dW for the blocks listed in ids[0..nids) (all nnz blocks in id order when ids is
 * NULL); out holds one b x b block per listed id, in the order listed. */
int orc_updat(const uint8_t* L, int64_t R, int64_t S, int b, int fa, int dt,
              const void* const* xs, const void* const* dys, int G, int64_t N,
              const int64_t* ids, int64_t nids, double* dw) {
    if (bad_args(L, R, S, b, fa, dt) || G < 1 || N < 0 || !xs || !dys || !dw) return -1;
    const int64_t C = R * b, K = S * b;
    int64_t nnz = 0;
    int64_t* id_of = make_ids(L, R, S, &nnz);
    if (!id_of) return -2;
    /* coordinates of every id, from the same scan */
    int64_t* cc = (int64_t*)malloc((size_t)(nnz > 0 ? nnz : 1) * sizeof(int64_t));
    int64_t* kk = (int64_t*)malloc((size_t)(nnz > 0 ? nnz : 1) * sizeof(int64_t));
    if (!cc || !kk) { free(id_of); free(cc); free(kk); return -2; }
    for (int64_t c = 0; c < R; c++)
        for (int64_t k = 0; k < S; k++)
            if (id_of[c * S + k] >= 0) { cc[id_of[c * S + k]] = c; kk[id_of[c * S + k]] = k; }
    if (!ids) nids = nnz;
    int rc = 0;
    for (int64_t t = 0; t < nids; t++)
        if (ids && (ids[t] < 0 || ids[t] >= nnz)) rc = -1;
    if (rc == 0) {
#pragma omp parallel for schedule(dynamic)
        for (int64_t t = 0; t < nids; t++) {
            int64_t id = ids ? ids[t] : t;
            int64_t c = cc[id], k = kk[id];
            for (int64_t i = 0; i < b; i++)
                for (int64_t j = 0; j < b; j++) {
                    double acc = 0.0;
                    for (int g = 0; g < G; g++)
                        for (int64_t n = 0; n < N; n++)
                            acc += orc_decode(xs[g], act_index(fa, N, C, n, c * b + i), dt) *
                                   orc_decode(dys[g], act_index(fa, N, K, n, k * b + j), dt);
                    dw[(t * b + i) * b + j] = acc;
                }
        }
    }
    free(id_of); free(cc); free(kk);
    return rc;
}

int orc_identity(const uint8_t* L, int64_t R, int64_t S, int b, double* w) {
    if (!L || R < 1 || S < 1 || b < 1 || !w) return -1;
    int64_t id = 0;
    for (int64_t c = 0; c < R; c++)
        for (int64_t k = 0; k < S; k++) {
            if (!L[c * S + k]) continue;
            for (int64_t i = 0; i < b; i++)
                for (int64_t j = 0; j < b; j++)
                    w[(id * b + i) * b + j] = (c == k && i == j) ? 1.0 : 0.0;
            id++;
        }
    return 0;
}

/* block_coord: the (c, k) of a block id under the row-major numbering. */
int orc_block_coord(const uint8_t* L, int64_t R, int64_t S, int64_t block, int64_t* c, int64_t* k) {
    if (!L || !c || !k || block < 0) return -1;
    int64_t id = 0;
    for (int64_t r = 0; r < R; r++)
        for (int64_t s = 0; s < S; s++)
            if (L[r * S + s]) {
                if (id == block) { *c = r; *k = s; return 0; }
                id++;
            }
    return -1;
}
