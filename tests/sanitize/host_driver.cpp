// Host-side driver for the sanitizer build of libbsmm (AddressSanitizer and
// UndefinedBehaviorSanitizer on the host code; no device code is compiled).  It runs
// the layout compiler over many layouts and every C-ABI argument check with fake device
// pointers, the same cases the CPU tests take through Python, and verifies the tables'
// invariants.  No GPU is used: any call that passes its checks stops at its first HIP
// runtime call with BSMM_ERR_DEVICE.  Exit status 0 when every check holds.
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <random>
#include <vector>

#include "bsmm.h"

static int g_fail = 0;
#define CHECK(c)                                                        \
    do {                                                                \
        if (!(c)) {                                                     \
            std::fprintf(stderr, "check failed: %s (line %d)\n", #c, __LINE__); \
            g_fail++;                                                   \
        }                                                               \
    } while (0)

static std::vector<int64_t> lut(bsmm_handle h, int which) {
    int64_t n = 0;
    CHECK(bsmm_debug_lut(h, which, nullptr, 0, &n) == BSMM_OK);
    std::vector<int64_t> v(n > 0 ? n : 1);
    CHECK(bsmm_debug_lut(h, which, v.data(), n, &n) == BSMM_OK);
    v.resize(n);
    return v;
}

// Tables of one plan against the layout they came from.
static void check_plan(const std::vector<uint8_t>& L, int64_t R, int64_t S, int b, int fa) {
    bsmm_handle h = nullptr;
    CHECK(bsmm_create(&h, L.data(), R, S, b, fa) == BSMM_OK);
    if (!h) return;
    int64_t nnz = 0;
    for (uint8_t v : L) nnz += v;
    int64_t ws[3];
    CHECK(bsmm_w_shape(h, ws) == BSMM_OK && ws[0] == nnz && ws[1] == b && ws[2] == b);
    const std::vector<int64_t> coords = lut(h, 0), colptr = lut(h, 1), colent = lut(h, 2), rowptr = lut(h, 3),
                               rowent = lut(h, 4);
    CHECK((int64_t)coords.size() == 2 * nnz);
    int64_t t = 0;
    for (int64_t c = 0; c < R; c++)
        for (int64_t k = 0; k < S; k++)
            if (L[c * S + k]) {   // ids in row-major order
                CHECK(coords[2 * t] == c && coords[2 * t + 1] == k);
                int64_t cc = -1, kk = -1;
                CHECK(bsmm_block_coord(h, t, &cc, &kk) == BSMM_OK && cc == c && kk == k);
                t++;
            }
    CHECK((int64_t)colptr.size() == S + 1 && colptr[S] == nnz && (int64_t)rowptr.size() == R + 1 && rowptr[R] == nnz);
    for (int64_t k = 0; k < S; k++)
        for (int64_t e = colptr[k]; e < colptr[k + 1]; e++) {
            const int64_t c = colent[2 * e], id = colent[2 * e + 1];
            CHECK(coords[2 * id] == c && coords[2 * id + 1] == k);
            if (e > colptr[k]) CHECK(colent[2 * (e - 1)] < c);
        }
    for (int64_t c = 0; c < R; c++)
        for (int64_t e = rowptr[c]; e < rowptr[c + 1]; e++) {
            const int64_t k = rowent[2 * e], id = rowent[2 * e + 1];
            CHECK(coords[2 * id] == c && coords[2 * id + 1] == k);
        }
    for (int which = 5; which < 20; which++) (void)lut(h, which);   // every table readable
    for (int pass = 0; pass < 4; pass++)
        for (int dt = 0; dt < 3; dt++)
            for (int64_t N : {0, 1, 64, 65, 512, 1024, 4096}) {
                const char* name = nullptr;
                CHECK(bsmm_kernel_name(h, pass, N, 1, (bsmm_dtype)dt, &name) == BSMM_OK && name);
                size_t bytes = 0;
                CHECK(bsmm_workspace_size(h, pass, N, (bsmm_dtype)dt, &bytes) == BSMM_OK);
            }
    bsmm_destroy(h);
}

int main() {
    std::mt19937 rng(7);
    // layouts: every block size and feature axis, densities from empty to full, odd shapes
    const int64_t shapes[][2] = {{1, 1}, {1, 7}, {7, 1}, {3, 5}, {16, 16}, {40, 24}, {64, 64}, {130, 9}};
    for (const auto& sh : shapes)
        for (int b : {8, 16, 32})
            for (int fa : {0, 1})
                for (double p : {0.0, 0.1, 0.5, 1.0}) {
                    std::vector<uint8_t> L(sh[0] * sh[1]);
                    std::bernoulli_distribution d(p);
                    for (auto& v : L) v = d(rng) ? 1 : 0;
                    check_plan(L, sh[0], sh[1], b, fa);
                }
    {   // a band and a long column / row (lists longer than the inline records)
        const int64_t R = 1100;
        std::vector<uint8_t> L(R * 3, 0);
        for (int64_t c = 0; c < R; c++) L[c * 3 + 1] = 1;
        check_plan(L, R, 3, 32, 1);
        std::vector<uint8_t> B(256 * 256, 0);
        for (int64_t c = 0; c < 256; c++)
            for (int64_t k = 0; k < 256; k++) B[c * 256 + k] = (c - k <= 2 && k - c <= 2) ? 1 : 0;
        check_plan(B, 256, 256, 32, 1);
    }
    // invalid plans
    bsmm_handle h = nullptr;
    const uint8_t one[4] = {1, 0, 2, 1};
    CHECK(bsmm_create(&h, one, 2, 2, 32, 1) == BSMM_ERR_INVALID_ARG && h == nullptr);
    CHECK(bsmm_create(&h, one, 2, 1, 12, 1) == BSMM_ERR_INVALID_ARG);
    CHECK(bsmm_create(&h, one, 2, 1, 32, 3) == BSMM_ERR_INVALID_ARG);
    CHECK(bsmm_create(&h, one, 0, 1, 32, 1) == BSMM_ERR_INVALID_ARG);
    CHECK(bsmm_create(&h, nullptr, 1, 1, 32, 1) == BSMM_ERR_INVALID_ARG);
    CHECK(bsmm_create(nullptr, one, 1, 1, 32, 1) == BSMM_ERR_INVALID_ARG);
    bsmm_destroy(nullptr);

    // call validation with fake device pointers (no GPU: a call that passes its checks
    // returns BSMM_ERR_DEVICE at its first runtime call)
    const uint8_t lay[6] = {1, 1, 0, 1, 0, 1};
    CHECK(bsmm_create(&h, lay, 2, 3, 8, 1) == BSMM_OK);
    void* good = (void*)0x10000;
    void* odd = (void*)0x10008;
    void* arr[8] = {good, good, good, good, good, good, good, good};
    void* bad[2] = {good, (void*)0x10004};
    CHECK(bsmm_fprop(h, good, good, good, 4, (bsmm_dtype)7, nullptr, 0, nullptr) == BSMM_ERR_INVALID_ARG);
    CHECK(bsmm_fprop(h, good, good, good, -1, BSMM_F32, nullptr, 0, nullptr) == BSMM_ERR_INVALID_ARG);
    CHECK(bsmm_fprop(h, nullptr, good, good, 4, BSMM_F32, nullptr, 0, nullptr) == BSMM_ERR_INVALID_ARG);
    CHECK(bsmm_fprop(h, odd, good, good, 4, BSMM_F32, nullptr, 0, nullptr) == BSMM_ERR_ALIGNMENT);
    CHECK(bsmm_fprop(h, good, good, good, int64_t(1) << 40, BSMM_F32, nullptr, 0, nullptr) == BSMM_ERR_UNSUPPORTED);
    CHECK(bsmm_fprop(h, nullptr, nullptr, nullptr, 0, BSMM_F32, nullptr, 0, nullptr) == BSMM_OK);
    CHECK(bsmm_bprop(h, good, odd, good, 4, BSMM_BF16, nullptr, 0, nullptr) == BSMM_ERR_ALIGNMENT);
    CHECK(bsmm_fprop(h, good, good, good, 4, BSMM_F32, nullptr, 0, nullptr) == BSMM_ERR_DEVICE);
    CHECK(bsmm_updat(h, (const void* const*)arr, (const void* const*)arr, 0, good, 4, BSMM_F32, BSMM_F32, nullptr, 0,
                     nullptr) == BSMM_ERR_INVALID_ARG);
    CHECK(bsmm_updat(h, (const void* const*)arr, (const void* const*)arr, 9, good, 4, BSMM_F32, BSMM_F32, nullptr, 0,
                     nullptr) == BSMM_ERR_INVALID_ARG);
    CHECK(bsmm_updat(h, (const void* const*)bad, (const void* const*)bad, 2, good, 4, BSMM_F32, BSMM_F32, nullptr, 0,
                     nullptr) == BSMM_ERR_ALIGNMENT);
    CHECK(bsmm_updat(h, nullptr, (const void* const*)arr, 1, good, 4, BSMM_F32, BSMM_F32, nullptr, 0, nullptr) ==
          BSMM_ERR_INVALID_ARG);
    CHECK(bsmm_updat_accumulate(h, (const void* const*)arr, (const void* const*)arr, 1, odd, 4, BSMM_F32, BSMM_F32,
                                nullptr, 0, nullptr) == BSMM_ERR_ALIGNMENT);
    CHECK(bsmm_updat_noalloc(h, (const void* const*)arr, (const void* const*)arr, 1, good, 4, BSMM_F32, (bsmm_dtype)5,
                             nullptr) == BSMM_ERR_INVALID_ARG);
    CHECK(bsmm_identity_init(h, odd, BSMM_F32, nullptr) == BSMM_ERR_ALIGNMENT);
    CHECK(bsmm_force_kernel(h, 0, "no such kernel") == BSMM_ERR_INVALID_ARG);
    CHECK(bsmm_force_kernel(h, 0, "list_n64") == BSMM_OK && bsmm_force_kernel(h, 0, nullptr) == BSMM_OK);
    CHECK(bsmm_debug_lut(h, 99, nullptr, 0, nullptr) == BSMM_ERR_INVALID_ARG);
    CHECK(bsmm_l2_normalize(h, good, nullptr, good, nullptr, -1.f, BSMM_F32, BSMM_F32, nullptr) == BSMM_ERR_INVALID_ARG);
    CHECK(bsmm_l2_normalize_grad(h, odd, good, nullptr, good, nullptr, 1e-6f, BSMM_F32, BSMM_F32, nullptr) ==
          BSMM_ERR_ALIGNMENT);
    for (int s = 0; s < 6; s++) CHECK(bsmm_status_string((bsmm_status)s)[0] == 'B');
    CHECK(bsmm_last_error() != nullptr);
    bsmm_destroy(h);

    // layer norm arguments
    size_t wsb = 0;
    CHECK(bsmm_layer_norm_workspace_size(64, 256, 0, 1, BSMM_BF16, &wsb) == BSMM_OK);
    CHECK(bsmm_layer_norm(good, (const float*)good, (const float*)good, good, nullptr, nullptr, 64, 256, 2, 1e-6f, 0,
                          BSMM_BF16, nullptr, 0, nullptr) == BSMM_ERR_INVALID_ARG);
    CHECK(bsmm_layer_norm(odd, (const float*)good, (const float*)good, good, nullptr, nullptr, 64, 256, 1, 1e-6f, 0,
                          BSMM_BF16, nullptr, 0, nullptr) == BSMM_ERR_ALIGNMENT);

    // SparseProj plans and arguments
    bsmm_proj_handle ph = nullptr;
    CHECK(bsmm_proj_create(&ph, 512, 256, 64, 32, nullptr) == BSMM_OK);
    int64_t nh = 0, np = 0;
    CHECK(bsmm_proj_info(ph, &nh, &np) == BSMM_OK && nh == 512 && np == 256);
    std::vector<int32_t> pl(256);
    CHECK(bsmm_proj_lut(ph, pl.data(), 256) == BSMM_OK && pl[32] == 64);
    CHECK(bsmm_proj_gather(ph, odd, good, 4, 1, BSMM_F32, nullptr) == BSMM_ERR_ALIGNMENT);
    CHECK(bsmm_proj_scatter(ph, good, good, 4, 2, BSMM_F32, nullptr) == BSMM_ERR_INVALID_ARG);
    bsmm_proj_destroy(ph);
    const int32_t dup[3] = {1, 1, 2};
    CHECK(bsmm_proj_create(&ph, 8, 3, 0, 1, dup) == BSMM_ERR_INVALID_ARG);
    CHECK(bsmm_proj_create(&ph, 8, 5, 0, 2, nullptr) == BSMM_ERR_INVALID_ARG);
    bsmm_proj_destroy(nullptr);

    // BlocksparseConv plans and arguments
    {
        const int32_t cidx[4] = {0, 1, 2, 3}, kidx[4] = {3, 2, 1, 0};
        const int64_t TRS[3] = {1, 3, 3}, DHW[3] = {1, 8, 8}, st[3] = {1, 1, 1}, dl[3] = {1, 1, 1}, pads[3] = {0, 1, 1};
        bsmm_conv_handle ch = nullptr;
        CHECK(bsmm_conv_create(&ch, 2, 2, 2, cidx, kidx, 4, 4, TRS, DHW, st, dl, 0, pads) == BSMM_OK);
        int64_t mpq[3], pd[3];
        CHECK(bsmm_conv_geometry(ch, mpq, pd) == BSMM_OK && mpq[1] == 8 && mpq[2] == 8);
        const char* nm = nullptr;
        for (int pass = 0; pass < 3; pass++) CHECK(bsmm_conv_kernel_name(ch, pass, BSMM_BF16, &nm) == BSMM_OK && nm);
        size_t cw = 0;
        CHECK(bsmm_conv_workspace_size(ch, 32, BSMM_BF16, &cw) == BSMM_OK);
        CHECK(bsmm_conv_fprop(ch, good, odd, good, 2, BSMM_BF16, nullptr) == BSMM_ERR_ALIGNMENT);
        bsmm_conv_destroy(ch);
        const int64_t big[3] = {1, 9, 9};
        CHECK(bsmm_conv_create(&ch, 2, 2, 2, cidx, kidx, 4, 4, big, DHW, st, dl, 1, pads) == BSMM_ERR_INVALID_ARG);
        const int32_t oob[4] = {0, 1, 2, 9};
        CHECK(bsmm_conv_create(&ch, 2, 2, 2, oob, kidx, 4, 4, TRS, DHW, st, dl, 0, pads) == BSMM_ERR_INVALID_ARG);
        bsmm_conv_destroy(nullptr);
    }
    std::printf("host driver: %s (%d failed checks)\n", g_fail ? "FAILED" : "ok", g_fail);
    return g_fail ? 1 : 0;
}
