// Host-side layout compiler: turns a 0/1 block layout into the look-up tables the
// kernels walk.  Pure C++ (no HIP calls), so it runs and is tested without a GPU.
//
// Layout semantics follow the kiteco/blocksparse README, "API Documentation" ›
// blocksparse.matmul › BlocksparseMatMul: __init__ takes an R x S array of zeros and
// ones and a block size of 8, 16 or 32; block_coord maps a block id to (c, k).  Ids
// are the row-major rank of a nonzero.
#include <algorithm>
#include <array>
#include <numeric>
#include <tuple>

#include "bsmm_internal.h"

namespace bsmm {

static std::vector<int32_t> order_by_length(const std::vector<int32_t>& ptr) {
    const int32_t n = (int32_t)ptr.size() - 1;
    std::vector<int32_t> ord(n);
    std::iota(ord.begin(), ord.end(), 0);
    std::stable_sort(ord.begin(), ord.end(), [&](int32_t a, int32_t b) {
        return (ptr[a + 1] - ptr[a]) > (ptr[b + 1] - ptr[b]);
    });
    return ord;
}

bool compile_layout(const uint8_t* layout, int64_t R, int64_t S, int b, int fa, HostLut& out,
                    std::string& err) {
    if (!layout) { err = "layout is NULL"; return false; }
    if (R < 1 || S < 1) { err = "layout must have at least one row and one column"; return false; }
    if (b != 8 && b != 16 && b != 32) { err = "block_size must be 8, 16 or 32"; return false; }
    if (fa != 0 && fa != 1) { err = "feature_axis must be 0 or 1"; return false; }
    if (R * (int64_t)b > INT32_MAX || S * (int64_t)b > INT32_MAX) {
        err = "feature dimension exceeds 2^31-1"; return false;
    }
    if (R * S > (int64_t)1 << 40) { err = "layout too large"; return false; }
    int64_t nnz = 0;
    for (int64_t t = 0; t < R * S; t++) {
        if (layout[t] > 1) { err = "layout entries must be 0 or 1"; return false; }
        nnz += layout[t];
    }
    if (nnz * (int64_t)b * b > INT32_MAX * (int64_t)64) { err = "too many blocks"; return false; }
    if (nnz > INT32_MAX / 2) { err = "too many blocks"; return false; }

    HostLut L;
    L.R = R; L.S = S; L.b = b; L.fa = fa; L.nnz = nnz;
    L.coords.resize(2 * nnz);
    L.colptr.assign(S + 1, 0);
    L.rowptr.assign(R + 1, 0);
    // ids: row-major scan; count per column and row on the way
    int32_t id = 0;
    for (int64_t c = 0; c < R; c++)
        for (int64_t k = 0; k < S; k++)
            if (layout[c * S + k]) {
                L.coords[2 * id] = (int32_t)c;
                L.coords[2 * id + 1] = (int32_t)k;
                L.colptr[k + 1]++;
                L.rowptr[c + 1]++;
                id++;
            }
    std::partial_sum(L.colptr.begin(), L.colptr.end(), L.colptr.begin());
    std::partial_sum(L.rowptr.begin(), L.rowptr.end(), L.rowptr.begin());
    // fprop lists (c ascending within each column) and bprop lists (k ascending within
    // each row): a single pass in id order visits c ascending and, within a row, k
    // ascending, so a counting sort keeps both orders.
    L.colent.resize(2 * nnz);
    L.rowent.resize(2 * nnz);
    std::vector<int32_t> cfill(L.colptr.begin(), L.colptr.end() - 1);
    std::vector<int32_t> rfill(L.rowptr.begin(), L.rowptr.end() - 1);
    for (int32_t t = 0; t < (int32_t)nnz; t++) {
        int32_t c = L.coords[2 * t], k = L.coords[2 * t + 1];
        int32_t pc = cfill[k]++;
        L.colent[2 * pc] = c;
        L.colent[2 * pc + 1] = t;
        int32_t pr = rfill[c]++;
        L.rowent[2 * pr] = k;
        L.rowent[2 * pr + 1] = t;
    }
    L.colorder = order_by_length(L.colptr);
    L.roworder = order_by_length(L.rowptr);
    auto work = [](const std::vector<int32_t>& order, const std::vector<int32_t>& ptr) {
        std::vector<int32_t> w(4 * order.size());
        for (size_t i = 0; i < order.size(); i++) {
            const int32_t o = order[i];
            w[4 * i] = o;
            w[4 * i + 1] = ptr[o];
            w[4 * i + 2] = ptr[o + 1] - ptr[o];
            w[4 * i + 3] = 0;
        }
        return w;
    };
    L.colwork = work(L.colorder, L.colptr);
    L.rowwork = work(L.roworder, L.rowptr);
    for (int64_t c = 0; c < R; c++)
        for (int32_t s = L.rowptr[c]; s < L.rowptr[c + 1]; s += 8) {
            const int32_t n = std::min<int32_t>(8, L.rowptr[c + 1] - s);
            // ids of row c are rowptr[c] .. rowptr[c+1]-1 (row-major numbering)
            L.ugroups.insert(L.ugroups.end(), {s, n, (int32_t)c, 0});
        }
    for (int64_t k = 0; k < S; k++) L.max_col = std::max(L.max_col, L.colptr[k + 1] - L.colptr[k]);
    for (int64_t c = 0; c < R; c++) L.max_row = std::max(L.max_row, L.rowptr[c + 1] - L.rowptr[c]);
    auto records = [](const std::vector<int32_t>& order, const std::vector<int32_t>& ptr,
                      const std::vector<int32_t>& ent, int32_t maxlen, std::vector<int32_t>& rec,
                      int32_t& rsi) {
        // an even entry count keeps every record 16-byte aligned
        const int32_t rs = std::max<int32_t>(2, (std::min<int32_t>(maxlen, kRecCap) + 1) & ~1);
        rsi = 4 + 2 * rs;
        rec.assign(order.size() * rsi, 0);
        for (size_t i = 0; i < order.size(); i++) {
            int32_t* r = rec.data() + i * rsi;
            const int32_t o = order[i], len = ptr[o + 1] - ptr[o];
            r[0] = o;
            r[1] = ptr[o];
            r[2] = len;
            for (int32_t e = 0; e < std::min(len, rs); e++) {
                r[4 + 2 * e] = ent[2 * (ptr[o] + e)];
                r[4 + 2 * e + 1] = ent[2 * (ptr[o] + e) + 1];
            }
        }
    };
    records(L.colorder, L.colptr, L.colent, L.max_col, L.colrec, L.col_rsi);
    records(L.roworder, L.rowptr, L.rowent, L.max_row, L.rowrec, L.row_rsi);
    if (b == 32) {
        // outer: the contraction index ascending; inner: its blocks, bucketed by group
        auto groups = [](int64_t nouter, int64_t nout, const std::vector<int32_t>& ptr,
                         const std::vector<int32_t>& ent, std::vector<int32_t>& gptr,
                         std::vector<int32_t>& gent) {
            const int64_t ng = (nout + kGroupOut - 1) / kGroupOut;
            std::vector<std::vector<int32_t>> lists(ng);
            for (int64_t u = 0; u < nouter; u++)
                for (int32_t e = ptr[u]; e < ptr[u + 1]; e++) {
                    const int32_t o = ent[2 * e], id = ent[2 * e + 1];
                    std::vector<int32_t>& v = lists[o / kGroupOut];
                    if (v.empty() || v[v.size() - kGroupInts] != (int32_t)u) v.resize(v.size() + kGroupInts, 0);
                    int32_t* r = v.data() + v.size() - kGroupInts;
                    r[0] = (int32_t)u;
                    r[1] |= 1 << (o % kGroupOut);
                    r[2 + o % kGroupOut] = id;
                }
            gptr.assign(ng + 1, 0);
            gent.clear();
            for (int64_t g = 0; g < ng; g++) {
                gent.insert(gent.end(), lists[g].begin(), lists[g].end());
                gptr[g + 1] = (int32_t)(gent.size() / kGroupInts);
            }
        };
        // fprop groups: rows c outer, the row's blocks (k, id); bprop: columns outer
        groups(R, S, L.rowptr, L.rowent, L.cgptr, L.cgent);
        groups(S, R, L.colptr, L.colent, L.rgptr, L.rgent);
        // weight-gradient tiles; ids of a tile row are consecutive in row-major order
        const int64_t TR = (R + kTileSide - 1) / kTileSide, TC = (S + kTileSide - 1) / kTileSide;
        std::vector<uint8_t> in_tile(nnz, 0);
        for (int64_t tr = 0; tr < TR; tr++)
            for (int64_t tc = 0; tc < TC; tc++) {
                std::vector<int32_t> pos(kTileSide * kTileSide, -1);   // row-major ids, -1 absent
                int32_t n = 0;
                for (int64_t c = tr * kTileSide; c < std::min<int64_t>(R, (tr + 1) * kTileSide); c++)
                    for (int32_t e = L.rowptr[c]; e < L.rowptr[c + 1]; e++) {
                        const int32_t k = L.rowent[2 * e];
                        if (k / kTileSide == tc) {
                            pos[(c - tr * kTileSide) * kTileSide + k % kTileSide] = L.rowent[2 * e + 1];
                            n++;
                        }
                    }
                if (n < kTileMin) continue;
                L.utiles.insert(L.utiles.end(), {(int32_t)(tr * kTileSide), (int32_t)(tc * kTileSide), n,
                                                 (int32_t)L.utblk.size()});
                for (int32_t id : pos)
                    if (id >= 0) in_tile[id] = 1;
                L.utblk.insert(L.utblk.end(), pos.begin(), pos.end());
            }
        // Processing order of the tiles: super-blocks of kSuperRows tile rows x kSuperCols
        // tile columns, row-major within and between super-blocks.  The weight-gradient
        // kernel hands each XCD a contiguous range of this order, so the tiles an XCD runs
        // at once form a compact block whose x rows and dy columns it reads from one L2
        // (in plain row-major order they were one tile row x every tile column, and each
        // dy column was fetched again for every tile row).
        {
            std::vector<int32_t> ord(L.utiles.size() / 4);
            std::iota(ord.begin(), ord.end(), 0);
            auto key = [&](int32_t i) {
                const int64_t tr = L.utiles[4 * i] / kTileSide, tc = L.utiles[4 * i + 1] / kTileSide;
                return std::make_tuple(tr / kSuperRows, tc / kSuperCols, tr, tc);
            };
            std::stable_sort(ord.begin(), ord.end(), [&](int32_t x, int32_t y) { return key(x) < key(y); });
            std::vector<int32_t> sorted;
            sorted.reserve(L.utiles.size());
            for (int32_t i : ord) sorted.insert(sorted.end(), L.utiles.begin() + 4 * i, L.utiles.begin() + 4 * i + 4);
            L.utiles.swap(sorted);
        }
        // the rest: per row, its blocks outside the tiles in groups of at most
        // kRestGroup, as even as possible (the slowest group sets the launch's time)
        for (int64_t c = 0; c < R; c++) {
            std::vector<int32_t> ids;
            for (int32_t e = L.rowptr[c]; e < L.rowptr[c + 1]; e++)
                if (!in_tile[L.rowent[2 * e + 1]]) ids.push_back(L.rowent[2 * e + 1]);
            const int32_t n = (int32_t)ids.size(), ng = (n + kRestGroup - 1) / kRestGroup;
            for (int32_t gi = 0, at = 0; gi < ng; gi++) {
                const int32_t cnt = n / ng + (gi < n % ng ? 1 : 0);
                L.urest.insert(L.urest.end(), {(int32_t)L.urids.size(), cnt, (int32_t)c, 1});
                L.urids.insert(L.urids.end(), ids.begin() + at, ids.begin() + at + cnt);
                at += cnt;
            }
        }
    }
    if (b == 8 || b == 16) {
        // small-block weight-gradient tiles (lut_format.h), in super-block order
        const int64_t TB = kSmallTileFeat / b;          // blocks per tile side
        const int64_t QB = b == 8 ? 2 : 1;              // blocks per quad side
        const int64_t TR = (R + TB - 1) / TB, TC = (S + TB - 1) / TB;
        std::vector<std::array<int64_t, 2>> order;
        for (int64_t tr = 0; tr < TR; tr++)
            for (int64_t tc = 0; tc < TC; tc++) order.push_back({tr, tc});
        std::stable_sort(order.begin(), order.end(), [](const std::array<int64_t, 2>& x, const std::array<int64_t, 2>& y) {
            return std::make_tuple(x[0] / kSuperRows, x[1] / kSuperCols, x[0], x[1]) <
                   std::make_tuple(y[0] / kSuperRows, y[1] / kSuperCols, y[0], y[1]);
        });
        // id of block (c, k), -1 if absent: rows are consecutive ids
        auto block_id = [&](int64_t c, int64_t k) -> int32_t {
            if (c >= R || k >= S) return -1;
            const int32_t* beg = L.rowent.data() + 2 * L.rowptr[c];
            int32_t lo = 0, hi = L.rowptr[c + 1] - L.rowptr[c];
            while (lo < hi) {   // entries ascending in k
                const int32_t mid = (lo + hi) / 2;
                if (beg[2 * mid] < k) lo = mid + 1; else hi = mid;
            }
            return lo < L.rowptr[c + 1] - L.rowptr[c] && beg[2 * lo] == k ? beg[2 * lo + 1] : -1;
        };
        for (const auto& tcell : order) {
            const int64_t tr = tcell[0], tc = tcell[1];
            std::vector<int32_t> ids(kSmallQuads * kSmallQuads * QB * QB, -1), mask(kSmallQuads, 0);
            int32_t n = 0;
            for (int64_t qi = 0; qi < kSmallQuads; qi++)
                for (int64_t qj = 0; qj < kSmallQuads; qj++)
                    for (int64_t di = 0; di < QB; di++)
                        for (int64_t dj = 0; dj < QB; dj++) {
                            const int32_t id = block_id(tr * TB + qi * QB + di, tc * TB + qj * QB + dj);
                            ids[((qi * kSmallQuads + qj) * QB + di) * QB + dj] = id;
                            if (id >= 0) {
                                mask[qi] |= 1 << qj;
                                n++;
                            }
                        }
            if (n == 0) continue;
            L.stiles.insert(L.stiles.end(), {(int32_t)(tr * kSmallTileFeat), (int32_t)(tc * kSmallTileFeat),
                                             (int32_t)L.stids.size(), 0});
            // quad rows to waves: wave w runs on SIMD w % 4 of its compute unit, so the
            // rows go to the four SIMDs (four rows each) fullest first, each to the SIMD
            // with the fewest quads so far, so that no SIMD's matrix core carries much
            // more than a quarter of the tile
            std::vector<int32_t> cnt(kSmallQuads, 0), order(kSmallQuads);
            for (int64_t qi = 0; qi < kSmallQuads; qi++) cnt[qi] = __builtin_popcount((uint32_t)mask[qi]);
            std::iota(order.begin(), order.end(), 0);
            std::stable_sort(order.begin(), order.end(), [&](int32_t x, int32_t y) { return cnt[x] > cnt[y]; });
            int32_t load[4] = {0, 0, 0, 0}, taken[4] = {0, 0, 0, 0}, rowof[kSmallQuads];
            for (int32_t r : order) {
                int best = -1;
                for (int sm = 0; sm < 4; sm++)
                    if (taken[sm] < kSmallQuads / 4 && (best < 0 || load[sm] < load[best])) best = sm;
                rowof[best + 4 * taken[best]] = r;
                taken[best]++;
                load[best] += cnt[r];
            }
            for (int wv = 0; wv < kSmallQuads; wv++) {
                const int32_t qi = rowof[wv];
                std::vector<int32_t> plan(kSmallPlanInts, 0);
                int32_t c = 0;
                for (int qj = 0; qj < kSmallQuads; qj++)
                    if ((mask[qi] >> qj) & 1) {
                        plan[1 + c / 4] |= (int32_t)((uint32_t)qj << (8 * (c % 4)));
                        c++;
                    }
                plan[0] = c;
                plan[5] = qi;
                L.stplan.insert(L.stplan.end(), plan.begin(), plan.end());
            }
            L.stids.insert(L.stids.end(), ids.begin(), ids.end());
        }
    }
    out = std::move(L);
    return true;
}

}  // namespace bsmm
