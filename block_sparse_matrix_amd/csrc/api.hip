// C ABI of libbsmm (declared and documented in include/bsmm.h): argument checks,
// lazy per-device upload of the layout tables, and dispatch to the kernel launchers.
// Every argument is validated before the first HIP call, so the error paths run
// without a GPU.
#include <hip/hip_runtime.h>

#include <cstdlib>
#include <cstring>
#include <map>
#include <mutex>
#include <new>
#include <string>
#include <vector>

#include "bsmm_internal.h"
#include "kernels.h"

using namespace bsmm;

namespace {

thread_local std::string g_err;

bsmm_status fail(bsmm_status s, const std::string& msg) {
    g_err = msg;
    return s;
}

bsmm_status dev_fail(hipError_t e, const char* what) {
    g_err = std::string(what) + ": " + hipGetErrorString(e);
    return BSMM_ERR_DEVICE;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

bool valid_dt(int dt) { return dt == BSMM_F32 || dt == BSMM_BF16 || dt == BSMM_F16; }

// ---- kernel timing (bsmm_profile_begin / bsmm_profile_end) ----
struct ProfRec {
    int pass;
    hipEvent_t e0, e1;
};
struct Prof {
    bool on = false;
    std::vector<ProfRec> recs;
    std::vector<hipEvent_t> pool;
    ~Prof() {
        for (auto e : pool) (void)hipEventDestroy(e);
    }
};
thread_local Prof g_prof;

hipEvent_t pool_event() {
    if (!g_prof.pool.empty()) {
        hipEvent_t e = g_prof.pool.back();
        g_prof.pool.pop_back();
        return e;
    }
    hipEvent_t e = nullptr;
    if (hipEventCreate(&e) != hipSuccess) return nullptr;
    return e;
}

// ---- per-device tables ----
template <typename V>
size_t bytes_of(const V& v) {
    return v.size() * sizeof(typename V::value_type);
}

// A handle's tables reach a device on its first call there: one allocation, filled by
// an asynchronous copy on the caller's stream from the host image the handle keeps
// (so the copy is ordered before the kernels that read it and never blocks the host).
// Refused while the stream is being captured into a graph: the allocation and the
// copy would become part of the graph.
bsmm_status upload_tables(const void* host, size_t bytes, void* stream, const char* what, void** out) {
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    hipError_t e = hipStreamIsCapturing((hipStream_t)stream, &cs);
    if (e != hipSuccess) return dev_fail(e, "hipStreamIsCapturing");
    if (cs != hipStreamCaptureStatusNone)
        return fail(BSMM_ERR_UNSUPPORTED, std::string("first use of the ") + what +
                                              " on this device inside a stream capture: the tables are uploaded on "
                                              "a handle's first call per device; make one call before capturing");
    void* p = nullptr;
    e = hipMalloc(&p, bytes > 0 ? bytes : 256);
    if (e != hipSuccess)
        return e == hipErrorOutOfMemory ? fail(BSMM_ERR_OOM, std::string("hipMalloc of the ") + what + " failed")
                                        : dev_fail(e, "hipMalloc");
    if (bytes > 0) e = hipMemcpyAsync(p, host, bytes, hipMemcpyHostToDevice, (hipStream_t)stream);
    if (e != hipSuccess) {
        (void)hipFree(p);
        return dev_fail(e, "hipMemcpyAsync of the tables");
    }
    *out = p;
    return BSMM_OK;
}

bsmm_status device_lut(bsmm_plan* h, void* stream, const DeviceLut** out, bool may_upload = true) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return dev_fail(e, "hipGetDevice");
    std::lock_guard<std::mutex> guard(h->mu);
    auto it = h->dev.find(dev);
    if (it != h->dev.end()) {
        *out = &it->second;
        return BSMM_OK;
    }
    if (!may_upload)
        return fail(BSMM_ERR_UNSUPPORTED,
                    "the layout tables are not on this device yet and this call allocates nothing: make one call "
                    "of an allocating entry point on this device first");
    const HostLut& L = h->lut;
    constexpr int NP = 23;
    const std::vector<int32_t>* parts[NP] = {&L.coords,  &L.colptr,   &L.colent,   &L.rowptr,  &L.rowent,
                                             &L.colorder, &L.roworder, &L.colwork, &L.rowwork, &L.ugroups,
                                             &L.colrec,  &L.rowrec,   &L.cgptr,    &L.cgent,   &L.rgptr,
                                             &L.rgent,   &L.utiles,   &L.utblk,    &L.urest,   &L.urids,
                                             &L.stiles,  &L.stplan,   &L.stids};
    size_t off[NP], total = 0;
    for (int i = 0; i < NP; i++) {
        off[i] = total;
        total += (bytes_of(*parts[i]) + 255) & ~(size_t)255;
    }
    if (total == 0) total = 256;
    if (h->image.empty()) {   // built once, kept for the copies to later devices
        h->image.assign(total, 0);
        for (int i = 0; i < NP; i++)
            if (!parts[i]->empty()) std::memcpy(h->image.data() + off[i], parts[i]->data(), bytes_of(*parts[i]));
    }
    void* base = nullptr;
    bsmm_status st = upload_tables(h->image.data(), total, stream, "layout tables", &base);
    if (st != BSMM_OK) return st;
    DeviceLut d;
    d.base = base;
    const char* b = (const char*)base;
    d.coords = (const int32_t*)(b + off[0]);
    d.colptr = (const int32_t*)(b + off[1]);
    d.colent = (const int32_t*)(b + off[2]);
    d.rowptr = (const int32_t*)(b + off[3]);
    d.rowent = (const int32_t*)(b + off[4]);
    d.colorder = (const int32_t*)(b + off[5]);
    d.roworder = (const int32_t*)(b + off[6]);
    d.colwork = (const int32_t*)(b + off[7]);
    d.rowwork = (const int32_t*)(b + off[8]);
    d.ugroups = (const int32_t*)(b + off[9]);
    d.colrec = (const int32_t*)(b + off[10]);
    d.rowrec = (const int32_t*)(b + off[11]);
    d.cgptr = (const int32_t*)(b + off[12]);
    d.cgent = (const int32_t*)(b + off[13]);
    d.rgptr = (const int32_t*)(b + off[14]);
    d.rgent = (const int32_t*)(b + off[15]);
    d.utiles = (const int32_t*)(b + off[16]);
    d.utblk = (const int32_t*)(b + off[17]);
    d.urest = (const int32_t*)(b + off[18]);
    d.urids = (const int32_t*)(b + off[19]);
    d.stiles = (const int32_t*)(b + off[20]);
    d.stplan = (const int32_t*)(b + off[21]);
    d.stids = (const int32_t*)(b + off[22]);
    d.nstiles = (int32_t)(L.stiles.size() / 4);
    d.nutiles = (int32_t)(L.utiles.size() / 4);
    d.nurest = (int32_t)(L.urest.size() / 4);
    d.nugroups = (int32_t)(L.ugroups.size() / 4);
    auto res = h->dev.emplace(dev, d);
    *out = &res.first->second;
    return BSMM_OK;
}

void set_groups(MMArgs& a, const std::vector<int32_t>& hptr, const int32_t* dptr, const int32_t* dent, int64_t nnz) {
    a.ngroups = hptr.empty() ? 0 : (int32_t)hptr.size() - 1;
    a.gptr = dptr;
    a.gent = dent;
    const int64_t entries = hptr.empty() ? 0 : hptr.back();
    a.gfill = entries ? (int32_t)(100 * nnz / (entries * kGroupOut)) : 0;
    a.gmax = 0;
    for (size_t g = 0; g + 1 < hptr.size(); g++) a.gmax = std::max(a.gmax, hptr[g + 1] - hptr[g]);
}

bsmm_status check_call(bsmm_handle h, int64_t N, int dt) {
    if (!h) return fail(BSMM_ERR_INVALID_ARG, "handle is NULL");
    if (N < 0) return fail(BSMM_ERR_INVALID_ARG, "N must be >= 0");
    if (N > INT32_MAX) return fail(BSMM_ERR_UNSUPPORTED, "N above 2^31-1");
    if (!valid_dt(dt)) return fail(BSMM_ERR_INVALID_ARG, "dtype must be BSMM_F32, BSMM_BF16 or BSMM_F16");
    return BSMM_OK;
}

bsmm_status check_ptr(const void* p, const char* name) {
    if (!p) return fail(BSMM_ERR_INVALID_ARG, std::string(name) + " is NULL");
    if (!aligned16(p)) return fail(BSMM_ERR_ALIGNMENT, std::string(name) + " is not 16-byte aligned");
    return BSMM_OK;
}

bsmm_status run_mm(bsmm_handle h, const void* in, const void* w, void* out, int64_t N, bsmm_dtype dt,
                   bool bprop) {
    bsmm_status s = check_call(h, N, dt);
    if (s != BSMM_OK) return s;
    if (N == 0) return BSMM_OK;
    const char* nin = bprop ? "dy" : "x";
    const char* nout = bprop ? "dx" : "y";
    if ((s = check_ptr(in, nin)) != BSMM_OK) return s;
    if ((s = check_ptr(out, nout)) != BSMM_OK) return s;
    const HostLut& L = h->lut;
    if (L.nnz > 0 && (s = check_ptr(w, "w")) != BSMM_OK) return s;
    const uint64_t es = dt == BSMM_F32 ? 4 : 2;
    const uint64_t feats = (uint64_t)(bprop ? L.S : L.R) * L.b;
    if ((uint64_t)N * feats * es > kMaxTensorBytes || (uint64_t)L.nnz * L.b * L.b * es > kMaxTensorBytes)
        return fail(BSMM_ERR_UNSUPPORTED, "an operand exceeds 2 GiB (the kernels use 32-bit offsets)");
    return BSMM_OK;
}

uint32_t bytes32(uint64_t v) { return (uint32_t)v; }

}  // namespace

namespace bsmm {
void prof_events(int pass, void** start, void** stop) {
    *start = *stop = nullptr;
    if (!g_prof.on) return;
    hipEvent_t e0 = pool_event(), e1 = pool_event();
    if (!e0 || !e1) return;
    g_prof.recs.push_back({pass, e0, e1});
    *start = e0;
    *stop = e1;
}
}  // namespace bsmm

namespace {

// Arguments of an fprop (transw false) or bprop launch; with d NULL only the fields
// the kernel choice reads are meaningful.
MMArgs mm_args(const HostLut& L, const DeviceLut* d, bool transw, int64_t N, int dt) {
    MMArgs a{};
    const bool bp = transw;
    if (d) {
        a.work = bp ? d->rowwork : d->colwork;
        a.ptr = bp ? d->rowptr : d->colptr;
        a.rec = bp ? d->rowrec : d->colrec;
        a.ent = bp ? d->rowent : d->colent;
    }
    a.rsi = bp ? L.row_rsi : L.col_rsi;
    a.rec_bytes = bytes32((uint64_t)(bp ? L.R : L.S) * a.rsi * 4);
    a.maxlen = bp ? L.max_row : L.max_col;
    set_groups(a, bp ? L.rgptr : L.cgptr, d ? (bp ? d->rgptr : d->cgptr) : nullptr,
               d ? (bp ? d->rgent : d->cgent) : nullptr, L.nnz);
    a.N = N;
    a.fin = (int32_t)((bp ? L.S : L.R) * L.b);
    a.fout = (int32_t)((bp ? L.R : L.S) * L.b);
    a.nout = (int32_t)(bp ? L.R : L.S);
    const uint64_t es = dt == BSMM_F32 ? 4 : 2;
    a.in_bytes = bytes32((uint64_t)N * a.fin * es);
    a.w_bytes = bytes32((uint64_t)L.nnz * L.b * L.b * es);
    return a;
}

bsmm_status mm_pass(bsmm_handle h, const void* in, const void* w, void* out, int64_t N, bsmm_dtype dt,
                    bool transw, void* stream) {
    bsmm_status s = run_mm(h, in, w, out, N, dt, transw);
    if (s != BSMM_OK || N == 0) return s;
    const DeviceLut* d = nullptr;
    if ((s = device_lut(h, stream, &d)) != BSMM_OK) return s;
    const HostLut& L = h->lut;
    MMArgs a = mm_args(L, d, transw, N, dt);
    a.in = in;
    a.w = w;
    a.out = out;
    const int pass = transw ? BSMM_PASS_BPROP : BSMM_PASS_FPROP;
    a.force = h->force[pass];
    if (mm_kind(a, dt, L.b, L.fa) < 0)
        return fail(BSMM_ERR_UNSUPPORTED, "the forced kernel does not apply to these arguments");
    hipError_t e = launch_mm(a, dt, L.b, L.fa, transw, stream, pass);
    return e == hipSuccess ? BSMM_OK : dev_fail(e, transw ? "bprop launch" : "fprop launch");
}

// Workspace of the dense-tile weight gradient (32x32 blocks, 16-bit activations): the
// tiles' split partial sums, then the split partial sums of the blocks outside them.
void updat_ws_parts(const HostLut& L, int64_t N, bsmm_dtype dt, size_t* tiles, size_t* rest) {
    *tiles = *rest = 0;
    if (N <= 0 || dt == BSMM_F32 || L.b != 32) return;
    const int nt = (int)(L.utiles.size() / 4);
    const int p = tile_split(nt);
    if (p > 1) *tiles = (size_t)p * nt * kTileSide * kTileSide * 32 * 32 * sizeof(float);
    if (nt * p >= 128)   // the tile kernel can be chosen (enough tiles x parts)
        *rest = (size_t)kRestSplit * L.urids.size() * 32 * 32 * sizeof(float);
}

UpArgs up_args(const HostLut& L, int64_t N, int group) {
    UpArgs a{};
    a.split = 1;
    a.rsplit = 1;
    a.nrids = (int32_t)L.urids.size();
    a.ntiles = (int32_t)(L.utiles.size() / 4);
    a.nrest = (int32_t)(L.urest.size() / 4);
    a.ngroups = (int32_t)(L.ugroups.size() / 4);
    a.nstiles = (int32_t)(L.stiles.size() / 4);
    a.N = N;
    a.C = (int32_t)(L.R * L.b);
    a.K = (int32_t)(L.S * L.b);
    a.nnz = (int32_t)L.nnz;
    a.G = N > 0 ? group : 1;
    return a;
}

}  // namespace

extern "C" {

bsmm_status bsmm_create(bsmm_handle* out, const uint8_t* layout, int64_t R, int64_t S, int block_size,
                        int feature_axis) {
    if (!out) return fail(BSMM_ERR_INVALID_ARG, "out is NULL");
    *out = nullptr;
    bsmm_plan* p = new (std::nothrow) bsmm_plan();
    if (!p) return fail(BSMM_ERR_OOM, "out of host memory");
    std::string err;
    bool ok = false;
    try {
        ok = compile_layout(layout, R, S, block_size, feature_axis, p->lut, err);
    } catch (const std::bad_alloc&) {
        delete p;
        return fail(BSMM_ERR_OOM, "out of host memory compiling the layout");
    }
    if (!ok) {
        delete p;
        return fail(BSMM_ERR_INVALID_ARG, err);
    }
    *out = p;
    return BSMM_OK;
}

void bsmm_destroy(bsmm_handle h) {
    if (!h) return;
    int cur = -1;
    bool have_cur = hipGetDevice(&cur) == hipSuccess;
    for (auto& kv : h->dev) {
        if (hipSetDevice(kv.first) == hipSuccess) (void)hipFree(kv.second.base);
    }
    if (have_cur && !h->dev.empty()) (void)hipSetDevice(cur);
    delete h;
}

bsmm_status bsmm_w_shape(bsmm_handle h, int64_t out[3]) {
    if (!h || !out) return fail(BSMM_ERR_INVALID_ARG, "NULL argument");
    out[0] = h->lut.nnz;
    out[1] = out[2] = h->lut.b;
    return BSMM_OK;
}

bsmm_status bsmm_i_shape(bsmm_handle h, int64_t N, int64_t out[2]) {
    if (!h || !out || N < 0) return fail(BSMM_ERR_INVALID_ARG, "NULL argument or N < 0");
    const int64_t C = h->lut.R * h->lut.b;
    out[0] = h->lut.fa ? N : C;
    out[1] = h->lut.fa ? C : N;
    return BSMM_OK;
}

bsmm_status bsmm_o_shape(bsmm_handle h, int64_t N, int64_t out[2]) {
    if (!h || !out || N < 0) return fail(BSMM_ERR_INVALID_ARG, "NULL argument or N < 0");
    const int64_t K = h->lut.S * h->lut.b;
    out[0] = h->lut.fa ? N : K;
    out[1] = h->lut.fa ? K : N;
    return BSMM_OK;
}

bsmm_status bsmm_block_coord(bsmm_handle h, int64_t block, int64_t* c, int64_t* k) {
    if (!h || !c || !k) return fail(BSMM_ERR_INVALID_ARG, "NULL argument");
    if (block < 0 || block >= h->lut.nnz) return fail(BSMM_ERR_INVALID_ARG, "block id out of range");
    *c = h->lut.coords[2 * block];
    *k = h->lut.coords[2 * block + 1];
    return BSMM_OK;
}

bsmm_status bsmm_plan_info(bsmm_handle h, int64_t out[5]) {
    if (!h || !out) return fail(BSMM_ERR_INVALID_ARG, "NULL argument");
    out[0] = h->lut.R;
    out[1] = h->lut.S;
    out[2] = h->lut.b;
    out[3] = h->lut.fa;
    out[4] = h->lut.nnz;
    return BSMM_OK;
}

bsmm_status bsmm_workspace_size(bsmm_handle h, int pass, int64_t N, bsmm_dtype dt, size_t* bytes) {
    if (!h || !bytes) return fail(BSMM_ERR_INVALID_ARG, "NULL argument");
    if (pass < BSMM_PASS_FPROP || pass > BSMM_PASS_IDENTITY) return fail(BSMM_ERR_INVALID_ARG, "bad pass");
    if (N < 0) return fail(BSMM_ERR_INVALID_ARG, "N must be >= 0");
    if (!valid_dt(dt)) return fail(BSMM_ERR_INVALID_ARG, "bad dtype");
    *bytes = 0;
    if (pass == BSMM_PASS_UPDAT) {
        size_t tb = 0, rb = 0;
        updat_ws_parts(h->lut, N, dt, &tb, &rb);
        *bytes = tb + rb;
    }
    return BSMM_OK;
}


bsmm_status bsmm_fprop(bsmm_handle h, const void* x, const void* w, void* y, int64_t N, bsmm_dtype dt,
                       void* ws, size_t ws_bytes, void* stream) {
    (void)ws;   // no fprop kernel takes a workspace
    (void)ws_bytes;
    return mm_pass(h, x, w, y, N, dt, false, stream);
}

bsmm_status bsmm_bprop(bsmm_handle h, const void* dy, const void* w, void* dx, int64_t N, bsmm_dtype dt,
                       void* ws, size_t ws_bytes, void* stream) {
    (void)ws;   // no bprop kernel takes a workspace
    (void)ws_bytes;
    return mm_pass(h, dy, w, dx, N, dt, true, stream);
}

bsmm_status bsmm_kernel_name(bsmm_handle h, int pass, int64_t N, int group, bsmm_dtype dt, const char** name) {
    if (!h || !name) return fail(BSMM_ERR_INVALID_ARG, "NULL argument");
    bsmm_status s = check_call(h, N, dt);
    if (s != BSMM_OK) return s;
    if (group < 1 || group > kMaxGroup) return fail(BSMM_ERR_INVALID_ARG, "group must be in [1, 8]");
    const HostLut& L = h->lut;
    *name = "none";
    if (pass == BSMM_PASS_FPROP || pass == BSMM_PASS_BPROP) {
        const bool tw = pass == BSMM_PASS_BPROP;
        MMArgs a = mm_args(L, nullptr, tw, N, dt);
        a.force = h->force[pass];
        if (N > 0 && (tw ? L.R : L.S) > 0) *name = mm_kind_name(mm_kind(a, dt, L.b, L.fa));
    } else if (pass == BSMM_PASS_UPDAT) {
        UpArgs a = up_args(L, N, group);
        a.force = h->force[BSMM_PASS_UPDAT];
        size_t tb = 0, rb = 0;
        updat_ws_parts(L, N, dt, &tb, &rb);
        if (tb > 0) a.split = tile_split(a.ntiles);   // as when the workspace is given
        if (L.nnz > 0) *name = updat_kind_name(updat_kind(a, dt, L.b, L.fa));
    } else if (pass == BSMM_PASS_IDENTITY) {
        if (L.nnz > 0) *name = "identity";
    } else {
        return fail(BSMM_ERR_INVALID_ARG, "bad pass");
    }
    return BSMM_OK;
}

}  // extern "C"

namespace {
// updat and its accumulating form (acc: dW += the sum instead of dW = the sum).
// noalloc: the caller's ws is the library's fixed scratch; the tables must already be
// on the device (no upload, so no allocation).
bsmm_status updat_call(bsmm_handle h, const void* const* xs, const void* const* dys, int group, void* dw,
                       int64_t N, bsmm_dtype dt, bsmm_dtype dw_dt, void* ws, size_t ws_bytes, void* stream,
                       bool acc, bool noalloc = false) {
    bsmm_status s = check_call(h, N, dt);
    if (s != BSMM_OK) return s;
    if (!valid_dt(dw_dt)) return fail(BSMM_ERR_INVALID_ARG, "dw dtype must be BSMM_F32, BSMM_BF16 or BSMM_F16");
    if (group < 1 || group > kMaxGroup) return fail(BSMM_ERR_INVALID_ARG, "group must be in [1, 8]");
    const HostLut& L = h->lut;
    if (L.nnz == 0) return BSMM_OK;
    if ((s = check_ptr(dw, "dw")) != BSMM_OK) return s;
    if (N > 0) {
        if (!xs || !dys) return fail(BSMM_ERR_INVALID_ARG, "xs / dys is NULL");
        for (int t = 0; t < group; t++) {
            if ((s = check_ptr(xs[t], "xs[t]")) != BSMM_OK) return s;
            if ((s = check_ptr(dys[t], "dys[t]")) != BSMM_OK) return s;
        }
    }
    {
        const uint64_t es = dt == BSMM_F32 ? 4 : 2;
        if ((uint64_t)N * L.R * L.b * es > kMaxTensorBytes || (uint64_t)N * L.S * L.b * es > kMaxTensorBytes)
            return fail(BSMM_ERR_UNSUPPORTED, "an activation exceeds 2 GiB (the kernels use 32-bit offsets)");
    }
    if (acc && N == 0) return BSMM_OK;   // the empty sum adds nothing
    const DeviceLut* d = nullptr;
    if ((s = device_lut(h, stream, &d, !noalloc)) != BSMM_OK) return s;
    UpArgs a = up_args(L, N, group);
    a.acc = acc ? 1 : 0;
    for (int t = 0; t < group; t++) {
        a.xs[t] = N > 0 ? xs[t] : nullptr;
        a.dys[t] = N > 0 ? dys[t] : nullptr;
    }
    a.dw = dw;
    a.coords = d->coords;
    a.dwdt = dw_dt;
    const uint64_t es = dt == BSMM_F32 ? 4 : 2;
    a.x_bytes = (uint32_t)((uint64_t)N * a.C * es);
    a.groups = d->ugroups;
    a.ngroups = d->nugroups;
    a.tiles = d->utiles;
    a.tblk = d->utblk;
    a.ntiles = d->nutiles;
    a.rest = d->urest;
    a.rids = d->urids;
    a.nrest = d->nurest;
    a.stiles = d->stiles;
    a.stplan = d->stplan;
    a.stids = d->stids;
    a.dy_bytes = (uint32_t)((uint64_t)N * a.K * es);
    a.force = h->force[BSMM_PASS_UPDAT];
    {   // a contraction split needs the workspace: the tiles' when it holds their parts,
        // the other blocks' when it holds both; without it, no split
        size_t tb = 0, rb = 0;
        updat_ws_parts(L, N, dt, &tb, &rb);
        const bool ok = ws && ((uintptr_t)ws & 15u) == 0;
        a.split = ok && tb > 0 && ws_bytes >= tb ? tile_split(a.ntiles) : 1;
        a.ws = (float*)ws;
        if (ok && rb > 0 && a.nrest > 0 && ws_bytes >= tb + rb) {
            a.rsplit = kRestSplit;
            a.rws = (float*)((char*)ws + tb);
        }
    }
    if (updat_kind(a, dt, L.b, L.fa) < 0)
        return fail(BSMM_ERR_UNSUPPORTED, "the forced kernel does not apply to these arguments");
    hipError_t e = launch_updat(a, dt, L.b, L.fa, stream);
    return e == hipSuccess ? BSMM_OK : dev_fail(e, "updat launch");
}
}  // namespace

extern "C" {

bsmm_status bsmm_updat(bsmm_handle h, const void* const* xs, const void* const* dys, int group, void* dw,
                       int64_t N, bsmm_dtype dt, bsmm_dtype dw_dt, void* ws, size_t ws_bytes, void* stream) {
    return updat_call(h, xs, dys, group, dw, N, dt, dw_dt, ws, ws_bytes, stream, false);
}

bsmm_status bsmm_updat_accumulate(bsmm_handle h, const void* const* xs, const void* const* dys, int group,
                                  void* dw, int64_t N, bsmm_dtype dt, bsmm_dtype dw_dt, void* ws, size_t ws_bytes,
                                  void* stream) {
    return updat_call(h, xs, dys, group, dw, N, dt, dw_dt, ws, ws_bytes, stream, true);
}

}  // extern "C"

// ---- weight gradient without allocation ----
// The split weight-gradient kernels keep fp32 partial sums in a workspace.  For callers
// that cannot allocate, bsmm_updat_noalloc uses this fixed device array instead: one
// copy per GPU, held until the process ends, shared by every call on that GPU.  Host
// code never passes `scratch` itself (on the host the name is only a stand-in); it
// passes the device address hipGetSymbolAddress reports for the current device.
constexpr size_t kScratchBytes = 128ull << 20;
static __device__ __align__(256) float scratch[kScratchBytes / sizeof(float)];

namespace {
std::mutex g_scratch_mu;
std::map<int, void*> g_scratch;   // device ordinal -> that device's scratch address

// The current device's scratch address, looked up once per device (first call there).
bsmm_status scratch_address(void** out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return dev_fail(e, "hipGetDevice");
    std::lock_guard<std::mutex> guard(g_scratch_mu);
    auto it = g_scratch.find(dev);
    if (it != g_scratch.end()) {
        *out = it->second;
        return BSMM_OK;
    }
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return dev_fail(e, "hipGetSymbolAddress of the scratch array");
    g_scratch.emplace(dev, p);
    *out = p;
    return BSMM_OK;
}
}  // namespace

extern "C" {

bsmm_status bsmm_updat_noalloc(bsmm_handle h, const void* const* xs, const void* const* dys, int group, void* dw,
                               int64_t N, bsmm_dtype dt, bsmm_dtype dw_dt, void* stream) {
    bsmm_status s = check_call(h, N, dt);
    if (s != BSMM_OK) return s;
    size_t need = 0;
    if ((s = bsmm_workspace_size(h, BSMM_PASS_UPDAT, N, dt, &need)) != BSMM_OK) return s;
    if (need > kScratchBytes)
        return fail(BSMM_ERR_UNSUPPORTED, "this weight gradient needs " + std::to_string(need) +
                                              " bytes of workspace, more than the " + std::to_string(kScratchBytes) +
                                              "-byte scratch of the allocation-free entry point");
    void* ws = nullptr;
    if (need > 0 && (s = scratch_address(&ws)) != BSMM_OK) return s;
    return updat_call(h, xs, dys, group, dw, N, dt, dw_dt, ws, need, stream, false, true);
}

bsmm_status bsmm_identity_init(bsmm_handle h, void* w, bsmm_dtype dt, void* stream) {
    if (!h) return fail(BSMM_ERR_INVALID_ARG, "handle is NULL");
    if (!valid_dt(dt)) return fail(BSMM_ERR_INVALID_ARG, "bad dtype");
    const HostLut& L = h->lut;
    if (L.nnz == 0) return BSMM_OK;
    bsmm_status s = check_ptr(w, "w");
    if (s != BSMM_OK) return s;
    const DeviceLut* d = nullptr;
    if ((s = device_lut(h, stream, &d)) != BSMM_OK) return s;
    hipError_t e = launch_identity(w, d->coords, L.nnz, L.b, dt, stream);
    return e == hipSuccess ? BSMM_OK : dev_fail(e, "identity_init launch");
}

const char* bsmm_status_string(bsmm_status s) {
    switch (s) {
    case BSMM_OK: return "BSMM_OK";
    case BSMM_ERR_INVALID_ARG: return "BSMM_ERR_INVALID_ARG";
    case BSMM_ERR_UNSUPPORTED: return "BSMM_ERR_UNSUPPORTED";
    case BSMM_ERR_ALIGNMENT: return "BSMM_ERR_ALIGNMENT";
    case BSMM_ERR_DEVICE: return "BSMM_ERR_DEVICE";
    case BSMM_ERR_OOM: return "BSMM_ERR_OOM";
    }
    return "unknown bsmm_status";
}

const char* bsmm_last_error(void) { return g_err.c_str(); }

bsmm_status bsmm_force_kernel(bsmm_handle h, int pass, const char* name) {
    if (!h) return fail(BSMM_ERR_INVALID_ARG, "handle is NULL");
    if (pass < BSMM_PASS_FPROP || pass > BSMM_PASS_UPDAT) return fail(BSMM_ERR_INVALID_ARG, "pass must be fprop, bprop or updat");
    if (!name || !*name) {
        h->force[pass] = 0;
        return BSMM_OK;
    }
    const int k = pass == BSMM_PASS_UPDAT ? updat_kind_of_name(name) : mm_kind_of_name(name);
    if (k == 0) return fail(BSMM_ERR_INVALID_ARG, std::string("unknown kernel name for this pass: ") + name);
    h->force[pass] = k;
    return BSMM_OK;
}

bsmm_status bsmm_debug_lut(bsmm_handle h, int which, int64_t* out, int64_t cap, int64_t* len) {
    if (!h || !len || cap < 0 || (cap > 0 && !out)) return fail(BSMM_ERR_INVALID_ARG, "bad argument");
    const HostLut& L = h->lut;
    const std::vector<int32_t>* v = nullptr;
    switch (which) {
    case 0: v = &L.coords; break;
    case 1: v = &L.colptr; break;
    case 2: v = &L.colent; break;
    case 3: v = &L.rowptr; break;
    case 4: v = &L.rowent; break;
    case 5: v = &L.colorder; break;
    case 6: v = &L.roworder; break;
    case 7: v = &L.colwork; break;
    case 8: v = &L.rowwork; break;
    case 9: v = &L.ugroups; break;
    case 10: v = &L.colrec; break;
    case 11: v = &L.rowrec; break;
    case 12: v = &L.cgptr; break;
    case 13: v = &L.cgent; break;
    case 14: v = &L.rgptr; break;
    case 15: v = &L.rgent; break;
    case 16: v = &L.utiles; break;
    case 17: v = &L.utblk; break;
    case 18: v = &L.urest; break;
    case 19: v = &L.urids; break;
    case 20: v = &L.stiles; break;
    case 21: v = &L.stplan; break;
    case 22: v = &L.stids; break;
    default: return fail(BSMM_ERR_INVALID_ARG, "which must be in [0, 22]");
    }
    *len = (int64_t)v->size();
    const int64_t n = cap < *len ? cap : *len;
    for (int64_t i = 0; i < n; i++) out[i] = (*v)[i];
    return BSMM_OK;
}

// ---- layer norm ----
namespace {
bsmm_status ln_check(int64_t N, int64_t C, int axis, bsmm_dtype dt) {
    if (N < 0 || C < 0) return fail(BSMM_ERR_INVALID_ARG, "N and C must be >= 0");
    if (axis != 0 && axis != 1) return fail(BSMM_ERR_INVALID_ARG, "axis must be 0 or 1");
    if (!valid_dt(dt)) return fail(BSMM_ERR_INVALID_ARG, "bad dtype");
    if (N > INT32_MAX || C > INT32_MAX || N * C > INT32_MAX)
        return fail(BSMM_ERR_UNSUPPORTED, "a tensor above 2^31 elements");
    return BSMM_OK;
}
bsmm_status ln_plan_call(LnArgs& a, int64_t N, int64_t C, int axis, bsmm_dtype dt, bool grad, bool aligned) {
    a.N = N;
    a.C = C;
    a.axis = axis;
    a.dt = dt;
    if (ln_plan(a, grad, aligned) != 0)
        return fail(BSMM_ERR_UNSUPPORTED, "axis 1 row longer than the register-resident kernels hold");
    return BSMM_OK;
}
bsmm_status ln_ws(int64_t N, int64_t C, int axis, bool grad, const void* ws, size_t ws_bytes) {
    const size_t need = ln_workspace_bytes(N, C, axis, grad);
    if (need == 0) return BSMM_OK;
    if (!ws || ws_bytes < need) return fail(BSMM_ERR_INVALID_ARG, "workspace smaller than bsmm_layer_norm_workspace_size");
    if (!aligned16(ws)) return fail(BSMM_ERR_ALIGNMENT, "ws is not 16-byte aligned");
    return BSMM_OK;
}
bool params_aligned(const float* g, const float* b) { return aligned16(g) && aligned16(b); }
}  // namespace

bsmm_status bsmm_layer_norm_workspace_size(int64_t N, int64_t C, int axis, int grad, bsmm_dtype dt, size_t* bytes) {
    if (!bytes) return fail(BSMM_ERR_INVALID_ARG, "bytes is NULL");
    bsmm_status s = ln_check(N, C, axis, dt);
    if (s != BSMM_OK) return s;
    *bytes = ln_workspace_bytes(N, C, axis, grad != 0);
    return BSMM_OK;
}

bsmm_status bsmm_layer_norm(const void* x, const float* g, const float* b, void* y, float* mean, float* rstd,
                            int64_t N, int64_t C, int axis, float epsilon, int relu, bsmm_dtype dt, void* ws,
                            size_t ws_bytes, void* stream) {
    if (!(epsilon >= 0.f) || epsilon > 3.0e38f) return fail(BSMM_ERR_INVALID_ARG, "epsilon must be finite and >= 0");
    if ((mean == nullptr) != (rstd == nullptr)) return fail(BSMM_ERR_INVALID_ARG, "mean and rstd: both or neither");
    bsmm_status s = ln_check(N, C, axis, dt);
    if (s != BSMM_OK || N == 0 || C == 0) return s;
    if (!g || !b) return fail(BSMM_ERR_INVALID_ARG, "g / b is NULL");
    if ((s = check_ptr(x, "x")) != BSMM_OK || (s = check_ptr(y, "y")) != BSMM_OK) return s;
    if ((s = ln_ws(N, C, axis, false, ws, ws_bytes)) != BSMM_OK) return s;
    LnArgs a{};
    // 16-byte parameter loads need aligned g, b (axis 1); else one value per load
    if ((s = ln_plan_call(a, N, C, axis, dt, false, axis == 0 || params_aligned(g, b))) != BSMM_OK) return s;
    a.x = x;
    a.y = y;
    a.g = g;
    a.b = b;
    a.mean = mean;
    a.rstd = rstd;
    a.ws = (float*)ws;
    a.eps = epsilon;
    a.relu = relu ? 1 : 0;
    prof_events(BSMM_PASS_LAYER_NORM, &a.e0, &a.e1);
    hipError_t e = launch_layer_norm(a, false, stream);
    return e == hipSuccess ? BSMM_OK : dev_fail(e, "layer_norm launch");
}

bsmm_status bsmm_layer_norm_grad(const void* dy, const void* x, const float* g, const float* b, const float* mean,
                                 const float* rstd, void* dx, float* dg, float* db, int64_t N, int64_t C, int axis,
                                 int relu, bsmm_dtype dt, void* ws, size_t ws_bytes, void* stream) {
    bsmm_status s = ln_check(N, C, axis, dt);
    if (s != BSMM_OK || C == 0) return s;
    if (!dg || !db) return fail(BSMM_ERR_INVALID_ARG, "dg / db is NULL");
    if (N == 0) {   // no vectors: the parameter gradients are zero
        hipError_t e = launch_ln_zero_params(dg, db, C, stream);
        return e == hipSuccess ? BSMM_OK : dev_fail(e, "layer_norm_grad launch");
    }
    if (!g || !b || !mean || !rstd) return fail(BSMM_ERR_INVALID_ARG, "NULL parameter or statistics");
    if ((s = check_ptr(x, "x")) != BSMM_OK || (s = check_ptr(dy, "dy")) != BSMM_OK ||
        (s = check_ptr(dx, "dx")) != BSMM_OK)
        return s;
    if ((s = ln_ws(N, C, axis, true, ws, ws_bytes)) != BSMM_OK) return s;
    LnArgs a{};
    if ((s = ln_plan_call(a, N, C, axis, dt, true, axis == 0 || params_aligned(g, b))) != BSMM_OK) return s;
    a.x = x;
    a.dy = dy;
    a.dx = dx;
    a.g = g;
    a.b = b;
    a.mean = const_cast<float*>(mean);
    a.rstd = const_cast<float*>(rstd);
    a.dg = dg;
    a.db = db;
    a.ws = (float*)ws;
    a.relu = relu ? 1 : 0;
    prof_events(BSMM_PASS_LAYER_NORM_GRAD, &a.e0, &a.e1);
    hipError_t e = launch_layer_norm(a, true, stream);
    return e == hipSuccess ? BSMM_OK : dev_fail(e, "layer_norm_grad launch");
}

// ---- weight normalisation ----
namespace {
bsmm_status wn_setup(bsmm_handle h, float epsilon, int dt1, int dt2, WnArgs& a, const DeviceLut** d,
                     void* stream) {
    if (!h) return fail(BSMM_ERR_INVALID_ARG, "handle is NULL");
    if (!valid_dt(dt1) || !valid_dt(dt2)) return fail(BSMM_ERR_INVALID_ARG, "bad dtype");
    if (!(epsilon > 0.f) || epsilon > 3.0e38f) return fail(BSMM_ERR_INVALID_ARG, "epsilon must be finite and > 0");
    a.S = h->lut.S;
    a.b = h->lut.b;
    a.eps = epsilon;
    if (h->lut.nnz == 0) return BSMM_OK;
    return device_lut(h, stream, d);
}
}  // namespace

bsmm_status bsmm_l2_normalize(bsmm_handle h, const void* w, const float* gain, void* w_out, float* norms,
                              float epsilon, bsmm_dtype w_dt, bsmm_dtype out_dt, void* stream) {
    WnArgs a{};
    if (h && h->lut.nnz > 0) {
        bsmm_status s;
        if ((s = check_ptr(w, "w")) != BSMM_OK || (s = check_ptr(w_out, "w_out")) != BSMM_OK) return s;
    }
    const DeviceLut* d = nullptr;
    bsmm_status s = wn_setup(h, epsilon, w_dt, out_dt, a, &d, stream);
    if (s != BSMM_OK || h->lut.nnz == 0) return s;
    a.w = w;
    a.out = w_out;
    a.gain = gain;
    a.norms = norms;
    a.colptr = d->colptr;
    a.colent = d->colent;
    a.w_dt = w_dt;
    a.out_dt = out_dt;
    prof_events(BSMM_PASS_L2_NORMALIZE, &a.e0, &a.e1);
    hipError_t e = launch_l2_normalize(a, false, stream);
    return e == hipSuccess ? BSMM_OK : dev_fail(e, "l2_normalize launch");
}

bsmm_status bsmm_l2_normalize_grad(bsmm_handle h, const void* dy, const void* w, const float* gain, void* dw,
                                   float* dgain, float epsilon, bsmm_dtype dy_dt, bsmm_dtype w_dt, void* stream) {
    WnArgs a{};
    if (h && h->lut.nnz > 0) {
        bsmm_status s;
        if ((s = check_ptr(dy, "dy")) != BSMM_OK || (s = check_ptr(w, "w")) != BSMM_OK ||
            (s = check_ptr(dw, "dw")) != BSMM_OK)
            return s;
    }
    const DeviceLut* d = nullptr;
    bsmm_status s = wn_setup(h, epsilon, dy_dt, w_dt, a, &d, stream);
    if (s != BSMM_OK || h->lut.nnz == 0) return s;
    a.w = w;
    a.dy = dy;
    a.out = dw;
    a.gain = gain;
    a.dgain = dgain;
    a.colptr = d->colptr;
    a.colent = d->colent;
    a.w_dt = w_dt;
    a.dy_dt = dy_dt;
    prof_events(BSMM_PASS_L2_NORMALIZE_GRAD, &a.e0, &a.e1);
    hipError_t e = launch_l2_normalize(a, true, stream);
    return e == hipSuccess ? BSMM_OK : dev_fail(e, "l2_normalize_grad launch");
}

bsmm_status bsmm_profile_begin(void) {
    g_prof.on = true;
    return BSMM_OK;
}

bsmm_status bsmm_profile_end(double ms[BSMM_NUM_PASSES], int64_t count[BSMM_NUM_PASSES]) {
    if (!g_prof.on) return fail(BSMM_ERR_INVALID_ARG, "profiling was not begun on this thread");
    g_prof.on = false;
    if (ms)
        for (int i = 0; i < BSMM_NUM_PASSES; i++) ms[i] = 0.0;
    if (count)
        for (int i = 0; i < BSMM_NUM_PASSES; i++) count[i] = 0;
    bsmm_status st = BSMM_OK;
    for (auto& r : g_prof.recs) {
        hipError_t e = hipEventSynchronize(r.e1);
        float t = 0.f;
        if (e == hipSuccess) e = hipEventElapsedTime(&t, r.e0, r.e1);
        if (e != hipSuccess && st == BSMM_OK) st = dev_fail(e, "profile event");
        if (r.pass >= 0 && r.pass < BSMM_NUM_PASSES) {
            if (ms) ms[r.pass] += t;
            if (count) count[r.pass] += 1;
        }
        g_prof.pool.push_back(r.e0);
        g_prof.pool.push_back(r.e1);
    }
    g_prof.recs.clear();
    return st;
}

}  // extern "C"

// ---- SparseProj ----
namespace {

bsmm_status proj_device(bsmm_proj_plan* h, void* stream, const int32_t** d) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return dev_fail(e, "hipGetDevice");
    std::lock_guard<std::mutex> guard(h->mu);
    auto it = h->dev.find(dev);
    if (it != h->dev.end()) {
        *d = it->second;
        return BSMM_OK;
    }
    if (h->image.empty()) {   // lut then inv, kept for the copies to later devices
        h->image = h->lut;
        h->image.insert(h->image.end(), h->inv.begin(), h->inv.end());
    }
    void* p = nullptr;
    bsmm_status st = upload_tables(h->image.data(), h->image.size() * sizeof(int32_t), stream, "projection map", &p);
    if (st != BSMM_OK) return st;
    h->dev.emplace(dev, (int32_t*)p);
    *d = (const int32_t*)p;
    return BSMM_OK;
}

// base / src / out per ProjMode (see kernels.h); widths follow from the mode
bsmm_status proj_call(bsmm_proj_handle h, int mode, const void* base, const void* src, void* out, int64_t N,
                      int fa, bsmm_dtype dt, void* stream) {
    if (!h) return fail(BSMM_ERR_INVALID_ARG, "handle is NULL");
    if (N < 0) return fail(BSMM_ERR_INVALID_ARG, "N must be >= 0");
    if (fa != 0 && fa != 1) return fail(BSMM_ERR_INVALID_ARG, "feature_axis must be 0 or 1");
    if (!valid_dt(dt)) return fail(BSMM_ERR_INVALID_ARG, "dtype must be BSMM_F32, BSMM_BF16 or BSMM_F16");
    const bool to_proj = mode == PROJ_GATHER || mode == PROJ_GATHER_MUL;
    const int64_t wout = to_proj ? h->nproj : h->nhidden, wsrc = to_proj ? h->nhidden : h->nproj;
    if (N == 0 || wout == 0) return BSMM_OK;
    bsmm_status s;
    if ((s = check_ptr(src, mode == PROJ_GATHER_MUL ? "b" : mode >= PROJ_ADD ? "y" : "x")) != BSMM_OK) return s;
    if ((s = check_ptr(out, mode == PROJ_GATHER ? "y" : mode == PROJ_SCATTER ? "y" : mode == PROJ_GATHER_MUL ? "g" : "z")) != BSMM_OK)
        return s;
    if (mode >= PROJ_ADD && (s = check_ptr(base, mode == PROJ_GATHER_MUL ? "a" : "x")) != BSMM_OK) return s;
    if (wsrc > 0 && (uint64_t)N > (uint64_t)INT64_MAX / 8 / (uint64_t)std::max(wout, wsrc))
        return fail(BSMM_ERR_UNSUPPORTED, "tensor too large");
    const int32_t* d = nullptr;
    if ((s = proj_device(h, stream, &d)) != BSMM_OK) return s;
    ProjArgs a{};
    a.base = base;
    a.src = src;
    a.out = out;
    a.map = to_proj ? d : d + h->nproj;
    a.N = N;
    a.wout = wout;
    a.wsrc = wsrc;
    a.mode = mode;
    a.fa = fa;
    a.dt = dt;
    hipError_t e = launch_proj(a, stream);
    return e == hipSuccess ? BSMM_OK : dev_fail(e, "SparseProj launch");
}

}  // namespace

extern "C" {

bsmm_status bsmm_proj_create(bsmm_proj_handle* out, int64_t nhidden, int64_t nproj, int64_t proj_stride,
                             int64_t block_size, const int32_t* gather_lut) {
    if (!out) return fail(BSMM_ERR_INVALID_ARG, "out is NULL");
    *out = nullptr;
    if (nhidden < 1 || nhidden > INT32_MAX) return fail(BSMM_ERR_INVALID_ARG, "nhidden must be in [1, 2^31-1]");
    std::vector<int32_t> lut;
    if (gather_lut) {
        if (nproj < 0 || nproj > nhidden) return fail(BSMM_ERR_INVALID_ARG, "nproj must be in [0, nhidden]");
        lut.assign(gather_lut, gather_lut + nproj);
    } else {
        if (block_size < 1) return fail(BSMM_ERR_INVALID_ARG, "block_size must be >= 1");
        const int64_t np = nproj > 0 ? nproj : nhidden;
        const int64_t st = proj_stride > 0 ? proj_stride : block_size;
        if (np % block_size != 0) return fail(BSMM_ERR_INVALID_ARG, "nproj must be a multiple of block_size");
        if (st < block_size) return fail(BSMM_ERR_INVALID_ARG, "proj_stride must be >= block_size");
        const int64_t nb = np / block_size;
        if (np > nhidden || (nb - 1) * st + block_size > nhidden)
            return fail(BSMM_ERR_INVALID_ARG, "the projected blocks run past nhidden");
        lut.reserve(np);
        for (int64_t j = 0; j < nb; j++)
            for (int64_t i = 0; i < block_size; i++) lut.push_back((int32_t)(j * st + i));
    }
    std::vector<int32_t> inv(nhidden, -1);
    for (size_t p = 0; p < lut.size(); p++) {
        const int32_t hf = lut[p];
        if (hf < 0 || hf >= nhidden) return fail(BSMM_ERR_INVALID_ARG, "gather_lut entry outside [0, nhidden)");
        if (inv[hf] >= 0) return fail(BSMM_ERR_INVALID_ARG, "gather_lut maps two projected features to one hidden feature");
        inv[hf] = (int32_t)p;
    }
    bsmm_proj_plan* p = new (std::nothrow) bsmm_proj_plan();
    if (!p) return fail(BSMM_ERR_OOM, "out of host memory");
    p->nhidden = nhidden;
    p->nproj = (int64_t)lut.size();
    p->lut = std::move(lut);
    p->inv = std::move(inv);
    *out = p;
    return BSMM_OK;
}

void bsmm_proj_destroy(bsmm_proj_handle h) {
    if (!h) return;
    for (auto& kv : h->dev) {
        int cur = 0;
        if (hipGetDevice(&cur) == hipSuccess && hipSetDevice(kv.first) == hipSuccess) {
            (void)hipFree(kv.second);
            (void)hipSetDevice(cur);
        }
    }
    delete h;
}

bsmm_status bsmm_proj_info(bsmm_proj_handle h, int64_t* nhidden, int64_t* nproj) {
    if (!h || !nhidden || !nproj) return fail(BSMM_ERR_INVALID_ARG, "NULL argument");
    *nhidden = h->nhidden;
    *nproj = h->nproj;
    return BSMM_OK;
}

bsmm_status bsmm_proj_lut(bsmm_proj_handle h, int32_t* out, int64_t cap) {
    if (!h || (cap > 0 && !out) || cap < 0) return fail(BSMM_ERR_INVALID_ARG, "bad argument");
    const int64_t n = std::min<int64_t>(cap, h->nproj);
    for (int64_t i = 0; i < n; i++) out[i] = h->lut[i];
    return BSMM_OK;
}

bsmm_status bsmm_proj_gather(bsmm_proj_handle h, const void* x, void* y, int64_t N, int feature_axis,
                             bsmm_dtype dt, void* stream) {
    return proj_call(h, PROJ_GATHER, nullptr, x, y, N, feature_axis, dt, stream);
}

bsmm_status bsmm_proj_scatter(bsmm_proj_handle h, const void* x, void* y, int64_t N, int feature_axis,
                              bsmm_dtype dt, void* stream) {
    return proj_call(h, PROJ_SCATTER, nullptr, x, y, N, feature_axis, dt, stream);
}

bsmm_status bsmm_proj_scatter_add(bsmm_proj_handle h, const void* x, const void* y, void* z, int64_t N,
                                  int feature_axis, bsmm_dtype dt, void* stream) {
    return proj_call(h, PROJ_ADD, x, y, z, N, feature_axis, dt, stream);
}

bsmm_status bsmm_proj_scatter_mul(bsmm_proj_handle h, const void* x, const void* y, void* z, int64_t N,
                                  int feature_axis, bsmm_dtype dt, void* stream) {
    return proj_call(h, PROJ_MUL, x, y, z, N, feature_axis, dt, stream);
}

bsmm_status bsmm_proj_gather_mul(bsmm_proj_handle h, const void* a, const void* b, void* g, int64_t N,
                                 int feature_axis, bsmm_dtype dt, void* stream) {
    return proj_call(h, PROJ_GATHER_MUL, a, b, g, N, feature_axis, dt, stream);
}

}  // extern "C"

// ---- BlocksparseConv ----
namespace {

// device copy of the conv tables; offsets (int32 elements) of each array in `off`
constexpr int kConvParts = 12;
bsmm_status conv_device(bsmm_conv_plan* h, void* stream, const int32_t** d, size_t off[kConvParts]) {
    const std::vector<int32_t>* parts[kConvParts] = {&h->cidx,    &h->kidx,    &h->kptr,   &h->kent,
                                                     &h->cptr,    &h->cent,    &h->gptr[0], &h->gblk[0],
                                                     &h->zch[0],  &h->gptr[1], &h->gblk[1], &h->zch[1]};
    size_t total = 0;
    for (int i = 0; i < kConvParts; i++) {
        off[i] = total;
        total += parts[i]->size();
    }
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return dev_fail(e, "hipGetDevice");
    std::lock_guard<std::mutex> guard(h->mu);
    auto it = h->dev.find(dev);
    if (it != h->dev.end()) {
        *d = it->second;
        return BSMM_OK;
    }
    if (h->image.empty() && total > 0) {   // kept for the copies to later devices
        h->image.reserve(total);
        for (int i = 0; i < kConvParts; i++) h->image.insert(h->image.end(), parts[i]->begin(), parts[i]->end());
    }
    void* p = nullptr;
    bsmm_status st = upload_tables(h->image.data(), total * sizeof(int32_t), stream, "conv tables", &p);
    if (st != BSMM_OK) return st;
    h->dev.emplace(dev, (int32_t*)p);
    *d = (const int32_t*)p;
    return BSMM_OK;
}

// the plan's sizes and geometry as kernel arguments (no device pointers)
ConvArgs conv_args(const bsmm_conv_plan* h, int dt) {
    ConvArgs x{};
    x.C = h->C;
    x.K = h->K;
    x.nb = h->nb;
    x.Bc = h->Bc;
    x.Bk = h->Bk;
    x.T = h->TRS[0]; x.R = h->TRS[1]; x.S = h->TRS[2];
    x.D = h->DHW[0]; x.H = h->DHW[1]; x.W = h->DHW[2];
    x.M = h->MPQ[0]; x.P = h->MPQ[1]; x.Q = h->MPQ[2];
    for (int i = 0; i < 3; i++) {
        x.st[i] = h->st[i];
        x.dl[i] = h->dl[i];
        x.pad[i] = h->pad[i];
    }
    x.dt = dt;
    return x;
}

// Workspace bytes of the filter gradient's contraction split for N images (0: none).
size_t conv_ws_bytes(const bsmm_conv_plan* h, int64_t N, int dt) {
    if (N <= 0 || h->nb == 0) return 0;
    ConvArgs x = conv_args(h, dt);
    x.N = N;
    x.a_bytes = x.b_bytes = 1;
    if (!conv_mfma_updat_ok(x) && !conv_gather_updat_ok(x)) return 0;
    const int p = conv_updat_parts(x);
    if (p <= 1) return 0;
    return (size_t)p * h->nb * h->Bc * h->TRS[0] * h->TRS[1] * h->TRS[2] * h->Bk * sizeof(float);
}

bsmm_status conv_call(bsmm_conv_handle h, int pass, const void* a, const void* b, void* out, int64_t N,
                      bsmm_dtype dt, void* stream, void* ws = nullptr, size_t ws_bytes = 0) {
    if (!h) return fail(BSMM_ERR_INVALID_ARG, "handle is NULL");
    if (N < 0) return fail(BSMM_ERR_INVALID_ARG, "N must be >= 0");
    if (!valid_dt(dt)) return fail(BSMM_ERR_INVALID_ARG, "dtype must be BSMM_F32, BSMM_BF16 or BSMM_F16");
    if (N == 0 && pass != 2) return BSMM_OK;   // updat with N = 0 writes dF = 0
    bsmm_status s;
    const char* na = pass == 1 ? "dO" : "I";
    const char* nb = pass == 2 ? "dO" : "F";
    const char* no = pass == 0 ? "O" : pass == 1 ? "dI" : "dF";
    if (pass == 2 && h->nb == 0) return BSMM_OK;
    if ((s = check_ptr(out, no)) != BSMM_OK) return s;
    if (N > 0 && (s = check_ptr(a, na)) != BSMM_OK) return s;
    if (N > 0 && (h->nb > 0 || pass == 2) && (s = check_ptr(b, nb)) != BSMM_OK) return s;
    const int64_t sp_in = (int64_t)h->DHW[0] * h->DHW[1] * h->DHW[2], sp_out = (int64_t)h->MPQ[0] * h->MPQ[1] * h->MPQ[2];
    if ((uint64_t)N > (uint64_t)INT64_MAX / 8 / (uint64_t)std::max<int64_t>(1, std::max(h->C * sp_in, h->K * sp_out)))
        return fail(BSMM_ERR_UNSUPPORTED, "tensor too large");
    const int32_t* d = nullptr;
    size_t off[kConvParts];
    if ((s = conv_device(h, stream, &d, off)) != BSMM_OK) return s;
    ConvArgs x = conv_args(h, dt);
    {
        const uint64_t es = dt == BSMM_F32 ? 4 : 2;
        const uint64_t ab = (uint64_t)N * es * (pass == 1 ? (uint64_t)h->K * sp_out : (uint64_t)h->C * sp_in);
        x.a_bytes = ab <= kMaxTensorBytes ? (uint32_t)ab : 0u;
        if (pass == 2) {   // b is dO
            const uint64_t bb = (uint64_t)N * es * (uint64_t)h->K * sp_out;
            x.b_bytes = bb <= kMaxTensorBytes ? (uint32_t)bb : 0u;
        }
    }
    x.a = a;
    x.b = b;
    x.out = out;
    x.cidx = d + off[0];
    x.kidx = d + off[1];
    x.lptr = pass == 0 ? d + off[2] : d + off[4];
    x.lent = pass == 0 ? d + off[3] : d + off[5];
    x.N = N;
    x.nparts = 1;
    if (pass == 2) {   // split the matrix-core filter gradient when the workspace allows it
        const size_t need = conv_ws_bytes(h, N, dt);
        if (need > 0 && ws && ws_bytes >= need && aligned16(ws)) {
            x.nparts = conv_updat_parts(x);
            x.ws = (float*)ws;
        }
    }
    if (pass < 2 && h->gok[pass] && h->gptr[pass].size() > 1) {
        if (conv_mfma_plan(x, pass))
            x.mfma = 1;
        else if (conv_gather_ok(x, pass) && (N == 0 || h->nb == 0 || aligned16(b)))
            x.mfma = 2;
    }
    if (x.mfma) {
        x.gptr = d + off[pass == 0 ? 6 : 9];
        x.gblk = d + off[pass == 0 ? 7 : 10];
        x.zch = d + off[pass == 0 ? 8 : 11];
        x.ngroups = (int)h->gptr[pass].size() - 1;
        x.nz = (int)h->zch[pass].size();
    }
    hipError_t e = launch_conv(x, pass, stream);
    return e == hipSuccess ? BSMM_OK : dev_fail(e, pass == 0 ? "conv fprop launch" : pass == 1 ? "conv bprop launch"
                                                                                             : "conv updat launch");
}

}  // namespace

extern "C" {

bsmm_status bsmm_conv_create(bsmm_conv_handle* out, int64_t nblocks, int64_t Bc, int64_t Bk, const int32_t* cidx,
                             const int32_t* kidx, int64_t C, int64_t K, const int64_t TRS[3], const int64_t DHW[3],
                             const int64_t strides[3], const int64_t dilates[3], int padding,
                             const int64_t pads[3]) {
    if (!out) return fail(BSMM_ERR_INVALID_ARG, "out is NULL");
    *out = nullptr;
    if (nblocks < 0 || nblocks > INT32_MAX / 2) return fail(BSMM_ERR_INVALID_ARG, "nblocks out of range");
    if (Bc < 1 || Bk < 1 || Bk > 64 || Bc > 65536) return fail(BSMM_ERR_INVALID_ARG, "Bc must be >= 1, Bk in [1, 64]");
    if (nblocks > 0 && (!cidx || !kidx)) return fail(BSMM_ERR_INVALID_ARG, "channel lists are NULL");
    if (C < 1 || K < 1 || C > INT32_MAX || K > INT32_MAX) return fail(BSMM_ERR_INVALID_ARG, "C and K must be >= 1");
    if (!TRS || !DHW || !strides || !dilates) return fail(BSMM_ERR_INVALID_ARG, "geometry arrays are NULL");
    if (padding < 0 || padding > 2 || (padding == 2 && !pads))
        return fail(BSMM_ERR_INVALID_ARG, "padding must be 0 (SAME), 1 (VALID) or 2 (explicit pads)");
    bsmm_conv_plan* p = new (std::nothrow) bsmm_conv_plan();
    if (!p) return fail(BSMM_ERR_OOM, "out of host memory");
    auto reject = [&](const char* msg) {
        delete p;
        return fail(BSMM_ERR_INVALID_ARG, msg);
    };
    for (int a = 0; a < 3; a++) {
        if (TRS[a] < 1 || DHW[a] < 1 || strides[a] < 1 || dilates[a] < 1 || TRS[a] > 4096 || DHW[a] > (1 << 20) ||
            strides[a] > 4096 || dilates[a] > 4096)
            return reject("filter, image, stride and dilation sizes must be >= 1");
        const int64_t X = DHW[a], F = TRS[a], st = strides[a], dl = dilates[a];
        int64_t o, pd;
        if (padding == 0) {            // SAME
            o = (X + st - 1) / st;
            pd = std::max<int64_t>(0, (o - 1) * st + (F - 1) * dl + 1 - X) / 2;
        } else if (padding == 1) {     // VALID
            pd = 0;
            o = X - (F - 1) * dl - 1 >= 0 ? (X - (F - 1) * dl - 1) / st + 1 : 0;
        } else {
            pd = pads[a];
            if (pd < 0 || pd > 4096) return reject("explicit pads must be in [0, 4096]");
            o = X + 2 * pd - (F - 1) * dl - 1 >= 0 ? (X + 2 * pd - (F - 1) * dl - 1) / st + 1 : 0;
        }
        if (o < 1) return reject("the filter does not fit the padded image");
        p->TRS[a] = (int)F;
        p->DHW[a] = (int)X;
        p->MPQ[a] = (int)o;
        p->st[a] = (int)st;
        p->dl[a] = (int)dl;
        p->pad[a] = (int)pd;
    }
    p->C = C;
    p->K = K;
    p->nb = (int)nblocks;
    p->Bc = (int)Bc;
    p->Bk = (int)Bk;
    p->cidx.assign(cidx ? cidx : nullptr, cidx ? cidx + nblocks * Bc : nullptr);
    p->kidx.assign(kidx ? kidx : nullptr, kidx ? kidx + nblocks * Bk : nullptr);
    for (int64_t b = 0; b < nblocks; b++) {
        for (int64_t i = 0; i < Bc; i++) {
            const int32_t c = p->cidx[b * Bc + i];
            if (c < 0 || c >= C) return reject("an input channel index is outside [0, C)");
            for (int64_t i2 = 0; i2 < i; i2++)
                if (p->cidx[b * Bc + i2] == c) return reject("a block lists an input channel twice");
        }
        for (int64_t j = 0; j < Bk; j++) {
            const int32_t k = p->kidx[b * Bk + j];
            if (k < 0 || k >= K) return reject("an output channel index is outside [0, K)");
            for (int64_t j2 = 0; j2 < j; j2++)
                if (p->kidx[b * Bk + j2] == k) return reject("a block lists an output channel twice");
        }
    }
    // per-channel (block, position) lists in block order: counting sort
    auto lists = [&](int64_t nch, int64_t per, const std::vector<int32_t>& idx, std::vector<int32_t>& ptr,
                     std::vector<int32_t>& ent) {
        ptr.assign(nch + 1, 0);
        for (int32_t v : idx) ptr[v + 1]++;
        for (int64_t c = 0; c < nch; c++) ptr[c + 1] += ptr[c];
        ent.assign(2 * idx.size(), 0);
        std::vector<int32_t> fill(ptr.begin(), ptr.end() - 1);
        for (int64_t b = 0; b < nblocks; b++)
            for (int64_t i = 0; i < per; i++) {
                const int32_t pos = fill[idx[b * per + i]]++;
                ent[2 * pos] = (int32_t)b;
                ent[2 * pos + 1] = (int32_t)i;
            }
    };
    lists(K, Bk, p->kidx, p->kptr, p->kent);
    lists(C, Bc, p->cidx, p->cptr, p->cent);
    // matrix-core grouping: blocks with identical output lists form a group; groups must
    // not share a channel
    auto group = [&](int pass, int64_t nch, int64_t per, const std::vector<int32_t>& idx) {
        std::map<std::vector<int32_t>, int32_t> gid;
        std::vector<std::vector<int32_t>> members;
        for (int64_t b = 0; b < nblocks; b++) {
            std::vector<int32_t> key(idx.begin() + b * per, idx.begin() + (b + 1) * per);
            auto it = gid.find(key);
            if (it == gid.end()) {
                it = gid.emplace(key, (int32_t)members.size()).first;
                members.emplace_back();
            }
            members[it->second].push_back((int32_t)b);
        }
        std::vector<int32_t> owner(nch, -1);
        bool ok = true;
        for (size_t g = 0; g < members.size(); g++) {
            const int64_t b = members[g][0];
            for (int64_t i = 0; i < per; i++) {
                int32_t& o = owner[idx[b * per + i]];
                if (o >= 0 && o != (int32_t)g) ok = false;
                o = (int32_t)g;
            }
        }
        p->gok[pass] = ok;
        p->gptr[pass].assign(1, 0);
        p->gblk[pass].clear();
        p->zch[pass].clear();
        if (!ok) return;
        for (auto& m : members) {
            p->gblk[pass].insert(p->gblk[pass].end(), m.begin(), m.end());
            p->gptr[pass].push_back((int32_t)p->gblk[pass].size());
        }
        for (int64_t c = 0; c < nch; c++)
            if (owner[c] < 0) p->zch[pass].push_back((int32_t)c);
    };
    group(0, K, Bk, p->kidx);
    group(1, C, Bc, p->cidx);
    *out = p;
    return BSMM_OK;
}

void bsmm_conv_destroy(bsmm_conv_handle h) {
    if (!h) return;
    for (auto& kv : h->dev) {
        int cur = 0;
        if (hipGetDevice(&cur) == hipSuccess && hipSetDevice(kv.first) == hipSuccess) {
            (void)hipFree(kv.second);
            (void)hipSetDevice(cur);
        }
    }
    delete h;
}

bsmm_status bsmm_conv_geometry(bsmm_conv_handle h, int64_t MPQ[3], int64_t pads[3]) {
    if (!h || !MPQ || !pads) return fail(BSMM_ERR_INVALID_ARG, "NULL argument");
    for (int a = 0; a < 3; a++) {
        MPQ[a] = h->MPQ[a];
        pads[a] = h->pad[a];
    }
    return BSMM_OK;
}

bsmm_status bsmm_conv_kernel_name(bsmm_conv_handle h, int pass, bsmm_dtype dt, const char** name) {
    if (!h || !name || pass < 0 || pass > 2) return fail(BSMM_ERR_INVALID_ARG, "bad argument");
    if (!valid_dt(dt)) return fail(BSMM_ERR_INVALID_ARG, "bad dtype");
    ConvArgs x = conv_args(h, dt);
    x.a_bytes = x.b_bytes = 1;   // the choice assuming the pass's inputs are below 2 GiB
    const bool grouped = pass < 2 && h->gok[pass] && h->gptr[pass].size() > 1;
    if (pass == 2)
        *name = conv_mfma_updat_ok(x) ? "matrix_core" : conv_gather_updat_ok(x) ? "matrix_core_gather" : "direct";
    else if (grouped && conv_mfma_plan(x, pass))
        *name = "matrix_core";
    else
        *name = grouped && conv_gather_ok(x, pass) ? "matrix_core_gather" : "direct";
    return BSMM_OK;
}

bsmm_status bsmm_conv_fprop(bsmm_conv_handle h, const void* F, const void* I, void* O, int64_t N, bsmm_dtype dt,
                            void* stream) {
    return conv_call(h, 0, I, F, O, N, dt, stream);
}

bsmm_status bsmm_conv_bprop(bsmm_conv_handle h, const void* F, const void* dO, void* dI, int64_t N, bsmm_dtype dt,
                            void* stream) {
    return conv_call(h, 1, dO, F, dI, N, dt, stream);
}

bsmm_status bsmm_conv_workspace_size(bsmm_conv_handle h, int64_t N, bsmm_dtype dt, size_t* bytes) {
    if (!h || !bytes || N < 0) return fail(BSMM_ERR_INVALID_ARG, "bad argument");
    if (!valid_dt(dt)) return fail(BSMM_ERR_INVALID_ARG, "bad dtype");
    *bytes = conv_ws_bytes(h, N, dt);
    return BSMM_OK;
}

bsmm_status bsmm_conv_updat(bsmm_conv_handle h, const void* I, const void* dO, float* dF, int64_t N, bsmm_dtype dt,
                            void* ws, size_t ws_bytes, void* stream) {
    return conv_call(h, 2, I, dO, dF, N, dt, stream, ws, ws_bytes);
}

}  // extern "C"
