// sata_api.cpp -- the C ABI of libsata (include/sata.h): argument checks, the
// tables handle and its workspace, and the launch sequence of each entry point.
//
// Prefill ([TA] "Feature maps and linear attention", evaluated by chunks):
//   for each segment of whole chunks (one segment unless the slice partials of
//   the whole sequence would exceed the workspace cap):
//     scan      per (head, feature slice), sequential over the segment's chunks:
//               partial readouts against the state, then the state update
//     finalize  per (head, chunk): intra-chunk direct part + sum of partials, y
//   The state of a slice is carried from one segment to the next through the
//   caller's state buffer (or a workspace copy when the caller passed none).
// Decode: one streaming read-modify-write kernel over the state, then a per-head
//   reduction of the partial readouts.
// Backward: a fp32 forward recompute (y and the normaliser of every row), then the
//   gradient scans of kern_backward.hip: dq with the forward state in chunk order,
//   dk and dv with its mirror in reverse chunk order.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <utility>
#include <vector>

#include "../../include/sata.h"
#include "launch.h"
#include "scan_mfma.h"
#include "tables.h"

// Per-handle kernel timer: HIP event pairs recorded around launches on the
// launch stream, resolved only by sata_read_timing.
struct KernelTimer {
    bool enabled = false;
    std::vector<std::pair<hipEvent_t, hipEvent_t>> pending[SATA_NUM_KERNELS];
    std::vector<hipEvent_t> pool;

    hipEvent_t take() {
        if (!pool.empty()) {
            hipEvent_t e = pool.back();
            pool.pop_back();
            return e;
        }
        hipEvent_t e = nullptr;
        if (hipEventCreate(&e) != hipSuccess) return nullptr;
        return e;
    }
    // Returns the start event (or nullptr when timing is off or an event failed).
    hipEvent_t begin(hipStream_t st) {
        if (!enabled) return nullptr;
        hipEvent_t e = take();
        if (e && hipEventRecord(e, st) != hipSuccess) {
            pool.push_back(e);
            return nullptr;
        }
        return e;
    }
    void end(int kind, hipEvent_t start, hipStream_t st) {
        if (!start) return;
        hipEvent_t e = take();
        if (!e || hipEventRecord(e, st) != hipSuccess) {
            pool.push_back(start);
            if (e) pool.push_back(e);
            return;
        }
        pending[kind].emplace_back(start, e);
    }
    void recycle() {
        for (auto& v : pending) {
            for (auto& pr : v) {
                pool.push_back(pr.first);
                pool.push_back(pr.second);
            }
            v.clear();
        }
    }
    void destroy() {
        recycle();
        for (hipEvent_t e : pool) (void)hipEventDestroy(e);
        pool.clear();
    }
};

// Default cap on the workspace of one call (about 11% of the 288 GB of an MI355X); a
// prefill whose slice partials need more runs in segments of whole readout windows.  Each
// segment boundary stores and reloads every head's state and restarts every workgroup:
// measured on the Long prefill (4 x 16 heads of 65536 tokens) 2 segments under this cap
// against 4 under 16 GiB cost 98.9 against 103.7 ms, on the Wide one (32 heads, d = 128)
// 4 segments against 7 cost 260 against 317 ms.  sata_prefill_workspace reports the need.
constexpr int64_t kDefaultWorkspace = 32LL << 30;

struct sata_tables {
    sata::HostTables h;
    KernelTimer timer;
    int device = -1;
    uint32_t* d_fidx = nullptr;
    float* d_qw = nullptr;
    uint32_t* d_fidx_h = nullptr;     // the same in the row order of the half-precision state
    float* d_qw_h = nullptr;
    sata::MfmaTables mfma;            // slice tables of the MFMA scan (may be empty)
    std::mutex mu;
    // one workspace per stream the handle is used on: calls on one stream run in order, and
    // calls on different streams never share workspace memory
    struct Workspace {
        hipStream_t stream;
        void* ptr;
        size_t bytes;
    };
    std::vector<Workspace> ws;
    int64_t ws_limit = kDefaultWorkspace;
    int cus = 0;                      // compute units of the device (256 assumed host-only)
    int split = 0;                    // two-level prefill: 0 automatic, 1 never, k >= 2 forced
    int mfma_slices = 0;              // feature slices of the matrix-core scan (0: not its shape)
};

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return code;
}

void clear_err() { g_err[0] = '\0'; }

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

int check_device(const sata_tables* t) {
    if (t->device < 0) return fail(SATA_ERR_ARG, "host-only handle: it has no device tables");
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) return fail(SATA_ERR_HIP, "hipGetDevice failed");
    if (dev != t->device)
        return fail(SATA_ERR_ARG, "handle was built on device %d but device %d is current",
                    t->device, dev);
    return SATA_OK;
}

// The workspace of stream `st`, grown to at least `bytes` (*out receives it).  Growth waits
// for `st` (the only user of that buffer), frees the old buffer and allocates.
int ensure_ws(sata_tables* t, size_t bytes, hipStream_t st, char** out) {
    sata_tables::Workspace* w = nullptr;
    for (auto& e : t->ws)
        if (e.stream == st) w = &e;
    if (!w) {
        t->ws.push_back(sata_tables::Workspace{st, nullptr, 0});
        w = &t->ws.back();
    }
    if (bytes > w->bytes) {
        if (w->ptr) {
            if (hipStreamSynchronize(st) != hipSuccess)
                return fail(SATA_ERR_HIP, "hipStreamSynchronize failed while growing the workspace");
            (void)hipFree(w->ptr);
            w->ptr = nullptr;
            w->bytes = 0;
        }
        const size_t rounded = (bytes + (1u << 20) - 1) & ~(size_t)((1u << 20) - 1);
        if (hipMalloc(&w->ptr, rounded) != hipSuccess) {
            (void)hipGetLastError();
            w->ptr = nullptr;
            return fail(SATA_ERR_OOM, "cannot allocate a %zu-byte workspace", rounded);
        }
        w->bytes = rounded;
    }
    if (out) *out = (char*)w->ptr;
    return SATA_OK;
}

int check_sizes(int d_K, int d_V, int P) {
    if (d_K < 1 || d_K > sata::kMaxD || d_V < 1 || d_V > sata::kMaxD || P < 1 || P > sata::kMaxP)
        return fail(SATA_ERR_UNSUPPORTED,
                    "unsupported sizes d_K=%d d_V=%d P=%d (need 1..128, 1..128, 1..5)", d_K,
                    d_V, P);
    return SATA_OK;
}

// How a prefill of these sizes runs: which scan, how the feature axis is sliced, how the
// sequence is cut (two-level sub-segments, or segments of whole readout windows under the
// workspace cap) and the workspace that takes.
struct PrefillPlan {
    bool mfma = false;
    int win = 1;                 // chunks per readout window
    int nslices = 0, slice_feats = 0;
    int nchunks = 0;
    int64_t part_chunk = 0;      // slice-partial bytes of one chunk of every head
    int64_t img_chunk = 0;       // operand-image bytes of one chunk of every head (matrix cores)
    int64_t per_chunk = 0;       // part_chunk + img_chunk
    int64_t fixed = 0;           // per-head input maxima (matrix cores)
    int64_t state_b = 0;         // bytes of one state per head, all heads
    int64_t s32_b = 0;           // fp32 working state of a call with a half-precision state
    int nsub = 1, sub_chunks = 0; // two-level form when nsub >= 2
    int pps = 1;                 // two-level: pieces per sub-segment in the update-only pass
    int seg = 0, nseg = 1;       // one-level form: segments of seg chunks
    int64_t ws_bytes = 0;
    // workspace layout (byte offsets): partials, carried state, operand images, maxima,
    // fp32 working state
    int64_t off_carrier = 0, off_img = 0, off_max = 0, off_s32 = 0;
};

int64_t round256(int64_t b) { return (b + 255) / 256 * 256; }

// Segment length of the one-level form: whole readout windows (a segment starts a new
// window, so results do not depend on the segmentation), at least one window, segments of
// nearly equal length (each boundary stores and reloads the state of every slice), and
// per_chunk * seg + carrier + fixed <= limit whenever one window fits.  `whole` is the
// need of a single segment over all nchunks chunks (no carrier).
int64_t segment_chunks(int64_t nchunks, int64_t win, int64_t per_chunk, int64_t carrier,
                       int64_t fixed, int64_t whole, int64_t limit) {
    if (whole <= limit) return nchunks;
    int64_t seg = (limit - carrier - fixed) / per_chunk;
    seg -= seg % win;
    if (seg < win) seg = win;                          // one window even above the cap
    if (seg >= nchunks) return nchunks;
    const int64_t ns = (nchunks + seg - 1) / seg;
    const int64_t even = (nchunks + ns - 1) / ns;      // <= seg, since ns segments of seg cover
    return (even + win - 1) / win * win;               // whole windows, still <= seg
}

int plan_prefill(const sata_tables* t, int B, int H, int n, int d_V, int chunk, bool bf16,
                 bool has_state, bool cont, bool f16state, PrefillPlan& pl) {
    const int d_K = t->h.d_K, P = t->h.P, L = chunk, cols = d_V + 1;
    const int64_t BH = (int64_t)B * H;
    pl = PrefillPlan();
    pl.nchunks = (int)(((int64_t)n + L - 1) / L);
    pl.mfma = t->mfma_slices > 0 && sata::mfma_shape(bf16, d_K, d_V, P, L);
    if (pl.mfma) {
        pl.nslices = t->mfma_slices;
        pl.slice_feats = sata::kRowsPerSlice * 8;
        pl.win = sata::mfma_window(d_K);
    } else {
        pl.win = 1;
        pl.slice_feats = sata::valu_slice_feats(d_K, d_V, L);
        if (pl.slice_feats == 0) return fail(SATA_ERR_UNSUPPORTED, "no fp32 scan slice fits LDS");
        pl.nslices = (int)((t->h.M + pl.slice_feats - 1) / pl.slice_feats);
    }
    pl.part_chunk = BH * pl.nslices * 4 *
                    (pl.mfma ? sata::tiled_partial_floats(L, d_V) : (int64_t)L * cols);
    if (pl.mfma) {
        // images of whole windows: q rows per window, tables per 128-token sub-chunk
        const int64_t win_bytes = sata::img_head_bytes(d_K, d_V, 1, sata::img_window(d_K) / sata::kImgLU);
        pl.img_chunk = BH * win_bytes / pl.win;
        pl.fixed = BH * 16 + 4 * 256;
    }
    pl.per_chunk = pl.part_chunk + pl.img_chunk;
    pl.state_b = BH * cols * t->h.M_pad * 4;
    pl.s32_b = f16state ? round256(pl.state_b) : 0;
    const int64_t limit = t->ws_limit;
    // the layout for segments of `chunks` chunks (images rounded up to whole windows)
    auto layout = [&](int64_t chunks, int64_t carrier_b) {
        const int64_t img_chunks = (chunks + pl.win - 1) / pl.win * pl.win;
        pl.off_carrier = round256(pl.part_chunk * chunks);
        pl.off_img = pl.off_carrier + round256(carrier_b);
        pl.off_max = pl.off_img + round256(pl.img_chunk * img_chunks);
        pl.off_s32 = pl.off_max + round256(pl.mfma ? BH * 16 : 0);
        pl.ws_bytes = pl.off_s32 + pl.s32_b;
    };

    // Two-level form: when the slices of all heads leave compute units idle, the sequence
    // is cut into nsub sub-segments of whole readout windows (at least 4 windows each).
    if (pl.mfma && t->split != 1) {
        const int64_t nwin = (pl.nchunks + pl.win - 1) / pl.win;
        int64_t nsub = 1;
        if (t->split >= 2) {
            nsub = t->split;
        } else {
            const int64_t cus = t->cus > 0 ? t->cus : 256;
            const int64_t wgs = BH * pl.nslices;                   // workgroups of one scan launch
            nsub = wgs < cus ? cus / wgs : 1;
            if (nsub > nwin / 4) nsub = nwin / 4;
        }
        if (nsub > nwin) nsub = nwin;
        int64_t sub_chunks = pl.nchunks, pps = 1;
        if (nsub >= 2) {
            sub_chunks = (nwin + nsub - 1) / nsub * pl.win;
            nsub = (pl.nchunks + sub_chunks - 1) / sub_chunks;     // no empty sub-segment
        }
        if (nsub >= 2) {
            // The update-only pass needs the local states of the first nsub - 1 sub-segments
            // alone (the last one's end state comes from the second pass); each is cut into
            // pps pieces of whole windows, as many as the idle compute units take.
            const int64_t cus = t->cus > 0 ? t->cus : 256;
            const int64_t sub_win = sub_chunks / pl.win;
            int64_t kmax = cus / (BH * pl.nslices * (nsub - 1));
            if (kmax > sub_win) kmax = sub_win;
            for (int64_t k = kmax; k >= 1; --k)
                if (sub_win % k == 0) {
                    pps = k;
                    break;
                }
            if (BH * (nsub - 1) * pps > 65535) pps = 1;
        }
        const int64_t carrier_b = pl.state_b * (nsub + (nsub - 1) * pps);   // starts, then pieces
        const int64_t need = pl.part_chunk * pl.nchunks + carrier_b + pl.fixed + pl.s32_b +
                             pl.img_chunk * ((pl.nchunks + pl.win - 1) / pl.win * pl.win) + 256;
        if (nsub >= 2 && BH * nsub <= 65535 && need <= limit) {
            pl.nsub = (int)nsub;
            pl.sub_chunks = (int)sub_chunks;
            pl.pps = (int)pps;
            pl.seg = pl.nchunks;
            pl.nseg = 1;
            layout(pl.nchunks, carrier_b);
            return SATA_OK;
        }
    }
    (void)cont;
    const int64_t carrier = has_state ? 0 : pl.state_b;
    const int64_t whole = pl.part_chunk * pl.nchunks +
                          pl.img_chunk * ((pl.nchunks + pl.win - 1) / pl.win * pl.win) + pl.fixed + pl.s32_b;
    pl.seg = (int)segment_chunks(pl.nchunks, pl.win, pl.per_chunk, carrier, pl.fixed + pl.s32_b,
                                 whole, limit);
    pl.nseg = (pl.nchunks + pl.seg - 1) / pl.seg;
    layout(pl.seg, !has_state && pl.nseg > 1 ? pl.state_b : 0);
    return SATA_OK;
}

// Checks shared by sata_prefill and the workspace query (no pointer is dereferenced).
int check_prefill_sizes(const sata_tables* t, int B, int H, int n, int d_K, int d_V, int P,
                        int chunk, sata_dtype in_dtype) {
    if (B < 1 || H < 1 || n < 1) return fail(SATA_ERR_ARG, "need B, H, n >= 1 (got %d %d %d)", B, H, n);
    int rc = check_sizes(d_K, d_V, P);
    if (rc) return rc;
    if (d_K != t->h.d_K || P != t->h.P)
        return fail(SATA_ERR_ARG, "handle built for d_K=%d P=%d, call has d_K=%d P=%d",
                    t->h.d_K, t->h.P, d_K, P);
    if (in_dtype != SATA_F32 && in_dtype != SATA_BF16)
        return fail(SATA_ERR_ARG, "unknown input dtype %d", (int)in_dtype);
    if (chunk != 16 && chunk != 32 && chunk != 64 && chunk != 128)
        return fail(SATA_ERR_UNSUPPORTED, "chunk must be 16, 32, 64 or 128 (got %d)", chunk);
    if (sata::finalize_lds_bytes(d_K, d_V, chunk) > 160 * 1024)
        return fail(SATA_ERR_UNSUPPORTED, "chunk=%d is too large for d_K=%d, d_V=%d", chunk,
                    d_K, d_V);
    if ((int64_t)B * H > 65535) return fail(SATA_ERR_UNSUPPORTED, "B*H must be <= 65535");
    return SATA_OK;
}

// Compact (half-precision) state layout of one head of this handle's d_K, P for d_V.
sata::State16Geom state16_geom(const sata_tables* t, int d_V) {
    sata::State16Geom g{};
    g.M = t->h.M;
    g.M_pad = t->h.M_pad;
    g.Mh = t->h.Mh;
    g.d_K = t->h.d_K;
    g.d_V = d_V;
    g.P = t->h.P;
    for (int p = 0; p < g.P; ++p) {
        g.off[p] = t->h.off[p];
        g.hoff[p] = t->h.hoff[p];
        g.m[p] = t->h.m[p];
    }
    g.z_off = sata::state16_header_bytes(d_V, g.P);
    g.v_off = g.z_off + 4 * g.Mh;
    g.head_bytes = sata::state16_head_bytes(g.Mh, d_V, g.P);
    return g;
}

constexpr int kPrefillFlags = SATA_PREFILL_CONTINUE | SATA_STATE_F16;

// Checks of the state conversions: count heads of d_V value columns.
int convert_args(const sata_tables* t, const void* a, const void* b, int count, int d_V) {
    if (!t) return fail(SATA_ERR_ARG, "handle is NULL");
    if (!a || !b) return fail(SATA_ERR_ARG, "state pointers must be non-NULL");
    if (count < 1 || count > 65535) return fail(SATA_ERR_ARG, "count must be in 1..65535 (got %d)", count);
    if (d_V < 1 || d_V > sata::kMaxD) return fail(SATA_ERR_UNSUPPORTED, "d_V=%d outside 1..128", d_V);
    if (!aligned16(a) || !aligned16(b)) return fail(SATA_ERR_ALIGN, "state pointers must be 16-byte aligned");
    return check_device(t);
}


}  // namespace

extern "C" {

const char* sata_last_error(void) { return g_err; }

int64_t sata_feature_dim(int d_K, int P) {
    if (d_K < 1 || d_K > sata::kMaxD || P < 1 || P > sata::kMaxP) return -1;
    return sata::feature_dim(d_K, P);
}

int64_t sata_state_stride(int d_K, int P) {
    if (d_K < 1 || d_K > sata::kMaxD || P < 1 || P > sata::kMaxP) return -1;
    return sata::state_stride(d_K, P);
}

int64_t sata_state_bytes(int B, int H, int d_K, int d_V, int P) {
    if (B < 1 || H < 1 || d_V < 1 || d_V > sata::kMaxD) return -1;
    const int64_t Mp = sata_state_stride(d_K, P);
    if (Mp < 0) return -1;
    return 4LL * B * H * (d_V + 1) * Mp;
}

int sata_tables_build(int d_K, int P, sata_tables** out) {
    clear_err();
    if (!out) return fail(SATA_ERR_ARG, "out is NULL");
    *out = nullptr;
    if (d_K < 1 || d_K > sata::kMaxD || P < 1 || P > sata::kMaxP)
        return fail(SATA_ERR_UNSUPPORTED, "unsupported d_K=%d P=%d", d_K, P);
    sata_tables* t = new (std::nothrow) sata_tables();
    if (!t) return fail(SATA_ERR_OOM, "host allocation failed");
    if (!sata::build_host_tables(d_K, P, t->h)) {
        delete t;
        return fail(SATA_ERR_ARG, "table construction failed for d_K=%d P=%d", d_K, P);
    }
    if (hipGetDevice(&t->device) != hipSuccess ||
        hipDeviceGetAttribute(&t->cus, hipDeviceAttributeMultiprocessorCount, t->device) != hipSuccess) {
        delete t;
        return fail(SATA_ERR_HIP, "hipGetDevice failed");
    }
    const size_t n = (size_t)t->h.M_pad, nh = (size_t)t->h.Mh;
    if (hipMalloc(&t->d_fidx, n * 4) != hipSuccess || hipMalloc(&t->d_qw, n * 4) != hipSuccess ||
        hipMalloc(&t->d_fidx_h, nh * 4) != hipSuccess || hipMalloc(&t->d_qw_h, nh * 4) != hipSuccess) {
        (void)hipGetLastError();
        sata_tables_free(t);
        return fail(SATA_ERR_OOM, "device allocation of the tables failed");
    }
    if (hipMemcpy(t->d_fidx, t->h.fidx.data(), n * 4, hipMemcpyHostToDevice) != hipSuccess ||
        hipMemcpy(t->d_qw, t->h.qw.data(), n * 4, hipMemcpyHostToDevice) != hipSuccess ||
        hipMemcpy(t->d_fidx_h, t->h.fidx_h.data(), nh * 4, hipMemcpyHostToDevice) != hipSuccess ||
        hipMemcpy(t->d_qw_h, t->h.qw_h.data(), nh * 4, hipMemcpyHostToDevice) != hipSuccess) {
        sata_tables_free(t);
        return fail(SATA_ERR_HIP, "copy of the tables to the device failed");
    }
    int rc = sata::build_mfma_tables(t->h, t->mfma);
    if (rc != SATA_OK) {
        sata_tables_free(t);
        return fail(rc, "MFMA slice tables failed");
    }
    t->mfma_slices = t->mfma.ok ? t->mfma.nslices : 0;
    *out = t;
    return SATA_OK;
}

int sata_tables_build_host(int d_K, int P, sata_tables** out) {
    clear_err();
    if (!out) return fail(SATA_ERR_ARG, "out is NULL");
    *out = nullptr;
    if (d_K < 1 || d_K > sata::kMaxD || P < 1 || P > sata::kMaxP)
        return fail(SATA_ERR_UNSUPPORTED, "unsupported d_K=%d P=%d", d_K, P);
    sata_tables* t = new (std::nothrow) sata_tables();
    if (!t) return fail(SATA_ERR_OOM, "host allocation failed");
    if (!sata::build_host_tables(d_K, P, t->h)) {
        delete t;
        return fail(SATA_ERR_ARG, "table construction failed for d_K=%d P=%d", d_K, P);
    }
    t->device = -1;
    t->mfma_slices = sata::mfma_slice_count(t->h);
    *out = t;
    return SATA_OK;
}

int sata_tables_get(const sata_tables* t, int p, const int32_t** M_p, const int32_t** C_p,
                    int64_t* m_p) {
    clear_err();
    if (!t) return fail(SATA_ERR_ARG, "handle is NULL");
    if (p < 0 || p >= t->h.P) return fail(SATA_ERR_ARG, "p=%d outside 0..%d", p, t->h.P - 1);
    if (M_p) *M_p = t->h.Mp[p].empty() ? nullptr : t->h.Mp[p].data();
    if (C_p) *C_p = t->h.Cp[p].data();
    if (m_p) *m_p = t->h.m[p];
    return SATA_OK;
}

void sata_tables_free(sata_tables* t) {
    if (!t) return;
    if (t->d_fidx) (void)hipFree(t->d_fidx);
    if (t->d_qw) (void)hipFree(t->d_qw);
    if (t->d_fidx_h) (void)hipFree(t->d_fidx_h);
    if (t->d_qw_h) (void)hipFree(t->d_qw_h);
    sata::free_mfma_tables(t->mfma);
    for (auto& e : t->ws)
        if (e.ptr) (void)hipFree(e.ptr);
    t->timer.destroy();
    delete t;
}

int sata_set_timing(sata_tables* t, int enable) {
    clear_err();
    if (!t) return fail(SATA_ERR_ARG, "handle is NULL");
    std::lock_guard<std::mutex> lock(t->mu);
    t->timer.recycle();
    t->timer.enabled = enable != 0;
    return SATA_OK;
}

int sata_read_timing(sata_tables* t, double* ms, int64_t* count) {
    clear_err();
    if (!t) return fail(SATA_ERR_ARG, "handle is NULL");
    std::lock_guard<std::mutex> lock(t->mu);
    int rc = SATA_OK;
    for (int k = 0; k < SATA_NUM_KERNELS; ++k) {
        double sum = 0.0;
        for (auto& pr : t->timer.pending[k]) {
            float e_ms = 0.0f;
            if (hipEventSynchronize(pr.second) != hipSuccess ||
                hipEventElapsedTime(&e_ms, pr.first, pr.second) != hipSuccess) {
                rc = fail(SATA_ERR_HIP, "reading a timing event failed");
                continue;
            }
            sum += e_ms;
        }
        if (ms) ms[k] = sum;
        if (count) count[k] = (int64_t)t->timer.pending[k].size();
    }
    t->timer.recycle();
    return rc;
}

int sata_set_prefill_split(sata_tables* t, int nsub) {
    clear_err();
    if (!t) return fail(SATA_ERR_ARG, "handle is NULL");
    if (nsub < 0 || nsub > 4096) return fail(SATA_ERR_ARG, "split must be in [0, 4096] (got %d)", nsub);
    std::lock_guard<std::mutex> lock(t->mu);
    t->split = nsub;
    return SATA_OK;
}

int sata_set_workspace_limit(sata_tables* t, int64_t bytes) {
    clear_err();
    if (!t) return fail(SATA_ERR_ARG, "handle is NULL");
    if (bytes < 0) return fail(SATA_ERR_ARG, "negative limit");
    std::lock_guard<std::mutex> lock(t->mu);
    t->ws_limit = bytes == 0 ? kDefaultWorkspace : bytes;
    return SATA_OK;
}

int sata_prefill_workspace(const sata_tables* t, int B, int H, int n, int d_K, int d_V, int P,
                           int chunk, sata_dtype in_dtype, int flags, int with_state,
                           int64_t* bytes, int* segments, int* segment_chunks_out, int* subsegments) {
    clear_err();
    if (!t) return fail(SATA_ERR_ARG, "handle is NULL");
    if (!bytes) return fail(SATA_ERR_ARG, "bytes is NULL");
    int rc = check_prefill_sizes(t, B, H, n, d_K, d_V, P, chunk, in_dtype);
    if (rc) return rc;
    if (flags & ~kPrefillFlags) return fail(SATA_ERR_ARG, "unknown flags 0x%x", flags);
    const bool cont = (flags & SATA_PREFILL_CONTINUE) != 0, f16 = (flags & SATA_STATE_F16) != 0;
    if (cont && !with_state) return fail(SATA_ERR_ARG, "SATA_PREFILL_CONTINUE needs a state buffer");
    if (f16 && !with_state) return fail(SATA_ERR_ARG, "SATA_STATE_F16 needs a state buffer");
    sata_tables* tm = const_cast<sata_tables*>(t);
    std::lock_guard<std::mutex> lock(tm->mu);
    PrefillPlan pl;
    rc = plan_prefill(t, B, H, n, d_V, chunk, in_dtype == SATA_BF16, with_state != 0, cont, f16, pl);
    if (rc) return rc;
    *bytes = pl.ws_bytes;
    if (segments) *segments = pl.nseg;
    if (segment_chunks_out) *segment_chunks_out = pl.seg;
    if (subsegments) *subsegments = pl.nsub;
    return SATA_OK;
}

int sata_decode_workspace(const sata_tables* t, int B, int H, int d_V, int64_t* bytes) {
    clear_err();
    if (!t) return fail(SATA_ERR_ARG, "handle is NULL");
    if (!bytes) return fail(SATA_ERR_ARG, "bytes is NULL");
    if (B < 1 || H < 1) return fail(SATA_ERR_ARG, "need B, H >= 1 (got %d %d)", B, H);
    if (d_V < 1 || d_V > sata::kMaxD) return fail(SATA_ERR_UNSUPPORTED, "d_V=%d outside 1..128", d_V);
    const int64_t f32 = sata::decode_partial_floats(B * H, d_V, t->h.M_pad) * 4;
    const int64_t f16 = sata::decode16_partial_floats(B * H, d_V, t->h.P, t->h.Mh) * 4;
    *bytes = f32 > f16 ? f32 : f16;
    return SATA_OK;
}

int sata_reserve_workspace(sata_tables* t, int64_t bytes, void* stream) {
    clear_err();
    if (!t) return fail(SATA_ERR_ARG, "handle is NULL");
    if (bytes < 0) return fail(SATA_ERR_ARG, "negative size");
    int rc = check_device(t);
    if (rc) return rc;
    std::lock_guard<std::mutex> lock(t->mu);
    return ensure_ws(t, (size_t)bytes, (hipStream_t)stream, nullptr);
}

int sata_prefill(const sata_tables* tc, const void* q, const void* k, const void* v, float* y,
                 void* state_arg, int B, int H, int n, int d_K, int d_V, int P, int chunk,
                 sata_dtype in_dtype, int flags, void* stream) {
    clear_err();
    sata_tables* t = const_cast<sata_tables*>(tc);
    if (!t) return fail(SATA_ERR_ARG, "handle is NULL");
    if (!q || !k || !v || !y) return fail(SATA_ERR_ARG, "q, k, v and y must be non-NULL");
    int rc = check_prefill_sizes(t, B, H, n, d_K, d_V, P, chunk, in_dtype);
    if (rc) return rc;
    if (flags & ~kPrefillFlags) return fail(SATA_ERR_ARG, "unknown flags 0x%x", flags);
    const bool cont = (flags & SATA_PREFILL_CONTINUE) != 0, f16 = (flags & SATA_STATE_F16) != 0;
    if (cont && !state_arg) return fail(SATA_ERR_ARG, "SATA_PREFILL_CONTINUE needs a state buffer");
    if (f16 && !state_arg) return fail(SATA_ERR_ARG, "SATA_STATE_F16 needs a state buffer");
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(y) ||
        (state_arg && !aligned16(state_arg)))
        return fail(SATA_ERR_ALIGN, "tensor pointers must be 16-byte aligned");
    rc = check_device(t);
    if (rc) return rc;

    std::lock_guard<std::mutex> lock(t->mu);
    PrefillPlan pl;
    rc = plan_prefill(t, B, H, n, d_V, chunk, in_dtype == SATA_BF16, state_arg != nullptr, cont, f16, pl);
    if (rc) return rc;
    const bool bf16 = in_dtype == SATA_BF16;
    const int BH = B * H, L = chunk, cols = d_V + 1;

    sata::PrefillSegArgs a{};
    a.q = q; a.k = k; a.v = v; a.y = y;
    a.fidx = t->d_fidx;
    a.qw = t->d_qw;
    for (int p = 0; p < P; ++p) a.alpha.a[p] = (float)t->h.alpha[p];
    a.M = t->h.M;
    a.M_pad = t->h.M_pad;
    a.BH = BH; a.n = n; a.d_K = d_K; a.d_V = d_V; a.P = P; a.L = L;
    a.bf16 = bf16;
    a.nslices = pl.nslices;
    a.slice_feats = pl.slice_feats;
    a.win = pl.win;
    a.partial_tiled = pl.mfma;
    a.mfma_rows = pl.mfma ? t->mfma.d_rows : nullptr;

    hipStream_t st = (hipStream_t)stream;
    char* ws = nullptr;
    rc = ensure_ws(t, (size_t)pl.ws_bytes, st, &ws);
    if (rc) return rc;
    a.partial = (float*)ws;

    // With a half-precision state the scans run on an fp32 working copy in the workspace:
    // unpacked from the caller's state first when it holds a prefix, packed into it at the end.
    const sata::State16Geom g16 = state16_geom(t, d_V);
    float* state = f16 ? (float*)(ws + pl.off_s32) : (float*)state_arg;
    if (f16 && cont) {
        hipEvent_t ev = t->timer.begin(st);
        const hipError_t e = sata::launch_state16_unpack((const uint8_t*)state_arg, state, g16, BH, st);
        t->timer.end(SATA_KERNEL_CONVERT, ev, st);
        if (e != hipSuccess) return fail(SATA_ERR_HIP, "state conversion failed: %s", hipGetErrorString(e));
    }
    auto finish = [&]() -> int {
        if (!f16) return SATA_OK;
        hipEvent_t ev = t->timer.begin(st);
        const hipError_t e = sata::launch_state16_pack(state, (uint8_t*)state_arg, g16, BH, st);
        t->timer.end(SATA_KERNEL_CONVERT, ev, st);
        if (e != hipSuccess) return fail(SATA_ERR_HIP, "state conversion failed: %s", hipGetErrorString(e));
        return SATA_OK;
    };

    // Matrix-core path: the per-head maxima of |q|, |k|, |v| over the whole sequence (they
    // fix the power-of-two scales of the fp16 operands), then, per segment, the operand
    // images of its whole windows (kern_prep.hip).
    const int R = sata::img_window(d_K);
    auto prep_images = [&](int c0, int c1, int nwin_stride) -> hipError_t {
        const int QB = sata::img_q_bytes(d_K), KTB = sata::img_kt_bytes(d_K);
        a.img_w0 = c0 / pl.win;
        a.img_nwin = nwin_stride;
        a.img_u0 = (int)((int64_t)c0 * L / sata::kImgLU);
        a.img_nsub = nwin_stride * (R / sata::kImgLU);
        char* img = ws + pl.off_img;
        a.qimg = (uint16_t*)img;
        a.kimg = (uint16_t*)(img + (int64_t)BH * a.img_nwin * QB);
        a.vimg = (uint16_t*)(img + (int64_t)BH * a.img_nwin * QB + (int64_t)BH * a.img_nsub * KTB);
        const int c1w = (c1 + pl.win - 1) / pl.win * pl.win;
        return sata::launch_prep_images(a, a.img_u0, (int)((int64_t)c1w * L / sata::kImgLU), st);
    };
    if (pl.mfma) {
        uint32_t* maxbits = (uint32_t*)(ws + pl.off_max);
        a.maxbits = maxbits;
        hipEvent_t ev = t->timer.begin(st);
        const hipError_t e = sata::launch_prep_max(a, maxbits, st);
        t->timer.end(SATA_KERNEL_PREP, ev, st);
        if (e != hipSuccess) return fail(SATA_ERR_HIP, "prep launch failed: %s", hipGetErrorString(e));
    }

    if (pl.nsub >= 2) {
        // Two-level form (the state recurrence as a prefix over segments, [TA] "Hardware
        // optimisation path"): the local states of the pieces of the first nsub - 1
        // sub-segments are accumulated in parallel (update-only scan), summed in order into
        // each sub-segment's starting state, and the sub-segments are then scanned in parallel
        // from those states; the last one's blocks store the final state.  Same sums as one
        // segment, in another order.
        const int64_t per_state = (int64_t)cols * t->h.M_pad;
        float* starts = (float*)(ws + pl.off_carrier);
        float* pieces = starts + (int64_t)BH * pl.nsub * per_state;
        hipEvent_t ev = t->timer.begin(st);
        hipError_t e = prep_images(0, pl.nchunks, (pl.nchunks + pl.win - 1) / pl.win);
        t->timer.end(SATA_KERNEL_PREP, ev, st);
        ev = t->timer.begin(st);
        a.c_begin = 0;                          // local states of the pieces, from zero
        a.c_end = (pl.nsub - 1) * pl.sub_chunks;
        a.nsub = (pl.nsub - 1) * pl.pps;
        a.sub_chunks = pl.sub_chunks / pl.pps;
        a.state = pieces;
        a.update_only = true;
        a.load_state = 0;
        a.store_state = 1;
        a.final_state = nullptr;
        if (e == hipSuccess) e = sata::launch_scan_mfma(a, t->mfma, st);
        if (e == hipSuccess)
            e = sata::launch_state_starts(pieces, cont ? state : nullptr, starts, BH, pl.nsub, pl.pps,
                                          per_state, st);
        a.c_end = pl.nchunks;                   // readouts and partials from the starts
        a.nsub = pl.nsub;
        a.sub_chunks = pl.sub_chunks;
        a.state = starts;
        a.update_only = false;
        a.load_state = 1;
        a.store_state = state ? 1 : 0;
        a.final_state = state;
        if (e == hipSuccess) e = sata::launch_scan_mfma(a, t->mfma, st);
        t->timer.end(SATA_KERNEL_SCAN, ev, st);
        if (e != hipSuccess)
            return fail(SATA_ERR_HIP, "two-level scan launch failed: %s", hipGetErrorString(e));
        ev = t->timer.begin(st);
        e = sata::launch_finalize(a, st);
        t->timer.end(SATA_KERNEL_FINALIZE, ev, st);
        if (e != hipSuccess)
            return fail(SATA_ERR_HIP, "finalize launch failed: %s", hipGetErrorString(e));
        return finish();
    }

    float* carrier = state;
    if (!carrier && pl.nseg > 1) carrier = (float*)(ws + pl.off_carrier);
    a.state = carrier;
    for (int s = 0; s < pl.nseg; ++s) {
        a.c_begin = s * pl.seg;
        a.c_end = (s + 1) * pl.seg < pl.nchunks ? (s + 1) * pl.seg : pl.nchunks;
        a.load_state = (s > 0 || cont) ? 1 : 0;
        a.store_state = (s < pl.nseg - 1 || state) ? 1 : 0;
        hipError_t e = hipSuccess;
        if (pl.mfma) {
            hipEvent_t ev = t->timer.begin(st);
            e = prep_images(a.c_begin, a.c_end, (pl.seg + pl.win - 1) / pl.win);
            t->timer.end(SATA_KERNEL_PREP, ev, st);
            if (e != hipSuccess) return fail(SATA_ERR_HIP, "prep launch failed: %s", hipGetErrorString(e));
        }
        hipEvent_t ev = t->timer.begin(st);
        e = pl.mfma ? sata::launch_scan_mfma(a, t->mfma, st) : sata::launch_scan_valu(a, st);
        t->timer.end(SATA_KERNEL_SCAN, ev, st);
        if (e != hipSuccess)
            return fail(SATA_ERR_HIP, "scan launch failed: %s", hipGetErrorString(e));
        ev = t->timer.begin(st);
        e = sata::launch_finalize(a, st);
        t->timer.end(SATA_KERNEL_FINALIZE, ev, st);
        if (e != hipSuccess)
            return fail(SATA_ERR_HIP, "finalize launch failed: %s", hipGetErrorString(e));
    }
    return finish();
}

int sata_prefill_backward(const sata_tables* tc, const void* q, const void* k, const void* v,
                          const float* dy, float* dq, float* dk, float* dv, int B, int H, int n,
                          int d_K, int d_V, int P, int chunk, sata_dtype in_dtype, void* stream) {
    clear_err();
    sata_tables* t = const_cast<sata_tables*>(tc);
    if (!t) return fail(SATA_ERR_ARG, "handle is NULL");
    if (!q || !k || !v || !dy || !dq || !dk || !dv)
        return fail(SATA_ERR_ARG, "q, k, v, dy, dq, dk and dv must be non-NULL");
    if (B < 1 || H < 1 || n < 1) return fail(SATA_ERR_ARG, "need B, H, n >= 1 (got %d %d %d)", B, H, n);
    int rc = check_sizes(d_K, d_V, P);
    if (rc) return rc;
    if (d_K != t->h.d_K || P != t->h.P)
        return fail(SATA_ERR_ARG, "handle built for d_K=%d P=%d, call has d_K=%d P=%d",
                    t->h.d_K, t->h.P, d_K, P);
    if (in_dtype != SATA_F32 && in_dtype != SATA_BF16)
        return fail(SATA_ERR_ARG, "unknown input dtype %d", (int)in_dtype);
    if (chunk != 16 && chunk != 32 && chunk != 64 && chunk != 128)
        return fail(SATA_ERR_UNSUPPORTED, "chunk must be 16, 32, 64 or 128 (got %d)", chunk);
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(dy) || !aligned16(dq) ||
        !aligned16(dk) || !aligned16(dv))
        return fail(SATA_ERR_ALIGN, "tensor pointers must be 16-byte aligned");
    const int L = chunk;
    const int SVf = sata::valu_slice_feats(d_K, d_V, L), SVb = sata::bwd_slice_feats(d_K, d_V, L);
    if (sata::finalize_lds_bytes(d_K, d_V, L) > 160 * 1024 || sata::bwd_fin_lds_bytes(d_K, d_V, L) > 160 * 1024 ||
        SVf == 0 || SVb == 0)
        return fail(SATA_ERR_UNSUPPORTED, "chunk=%d is too large for the backward at d_K=%d, d_V=%d", chunk,
                    d_K, d_V);
    if ((int64_t)B * H > 65535) return fail(SATA_ERR_UNSUPPORTED, "B*H must be <= 65535");
    rc = check_device(t);
    if (rc) return rc;

    const bool bf16 = in_dtype == SATA_BF16;
    const int BH = B * H, cols = d_V + 1;
    const int nchunks = (int)(((int64_t)n + L - 1) / L);
    const int64_t M = t->h.M, M_pad = t->h.M_pad;
    const int nslf = (int)((M + SVf - 1) / SVf), nslb = (int)((M + SVb - 1) / SVb);
    auto r256 = [](int64_t b) { return (b + 255) / 256 * 256; };
    const int64_t y_b = r256((int64_t)BH * n * d_V * 4), den_b = r256((int64_t)BH * n * 4);
    const int ucols = (cols + 3) / 4 * 4;
    const int64_t u_b = r256((int64_t)BH * n * ucols * 4), st_b = r256((int64_t)BH * cols * M_pad * 4);
    const int64_t fixed = y_b + den_b + u_b + st_b;
    int64_t per_chunk = (int64_t)BH * nslf * L * cols * 4;                    // forward recompute
    const int64_t per_q = (int64_t)BH * nslb * L * d_K * 4;
    const int64_t per_kv = (int64_t)BH * nslb * L * (d_K + d_V) * 4;
    if (per_q > per_chunk) per_chunk = per_q;
    if (per_kv > per_chunk) per_chunk = per_kv;
    int64_t seg = nchunks;
    if (fixed + per_chunk * seg > t->ws_limit) {
        seg = (t->ws_limit - fixed) / per_chunk;
        if (seg < 1) seg = 1;
        const int64_t ns = (nchunks + seg - 1) / seg;
        seg = (nchunks + ns - 1) / ns;
    }
    const int nseg = (int)((nchunks + seg - 1) / seg);

    std::lock_guard<std::mutex> lock(t->mu);
    hipStream_t st = (hipStream_t)stream;
    char* base = nullptr;
    rc = ensure_ws(t, (size_t)(fixed + per_chunk * seg), st, &base);
    if (rc) return rc;
    float* y_ws = (float*)base;
    float* den_ws = (float*)(base + y_b);
    float* u_ws = (float*)(base + y_b + den_b);
    float* carrier = (float*)(base + y_b + den_b + u_b);
    float* part = (float*)(base + fixed);
    hipEvent_t ev = t->timer.begin(st);

    // forward recompute in fp32: y and the normaliser D of every row
    sata::PrefillSegArgs a{};
    a.q = q; a.k = k; a.v = v; a.y = y_ws; a.den = den_ws;
    a.fidx = t->d_fidx;
    a.qw = t->d_qw;
    for (int p = 0; p < P; ++p) a.alpha.a[p] = (float)t->h.alpha[p];
    a.M = M; a.M_pad = M_pad;
    a.BH = BH; a.n = n; a.d_K = d_K; a.d_V = d_V; a.P = P; a.L = L;
    a.bf16 = bf16;
    a.win = 1;
    a.partial_tiled = false;
    a.slice_feats = SVf;
    a.nslices = nslf;
    a.partial = part;
    a.state = carrier;
    hipError_t e = hipSuccess;
    for (int s = 0; s < nseg && e == hipSuccess; ++s) {
        a.c_begin = (int)(s * seg);
        a.c_end = (int)((s + 1) * seg < nchunks ? (s + 1) * seg : nchunks);
        a.load_state = s > 0 ? 1 : 0;
        a.store_state = s < nseg - 1 ? 1 : 0;
        e = sata::launch_scan_valu(a, st);
        if (e == hipSuccess) e = sata::launch_finalize_fp32(a, st);
    }
    // u = [dy / D | -(dy . y) / D]
    sata::BwdArgs b{};
    b.q = q; b.k = k; b.v = v;
    b.dy = dy; b.y = y_ws; b.den = den_ws; b.u = u_ws; b.u_out = u_ws; b.ucols = ucols;
    b.dq = dq; b.dk = dk; b.dv = dv;
    b.state = carrier;
    b.fidx = t->d_fidx;
    b.qw = t->d_qw;
    b.alpha = a.alpha;
    b.M = M; b.M_pad = M_pad;
    b.BH = BH; b.n = n; b.d_K = d_K; b.d_V = d_V; b.P = P; b.L = L;
    b.nslices = nslb;
    b.slice_feats = SVb;
    b.bf16 = bf16;
    if (e == hipSuccess) e = sata::launch_bwd_u(b, st);
    // dq: chunks in order, the forward state S carried between segments
    b.part = part;
    b.part2 = nullptr;
    for (int s = 0; s < nseg && e == hipSuccess; ++s) {
        b.c_begin = (int)(s * seg);
        b.c_end = (int)((s + 1) * seg < nchunks ? (s + 1) * seg : nchunks);
        b.load_state = s > 0 ? 1 : 0;
        b.store_state = s < nseg - 1 ? 1 : 0;
        e = sata::launch_bwd_q(b, st);
        if (e == hipSuccess) e = sata::launch_bwd_fin(b, 0, st);
    }
    // dk, dv: chunks in reverse, the mirror state R carried between segments
    for (int s = nseg - 1; s >= 0 && e == hipSuccess; --s) {
        b.c_begin = (int)(s * seg);
        b.c_end = (int)((s + 1) * seg < nchunks ? (s + 1) * seg : nchunks);
        b.part = part;
        b.part2 = part + (int64_t)BH * (b.c_end - b.c_begin) * nslb * L * d_K;
        b.load_state = s < nseg - 1 ? 1 : 0;
        b.store_state = s > 0 ? 1 : 0;
        e = sata::launch_bwd_kv(b, st);
        if (e == hipSuccess) e = sata::launch_bwd_fin(b, 1, st);
    }
    t->timer.end(SATA_KERNEL_BACKWARD, ev, st);
    if (e != hipSuccess) return fail(SATA_ERR_HIP, "backward launch failed: %s", hipGetErrorString(e));
    return SATA_OK;
}

}  // extern "C"

namespace {

// Decode step shared by the dense, the pool and the allocation-free forms: BH = batch
// entries x H heads; slots == NULL for the dense forms; noalloc: the partial readouts go to
// the fixed device scratch, and nothing is allocated (no workspace, no timing events);
// f16: the states are compact half-precision states.
int decode_impl(sata_tables* t, void* state, const int32_t* slots, int64_t pool, const void* q,
                const void* k, const void* v, float* y, int B, int H, int d_K, int d_V, int P,
                sata_dtype in_dtype, void* stream, bool noalloc = false, bool f16 = false) {
    int rc = check_sizes(d_K, d_V, P);
    if (rc) return rc;
    if (d_K != t->h.d_K || P != t->h.P)
        return fail(SATA_ERR_ARG, "handle built for d_K=%d P=%d, call has d_K=%d P=%d",
                    t->h.d_K, t->h.P, d_K, P);
    if (in_dtype != SATA_F32 && in_dtype != SATA_BF16)
        return fail(SATA_ERR_ARG, "unknown input dtype %d", (int)in_dtype);
    if (!aligned16(state) || !aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(y))
        return fail(SATA_ERR_ALIGN, "tensor pointers must be 16-byte aligned");
    if ((int64_t)B * H > 65535) return fail(SATA_ERR_UNSUPPORTED, "B*H must be <= 65535");
    const int64_t part_bytes = f16 ? sata::decode16_partial_floats(B * H, d_V, P, t->h.Mh) * 4
                                   : sata::decode_partial_floats(B * H, d_V, t->h.M_pad) * 4;
    if (noalloc && part_bytes > sata::kNoAllocScratchBytes)
        return fail(SATA_ERR_UNSUPPORTED,
                    "the allocation-free decode step holds %lld bytes of partials; B=%d H=%d "
                    "d_V=%d needs %lld", (long long)sata::kNoAllocScratchBytes, B, H, d_V,
                    (long long)part_bytes);
    rc = check_device(t);
    if (rc) return rc;
    hipStream_t st = (hipStream_t)stream;

    if (f16) {
        sata::Decode16Args a{};
        a.state = (uint8_t*)state; a.q = q; a.k = k; a.v = v; a.y = y;
        a.fidx_h = t->d_fidx_h;
        a.qw_h = t->d_qw_h;
        a.g = state16_geom(t, d_V);
        a.BH = B * H;
        a.nblk = sata::decode16_blocks(t->h.Mh);
        a.bf16 = in_dtype == SATA_BF16;
        a.slots = slots;
        a.pool = pool;
        a.H = H;
        std::lock_guard<std::mutex> lock(t->mu);
        char* ws = nullptr;
        rc = ensure_ws(t, (size_t)part_bytes, st, &ws);
        if (rc) return rc;
        a.partial = (float*)ws;
        hipEvent_t ev = t->timer.begin(st);
        hipError_t e = sata::launch_decode16(a, st);
        t->timer.end(SATA_KERNEL_DECODE, ev, st);
        if (e != hipSuccess) return fail(SATA_ERR_HIP, "decode launch failed: %s", hipGetErrorString(e));
        ev = t->timer.begin(st);
        e = sata::launch_decode16_reduce(a, st);
        t->timer.end(SATA_KERNEL_DECODE_REDUCE, ev, st);
        if (e != hipSuccess)
            return fail(SATA_ERR_HIP, "decode reduction launch failed: %s", hipGetErrorString(e));
        return SATA_OK;
    }

    sata::DecodeArgs a{};
    a.state = (float*)state; a.q = q; a.k = k; a.v = v; a.y = y;
    a.fidx = t->d_fidx;
    a.qw = t->d_qw;
    a.M = t->h.M;
    a.M_pad = t->h.M_pad;
    a.BH = B * H; a.d_K = d_K; a.d_V = d_V; a.P = P;
    a.nblk = sata::decode_blocks(t->h.M_pad);
    a.bf16 = in_dtype == SATA_BF16;
    a.slots = slots;
    a.pool = pool;
    a.H = H;

    if (noalloc) {
        hipError_t e = sata::noalloc_scratch(t->device, &a.partial);
        if (e != hipSuccess)
            return fail(SATA_ERR_HIP, "address of the decode scratch: %s", hipGetErrorString(e));
        e = sata::launch_decode(a, st);
        if (e == hipSuccess) e = sata::launch_decode_reduce(a, st);
        if (e != hipSuccess) return fail(SATA_ERR_HIP, "decode launch failed: %s", hipGetErrorString(e));
        return SATA_OK;
    }
    std::lock_guard<std::mutex> lock(t->mu);
    char* ws = nullptr;
    rc = ensure_ws(t, (size_t)part_bytes, st, &ws);
    if (rc) return rc;
    a.partial = (float*)ws;
    hipEvent_t ev = t->timer.begin(st);
    hipError_t e = sata::launch_decode(a, st);
    t->timer.end(SATA_KERNEL_DECODE, ev, st);
    if (e != hipSuccess) return fail(SATA_ERR_HIP, "decode launch failed: %s", hipGetErrorString(e));
    ev = t->timer.begin(st);
    e = sata::launch_decode_reduce(a, st);
    t->timer.end(SATA_KERNEL_DECODE_REDUCE, ev, st);
    if (e != hipSuccess)
        return fail(SATA_ERR_HIP, "decode reduction launch failed: %s", hipGetErrorString(e));
    return SATA_OK;
}

}  // namespace

extern "C" {

int sata_decode_step(const sata_tables* tc, float* state, const void* q, const void* k,
                     const void* v, float* y, int B, int H, int d_K, int d_V, int P,
                     sata_dtype in_dtype, void* stream) {
    clear_err();
    sata_tables* t = const_cast<sata_tables*>(tc);
    if (!t) return fail(SATA_ERR_ARG, "handle is NULL");
    if (!state || !q || !k || !v || !y)
        return fail(SATA_ERR_ARG, "state, q, k, v and y must be non-NULL");
    if (B < 1 || H < 1) return fail(SATA_ERR_ARG, "need B, H >= 1 (got %d %d)", B, H);
    return decode_impl(t, state, nullptr, 0, q, k, v, y, B, H, d_K, d_V, P, in_dtype, stream);
}

int sata_decode_step_noalloc(const sata_tables* tc, float* state, const void* q, const void* k,
                             const void* v, float* y, int B, int H, int d_K, int d_V, int P,
                             sata_dtype in_dtype, void* stream) {
    clear_err();
    sata_tables* t = const_cast<sata_tables*>(tc);
    if (!t) return fail(SATA_ERR_ARG, "handle is NULL");
    if (!state || !q || !k || !v || !y)
        return fail(SATA_ERR_ARG, "state, q, k, v and y must be non-NULL");
    if (B < 1 || H < 1) return fail(SATA_ERR_ARG, "need B, H >= 1 (got %d %d)", B, H);
    return decode_impl(t, state, nullptr, 0, q, k, v, y, B, H, d_K, d_V, P, in_dtype, stream, true);
}

int sata_decode_step_pool(const sata_tables* tc, float* state_pool, int64_t pool_size,
                          const int32_t* slots, int count, const void* q, const void* k,
                          const void* v, float* y, int H, int d_K, int d_V, int P,
                          sata_dtype in_dtype, void* stream) {
    clear_err();
    sata_tables* t = const_cast<sata_tables*>(tc);
    if (!t) return fail(SATA_ERR_ARG, "handle is NULL");
    if (!state_pool || !slots || !q || !k || !v || !y)
        return fail(SATA_ERR_ARG, "state_pool, slots, q, k, v and y must be non-NULL");
    if (count < 1 || H < 1 || pool_size < 1)
        return fail(SATA_ERR_ARG, "need count, H, pool_size >= 1 (got %d %d %lld)", count, H,
                    (long long)pool_size);
    if (((uintptr_t)slots & 3) != 0) return fail(SATA_ERR_ALIGN, "slots must be 4-byte aligned");
    return decode_impl(t, state_pool, slots, pool_size, q, k, v, y, count, H, d_K, d_V, P,
                       in_dtype, stream);
}

int sata_decode_step_f16(const sata_tables* tc, void* state16, const void* q, const void* k,
                         const void* v, float* y, int B, int H, int d_K, int d_V, int P,
                         sata_dtype in_dtype, void* stream) {
    clear_err();
    sata_tables* t = const_cast<sata_tables*>(tc);
    if (!t) return fail(SATA_ERR_ARG, "handle is NULL");
    if (!state16 || !q || !k || !v || !y)
        return fail(SATA_ERR_ARG, "state16, q, k, v and y must be non-NULL");
    if (B < 1 || H < 1) return fail(SATA_ERR_ARG, "need B, H >= 1 (got %d %d)", B, H);
    return decode_impl(t, state16, nullptr, 0, q, k, v, y, B, H, d_K, d_V, P, in_dtype, stream,
                       false, true);
}

int sata_decode_step_pool_f16(const sata_tables* tc, void* state16_pool, int64_t pool_size,
                              const int32_t* slots, int count, const void* q, const void* k,
                              const void* v, float* y, int H, int d_K, int d_V, int P,
                              sata_dtype in_dtype, void* stream) {
    clear_err();
    sata_tables* t = const_cast<sata_tables*>(tc);
    if (!t) return fail(SATA_ERR_ARG, "handle is NULL");
    if (!state16_pool || !slots || !q || !k || !v || !y)
        return fail(SATA_ERR_ARG, "state16_pool, slots, q, k, v and y must be non-NULL");
    if (count < 1 || H < 1 || pool_size < 1)
        return fail(SATA_ERR_ARG, "need count, H, pool_size >= 1 (got %d %d %lld)", count, H,
                    (long long)pool_size);
    if (((uintptr_t)slots & 3) != 0) return fail(SATA_ERR_ALIGN, "slots must be 4-byte aligned");
    return decode_impl(t, state16_pool, slots, pool_size, q, k, v, y, count, H, d_K, d_V, P,
                       in_dtype, stream, false, true);
}

int64_t sata_state16_stride(int d_K, int P) {
    if (d_K < 1 || d_K > sata::kMaxD || P < 1 || P > sata::kMaxP) return -1;
    return sata::state16_stride(d_K, P);
}

int64_t sata_state16_bytes(int B, int H, int d_K, int d_V, int P) {
    if (B < 1 || H < 1 || d_V < 1 || d_V > sata::kMaxD) return -1;
    const int64_t Mh = sata_state16_stride(d_K, P);
    if (Mh < 0) return -1;
    return (int64_t)B * H * sata::state16_head_bytes(Mh, d_V, P);
}

int sata_state_pack_f16(const sata_tables* t, const float* state, void* state16, int count, int d_V,
                        void* stream) {
    clear_err();
    int rc = convert_args(t, state, state16, count, d_V);
    if (rc) return rc;
    const hipError_t e = sata::launch_state16_pack(state, (uint8_t*)state16, state16_geom(t, d_V), count,
                                                   (hipStream_t)stream);
    if (e != hipSuccess) return fail(SATA_ERR_HIP, "state conversion failed: %s", hipGetErrorString(e));
    return SATA_OK;
}

int sata_state_unpack_f16(const sata_tables* t, const void* state16, float* state, int count, int d_V,
                          void* stream) {
    clear_err();
    int rc = convert_args(t, state16, state, count, d_V);
    if (rc) return rc;
    const hipError_t e = sata::launch_state16_unpack((const uint8_t*)state16, state, state16_geom(t, d_V),
                                                     count, (hipStream_t)stream);
    if (e != hipSuccess) return fail(SATA_ERR_HIP, "state conversion failed: %s", hipGetErrorString(e));
    return SATA_OK;
}

}  // extern "C"
