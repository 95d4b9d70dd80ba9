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

// Default cap on the slice-partial workspace of one prefill call (about 11% of the
// 288 GB of an MI355X); a call that needs more runs in segments of whole chunks.
constexpr int64_t kDefaultWorkspace = 32LL << 30;

struct sata_tables {
    sata::HostTables h;
    KernelTimer timer;
    int device = -1;
    uint32_t* d_fidx = nullptr;
    float* d_qw = nullptr;
    sata::MfmaTables mfma;            // slice tables of the MFMA scan (may be empty)
    std::mutex mu;
    void* ws = nullptr;
    size_t ws_bytes = 0;
    int64_t ws_limit = kDefaultWorkspace;
    int cus = 0;                      // compute units of the device
    int split = 0;                    // two-level prefill: 0 automatic, 1 never, k >= 2 forced
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

// Grow the handle's workspace to at least `bytes`.  Growth waits for `st` (calls
// on one handle are issued on one stream), frees the old buffer and allocates.
int ensure_ws(sata_tables* t, size_t bytes, hipStream_t st) {
    if (bytes <= t->ws_bytes) return SATA_OK;
    if (t->ws) {
        if (hipStreamSynchronize(st) != hipSuccess)
            return fail(SATA_ERR_HIP, "hipStreamSynchronize failed while growing the workspace");
        (void)hipFree(t->ws);
        t->ws = nullptr;
        t->ws_bytes = 0;
    }
    const size_t rounded = (bytes + (1u << 20) - 1) & ~(size_t)((1u << 20) - 1);
    if (hipMalloc(&t->ws, rounded) != hipSuccess) {
        (void)hipGetLastError();
        t->ws = nullptr;
        return fail(SATA_ERR_OOM, "cannot allocate a %zu-byte workspace", rounded);
    }
    t->ws_bytes = rounded;
    return SATA_OK;
}

int check_sizes(int d_K, int d_V, int P) {
    if (d_K < 1 || d_K > sata::kMaxD || d_V < 1 || d_V > sata::kMaxD || P < 1 || P > sata::kMaxP)
        return fail(SATA_ERR_UNSUPPORTED,
                    "unsupported sizes d_K=%d d_V=%d P=%d (need 1..128, 1..128, 1..5)", d_K,
                    d_V, P);
    return SATA_OK;
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
    const size_t n = (size_t)t->h.M_pad;
    if (hipMalloc(&t->d_fidx, n * 4) != hipSuccess || hipMalloc(&t->d_qw, n * 4) != hipSuccess) {
        (void)hipGetLastError();
        sata_tables_free(t);
        return fail(SATA_ERR_OOM, "device allocation of the tables failed");
    }
    if (hipMemcpy(t->d_fidx, t->h.fidx.data(), n * 4, hipMemcpyHostToDevice) != hipSuccess ||
        hipMemcpy(t->d_qw, t->h.qw.data(), n * 4, hipMemcpyHostToDevice) != hipSuccess) {
        sata_tables_free(t);
        return fail(SATA_ERR_HIP, "copy of the tables to the device failed");
    }
    int rc = sata::build_mfma_tables(t->h, t->mfma);
    if (rc != SATA_OK) {
        sata_tables_free(t);
        return fail(rc, "MFMA slice tables failed");
    }
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
    sata::free_mfma_tables(t->mfma);
    if (t->ws) (void)hipFree(t->ws);
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

int sata_prefill(const sata_tables* tc, const void* q, const void* k, const void* v, float* y,
                 float* state, int B, int H, int n, int d_K, int d_V, int P, int chunk,
                 sata_dtype in_dtype, int flags, void* stream) {
    clear_err();
    sata_tables* t = const_cast<sata_tables*>(tc);
    if (!t) return fail(SATA_ERR_ARG, "handle is NULL");
    if (!q || !k || !v || !y) return fail(SATA_ERR_ARG, "q, k, v and y must be non-NULL");
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
    if (flags & ~SATA_PREFILL_CONTINUE) return fail(SATA_ERR_ARG, "unknown flags 0x%x", flags);
    const bool cont = (flags & SATA_PREFILL_CONTINUE) != 0;
    if (cont && !state) return fail(SATA_ERR_ARG, "SATA_PREFILL_CONTINUE needs a state buffer");
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(y) ||
        (state && !aligned16(state)))
        return fail(SATA_ERR_ALIGN, "tensor pointers must be 16-byte aligned");
    if (sata::finalize_lds_bytes(d_K, d_V, chunk) > 160 * 1024)
        return fail(SATA_ERR_UNSUPPORTED, "chunk=%d is too large for d_K=%d, d_V=%d", chunk,
                    d_K, d_V);
    if ((int64_t)B * H > 65535) return fail(SATA_ERR_UNSUPPORTED, "B*H must be <= 65535");
    rc = check_device(t);
    if (rc) return rc;

    const bool bf16 = in_dtype == SATA_BF16;
    const int BH = B * H, L = chunk, cols = d_V + 1;
    const int nchunks = (int)(((int64_t)n + L - 1) / L);

    sata::PrefillSegArgs a{};
    a.q = q; a.k = k; a.v = v; a.y = y;
    a.fidx = t->d_fidx;
    a.qw = t->d_qw;
    for (int p = 0; p < P; ++p) a.alpha.a[p] = (float)t->h.alpha[p];
    a.M = t->h.M;
    a.M_pad = t->h.M_pad;
    a.BH = BH; a.n = n; a.d_K = d_K; a.d_V = d_V; a.P = P; a.L = L;
    a.bf16 = bf16;

    const bool use_mfma = sata::mfma_supported(t->mfma, bf16, d_K, d_V, P, L);
    if (use_mfma) {
        a.nslices = t->mfma.nslices;
        a.slice_feats = t->mfma.slice_feats;
        a.mfma_rows = t->mfma.d_rows;
        a.win = sata::mfma_window(d_K);
        a.partial_tiled = true;
    } else {
        a.win = 1;
        a.partial_tiled = false;
        a.slice_feats = sata::valu_slice_feats(d_K, d_V, L);
        if (a.slice_feats == 0) return fail(SATA_ERR_UNSUPPORTED, "no VALU slice fits LDS");
        a.nslices = (int)((t->h.M + a.slice_feats - 1) / a.slice_feats);
        a.mfma_rows = nullptr;
    }

    std::lock_guard<std::mutex> lock(t->mu);
    hipStream_t st = (hipStream_t)stream;
    const int64_t per_chunk = (int64_t)BH * a.nslices * 4 *
                              (a.partial_tiled ? sata::tiled_partial_floats(L, d_V) : (int64_t)L * cols);
    const int64_t state_b = (int64_t)BH * cols * t->h.M_pad * 4;

    // Two-level form (the state recurrence as a prefix over segments, [TA] "Hardware
    // optimisation path"): when the slices of all heads leave compute units idle, the
    // sequence is cut into nsub sub-segments of whole readout windows.  Their local states
    // are accumulated in parallel (update-only scan), turned into each sub-segment's
    // starting state by a prefix sum, and the sub-segments are then scanned in parallel from
    // those states.  Same sums as one segment, in another order.
    if (use_mfma && t->split != 1) {
        const int64_t nwin = (nchunks + a.win - 1) / a.win;
        int64_t nsub = 1;
        if (t->split >= 2) {
            nsub = t->split;
        } else {
            const int64_t wgs = (int64_t)BH * a.nslices;            // workgroups of one scan launch
            nsub = wgs < t->cus ? t->cus / wgs : 1;
            if (nsub > nwin / 4) nsub = nwin / 4;                   // at least 4 windows each
        }
        if (nsub > nwin) nsub = nwin;
        int64_t sub_chunks = nchunks;
        if (nsub >= 2) {
            sub_chunks = (nwin + nsub - 1) / nsub * a.win;
            nsub = (nchunks + sub_chunks - 1) / sub_chunks;         // no empty sub-segment
        }
        const int64_t need = per_chunk * nchunks + state_b * nsub;
        if (nsub >= 2 && BH * nsub <= 65535 && need <= t->ws_limit) {
            rc = ensure_ws(t, (size_t)need, st);
            if (rc) return rc;
            a.partial = (float*)t->ws;
            float* starts = (float*)((char*)t->ws + per_chunk * nchunks);
            a.c_begin = 0;
            a.c_end = nchunks;
            a.nsub = (int)nsub;
            a.sub_chunks = (int)sub_chunks;
            a.state = starts;
            hipEvent_t ev = t->timer.begin(st);
            a.update_only = true;                   // local states from zero
            a.load_state = 0;
            a.store_state = 1;
            hipError_t e = sata::launch_scan_mfma(a, t->mfma, st);
            if (e == hipSuccess)
                e = sata::launch_state_prefix(starts, cont ? state : nullptr, state, BH, (int)nsub,
                                              (int64_t)cols * t->h.M_pad, st);
            a.update_only = false;                  // readouts and partials from the starts
            a.load_state = 1;
            a.store_state = 0;
            if (e == hipSuccess) e = sata::launch_scan_mfma(a, t->mfma, st);
            t->timer.end(SATA_KERNEL_SCAN, ev, st);
            if (e != hipSuccess)
                return fail(SATA_ERR_HIP, "two-level scan launch failed: %s", hipGetErrorString(e));
            ev = t->timer.begin(st);
            e = sata::launch_finalize(a, st);
            t->timer.end(SATA_KERNEL_FINALIZE, ev, st);
            if (e != hipSuccess)
                return fail(SATA_ERR_HIP, "finalize launch failed: %s", hipGetErrorString(e));
            return SATA_OK;
        }
    }

    int64_t seg = nchunks;
    if (per_chunk * seg > t->ws_limit) {
        seg = (t->ws_limit - (state ? 0 : state_b)) / per_chunk;
        if (seg < a.win) seg = a.win;            // at least one readout window
        // equal segments: every segment boundary stores and reloads the state, so no
        // segment should be much shorter than the others
        const int64_t ns = (nchunks + seg - 1) / seg;
        seg = (nchunks + ns - 1) / ns;
        // whole readout windows per segment: a segment starts a new window, so the
        // windows (and the results) do not depend on the segmentation
        seg -= seg % a.win;
    }
    const int nseg = (int)((nchunks + seg - 1) / seg);
    float* carrier = state;
    size_t need = (size_t)(per_chunk * seg);
    if (!state && nseg > 1) need += (size_t)state_b;
    rc = ensure_ws(t, need, st);
    if (rc) return rc;
    a.partial = (float*)t->ws;
    if (!carrier && nseg > 1) carrier = (float*)((char*)t->ws + per_chunk * seg);
    a.state = carrier;

    for (int s = 0; s < nseg; ++s) {
        a.c_begin = (int)(s * seg);
        a.c_end = (int)((s + 1) * seg < nchunks ? (s + 1) * seg : nchunks);
        a.load_state = (s > 0 || cont) ? 1 : 0;
        a.store_state = (s < nseg - 1 || state) ? 1 : 0;
        hipEvent_t ev = t->timer.begin(st);
        hipError_t e = use_mfma ? sata::launch_scan_mfma(a, t->mfma, st)
                                : sata::launch_scan_valu(a, st);
        t->timer.end(SATA_KERNEL_SCAN, ev, st);
        if (e != hipSuccess)
            return fail(SATA_ERR_HIP, "scan launch failed: %s", hipGetErrorString(e));
        ev = t->timer.begin(st);
        e = sata::launch_finalize(a, st);
        t->timer.end(SATA_KERNEL_FINALIZE, ev, st);
        if (e != hipSuccess)
            return fail(SATA_ERR_HIP, "finalize launch failed: %s", hipGetErrorString(e));
    }
    return SATA_OK;
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
    rc = ensure_ws(t, (size_t)(fixed + per_chunk * seg), st);
    if (rc) return rc;
    char* base = (char*)t->ws;
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

// Decode step shared by the dense and the pool forms: BH = batch entries x H heads;
// slots == NULL for the dense form.
int decode_impl(sata_tables* t, float* state, const int32_t* slots, int64_t pool, const void* q,
                const void* k, const void* v, float* y, int B, int H, int d_K, int d_V, int P,
                sata_dtype in_dtype, void* stream) {
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
    rc = check_device(t);
    if (rc) return rc;

    sata::DecodeArgs a{};
    a.state = state; a.q = q; a.k = k; a.v = v; a.y = y;
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

    std::lock_guard<std::mutex> lock(t->mu);
    hipStream_t st = (hipStream_t)stream;
    rc = ensure_ws(t, (size_t)sata::decode_partial_floats(a.BH, d_V, a.M_pad) * 4, st);
    if (rc) return rc;
    a.partial = (float*)t->ws;
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

}  // extern "C"
