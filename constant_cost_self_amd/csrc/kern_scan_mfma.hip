// kern_scan_mfma.hip -- bf16 MFMA chunked prefill scan for gfx950.
//
// The inter-chunk half of the chunked prefill ([TA] "Feature maps and linear
// attention": the state recurrence, evaluated chunk by chunk):
//     readout   part[t][j] = sum_f qw_f phi_f(q_t) S[f][j]      (S before the chunk)
//     update    S[f][j]   += sum_t phi_f(k_t) u_t[j],   u_t = [v_t | 1]
// Both are dense contractions over a 64-token chunk and a slice of the feature
// axis, run as v_mfma_f32_16x16x32_bf16 with fp32 accumulation:
//     readout  (64 tokens x 32 features) x (32 features x 16 columns)
//     update   (16 features x 32 tokens) x (32 tokens x 16 columns)
// with d_V + 1 = 65 columns padded to 5 tiles of 16.
//
// Work split.  One workgroup (4 waves) owns one slice of 64 rows = 512 kernel
// features of one head and walks all chunks of the segment in order; its fp32
// state slice never leaves the registers (8 update tiles x 5 column tiles x 4
// VGPRs = 160 per lane per wave).  A wave owns 16 rows of one l-block b: its
// kernel features are (parent a, l = 8b + e), e = 0..7 (see mfma_rows.cpp).
// Feature tiles are never written to HBM: per chunk the wave keeps the 8
// coordinates x_{8b..8b+7} of its tokens in registers and builds
//     query side  q^(a, l)[t] = (W_a q_a[t]) * q_l[t]        (W_a = alpha_p C(a) p)
//     key side    k^(a, l)[t] = kpar_a[t] * k_l[t] * c_(a,l)  (c: 0 / 1/(1+m) / 1)
// directly in the MFMA operand layout, where q_a, kpar_a are the parent products
// (kpar_a from a per-chunk LDS table).  The readout uses the register state
// converted to bf16 in place: the update's accumulator layout (lane = column,
// 4 rows each) concatenated over two tiles is exactly a 32-deep B operand, as
// long as the query operand uses the same feature order, which it does.
//
// Per chunk: stage q, k (fp32) and [v | 1] (bf16) in LDS; build the parent-product
// table; readout MFMAs (per-wave accumulators) written to LDS; update MFMAs; sum
// the 4 waves' readouts and write one 64 x (d_V + 1) partial per slice and chunk.
#include "scan_mfma.h"

#include <hip/hip_runtime.h>

namespace sata {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4v __attribute__((ext_vector_type(4)));

constexpr int kL = 64;     // chunk length of the MFMA scan

template <int D, int NCT>
struct Layout {
    static constexpr int QS = D + 12;        // qs row stride (floats): coords 0..D+7 + pad
    static constexpr int KT = 68;            // kT / kpar row stride (floats): 64 tokens + pad
    static constexpr int VT = 72;            // vT row stride (bf16): 64 tokens + pad
    static constexpr int UR = NCT * 16 + 4;  // per-wave readout row stride (floats)
    static constexpr int qs = 0;
    static constexpr int kt = qs + kL * QS;
    static constexpr int kp = kt + (D + 8) * KT;
    static constexpr int ur = kp + kRowsPerSlice * KT;
    static constexpr int vt_bytes = (ur + kWavesPerSlice * kL * UR) * 4;
    static constexpr int bytes = vt_bytes + NCT * 16 * VT * 2;
};

__device__ inline float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ inline float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

__device__ inline bf16x8 pack_bf16(const float* x) {
    bf16x8 r;
#pragma unroll
    for (int e = 0; e < 8; ++e) r[e] = (__bf16)x[e];
    return r;
}

__device__ inline bf16x8 pack_tiles(const f32x4v& lo, const f32x4v& hi) {
    bf16x8 r;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        r[e] = (__bf16)lo[e];
        r[4 + e] = (__bf16)hi[e];
    }
    return r;
}

struct RowPtrs {
    const uint32_t* parent;
    const float* weight;
    const float* kscale;
    const int32_t* canon;
    const int32_t* wave_lblock;
};

template <int D, int NCT>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void scan_mfma_kernel(PrefillSegArgs a, RowPtrs rt) {
    using LY = Layout<D, NCT>;
    constexpr int KS = kRowsPerWave / 4;     // readout K-steps per wave (32 features each)
    constexpr int NT = 2 * KS;               // update tiles per wave (16 features each)
    extern __shared__ __align__(16) unsigned char lds_raw[];
    float* lds = reinterpret_cast<float*>(lds_raw);
    float* qs = lds + LY::qs;
    float* kT = lds + LY::kt;
    float* kpar = lds + LY::kp;
    float* ured = lds + LY::ur;
    __bf16* vT = reinterpret_cast<__bf16*>(lds_raw + LY::vt_bytes);

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int g = lane >> 4, li = lane & 15;
    const int slice = blockIdx.x;
    const int64_t bh = blockIdx.y;
    const int d_V = a.d_V, cols = d_V + 1;
    const int nch = a.c_end - a.c_begin;
    const int row_wg = slice * kRowsPerSlice;               // first row of the workgroup
    const int row_w = row_wg + w * kRowsPerWave;            // first row of this wave
    const int lb = rt.wave_lblock[slice * kWavesPerSlice + w];

    const uint16_t* q = static_cast<const uint16_t*>(a.q) + bh * (int64_t)a.n * D;
    const uint16_t* k = static_cast<const uint16_t*>(a.k) + bh * (int64_t)a.n * D;
    const uint16_t* v = static_cast<const uint16_t*>(a.v) + bh * (int64_t)a.n * d_V;
    float* state = a.state ? a.state + bh * (int64_t)cols * a.M_pad : nullptr;

    // per-lane row constants
    uint32_t pc[KS];
    float Wq[KS];
#pragma unroll
    for (int s = 0; s < KS; ++s) {
        pc[s] = rt.parent[row_w + 4 * s + g];
        Wq[s] = rt.weight[row_w + 4 * s + g];
    }
    float cK[NT];
    bool ones[NT];
#pragma unroll
    for (int T = 0; T < NT; ++T) {
        const int s = T >> 1, h = T & 1;
        cK[T] = rt.kscale[(row_w + 4 * s + (li >> 2)) * 8 + 4 * h + (li & 3)];
        ones[T] = __all(cK[T] == 1.0f);
    }

    // resident state slice, update-accumulator layout: lane (column 16 ct + li, g)
    // register r of tile T = 2 s + h holds kernel feature (row 4 s + g, element 4 h + r).
    f32x4v S[NT][NCT];
#pragma unroll
    for (int T = 0; T < NT; ++T)
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) S[T][ct] = f32x4v{0.0f, 0.0f, 0.0f, 0.0f};
    if (a.load_state) {
        // through LDS, half of the tiles at a time: plain gather loop, then a
        // register fill with compile-time indices
#pragma unroll
        for (int ph = 0; ph < 2; ++ph) {
            __syncthreads();
            for (int idx = tid; idx < kWavesPerSlice * 64 * cols; idx += 256) {
                const int ww = idx / (64 * cols), rem = idx % (64 * cols);
                const int fl = rem / cols, j = rem % cols;
                const int T = (NT / 2) * ph + fl / 16, rho = fl % 16;
                const int fi = (row_wg + ww * kRowsPerWave + 4 * (T >> 1) + (rho >> 2)) * 8 +
                               4 * (T & 1) + (rho & 3);
                const int F = rt.canon[fi];
                ured[(ww * 64 + fl) * LY::UR + j] =
                    F >= 0 ? rt.kscale[fi] * state[(int64_t)j * a.M_pad + F] : 0.0f;
            }
            __syncthreads();
#pragma unroll
            for (int Tl = 0; Tl < NT / 2; ++Tl)
#pragma unroll
                for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int j = 16 * ct + li;
                        S[(NT / 2) * ph + Tl][ct][r] =
                            j < cols ? ured[(w * 64 + Tl * 16 + 4 * g + r) * LY::UR + j] : 0.0f;
                    }
        }
        __syncthreads();
    }

    // constant columns of [v | 1] beyond d_V
    for (int idx = tid; idx < (NCT * 16 - cols) * kL; idx += 256) {
        const int j = cols + idx / kL, t = idx % kL;
        vT[j * LY::VT + t] = (__bf16)0.0f;
    }

    for (int c = a.c_begin; c < a.c_end; ++c) {
        const int64_t t0 = (int64_t)c * kL;
        const int nvalid = (int)((a.n - t0) < kL ? (a.n - t0) : kL);

        // ---- stage the chunk -------------------------------------------------
        for (int idx = tid; idx < kL * (D / 4); idx += 256) {
            const int t = idx / (D / 4), c4 = idx % (D / 4);
            f32x4v x = {0.0f, 0.0f, 0.0f, 0.0f};
            if (t < nvalid) {
                const uint2 raw = *reinterpret_cast<const uint2*>(q + (t0 + t) * D + 4 * c4);
                x = f32x4v{bf16_lo(raw.x), bf16_hi(raw.x), bf16_lo(raw.y), bf16_hi(raw.y)};
            }
            *reinterpret_cast<f32x4v*>(qs + t * LY::QS + 4 * c4) = x;
        }
        for (int idx = tid; idx < kL * 8; idx += 256) {
            const int t = idx >> 3, e = idx & 7;
            qs[t * LY::QS + D + e] = e == 0 ? 1.0f : 0.0f;
            kT[(D + e) * LY::KT + t] = e == 0 ? 1.0f : 0.0f;
        }
        for (int idx = tid; idx < kL * (D / 4); idx += 256) {
            const int t = idx % kL, c4 = idx / kL;
            float x0 = 0.0f, x1 = 0.0f, x2 = 0.0f, x3 = 0.0f;
            if (t < nvalid) {
                const uint2 raw = *reinterpret_cast<const uint2*>(k + (t0 + t) * D + 4 * c4);
                x0 = bf16_lo(raw.x); x1 = bf16_hi(raw.x); x2 = bf16_lo(raw.y); x3 = bf16_hi(raw.y);
            }
            kT[(4 * c4 + 0) * LY::KT + t] = x0;
            kT[(4 * c4 + 1) * LY::KT + t] = x1;
            kT[(4 * c4 + 2) * LY::KT + t] = x2;
            kT[(4 * c4 + 3) * LY::KT + t] = x3;
        }
        for (int idx = tid; idx < kL * (d_V / 4); idx += 256) {
            const int t = idx % kL, c4 = idx / kL;
            uint2 raw = {0u, 0u};
            if (t < nvalid) raw = *reinterpret_cast<const uint2*>(v + (t0 + t) * d_V + 4 * c4);
            uint16_t* vt16 = reinterpret_cast<uint16_t*>(vT);
            vt16[(4 * c4 + 0) * LY::VT + t] = (uint16_t)(raw.x & 0xffffu);
            vt16[(4 * c4 + 1) * LY::VT + t] = (uint16_t)(raw.x >> 16);
            vt16[(4 * c4 + 2) * LY::VT + t] = (uint16_t)(raw.y & 0xffffu);
            vt16[(4 * c4 + 3) * LY::VT + t] = (uint16_t)(raw.y >> 16);
        }
        for (int t = tid; t < kL; t += 256) vT[d_V * LY::VT + t] = (__bf16)(t < nvalid ? 1.0f : 0.0f);
        __syncthreads();

        // ---- parent products of the key side, one per row of the slice --------
        for (int idx = tid; idx < kRowsPerSlice * kL; idx += 256) {
            const int r = idx / kL, t = idx % kL;
            const uint32_t p3 = rt.parent[row_wg + r];
            const float x = kT[(p3 & 1023u) * LY::KT + t] * kT[((p3 >> 10) & 1023u) * LY::KT + t] *
                            kT[((p3 >> 20) & 1023u) * LY::KT + t];
            kpar[r * LY::KT + t] = x;
        }
        __syncthreads();

        // ---- readout: U = Q^ . bf16(S) ------------------------------------------
        f32x4v U[4][NCT];
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct) U[mt][ct] = f32x4v{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            bf16x8 Sb[NCT];
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct) Sb[ct] = pack_tiles(S[2 * s][ct], S[2 * s + 1][ct]);
            const uint32_t p3 = pc[s];
            const int i0 = p3 & 1023u, i1 = (p3 >> 10) & 1023u, i2 = (p3 >> 20) & 1023u;
#pragma unroll
            for (int mt = 0; mt < 4; ++mt) {
                const float* qrow = qs + (16 * mt + li) * LY::QS;
                const f32x4v q0 = *reinterpret_cast<const f32x4v*>(qrow + 8 * lb);
                const f32x4v q1 = *reinterpret_cast<const f32x4v*>(qrow + 8 * lb + 4);
                const float qp = Wq[s] * qrow[i0] * qrow[i1] * qrow[i2];
                float x[8];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    x[e] = qp * q0[e];
                    x[4 + e] = qp * q1[e];
                }
                const bf16x8 A = pack_bf16(x);
#pragma unroll
                for (int ct = 0; ct < NCT; ++ct)
                    U[mt][ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, Sb[ct], U[mt][ct], 0, 0, 0);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        {
            float* ur = ured + w * kL * LY::UR;
#pragma unroll
            for (int mt = 0; mt < 4; ++mt)
#pragma unroll
                for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
                    for (int r = 0; r < 4; ++r) ur[(16 * mt + 4 * g + r) * LY::UR + 16 * ct + li] = U[mt][ct][r];
        }

        // ---- update: S += K^^T . [v | 1] ------------------------------------------
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
            bf16x8 Vop[NCT];
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct)
                Vop[ct] = *reinterpret_cast<const bf16x8*>(vT + (16 * ct + li) * LY::VT + 32 * kk + 8 * g);
#pragma unroll
            for (int T = 0; T < NT; ++T) {
                const int s = T >> 1, h = T & 1;
                const float* kp = kpar + (w * kRowsPerWave + 4 * s + (li >> 2)) * LY::KT + 32 * kk + 8 * g;
                const float* kv = kT + (8 * lb + 4 * h + (li & 3)) * LY::KT + 32 * kk + 8 * g;
                const f32x4v p0 = *reinterpret_cast<const f32x4v*>(kp);
                const f32x4v p1 = *reinterpret_cast<const f32x4v*>(kp + 4);
                const f32x4v v0 = *reinterpret_cast<const f32x4v*>(kv);
                const f32x4v v1 = *reinterpret_cast<const f32x4v*>(kv + 4);
                float x[8];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    x[e] = p0[e] * v0[e];
                    x[4 + e] = p1[e] * v1[e];
                }
                if (!ones[T]) {
#pragma unroll
                    for (int e = 0; e < 8; ++e) x[e] *= cK[T];
                }
                const bf16x8 A = pack_bf16(x);
#pragma unroll
                for (int ct = 0; ct < NCT; ++ct)
                    S[T][ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, Vop[ct], S[T][ct], 0, 0, 0);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        __syncthreads();

        // ---- sum the 4 waves' readouts into this slice's partial ------------------
        float* part = a.partial + ((bh * nch + (c - a.c_begin)) * a.nslices + slice) * (int64_t)kL * cols;
        for (int idx = tid; idx < kL * cols; idx += 256) {
            const int t = idx / cols, j = idx % cols;
            float s = 0.0f;
#pragma unroll
            for (int ww = 0; ww < kWavesPerSlice; ++ww) s += ured[(ww * kL + t) * LY::UR + j];
            part[idx] = s;
        }
    }

    if (a.store_state) {
        // through LDS as for the load; internal S' = c S is scaled back by 1/c
#pragma unroll
        for (int ph = 0; ph < 2; ++ph) {
            __syncthreads();
#pragma unroll
            for (int Tl = 0; Tl < NT / 2; ++Tl)
#pragma unroll
                for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        ured[(w * 64 + Tl * 16 + 4 * g + r) * LY::UR + 16 * ct + li] =
                            S[(NT / 2) * ph + Tl][ct][r];
            __syncthreads();
            for (int idx = tid; idx < kWavesPerSlice * 64 * cols; idx += 256) {
                const int ww = idx / (64 * cols), rem = idx % (64 * cols);
                const int fl = rem / cols, j = rem % cols;
                const int T = (NT / 2) * ph + fl / 16, rho = fl % 16;
                const int fi = (row_wg + ww * kRowsPerWave + 4 * (T >> 1) + (rho >> 2)) * 8 +
                               4 * (T & 1) + (rho & 3);
                const int F = rt.canon[fi];
                if (F >= 0) state[(int64_t)j * a.M_pad + F] = ured[(ww * 64 + fl) * LY::UR + j] / rt.kscale[fi];
            }
        }
        if (slice == 0) {
            const int64_t padn = a.M_pad - a.M;
            for (int64_t idx = tid; idx < cols * padn; idx += 256)
                state[(idx / padn) * a.M_pad + a.M + idx % padn] = 0.0f;
        }
    }
}

template <int D, int NCT>
hipError_t launch_t(const PrefillSegArgs& a, const MfmaTables& m, hipStream_t st) {
    using LY = Layout<D, NCT>;
    static_assert(LY::bytes <= 160 * 1024, "LDS budget");
    RowPtrs rt{m.parent, m.weight, m.kscale, m.canon, m.wave_lblock};
    hipError_t e = hipFuncSetAttribute((const void*)scan_mfma_kernel<D, NCT>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, LY::bytes);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((scan_mfma_kernel<D, NCT>), dim3(a.nslices, a.BH), dim3(256), LY::bytes, st,
                       a, rt);
    return hipGetLastError();
}

}  // namespace

int build_mfma_tables(const HostTables& h, MfmaTables& m) {
    m = MfmaTables();
    MfmaHostRows r;
    if (!build_mfma_rows(h, r)) return 0;        // not an MFMA shape: the VALU scan is used
    const size_t nr = (size_t)r.nrows, nw = r.wave_lblock.size();
    const size_t bytes = nr * 4 + nr * 4 + nr * 8 * 4 + nr * 8 * 4 + nw * 4;
    char* base = nullptr;
    if (hipMalloc(&base, bytes) != hipSuccess) {
        (void)hipGetLastError();
        return -5;
    }
    size_t off = 0;
    auto put = [&](const void* src, size_t n) -> void* {
        void* dst = base + off;
        off += n;
        return hipMemcpy(dst, src, n, hipMemcpyHostToDevice) == hipSuccess ? dst : nullptr;
    };
    m.parent = (const uint32_t*)put(r.parent.data(), nr * 4);
    m.weight = (const float*)put(r.weight.data(), nr * 4);
    m.kscale = (const float*)put(r.kscale.data(), nr * 8 * 4);
    m.canon = (const int32_t*)put(r.canon.data(), nr * 8 * 4);
    m.wave_lblock = (const int32_t*)put(r.wave_lblock.data(), nw * 4);
    m.d_rows = base;
    if (!m.parent || !m.weight || !m.kscale || !m.canon || !m.wave_lblock) {
        free_mfma_tables(m);
        return -4;
    }
    m.nslices = r.nrows / kRowsPerSlice;
    m.slice_feats = kRowsPerSlice * 8;
    m.d_K = r.d_K;
    m.P = r.P;
    m.ok = true;
    return 0;
}

void free_mfma_tables(MfmaTables& m) {
    if (m.d_rows) (void)hipFree(m.d_rows);
    m = MfmaTables();
}

bool mfma_supported(const MfmaTables& m, bool bf16, int d_K, int d_V, int P, int L) {
    return m.ok && bf16 && d_K == m.d_K && P == m.P && L == kL && d_K == 64 && d_V % 4 == 0 &&
           d_V + 1 <= 80 && d_V + 1 > 64;
}

hipError_t launch_scan_mfma(const PrefillSegArgs& a, const MfmaTables& m, hipStream_t st) {
    return launch_t<64, 5>(a, m, st);
}

}  // namespace sata
