// kern_prefill_valu.hip -- fp32 chunked prefill scan (gfx950).
//
// The inter-chunk half of the chunked prefill ([TA] "Feature maps and linear
// attention": the state recurrence evaluated chunk by chunk).  A block owns one
// slice of `SV` consecutive features of one head's state, S[f][0..d_V] (column
// d_V is Z), keeps it in LDS for the whole segment and walks the chunks in order.
// For chunk c with tokens t0..t0+L-1:
//     readout   part[t][j] = sum_{f in slice} qw[f] phi_f(q_t) S[f][j]   (S before c)
//     update    S[f][j]   += sum_t phi_f(k_t) u_t[j],   u_t = [v_t | 1]
// The readout of every slice is written as a partial sum ([column][token] within
// the chunk); the finalize kernel adds
// the partials of all slices to the intra-chunk part.  Arithmetic is fp32 (the two
// contractions on the matrix cores with fp32 operands, mfma_gemm): this is the path for
// fp32 inputs and for sizes the fp16-operand MFMA scan does not cover.  Tokens past n in
// the last chunk get u = 0 and so never enter the state.
#include "launch.h"
#include "sata_common.h"

namespace sata {

namespace {

__host__ __device__ inline int64_t valu_lds_floats(int SV, int d_K, int d_V, int L) {
    const int cols = d_V + 1;
    return (int64_t)SV * cols + 2LL * L * (d_K + 1) + (int64_t)L * cols + (int64_t)L * (SV + 1) + 2LL * SV;
}

template <typename In, int NIDX>
__global__ __launch_bounds__(kScanThreads) void scan_valu_kernel(PrefillSegArgs a) {
    using T = typename In::T;
    extern __shared__ float lds[];
    const int slice = blockIdx.x;
    const int64_t bh = blockIdx.y;
    const int tid = threadIdx.x;
    const int SV = a.slice_feats, L = a.L, d_K = a.d_K, d_V = a.d_V, cols = d_V + 1;
    const int64_t F0 = (int64_t)slice * SV;

    float* Ssl = lds;                              // [SV][cols]
    float* xq = Ssl + SV * cols;                   // [L][d_K+1], coordinate d_K == 1
    float* xk = xq + L * (d_K + 1);                // [L][d_K+1]
    float* us = xk + L * (d_K + 1);                // [L][cols]
    const int SVP = SV + 1;                        // row stride of 1 modulo 64 floats
    float* hat = us + L * cols;                    // [L][SVP]
    uint32_t* sfi = reinterpret_cast<uint32_t*>(hat + L * SVP);  // [SV] packed indices
    float* sqw = reinterpret_cast<float*>(sfi + SV);             // [SV] query weights
    for (int f = tid; f < SV; f += kScanThreads) {   // tables are M_pad long (padding: weight 0)
        const int64_t F = F0 + f;
        sfi[f] = F < a.M_pad ? a.fidx[F] : 0u;
        sqw[f] = F < a.M_pad ? a.qw[F] : 0.0f;
    }

    const T* q = static_cast<const T*>(a.q) + bh * a.n * d_K;
    const T* k = static_cast<const T*>(a.k) + bh * a.n * d_K;
    const T* v = static_cast<const T*>(a.v) + bh * a.n * d_V;
    float* state = a.state ? a.state + bh * (int64_t)cols * a.M_pad : nullptr;

    for (int idx = tid; idx < SV * cols; idx += kScanThreads) {
        const int f = idx / cols, j = idx % cols;
        const int64_t F = F0 + f;
        Ssl[idx] = (a.load_state && F < a.M_pad) ? state[(int64_t)j * a.M_pad + F] : 0.0f;
    }

    const int nch = a.c_end - a.c_begin;
    // the next chunk's rows are loaded into registers while this chunk is computed
    using Stage = RowStage<In, kScanThreads, 2>;
    Stage sq, sk, sv;
    const bool staged = Stage::fits(L, d_K) && Stage::fits(L, d_V);
    auto issue = [&](int c) {
        const int64_t t0 = (int64_t)c * L;
        const int nvalid = (int)((a.n - t0) < L ? (a.n - t0) : L);
        sq.issue(q, t0, nvalid, L, d_K);
        sk.issue(k, t0, nvalid, L, d_K);
        sv.issue(v, t0, nvalid, L, d_V);
    };
    if (staged) issue(a.c_begin);
    for (int c = a.c_begin; c < a.c_end; ++c) {
        const int64_t t0 = (int64_t)c * L;
        const int nvalid = (int)((a.n - t0) < L ? (a.n - t0) : L);
        __syncthreads();
        if (staged) {
            sq.commit(xq, d_K + 1, L, d_K, d_K);
            sk.commit(xk, d_K + 1, L, d_K, d_K);
            sv.commit(us, cols, L, d_V, d_V);
        } else {
            load_rows<In, kScanThreads>(q, t0, nvalid, L, d_K, xq, d_K + 1);
            load_rows<In, kScanThreads>(k, t0, nvalid, L, d_K, xk, d_K + 1);
            load_rows<In, kScanThreads>(v, t0, nvalid, L, d_V, us, cols);
        }
        for (int t = tid; t < L; t += kScanThreads) {      // coordinate d_K == 1; u = [v | 1]
            xq[t * (d_K + 1) + d_K] = 1.0f;
            xk[t * (d_K + 1) + d_K] = 1.0f;
            us[t * cols + d_V] = t < nvalid ? 1.0f : 0.0f;
        }
        __syncthreads();
        if (staged && c + 1 < a.c_end) issue(c + 1);        // in flight during this chunk
        // weighted query features of the slice
        // (a thread owns feature tid % SV, a power of two, for tokens tid / SV + k NT / SV)
        const int fo = tid & (SV - 1);
        const bool flive = F0 + fo < a.M;
        const uint32_t fi = sfi[fo];
        const float fw = sqw[fo];
        for (int t = tid / SV; t < L; t += kScanThreads / SV)
            hat[t * SVP + fo] = flive ? fw * feature_value_n<NIDX>(xq + t * (d_K + 1), fi) : 0.0f;
        __syncthreads();
        // readout against the state of the chunks before c
        float* part = a.partial +
                      (((bh * nch + (c - a.c_begin)) * a.nslices + slice) * (int64_t)L) * cols;
        mfma_gemm<kScanThreads>(L, cols, SV, hat, SVP, 1, Ssl, cols, 1, [&](int t, int j, float c) { part[j * L + t] = c; });
        __syncthreads();
        // key features of the slice
        for (int t = tid / SV; t < L; t += kScanThreads / SV)
            hat[t * SVP + fo] = flive ? feature_value_n<NIDX>(xk + t * (d_K + 1), fi) : 0.0f;
        __syncthreads();
        // state update with the chunk
        mfma_gemm<kScanThreads>(SV, cols, L, hat, 1, SVP, us, cols, 1, [&](int f, int j, float c) { Ssl[f * cols + j] += c; });
    }
    __syncthreads();
    if (a.store_state) {
        for (int idx = tid; idx < SV * cols; idx += kScanThreads) {
            const int j = idx / SV, f = idx % SV;
            const int64_t F = F0 + f;
            if (F < a.M_pad) state[(int64_t)j * a.M_pad + F] = Ssl[f * cols + j];
        }
    }
}

}  // namespace

// a power of two no larger than the block (the feature loops rely on it)
int valu_slice_feats(int d_K, int d_V, int L) {
    for (int SV = 256; SV >= 16; SV >>= 1)
        if (valu_lds_floats(SV, d_K, d_V, L) * 4 <= 96 * 1024) return SV;
    return 0;
}

namespace {

template <int NIDX>
hipError_t launch_scan_valu_n(const PrefillSegArgs& a, hipStream_t st) {
    const size_t lds = (size_t)valu_lds_floats(a.slice_feats, a.d_K, a.d_V, a.L) * 4;
    dim3 grid(a.nslices, a.BH);
    auto kernel = a.bf16 ? scan_valu_kernel<InBF16, NIDX> : scan_valu_kernel<InF32, NIDX>;
    hipError_t e = hipFuncSetAttribute((const void*)kernel, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kernel, grid, dim3(kScanThreads), lds, st, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_scan_valu(const PrefillSegArgs& a, hipStream_t st) {
    switch (a.P - 1) {                 // slots per feature
        case 0: return launch_scan_valu_n<0>(a, st);
        case 1: return launch_scan_valu_n<1>(a, st);
        case 2: return launch_scan_valu_n<2>(a, st);
        case 3: return launch_scan_valu_n<3>(a, st);
        default: return launch_scan_valu_n<4>(a, st);
    }
}

}  // namespace sata
