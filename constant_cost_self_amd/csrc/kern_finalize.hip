// kern_finalize.hip -- intra-chunk part, slice reduction and normalisation (gfx950).
//
// For every chunk of L tokens of a head, the rows T of the chunk attend to the
// earlier tokens of the same chunk directly, with the truncated kernel on the
// plain dot product ([TA] "Feature maps and linear attention": w(q,k) =
// sum_{p<P} alpha_p (q.k)^p), and to everything before the chunk through the
// state (the slice partials written by the scan):
//     U[T][j] = sum_{t0<=t<=T} w(q_T, k_t) u_t[j]  +  sum_slices part[slice][T][j]
//     y[T][j] = U[T][j] / U[T][d_V]               (u_t = [v_t | 1])
// One block per (chunk, head); fp32 arithmetic; w by Horner's rule.
#include "launch.h"
#include "sata_common.h"

namespace sata {

namespace {

__host__ __device__ inline int64_t finalize_lds_floats(int d_K, int d_V, int L) {
    const int wide = (d_K + 1) > (d_V + 1) ? (d_K + 1) : (d_V + 1);
    return (int64_t)L * (L + 1) + 2LL * L * wide;
}

template <typename In>
__global__ __launch_bounds__(kThreads) void finalize_kernel(PrefillSegArgs a) {
    using T = typename In::T;
    extern __shared__ float lds[];
    const int cl = blockIdx.x;                  // chunk within the segment
    const int64_t bh = blockIdx.y;
    const int c = a.c_begin + cl;
    const int tid = threadIdx.x;
    const int L = a.L, d_K = a.d_K, d_V = a.d_V, cols = d_V + 1, ks = d_K + 1;
    const int wide = ks > cols ? ks : cols;
    const int nch = a.c_end - a.c_begin;
    const int64_t t0 = (int64_t)c * L;
    const int nvalid = (int)((a.n - t0) < L ? (a.n - t0) : L);

    float* W = lds;                              // [L][L+1]
    float* xq = W + L * (L + 1);                 // [L][d_K+1]   (phase 1)
    float* xk = xq + L * ks;                     // [L][d_K+1]   (phase 1)
    float* us = W + L * (L + 1);                 // [L][cols]    (phase 2)
    float* num = us + L * wide;                  // [L][cols]    (phase 2)

    const T* q = static_cast<const T*>(a.q) + (bh * a.n + t0) * d_K;
    const T* k = static_cast<const T*>(a.k) + (bh * a.n + t0) * d_K;
    const T* v = static_cast<const T*>(a.v) + (bh * a.n + t0) * d_V;

    for (int idx = tid; idx < L * d_K; idx += kThreads) {
        const int t = idx / d_K, i = idx % d_K;
        xq[t * ks + i] = t < nvalid ? In::load(q, idx) : 0.0f;
        xk[t * ks + i] = t < nvalid ? In::load(k, idx) : 0.0f;
    }
    __syncthreads();
    for (int idx = tid; idx < L * L; idx += kThreads) {
        const int T_ = idx / L, s = idx % L;
        float w = 0.0f;
        if (s <= T_ && T_ < nvalid) {
            const float* qa = xq + T_ * ks;
            const float* kb = xk + s * ks;
            float x = 0.0f;
            for (int i = 0; i < d_K; ++i) x = fmaf(qa[i], kb[i], x);
            w = taylor_weight(x, a.alpha, a.P);
        }
        W[T_ * (L + 1) + s] = w;
    }
    __syncthreads();
    for (int idx = tid; idx < L * cols; idx += kThreads) {
        const int t = idx / cols, j = idx % cols;
        float u = 0.0f;
        if (t < nvalid) u = j < d_V ? In::load(v, (int64_t)t * d_V + j) : 1.0f;
        us[idx] = u;
    }
    __syncthreads();
    const float* part = a.partial + ((bh * nch + cl) * (int64_t)a.nslices) * L * cols;
    for (int idx = tid; idx < L * cols; idx += kThreads) {
        const int j = idx / L, T_ = idx % L;      // token fastest: coalesced partial reads
        const float* wr = W + T_ * (L + 1);
        float acc = 0.0f;
        for (int s = 0; s <= T_; ++s) acc = fmaf(wr[s], us[s * cols + j], acc);
        // slice partials: read once, four independent sums to keep loads in flight
        const float* p = part + j * L + T_;           // partials are [column][token]
        const int64_t stride = (int64_t)L * cols;
        float a0 = 0.0f, a1 = 0.0f, a2 = 0.0f, a3 = 0.0f;
        int sl = 0;
        for (; sl + 4 <= a.nslices; sl += 4) {
            a0 += __builtin_nontemporal_load(p + (sl + 0) * stride);
            a1 += __builtin_nontemporal_load(p + (sl + 1) * stride);
            a2 += __builtin_nontemporal_load(p + (sl + 2) * stride);
            a3 += __builtin_nontemporal_load(p + (sl + 3) * stride);
        }
        for (; sl < a.nslices; ++sl) a0 += __builtin_nontemporal_load(p + sl * stride);
        num[T_ * cols + j] = acc + ((a0 + a1) + (a2 + a3));
    }
    __syncthreads();
    float* y = a.y + (bh * a.n + t0) * d_V;
    for (int idx = tid; idx < nvalid * d_V; idx += kThreads) {
        const int t = idx / d_V, j = idx % d_V;
        y[idx] = num[t * cols + j] / num[t * cols + d_V];
    }
}

}  // namespace

int64_t finalize_lds_bytes(int d_K, int d_V, int L) { return finalize_lds_floats(d_K, d_V, L) * 4; }

hipError_t launch_finalize(const PrefillSegArgs& a, hipStream_t st) {
    const size_t lds = (size_t)finalize_lds_bytes(a.d_K, a.d_V, a.L);
    dim3 grid(a.c_end - a.c_begin, a.BH);
    if (a.bf16) {
        hipError_t e = hipFuncSetAttribute((const void*)finalize_kernel<InBF16>,
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL(finalize_kernel<InBF16>, grid, dim3(kThreads), lds, st, a);
    } else {
        hipError_t e = hipFuncSetAttribute((const void*)finalize_kernel<InF32>,
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL(finalize_kernel<InF32>, grid, dim3(kThreads), lds, st, a);
    }
    return hipGetLastError();
}

}  // namespace sata
