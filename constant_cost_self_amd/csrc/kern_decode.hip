// kern_decode.hip -- one-token decode step over a batch of heads (gfx950).
//
// Per head ([TA] "Feature maps and linear attention": the recurrences
// Z_T = Z_{T-1} + phi(k_T), S_T = S_{T-1} + phi(k_T) v_T^T, then the readout):
//     S[f][j] += phi_f(k) u[j]          u = [v | 1]
//     acc[j]   = sum_f qw[f] phi_f(q) S[f][j]
//     y[j]     = acc[j] / acc[d_V]
// where qw[f] = alpha_p C_p[f].  The state is the fp32 array [cols][M_pad] of the
// head (cols = d_V + 1), read and written in place exactly once: the step is a
// streaming read-modify-write and is bound by HBM bandwidth (8 bytes of traffic
// per state entry for 4 flops).
//
// Kernel 1 (decode_step_kernel): grid (feature blocks, heads), 256 threads.  A
// thread owns 4 consecutive features per group and walks all columns with 16-byte
// non-temporal loads/stores, so each wave touches 1 KiB contiguous per column.
// The per-thread partial readouts are reduced over the block and written as one
// row of `cols` partial sums per (head, block).
// Kernel 2 (decode_finalize_kernel): one block per head sums the partial rows and
// divides by the normaliser column.
// Pool form ([HW] "The fixed-size hidden state of SATA attention": the state's memory
// is allocated up front and requests share the device in turns): batch entry b uses
// the state in slot slots[b] of a preallocated pool instead of state b.
#include "launch.h"
#include "sata_common.h"

namespace sata {

namespace {

constexpr int kDecGroups = 1;                         // feature groups per thread (measured best)
constexpr int kDecFeatPerBlock = kThreads * 4 * kDecGroups;   // 1024

template <typename In, int CMAX>
__global__ __launch_bounds__(kThreads) void decode_step_kernel(
    float* __restrict__ state, const typename In::T* __restrict__ q,
    const typename In::T* __restrict__ k, const typename In::T* __restrict__ v,
    const uint32_t* __restrict__ fidx, const float* __restrict__ qw,
    float* __restrict__ partial, int64_t M, int64_t M_pad, int d_K, int d_V, int P,
    int nblk, const int32_t* __restrict__ slots, int64_t pool, int H) {
    const int blk = blockIdx.x;
    const int64_t bh = blockIdx.y;
    const int tid = threadIdx.x;
    const int cols = d_V + 1;
    // state of this head: its own (dense form) or the one in its entry's pool slot; an
    // entry whose slot is outside the pool leaves the pool alone and reads out NaN
    int64_t sh = bh;
    if (slots) {
        const int64_t s = slots[bh / H];
        if (s < 0 || s >= pool) {
            for (int j = tid; j < cols; j += kThreads) partial[(bh * nblk + blk) * cols + j] = __builtin_nanf("");
            return;
        }
        sh = s * H + bh % H;
    }

    __shared__ float xq[kMaxD + 1];
    __shared__ float xk[kMaxD + 1];
    __shared__ float us[kMaxD + 1];
    __shared__ float red[kThreads / 64][CMAX];

    for (int i = tid; i <= d_K; i += kThreads) {
        xq[i] = i < d_K ? In::load(q, bh * d_K + i) : 1.0f;
        xk[i] = i < d_K ? In::load(k, bh * d_K + i) : 1.0f;
    }
    for (int j = tid; j < cols; j += kThreads)
        us[j] = j < d_V ? In::load(v, bh * d_V + j) : 1.0f;
    __syncthreads();

    float acc[CMAX];
#pragma unroll
    for (int j = 0; j < CMAX; ++j) acc[j] = 0.0f;

    float* __restrict__ S = state + sh * (int64_t)cols * M_pad;
    const int nidx = P - 1;

    for (int g = 0; g < kDecGroups; ++g) {
        const int64_t f0 = (int64_t)blk * kDecFeatPerBlock + ((int64_t)g * kThreads + tid) * 4;
        if (f0 >= M_pad) break;
        float pk[4], pq[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int64_t f = f0 + e;
            if (f < M) {
                const uint32_t packed = fidx[f];
                pk[e] = feature_value(xk, packed, nidx);
                pq[e] = qw[f] * feature_value(xq, packed, nidx);
            } else {
                pk[e] = 0.0f;
                pq[e] = 0.0f;
            }
        }
#pragma unroll
        for (int j = 0; j < CMAX; ++j) {
            if (j < cols) {
                f32x4* p = reinterpret_cast<f32x4*>(S + (int64_t)j * M_pad + f0);
                f32x4 s = __builtin_nontemporal_load(p);
                const float u = us[j];
                s.x = fmaf(pk[0], u, s.x);
                s.y = fmaf(pk[1], u, s.y);
                s.z = fmaf(pk[2], u, s.z);
                s.w = fmaf(pk[3], u, s.w);
                __builtin_nontemporal_store(s, p);
                acc[j] = fmaf(pq[0], s.x, acc[j]);
                acc[j] = fmaf(pq[1], s.y, acc[j]);
                acc[j] = fmaf(pq[2], s.z, acc[j]);
                acc[j] = fmaf(pq[3], s.w, acc[j]);
            }
        }
    }

    // block reduction of acc[0..cols)
    const int lane = tid & 63, wave = tid >> 6;
#pragma unroll
    for (int j = 0; j < CMAX; ++j) {
        float a = acc[j];
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) a += __shfl_xor(a, off, 64);
        if (lane == 0) red[wave][j] = a;
    }
    __syncthreads();
    for (int j = tid; j < cols; j += kThreads) {
        float s = 0.0f;
#pragma unroll
        for (int w = 0; w < kThreads / 64; ++w) s += red[w][j];
        partial[(bh * nblk + blk) * cols + j] = s;
    }
}

__global__ __launch_bounds__(kThreads) void decode_finalize_kernel(
    const float* __restrict__ partial, float* __restrict__ y, int d_V, int nblk) {
    const int64_t bh = blockIdx.x;
    const int cols = d_V + 1;
    __shared__ float num[kMaxD + 1];
    for (int j = threadIdx.x; j < cols; j += kThreads) {
        float s = 0.0f;
        for (int b = 0; b < nblk; ++b) s += partial[(bh * nblk + b) * cols + j];
        num[j] = s;
    }
    __syncthreads();
    for (int j = threadIdx.x; j < d_V; j += kThreads) y[bh * d_V + j] = num[j] / num[d_V];
}

template <typename In, int CMAX>
hipError_t launch_decode_t(const DecodeArgs& a, hipStream_t st) {
    dim3 grid(a.nblk, a.BH);
    hipLaunchKernelGGL((decode_step_kernel<In, CMAX>), grid, dim3(kThreads), 0, st,
                       a.state, static_cast<const typename In::T*>(a.q),
                       static_cast<const typename In::T*>(a.k),
                       static_cast<const typename In::T*>(a.v), a.fidx, a.qw, a.partial, a.M,
                       a.M_pad, a.d_K, a.d_V, a.P, a.nblk, a.slots, a.pool, a.H);
    return hipGetLastError();
}

template <typename In>
hipError_t launch_decode_in(const DecodeArgs& a, hipStream_t st) {
    const int cols = a.d_V + 1;
    if (cols <= 9) return launch_decode_t<In, 9>(a, st);
    if (cols <= 17) return launch_decode_t<In, 17>(a, st);
    if (cols <= 33) return launch_decode_t<In, 33>(a, st);
    if (cols <= 65) return launch_decode_t<In, 65>(a, st);
    return launch_decode_t<In, 129>(a, st);
}

}  // namespace

int decode_blocks(int64_t M_pad) { return (int)((M_pad + kDecFeatPerBlock - 1) / kDecFeatPerBlock); }

hipError_t launch_decode(const DecodeArgs& a, hipStream_t st) {
    return a.bf16 ? launch_decode_in<InBF16>(a, st) : launch_decode_in<InF32>(a, st);
}

hipError_t launch_decode_reduce(const DecodeArgs& a, hipStream_t st) {
    hipLaunchKernelGGL(decode_finalize_kernel, dim3(a.BH), dim3(kThreads), 0, st, a.partial,
                       a.y, a.d_V, a.nblk);
    return hipGetLastError();
}

}  // namespace sata
