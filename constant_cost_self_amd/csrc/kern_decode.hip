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
// Kernel 1 (decode_sweep_kernel): workgroup (g, b) of head h updates 1024 features of
// four columns of the state, two 16-byte non-temporal loads and stores per thread and
// column, all loads issued before any arithmetic.  Consecutive workgroups take
// consecutive feature blocks of the same four columns, so the workgroups in flight
// stream four contiguous windows of HBM.  phi(k) and the weighted phi(q) of a thread's
// 8 features are computed once (packed index table, q and k staged in LDS per wave)
// and serve the four columns.  Measured on MI355X at d = 64, P = 4: one column per
// workgroup recomputes the features 65 times and reaches about 3.5-4.6 TB/s, one
// thread walking all 65 columns about 5.1 TB/s, four columns about 5.6 TB/s.  Each
// wave writes its partial readout of each column.
// Kernel 2 (decode_finalize_kernel): per head, one workgroup per 16 value columns sums
// their partials and the normaliser column's, and divides.
// Pool form ([HW] "The fixed-size hidden state of SATA attention": the state's memory
// is allocated up front and requests share the device in turns): batch entry b uses
// the state in slot slots[b] of a preallocated pool instead of state b.
#include <mutex>

#include "launch.h"
#include "sata_common.h"

namespace sata {

// Fixed scratch of the allocation-free decode step: the partial readouts of one call, in a
// file-scope device array that each GPU holds until the process ends.  Host code must not
// pass `scratch` itself to a kernel (on the host it is only a stand-in symbol): its device
// address is taken once per device with hipGetSymbolAddress and that address is used.
static __device__ __align__(256) float scratch[kNoAllocScratchBytes / 4];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
float* g_scratch_ptr[kMaxDevices] = {};
}  // namespace

hipError_t noalloc_scratch(int device, float** ptr) {
    *ptr = nullptr;
    if (device < 0 || device >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[device]) {
        void* p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        g_scratch_ptr[device] = static_cast<float*>(p);
    }
    *ptr = g_scratch_ptr[device];
    return hipSuccess;
}

namespace {

constexpr int kDecThreads = 128;                         // block size of the sweep
constexpr int kDecVec = 2;                               // 16-byte groups per thread
constexpr int kDecCols = 4;                              // state columns per workgroup
constexpr int kDecFeatPerBlock = kDecThreads * 4 * kDecVec;
constexpr int kDecWaves = kDecThreads / 64;
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// grid (ceil(cols / kDecCols) * nblk, BH): x = column group * nblk + feature block
template <typename In, int NIDX>
__global__ __launch_bounds__(kDecThreads) void decode_sweep_kernel(
    float* __restrict__ state, const typename In::T* __restrict__ q,
    const typename In::T* __restrict__ k, const typename In::T* __restrict__ v,
    const uint32_t* __restrict__ fidx, const float* __restrict__ qw,
    float* __restrict__ partial, int64_t M, int64_t M_pad, int d_K, int d_V,
    int nblk, const int32_t* __restrict__ slots, int64_t pool, int H) {
    const int cols = d_V + 1;
    const int64_t bh = blockIdx.y;
    const int fb = (int)(blockIdx.x % nblk);
    const int j0 = (int)(blockIdx.x / nblk) * kDecCols;
    const int ncol = min(kDecCols, cols - j0);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    // partial readouts: [BH][cols][nblk][kDecWaves]
    const int64_t pstride = (int64_t)nblk * kDecWaves;
    float* __restrict__ pw = partial + (bh * cols + j0) * pstride + fb * kDecWaves + wave;

    // state of this head: its own (dense form) or the one in its entry's pool slot; an
    // entry whose slot is outside the pool leaves the pool alone and reads out NaN
    int64_t sh = bh;
    if (slots) {
        const int64_t s = slots[bh / H];
        if (s < 0 || s >= pool) {
            if (lane == 0)
                for (int c = 0; c < ncol; ++c) pw[c * pstride] = __builtin_nanf("");
            return;
        }
        sh = s * H + bh % H;
    }

    // The small inputs (q, k, v, the features' index rows and query weights) are loaded
    // before the state, so that the features are computed while the state is in flight
    // (loads complete in order).  Every load is unconditional, from a valid place (indices
    // past the end clamped), so that no wait comes before the state loads are all issued;
    // only live features and columns are used and stored.  The tables are M_pad long
    // (padding rows have weight 0 and an all-sentinel index row).
    const int ti0 = min(lane, d_K - 1), ti1 = min(lane + 64, d_K - 1);
    const float q0 = In::load(q, bh * d_K + ti0), q1 = In::load(q, bh * d_K + ti1);
    const float k0 = In::load(k, bh * d_K + ti0), k1 = In::load(k, bh * d_K + ti1);
    float u[kDecCols];
#pragma unroll
    for (int c = 0; c < kDecCols; ++c) u[c] = In::load(v, bh * d_V + min(j0 + c, d_V - 1));
    const int64_t f0 = (int64_t)fb * kDecFeatPerBlock + tid * 4;
    int64_t fl[kDecVec];
    u32x4 packed[kDecVec];
    f32x4 w[kDecVec];
#pragma unroll
    for (int g = 0; g < kDecVec; ++g) {
        fl[g] = min(f0 + g * kDecThreads * 4, M_pad - 4);
        packed[g] = *reinterpret_cast<const u32x4*>(fidx + fl[g]);
        w[g] = *reinterpret_cast<const f32x4*>(qw + fl[g]);
    }
    float* __restrict__ base = state + (sh * cols + j0) * M_pad;
    f32x4 s[kDecVec][kDecCols];
#pragma unroll
    for (int g = 0; g < kDecVec; ++g)
#pragma unroll
        for (int c = 0; c < kDecCols; ++c)
            s[g][c] = __builtin_nontemporal_load(
                reinterpret_cast<const f32x4*>(base + min(c, ncol - 1) * M_pad + fl[g]));

    // this wave's copy of the head's q and k coordinates and the constant 1 (index d_K)
    __shared__ float xs[kDecWaves][2][kMaxD + 1];
    float* xq = xs[wave][0];
    float* xk = xs[wave][1];
    if (lane < d_K) { xq[lane] = q0; xk[lane] = k0; }
    if (lane + 64 < d_K) { xq[lane + 64] = q1; xk[lane + 64] = k1; }
    if (lane == 0) { xq[d_K] = 1.0f; xk[d_K] = 1.0f; }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

    float acc[kDecCols];
#pragma unroll
    for (int c = 0; c < kDecCols; ++c) acc[c] = 0.0f;
#pragma unroll
    for (int g = 0; g < kDecVec; ++g) {
        const int64_t f = f0 + g * kDecThreads * 4;
        // phi(k) masked to f < M keeps the padding of S at zero
        float pk[4], pq[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            pk[e] = f + e < M ? feature_value_n<NIDX>(xk, packed[g][e]) : 0.0f;
            pq[e] = w[g][e] * feature_value_n<NIDX>(xq, packed[g][e]);
        }
        if (f < M_pad) {
#pragma unroll
            for (int c = 0; c < kDecCols; ++c) {
                if (c < ncol) {
                    const float uc = j0 + c < d_V ? u[c] : 1.0f;
                    f32x4 t = s[g][c];
                    t.x = fmaf(pk[0], uc, t.x);
                    t.y = fmaf(pk[1], uc, t.y);
                    t.z = fmaf(pk[2], uc, t.z);
                    t.w = fmaf(pk[3], uc, t.w);
                    __builtin_nontemporal_store(t, reinterpret_cast<f32x4*>(base + c * M_pad + f));
                    acc[c] = fmaf(pq[0], t.x, fmaf(pq[1], t.y, fmaf(pq[2], t.z, fmaf(pq[3], t.w, acc[c]))));
                }
            }
        }
    }
#pragma unroll
    for (int c = 0; c < kDecCols; ++c) {
        const float a = wave_sum64(acc[c]);
        if (lane == 0 && c < ncol) pw[c * pstride] = a;
    }
}

// grid (BH, ceil(d_V / 16)): workgroup (h, c) writes y of head h for value columns 16 c ..
// 16 c + 15: each wave sums the partials of one of those columns (lanes over the feature
// blocks and waves of the column) and of the normaliser column, then y = num / normaliser
constexpr int kFinCols = 16;

__global__ __launch_bounds__(kThreads) void decode_finalize_kernel(
    const float* __restrict__ partial, float* __restrict__ y, int d_V, int nblk) {
    const int64_t bh = blockIdx.x;
    const int cols = d_V + 1;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int per_col = nblk * kDecWaves;
    const int j0 = blockIdx.y * kFinCols;
    const int nc = min(kFinCols, d_V - j0);
    __shared__ float num[kFinCols + 1];
    for (int c = wave; c <= nc; c += kThreads / 64) {
        const int j = c < nc ? j0 + c : d_V;
        const float* pc = partial + (bh * cols + j) * per_col;
        float s = 0.0f;
        for (int i = lane; i < per_col; i += 64) s += pc[i];
        s = wave_sum64(s);
        if (lane == 0) num[c < nc ? c : kFinCols] = s;
    }
    __syncthreads();
    if ((int)threadIdx.x < nc) y[bh * d_V + j0 + threadIdx.x] = num[threadIdx.x] / num[kFinCols];
}

template <typename In, int NIDX>
hipError_t launch_decode_n(const DecodeArgs& a, hipStream_t st) {
    const unsigned per_head = (unsigned)((a.d_V + kDecCols) / kDecCols * a.nblk);
    hipLaunchKernelGGL((decode_sweep_kernel<In, NIDX>), dim3(per_head, a.BH), dim3(kDecThreads), 0, st,
                       a.state, static_cast<const typename In::T*>(a.q),
                       static_cast<const typename In::T*>(a.k),
                       static_cast<const typename In::T*>(a.v), a.fidx, a.qw, a.partial, a.M,
                       a.M_pad, a.d_K, a.d_V, a.nblk, a.slots, a.pool, a.H);
    return hipGetLastError();
}

template <typename In>
hipError_t launch_decode_in(const DecodeArgs& a, hipStream_t st) {
    switch (a.P) {
        case 1: return launch_decode_n<In, 0>(a, st);
        case 2: return launch_decode_n<In, 1>(a, st);
        case 3: return launch_decode_n<In, 2>(a, st);
        case 4: return launch_decode_n<In, 3>(a, st);
        default: return launch_decode_n<In, 4>(a, st);
    }
}

}  // namespace

int decode_blocks(int64_t M_pad) { return (int)((M_pad + kDecFeatPerBlock - 1) / kDecFeatPerBlock); }

int64_t decode_partial_floats(int BH, int d_V, int64_t M_pad) {
    return (int64_t)BH * (d_V + 1) * decode_blocks(M_pad) * kDecWaves;
}

hipError_t launch_decode(const DecodeArgs& a, hipStream_t st) {
    return a.bf16 ? launch_decode_in<InBF16>(a, st) : launch_decode_in<InF32>(a, st);
}

hipError_t launch_decode_reduce(const DecodeArgs& a, hipStream_t st) {
    hipLaunchKernelGGL(decode_finalize_kernel, dim3(a.BH, (a.d_V + kFinCols - 1) / kFinCols),
                       dim3(kThreads), 0, st, a.partial, a.y, a.d_V, a.nblk);
    return hipGetLastError();
}

}  // namespace sata
