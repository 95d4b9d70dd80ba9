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
// Kernel 1 (decode_sweep_kernel): workgroup (g, b) of head h updates 2048 features of
// four columns of the state, two 16-byte non-temporal loads and stores per thread and
// column, all loads issued before any arithmetic.  Consecutive workgroups take
// consecutive feature blocks of the same four columns, so the workgroups in flight
// stream four contiguous windows of HBM.  phi(k) and the weighted phi(q) of a thread's
// 8 features are computed once (packed index table, q and k staged in LDS per wave)
// and serve the four columns.  Measured on MI355X at d = 64, P = 4: one column per
// workgroup recomputes the features 65 times and reaches about 3.5-4.6 TB/s, one
// thread walking all 65 columns about 5.1 TB/s, four columns about 5.6 TB/s.  Each
// wave writes its partial readout of each column.
// Kernel 2 (decode_finalize_kernel): one workgroup per head sums the partials of
// every column and divides by the normaliser column.
// Pool form ([HW] "The fixed-size hidden state of SATA attention": the state's memory
// is allocated up front and requests share the device in turns): batch entry b uses
// the state in slot slots[b] of a preallocated pool instead of state b.
#include "launch.h"
#include "sata_common.h"

namespace sata {

namespace {

constexpr int kDecVec = 2;                               // 16-byte groups per thread
constexpr int kDecCols = 4;                              // state columns per workgroup
constexpr int kDecFeatPerBlock = kThreads * 4 * kDecVec; // 2048 features
constexpr int kDecWaves = kThreads / 64;
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// DPP lane exchange of a float (CTRL is the DPP control word)
template <int CTRL>
__device__ inline float dpp_f(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xf, 0xf, false));
}

// sum over the 64 lanes of a wave: DPP within rows of 16 lanes (quad swaps, then the
// half-row and row mirrors), then the four row sums read out to scalars
__device__ inline float wave_sum(float x) {
    x += dpp_f<0xB1>(x);      // quad_perm [1,0,3,2]
    x += dpp_f<0x4E>(x);      // quad_perm [2,3,0,1]
    x += dpp_f<0x141>(x);     // row_half_mirror
    x += dpp_f<0x140>(x);     // row_mirror
    const int b = __float_as_int(x);
    return (__int_as_float(__builtin_amdgcn_readlane(b, 0)) +
            __int_as_float(__builtin_amdgcn_readlane(b, 16))) +
           (__int_as_float(__builtin_amdgcn_readlane(b, 32)) +
            __int_as_float(__builtin_amdgcn_readlane(b, 48)));
}

// grid (ceil(cols / kDecCols) * nblk, BH): x = column group * nblk + feature block
template <typename In>
__global__ __launch_bounds__(kThreads) void decode_sweep_kernel(
    float* __restrict__ state, const typename In::T* __restrict__ q,
    const typename In::T* __restrict__ k, const typename In::T* __restrict__ v,
    const uint32_t* __restrict__ fidx, const float* __restrict__ qw,
    float* __restrict__ partial, int64_t M, int64_t M_pad, int d_K, int d_V, int P,
    int nblk, const int32_t* __restrict__ slots, int64_t pool, int H) {
    const int cols = d_V + 1;
    const int64_t bh = blockIdx.y;
    const int fb = (int)(blockIdx.x % nblk);
    const int j0 = (int)(blockIdx.x / nblk) * kDecCols;
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
                for (int c = 0; c < kDecCols && j0 + c < cols; ++c) pw[c * pstride] = __builtin_nanf("");
            return;
        }
        sh = s * H + bh % H;
    }

    // issue every state load first; the tables are M_pad long (padding rows have weight 0
    // and an all-sentinel index row)
    float* __restrict__ base = state + (sh * cols + j0) * M_pad;
    const int64_t f0 = (int64_t)fb * kDecFeatPerBlock + tid * 4;
    f32x4 s[kDecVec][kDecCols];
    u32x4 packed[kDecVec];
    f32x4 w[kDecVec];
#pragma unroll
    for (int g = 0; g < kDecVec; ++g) {
        const int64_t f = f0 + g * kThreads * 4;
        if (f < M_pad) {
#pragma unroll
            for (int c = 0; c < kDecCols; ++c)
                if (j0 + c < cols)
                    s[g][c] = __builtin_nontemporal_load(reinterpret_cast<f32x4*>(base + c * M_pad + f));
            packed[g] = *reinterpret_cast<const u32x4*>(fidx + f);
            w[g] = *reinterpret_cast<const f32x4*>(qw + f);
        }
    }

    // this wave's copy of the head's q and k coordinates and the constant 1 (index d_K)
    __shared__ float xs[kDecWaves][2][kMaxD + 1];
    float* xq = xs[wave][0];
    float* xk = xs[wave][1];
    for (int i = lane; i <= d_K; i += 64) {
        xq[i] = i < d_K ? In::load(q, bh * d_K + i) : 1.0f;
        xk[i] = i < d_K ? In::load(k, bh * d_K + i) : 1.0f;
    }
    float u[kDecCols];
#pragma unroll
    for (int c = 0; c < kDecCols; ++c) u[c] = j0 + c < d_V ? In::load(v, bh * d_V + j0 + c) : 1.0f;
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

    float acc[kDecCols];
#pragma unroll
    for (int c = 0; c < kDecCols; ++c) acc[c] = 0.0f;
    const int nidx = P - 1;
#pragma unroll
    for (int g = 0; g < kDecVec; ++g) {
        const int64_t f = f0 + g * kThreads * 4;
        if (f < M_pad) {
            // phi(k) masked to f < M keeps the padding of S at zero
            float pk[4], pq[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                pk[e] = f + e < M ? feature_value(xk, packed[g][e], nidx) : 0.0f;
                pq[e] = w[g][e] * feature_value(xq, packed[g][e], nidx);
            }
#pragma unroll
            for (int c = 0; c < kDecCols; ++c) {
                if (j0 + c < cols) {
                    f32x4 t = s[g][c];
                    t.x = fmaf(pk[0], u[c], t.x);
                    t.y = fmaf(pk[1], u[c], t.y);
                    t.z = fmaf(pk[2], u[c], t.z);
                    t.w = fmaf(pk[3], u[c], t.w);
                    __builtin_nontemporal_store(t, reinterpret_cast<f32x4*>(base + c * M_pad + f));
                    acc[c] = fmaf(pq[0], t.x, fmaf(pq[1], t.y, fmaf(pq[2], t.z, fmaf(pq[3], t.w, acc[c]))));
                }
            }
        }
    }
#pragma unroll
    for (int c = 0; c < kDecCols; ++c) {
        const float a = wave_sum(acc[c]);
        if (lane == 0 && j0 + c < cols) pw[c * pstride] = a;
    }
}

// one workgroup per head: wave w sums the partials of columns w, w + 4, ... (lanes
// over the feature blocks and waves of the column), then y = num / normaliser
__global__ __launch_bounds__(kThreads) void decode_finalize_kernel(
    const float* __restrict__ partial, float* __restrict__ y, int d_V, int nblk) {
    const int64_t bh = blockIdx.x;
    const int cols = d_V + 1;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int per_col = nblk * kDecWaves;
    __shared__ float num[kMaxD + 1];
    for (int j = wave; j < cols; j += kDecWaves) {
        const float* pc = partial + (bh * cols + j) * per_col;
        float s = 0.0f;
        for (int i = lane; i < per_col; i += 64) s += pc[i];
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) s += __shfl_xor(s, off, 64);
        if (lane == 0) num[j] = s;
    }
    __syncthreads();
    for (int j = threadIdx.x; j < d_V; j += kThreads) y[bh * d_V + j] = num[j] / num[d_V];
}

template <typename In>
hipError_t launch_decode_in(const DecodeArgs& a, hipStream_t st) {
    const unsigned per_head = (unsigned)((a.d_V + kDecCols) / kDecCols * a.nblk);
    hipLaunchKernelGGL((decode_sweep_kernel<In>), dim3(per_head, a.BH), dim3(kThreads), 0, st,
                       a.state, static_cast<const typename In::T*>(a.q),
                       static_cast<const typename In::T*>(a.k),
                       static_cast<const typename In::T*>(a.v), a.fidx, a.qw, a.partial, a.M,
                       a.M_pad, a.d_K, a.d_V, a.P, a.nblk, a.slots, a.pool, a.H);
    return hipGetLastError();
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
    hipLaunchKernelGGL(decode_finalize_kernel, dim3(a.BH), dim3(kThreads), 0, st, a.partial,
                       a.y, a.d_V, a.nblk);
    return hipGetLastError();
}

}  // namespace sata
