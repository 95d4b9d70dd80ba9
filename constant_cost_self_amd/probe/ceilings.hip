// ceilings.hip -- measured hardware ceilings for the benchmark (gfx950); not part of
// libsata.  Each probe does the simplest work with the same shape of traffic or of
// matrix instructions as a kernel of the path, so the path's figures can be quoted as a
// fraction of what the device reaches, not only of its data-sheet peaks.
//
//   probe_rmw   in-place read-modify-write of n floats, one linear sweep: each thread
//               loads one 16-byte vector (non-temporal), computes x = a x + b and stores
//               it back (non-temporal).  The decode step's traffic: every state byte read
//               and written once.
//   probe_mfma  back-to-back v_mfma_f32_16x16x32_f16 from 8 waves per workgroup (two per
//               SIMD, the prefill scan's occupancy), four independent accumulator chains
//               per wave; the accumulators are summed and stored so nothing is dead.
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

namespace {

__global__ __launch_bounds__(256) void rmw_kernel(float* __restrict__ x, int64_t n4, float a, float b) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= n4) return;
    f32x4* p = reinterpret_cast<f32x4*>(x) + i;
    f32x4 v = __builtin_nontemporal_load(p);
    v = v * a + b;
    __builtin_nontemporal_store(v, p);
}

__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
void mfma_kernel(float* __restrict__ out, int iters) {
    const int tid = threadIdx.x;
    f16x8 A, B;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        A[e] = (_Float16)(1.0f + 0.001f * ((tid + e) & 7));
        B[e] = (_Float16)(1.0f - 0.001f * ((tid * 3 + e) & 7));
    }
    f32x4 c0 = {0, 0, 0, 0}, c1 = c0, c2 = c0, c3 = c0;
    for (int i = 0; i < iters; ++i) {
        c0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(A, B, c0, 0, 0, 0);
        c1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(A, B, c1, 0, 0, 0);
        c2 = __builtin_amdgcn_mfma_f32_16x16x32_f16(A, B, c2, 0, 0, 0);
        c3 = __builtin_amdgcn_mfma_f32_16x16x32_f16(A, B, c3, 0, 0, 0);
    }
    const f32x4 s = (c0 + c1) + (c2 + c3);
    out[(int64_t)blockIdx.x * 512 + tid] = (s[0] + s[1]) + (s[2] + s[3]);
}

}  // namespace

extern "C" {

// In-place read-modify-write of x[0 .. n) (n a multiple of 4, x 16-byte aligned) on
// `stream`.  Returns 0 or a hipError_t.
int probe_rmw(float* x, int64_t n, float a, float b, void* stream) {
    if (!x || n <= 0 || (n & 3) || ((uintptr_t)x & 15)) return (int)hipErrorInvalidValue;
    const int64_t n4 = n / 4;
    hipLaunchKernelGGL(rmw_kernel, dim3((unsigned)((n4 + 255) / 256)), dim3(256), 0, (hipStream_t)stream, x, n4, a, b);
    return (int)hipGetLastError();
}

// `blocks` workgroups of 512 threads, each wave issuing 4 * iters MFMAs of 16x16x32
// (16384 flops each); out receives blocks * 512 floats.  Flops = blocks * 8 * 4 * iters * 16384.
int probe_mfma(float* out, int blocks, int iters, void* stream) {
    if (!out || blocks < 1 || iters < 1) return (int)hipErrorInvalidValue;
    hipLaunchKernelGGL(mfma_kernel, dim3((unsigned)blocks), dim3(512), 0, (hipStream_t)stream, out, iters);
    return (int)hipGetLastError();
}

}  // extern "C"
