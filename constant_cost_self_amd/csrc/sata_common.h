// sata_common.h -- device helpers shared by the SATA kernels (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sata {

constexpr int kMaxP = 5;          // P <= 5: up to 4 indices per feature, 8 bits each
constexpr int kMaxD = 128;        // d_K, d_V <= 128
constexpr int kThreads = 256;     // block size of the VALU kernels

// Native 4 x fp32 vector (16-byte global accesses, usable with the builtins).
typedef float f32x4 __attribute__((ext_vector_type(4)));

// Input element types.  bf16 is carried as its raw 16 bits.
struct InF32 {
    using T = float;
    __device__ static inline float load(const T* p, int64_t i) { return p[i]; }
};
struct InBF16 {
    using T = uint16_t;
    __device__ static inline float load(const T* p, int64_t i) {
        return __uint_as_float(static_cast<uint32_t>(p[i]) << 16);
    }
};

// alpha_p = 1 / (p! c^p), c = sqrt(d_K), rounded once to fp32 on the host.
struct Alpha {
    float a[kMaxP];
};

// A feature f of degree p is the product of p coordinates; its indices are
// packed one per byte (low byte first) in fidx[f].  Unused bytes hold the
// sentinel index d_K, which the kernels map to a stored coordinate equal to 1,
// so every feature is a product of exactly P-1 gathered values.
__device__ inline float feature_value(const float* x, uint32_t packed, int nidx) {
    float prod = 1.0f;
    for (int s = 0; s < nidx; ++s) prod *= x[(packed >> (8 * s)) & 0xffu];
    return prod;
}

// Truncated kernel w(x) = sum_{p<P} alpha_p x^p by Horner's rule.
__device__ inline float taylor_weight(float x, const Alpha& al, int P) {
    float w = al.a[P - 1];
    for (int p = P - 2; p >= 0; --p) w = fmaf(w, x, al.a[p]);
    return w;
}

__device__ inline int64_t ceil_div64(int64_t a, int64_t b) { return (a + b - 1) / b; }

}  // namespace sata
