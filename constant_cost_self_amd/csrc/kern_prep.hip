// kern_prep.hip -- operand images of the matrix-core prefill scan (gfx950).
//
// The scan's contractions take fp16 operands built from q, k and v ([TA] "Feature maps and
// linear attention": the feature products of the query and key coordinates, and [v | 1]).
// Every feature slice of a head needs the same coordinates in the same layout, so they are
// converted once per prefill here instead of once per slice inside the scan:
//   prep_max_kernel     max |q|, |k|, |v| of every head (float bits, atomicMax): each input
//                       is scaled by the power of two 2^-s that brings its maximum into
//                       [1, 2), so feature products of any input magnitude stay inside
//                       fp16's range; the scan folds the scales back in exactly.
//   prep_images_kernel  per 128-token update sub-chunk of a head: the coordinate-major key
//                       table, the value tables of each group of 64 value columns (with the
//                       normaliser's row of ones in group 0) and the fp16 query rows of the
//                       readout window, in the byte layout the scan copies into LDS with
//                       direct-to-LDS loads (scan_mfma.h).
// Both are streaming passes over q, k, v (about 0.1% of the scan's time on the Long shape).
#include "scan_mfma.h"

namespace sata {

namespace {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

__device__ inline float bf16f(uint32_t b16) { return __uint_as_float(b16 << 16); }

// largest |x| of the 8 bf16 values of a 16-byte piece, as the bits of a non-negative float
// (which order like unsigned integers)
__device__ inline uint32_t absmax8(const uint4& r) {
    const uint32_t w[4] = {r.x, r.y, r.z, r.w};
    uint32_t m = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const uint32_t lo = (w[e] & 0x7fffu) << 16, hi = (w[e] >> 16 & 0x7fffu) << 16;
        m = m > lo ? m : lo;
        m = m > hi ? m : hi;
    }
    return m;
}

__device__ inline uint32_t wave_max_u32(uint32_t x) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
        const uint32_t y = (uint32_t)__shfl_xor((int)x, off, 64);
        x = x > y ? x : y;
    }
    return x;
}

__global__ __launch_bounds__(256) void prep_zero_kernel(uint32_t* __restrict__ p, int n) {
    const int i = blockIdx.x * 256 + threadIdx.x;
    if (i < n) p[i] = 0u;
}

// grid (blocks per head, BH): grid-stride over the head's 16-byte pieces of q, k and v
__global__ __launch_bounds__(256) void prep_max_kernel(const uint16_t* __restrict__ q,
                                                       const uint16_t* __restrict__ k,
                                                       const uint16_t* __restrict__ v, int64_t n,
                                                       int d_K, int d_V, uint32_t* __restrict__ maxbits) {
    const int64_t bh = blockIdx.y;
    const int64_t nqk = n * d_K / 8, nv = n * d_V / 8;
    const uint4* q4 = reinterpret_cast<const uint4*>(q + bh * n * d_K);
    const uint4* k4 = reinterpret_cast<const uint4*>(k + bh * n * d_K);
    const uint4* v4 = reinterpret_cast<const uint4*>(v + bh * n * d_V);
    const int64_t stride = (int64_t)gridDim.x * 256;
    uint32_t mq = 0, mk = 0, mv = 0;
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < nqk; i += stride) {
        const uint32_t a = absmax8(q4[i]), b = absmax8(k4[i]);
        mq = mq > a ? mq : a;
        mk = mk > b ? mk : b;
    }
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < nv; i += stride) {
        const uint32_t c = absmax8(v4[i]);
        mv = mv > c ? mv : c;
    }
    mq = wave_max_u32(mq);
    mk = wave_max_u32(mk);
    mv = wave_max_u32(mv);
    if ((threadIdx.x & 63) == 0) {
        atomicMax(&maxbits[bh * 4 + 0], mq);
        atomicMax(&maxbits[bh * 4 + 1], mk);
        atomicMax(&maxbits[bh * 4 + 2], mv);
    }
}

// grid (sub-chunks, BH): the images of 128-token update sub-chunk u_begin + blockIdx.x
template <int D, int DV>
__global__ __launch_bounds__(256) void prep_images_kernel(PrefillSegArgs a, int u_begin) {
    constexpr int LU = kImgLU, XR = img_xr(D), TS = img_ts(), R = img_window(D), NG = DV / 64;
    constexpr int PR = TS / 8;                         // 16-byte pieces per table row (17)
    constexpr int KS = D + 2, VS = DV + 2;             // LDS row strides (halves)
    __shared__ uint16_t ks[LU * KS];
    __shared__ uint16_t vs[LU * VS];
    const int u = u_begin + blockIdx.x;
    const int64_t bh = blockIdx.y;
    const int tid = threadIdx.x;
    const int64_t t0 = (int64_t)u * LU;
    const int nvalid = (int)(a.n - t0 < LU ? a.n - t0 : LU);
    const float fq = ldexpf(1.0f, -prep_scale_exp(a.maxbits[bh * 4 + 0]));
    const float fk = ldexpf(1.0f, -prep_scale_exp(a.maxbits[bh * 4 + 1]));
    const float fv = ldexpf(1.0f, -prep_scale_exp(a.maxbits[bh * 4 + 2]));
    const uint16_t* q = static_cast<const uint16_t*>(a.q) + (bh * a.n + t0) * D;
    const uint16_t* k = static_cast<const uint16_t*>(a.k) + (bh * a.n + t0) * D;
    const uint16_t* v = static_cast<const uint16_t*>(a.v) + (bh * a.n + t0) * DV;

    // the sub-chunk's key and value rows (bf16) in LDS; rows past the sequence are zero
    for (int pc = tid; pc < LU * (D / 8); pc += 256) {
        const int t = pc / (D / 8), c8 = pc % (D / 8);
        uint4 x = uint4{0u, 0u, 0u, 0u};
        if (t < nvalid) x = *reinterpret_cast<const uint4*>(k + (int64_t)t * D + 8 * c8);
        uint32_t* dst = reinterpret_cast<uint32_t*>(ks + t * KS + 8 * c8);
        dst[0] = x.x; dst[1] = x.y; dst[2] = x.z; dst[3] = x.w;
    }
    for (int pc = tid; pc < LU * (DV / 8); pc += 256) {
        const int t = pc / (DV / 8), c8 = pc % (DV / 8);
        uint4 x = uint4{0u, 0u, 0u, 0u};
        if (t < nvalid) x = *reinterpret_cast<const uint4*>(v + (int64_t)t * DV + 8 * c8);
        uint32_t* dst = reinterpret_cast<uint32_t*>(vs + t * VS + 8 * c8);
        dst[0] = x.x; dst[1] = x.y; dst[2] = x.z; dst[3] = x.w;
    }
    // the query rows of this sub-chunk, straight from global memory: coordinates q 2^-s_q,
    // then the constant slot (1, 0, ..., 0); rows past the sequence are zero
    {
        const int64_t win = t0 / R;
        const int r0 = (int)(t0 % R);
        uint16_t* qi = a.qimg + ((bh * a.img_nwin + (win - a.img_w0)) * R + r0) * XR;
        for (int pc = tid; pc < LU * (XR / 8); pc += 256) {
            const int t = pc / (XR / 8), c8 = pc % (XR / 8);
            f16x8 o = f16x8{0, 0, 0, 0, 0, 0, 0, 0};
            if (c8 == D / 8) {
                o[0] = (_Float16)1.0f;
            } else if (t < nvalid) {
                const uint4 x = *reinterpret_cast<const uint4*>(q + (int64_t)t * D + 8 * c8);
                const uint32_t w[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    o[2 * e] = (_Float16)(bf16f(w[e] & 0xffffu) * fq);
                    o[2 * e + 1] = (_Float16)(bf16f(w[e] >> 16) * fq);
                }
            }
            *reinterpret_cast<f16x8*>(qi + t * XR + 8 * c8) = o;
        }
    }
    __syncthreads();

    // key table [XR][TS]: coordinate rows over the sub-chunk's tokens, then the constant
    // coordinate (1 for the tokens that exist), zero rows and padding
    {
        uint16_t* kt = a.kimg + (bh * a.img_nsub + (u - a.img_u0)) * (int64_t)(img_kt_bytes(D) / 2);
        for (int pc = tid; pc < img_kt_bytes(D) / 16; pc += 256) {
            f16x8 o = f16x8{0, 0, 0, 0, 0, 0, 0, 0};
            const int c = pc / PR, p8 = pc % PR;
            if (c < XR && p8 < LU / 8) {
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const int t = 8 * p8 + e;
                    float x = 0.0f;
                    if (t < nvalid) x = c < D ? bf16f(ks[t * KS + c]) * fk : (c == D ? 1.0f : 0.0f);
                    o[e] = (_Float16)x;
                }
            }
            *reinterpret_cast<f16x8*>(kt + 8 * pc) = o;
        }
    }
    // value tables [rows][TS] per group of 64 value columns; group 0 ends with the ones row
#pragma unroll
    for (int G = 0; G < NG; ++G) {
        uint16_t* vt = a.vimg + ((bh * NG + G) * a.img_nsub + (u - a.img_u0)) * (int64_t)(img_vt_bytes() / 2);
        const int rows = G == 0 ? 65 : 64;
        for (int pc = tid; pc < img_vt_bytes() / 16; pc += 256) {
            f16x8 o = f16x8{0, 0, 0, 0, 0, 0, 0, 0};
            const int j = pc / PR, p8 = pc % PR;
            if (j < rows && p8 < LU / 8) {
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const int t = 8 * p8 + e;
                    float x = 0.0f;
                    if (t < nvalid) x = j < 64 ? bf16f(vs[t * VS + 64 * G + j]) * fv : 1.0f;
                    o[e] = (_Float16)x;
                }
            }
            *reinterpret_cast<f16x8*>(vt + 8 * pc) = o;
        }
    }
}

template <int D, int DV>
hipError_t launch_images_t(const PrefillSegArgs& a, int u_begin, int u_end, hipStream_t st) {
    hipLaunchKernelGGL((prep_images_kernel<D, DV>), dim3(u_end - u_begin, a.BH), dim3(256), 0, st, a, u_begin);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_prep_max(const PrefillSegArgs& a, uint32_t* maxbits, hipStream_t st) {
    const int nz = a.BH * 4;
    hipLaunchKernelGGL(prep_zero_kernel, dim3((nz + 255) / 256), dim3(256), 0, st, maxbits, nz);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t pieces = (int64_t)a.n * a.d_K / 8;
    int64_t blocks = (pieces + 256 * 8 - 1) / (256 * 8);                 // about 8 pieces per thread
    if (blocks > 64) blocks = 64;
    if (blocks < 1) blocks = 1;
    hipLaunchKernelGGL(prep_max_kernel, dim3((unsigned)blocks, a.BH), dim3(256), 0, st,
                       static_cast<const uint16_t*>(a.q), static_cast<const uint16_t*>(a.k),
                       static_cast<const uint16_t*>(a.v), (int64_t)a.n, a.d_K, a.d_V, maxbits);
    return hipGetLastError();
}

hipError_t launch_prep_images(const PrefillSegArgs& a, int u_begin, int u_end, hipStream_t st) {
    if (u_end <= u_begin) return hipSuccess;
    if (a.d_K == 64) return a.d_V == 64 ? launch_images_t<64, 64>(a, u_begin, u_end, st)
                                         : launch_images_t<64, 128>(a, u_begin, u_end, st);
    return a.d_V == 64 ? launch_images_t<128, 64>(a, u_begin, u_end, st)
                       : launch_images_t<128, 128>(a, u_begin, u_end, st);
}

}  // namespace sata
