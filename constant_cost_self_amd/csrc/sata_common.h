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
// so every feature is a product of exactly NIDX = P-1 gathered values.
template <int NIDX>
__device__ inline float feature_value_n(const float* x, uint32_t packed) {
    float prod = 1.0f;
#pragma unroll
    for (int s = 0; s < NIDX; ++s) prod *= x[(packed >> (8 * s)) & 0xffu];
    return prod;
}

// Truncated kernel w(x) = sum_{p<P} alpha_p x^p by Horner's rule.
__device__ inline float taylor_weight(float x, const Alpha& al, int P) {
    float w = al.a[P - 1];
    for (int p = P - 2; p >= 0; --p) w = fmaf(w, x, al.a[p]);
    return w;
}

// DPP lane exchange of a float within rows of 16 lanes (CTRL is the DPP control word)
template <int CTRL>
__device__ inline float dpp_row(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xf, 0xf, false));
}

// Sum and maximum over the 64 lanes of a wave, returned in every lane: DPP within rows of
// 16 lanes (quad swaps, then the half-row and row mirrors), then the four row results read
// out to scalars.
__device__ inline float wave_sum64(float x) {
    x += dpp_row<0xB1>(x);      // quad_perm [1,0,3,2]
    x += dpp_row<0x4E>(x);      // quad_perm [2,3,0,1]
    x += dpp_row<0x141>(x);     // row_half_mirror
    x += dpp_row<0x140>(x);     // row_mirror
    const int b = __float_as_int(x);
    return (__int_as_float(__builtin_amdgcn_readlane(b, 0)) +
            __int_as_float(__builtin_amdgcn_readlane(b, 16))) +
           (__int_as_float(__builtin_amdgcn_readlane(b, 32)) +
            __int_as_float(__builtin_amdgcn_readlane(b, 48)));
}
__device__ inline float wave_max64(float x) {
    x = fmaxf(x, dpp_row<0xB1>(x));
    x = fmaxf(x, dpp_row<0x4E>(x));
    x = fmaxf(x, dpp_row<0x141>(x));
    x = fmaxf(x, dpp_row<0x140>(x));
    const int b = __float_as_int(x);
    return fmaxf(fmaxf(__int_as_float(__builtin_amdgcn_readlane(b, 0)),
                       __int_as_float(__builtin_amdgcn_readlane(b, 16))),
                 fmaxf(__int_as_float(__builtin_amdgcn_readlane(b, 32)),
                       __int_as_float(__builtin_amdgcn_readlane(b, 48))));
}

__device__ inline int64_t ceil_div64(int64_t a, int64_t b) { return (a + b - 1) / b; }

constexpr int kScanThreads = 512;    // block size of the fp32 scan kernels (2 waves per SIMD)

// dst[t * ds + i] = src[(row0 + t) * d + i] as fp32 for t < L, i < d; rows t >= nvalid are
// zero.  16-byte loads when a row is a whole number of 16-byte pieces (the base is
// 16-byte aligned), else one element per load.  All NT threads of the block take part.
template <typename In, int NT>
__device__ inline void load_rows(const typename In::T* src, int64_t row0, int nvalid, int L, int d,
                                 float* dst, int ds) {
    using T = typename In::T;
    constexpr int VE = 16 / sizeof(T);
    if ((d * (int)sizeof(T)) % 16 == 0) {
        const int pr = d / VE;                                  // 16-byte pieces per row
        for (int idx = threadIdx.x; idx < L * pr; idx += NT) {
            const int t = idx / pr, c = idx % pr;
            float* o = dst + t * ds + c * VE;
            if (t < nvalid) {
                const uint4 x = *reinterpret_cast<const uint4*>(src + (row0 + t) * d + c * VE);
                const uint32_t w[4] = {x.x, x.y, x.z, x.w};
                if (sizeof(T) == 2) {
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        o[2 * e] = __uint_as_float(w[e] << 16);
                        o[2 * e + 1] = __uint_as_float(w[e] & 0xffff0000u);
                    }
                } else {
#pragma unroll
                    for (int e = 0; e < 4; ++e) o[e] = __uint_as_float(w[e]);
                }
            } else {
#pragma unroll
                for (int e = 0; e < VE; ++e) o[e] = 0.0f;
            }
        }
    } else {
        for (int idx = threadIdx.x; idx < L * d; idx += NT) {
            const int t = idx / d, i = idx % d;
            dst[t * ds + i] = t < nvalid ? In::load(src, (row0 + t) * d + i) : 0.0f;
        }
    }
}

// The rows of one chunk held in registers between their global load and their LDS write,
// so that the next chunk's loads are in flight while the current chunk is computed.  A
// thread holds up to MAXP 16-byte pieces (piece idx = tid + p NT of the L x pr pieces, row
// idx / pr); fits() says whether the rows are whole 16-byte pieces that MAXP pieces per
// thread cover, and the caller loads with load_rows otherwise.  Rows t >= nvalid are zero.
template <typename In, int NT, int MAXP>
struct RowStage {
    using T = typename In::T;
    static constexpr int VE = 16 / sizeof(T);
    uint4 r[MAXP];
    __device__ static bool fits(int L, int d) {
        return (d * (int)sizeof(T)) % 16 == 0 && L * (d / VE) <= MAXP * NT;
    }
    __device__ void issue(const T* src, int64_t row0, int nvalid, int L, int d) {
        const int pr = d / VE;
#pragma unroll
        for (int p = 0; p < MAXP; ++p) {
            const int idx = threadIdx.x + p * NT, t = idx / pr, c = idx % pr;
            r[p] = make_uint4(0u, 0u, 0u, 0u);
            if (idx < L * pr && t < nvalid) r[p] = *reinterpret_cast<const uint4*>(src + (row0 + t) * d + c * VE);
        }
    }
    // dst[t * ds + i] for the first dcols elements of each row
    __device__ void commit(float* dst, int ds, int L, int d, int dcols) const {
        const int pr = d / VE;
#pragma unroll
        for (int p = 0; p < MAXP; ++p) {
            const int idx = threadIdx.x + p * NT, t = idx / pr, c = idx % pr;
            if (idx >= L * pr) continue;
            float* o = dst + t * ds + c * VE;
            const uint32_t w[4] = {r[p].x, r[p].y, r[p].z, r[p].w};
            if (sizeof(T) == 2) {
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    if (c * VE + 2 * e < dcols) o[2 * e] = __uint_as_float(w[e] << 16);
                    if (c * VE + 2 * e + 1 < dcols) o[2 * e + 1] = __uint_as_float(w[e] & 0xffff0000u);
                }
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    if (c * VE + e < dcols) o[e] = __uint_as_float(w[e]);
            }
        }
    }
};

// C(m, n) = sum_{k < K} A(m, k) B(k, n) for m < Mo, n < No, with A(m, k) = A[m sam + k sak]
// and B(k, n) = B[k sbk + n sbn] in LDS, on the matrix cores (v_mfma_f32_16x16x4_f32: fp32
// operands and accumulation), by the NT threads of a block; out(m, n, c) receives each
// result.  A wave computes units of two 16 x 16 output tiles side by side (rows m0..,
// columns n0.. and n0 + 16..), which share the A operand: unit w, w + NT/64, ...
// In step j of a unit the 16 lanes of group g = lane / 16 take
// k = g KQ + j (KQ = ceil(K / 4)): lane i + 16 g holds A(m0 + i, k) and B(k, n0 + i), and
// register r of a tile's accumulator is C(m0 + 4 g + r, n0 + i).  With row strides of 1
// modulo 64 floats (65, 129, L + 1, SV + 1) the 64 lanes of a load hit 64 different LDS
// banks.  A last column past whole pairs of tiles (the normaliser of [v | 1], No = 32 q + 1)
// is a dot product per row on the vector ALUs instead of a unit of its own.  K >= 1.
template <int NT, typename Out>
__device__ inline void mfma_gemm(int Mo, int No, int K, const float* A, int sam, int sak, const float* B,
                                 int sbk, int sbn, Out out) {
    constexpr int NW = NT / 64;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int i = lane & 15, g = lane >> 4;
    const int rem = (No % 32 == 1 && No > 32) ? 1 : 0;
    const int Nm = No - rem;
    const int pairs_n = (Nm + 31) / 32, units = (Mo + 15) / 16 * pairs_n;
    const int KQ = (K + 3) / 4;
    for (int unit = w; unit < units; unit += NW) {
        const int m0 = unit / pairs_n * 16, n0 = unit % pairs_n * 32;
        const bool mv = m0 + i < Mo, nv0 = n0 + i < Nm, nv1 = n0 + 16 + i < Nm;
        // rows of A past Mo and columns of B past Nm are read from valid places and only
        // reach outputs that are dropped
        const float* Ap = A + (mv ? m0 + i : Mo - 1) * sam;
        const float* Bp0 = B + (nv0 ? n0 + i : Nm - 1) * sbn;
        const float* Bp1 = B + (nv1 ? n0 + 16 + i : Nm - 1) * sbn;
        const int kb = g * KQ;
        const int kl = K - kb < KQ ? K - kb : KQ;          // live steps of this lane group
        // steps live in every lane group, in whole groups of four: no clamps, one address
        // add per load
        const int jm = (K - 3 * KQ > 0 ? K - 3 * KQ : 0) & ~3;
        f32x4 acc0 = {0.0f, 0.0f, 0.0f, 0.0f}, acc1 = {0.0f, 0.0f, 0.0f, 0.0f};
        const float* pa = Ap + kb * sak;
        const float* pb0 = Bp0 + kb * sbk;
        const float* pb1 = Bp1 + kb * sbk;
        // two register sets take turns, so the next group's operands are loaded before this
        // group's MFMAs without copies between them
        auto ld4 = [&](float* ra, float* rb0, float* rb1) {
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                ra[u] = pa[u * sak];
                rb0[u] = pb0[u * sbk];
                rb1[u] = pb1[u * sbk];
            }
            pa += 4 * sak;
            pb0 += 4 * sbk;
            pb1 += 4 * sbk;
        };
        auto mma4 = [&](const float* ra, const float* rb0, const float* rb1) {
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                acc0 = __builtin_amdgcn_mfma_f32_16x16x4f32(ra[u], rb0[u], acc0, 0, 0, 0);
                acc1 = __builtin_amdgcn_mfma_f32_16x16x4f32(ra[u], rb1[u], acc1, 0, 0, 0);
            }
        };
        // (the loop body has no branches, so the compiler can wait for the older set alone)
        float xa[4], xb0[4], xb1[4], ya[4], yb0[4], yb1[4];
        if (jm > 0) {
            ld4(xa, xb0, xb1);                           // group 0
            int j = 0;
            for (; j + 12 <= jm; j += 8) {               // groups j + 4 and j + 8 exist
                ld4(ya, yb0, yb1);
                __builtin_amdgcn_sched_barrier(0);       // keep each group's loads ahead
                mma4(xa, xb0, xb1);
                __builtin_amdgcn_sched_barrier(0);
                ld4(xa, xb0, xb1);
                __builtin_amdgcn_sched_barrier(0);
                mma4(ya, yb0, yb1);
                __builtin_amdgcn_sched_barrier(0);
            }
            if (j + 8 <= jm) {                           // groups j and j + 4 remain
                ld4(ya, yb0, yb1);
                mma4(xa, xb0, xb1);
                mma4(ya, yb0, yb1);
            } else {                                     // group j remains
                mma4(xa, xb0, xb1);
            }
        }
        // the rest (at most 7 steps): loads from clamped, always valid positions, all issued
        // first; a dead step is zeroed on the A side alone
        if (jm < KQ) {
            float ta[8], tb0[8], tb1[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int j = jm + u;
                const int k = kb + j < K ? kb + j : K - 1;
                ta[u] = j < kl ? Ap[k * sak] : 0.0f;
                tb0[u] = Bp0[k * sbk];
                tb1[u] = Bp1[k * sbk];
            }
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                if (jm + u < KQ) {
                    acc0 = __builtin_amdgcn_mfma_f32_16x16x4f32(ta[u], tb0[u], acc0, 0, 0, 0);
                    acc1 = __builtin_amdgcn_mfma_f32_16x16x4f32(ta[u], tb1[u], acc1, 0, 0, 0);
                }
            }
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int m = m0 + 4 * g + r;
            if (m < Mo) {
                if (nv0) out(m, n0 + i, acc0[r]);
                if (nv1) out(m, n0 + 16 + i, acc1[r]);
            }
        }
    }
    if (rem) {
        // C(m, Nm) for every row: 8 lanes per row, each summing every 8th k, then the 8 partial
        // sums of a row added across its lanes
        const float* Bc = B + Nm * sbn;
        for (int base = 0; base < Mo * 8; base += NT) {
            const int idx = base + threadIdx.x, m = idx >> 3, sub = idx & 7;
            const int mm = m < Mo ? m : Mo - 1;
            float c = 0.0f;
            for (int k = sub; k < K; k += 8) c = fmaf(A[mm * sam + k * sak], Bc[k * sbk], c);
            c += __shfl_xor(c, 1, 64);
            c += __shfl_xor(c, 2, 64);
            c += __shfl_xor(c, 4, 64);
            if (sub == 0 && m < Mo) out(m, Nm, c);
        }
    }
}

}  // namespace sata
