// kern_finalize.hip -- intra-chunk part, slice reduction and normalisation (gfx950).
//
// The scan reads the state out once per window of `win` chunks (the state before
// the window's first chunk).  The rows T of a chunk attend to the earlier tokens of
// their window directly, with the truncated kernel on the plain dot product ([TA]
// "Feature maps and linear attention": w(q,k) = sum_{p<P} alpha_p (q.k)^p), and to
// everything before the window through the state (the slice partials):
//     U[T][j] = sum_{t_w<=t<=T} w(q_T, k_t) u_t[j]  +  sum_slices part[slice][T][j]
//     y[T][j] = U[T][j] / U[T][d_V]               (u_t = [v_t | 1])
// with t_w the window's first token.  One block per (chunk, head).  The fp32 kernel
// below serves win = 1 (fp32 arithmetic, w by Horner's rule).
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
    const int64_t stride = (int64_t)L * cols;
    // four tokens T0 .. T0 + 3 of one column per thread (L is a multiple of 4): the slice
    // partials ([column][token]) with 16-byte loads, 8 slices in flight
    for (int q4 = tid; q4 < L * cols / 4; q4 += kThreads) {
        const int idx = 4 * q4, j = idx / L, T0 = idx % L;
        f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
        for (int s = 0; s <= T0 + 3; ++s) {
            const float u = us[s * cols + j];
#pragma unroll
            for (int e = 0; e < 4; ++e)
                if (s <= T0 + e) acc[e] = fmaf(W[(T0 + e) * (L + 1) + s], u, acc[e]);
        }
        const float* p = part + idx;
        f32x4 ps[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) ps[u] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
        int sl = 0;
        for (; sl + 8 <= a.nslices; sl += 8)
#pragma unroll
            for (int u = 0; u < 8; ++u) ps[u] += __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p + (sl + u) * stride));
        for (; sl < a.nslices; ++sl) ps[0] += __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p + sl * stride));
        const f32x4 sum = ((ps[0] + ps[1]) + (ps[2] + ps[3])) + ((ps[4] + ps[5]) + (ps[6] + ps[7]));
#pragma unroll
        for (int e = 0; e < 4; ++e) num[(T0 + e) * cols + j] = acc[e] + sum[e];
    }
    __syncthreads();
    float* y = a.y + (bh * a.n + t0) * d_V;
    for (int idx = tid; idx < nvalid * d_V; idx += kThreads) {
        const int t = idx / d_V, j = idx % d_V;
        y[idx] = num[t * cols + j] / num[t * cols + d_V];
    }
    if (a.den)
        for (int t = tid; t < nvalid; t += kThreads) a.den[bh * a.n + t0 + t] = num[t * cols + d_V];
}

// ---------------------------------------------------------------------------
// MFMA variant for bf16 inputs, L = 64, d_K in {64, 128}, d_V in {64, 128}.
// Same quantities, computed transposed so that no layout change is needed:
//     S^T[j][i] = k_j . q_i            v_mfma_f32_16x16x32_bf16 (exact products)
//     W^T[j][i] = w(S^T[j][i]) for live pairs, else 0           (fp32, Horner)
//     O^T[c][i] = sum_j U^T[c][j] W^T[j][i]     v_mfma_f32_16x16x32_f16, W^T in fp16
// summed over the key chunks of the window: a pair is live when i < nvalid and the key
// chunk precedes the query chunk, or is the query chunk and j <= i.
// The accumulator layout of two 16-key tiles of W^T is the B operand of the second
// contraction when the A operand (U^T, [column][token] in LDS) lists its keys in
// the same order: keys {4 g + r, 16 + 4 g + r} for lane group g.  Wave w owns
// query tile w (16 tokens) and keeps its direct part in registers while the slice
// partials are summed into the LDS the q, k, v tables held.  The slice partials ([column][token] per slice, or in
// the MFMA scan's tile order) are summed first by all threads with 16-byte loads
// (the memory-bound part).
// ---------------------------------------------------------------------------
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

template <int DK, int DV>
struct FinLayout {
    static constexpr int L = 64;
    static constexpr int XR = DK + 8;                  // q/k row (bf16)
    static constexpr int TS = L + 8;                   // U^T row (fp16)
    static constexpr int COLS = DV + 1;
    static constexpr int NS = COLS + 3;                // num row (floats)
    // q, k and [v | 1] for the direct part, then (same bytes) the sums of the partials
    static constexpr int qs = 0;
    static constexpr int ks = qs + L * XR * 2;
    static constexpr int vt = ks + L * XR * 2;
    static constexpr int tables = vt + ((COLS * TS * 2 + 15) / 16) * 16;
    static constexpr int num = 0;
    static constexpr int zs = num + L * NS * 4;        // normaliser partial sums [16 groups][L]
    static constexpr int sums_end = zs + 16 * L * 4;
    static constexpr int bytes = tables > sums_end ? tables : sums_end;
};

template <int DK, int DV, bool TILED>
__global__ __launch_bounds__(256) void finalize_mfma_kernel(PrefillSegArgs a) {
    using LY = FinLayout<DK, DV>;
    constexpr int L = LY::L, XR = LY::XR, TS = LY::TS, COLS = LY::COLS, NS = LY::NS;
    constexpr int NCT = (COLS + 15) / 16;              // column tiles of U (last one: the normaliser)
    extern __shared__ __align__(16) unsigned char fl[];
    uint16_t* qs = reinterpret_cast<uint16_t*>(fl + LY::qs);
    uint16_t* ks = reinterpret_cast<uint16_t*>(fl + LY::ks);
    _Float16* vt = reinterpret_cast<_Float16*>(fl + LY::vt);
    float* num = reinterpret_cast<float*>(fl + LY::num);

    const int cl = blockIdx.x;                  // chunk within the segment
    const int64_t bh = blockIdx.y;
    const int c = a.c_begin + cl;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int g = lane >> 4, li = lane & 15;
    const int nch = a.c_end - a.c_begin;
    const int64_t t0 = (int64_t)c * L;
    const int nvalid = (int)((a.n - t0) < L ? (a.n - t0) : L);

    const uint16_t* q = static_cast<const uint16_t*>(a.q) + (bh * a.n + t0) * DK;
    const uint16_t* k = static_cast<const uint16_t*>(a.k) + (bh * a.n + t0) * DK;
    const uint16_t* v = static_cast<const uint16_t*>(a.v) + (bh * a.n + t0) * DV;
    // the head's value scale (the matrix-core scan's v' = v 2^-s_v): the fp16 [v | 1] table
    // holds v', whatever the magnitude of v
    const int s_v = a.maxbits ? prep_scale_exp(a.maxbits[bh * 4 + 2]) : 0;
    const float vsc = ldexpf(1.0f, -s_v);

    for (int idx = tid; idx < L * DK / 8; idx += 256) {
        const int t = idx / (DK / 8), s8 = idx % (DK / 8);
        uint4 xq = uint4{0u, 0u, 0u, 0u};
        if (t < nvalid) xq = *reinterpret_cast<const uint4*>(q + t * DK + 8 * s8);
        *reinterpret_cast<uint4*>(qs + t * XR + 8 * s8) = xq;
    }
    // keys and [v | 1] of key chunk kc (zero past the sequence's end)
    auto load_kv = [&](int kc) {
        const int64_t dt = (int64_t)(kc - c) * L;
        const int nvk = (int)((a.n - (int64_t)kc * L) < L ? (a.n - (int64_t)kc * L) : L);
        for (int idx = tid; idx < L * DK / 8; idx += 256) {
            const int t = idx / (DK / 8), s8 = idx % (DK / 8);
            uint4 xk = uint4{0u, 0u, 0u, 0u};
            if (t < nvk) xk = *reinterpret_cast<const uint4*>(k + (dt + t) * DK + 8 * s8);
            *reinterpret_cast<uint4*>(ks + t * XR + 8 * s8) = xk;
        }
        for (int idx = tid; idx < L * DV / 8; idx += 256) {
            const int t = idx % L, c8 = idx / L;
            uint4 x = uint4{0u, 0u, 0u, 0u};
            if (t < nvk) x = *reinterpret_cast<const uint4*>(v + (dt + t) * DV + 8 * c8);
            const uint32_t xw[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                vt[(8 * c8 + 2 * e) * TS + t] = (_Float16)(__uint_as_float(xw[e] << 16) * vsc);
                vt[(8 * c8 + 2 * e + 1) * TS + t] = (_Float16)(__uint_as_float(xw[e] & 0xffff0000u) * vsc);
            }
        }
        if (tid < L) vt[DV * TS + tid] = (_Float16)(tid < nvk ? 1.0f : 0.0f);
    };
    const int cw = a.c_begin + (cl / a.win) * a.win;     // first chunk of this chunk's window
    load_kv(cw);

    __syncthreads();

    // wave w: query tile w, over the key chunks of the window (the last one causal).  The
    // weights enter the fp16 contraction as w 2^-e, with e a running power of two per query
    // (lane column li): a key chunk whose largest |w| needs a larger e rescales the fp32
    // accumulators first, so no weight of any magnitude overflows fp16.
    const int iq = 16 * w + li;                 // this lane's query token
    f32x4_t O[NCT];
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) O[ct] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
    int e_cur = -200;                           // no weight yet
    for (int kc = cw; kc <= c; ++kc) {
        if (kc > cw) {
            __syncthreads();                    // the previous key chunk is consumed
            load_kv(kc);
            __syncthreads();
        }
        // S^T tiles over the 4 key tiles, then the weights
        float wv[4][4];                         // keys 16 kt + 4 g + r of query iq
        float wmax = 0.0f;
#pragma unroll
        for (int kt = 0; kt < 4; ++kt) {
            f32x4_t st = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int kd = 0; kd < DK / 32; ++kd) {
                const bf16x8_t A = *reinterpret_cast<const bf16x8_t*>(ks + (16 * kt + li) * XR + 32 * kd + 8 * g);
                const bf16x8_t B = *reinterpret_cast<const bf16x8_t*>(qs + iq * XR + 32 * kd + 8 * g);
                st = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, B, st, 0, 0, 0);
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int j = 16 * kt + 4 * g + r;      // key token within chunk kc
                const float wgt = taylor_weight(st[r], a.alpha, a.P);
                // earlier chunks of the window are whole; chunk c is causal
                const bool live = iq < nvalid && (kc < c || j <= iq);
                wv[kt][r] = live ? wgt : 0.0f;
                wmax = fmaxf(wmax, fabsf(wv[kt][r]));
            }
        }
        // the query's largest |w| in this key chunk (its keys lie in lane groups g = 0..3)
        wmax = fmaxf(wmax, __shfl_xor(wmax, 16, 64));
        wmax = fmaxf(wmax, __shfl_xor(wmax, 32, 64));
        if (wmax > 0.0f) {
            int e = (int)((__float_as_uint(wmax) >> 23) & 0xffu) - 127 - 13;   // |w| 2^-e < 2^14
            e = e < -120 ? -120 : (e > 120 ? 120 : e);
            if (e > e_cur) {
                const float f = ldexpf(1.0f, e_cur - e);
#pragma unroll
                for (int ct = 0; ct < NCT; ++ct) O[ct] *= f;
                e_cur = e;
            }
        }
        f16x8_t Wb[2];                          // B operands: keys {32 ks + 4 g + r, 32 ks + 16 + 4 g + r}
        {
            const float f = e_cur > -200 ? ldexpf(1.0f, -e_cur) : 0.0f;   // all weights 0 so far
#pragma unroll
            for (int kt = 0; kt < 4; ++kt)
#pragma unroll
                for (int r = 0; r < 4; ++r) Wb[kt >> 1][4 * (kt & 1) + r] = (_Float16)(wv[kt][r] * f);
        }
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) {
            const int row = 16 * ct + li < COLS ? 16 * ct + li : DV;   // dead columns read the ones row
#pragma unroll
            for (int kq = 0; kq < 2; ++kq) {
                const f16x4_t lo = *reinterpret_cast<const f16x4_t*>(vt + row * TS + 32 * kq + 4 * g);
                const f16x4_t hi = *reinterpret_cast<const f16x4_t*>(vt + row * TS + 32 * kq + 16 + 4 * g);
                const f16x8_t A = f16x8_t{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
                O[ct] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A, Wb[kq], O[ct], 0, 0, 0);
            }
        }
    }
    // the tables are consumed: the partial sums reuse their LDS
    __syncthreads();

    // slice partials: num[t][col] = sum over slices.  Value columns: items of 16 bytes per
    // thread, all of them loaded together, several slices at a time (16 loads in flight).
    // The normaliser column (16 items) is split over 16 slice groups, one per thread, so
    // that no thread walks the slices alone at the end; the groups' sums are added in order.
    {
        const int64_t stride = TILED ? tiled_partial_floats(L, DV) : (int64_t)L * COLS;
        const float* part = a.partial + ((bh * nch + cl) * (int64_t)a.nslices) * stride;
        if constexpr (TILED) {
            // items of 8 fp16: [token tile][tile pair][lane (li, g)], tokens 16 tile + 4 g + r,
            // columns 32 pair + li (halves r) and 32 pair + 16 + li (halves 4 + r); each slice's
            // items of token tile tt and column group G carry the scale at [L d_V / 2 + L +
            // tt NG + G], and the sum is in units of 2^s_v (the head's value scale)
            constexpr int NVP = DV / 32, NG = DV / 64, NI = L * DV / 8 / 256, SB = 16 / NI;
            static_assert(NI * 256 * 8 == L * DV && SB * NI == 16, "whole items per thread");
            const float* p[NI];
            const float* ps[NI];
#pragma unroll
            for (int i = 0; i < NI; ++i) {
                const int item = tid + 256 * i, pr = (item / 64) % NVP, tt = item / 64 / NVP;
                p[i] = part + 4 * item;
                ps[i] = part + L * DV / 2 + L + tt * NG + pr / 2;
            }
            f32x4_t acc[NI][2];
#pragma unroll
            for (int i = 0; i < NI; ++i) acc[i][0] = acc[i][1] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
            auto add = [&](f32x4_t* ac, f32x4_t raw, float sc) {
                const f16x8_t h = __builtin_bit_cast(f16x8_t, raw);
                ac[0] += f32x4_t{(float)h[0], (float)h[1], (float)h[2], (float)h[3]} * sc;
                ac[1] += f32x4_t{(float)h[4], (float)h[5], (float)h[6], (float)h[7]} * sc;
            };
            int sl = 0;
            for (; sl + SB <= a.nslices; sl += SB) {
                f32x4_t x[SB][NI];
                float sc[SB][NI];
#pragma unroll
                for (int u = 0; u < SB; ++u)
#pragma unroll
                    for (int i = 0; i < NI; ++i) {
                        x[u][i] = __builtin_nontemporal_load(reinterpret_cast<const f32x4_t*>(p[i] + (sl + u) * stride));
                        sc[u][i] = ps[i][(sl + u) * stride];
                    }
#pragma unroll
                for (int u = 0; u < SB; ++u)
#pragma unroll
                    for (int i = 0; i < NI; ++i) add(acc[i], x[u][i], sc[u][i]);
            }
            for (; sl < a.nslices; ++sl)
#pragma unroll
                for (int i = 0; i < NI; ++i)
                    add(acc[i], __builtin_nontemporal_load(reinterpret_cast<const f32x4_t*>(p[i] + sl * stride)),
                        ps[i][sl * stride]);
            const float vs = ldexpf(1.0f, prep_scale_exp(a.maxbits[bh * 4 + 2]));
#pragma unroll
            for (int i = 0; i < NI; ++i) {
                const int item = tid + 256 * i, ln = item % 64, pr = (item / 64) % NVP, tt = item / 64 / NVP;
                const int col = 32 * pr + (ln & 15), t0 = 16 * tt + 4 * (ln >> 4);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    num[(t0 + e) * NS + col] = acc[i][0][e] * vs;
                    num[(t0 + e) * NS + col + 16] = acc[i][1][e] * vs;
                }
            }
        } else {
            // items of 4 tokens of one value column, [column][token]
            constexpr int NI = DV * (L / 4) / 256;
            static_assert(NI * 256 == DV * (L / 4), "whole items per thread");
            const float* p[NI];
#pragma unroll
            for (int i = 0; i < NI; ++i) {
                const int item = tid + 256 * i;
                p[i] = part + (item / (L / 4)) * L + 4 * (item % (L / 4));
            }
            f32x4_t acc[NI];
#pragma unroll
            for (int i = 0; i < NI; ++i) acc[i] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
            int sl = 0;
            for (; sl + 4 <= a.nslices; sl += 4) {
                f32x4_t x[4][NI];
#pragma unroll
                for (int u = 0; u < 4; ++u)
#pragma unroll
                    for (int i = 0; i < NI; ++i)
                        x[u][i] = __builtin_nontemporal_load(reinterpret_cast<const f32x4_t*>(p[i] + (sl + u) * stride));
#pragma unroll
                for (int i = 0; i < NI; ++i) acc[i] += (x[0][i] + x[1][i]) + (x[2][i] + x[3][i]);
            }
            for (; sl < a.nslices; ++sl)
#pragma unroll
                for (int i = 0; i < NI; ++i)
                    acc[i] += __builtin_nontemporal_load(reinterpret_cast<const f32x4_t*>(p[i] + sl * stride));
#pragma unroll
            for (int i = 0; i < NI; ++i) {
                const int item = tid + 256 * i, col = item / (L / 4), t0 = 4 * (item % (L / 4));
#pragma unroll
                for (int e = 0; e < 4; ++e) num[(t0 + e) * NS + col] = acc[i][e];
            }
        }
        // normaliser column: token quad tid % 16, slices tid / 16, tid / 16 + 16, ...; the 16
        // slice groups are then added in a fixed order (no atomics: y is reproducible)
        const int tg = tid % (L / 4), sg = tid / (L / 4);
        const float* pz = part + (TILED ? L * DV / 2 : L * DV) + 4 * tg;
        f32x4_t z = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
        for (int s2 = sg; s2 < a.nslices; s2 += 256 / (L / 4))
            z += __builtin_nontemporal_load(reinterpret_cast<const f32x4_t*>(pz + s2 * stride));
        float* zs = reinterpret_cast<float*>(fl + LY::zs);
        *reinterpret_cast<f32x4_t*>(zs + sg * L + 4 * tg) = z;
        __syncthreads();
        if (tid < L) {
            float acc = 0.0f;
#pragma unroll
            for (int i = 0; i < 256 / (L / 4); ++i) acc += zs[i * L + tid];
            num[tid * NS + DV] = acc;
        }
    }
    __syncthreads();
    {   // the direct part in true units: 2^e_cur, and 2^s_v for the value columns
        const float fz = ldexpf(1.0f, e_cur), fv = ldexpf(1.0f, e_cur + s_v);
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int col = 16 * ct + 4 * g + r;
                if (col < COLS) num[iq * NS + col] += O[ct][r] * (col < DV ? fv : fz);
            }
    }
    __syncthreads();
    float* y = a.y + (bh * a.n + t0) * DV;
    for (int idx = tid; idx < nvalid * DV; idx += 256) {
        const int t = idx / DV, j = idx % DV;
        y[idx] = num[t * NS + j] / num[t * NS + DV];
    }
}

template <int DK, int DV, bool TILED>
hipError_t launch_fin_mfma_t(const PrefillSegArgs& a, hipStream_t st) {
    constexpr int bytes = FinLayout<DK, DV>::bytes;
    hipError_t e = hipFuncSetAttribute((const void*)finalize_mfma_kernel<DK, DV, TILED>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((finalize_mfma_kernel<DK, DV, TILED>), dim3(a.c_end - a.c_begin, a.BH), dim3(256), bytes, st, a);
    return hipGetLastError();
}

template <int DK, int DV>
hipError_t launch_fin_mfma(const PrefillSegArgs& a, hipStream_t st) {
    return a.partial_tiled ? launch_fin_mfma_t<DK, DV, true>(a, st) : launch_fin_mfma_t<DK, DV, false>(a, st);
}

}  // namespace

int64_t finalize_lds_bytes(int d_K, int d_V, int L) { return finalize_lds_floats(d_K, d_V, L) * 4; }

hipError_t launch_finalize(const PrefillSegArgs& a, hipStream_t st) {
    if (a.bf16 && a.L == 64 && (a.d_K == 64 || a.d_K == 128) && (a.d_V == 64 || a.d_V == 128)) {
        if (a.d_K == 64) return a.d_V == 64 ? launch_fin_mfma<64, 64>(a, st) : launch_fin_mfma<64, 128>(a, st);
        return a.d_V == 64 ? launch_fin_mfma<128, 64>(a, st) : launch_fin_mfma<128, 128>(a, st);
    }
    return launch_finalize_fp32(a, st);
}

hipError_t launch_finalize_fp32(const PrefillSegArgs& a, hipStream_t st) {
    // windows and the tiled partial layout come only with the MFMA scan
    if (a.win != 1 || a.partial_tiled) return hipErrorInvalidValue;
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
