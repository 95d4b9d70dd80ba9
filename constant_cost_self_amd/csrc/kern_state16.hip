// kern_state16.hip -- the state kept in half precision (gfx950): the decode step over it and
// the conversions from and to the fp32 state.
//
// [TA] "Hidden-state size and compute analysis" sizes a head's state in Float16 (about 6.2 MB
// at d_K = d_V = 64, P = 4).  Here the d_V value columns are stored as fp16 and the
// normaliser column Z stays fp32: its degree-0 entry counts the tokens, and fp16 holds
// consecutive integers only up to 2048.  The bytes of a decode step fall from
// 8 (d_V + 1) M_pad to about 4 (d_V + 1) Mh per head.  Arithmetic is fp32; every write
// rounds a value entry to fp16 (to nearest even).  The layout of one head is in launch.h
// (State16Geom): degree block p of every column starts at row hoff[p], a multiple of 64, so
// each thread's 8 consecutive rows share one degree.
//
// Range.  The entries of one degree block of one column share a power-of-two exponent e,
// chosen so that the block's largest stored entry |S| 2^-e stays below 2^15 (fp16's largest
// finite value is 65504).  It comes from a bound on the block known before the entries are
// written:  a decode step adds phi_f(k) u_j to an entry, |phi_f(k)| <= kinf^p for a monomial
// of degree p (kinf = max_i |k_i|), and the old entries are at most bound (1 + 2^-11) after
// their own fp16 rounding, so
//     |S_new| <= bound (1 + 2^-10) + kinf^p |u_j|.
// The step also finds the new block maxima (each wave writes its own, the per-head kernel
// reduces them), which become the bounds of the next step: the exponent follows the entries
// up and down instead of growing with the context, and no finite input overflows.  For exponent e = floor(log2 b) - 14 the
// stored values are below 2^15 whenever the entries are at most b.
#include "launch.h"
#include "sata_common.h"

namespace sata {

namespace {

constexpr int kH16Feat = 8;                         // rows per thread (one 16-byte fp16 load)
constexpr int kH16Cols = 8;                         // value columns per workgroup
constexpr int kSweepThreads = 128;                  // block size of the sweep
constexpr int kH16Block = kSweepThreads * kH16Feat; // rows per sweep workgroup
constexpr int kH16Waves = kSweepThreads / 64;       // waves per sweep workgroup
constexpr int kFinWaves = kThreads / 64;            // waves of the other kernels' blocks
constexpr int kH16WaveRows = 64 * kH16Feat;         // rows of one wave: one slot of block maxima
static_assert(kH16Cols == 8, "the wave reductions take 8 values per lane");
constexpr float kGrow = 1.0009765625f;              // 1 + 2^-10
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f2 __attribute__((ext_vector_type(2)));
typedef _Float16 h2 __attribute__((ext_vector_type(2)));

// exponent of a block whose entries are at most b: floor(log2 b) - 14 from the float bits (0
// and subnormal b give -141, inf and NaN 114; the stored values stay below 2^15 in every case)
__device__ inline int s16_exp(float b) { return (int)((__float_as_uint(b) >> 23) & 0xffu) - 141; }

// bound on the entries of degree block p of a column after phi(k) u is added to them
__device__ inline float s16_bound(float bound, float kinf, int p, float ua) {
    float pw = 1.0f;
    for (int s = 0; s < p; ++s) pw *= kinf;
    return fmaf(bound, kGrow, pw * ua);
}

__device__ inline float h2f(uint32_t bits) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(bits & 0xffffu));
}
__device__ inline uint32_t f2h(float x) { return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)x); }

struct Head16 {
    int32_t* expo;
    float* bound;
    float* Z;
    uint16_t* V;
};

__device__ inline Head16 head16(uint8_t* base, const State16Geom& g) {
    const int pd = g.P * g.d_V;
    Head16 h;
    h.expo = reinterpret_cast<int32_t*>(base);
    h.bound = reinterpret_cast<float*>(base) + pd;
    h.Z = reinterpret_cast<float*>(base + g.z_off);
    h.V = reinterpret_cast<uint16_t*>(base + g.v_off);
    return h;
}

// Sum (or maximum) over the 64 lanes of a wave of each of 8 values per lane, which the lanes
// have written column-major to the wave's own 512 floats of LDS (lds[c * 64 + lane]): lane
// 8 c + i combines the values of column c held by lanes 8 i .. 8 i + 7, then the 8 lanes of
// each column combine by DPP (quad swaps and the half-row mirror).  Lane 8 c returns column
// c's result.
template <bool MAX>
__device__ inline float wave_reduce8(const float* lds, int lane) {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    const f32x4* src = reinterpret_cast<const f32x4*>(lds + (lane >> 3) * 64 + (lane & 7) * 8);
    const f32x4 a = src[0], b = src[1];
    float r;
    if (MAX) {
        r = fmaxf(fmaxf(fmaxf(a.x, a.y), fmaxf(a.z, a.w)), fmaxf(fmaxf(b.x, b.y), fmaxf(b.z, b.w)));
        r = fmaxf(r, dpp_row<0xB1>(r));
        r = fmaxf(r, dpp_row<0x4E>(r));
        r = fmaxf(r, dpp_row<0x141>(r));
    } else {
        r = ((a.x + a.y) + (a.z + a.w)) + ((b.x + b.y) + (b.z + b.w));
        r += dpp_row<0xB1>(r);
        r += dpp_row<0x4E>(r);
        r += dpp_row<0x141>(r);
    }
    // the LDS may be written again after this
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    return r;
}

// max_i |k_i| of head bh, in every lane of the calling wave
template <typename In>
__device__ inline float head_kinf(const typename In::T* k, int64_t bh, int d_K, int lane) {
    float a = 0.0f;
    for (int i = lane; i < d_K; i += 64) a = fmaxf(a, fabsf(In::load(k, bh * d_K + i)));
    return wave_max64(a);
}

// Decode step, kernel 1.  grid (ceil(d_V / 8) nblk, BH): x = column group * nblk + row
// block.  Group g takes the fp16 value columns 8 g .. 8 g + 7 (those below d_V), and group 0
// also the fp32 normaliser column.  A thread takes 8 consecutive rows of each of its columns
// (one 16-byte non-temporal load and store per fp16 column, two per fp32 one, all loads
// issued before any arithmetic) and computes their 8 features once for all of them:
//     S[f][j] = V[j][f] 2^e_in + phi_f(k) u_j      (u = [v | 1]),   V[j][f] = S[f][j] 2^-e_out
//     partial readout  sum_f alpha_p C_p[f] phi_f(q) S[f][j]  per wave,
// with the readout taken from the fp32 entries before their rounding.  Pool form as the fp32
// step: batch entry b uses slot slots[b]; an entry whose slot is outside the pool leaves the
// pool alone and reads out NaN.  Row blocks of 1024 leave little of a head's last block idle
// (48000 rows at d = 64: 47 blocks, the last 7/8 full).
template <typename In, int NIDX>
__global__ __launch_bounds__(kSweepThreads) void decode16_sweep_kernel(const Decode16Args a) {
    using T = typename In::T;
    const State16Geom& g = a.g;
    const int d_K = g.d_K, d_V = g.d_V, P = g.P, cols = d_V + 1, nblk = a.nblk;
    const int64_t bh = blockIdx.y;
    const int grp = (int)(blockIdx.x / nblk), fb = (int)(blockIdx.x % nblk);
    const bool withz = grp == 0;
    const int j0 = grp * kH16Cols;
    const int ncol = min(kH16Cols, d_V - j0);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const T* q = static_cast<const T*>(a.q);
    const T* k = static_cast<const T*>(a.k);
    const T* v = static_cast<const T*>(a.v);
    // partial readouts [BH][cols][nblk * kH16Waves], then the block maxima of each wave
    // [BH][P][d_V][nblk * kH16Waves]: slot fb * kH16Waves + wave covers kH16WaveRows rows
    const int64_t pstride = (int64_t)nblk * kH16Waves;
    const int slot = fb * kH16Waves + wave;
    float* __restrict__ pw = a.partial + (bh * cols + j0) * pstride + slot;
    float* __restrict__ pwz = a.partial + (bh * cols + d_V) * pstride + slot;
    float* __restrict__ pmax = a.partial + (int64_t)a.BH * cols * pstride + bh * P * d_V * pstride + slot;

    int64_t sh = bh;
    if (a.slots) {
        const int64_t s = a.slots[bh / a.H];
        if (s < 0 || s >= a.pool) {
            if (lane == 0) {
                for (int c = 0; c < ncol; ++c) pw[c * pstride] = __builtin_nanf("");
                if (withz) *pwz = __builtin_nanf("");
            }
            return;
        }
        sh = s * a.H + bh % a.H;
    }
    const Head16 hd = head16(a.state + sh * g.head_bytes, g);
    const int64_t Mh = g.Mh;
    const int64_t f0 = (int64_t)fb * kH16Block + tid * kH16Feat;
    const bool live = f0 < Mh;

    // degree block of this thread's rows, its first row and its row count
    int p = 0;
    int64_t hstart = 0, mcount = g.m[0];
#pragma unroll
    for (int s = 1; s < kMaxP; ++s) {
        if (s < P && f0 >= g.hoff[s]) {
            p = s;
            hstart = g.hoff[s];
            mcount = g.m[s];
        }
    }
    // The small inputs (q, k, v, this lane's header entries, the rows' feature indices and
    // query weights) are loaded before the state, so that the features are computed while the
    // state is still in flight (loads complete in order).  Every load is
    // unconditional, from a valid place (indices past the end clamped; rows past Mh and columns
    // past the group's last read the last ones), so that no wait comes before the state loads
    // are all issued; only live rows and columns are used and stored.  Each wave stages its own
    // q and k and takes its own exponents: the sweep has no workgroup barrier.
    const int ti0 = min(lane, d_K - 1), ti1 = min(lane + 64, d_K - 1);
    const float q0 = In::load(q, bh * d_K + ti0), q1 = In::load(q, bh * d_K + ti1);
    const float k0 = In::load(k, bh * d_K + ti0), k1 = In::load(k, bh * d_K + ti1);
    float u[kH16Cols];
    int h_e[kH16Cols];
    float h_b[kH16Cols];
#pragma unroll
    for (int c = 0; c < kH16Cols; ++c) {
        const int j = j0 + min(c, ncol - 1);
        u[c] = In::load(v, bh * d_V + j);
        h_e[c] = hd.expo[p * d_V + j];
        h_b[c] = hd.bound[p * d_V + j];
    }
    const int64_t fl = live ? f0 : Mh - kH16Feat;
    const u32x4 pk[2] = {*reinterpret_cast<const u32x4*>(a.fidx_h + fl),
                         *reinterpret_cast<const u32x4*>(a.fidx_h + fl + 4)};
    const f32x4 wq[2] = {*reinterpret_cast<const f32x4*>(a.qw_h + fl),
                         *reinterpret_cast<const f32x4*>(a.qw_h + fl + 4)};
    u32x4 hv[kH16Cols];
#pragma unroll
    for (int c = 0; c < kH16Cols; ++c) {
        const int cc = c < ncol ? c : ncol - 1;
        hv[c] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(hd.V + (int64_t)(j0 + cc) * Mh + fl));
    }
    f32x4 zv[2];
    if (withz) {
        zv[0] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(hd.Z + fl));
        zv[1] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(hd.Z + fl + 4));
    }
    const float kinf = wave_max64(fmaxf(fabsf(k0), fabsf(k1)));
    const int ek = kinf > 0.0f ? (int)((__float_as_uint(kinf) >> 23) & 0xffu) - 127 : 0;
    // this wave's copy of q and k 2^-ek, the constant 1 at index d_K
    __shared__ float xs[kH16Waves][2][kMaxD + 1];
    float* xq = xs[wave][0];
    float* xk = xs[wave][1];
    if (lane < d_K) { xq[lane] = q0; xk[lane] = ldexpf(k0, -ek); }
    if (lane + 64 < d_K) { xq[lane + 64] = q1; xk[lane + 64] = ldexpf(k1, -ek); }
    if (lane == 0) { xq[d_K] = 1.0f; xk[d_K] = 1.0f; }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

    // Features of the 8 rows: phi'_f = phi_f(k) 2^-kp (kp = p ek) from the scaled k; with
    // u_j 2^(kp - e_out) their product is the increment in units of 2^e_out, and neither factor
    // overflows (2^e_out is at least 2^-15 kinf^p |u_j|).
    const int kp = p * ek;
    float fk[kH16Feat], fq[kH16Feat];
#pragma unroll
    for (int e = 0; e < kH16Feat; ++e) {
        const uint32_t pkd = pk[e >> 2][e & 3];
        const bool valid = live && f0 + e - hstart < mcount;     // rows past m_p stay zero
        fk[e] = valid ? feature_value_n<NIDX>(xk, pkd) : 0.0f;
        fq[e] = live ? wq[e >> 2][e & 3] * feature_value_n<NIDX>(xq, pkd) : 0.0f;
    }

    // Value columns, in units of 2^e_out of their block: S' = V 2^(e_in - e_out) + phi' u',
    // stored as fp16 (one packed conversion per two rows); the readout and the block maximum
    // are taken in these units, scaled once per column and put in LDS for the wave reductions.
    __shared__ float s_acc[kH16Waves][8 * 64], s_mx[kH16Waves][8 * 64];
    float* lacc = s_acc[wave];
    float* lmx = s_mx[wave];
#pragma unroll
    for (int c = 0; c < kH16Cols; ++c) {
        float a = 0.0f, m = 0.0f;
        if (live && c < ncol) {
                const int ein = h_e[c], eout = s16_exp(s16_bound(h_b[c], kinf, p, fabsf(u[c])));
                const float uc = ldexpf(u[c], kp - eout);
                const u32x4 h = hv[c];
                float sv[kH16Feat];
                if (ein == eout) {
#pragma unroll
                    for (int e = 0; e < kH16Feat; ++e) sv[e] = fmaf(fk[e], uc, h2f(h[e >> 1] >> (16 * (e & 1))));
                } else {
                    const float r = ldexpf(1.0f, ein - eout);
#pragma unroll
                    for (int e = 0; e < kH16Feat; ++e) sv[e] = fmaf(fk[e], uc, h2f(h[e >> 1] >> (16 * (e & 1))) * r);
                }
#pragma unroll
                for (int e = 0; e < kH16Feat; ++e) {
                    a = fmaf(fq[e], sv[e], a);
                    m = fmaxf(m, fabsf(sv[e]));
                }
                a = ldexpf(a, eout);
                m = ldexpf(m, eout);
                u32x4 o;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const f2 two = {sv[2 * i], sv[2 * i + 1]};
                    o[i] = __builtin_bit_cast(uint32_t, __builtin_convertvector(two, h2));
                }
                __builtin_nontemporal_store(o, reinterpret_cast<u32x4*>(hd.V + (int64_t)(j0 + c) * Mh + f0));
        }
        lacc[c * 64 + lane] = a;
        lmx[c * 64 + lane] = m;
        __builtin_amdgcn_sched_barrier(0);        // one column at a time: few live registers
    }
    float accz = 0.0f;
    if (withz && live) {
        f32x4 z0 = zv[0], z1 = zv[1];
        z0.x += ldexpf(fk[0], kp); z0.y += ldexpf(fk[1], kp); z0.z += ldexpf(fk[2], kp); z0.w += ldexpf(fk[3], kp);
        z1.x += ldexpf(fk[4], kp); z1.y += ldexpf(fk[5], kp); z1.z += ldexpf(fk[6], kp); z1.w += ldexpf(fk[7], kp);
        __builtin_nontemporal_store(z0, reinterpret_cast<f32x4*>(hd.Z + f0));
        __builtin_nontemporal_store(z1, reinterpret_cast<f32x4*>(hd.Z + f0 + 4));
        accz = fmaf(fq[0], z0.x, fmaf(fq[1], z0.y, fmaf(fq[2], z0.z, fmaf(fq[3], z0.w,
               fmaf(fq[4], z1.x, fmaf(fq[5], z1.y, fmaf(fq[6], z1.z, fq[7] * z1.w)))))));
    }
    {
        const float t = wave_reduce8<false>(lacc, lane);
        if ((lane & 7) == 0 && (lane >> 3) < ncol) pw[(lane >> 3) * pstride] = t;
    }
    if (withz) {
        const float t = wave_sum64(accz);
        if (lane == 0) *pwz = t;
    }
    // this wave's largest |entry| of every degree block its rows meet (rows increase with the
    // lane, so lanes 0 and 63 hold the first and the last degree; lanes past Mh have the last
    // degree and no entries)
    const int plo = __builtin_amdgcn_readfirstlane(p), phi = __builtin_amdgcn_readlane(p, 63);
    if (plo == phi) {
        const float m = wave_reduce8<true>(lmx, lane);
        if ((lane & 7) == 0 && (lane >> 3) < ncol) pmax[((int64_t)plo * d_V + j0 + (lane >> 3)) * pstride] = m;
    } else {
        // rows of several degrees: each degree's maxima from this lane's entries of it alone
        // (the readout's LDS is free again)
        for (int pp = plo; pp <= phi; ++pp) {
#pragma unroll
            for (int c = 0; c < kH16Cols; ++c) lacc[c * 64 + lane] = p == pp ? lmx[c * 64 + lane] : 0.0f;
            const float m = wave_reduce8<true>(lacc, lane);
            if ((lane & 7) == 0 && (lane >> 3) < ncol) pmax[((int64_t)pp * d_V + j0 + (lane >> 3)) * pstride] = m;
        }
    }
}

// Decode step, kernel 2.  grid (BH, NY + NB): per head, NY = ceil(d_V / 16) workgroups
// write y for 16 value columns each (the sums of their partials over the normaliser's), and
// NB = ceil(P d_V / 64) workgroups move the header of 64 (degree, column) blocks each to the
// step just taken: the exponent the sweep wrote with (the same arithmetic on the same header
// entries and inputs), and as the new bound the block maximum, the largest of the waves'
// maxima over the slots (kH16WaveRows rows each) that meet the block.  A wave reduces one
// column or one block at a time, its lanes over the slots.
constexpr int kFinCols = 16;
constexpr int kFinBlocks = 64;

template <typename In>
__global__ __launch_bounds__(kThreads) void decode16_finalize_kernel(const Decode16Args a) {
    using T = typename In::T;
    const State16Geom& g = a.g;
    const int64_t bh = blockIdx.x;
    const int d_V = g.d_V, cols = d_V + 1;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int nslot = a.nblk * kH16Waves;
    const int ny = (d_V + kFinCols - 1) / kFinCols;
    const T* k = static_cast<const T*>(a.k);
    const T* v = static_cast<const T*>(a.v);
    if ((int)blockIdx.y < ny) {
        // y: the normaliser column and columns j0 .. j0 + 15
        __shared__ float num[kFinCols + 1];
        const int j0 = blockIdx.y * kFinCols;
        const int nc = min(kFinCols, d_V - j0);
        for (int c = wave; c <= nc; c += kFinWaves) {
            const int j = c < nc ? j0 + c : d_V;
            const float* pc = a.partial + (bh * cols + j) * nslot;
            float s = 0.0f;
            for (int i = lane; i < nslot; i += 64) s += pc[i];
            s = wave_sum64(s);
            if (lane == 0) num[c < nc ? c : kFinCols] = s;
        }
        __syncthreads();
        if ((int)threadIdx.x < nc) a.y[bh * d_V + j0 + threadIdx.x] = num[threadIdx.x] / num[kFinCols];
        return;
    }
    int64_t sh = bh;
    if (a.slots) {
        const int64_t s = a.slots[bh / a.H];
        if (s < 0 || s >= a.pool) return;
        sh = s * a.H + bh % a.H;
    }
    const Head16 hd = head16(a.state + sh * g.head_bytes, g);
    const float kinf = head_kinf<In>(k, bh, g.d_K, lane);
    const float* pmax = a.partial + (int64_t)a.BH * cols * nslot + bh * g.P * d_V * nslot;
    const int b0 = (blockIdx.y - ny) * kFinBlocks;
    const int b1 = min(b0 + kFinBlocks, g.P * d_V);
    for (int idx = b0 + wave; idx < b1; idx += kFinWaves) {
        const int p = idx / d_V;
        const int j = idx - p * d_V;
        int64_t r0 = g.hoff[0], r1 = g.Mh;
#pragma unroll
        for (int s = 0; s < kMaxP; ++s) {
            if (s == p) r0 = g.hoff[s];
            if (s == p + 1 && s < g.P) r1 = g.hoff[s];
        }
        const float* pb = pmax + (int64_t)idx * nslot;
        float m = 0.0f;
        for (int64_t i = r0 / kH16WaveRows + lane; i <= (r1 - 1) / kH16WaveRows; i += 64) m = fmaxf(m, pb[i]);
        m = wave_max64(m);
        if (lane == 0) {
            const float ua = fabsf(In::load(v, bh * d_V + j));
            hd.expo[idx] = s16_exp(s16_bound(hd.bound[idx], kinf, p, ua));
            hd.bound[idx] = m;
        }
    }
}

// fp32 state -> compact state.  grid (d_V + 1, count): workgroup (j, h) converts column j of
// head h.  A value column takes each degree block in turn: its largest |entry| (the block's
// bound), the exponent, then the fp16 entries (8 rows, one 16-byte store per thread).
__global__ __launch_bounds__(kThreads) void state16_pack_kernel(const float* __restrict__ src,
                                                                uint8_t* __restrict__ dst,
                                                                const State16Geom g) {
    const int j = blockIdx.x;
    const int64_t h = blockIdx.y;
    const int d_V = g.d_V, cols = d_V + 1;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const float* s = src + (h * cols + j) * g.M_pad;
    const Head16 hd = head16(dst + h * g.head_bytes, g);
    __shared__ float red[kFinWaves];
    for (int p = 0; p < g.P; ++p) {
        const int64_t off = g.off[p], hoff = g.hoff[p], m = g.m[p], mr = (m + 63) / 64 * 64;
        if (j == d_V) {
            for (int64_t r = tid; r < mr; r += kThreads) hd.Z[hoff + r] = r < m ? s[off + r] : 0.0f;
            continue;
        }
        float mx = 0.0f;
        for (int64_t r = tid; r < m; r += kThreads) mx = fmaxf(mx, fabsf(s[off + r]));
        mx = wave_max64(mx);
        if (lane == 0) red[wave] = mx;
        __syncthreads();
        mx = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
        __syncthreads();                               // red is written again for the next block
        const int e = -s16_exp(mx);
        uint16_t* vj = hd.V + (int64_t)j * g.Mh + hoff;
        for (int64_t r0 = (int64_t)tid * 8; r0 < mr; r0 += kThreads * 8) {
            u32x4 o;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int64_t r = r0 + 2 * i;
                const uint32_t lo = r < m ? f2h(ldexpf(s[off + r], e)) : 0u;
                const uint32_t hi = r + 1 < m ? f2h(ldexpf(s[off + r + 1], e)) : 0u;
                o[i] = lo | (hi << 16);
            }
            *reinterpret_cast<u32x4*>(vj + r0) = o;
        }
        if (tid == 0) {
            hd.expo[p * d_V + j] = -e;
            hd.bound[p * d_V + j] = mx;
        }
    }
}

// compact state -> fp32 state: grid (d_V + 1, count), workgroup (j, h) writes column j of
// head h, rows past M zero.
__global__ __launch_bounds__(kThreads) void state16_unpack_kernel(const uint8_t* __restrict__ src,
                                                                  float* __restrict__ dst,
                                                                  const State16Geom g) {
    const int j = blockIdx.x;
    const int64_t h = blockIdx.y;
    const int d_V = g.d_V, cols = d_V + 1, tid = threadIdx.x;
    float* d = dst + (h * cols + j) * g.M_pad;
    const Head16 hd = head16(const_cast<uint8_t*>(src) + h * g.head_bytes, g);
    for (int p = 0; p < g.P; ++p) {
        const int64_t off = g.off[p], hoff = g.hoff[p], m = g.m[p];
        if (j == d_V) {
            for (int64_t r = tid; r < m; r += kThreads) d[off + r] = hd.Z[hoff + r];
        } else {
            const int e = hd.expo[p * d_V + j];
            const uint16_t* vj = hd.V + (int64_t)j * g.Mh + hoff;
            for (int64_t r = tid; r < m; r += kThreads) d[off + r] = ldexpf(h2f(vj[r]), e);
        }
    }
    for (int64_t f = g.M + tid; f < g.M_pad; f += kThreads) d[f] = 0.0f;
}

template <int NIDX>
hipError_t launch_sweep16(const Decode16Args& a, dim3 grid, hipStream_t st) {
    if (a.bf16)
        hipLaunchKernelGGL((decode16_sweep_kernel<InBF16, NIDX>), grid, dim3(kSweepThreads), 0, st, a);
    else
        hipLaunchKernelGGL((decode16_sweep_kernel<InF32, NIDX>), grid, dim3(kSweepThreads), 0, st, a);
    return hipGetLastError();
}

}  // namespace

int decode16_blocks(int64_t Mh) { return (int)((Mh + kH16Block - 1) / kH16Block); }

int64_t decode16_partial_floats(int BH, int d_V, int P, int64_t Mh) {
    return (int64_t)BH * (d_V + 1 + (int64_t)P * d_V) * decode16_blocks(Mh) * kH16Waves;
}

hipError_t launch_decode16(const Decode16Args& a, hipStream_t st) {
    const int ngv = (a.g.d_V + kH16Cols - 1) / kH16Cols;
    const dim3 grid((unsigned)(ngv * a.nblk), (unsigned)a.BH);
    switch (a.g.P) {
        case 1: return launch_sweep16<0>(a, grid, st);
        case 2: return launch_sweep16<1>(a, grid, st);
        case 3: return launch_sweep16<2>(a, grid, st);
        case 4: return launch_sweep16<3>(a, grid, st);
        default: return launch_sweep16<4>(a, grid, st);
    }
}

hipError_t launch_decode16_reduce(const Decode16Args& a, hipStream_t st) {
    const int ny = (a.g.d_V + kFinCols - 1) / kFinCols;
    const int nb = (a.g.P * a.g.d_V + kFinBlocks - 1) / kFinBlocks;
    const dim3 grid((unsigned)a.BH, (unsigned)(ny + nb));
    if (a.bf16)
        hipLaunchKernelGGL(decode16_finalize_kernel<InBF16>, grid, dim3(kThreads), 0, st, a);
    else
        hipLaunchKernelGGL(decode16_finalize_kernel<InF32>, grid, dim3(kThreads), 0, st, a);
    return hipGetLastError();
}

hipError_t launch_state16_pack(const float* src, uint8_t* dst, const State16Geom& g, int count,
                               hipStream_t st) {
    hipLaunchKernelGGL(state16_pack_kernel, dim3(g.d_V + 1, count), dim3(kThreads), 0, st, src, dst, g);
    return hipGetLastError();
}

hipError_t launch_state16_unpack(const uint8_t* src, float* dst, const State16Geom& g, int count,
                                 hipStream_t st) {
    hipLaunchKernelGGL(state16_unpack_kernel, dim3(g.d_V + 1, count), dim3(kThreads), 0, st, src, dst, g);
    return hipGetLastError();
}

}  // namespace sata
