// kern_backward.hip -- gradients of the chunked prefill (fp32, gfx950).
//
// For a loss with dL/dy = dy, the chain rule through y_T = N_T / D_T ([TA] "Feature maps
// and linear attention": N_T = sum_{t<=T} w(q_T.k_t) v_t, D_T = sum_{t<=T} w(q_T.k_t))
// gives, with u_T = [g_T | h_T], g_T = dy_T / D_T and h_T = -(dy_T . y_T) / D_T,
// c_Tt = g_T . v_t + h_T and w'(x) = sum_{p>=1} p alpha_p x^{p-1}:
//     dv_t = sum_{T>=t} w(q_T.k_t) g_T
//     dq_T = sum_{t<=T} c_Tt w'(q_T.k_t) k_t
//     dk_t = sum_{T>=t} c_Tt w'(q_T.k_t) q_T
// In the feature form ([TA] "Feature maps and linear attention": w(q,k) =
// sum_f qw_f phi_f(q) phi_f(k)) the parts across chunks are contractions with two
// fixed-size states:
//     S_T = sum_{t<=T} phi(k_t) [v_t | 1]^T     (the forward state)
//     R_t = sum_{T>=t} qw phi(q_T) u_T^T         (its mirror, accumulated backwards)
//     dq_T = sum_f (S[f] . u_T) d(qw_f phi_f)/dq (q_T)
//     dk_t = sum_f (R[f] . [v_t | 1]) d phi_f/dk (k_t),     dv_t = sum_f phi_f(k_t) R[f][0:d_V]
// and the pairs inside a chunk are taken directly.  A feature is a product of P-1
// gathered coordinates (index d_K stands for the constant 1), so its derivative along
// coordinate i collects, for every slot holding i, the product of the other slots.
//
// Kernels:
//   bwd_u_kernel      u_T from dy, y and D (one thread per token)
//   bwd_q_kernel      per (feature slice, head), chunks in order: a_T[f] = S[f] . u_T,
//                     dq partials by scattering a_T[f] qw_f dphi_f into LDS, then the
//                     update S += phi(k)^T [v | 1]
//   bwd_kv_kernel     per (feature slice, head), chunks in reverse: b_t[f] = R[f].[v|1],
//                     dk partials by scattering, dv partials by a readout of R, then
//                     R += (qw phi(q))^T u
//   bwd_fin_kernel    per (chunk, head): sum of the slice partials plus the direct part
//                     of the chunk's pairs
// The state contractions run on the matrix cores with fp32 operands (mfma_gemm); the
// scatter follows a per-slice plan (build_plan) instead of atomics.
#include "launch.h"
#include "sata_common.h"

namespace sata {

namespace {

constexpr int kScanWaves = kScanThreads / 64;
constexpr int kMaxSlots = 4;                       // P - 1 gathered slots per feature, P <= 5

// LDS floats of a feature table: [L][SV + 1] or [SV][L + 1] (row strides of 1 modulo 64
// floats for the matrix-core loads)
__host__ __device__ inline int64_t bwd_table_floats(int SV, int L) { return (int64_t)(L + 1) * (SV + 1); }

// LDS floats of the scan kernels: state slice, x_q, x_k, u, [v | 1], three feature tables,
// the gradient rows, the slice's index rows and weights, then the scatter plan (entries of
// two words, coordinate offsets, wave ranges) at an even offset
__host__ __device__ inline int64_t bwd_scan_lds_floats(int SV, int d_K, int d_V, int L) {
    const int cols = d_V + 1, ks = d_K + 1;
    int64_t base = (int64_t)SV * cols + 2LL * L * ks + 2LL * L * cols + 3 * bwd_table_floats(SV, L) +
                   (int64_t)L * ks + 2LL * SV;
    base += base & 1;
    return base + 2LL * kMaxSlots * SV + (d_K + 1) + (kScanWaves + 1) + kScanWaves;
}

// LDS floats of the finalize: x_q, x_k, [v | 1], u, and two L x (L + 1) pair tables
__host__ __device__ inline int64_t bwd_fin_lds_floats(int d_K, int d_V, int L) {
    const int cols = d_V + 1;
    return 2LL * L * d_K + 2LL * L * cols + 2LL * L * (L + 1);
}

// The chunk's q, k, v and u rows staged in registers (see RowStage).
template <typename In>
struct ChunkStage {
    RowStage<In, kScanThreads, 2> q, k, v;
    RowStage<InF32, kScanThreads, 3> u;
    __device__ static bool fits(const BwdArgs& a) {
        return RowStage<In, kScanThreads, 2>::fits(a.L, a.d_K) && RowStage<In, kScanThreads, 2>::fits(a.L, a.d_V) &&
               RowStage<InF32, kScanThreads, 3>::fits(a.L, a.ucols);
    }
    __device__ void issue(const BwdArgs& a, int64_t bh, int c) {
        using T = typename In::T;
        const int64_t t0 = (int64_t)c * a.L;
        const int nvalid = (int)((a.n - t0) < a.L ? (a.n - t0) : a.L);
        q.issue(static_cast<const T*>(a.q) + bh * a.n * a.d_K, t0, nvalid, a.L, a.d_K);
        k.issue(static_cast<const T*>(a.k) + bh * a.n * a.d_K, t0, nvalid, a.L, a.d_K);
        v.issue(static_cast<const T*>(a.v) + bh * a.n * a.d_V, t0, nvalid, a.L, a.d_V);
        u.issue(a.u + bh * a.n * a.ucols, t0, nvalid, a.L, a.ucols);
    }
    __device__ void commit(const BwdArgs& a, float* xq, float* xk, float* uu, float* vv) const {
        const int cols = a.d_V + 1, ks = a.d_K + 1;
        q.commit(xq, ks, a.L, a.d_K, a.d_K);
        k.commit(xk, ks, a.L, a.d_K, a.d_K);
        v.commit(vv, cols, a.L, a.d_V, a.d_V);
        u.commit(uu, cols, a.L, a.ucols, cols);
    }
};

// coordinate d_K is the constant 1; the last column of [v | 1] is 1 for the tokens
__device__ inline void chunk_constants(const BwdArgs& a, int nvalid, float* xq, float* xk, float* vv) {
    const int d_K = a.d_K, d_V = a.d_V, cols = d_V + 1, ks = d_K + 1;
    for (int t = threadIdx.x; t < a.L; t += kScanThreads) {
        xq[t * ks + d_K] = 1.0f;
        xk[t * ks + d_K] = 1.0f;
        vv[t * cols + d_V] = t < nvalid ? 1.0f : 0.0f;
    }
}

// The chunk's rows straight from global memory (when they do not fit a ChunkStage).
template <typename In>
__device__ inline void load_chunk(const BwdArgs& a, int64_t bh, int64_t t0, int nvalid, float* xq,
                                  float* xk, float* uu, float* vv) {
    using T = typename In::T;
    const int d_K = a.d_K, d_V = a.d_V, cols = d_V + 1, ks = d_K + 1, L = a.L, uc = a.ucols;
    load_rows<In, kScanThreads>(static_cast<const T*>(a.q) + bh * a.n * d_K, t0, nvalid, L, d_K, xq, ks);
    load_rows<In, kScanThreads>(static_cast<const T*>(a.k) + bh * a.n * d_K, t0, nvalid, L, d_K, xk, ks);
    load_rows<In, kScanThreads>(static_cast<const T*>(a.v) + bh * a.n * d_V, t0, nvalid, L, d_V, vv, cols);
    // u rows are padded to uc floats (a multiple of 4): 16-byte loads
    const float* u = a.u + (bh * a.n + t0) * uc;
    const int pr = uc / 4;
    for (int idx = threadIdx.x; idx < L * pr; idx += kScanThreads) {
        const int t = idx / pr, c = idx % pr;
        float4 x = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
        if (t < nvalid) x = *reinterpret_cast<const float4*>(u + (int64_t)t * uc + 4 * c);
        const float xv[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
        for (int e = 0; e < 4; ++e)
            if (4 * c + e < cols) uu[t * cols + 4 * c + e] = xv[e];
    }
}

// the slice's packed index rows and query weights, copied to LDS once per block (the
// tables are M_pad long: padding rows have weight 0 and an all-sentinel index row)
__device__ inline void stage_slice(const BwdArgs& a, int64_t F0, int SV, uint32_t* sfi, float* sqw) {
    for (int f = threadIdx.x; f < SV; f += kScanThreads) {
        const int64_t F = F0 + f;
        sfi[f] = F < a.M_pad ? a.fidx[F] : 0u;
        sqw[f] = F < a.M_pad ? a.qw[F] : 0.0f;
    }
}

// Scatter plan of a slice, built once per block.  When coordinate i fills m of the slots of
// feature f, d phi_f / d x_i = m x_i^(m-1) prod(other slots), so the slice's gradient along i
// sums one entry per feature holding i.  The entries are grouped by coordinate (the
// constant-1 slot has no gradient) and split into eight equal ranges, one per wave (one
// coordinate of a slice can hold every feature, so ranges of whole coordinates would leave
// waves idle).  A wave sums each run of one coordinate in its range, for every token, in one
// lane's register and writes it once.  The run that holds a coordinate's first entry is
// written into the gradient rows; a wave whose range starts inside a coordinate writes that
// first run to its own carry row instead, and the copy-out adds the carries: no two waves
// write one place, and no LDS atomics are needed.
// Entry: x = feature | coordinate << 16 | m << 24 | (first entry of its coordinate) << 30
//            | (last entry of its coordinate) << 31,
//        y = the other NIDX - 1 slots (one copy of the coordinate taken out), 8 bits each.
// carry_coord[w]: the coordinate of wave w's carry row, or -1.
template <int NIDX>
__device__ inline void build_plan(const BwdArgs& a, int64_t F0, int SV, const uint32_t* sfi, uint2* ent,
                                  int* off, int* wave_begin, int* carry_coord) {
    const int tid = threadIdx.x, d_K = a.d_K;
    const int nf = (int)((a.M - F0) < SV ? (a.M - F0) : SV);     // live features of the slice
    __syncthreads();                                              // sfi is written by other waves
    if (tid < d_K) {
        int cnt = 0;
        for (int f = 0; f < nf; ++f) {
            bool has = false;
#pragma unroll
            for (int sl = 0; sl < NIDX; ++sl) has |= ((sfi[f] >> (8 * sl)) & 0xffu) == (uint32_t)tid;
            cnt += has;
        }
        off[tid + 1] = cnt;
    }
    __syncthreads();
    if (tid == 0) {
        off[0] = 0;
        for (int i = 0; i < d_K; ++i) off[i + 1] += off[i];
        const int E = off[d_K];
        for (int w = 0; w <= kScanWaves; ++w) wave_begin[w] = E * w / kScanWaves;
    }
    __syncthreads();
    if (tid < d_K) {
        int pos = off[tid];
        const int end = off[tid + 1];
        for (int f = 0; f < nf; ++f) {
            uint32_t m = 0, others = 0;
            int no = 0;
#pragma unroll
            for (int sl = 0; sl < NIDX; ++sl) {
                const uint32_t c = (sfi[f] >> (8 * sl)) & 0xffu;
                if (c == (uint32_t)tid && m++ == 0) continue;
                others |= c << (8 * no++);
            }
            if (m) {
                const uint32_t first = pos == off[tid] ? 1u << 30 : 0u;
                const uint32_t last = pos + 1 == end ? 1u << 31 : 0u;
                ent[pos++] = make_uint2((uint32_t)f | (uint32_t)tid << 16 | m << 24 | first | last, others);
            }
        }
    }
    __syncthreads();
    if (tid < kScanWaves) {
        const int e = wave_begin[tid];
        carry_coord[tid] = (e < wave_begin[tid + 1] && !((ent[e].x >> 30) & 1u)) ? (int)((ent[e].x >> 16) & 0xffu) : -1;
    }
    __syncthreads();
}

// g[t][i] = sum over the plan entries (f, i) of this wave's range of coef[f cs + t] m prod(other
// slots of x_t), lanes over tokens; rows t >= nvalid are written 0.  A first run that continues
// the previous wave's coordinate goes to carry[w L + t] instead.
// The wave's entries come in batches of 64, one per lane, and are read out of the lanes by
// index (the range is uniform over the wave); then eight entries at a time, all their LDS
// reads issued before their sums.
template <int NIDX>
__device__ inline void scatter_planned(float* __restrict__ g, const float* __restrict__ x,
                                       const float* __restrict__ coef, const uint2* __restrict__ ent,
                                       const int* __restrict__ wave_begin, const int* __restrict__ carry_coord,
                                       float* __restrict__ carry, int L, int cs, int ks, int nvalid) {
    constexpr int U = 8;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int e0 = __builtin_amdgcn_readfirstlane(wave_begin[w]);
    const int e1 = __builtin_amdgcn_readfirstlane(wave_begin[w + 1]);
    for (int tb = 0; tb < L; tb += 64) {
        const int t = tb + lane;
        const int tt = t < L ? t : L - 1;
        const float* xr = x + tt * ks;
        const float* cr = coef + tt;
        float acc = 0.0f;
        bool owner = __builtin_amdgcn_readfirstlane(carry_coord[w]) < 0;
        for (int eb = e0; eb < e1; eb += 64) {
            const int ne = e1 - eb < 64 ? e1 - eb : 64;
            const uint2 mine = ent[eb + (lane < ne ? lane : ne - 1)];
            for (int j = 0; j < ne; j += U) {
                uint32_t ex[U], ey[U];
                float p[U];
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    const int jj = j + u < ne ? j + u : ne - 1;
                    ex[u] = __builtin_amdgcn_readlane(mine.x, jj);
                    ey[u] = __builtin_amdgcn_readlane(mine.y, jj);
                }
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    p[u] = cr[(int)(ex[u] & 0xffffu) * cs] * (float)((ex[u] >> 24) & 7u);
#pragma unroll
                    for (int sl = 0; sl < NIDX - 1; ++sl) p[u] *= xr[(ey[u] >> (8 * sl)) & 0xffu];
                }
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    if (j + u < ne) {
                        acc += p[u];
                        if ((ex[u] >> 31) || eb + j + u + 1 == e1) {     // end of a run
                            const float r = t < nvalid ? acc : 0.0f;
                            if (t < L) {
                                if (owner) g[t * ks + ((ex[u] >> 16) & 0xffu)] = r;
                                else carry[w * L + t] = r;
                            }
                            owner = true;
                            acc = 0.0f;
                        }
                    }
                }
            }
        }
    }
}

// part[t][i] = g[t][i] plus the carry rows of coordinate i (t < L, i < d_K), all threads.
// Columns without a carry are copied by the first loop (uniform compares, no extra loads);
// each carried column is written once by the second, from the first wave that carries it
// (the waves carrying one coordinate are consecutive).
__device__ inline void copy_grad_rows(float* part, const float* g, const float* carry, const int* carry_coord,
                                      int L, int d_K, int ks) {
    int cc[kScanWaves];
#pragma unroll
    for (int w = 0; w < kScanWaves; ++w) cc[w] = __builtin_amdgcn_readfirstlane(carry_coord[w]);
    for (int idx = threadIdx.x; idx < L * d_K; idx += kScanThreads) {
        const int t = idx / d_K, i = idx % d_K;
        bool carried = false;
#pragma unroll
        for (int w = 1; w < kScanWaves; ++w) carried |= cc[w] == i;
        if (!carried) part[idx] = g[t * ks + i];
    }
    for (int idx = threadIdx.x; idx < (kScanWaves - 1) * L; idx += kScanThreads) {
        const int w = 1 + idx / L, t = idx % L;
        const int c = carry_coord[w];
        if (c >= 0 && carry_coord[w - 1] != c) {
            float v = g[t * ks + c];
            for (int w2 = w; w2 < kScanWaves && carry_coord[w2] == c; ++w2) v += carry[w2 * L + t];
            part[t * d_K + c] = v;
        }
    }
}

template <typename In, int NIDX>
__global__ __launch_bounds__(kScanThreads) void bwd_q_kernel(BwdArgs a) {
    extern __shared__ float lds[];
    const int slice = blockIdx.x;
    const int64_t bh = blockIdx.y;
    const int tid = threadIdx.x;
    const int SV = a.slice_feats, L = a.L, d_K = a.d_K, d_V = a.d_V, cols = d_V + 1, ks = d_K + 1;
    const int64_t F0 = (int64_t)slice * SV;
    float* Ssl = lds;                              // [SV][cols]
    float* xq = Ssl + SV * cols;                   // [L][ks]
    float* xk = xq + L * ks;                       // [L][ks]
    float* uu = xk + L * ks;                       // [L][cols]
    float* vv = uu + L * cols;                     // [L][cols]
    const int LP = L + 1, SVP = SV + 1;
    float* hat = vv + L * cols;                    // [SV][LP] qw a_T; two more tables follow
    float* gq = hat + 3 * bwd_table_floats(SV, L); // [L][ks] (the layout of bwd_kv_kernel)
    uint32_t* sfi = reinterpret_cast<uint32_t*>(gq + L * ks);   // [SV] packed indices
    float* sqw = reinterpret_cast<float*>(sfi + SV);             // [SV] query weights, 0 past M
    uint2* ent = reinterpret_cast<uint2*>(lds + ((sqw + SV - lds + 1) & ~int64_t(1)));  // plan
    int* off = reinterpret_cast<int*>(ent + kMaxSlots * SV);
    int* wave_begin = off + d_K + 1;
    int* carry_coord = wave_begin + kScanWaves + 1;
    float* state = a.state + bh * (int64_t)cols * a.M_pad;
    stage_slice(a, F0, SV, sfi, sqw);
    build_plan<NIDX>(a, F0, SV, sfi, ent, off, wave_begin, carry_coord);

    for (int idx = tid; idx < SV * cols; idx += kScanThreads) {
        const int f = idx / cols, j = idx % cols;
        const int64_t F = F0 + f;
        Ssl[idx] = (a.load_state && F < a.M_pad) ? state[(int64_t)j * a.M_pad + F] : 0.0f;
    }
    const int nch = a.c_end - a.c_begin;
    ChunkStage<In> stage;
    const bool staged = ChunkStage<In>::fits(a);
    if (staged) stage.issue(a, bh, a.c_begin);
    for (int c = a.c_begin; c < a.c_end; ++c) {
        const int64_t t0 = (int64_t)c * L;
        const int nvalid = (int)((a.n - t0) < L ? (a.n - t0) : L);
        __syncthreads();
        if (staged) stage.commit(a, xq, xk, uu, vv);
        else load_chunk<In>(a, bh, t0, nvalid, xq, xk, uu, vv);
        chunk_constants(a, nvalid, xq, xk, vv);
        for (int idx = tid; idx < L * ks; idx += kScanThreads) gq[idx] = 0.0f;
        __syncthreads();
        if (staged && c + 1 < a.c_end) stage.issue(a, bh, c + 1);     // in flight during this chunk
        // qw_f a_T[f], a_T[f] = S[f] . u_T against the state before the chunk, stored [f][t]
        mfma_gemm<kScanThreads>(L, SV, cols, uu, cols, 1, Ssl, 1, cols,
                                [&](int t, int f, float c) { hat[f * LP + t] = c * sqw[f]; });
        __syncthreads();
        // dq partial: sum_f qw_f a_T[f] d phi_f / dq, and in the same phase the key features
        // (third table) for the update
        float* carry = hat + bwd_table_floats(SV, L);      // [waves][L] in the second table
        float* hk = hat + 2 * bwd_table_floats(SV, L);     // [L][SVP] phi(k)
        scatter_planned<NIDX>(gq, xq, hat, ent, wave_begin, carry_coord, carry, L, LP, ks, nvalid);
        {   // a thread owns feature tid % SV (a power of two) for tokens tid / SV + k NT / SV
            const int f = tid & (SV - 1);
            const bool live = F0 + f < a.M;
            const uint32_t fi = sfi[f];
            for (int t = tid / SV; t < L; t += kScanThreads / SV)
                hk[t * SVP + f] = live ? feature_value_n<NIDX>(xk + t * ks, fi) : 0.0f;
        }
        __syncthreads();
        float* part = a.part + (((bh * nch + (c - a.c_begin)) * a.nslices + slice) * (int64_t)L) * d_K;
        copy_grad_rows(part, gq, carry, carry_coord, L, d_K, ks);
        // the update S += phi(k)^T [v | 1]
        mfma_gemm<kScanThreads>(SV, cols, L, hk, 1, SVP, vv, cols, 1, [&](int f, int j, float c) { Ssl[f * cols + j] += c; });
    }
    __syncthreads();
    if (a.store_state) {
        for (int idx = tid; idx < SV * cols; idx += kScanThreads) {
            const int j = idx / SV, f = idx % SV;
            const int64_t F = F0 + f;
            if (F < a.M_pad) state[(int64_t)j * a.M_pad + F] = Ssl[f * cols + j];
        }
    }
}

template <typename In, int NIDX>
__global__ __launch_bounds__(kScanThreads) void bwd_kv_kernel(BwdArgs a) {
    extern __shared__ float lds[];
    const int slice = blockIdx.x;
    const int64_t bh = blockIdx.y;
    const int tid = threadIdx.x;
    const int SV = a.slice_feats, L = a.L, d_K = a.d_K, d_V = a.d_V, cols = d_V + 1, ks = d_K + 1;
    const int64_t F0 = (int64_t)slice * SV;
    float* Rsl = lds;                              // [SV][cols]
    float* xq = Rsl + SV * cols;                   // [L][ks]
    float* xk = xq + L * ks;                       // [L][ks]
    float* uu = xk + L * ks;                       // [L][cols]
    float* vv = uu + L * cols;                     // [L][cols]
    const int LP = L + 1, SVP = SV + 1;
    const int64_t TAB = bwd_table_floats(SV, L);
    float* hk = vv + L * cols;                     // [L][SVP] phi(k)
    float* hq = hk + TAB;                          // [L][SVP] qw phi(q)
    float* bb = hq + TAB;                          // [SV][LP] R[f] . [v_t | 1]
    float* gk = bb + TAB;                          // [L][ks]
    uint32_t* sfi = reinterpret_cast<uint32_t*>(gk + L * ks);   // [SV] packed indices
    float* sqw = reinterpret_cast<float*>(sfi + SV);             // [SV] query weights, 0 past M
    uint2* ent = reinterpret_cast<uint2*>(lds + ((sqw + SV - lds + 1) & ~int64_t(1)));  // plan
    int* off = reinterpret_cast<int*>(ent + kMaxSlots * SV);
    int* wave_begin = off + d_K + 1;
    int* carry_coord = wave_begin + kScanWaves + 1;
    float* state = a.state + bh * (int64_t)cols * a.M_pad;
    stage_slice(a, F0, SV, sfi, sqw);
    build_plan<NIDX>(a, F0, SV, sfi, ent, off, wave_begin, carry_coord);

    for (int idx = tid; idx < SV * cols; idx += kScanThreads) {
        const int f = idx / cols, j = idx % cols;
        const int64_t F = F0 + f;
        Rsl[idx] = (a.load_state && F < a.M_pad) ? state[(int64_t)j * a.M_pad + F] : 0.0f;
    }
    const int nch = a.c_end - a.c_begin;
    ChunkStage<In> stage;
    const bool staged = ChunkStage<In>::fits(a);
    if (staged) stage.issue(a, bh, a.c_end - 1);
    for (int c = a.c_end - 1; c >= a.c_begin; --c) {
        const int64_t t0 = (int64_t)c * L;
        const int nvalid = (int)((a.n - t0) < L ? (a.n - t0) : L);
        __syncthreads();
        if (staged) stage.commit(a, xq, xk, uu, vv);
        else load_chunk<In>(a, bh, t0, nvalid, xq, xk, uu, vv);
        chunk_constants(a, nvalid, xq, xk, vv);
        for (int idx = tid; idx < L * ks; idx += kScanThreads) gk[idx] = 0.0f;
        __syncthreads();
        if (staged && c > a.c_begin) stage.issue(a, bh, c - 1);      // in flight during this chunk
        {   // a thread owns feature tid % SV (a power of two) for tokens tid / SV + k NT / SV
            const int f = tid & (SV - 1);
            const bool fl = F0 + f < a.M;
            const uint32_t fi = sfi[f];
            const float w = sqw[f];
            for (int t = tid / SV; t < L; t += kScanThreads / SV) {
                const bool live = fl && t < nvalid;
                hk[t * SVP + f] = live ? feature_value_n<NIDX>(xk + t * ks, fi) : 0.0f;
                hq[t * SVP + f] = live ? w * feature_value_n<NIDX>(xq + t * ks, fi) : 0.0f;
            }
        }
        __syncthreads();
        const int64_t pbase = ((bh * nch + (c - a.c_begin)) * a.nslices + slice) * (int64_t)L;
        // b_t[f] = R[f] . [v_t | 1] and the dv partial sum_f phi_f(k_t) R[f][j], against
        // the chunks after c
        mfma_gemm<kScanThreads>(L, SV, cols, vv, cols, 1, Rsl, 1, cols, [&](int t, int f, float c) { bb[f * LP + t] = c; });
        float* pv = a.part2 + pbase * d_V;
        mfma_gemm<kScanThreads>(L, d_V, SV, hk, SVP, 1, Rsl, cols, 1, [&](int t, int j, float c) { pv[t * d_V + j] = c; });
        __syncthreads();
        // dk partial: sum_f b_t[f] d phi_f / dk
        // the carry rows take the key-feature table, which the dv partial has finished with
        scatter_planned<NIDX>(gk, xk, bb, ent, wave_begin, carry_coord, hk, L, LP, ks, nvalid);
        __syncthreads();
        float* pk = a.part + pbase * d_K;
        copy_grad_rows(pk, gk, hk, carry_coord, L, d_K, ks);
        // R += (qw phi(q))^T u with the chunk's queries
        mfma_gemm<kScanThreads>(SV, cols, L, hq, 1, SVP, uu, cols, 1, [&](int f, int j, float c) { Rsl[f * cols + j] += c; });
    }
    __syncthreads();
    if (a.store_state) {
        for (int idx = tid; idx < SV * cols; idx += kScanThreads) {
            const int j = idx / SV, f = idx % SV;
            const int64_t F = F0 + f;
            if (F < a.M_pad) state[(int64_t)j * a.M_pad + F] = Rsl[f * cols + j];
        }
    }
}

// u_T = [dy_T / D_T | -(dy_T . y_T) / D_T], one thread per token
__global__ __launch_bounds__(kThreads) void bwd_u_kernel(BwdArgs a) {
    const int64_t tok = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    if (tok >= (int64_t)a.BH * a.n) return;
    const int d_V = a.d_V;
    const float inv = 1.0f / a.den[tok];
    const float* dy = a.dy + tok * d_V;
    const float* y = a.y + tok * d_V;
    float* u = a.u_out + tok * a.ucols;
    float h = 0.0f;
    for (int j = 0; j < d_V; ++j) {
        u[j] = dy[j] * inv;
        h = fmaf(dy[j], y[j], h);
    }
    u[d_V] = -h * inv;
}

// sum over the slices of one partial entry: 8 independent loads in flight per thread
__device__ inline float slice_sum(const float* p, int64_t stride, int nslices) {
    float s[8] = {0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f};
    int sl = 0;
    for (; sl + 8 <= nslices; sl += 8)
#pragma unroll
        for (int u = 0; u < 8; ++u) s[u] += __builtin_nontemporal_load(p + (sl + u) * stride);
    for (; sl < nslices; ++sl) s[0] += __builtin_nontemporal_load(p + sl * stride);
    return ((s[0] + s[1]) + (s[2] + s[3])) + ((s[4] + s[5]) + (s[6] + s[7]));
}

// sum over the slices of four consecutive partial entries (16-byte aligned): 8 independent
// 16-byte loads in flight per thread
__device__ inline f32x4 slice_sum4(const float* p, int64_t stride, int nslices) {
    f32x4 s[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) s[u] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    int sl = 0;
    for (; sl + 8 <= nslices; sl += 8)
#pragma unroll
        for (int u = 0; u < 8; ++u) s[u] += __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p + (sl + u) * stride));
    for (; sl < nslices; ++sl) s[0] += __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p + sl * stride));
    return ((s[0] + s[1]) + (s[2] + s[3])) + ((s[4] + s[5]) + (s[6] + s[7]));
}

// out[r][c] (r < nvalid, c < d; row stride d) = the chunk's pair sum plus the slice partials,
// four consecutive columns per thread with 16-byte loads and stores when d is a multiple of 4,
// else one column.  pair(r, c) returns the pair sum of one entry.
template <typename Pair>
__device__ inline void fin_rows(float* out, const float* part, int64_t pstride, int nslices, int nvalid, int d,
                                Pair pair) {
    if (d % 4 == 0) {
        for (int q4 = threadIdx.x; q4 < nvalid * d / 4; q4 += kThreads) {
            const int idx = 4 * q4, r = idx / d, c = idx % d;
            f32x4 v = slice_sum4(part + idx, pstride, nslices);
#pragma unroll
            for (int e = 0; e < 4; ++e) v[e] += pair(r, c + e);
            *reinterpret_cast<f32x4*>(out + idx) = v;
        }
    } else {
        for (int idx = threadIdx.x; idx < nvalid * d; idx += kThreads)
            out[idx] = pair(idx / d, idx % d) + slice_sum(part + idx, pstride, nslices);
    }
}

// MODE 0: dq; MODE 1: dk and dv.  Sum of the slice partials plus the chunk's pairs.
template <typename In, int MODE>
__global__ __launch_bounds__(kThreads) void bwd_fin_kernel(BwdArgs a) {
    using T = typename In::T;
    extern __shared__ float lds[];
    const int cl = blockIdx.x;
    const int64_t bh = blockIdx.y;
    const int c = a.c_begin + cl;
    const int tid = threadIdx.x;
    const int L = a.L, d_K = a.d_K, d_V = a.d_V, cols = d_V + 1;
    const int nch = a.c_end - a.c_begin;
    const int64_t t0 = (int64_t)c * L;
    const int nvalid = (int)((a.n - t0) < L ? (a.n - t0) : L);
    float* xq = lds;                     // [L][d_K]
    float* xk = xq + L * d_K;            // [L][d_K]
    float* vv = xk + L * d_K;            // [L][cols]: v (the last column unused)
    float* uu = vv + L * cols;           // [L][cols]
    float* cw = uu + L * cols;           // [L][L + 1]: c_Tt w'(x_Tt), live pairs
    float* ww = cw + L * (L + 1);        // [L][L + 1]: w(x_Tt), live pairs
    const T* q = static_cast<const T*>(a.q) + (bh * a.n + t0) * d_K;
    const T* k = static_cast<const T*>(a.k) + (bh * a.n + t0) * d_K;
    const T* v = static_cast<const T*>(a.v) + (bh * a.n + t0) * d_V;
    const float* u = a.u + (bh * a.n + t0) * a.ucols;
    for (int idx = tid; idx < L * d_K; idx += kThreads) {
        const int t = idx / d_K;
        xq[idx] = t < nvalid ? In::load(q, idx) : 0.0f;
        xk[idx] = t < nvalid ? In::load(k, idx) : 0.0f;
    }
    for (int idx = tid; idx < L * cols; idx += kThreads) {
        const int t = idx / cols, j = idx % cols;
        vv[idx] = (t < nvalid && j < d_V) ? In::load(v, (int64_t)t * d_V + j) : 0.0f;
        uu[idx] = t < nvalid ? u[(int64_t)t * a.ucols + j] : 0.0f;
    }
    __syncthreads();
    for (int idx = tid; idx < L * L; idx += kThreads) {
        const int Tq = idx / L, t = idx % L;
        float cv = 0.0f, wv = 0.0f;
        if (t <= Tq && Tq < nvalid) {
            float x = 0.0f;
            for (int i = 0; i < d_K; ++i) x = fmaf(xq[Tq * d_K + i], xk[t * d_K + i], x);
            // w and w' by Horner's rule
            float w = a.alpha.a[a.P - 1], wp = 0.0f;
            for (int p = a.P - 2; p >= 0; --p) {
                wp = fmaf(wp, x, w);
                w = fmaf(w, x, a.alpha.a[p]);
            }
            float cc = uu[Tq * cols + d_V];
            for (int j = 0; j < d_V; ++j) cc = fmaf(uu[Tq * cols + j], vv[t * cols + j], cc);
            cv = cc * wp;
            wv = w;
        }
        cw[Tq * (L + 1) + t] = cv;
        ww[Tq * (L + 1) + t] = wv;
    }
    __syncthreads();
    const int64_t slice_stride = (int64_t)L;
    if (MODE == 0) {
        const float* part = a.part + ((bh * nch + cl) * (int64_t)a.nslices) * L * d_K;
        float* dq = a.dq + (bh * a.n + t0) * d_K;
        fin_rows(dq, part, slice_stride * d_K, a.nslices, nvalid, d_K, [&](int Tq, int i) {
            float acc = 0.0f;
            for (int t = 0; t <= Tq; ++t) acc = fmaf(cw[Tq * (L + 1) + t], xk[t * d_K + i], acc);
            return acc;
        });
    } else {
        const int64_t pb = (bh * nch + cl) * (int64_t)a.nslices * L;
        const float* pk = a.part + pb * d_K;
        const float* pv = a.part2 + pb * d_V;
        float* dk = a.dk + (bh * a.n + t0) * d_K;
        float* dv = a.dv + (bh * a.n + t0) * d_V;
        fin_rows(dk, pk, slice_stride * d_K, a.nslices, nvalid, d_K, [&](int t, int i) {
            float acc = 0.0f;
            for (int Tq = t; Tq < nvalid; ++Tq) acc = fmaf(cw[Tq * (L + 1) + t], xq[Tq * d_K + i], acc);
            return acc;
        });
        fin_rows(dv, pv, slice_stride * d_V, a.nslices, nvalid, d_V, [&](int t, int j) {
            float acc = 0.0f;
            for (int Tq = t; Tq < nvalid; ++Tq) acc = fmaf(ww[Tq * (L + 1) + t], uu[Tq * cols + j], acc);
            return acc;
        });
    }
}

template <typename K>
hipError_t launch_lds(K kernel, dim3 grid, int threads, size_t lds, const BwdArgs& a, hipStream_t st) {
    hipError_t e = hipFuncSetAttribute((const void*)kernel, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kernel, grid, dim3(threads), lds, st, a);
    return hipGetLastError();
}

}  // namespace

// a power of two no larger than the block (the feature loops rely on it)
int bwd_slice_feats(int d_K, int d_V, int L) {
    for (int SV = 128; SV >= 16; SV >>= 1)
        if (bwd_scan_lds_floats(SV, d_K, d_V, L) * 4 <= 150 * 1024) return SV;
    return 0;
}

int64_t bwd_fin_lds_bytes(int d_K, int d_V, int L) { return bwd_fin_lds_floats(d_K, d_V, L) * 4; }

hipError_t launch_bwd_u(const BwdArgs& a, hipStream_t st) {
    const int64_t toks = (int64_t)a.BH * a.n;
    hipLaunchKernelGGL(bwd_u_kernel, dim3((unsigned)((toks + kThreads - 1) / kThreads)), dim3(kThreads), 0, st, a);
    return hipGetLastError();
}

template <int NIDX>
hipError_t launch_bwd_scans(const BwdArgs& a, bool kv, hipStream_t st) {
    const size_t lds = (size_t)bwd_scan_lds_floats(a.slice_feats, a.d_K, a.d_V, a.L) * 4;
    const dim3 grid(a.nslices, a.BH);
    if (kv)
        return a.bf16 ? launch_lds(bwd_kv_kernel<InBF16, NIDX>, grid, kScanThreads, lds, a, st)
                      : launch_lds(bwd_kv_kernel<InF32, NIDX>, grid, kScanThreads, lds, a, st);
    return a.bf16 ? launch_lds(bwd_q_kernel<InBF16, NIDX>, grid, kScanThreads, lds, a, st)
                  : launch_lds(bwd_q_kernel<InF32, NIDX>, grid, kScanThreads, lds, a, st);
}

hipError_t launch_bwd_scan(const BwdArgs& a, bool kv, hipStream_t st) {
    switch (a.P - 1) {                 // slots per feature
        case 0: return launch_bwd_scans<0>(a, kv, st);
        case 1: return launch_bwd_scans<1>(a, kv, st);
        case 2: return launch_bwd_scans<2>(a, kv, st);
        case 3: return launch_bwd_scans<3>(a, kv, st);
        default: return launch_bwd_scans<4>(a, kv, st);
    }
}

hipError_t launch_bwd_q(const BwdArgs& a, hipStream_t st) { return launch_bwd_scan(a, false, st); }

hipError_t launch_bwd_kv(const BwdArgs& a, hipStream_t st) { return launch_bwd_scan(a, true, st); }

hipError_t launch_bwd_fin(const BwdArgs& a, int mode, hipStream_t st) {
    const size_t lds = (size_t)bwd_fin_lds_bytes(a.d_K, a.d_V, a.L);
    const dim3 grid(a.c_end - a.c_begin, a.BH);
    if (mode == 0)
        return a.bf16 ? launch_lds(bwd_fin_kernel<InBF16, 0>, grid, kThreads, lds, a, st)
                      : launch_lds(bwd_fin_kernel<InF32, 0>, grid, kThreads, lds, a, st);
    return a.bf16 ? launch_lds(bwd_fin_kernel<InBF16, 1>, grid, kThreads, lds, a, st)
                  : launch_lds(bwd_fin_kernel<InF32, 1>, grid, kThreads, lds, a, st);
}

}  // namespace sata
