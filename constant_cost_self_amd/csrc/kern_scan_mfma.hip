// kern_scan_mfma.hip -- bf16 MFMA chunked prefill scan for gfx950.
//
// The inter-chunk half of the chunked prefill ([TA] "Feature maps and linear
// attention": the state recurrence, evaluated chunk by chunk):
//     readout   part[t][j] = sum_f qw_f phi_f(q_t) S[f][j]      (S before the chunk)
//     update    S[f][j]   += sum_t phi_f(k_t) u_t[j],   u_t = [v_t | 1]
// Both are dense contractions over a 64-token chunk and a slice of the feature
// axis, run as v_mfma_f32_16x16x32_bf16 with fp32 accumulation:
//     readout  (64 tokens x 32 features) x (32 features x 16 columns)
//     update   (16 features x 32 tokens) x (32 tokens x 16 columns)
//
// Work split.  The columns of [v | 1] are cut into groups of 64 value columns;
// group 0 also carries the normaliser column (65 columns, 5 tiles of 16), the
// others 4 tiles.  One workgroup (4 waves) owns one slice of 64 rows = 512 kernel
// features of one head for one column group, and walks all chunks of the segment
// in order; its fp32 state never leaves the registers (8 update tiles x 5 column
// tiles x 4 = 160 accumulator registers per lane per wave).  A wave owns 16 rows
// of one l-block b: its kernel features are (parent a, l = 8b + e), e = 0..7 (see
// mfma_rows.cpp).  Feature tiles are never written to HBM: per chunk the wave keeps
// the 8 coordinates x_{8b..8b+7} of its tokens in registers and builds
//     query side  q^(a, l)[t] = (W_a q_a[t]) * q_l[t]        (W_a = alpha_p C(a) p)
//     key side    k^(a, l)[t] = kpar_a[t] * k_l[t] * c_(a,l)  (c: 0 / 1/(1+m) / 1)
// directly in the MFMA operand layout (q_a, kpar_a: parent products).  The readout
// takes the state packed to bf16 after its last update of the previous chunk: the
// update's accumulator layout (lane = column, 4 rows each) over two tiles is a
// 32-deep B operand when the query operand uses the same feature order.
//
// Per chunk: q, k, v arrive in LDS by direct-to-LDS loads issued during the
// previous chunk; parent products of the key side go to an LDS table; readout
// MFMAs (per-wave accumulators) go to four LDS regions; update MFMAs; the sum of
// the four regions is this slice's partial readout, written at the start of the
// next chunk.
#include "scan_mfma.h"

#include <hip/hip_runtime.h>

namespace sata {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4v __attribute__((ext_vector_type(4)));

constexpr int kL = 64;     // chunk length of the MFMA scan

template <int D, int NCT>
struct Layout {
    static constexpr int XR = D + 8;         // raw q/k row (bf16): D coords, 1, then 7 zeros
    static constexpr int XSLOTS = XR / 8;    // 16-byte slots per raw row
    static constexpr int VG = 64;            // value columns per column group
    static constexpr int KP = 68;            // kpar row stride (floats): 64 tokens + pad
    static constexpr int VT = 72;            // vT row stride (bf16): 64 tokens + pad
    static constexpr int UT = 68;            // readout region row stride (floats, rows = columns)
    static constexpr int rawq = 0;                                  // bytes
    static constexpr int rawk = rawq + kL * XR * 2;
    static constexpr int rawv = rawk + kL * XR * 2;
    static constexpr int vt = rawv + kL * VG * 2;
    static constexpr int kp = vt + NCT * 16 * VT * 2;
    static constexpr int ur = kp + kRowsPerSlice * KP * 4;
    static constexpr int bytes = ur + kWavesPerSlice * NCT * 16 * UT * 4;
    // state load/store staging (outside the chunk loop) aliases the readout regions
    static constexpr int IO = NCT * 16 + 4;                         // floats per feature row
    static constexpr int io_rows = kWavesPerSlice * 32;             // 2 tiles per wave per phase
    static_assert(io_rows * IO * 4 <= kWavesPerSlice * NCT * 16 * UT * 4, "state staging size");
    static_assert(rawk % 16 == 0 && rawv % 16 == 0 && vt % 16 == 0 && kp % 16 == 0 && ur % 16 == 0,
                  "16-byte alignment of LDS regions");
    static_assert((kL * XSLOTS) % 64 == 0, "whole DMA blocks per raw chunk");
};

__device__ inline float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ inline float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ inline float bf16_at(const uint16_t* p, int i) { return __uint_as_float((uint32_t)p[i] << 16); }

__device__ inline bf16x8 pack_bf16(const float* x) {
    bf16x8 r;
#pragma unroll
    for (int e = 0; e < 8; ++e) r[e] = (__bf16)x[e];
    return r;
}

__device__ inline bf16x8 pack_tiles(const f32x4v& lo, const f32x4v& hi) {
    bf16x8 r;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        r[e] = (__bf16)lo[e];
        r[4 + e] = (__bf16)hi[e];
    }
    return r;
}

struct RowPtrs {
    const uint32_t* parent;
    const float* weight;
    const float* kscale;
    const int32_t* canon;
    const int32_t* wave_lblock;
    const uint16_t* one_row;     // 8 bf16: 1, 0, ..., 0 (the constant coordinates d..d+7)
};

// Direct-to-LDS copies of one chunk.  A wave instruction moves 64 lanes x 16 bytes
// into a contiguous 1 KiB block; lane i fills bytes [16 i, 16 i + 16).  q and k rows
// get one more slot holding the constant coordinates (1, 0, ..., 0).  Rows past n
// read row 0 of the chunk instead (masked later).
template <int D, int NCT>
__device__ inline void prefetch_x(const uint16_t* x, const uint16_t* one_row, int64_t t0, int nvalid,
                                  unsigned char* dst, int w, int lane) {
    using LY = Layout<D, NCT>;
    constexpr int NBLK = kL * LY::XSLOTS / 64;
#pragma unroll
    for (int blk = w; blk < NBLK; blk += kWavesPerSlice) {
        const int sl = blk * 64 + lane;
        const int t = sl / LY::XSLOTS, cs = sl % LY::XSLOTS;
        const void* src = cs == D / 8 ? (const void*)one_row
                                      : (const void*)(x + (t0 + (t < nvalid ? t : 0)) * D + 8 * cs);
        __builtin_amdgcn_global_load_lds(src, (void __attribute__((address_space(3)))*)(dst + blk * 1024),
                                         16, 0, 0);
    }
}

// The 64 value columns [col0, col0 + 64) of the chunk's v rows (row length d_V).
template <int D, int NCT>
__device__ inline void prefetch_v(const uint16_t* v, int64_t t0, int nvalid, int d_V, int col0,
                                  unsigned char* dst, int w, int lane) {
#pragma unroll
    for (int blk = w; blk < kL * 8 / 64; blk += kWavesPerSlice) {
        const int sl = blk * 64 + lane;
        const int t = sl >> 3, cs = sl & 7;
        const uint16_t* src = v + (t0 + (t < nvalid ? t : 0)) * d_V + col0 + 8 * cs;
        __builtin_amdgcn_global_load_lds((const void*)src,
                                         (void __attribute__((address_space(3)))*)(dst + blk * 1024), 16, 0, 0);
    }
}

template <int D, int DV, int G, int NPC>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void scan_mfma_kernel(PrefillSegArgs a, RowPtrs rt) {
    constexpr bool ONES = G == 0;            // group 0 carries the normaliser column
    constexpr int col0 = 64 * G;             // first value column of the group
    constexpr int NCT = ONES ? 5 : 4;        // column tiles of this group
    constexpr int NCL = ONES ? 65 : 64;      // live columns of this group
    using LY = Layout<D, NCT>;
    constexpr int KS = kRowsPerWave / 4;     // readout K-steps per wave (32 features each)
    constexpr int NT = 2 * KS;               // update tiles per wave (16 features each)
    constexpr int XR = LY::XR;
    extern __shared__ __align__(16) unsigned char lds_raw[];
    const uint16_t* rq = reinterpret_cast<const uint16_t*>(lds_raw + LY::rawq);
    const uint16_t* rk = reinterpret_cast<const uint16_t*>(lds_raw + LY::rawk);
    const uint16_t* rv = reinterpret_cast<const uint16_t*>(lds_raw + LY::rawv);
    uint16_t* vt16 = reinterpret_cast<uint16_t*>(lds_raw + LY::vt);
    float* kpar = reinterpret_cast<float*>(lds_raw + LY::kp);
    float* ured = reinterpret_cast<float*>(lds_raw + LY::ur);

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int g = lane >> 4, li = lane & 15;
    const int slice = blockIdx.x;
    const int64_t bh = blockIdx.y;
    constexpr int d_V = DV, cols = DV + 1;
    const int nch = a.c_end - a.c_begin;
    const int row_w = slice * kRowsPerSlice + w * kRowsPerWave;   // first row of this wave
    const int lb = rt.wave_lblock[slice * kWavesPerSlice + w];
    // global column of local column j of this group (local 64 is the normaliser)
    auto gcol = [&](int j) { return (ONES && j == 64) ? d_V : col0 + j; };

    const uint16_t* q = static_cast<const uint16_t*>(a.q) + bh * (int64_t)a.n * D;
    const uint16_t* k = static_cast<const uint16_t*>(a.k) + bh * (int64_t)a.n * D;
    const uint16_t* v = static_cast<const uint16_t*>(a.v) + bh * (int64_t)a.n * d_V;
    float* state = a.state ? a.state + bh * (int64_t)cols * a.M_pad : nullptr;

    auto nvalid_of = [&](int c) {
        const int64_t r = a.n - (int64_t)c * kL;
        return (int)(r < kL ? r : kL);
    };
    {   // first chunk in flight while the state is being set up
        const int64_t t0 = (int64_t)a.c_begin * kL;
        const int nv = nvalid_of(a.c_begin);
        prefetch_x<D, NCT>(q, rt.one_row, t0, nv, lds_raw + LY::rawq, w, lane);
        prefetch_x<D, NCT>(k, rt.one_row, t0, nv, lds_raw + LY::rawk, w, lane);
        prefetch_v<D, NCT>(v, t0, nv, d_V, col0, lds_raw + LY::rawv, w, lane);
    }

    // per-lane row constants: query weight and LDS addresses of the parent coordinates
    // of row 4 s + g in this lane's token row of the raw q buffer (m-tile 0)
    uint32_t qoff[KS][NPC > 0 ? NPC : 1];
    float Wq[KS];
#pragma unroll
    for (int s = 0; s < KS; ++s) {
        const uint32_t p3 = rt.parent[row_w + 4 * s + g];
#pragma unroll
        for (int e = 0; e < NPC; ++e)
            qoff[s][e] = (uint32_t)(LY::rawq + (li * XR + ((p3 >> (10 * e)) & 1023u)) * 2);
        Wq[s] = rt.weight[row_w + 4 * s + g];
    }
    float cK[NT];
    bool ones[NT];
#pragma unroll
    for (int T = 0; T < NT; ++T) {
        const int s = T >> 1, h = T & 1;
        cK[T] = rt.kscale[(row_w + 4 * s + (li >> 2)) * 8 + 4 * h + (li & 3)];
        ones[T] = __all(cK[T] == 1.0f);
    }

    // Resident state slice, update-accumulator layout: lane (column 16 ct + li, g)
    // register r of tile T = 2 s + h holds kernel feature (row 4 s + g, element 4 h + r).
    f32x4v S[NT][NCT];
#pragma unroll
    for (int T = 0; T < NT; ++T)
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) S[T][ct] = f32x4v{0.0f, 0.0f, 0.0f, 0.0f};
    if (a.load_state) {
        // through LDS, 2 tiles per wave at a time: plain gather loop, then a register
        // fill with compile-time indices (keeps the unrolled code free of table loads)
        float* io = ured;
        const int row_wg = slice * kRowsPerSlice;
#pragma unroll
        for (int ph = 0; ph < NT / 2; ++ph) {
            __syncthreads();
            for (int idx = tid; idx < LY::io_rows * NCL; idx += 256) {
                const int fr = idx / NCL, j = idx % NCL;
                const int ww = fr / 32, fl = fr % 32;
                const int T = 2 * ph + fl / 16, rho = fl % 16;
                const int fi = (row_wg + ww * kRowsPerWave + 4 * (T >> 1) + (rho >> 2)) * 8 +
                               4 * (T & 1) + (rho & 3);
                const int F = rt.canon[fi];
                io[fr * LY::IO + j] = F >= 0 ? rt.kscale[fi] * state[(int64_t)gcol(j) * a.M_pad + F] : 0.0f;
            }
            __syncthreads();
#pragma unroll
            for (int Tl = 0; Tl < 2; ++Tl)
#pragma unroll
                for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int j = 16 * ct + li;
                        S[2 * ph + Tl][ct][r] = j < NCL ? io[(w * 32 + Tl * 16 + 4 * g + r) * LY::IO + j] : 0.0f;
                    }
        }
    }
    // bf16 copy of the state in the readout's B-operand layout, refreshed at the end of
    // every update (tile pair s covers the readout's K-step s)
    bf16x8 Sb[KS][NCT];
#pragma unroll
    for (int s2 = 0; s2 < KS; ++s2)
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) Sb[s2][ct] = pack_tiles(S[2 * s2][ct], S[2 * s2 + 1][ct]);

    // columns of [v | 1] past the live ones are zero for good
    __syncthreads();
    for (int idx = tid; idx < (NCT * 16 - NCL) * kL; idx += 256) {
        const int j = NCL + idx / kL, t = idx % kL;
        vt16[j * LY::VT + t] = 0;
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();

    // A slice's partial readout of chunk c (the sum of the 4 waves' regions, [col][token])
    // is written at the start of chunk c + 1, so the stores complete during that chunk.
    auto write_partial = [&](int c) {
        float* pp = a.partial + ((bh * nch + (c - a.c_begin)) * a.nslices + slice) * (int64_t)kL * cols + lane;
        const float* up = ured + w * LY::UT + lane;
        constexpr int WS = NCT * 16 * LY::UT;                  // one wave's region
        constexpr int NJ = (NCL + 3) / 4;                      // columns per wave (last one partial)
#pragma unroll
        for (int i = 0; i < NJ; ++i) {
            const int j = w + 4 * i;
            if (i < NJ - 1 || j < NCL)
                pp[gcol(j) * kL] = (up[4 * i * LY::UT] + up[4 * i * LY::UT + WS]) +
                                   (up[4 * i * LY::UT + 2 * WS] + up[4 * i * LY::UT + 3 * WS]);
        }
    };

    for (int c = a.c_begin; c < a.c_end; ++c) {
        const int nvalid = nvalid_of(c);
        const int64_t t1 = (int64_t)(c + 1) * kL;
        const bool more = c + 1 < a.c_end;
        const int nvalid1 = more ? nvalid_of(c + 1) : 0;
        if (c > a.c_begin) write_partial(c - 1);

        // ---- P1: value columns transposed to bf16, key parent products ---------------
        {
            constexpr int NV = kL * LY::VG / 4 / 256;
            uint2 r2[NV];
#pragma unroll
            for (int it = 0; it < NV; ++it) {            // all reads first: no LDS round trips
                const int idx = tid + 256 * it;
                r2[it] = *reinterpret_cast<const uint2*>(rv + (idx / (LY::VG / 4)) * LY::VG + 4 * (idx % (LY::VG / 4)));
            }
#pragma unroll
            for (int it = 0; it < NV; ++it) {
                const int idx = tid + 256 * it;
                const int t = idx / (LY::VG / 4), c4 = idx % (LY::VG / 4);
                const uint2 x = t < nvalid ? r2[it] : uint2{0u, 0u};
                uint16_t* dst = vt16 + 4 * c4 * LY::VT + t;
                dst[0] = (uint16_t)(x.x & 0xffffu);
                dst[LY::VT] = (uint16_t)(x.x >> 16);
                dst[2 * LY::VT] = (uint16_t)(x.y & 0xffffu);
                dst[3 * LY::VT] = (uint16_t)(x.y >> 16);
            }
        }
        if (ONES && tid < kL) vt16[64 * LY::VT + tid] = tid < nvalid ? (uint16_t)0x3f80u : (uint16_t)0u;
        {
            // each wave builds the parent products of its own 16 rows; lane = token.
            // The parent words are wave-uniform (scalar loads).
            const uint16_t* xrow = rk + lane * XR;
            float* kdst = kpar + (w * kRowsPerWave) * LY::KP + lane;
            const bool tv = lane < nvalid;
            const int row_u = __builtin_amdgcn_readfirstlane(row_w);
            float kp[kRowsPerWave];
#pragma unroll
            for (int i = 0; i < kRowsPerWave; ++i) {      // all reads first: no LDS round trips
                const uint32_t p3 = rt.parent[row_u + i];
                kp[i] = 1.0f;
#pragma unroll
                for (int e = 0; e < NPC; ++e) kp[i] *= bf16_at(xrow, (p3 >> (10 * e)) & 1023u);
            }
#pragma unroll
            for (int i = 0; i < kRowsPerWave; ++i) kdst[i * LY::KP] = tv ? kp[i] : 0.0f;
        }
        __syncthreads();                                               // B1
        if (more) prefetch_v<D, NCT>(v, t1, nvalid1, d_V, col0, lds_raw + LY::rawv, w, lane);

        // ---- P2: readout U = Q^ . bf16(S) ------------------------------------------
        {
            f32x4v U[4][NCT];
#pragma unroll
            for (int mt = 0; mt < 4; ++mt)
#pragma unroll
                for (int ct = 0; ct < NCT; ++ct) U[mt][ct] = f32x4v{0.0f, 0.0f, 0.0f, 0.0f};
            float qreg[4][8];
#pragma unroll
            for (int mt = 0; mt < 4; ++mt) {
                const uint4 raw = *reinterpret_cast<const uint4*>(rq + (16 * mt + li) * XR + 8 * lb);
                qreg[mt][0] = bf16_lo(raw.x); qreg[mt][1] = bf16_hi(raw.x);
                qreg[mt][2] = bf16_lo(raw.y); qreg[mt][3] = bf16_hi(raw.y);
                qreg[mt][4] = bf16_lo(raw.z); qreg[mt][5] = bf16_hi(raw.z);
                qreg[mt][6] = bf16_lo(raw.w); qreg[mt][7] = bf16_hi(raw.w);
            }
#pragma unroll
            for (int s = 0; s < KS; ++s) {
#pragma unroll
                for (int mt = 0; mt < 4; ++mt) {
                    float qp = Wq[s];
#pragma unroll
                    for (int e = 0; e < NPC; ++e)
                        qp *= bf16_at(reinterpret_cast<const uint16_t*>(lds_raw + qoff[s][e] + mt * 16 * XR * 2), 0);
                    float x[8];
#pragma unroll
                    for (int e = 0; e < 8; ++e) x[e] = qp * qreg[mt][e];
                    const bf16x8 A = pack_bf16(x);
#pragma unroll
                    for (int ct = 0; ct < NCT; ++ct)
                        U[mt][ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, Sb[s][ct], U[mt][ct], 0, 0, 0);
                }
                __builtin_amdgcn_sched_barrier(0x100);   // only LDS reads may move across
            }
            // this wave's readout, column-major: ured[w][col][token], 4 tokens per store
            float* ur = ured + w * (NCT * 16 * LY::UT);
#pragma unroll
            for (int mt = 0; mt < 4; ++mt)
#pragma unroll
                for (int ct = 0; ct < NCT; ++ct)
                    *reinterpret_cast<f32x4v*>(ur + (16 * ct + li) * LY::UT + 16 * mt + 4 * g) = U[mt][ct];
        }
        // the wave's key coordinates k_l (l = 8 lb + 4 h + li % 4) for its tokens
        float kreg[2][2][8];
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int kk = 0; kk < 2; ++kk)
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    kreg[h][kk][e] = bf16_at(rk, (32 * kk + 8 * g + e) * XR + 8 * lb + 4 * h + (li & 3));
        __syncthreads();                                               // B2
        // the raw q/k buffers are free: the next chunk streams in during the update
        if (more) {
            prefetch_x<D, NCT>(q, rt.one_row, t1, nvalid1, lds_raw + LY::rawq, w, lane);
            prefetch_x<D, NCT>(k, rt.one_row, t1, nvalid1, lds_raw + LY::rawk, w, lane);
        }

        // ---- P3: update S += K^^T . [v | 1] ------------------------------------------
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
            bf16x8 Vop[NCT];
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct)
                Vop[ct] = *reinterpret_cast<const bf16x8*>(vt16 + (16 * ct + li) * LY::VT + 32 * kk + 8 * g);
#pragma unroll
            for (int s = 0; s < KS; ++s) {
                const float* kpr = kpar + (w * kRowsPerWave + 4 * s + (li >> 2)) * LY::KP + 32 * kk + 8 * g;
                const f32x4v p0 = *reinterpret_cast<const f32x4v*>(kpr);
                const f32x4v p1 = *reinterpret_cast<const f32x4v*>(kpr + 4);
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const int T = 2 * s + h;
                    float x[8];
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        x[e] = p0[e] * kreg[h][kk][e];
                        x[4 + e] = p1[e] * kreg[h][kk][4 + e];
                    }
                    if (!ones[T]) {
#pragma unroll
                        for (int e = 0; e < 8; ++e) x[e] *= cK[T];
                    }
                    const bf16x8 A = pack_bf16(x);
#pragma unroll
                    for (int ct = 0; ct < NCT; ++ct)
                        S[T][ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, Vop[ct], S[T][ct], 0, 0, 0);
                }
                // on the last token step, tile pair s - 1 is final: pack it for the next
                // readout while pair s is still in the matrix pipe
                if (kk == 1 && s > 0) {
#pragma unroll
                    for (int ct = 0; ct < NCT; ++ct) Sb[s - 1][ct] = pack_tiles(S[2 * s - 2][ct], S[2 * s - 1][ct]);
                }
                __builtin_amdgcn_sched_barrier(0x100);   // only LDS reads may move across
            }
        }
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) Sb[KS - 1][ct] = pack_tiles(S[2 * KS - 2][ct], S[2 * KS - 1][ct]);
        __builtin_amdgcn_s_waitcnt(0);          // the next chunk has landed
        __syncthreads();                                               // B3
    }
    if (a.c_end > a.c_begin) write_partial(a.c_end - 1);

    if (a.store_state) {
        // through LDS as for the load; the internal S' = c S is scaled back by 1/c
        float* io = ured;
        const int row_wg = slice * kRowsPerSlice;
#pragma unroll
        for (int ph = 0; ph < NT / 2; ++ph) {
            __syncthreads();
#pragma unroll
            for (int Tl = 0; Tl < 2; ++Tl)
#pragma unroll
                for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        io[(w * 32 + Tl * 16 + 4 * g + r) * LY::IO + 16 * ct + li] = S[2 * ph + Tl][ct][r];
            __syncthreads();
            for (int idx = tid; idx < LY::io_rows * NCL; idx += 256) {
                const int fr = idx / NCL, j = idx % NCL;
                const int ww = fr / 32, fl = fr % 32;
                const int T = 2 * ph + fl / 16, rho = fl % 16;
                const int fi = (row_wg + ww * kRowsPerWave + 4 * (T >> 1) + (rho >> 2)) * 8 +
                               4 * (T & 1) + (rho & 3);
                const int F = rt.canon[fi];
                if (F >= 0) state[(int64_t)gcol(j) * a.M_pad + F] = io[fr * LY::IO + j] / rt.kscale[fi];
            }
        }
        if (slice == 0) {
            const int64_t padn = a.M_pad - a.M;
            for (int64_t idx = tid; idx < NCL * padn; idx += 256)
                state[(int64_t)gcol((int)(idx / padn)) * a.M_pad + a.M + idx % padn] = 0.0f;
        }
    }
}

template <int D, int DV, int G, int NPC>
hipError_t launch_t(const PrefillSegArgs& a, const MfmaTables& m, hipStream_t st) {
    using LY = Layout<D, G == 0 ? 5 : 4>;
    static_assert(LY::bytes <= 160 * 1024, "LDS budget");
    RowPtrs rt{m.parent, m.weight, m.kscale, m.canon, m.wave_lblock, m.one_row};
    hipError_t e = hipFuncSetAttribute((const void*)scan_mfma_kernel<D, DV, G, NPC>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, LY::bytes);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((scan_mfma_kernel<D, DV, G, NPC>), dim3(a.nslices, a.BH), dim3(256), LY::bytes, st,
                       a, rt);
    return hipGetLastError();
}

// one launch per column group of 64 value columns; group 0 carries the normaliser
template <int D, int NPC>
hipError_t launch_groups(const PrefillSegArgs& a, const MfmaTables& m, hipStream_t st) {
    if (a.d_V == 64) return launch_t<D, 64, 0, NPC>(a, m, st);
    hipError_t e = launch_t<D, 128, 0, NPC>(a, m, st);
    return e == hipSuccess ? launch_t<D, 128, 1, NPC>(a, m, st) : e;
}

template <int D>
hipError_t launch_d(const PrefillSegArgs& a, const MfmaTables& m, hipStream_t st) {
    switch (a.P) {
        case 2: return launch_groups<D, 0>(a, m, st);
        case 3: return launch_groups<D, 1>(a, m, st);
        case 4: return launch_groups<D, 2>(a, m, st);
        default: return launch_groups<D, 3>(a, m, st);
    }
}

}  // namespace

int build_mfma_tables(const HostTables& h, MfmaTables& m) {
    m = MfmaTables();
    MfmaHostRows r;
    if (!build_mfma_rows(h, r)) return 0;        // not an MFMA shape: the VALU scan is used
    const size_t nr = (size_t)r.nrows, nw = r.wave_lblock.size();
    const size_t bytes = 16 + nr * 4 + nr * 4 + nr * 8 * 4 + nr * 8 * 4 + nw * 4;
    char* base = nullptr;
    if (hipMalloc(&base, bytes) != hipSuccess) {
        (void)hipGetLastError();
        return -5;
    }
    size_t off = 0;
    auto put = [&](const void* src, size_t n) -> void* {
        void* dst = base + off;
        off += n;
        return hipMemcpy(dst, src, n, hipMemcpyHostToDevice) == hipSuccess ? dst : nullptr;
    };
    const uint16_t one_row[8] = {0x3f80u, 0, 0, 0, 0, 0, 0, 0};
    m.one_row = (const uint16_t*)put(one_row, 16);
    m.parent = (const uint32_t*)put(r.parent.data(), nr * 4);
    m.weight = (const float*)put(r.weight.data(), nr * 4);
    m.kscale = (const float*)put(r.kscale.data(), nr * 8 * 4);
    m.canon = (const int32_t*)put(r.canon.data(), nr * 8 * 4);
    m.wave_lblock = (const int32_t*)put(r.wave_lblock.data(), nw * 4);
    m.d_rows = base;
    if (!m.one_row || !m.parent || !m.weight || !m.kscale || !m.canon || !m.wave_lblock) {
        free_mfma_tables(m);
        return -4;
    }
    m.nslices = r.nrows / kRowsPerSlice;
    m.slice_feats = kRowsPerSlice * 8;
    m.d_K = r.d_K;
    m.P = r.P;
    m.ok = true;
    return 0;
}

void free_mfma_tables(MfmaTables& m) {
    if (m.d_rows) (void)hipFree(m.d_rows);
    m = MfmaTables();
}

bool mfma_supported(const MfmaTables& m, bool bf16, int d_K, int d_V, int P, int L) {
    return m.ok && bf16 && d_K == m.d_K && P == m.P && P >= 2 && P <= 5 && L == kL &&
           (d_K == 64 || d_K == 128) && (d_V == 64 || d_V == 128);
}

hipError_t launch_scan_mfma(const PrefillSegArgs& a, const MfmaTables& m, hipStream_t st) {
    return a.d_K == 64 ? launch_d<64>(a, m, st) : launch_d<128>(a, m, st);
}

}  // namespace sata
