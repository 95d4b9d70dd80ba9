// kern_scan_mfma.hip -- MFMA chunked prefill scan for gfx950 (fp16 operands, fp32 state).
//
// The inter-chunk half of the chunked prefill ([TA] "Feature maps and linear
// attention": the state recurrence, evaluated chunk by chunk):
//     readout   part[t][j] = sum_f qw_f phi_f(q_t) S[f][j]      (S before the chunk)
//     update    S[f][j]   += sum_t phi_f(k_t) u_t[j],   u_t = [v_t | 1]
// Both are dense contractions over a 64-token chunk and a slice of the feature
// axis, run as v_mfma_f32_16x16x32_f16 with fp32 accumulation:
//     readout  (64 tokens x 32 features) x (32 features x 16 columns)
//     update   (16 features x 32 tokens) x (32 tokens x 16 columns)
//
// Operands are fp16, not bf16: gfx950 multiplies fp16 pairs in one VALU
// instruction (bf16 only one value at a time) and converts two fp32 values to fp16
// in one, and the operand building is what bounds this kernel; the matrix rate of
// the two types is the same, and fp16 keeps 3 more mantissa bits.  Exact powers of
// two keep every operand inside fp16's range: the [v | 1] operand carries 2^-8
// (the internal state is S' = 2^-8 c S, with c the key-side factor below), the
// query operand 2^12, and the readout is scaled back by 2^-4 before it is stored.
// The state stays fp32 in registers; its fp16 copy only feeds the readout.
//
// Work split.  The columns of [v | 1] are cut into groups of 64 value columns;
// group 0 also carries the normaliser column (65 columns, 5 tiles of 16), the
// others 4 tiles.  One workgroup (4 waves) owns one slice of 64 rows = 512 kernel
// features of one head for one column group, and walks all chunks of the segment
// in order; its fp32 state never leaves the registers (8 update tiles x 5 column
// tiles x 4 = 160 registers per lane per wave).  A wave owns 16 rows of one
// l-block b: its kernel features are (parent a, l = 8b + e), e = 0..7 (see
// mfma_rows.cpp).  Feature tiles are never written to HBM: per chunk the wave
// builds
//     query side  q^(a, l)[t] = (W_a q_a[t]) * q_l[t]        (W_a = alpha_p C(a) p)
//     key side    k^(a, l)[t] = kpar_a[t] * k_l[t] * c_(a,l)  (c: 0 / 1/(1+m) / 1)
// directly in the MFMA operand layout (q_a, kpar_a: parent products).  The readout
// takes the state packed to fp16 after its last update of the previous chunk: the
// update's accumulator layout (lane = column, 4 rows each) over two tiles is a
// 32-deep B operand when the query operand uses the same feature order.
//
// Per chunk: q, k, v arrive in LDS (bf16) by direct-to-LDS loads issued during the
// previous chunk; the values are moved to fp16 token-major tables (v transposed,
// each wave's 8 key coordinates, the key parent products); readout MFMAs
// (per-wave accumulators) go to four LDS regions; update MFMAs; the sum of the
// four regions is this slice's partial readout, written at the start of the next
// chunk.
#include "scan_mfma.h"

#include <hip/hip_runtime.h>

namespace sata {

namespace {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4v __attribute__((ext_vector_type(4)));

constexpr int kL = 64;                      // chunk length of the MFMA scan
constexpr float kVScale = 1.0f / 256.0f;    // on the [v | 1] operand of the update
constexpr float kQScale = 4096.0f;          // on the query operand of the readout
constexpr float kUScale = 1.0f / 16.0f;     // 1 / (kQScale kVScale): readout back to S's units

template <int D, int NCT>
struct Layout {
    static constexpr int XR = D + 8;         // raw q/k row (bf16): D coords, 1, then 7 zeros
    static constexpr int XSLOTS = XR / 8;    // 16-byte slots per raw row
    static constexpr int VG = 64;            // value columns per column group
    static constexpr int TS = 72;            // fp16 token-major row stride: 64 tokens + pad
    static constexpr int UT = 68;            // readout region row stride (floats, rows = columns)
    static constexpr int rawq = 0;                                  // bytes
    static constexpr int rawk = rawq + kL * XR * 2;
    static constexpr int rawv = rawk + kL * XR * 2;
    static constexpr int vt = rawv + kL * VG * 2;                   // [NCT*16 columns][TS]
    static constexpr int kt = vt + NCT * 16 * TS * 2;               // [wave][8 coordinates][TS]
    static constexpr int kp = kt + kWavesPerSlice * 8 * TS * 2;     // [64 rows][TS]
    static constexpr int ur = kp + kRowsPerSlice * TS * 2;
    static constexpr int bytes = ur + kWavesPerSlice * NCT * 16 * UT * 4;
    // state load/store staging (outside the chunk loop) aliases the readout regions
    static constexpr int IO = NCT * 16 + 4;                         // floats per feature row
    static constexpr int io_rows = kWavesPerSlice * 32;             // 2 tiles per wave per phase
    static_assert(io_rows * IO * 4 <= kWavesPerSlice * NCT * 16 * UT * 4, "state staging size");
    static_assert(rawk % 16 == 0 && rawv % 16 == 0 && vt % 16 == 0 && kt % 16 == 0 && kp % 16 == 0 &&
                  ur % 16 == 0, "16-byte alignment of LDS regions");
    static_assert((kL * XSLOTS) % 64 == 0, "whole DMA blocks per raw chunk");
};

__device__ inline float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ inline float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ inline float bf16_at(const uint16_t* p, int i) { return __uint_as_float((uint32_t)p[i] << 16); }

// 8 bf16 values (one 16-byte slot) to fp16; exact for |x| in fp16's normal range
__device__ inline f16x8 bf16x8_to_f16(const uint4& r) {
    f16x8 o;
    o[0] = (_Float16)bf16_lo(r.x); o[1] = (_Float16)bf16_hi(r.x);
    o[2] = (_Float16)bf16_lo(r.y); o[3] = (_Float16)bf16_hi(r.y);
    o[4] = (_Float16)bf16_lo(r.z); o[5] = (_Float16)bf16_hi(r.z);
    o[6] = (_Float16)bf16_lo(r.w); o[7] = (_Float16)bf16_hi(r.w);
    return o;
}

__device__ inline f16x8 pack_tiles(const f32x4v& lo, const f32x4v& hi) {
    f16x8 r;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        r[e] = (_Float16)lo[e];
        r[4 + e] = (_Float16)hi[e];
    }
    return r;
}

// the key-side factor as the update applies it (rounded to fp16)
__device__ inline float kfactor(float c) { return (float)(_Float16)c; }

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
    constexpr int XR = LY::XR, TS = LY::TS;
    extern __shared__ __align__(16) unsigned char lds_raw[];
    const uint16_t* rq = reinterpret_cast<const uint16_t*>(lds_raw + LY::rawq);
    const uint16_t* rk = reinterpret_cast<const uint16_t*>(lds_raw + LY::rawk);
    const uint16_t* rv = reinterpret_cast<const uint16_t*>(lds_raw + LY::rawv);
    _Float16* vt = reinterpret_cast<_Float16*>(lds_raw + LY::vt);
    _Float16* kt = reinterpret_cast<_Float16*>(lds_raw + LY::kt);
    _Float16* kp = reinterpret_cast<_Float16*>(lds_raw + LY::kp);
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

    // per-lane row constants: query weight (with the operand scale) and LDS addresses of
    // the parent coordinates of row 4 s + g in this lane's token row of the raw q buffer
    uint32_t qoff[KS][NPC > 0 ? NPC : 1];
    float Wq[KS];
#pragma unroll
    for (int s = 0; s < KS; ++s) {
        const uint32_t p3 = rt.parent[row_w + 4 * s + g];
#pragma unroll
        for (int e = 0; e < NPC; ++e)
            qoff[s][e] = (uint32_t)(LY::rawq + (li * XR + ((p3 >> (10 * e)) & 1023u)) * 2);
        Wq[s] = rt.weight[row_w + 4 * s + g] * kQScale;
    }
    // key-side factor of this lane's feature in update tile T
    _Float16 cK[NT];
#pragma unroll
    for (int T = 0; T < NT; ++T) {
        const int s = T >> 1, h = T & 1;
        cK[T] = (_Float16)rt.kscale[(row_w + 4 * s + (li >> 2)) * 8 + 4 * h + (li & 3)];
    }

    // Resident state slice S', update-accumulator layout: lane (column 16 ct + li, g)
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
                io[fr * LY::IO + j] =
                    F >= 0 ? kfactor(rt.kscale[fi]) * kVScale * state[(int64_t)gcol(j) * a.M_pad + F] : 0.0f;
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

    // fp16 copy of the state in the readout's B-operand layout, refreshed at the end of
    // every update (tile pair s covers the readout's K-step s)
    f16x8 Sb[KS][NCT];
#pragma unroll
    for (int s2 = 0; s2 < KS; ++s2)
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) Sb[s2][ct] = pack_tiles(S[2 * s2][ct], S[2 * s2 + 1][ct]);

    // columns of [v | 1] past the live ones are zero for good
    __syncthreads();
    for (int idx = tid; idx < (NCT * 16 - NCL) * TS; idx += 256) vt[NCL * TS + idx] = (_Float16)0.0f;
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
                pp[gcol(j) * kL] = ((up[4 * i * LY::UT] + up[4 * i * LY::UT + WS]) +
                                    (up[4 * i * LY::UT + 2 * WS] + up[4 * i * LY::UT + 3 * WS])) * kUScale;
        }
    };

    for (int c = a.c_begin; c < a.c_end; ++c) {
        const int nvalid = nvalid_of(c);
        const int64_t t1 = (int64_t)(c + 1) * kL;
        const bool more = c + 1 < a.c_end;
        const int nvalid1 = more ? nvalid_of(c + 1) : 0;
        if (c > a.c_begin) write_partial(c - 1);

        // ---- P1: fp16 tables of the chunk -------------------------------------------
        {   // value columns, transposed to [column][token] and scaled; zero past nvalid
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
                _Float16* dst = vt + 4 * c4 * TS + t;
                dst[0] = (_Float16)(bf16_lo(x.x) * kVScale);
                dst[TS] = (_Float16)(bf16_hi(x.x) * kVScale);
                dst[2 * TS] = (_Float16)(bf16_lo(x.y) * kVScale);
                dst[3 * TS] = (_Float16)(bf16_hi(x.y) * kVScale);
            }
        }
        if (ONES && tid < kL) vt[64 * TS + tid] = (_Float16)(tid < nvalid ? kVScale : 0.0f);
        {
            // each wave: its 8 key coordinates l = 8 lb + e, transposed (lane = token), and
            // the parent products of its 16 rows, zero past nvalid.  The parent words are
            // wave-uniform (scalar loads).
            const uint16_t* xrow = rk + lane * XR;
            const f16x8 kx = bf16x8_to_f16(*reinterpret_cast<const uint4*>(xrow + 8 * lb));
            _Float16* ktw = kt + w * 8 * TS + lane;
#pragma unroll
            for (int e = 0; e < 8; ++e) ktw[e * TS] = kx[e];
            _Float16* kdst = kp + (w * kRowsPerWave) * TS + lane;
            const bool tv = lane < nvalid;
            const int row_u = __builtin_amdgcn_readfirstlane(row_w);
            float kpv[kRowsPerWave];
#pragma unroll
            for (int i = 0; i < kRowsPerWave; ++i) {      // all reads first: no LDS round trips
                const uint32_t p3 = rt.parent[row_u + i];
                kpv[i] = 1.0f;
#pragma unroll
                for (int e = 0; e < NPC; ++e) kpv[i] *= bf16_at(xrow, (p3 >> (10 * e)) & 1023u);
            }
#pragma unroll
            for (int i = 0; i < kRowsPerWave; ++i) kdst[i * TS] = (_Float16)(tv ? kpv[i] : 0.0f);
        }
        __syncthreads();                                               // B1
        // raw k and v are free: the next chunk streams in during the readout and update
        if (more) {
            prefetch_x<D, NCT>(k, rt.one_row, t1, nvalid1, lds_raw + LY::rawk, w, lane);
            prefetch_v<D, NCT>(v, t1, nvalid1, d_V, col0, lds_raw + LY::rawv, w, lane);
        }

        // ---- P2: readout U = Q^ . fp16(S') ------------------------------------------
        {
            f32x4v U[4][NCT];
#pragma unroll
            for (int mt = 0; mt < 4; ++mt)
#pragma unroll
                for (int ct = 0; ct < NCT; ++ct) U[mt][ct] = f32x4v{0.0f, 0.0f, 0.0f, 0.0f};
            f16x8 qreg[4];
#pragma unroll
            for (int mt = 0; mt < 4; ++mt)
                qreg[mt] = bf16x8_to_f16(*reinterpret_cast<const uint4*>(rq + (16 * mt + li) * XR + 8 * lb));
#pragma unroll
            for (int s = 0; s < KS; ++s) {
#pragma unroll
                for (int mt = 0; mt < 4; ++mt) {
                    float qp = Wq[s];
#pragma unroll
                    for (int e = 0; e < NPC; ++e)
                        qp *= bf16_at(reinterpret_cast<const uint16_t*>(lds_raw + qoff[s][e] + mt * 16 * XR * 2), 0);
                    const f16x8 A = qreg[mt] * (_Float16)qp;
#pragma unroll
                    for (int ct = 0; ct < NCT; ++ct)
                        U[mt][ct] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A, Sb[s][ct], U[mt][ct], 0, 0, 0);
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
        __syncthreads();                                               // B2
        // raw q is free
        if (more) prefetch_x<D, NCT>(q, rt.one_row, t1, nvalid1, lds_raw + LY::rawq, w, lane);

        // ---- P3: update S' += K^^T . [v | 1] ----------------------------------------
        // this lane's key coordinates l = 8 lb + 4 h + li % 4 over its 8 tokens of step kk
        f16x8 kreg[2][2];
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int kk = 0; kk < 2; ++kk)
                kreg[h][kk] = *reinterpret_cast<const f16x8*>(kt + (w * 8 + 4 * h + (li & 3)) * TS + 32 * kk + 8 * g);
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
            f16x8 Vop[NCT];
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct)
                Vop[ct] = *reinterpret_cast<const f16x8*>(vt + (16 * ct + li) * TS + 32 * kk + 8 * g);
#pragma unroll
            for (int s = 0; s < KS; ++s) {
                const f16x8 kp8 = *reinterpret_cast<const f16x8*>(
                    kp + (w * kRowsPerWave + 4 * s + (li >> 2)) * TS + 32 * kk + 8 * g);
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const int T = 2 * s + h;
                    const f16x8 A = kp8 * kreg[h][kk] * cK[T];
#pragma unroll
                    for (int ct = 0; ct < NCT; ++ct)
                        S[T][ct] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A, Vop[ct], S[T][ct], 0, 0, 0);
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
        // through LDS as for the load; S = S' / (2^-8 c)
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
                if (F >= 0)
                    state[(int64_t)gcol(j) * a.M_pad + F] = io[fr * LY::IO + j] / (kfactor(rt.kscale[fi]) * kVScale);
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
