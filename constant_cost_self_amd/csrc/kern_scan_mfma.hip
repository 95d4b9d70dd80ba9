// kern_scan_mfma.hip -- MFMA chunked prefill scan for gfx950 (fp16 operands, fp32 state).
//
// The inter-chunk half of the chunked prefill ([TA] "Feature maps and linear
// attention": the state recurrence, evaluated chunk by chunk):
//     readout   part[t][j] = sum_f qw_f phi_f(q_t) S[f][j]      (S before the window)
//     update    S[f][j]   += sum_t phi_f(k_t) u_t[j],   u_t = [v_t | 1]
// The readout is taken once per window of NSUB chunks of L = 64 tokens (R = 256
// tokens at d_K = 64, 128 at d_K = 128) against the state before the window; the
// finalize adds the direct part of the window's earlier chunks.  The update runs
// chunk by chunk.  Both are dense contractions over tokens and a slice of the
// feature axis, run as v_mfma_f32_16x16x32_f16 with fp32 accumulation:
//     readout  (16 tokens x 32 features) x (32 features x 16 columns)
//     update   (16 features x 32 tokens) x (32 tokens x 16 columns)
//
// Operands are fp16, not bf16: gfx950 multiplies fp16 pairs in one VALU
// instruction (bf16 only one value at a time) and converts two fp32 values to fp16
// in one, and operand building competes with the matrix pipe for issue slots; the
// matrix rate of the two types is the same, and fp16 keeps 3 more mantissa bits.
// Exact powers of two keep every operand inside fp16's range: the [v | 1] operand
// carries 2^-8 (the internal state is S' = 2^-8 c S, with c the key-side factor
// below), the query operand 2^12, and the readout is scaled back by 2^-4.
//
// Work split.  The columns of [v | 1] are cut into groups of 64 value columns;
// group 0 also carries the normaliser column (65 columns, 5 tiles of 16), the
// others 4 tiles.  One workgroup of 8 waves (two per SIMD, so that one wave's
// waits overlap the other's matrix work) owns one slice of 64 rows = 512 kernel
// features of one head for one column group, and walks all chunks of the segment
// in order.  Wave w owns rows 8w .. 8w+7: kernel features (parent a, l = 8b + e),
// e = 0..7, with one l-block b per wave (see mfma_rows.cpp); its fp32 state never
// leaves the registers (4 update tiles x 5 column tiles x 4 = 80 registers).
// Feature tiles are never written to HBM: per chunk the operands are built as
//     query side  q^(a, l)[t] = (W_a q_a[t]) * q_l[t]        (W_a = alpha_p C(a) p)
//     key side    k^(a, l)[t] = kpar_a[t] * k_l[t] * c_(a,l)  (c: 0 / 1/(1+m) / 1)
// directly in the MFMA operand layout (q_a, kpar_a: parent products).
//
// The readout is split by tokens, not by features: wave w computes R / 8 tokens of
// the window (two or one 16-token tiles) over all 512 features of the slice, so the
// slice's partial readout leaves the registers straight to HBM with no exchange
// between waves.  Its B operand, the state packed to fp16 after the previous
// window's last update, is shared through LDS and read once per window: the
// update's accumulator layout (lane = column, 4 rows each) over two tiles is a
// 32-deep B operand when the query operand uses the same feature order.  A larger
// window gives each B byte more tokens (R / 8 per wave) without more registers.
//
// Per window: the window's q arrives in LDS (bf16) by direct-to-LDS loads issued
// during the previous window and is converted to fp16 in place; readout.  Per chunk:
// k and v arrive by direct-to-LDS loads a chunk ahead; v (transposed, scaled) and
// all key coordinates go to fp16 token-major tables; update.  After the window's last
// update the fp16 state goes to LDS.
#include "scan_mfma.h"

#include <hip/hip_runtime.h>

namespace sata {

namespace {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4v __attribute__((ext_vector_type(4)));

constexpr int kWaves = kWavesPerSlice;      // 8 waves, 8 rows each
constexpr int kL = 64;                      // chunk length (partials, finalize)
constexpr int kLU = 128;                    // tokens per state update
constexpr float kVScale = 1.0f / 256.0f;    // on the [v | 1] operand of the update
constexpr float kQScale = 4096.0f;          // on the query operand of the readout
constexpr float kUScale = 1.0f / 16.0f;     // 1 / (kQScale kVScale): readout back to S's units

template <int D, int NCT>
struct Layout {
    static constexpr int L = kL;                     // chunk (partials)
    static constexpr int LU = kLU;                   // update sub-chunk
    static constexpr int R = D == 64 ? 256 : 128;    // readout window (tokens)
    static constexpr int NSUB = R / L;               // chunks per window
    static constexpr int TW = R / kWaves;            // readout tokens per wave (32 or 16)
    static constexpr int MTW = TW / 16;              // readout token tiles per wave
    static constexpr int KS = kRowsPerSlice / 4;     // readout K-steps (32 features each)
    static constexpr int XR = D + 8;                 // raw q/k row: D coords, 1, then 7 zeros
    static constexpr int XSLOTS = XR / 8;            // 16-byte slots per raw row
    static constexpr int TS = LU + 8;                // fp16 token-major row stride of the tables
    static constexpr int VROWS = NCT == 5 ? 65 : 64;
    static constexpr int sb = 0;                                    // [4 ct][KS][64 lanes] x 16 B
    static constexpr int sb4 = sb + 4 * KS * 64 * 16;               // normaliser tile: [KS][4 g] x 16 B
    // the update's tables alias the fp16 state: they live between the window's readout
    // and the next window's state copy
    static constexpr int vt = 0;                                    // [VROWS][TS]
    static constexpr int kT = vt + VROWS * TS * 2;                  // [XR coordinates][TS] fp16 keys
    static constexpr int tables_end = kT + XR * TS * 2;
    static constexpr int sb_end = sb4 + (NCT == 5 ? KS * 4 * 16 : 0);
    static constexpr int qt = ((tables_end > sb_end ? tables_end : sb_end) + 15) / 16 * 16;  // window's q rows
    static constexpr int rawk = qt + R * XR * 2;                    // one sub-chunk of raw k
    static constexpr int rawv = rawk + LU * XR * 2;                 // one sub-chunk of raw v (64 columns)
    static constexpr int ri = rawv + LU * 64 * 2;                   // [64 rows] readout row constants
    static constexpr int bytes = ri + kRowsPerSlice * 8;
    // state load/store staging (outside the chunk loop) aliases the fp16 state area
    static constexpr int IO = 68;                                   // floats per feature row
    static constexpr int io_rows = kWaves * 16;                     // one tile per wave per phase
    static constexpr int cf = sb + io_rows * IO * 4;                // [512] canonical index, [512] factor
    static_assert(cf + kRowsPerSlice * 8 * 8 <= 4 * KS * 64 * 16, "state staging size");
    static_assert(qt % 16 == 0 && rawk % 16 == 0 && rawv % 16 == 0 && kT % 16 == 0 && ri % 16 == 0,
                  "16-byte alignment of LDS regions");
    static_assert((R * XSLOTS) % 64 == 0 && (LU * XSLOTS) % 64 == 0, "whole DMA blocks per raw chunk");
    static_assert(TW % 16 == 0 && L % TW == 0 && KS == 16 && R % LU == 0, "readout tiling");
};

__device__ inline float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ inline float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

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

// An LDS byte address the compiler may not re-derive: the constant parts of the
// accesses made from it then fit the 16-bit offset field of ds_read/ds_write, and one
// register serves a whole table.
__device__ inline uint32_t lds_base(uint32_t a) {
    asm volatile("" : "+v"(a));
    return a;
}
template <typename T>
__device__ inline const T& lds_at(const unsigned char* lds, uint32_t base, uint32_t off) {
    return *reinterpret_cast<const T*>(lds + base + off);
}

// Workgroup barrier for the chunk loop: this wave's LDS accesses have completed and
// at most VM of its vector-memory operations are still outstanding (63: no wait).
// Unlike __syncthreads() it does not wait for outstanding global stores unless VM
// asks for it (they retire in order with the loads on this architecture).
template <int VM>
__device__ inline void lds_barrier() {
    static_assert(VM >= 0 && VM <= 63, "vmcnt range");
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt((VM & 15) | (7 << 4) | (0 << 8) | ((VM >> 4) << 14));
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

struct RowPtrs {
    const uint32_t* parent;
    const float* weight;
    const float* kscale;
    const int32_t* canon;
    const int32_t* wave_lblock;
};

// Direct-to-LDS copies of ROWS rows of q or k.  A wave instruction moves 64 lanes x
// 16 bytes into a contiguous 1 KiB block; lane i fills bytes [16 i, 16 i + 16).  The
// slot after each row's D coordinates holds the constant coordinates (1, 0, ..., 0),
// written once: its lanes are masked off.  Rows past n read row 0 of the chunk
// instead (masked later).  Addresses are a uniform base plus 32-bit lane offsets.
template <int D, int ROWS>
__device__ inline void prefetch_x(const uint16_t* x0, int nvalid, unsigned char* dst, int w, int lane) {
    constexpr int XSLOTS = (D + 8) / 8;
    constexpr int NBLK = ROWS * XSLOTS / 64;
    for (int blk = w; blk < NBLK; blk += kWaves) {
        const int sl = blk * 64 + lane;
        const int t = sl / XSLOTS, cs = sl % XSLOTS;
        if (cs != D / 8)
            __builtin_amdgcn_global_load_lds((const void*)(x0 + ((t < nvalid ? t : 0) * D + 8 * cs)),
                                             (void __attribute__((address_space(3)))*)(dst + blk * 1024), 16, 0, 0);
    }
}

// The 64 value columns [col0, col0 + 64) of a sub-chunk's v rows (row length d_V), v0
// at its first row and column col0, stored column-group major per 64 tokens: wave w
// moves columns 8w .. 8w+7 of tokens 64 h + lane into 1 KiB block 8 h + w.  Rows past
// nvalid read row 0 instead (masked later).
template <int ROWS>
__device__ inline void prefetch_v(const uint16_t* v0, int nvalid, int d_V, unsigned char* dst, int w, int lane) {
#pragma unroll
    for (int h = 0; h < ROWS / 64; ++h) {
        const int t = 64 * h + lane;
        __builtin_amdgcn_global_load_lds((const void*)(v0 + ((t < nvalid ? t : 0) * d_V + 8 * w)),
                                         (void __attribute__((address_space(3)))*)(dst + (8 * h + w) * 1024), 16, 0, 0);
    }
}

template <int D, int DV, int G, int NPC>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
void scan_mfma_kernel(PrefillSegArgs a, RowPtrs rt) {
    constexpr bool ONES = G == 0;            // group 0 carries the normaliser column
    constexpr int col0 = 64 * G;             // first value column of the group
    constexpr int NCT = ONES ? 5 : 4;        // column tiles of this group
    constexpr int NCL = ONES ? 65 : 64;      // live columns of this group
    using LY = Layout<D, NCT>;
    constexpr int L = kL, LU = LY::LU, XR = LY::XR, TS = LY::TS, NSUB = LY::NSUB, R = LY::R, TW = LY::TW;
    constexpr int MTW = LY::MTW, KS = LY::KS;
    extern __shared__ __align__(16) unsigned char lds_raw[];
    const uint16_t* rk = reinterpret_cast<const uint16_t*>(lds_raw + LY::rawk);
    _Float16* vt = reinterpret_cast<_Float16*>(lds_raw + LY::vt);
    _Float16* kT = reinterpret_cast<_Float16*>(lds_raw + LY::kT);
    f16x8* sb = reinterpret_cast<f16x8*>(lds_raw + LY::sb);
    f16x8* sb4 = reinterpret_cast<f16x8*>(lds_raw + LY::sb4);

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int g = lane >> 4, li = lane & 15;
    const int slice = blockIdx.x;
    const int64_t bh = blockIdx.y / a.nsub;
    const int sub = blockIdx.y % a.nsub;
    constexpr int d_V = DV, cols = DV + 1;
    const int nch = a.c_end - a.c_begin;       // chunks of the partial buffer
    // the chunks this block scans: its sub-segment (the whole range when nsub = 1)
    const int cb = a.c_begin + sub * a.sub_chunks;
    const int ce = a.nsub > 1 && cb + a.sub_chunks < a.c_end ? cb + a.sub_chunks : a.c_end;
    const int row_s = slice * kRowsPerSlice;                 // first row of the slice
    const int lb_w = rt.wave_lblock[slice * kWaves + w];     // l-block of this wave's update rows
    // global column of local column j of this group (local 64 is the normaliser)
    auto gcol = [&](int j) { return (ONES && j == 64) ? d_V : col0 + j; };

    const uint16_t* q = static_cast<const uint16_t*>(a.q) + bh * (int64_t)a.n * D;
    const uint16_t* k = static_cast<const uint16_t*>(a.k) + bh * (int64_t)a.n * D;
    const uint16_t* v = static_cast<const uint16_t*>(a.v) + bh * (int64_t)a.n * d_V;
    float* state = a.state ? a.state + (bh * a.nsub + sub) * (int64_t)cols * a.M_pad : nullptr;

    // tokens of [c L, c L + len) that exist
    auto nvalid_of = [&](int c, int len) {
        const int64_t r = a.n - (int64_t)c * L;
        return (int)(r < len ? r : len);
    };
    // tokens of [c L, c L + LU) that belong to the segment (the update stops at its end)
    const int64_t seg_end = (int64_t)ce * L < a.n ? (int64_t)ce * L : a.n;
    auto nupd_of = [&](int c) {
        const int64_t r = seg_end - (int64_t)c * L;
        return (int)(r < LU ? r : LU);
    };
    auto prefetch_q = [&](int cw) {
        prefetch_x<D, R>(q + (int64_t)cw * L * D, nvalid_of(cw, R), lds_raw + LY::qt, w, lane);
    };
    auto prefetch_kv = [&](int c) {        // the update sub-chunk starting at chunk c
        const int64_t t0 = (int64_t)c * L;
        const int nv = nupd_of(c);
        prefetch_x<D, LU>(k + t0 * D, nv, lds_raw + LY::rawk, w, lane);
        prefetch_v<LU>(v + t0 * d_V + col0, nv, d_V, lds_raw + LY::rawv, w, lane);
    };
    // the constant coordinate slot of every raw q and k row, for good
    for (int t = tid; t < R + LU; t += 512) {
        uint16_t* row = reinterpret_cast<uint16_t*>(lds_raw + (t < R ? LY::qt : LY::rawk)) + (t < R ? t : t - R) * XR + D;
        *reinterpret_cast<uint4*>(row) = uint4{0x3f80u, 0u, 0u, 0u};
    }
    // the first window's q and first sub-chunk's k, v in flight while the state is set up
    if (!a.update_only) prefetch_q(cb);
    prefetch_kv(cb);

    // readout constants of the slice's rows (K-step s covers rows 4 s .. 4 s + 3, lane group
    // g row 4 s + g), in LDS: the parent coordinates as byte offsets in a q row (10 bits
    // each) and the query weight with the operand scale (fp16 bits)
    if (tid < kRowsPerSlice) {
        const int row = row_s + tid;
        const uint32_t p3 = rt.parent[row];
        uint32_t o = 0;
#pragma unroll
        for (int e = 0; e < NPC; ++e) o |= (((p3 >> (10 * e)) & 1023u) * 2u) << (10 * e);
        const _Float16 wq = (_Float16)(rt.weight[row] * kQScale);
        reinterpret_cast<uint2*>(lds_raw + LY::ri)[tid] = uint2{o, (uint32_t)__builtin_bit_cast(uint16_t, wq)};
    }
    // l-blocks of the slice's row octets (uniform)
    int lbg[KS / 2];
#pragma unroll
    for (int gi = 0; gi < KS / 2; ++gi) lbg[gi] = __builtin_amdgcn_readfirstlane(rt.wave_lblock[slice * kWaves + gi]);
    // key parents of this lane's update rows 8 w + 4 s + li / 4: byte offsets of their
    // coordinate rows in the key table (a missing parent is the constant coordinate d,
    // which is 1 for the chunk's tokens and 0 past them)
    constexpr int NPR = NPC > 0 ? NPC : 1;
    uint32_t kpa[2][NPR];
#pragma unroll
    for (int s = 0; s < 2; ++s) {
        const uint32_t p3 = rt.parent[row_s + 8 * w + 4 * s + (li >> 2)];
#pragma unroll
        for (int e = 0; e < NPR; ++e)
            kpa[s][e] = lds_base(LY::kT + (((p3 >> (10 * e)) & 1023u) * TS + 8 * g) * 2);
    }
    // key-side factor of this lane's feature in update tile T (rows 4 (T / 2) + li / 4)
    _Float16 cK[4];
#pragma unroll
    for (int T = 0; T < 4; ++T)
        cK[T] = (_Float16)rt.kscale[(row_s + 8 * w + 4 * (T >> 1) + (li >> 2)) * 8 + 4 * (T & 1) + (li & 3)];

    // Resident state slice S', update-accumulator layout: lane (column 16 ct + li, g)
    // register r of tile T holds kernel feature (row 8 w + 4 (T / 2) + g, element 4 (T % 2) + r).
    f32x4v S[4][NCT];
#pragma unroll
    for (int T = 0; T < 4; ++T)
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) S[T][ct] = f32x4v{0.0f, 0.0f, 0.0f, 0.0f};
    // State I/O at the segment's ends goes through LDS, one update tile per wave at a time.
    // The slice's canonical feature index and key-side factor per kernel feature are staged
    // in LDS first; consecutive threads then take consecutive kernel features of one column
    // (mostly consecutive canonical features: few cache lines per wave), and every thread
    // issues all its loads before it writes any of them.
    constexpr int NIO = (LY::io_rows * NCL + 511) / 512, IOB = 6;
    int32_t* cf_idx = reinterpret_cast<int32_t*>(lds_raw + LY::cf);
    float* cf_fac = reinterpret_cast<float*>(lds_raw + LY::cf) + kRowsPerSlice * 8;
    // kernel feature (within the slice) of staging row fr of update tile T
    auto kf_of = [](int T, int fr) {
        const int ww = fr / 16, rho = fr % 16;
        return (8 * ww + 4 * (T >> 1) + (rho >> 2)) * 8 + 4 * (T & 1) + (rho & 3);
    };
    if (a.load_state) {
        const int fi = row_s * 8 + tid;
        cf_idx[tid] = rt.canon[fi];
        cf_fac[tid] = kfactor(rt.kscale[fi]) * kVScale;
    }
    if (a.load_state) {
        float* io = reinterpret_cast<float*>(lds_raw + LY::sb);
#pragma unroll
        for (int T = 0; T < 4; ++T) {
            __syncthreads();
            // batches of IOB loads in flight per thread
            for (int i0 = 0; i0 < NIO; i0 += IOB) {
                float vals[IOB];
#pragma unroll
                for (int i = 0; i < IOB; ++i) {
                    const int idx = tid + 512 * (i0 + i);
                    float x = 0.0f;
                    if (idx < LY::io_rows * NCL) {
                        const int j = idx / LY::io_rows, kf = kf_of(T, idx % LY::io_rows);
                        const int F = cf_idx[kf];
                        if (F >= 0) x = state[(int64_t)gcol(j) * a.M_pad + F] * cf_fac[kf];
                    }
                    vals[i] = x;
                }
#pragma unroll
                for (int i = 0; i < IOB; ++i) {
                    const int idx = tid + 512 * (i0 + i);
                    if (idx < LY::io_rows * NCL) io[(idx % LY::io_rows) * LY::IO + idx / LY::io_rows] = vals[i];
                }
            }
            __syncthreads();
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int j = 16 * ct + li;
                    S[T][ct][r] = j < NCL ? io[(w * 16 + 4 * g + r) * LY::IO + j] : 0.0f;
                }
        }
    }

    // fp16 copy of this wave's state for the readout (K-steps 2 w, 2 w + 1)
    auto store_sb = [&]() {
#pragma unroll
        for (int s = 0; s < 2; ++s)
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct) {
                const f16x8 p = pack_tiles(S[2 * s][ct], S[2 * s + 1][ct]);
                if (ct < 4) sb[(ct * KS + 2 * w + s) * 64 + lane] = p;
                else if (li == 0) sb4[(2 * w + s) * 4 + g] = p;
            }
    };
    __syncthreads();                         // staging reads done before the area is reused

    // per-lane LDS bases of the contraction's operand tables (byte addresses)
    const uint32_t a_sb = lds_base(LY::sb + lane * 16);                           // [ct][K-step][lane]
    const uint32_t a_sb4 = lds_base(LY::sb4 + g * 16);                            // [K-step][g]
    const uint32_t a_vt = lds_base(LY::vt + (li * TS + 8 * g) * 2);               // row 16 ct + li
    const uint32_t a_vt4 = lds_base(LY::vt + (64 * TS + 8 * g) * 2);              // the ones row
    const uint32_t a_kt = lds_base(LY::kT + ((8 * lb_w + (li & 3)) * TS + 8 * g) * 2);
    const uint32_t a_q = lds_base(LY::qt + (TW * w + li) * XR * 2);               // token row, tile 0
    const uint32_t a_ri = lds_base(LY::ri + g * 8);                               // row 4 s + g

    // fp16 tables of the update sub-chunk starting at chunk c from its raw k and v.  A
    // thread takes two consecutive tokens of one 16-byte slot: both raw rows are read
    // before any conversion, and each transposed table row gets 4-byte token pairs.
    auto build_tables = [&](int c) {
        const int nvalid = nupd_of(c);
        static_assert(LU == 128, "one token pair per lane");
        const int t0 = 2 * lane;                                    // this lane's tokens t0, t0 + 1
        const uint32_t m0 = t0 < nvalid ? 0xffffffffu : 0u, m1 = t0 + 1 < nvalid ? 0xffffffffu : 0u;
        constexpr int NKS = D / 8 / kWaves;                         // key slots per thread (1 or 2)
        uint4 kx[NKS][2], vx[2];
        // raw v: block 8 h + w holds columns 8 w .. 8 w + 7 of tokens 64 h + (0 .. 63)
        const uint4* rv = reinterpret_cast<const uint4*>(lds_raw + LY::rawv) + (8 * (t0 >> 6) + w) * 64 + (t0 & 63);
        vx[0] = rv[0];
        vx[1] = rv[1];
#pragma unroll
        for (int j = 0; j < NKS; ++j) {
            const int cs = w + kWaves * j;
            kx[j][0] = *reinterpret_cast<const uint4*>(rk + t0 * XR + 8 * cs);
            kx[j][1] = *reinterpret_cast<const uint4*>(rk + (t0 + 1) * XR + 8 * cs);
        }
        auto mask = [&](uint4& x, uint32_t m) { x.x &= m; x.y &= m; x.z &= m; x.w &= m; };
        mask(vx[0], m0);
        mask(vx[1], m1);
        {   // v: [column][token], scaled
            const uint32_t a0[4] = {vx[0].x, vx[0].y, vx[0].z, vx[0].w};
            const uint32_t a1[4] = {vx[1].x, vx[1].y, vx[1].z, vx[1].w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const f16x2 lo = __builtin_convertvector(f32x2{bf16_lo(a0[e]), bf16_lo(a1[e])} * kVScale, f16x2);
                const f16x2 hi = __builtin_convertvector(f32x2{bf16_hi(a0[e]), bf16_hi(a1[e])} * kVScale, f16x2);
                *reinterpret_cast<f16x2*>(vt + (8 * w + 2 * e) * TS + t0) = lo;
                *reinterpret_cast<f16x2*>(vt + (8 * w + 2 * e + 1) * TS + t0) = hi;
            }
        }
#pragma unroll
        for (int j = 0; j < NKS; ++j) {   // keys: every coordinate to [coordinate][token]
            const int cs = w + kWaves * j;
            mask(kx[j][0], m0);
            mask(kx[j][1], m1);
            const uint32_t a0[4] = {kx[j][0].x, kx[j][0].y, kx[j][0].z, kx[j][0].w};
            const uint32_t a1[4] = {kx[j][1].x, kx[j][1].y, kx[j][1].z, kx[j][1].w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const f16x2 lo = __builtin_convertvector(f32x2{bf16_lo(a0[e]), bf16_lo(a1[e])}, f16x2);
                const f16x2 hi = __builtin_convertvector(f32x2{bf16_hi(a0[e]), bf16_hi(a1[e])}, f16x2);
                *reinterpret_cast<f16x2*>(kT + (8 * cs + 2 * e) * TS + t0) = lo;
                *reinterpret_cast<f16x2*>(kT + (8 * cs + 2 * e + 1) * TS + t0) = hi;
            }
        }
        {   // the constant key coordinate d (1 for the tokens, 0 past them), then
            // coordinates d + 1 .. d + 7 (zeros): row d + w, this lane's token pair
            const _Float16 one0 = (_Float16)(w == 0 && t0 < nvalid ? 1.0f : 0.0f);
            const _Float16 one1 = (_Float16)(w == 0 && t0 + 1 < nvalid ? 1.0f : 0.0f);
            *reinterpret_cast<f16x2*>(kT + (D + w) * TS + t0) = f16x2{one0, one1};
            // the ones row of [v | 1]
            if (ONES && w == 0)
                *reinterpret_cast<f16x2*>(vt + 64 * TS + t0) =
                    f16x2{(_Float16)(t0 < nvalid ? kVScale : 0.0f), (_Float16)(t0 + 1 < nvalid ? kVScale : 0.0f)};
        }
    };

    // update S' += K^^T . [v | 1] of this wave's rows over the sub-chunk in the tables
    auto update = [&]() {
#pragma unroll
        for (int kk = 0; kk < LU / 32; ++kk) {
            f16x8 Vop[NCT], kreg[2];
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct)
                Vop[ct] = ct < 4 ? lds_at<f16x8>(lds_raw, a_vt, (16 * ct * TS + 32 * kk) * 2)
                                 : lds_at<f16x8>(lds_raw, a_vt4, 32 * kk * 2);
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) kreg[hh] = lds_at<f16x8>(lds_raw, a_kt, (4 * hh * TS + 32 * kk) * 2);
#pragma unroll
            for (int s = 0; s < 2; ++s) {
                // parent product of this lane's row for its 8 tokens
                f16x8 kp8 = lds_at<f16x8>(lds_raw, kpa[s][0], 32 * kk * 2);
#pragma unroll
                for (int e = 1; e < NPR; ++e) kp8 = kp8 * lds_at<f16x8>(lds_raw, kpa[s][e], 32 * kk * 2);
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const int T = 2 * s + h;
                    const f16x8 Au = kp8 * kreg[h] * cK[T];
#pragma unroll
                    for (int ct = 0; ct < NCT; ++ct)
                        S[T][ct] = __builtin_amdgcn_mfma_f32_16x16x32_f16(Au, Vop[ct], S[T][ct], 0, 0, 0);
                }
            }
        }
    };

    // Windows of NSUB chunks: one readout of the window's R tokens against the state
    // before the window, then the window's updates, LU tokens each.  The finalize adds
    // the direct part of the window's earlier chunks.
    for (int cw = cb; cw < ce; cw += NSUB) {
        const int nchw = ce - cw < NSUB ? ce - cw : NSUB;             // chunks of the window
        const bool next_w = cw + NSUB < ce;
        lds_barrier<0>();           // the window's q and first k, v landed; the updates are done
        if (!a.update_only) {

        // ---- fp16 state for the readout (over the previous window's tables); q to fp16 --
        store_sb();
        {
            constexpr int NQ = (R * LY::XSLOTS + 511) / 512;
            uint4 r[NQ];
#pragma unroll
            for (int i = 0; i < NQ; ++i) {
                const int sl = tid + 512 * i;
                if (sl < R * LY::XSLOTS) r[i] = reinterpret_cast<const uint4*>(lds_raw + LY::qt)[sl];
            }
#pragma unroll
            for (int i = 0; i < NQ; ++i) {
                const int sl = tid + 512 * i;
                // the constant slot is written as fp16 (1, 0, ..., 0); loads never refill it
                const f16x8 h = sl % LY::XSLOTS == D / 8 ? f16x8{1, 0, 0, 0, 0, 0, 0, 0} : bf16x8_to_f16(r[i]);
                if (sl < R * LY::XSLOTS) reinterpret_cast<f16x8*>(lds_raw + LY::qt)[sl] = h;
            }
        }
        lds_barrier<63>();

        // ---- readout: window tokens TW w .. TW w + TW - 1 over the slice's K-steps --------
        f32x4v U[MTW][NCT];
#pragma unroll
        for (int m = 0; m < MTW; ++m)
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct) U[m][ct] = f32x4v{0.0f, 0.0f, 0.0f, 0.0f};
        {
            // software-pipelined: the B operands of K-step s + 1 are requested before the
            // MFMAs of step s
            f16x8 B[2][NCT], qreg[MTW];
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct)
                B[0][ct] = ct < 4 ? lds_at<f16x8>(lds_raw, a_sb, ct * KS * 64 * 16) : lds_at<f16x8>(lds_raw, a_sb4, 0);
#pragma unroll
            for (int s = 0; s < KS; ++s) {
                if (s + 1 < KS) {
#pragma unroll
                    for (int ct = 0; ct < NCT; ++ct)
                        B[(s + 1) & 1][ct] = ct < 4 ? lds_at<f16x8>(lds_raw, a_sb, (ct * KS * 64 + (s + 1) * 64) * 16)
                                                    : lds_at<f16x8>(lds_raw, a_sb4, (s + 1) * 64);
                }
                if (s % 2 == 0) {
#pragma unroll
                    for (int m = 0; m < MTW; ++m)
                        qreg[m] = lds_at<f16x8>(lds_raw, a_q + 16u * (uint32_t)lbg[s / 2], m * 16 * XR * 2);
                }
                const uint2 rc = lds_at<uint2>(lds_raw, a_ri, s * 4 * 8);
#pragma unroll
                for (int m = 0; m < MTW; ++m) {
                    _Float16 qp = __builtin_bit_cast(_Float16, (uint16_t)rc.y);
#pragma unroll
                    for (int e = 0; e < NPC; ++e)
                        qp *= lds_at<_Float16>(lds_raw, a_q + ((rc.x >> (10 * e)) & 1023u), m * 16 * XR * 2);
                    const f16x8 A = qreg[m] * qp;
#pragma unroll
                    for (int ct = 0; ct < NCT; ++ct)
                        U[m][ct] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A, B[s & 1][ct], U[m][ct], 0, 0, 0);
                }
            }
        }
        {   // this wave's tokens lie in one chunk.  Partials in HBM, per (chunk, slice), in
            // the tiled layout (launch.h): a lane's accumulators of two adjacent column tiles
            // as one 16-byte store of fp16, so that one store instruction writes 1 KiB
            // contiguously; then the normaliser column in fp32, [token] (its lanes li = 0
            // write 16 bytes each)
            const int cs = (TW * w) / L;
            if (cs < nchw) {
                const int c = cw + cs;
                constexpr int NVP = d_V / 32;                       // value column-tile pairs of the head
                constexpr float ps = kUScale * kPartialScale;
                float* pp = a.partial + ((bh * nch + (c - a.c_begin)) * a.nslices + slice) * tiled_partial_floats(L, d_V);
                _Float16* ph = reinterpret_cast<_Float16*>(pp);
#pragma unroll
                for (int m = 0; m < MTW; ++m) {
                    const int mg = ((TW * w) % L) / 16 + m;         // token tile within the chunk
#pragma unroll
                    for (int cp = 0; cp < 2; ++cp) {
                        const f32x4v lo = U[m][2 * cp] * ps, hi = U[m][2 * cp + 1] * ps;
                        const f16x8 h = {(_Float16)lo[0], (_Float16)lo[1], (_Float16)lo[2], (_Float16)lo[3],
                                         (_Float16)hi[0], (_Float16)hi[1], (_Float16)hi[2], (_Float16)hi[3]};
                        *reinterpret_cast<f16x8*>(ph + ((mg * NVP + 2 * G + cp) * 64 + lane) * 8) = h;
                    }
                    if constexpr (ONES) {
                        if (li == 0) *reinterpret_cast<f32x4v*>(pp + L * d_V / 2 + 16 * mg + 4 * g) = U[m][NCT - 1] * kUScale;
                    }
                }
            }
        }
        lds_barrier<63>();          // every readout is done: the state copy and q are free
        if (next_w) prefetch_q(cw + NSUB);
        }   // readout

        // ---- the window's updates ----------------------------------------------------------
        for (int cu = cw; cu < cw + nchw; cu += LU / L) {
            if (cu > cw) lds_barrier<0>();    // k, v of this sub-chunk landed; the last update is done
            build_tables(cu);
            lds_barrier<63>();
            // next raw k, v: this window's next sub-chunk, or the next window's first
            if (cu + LU / L < ce) prefetch_kv(cu + LU / L);
            update();
        }
    }
    __builtin_amdgcn_s_waitcnt(0);

    if (a.store_state) {
        // through LDS as for the load; S = S' / (2^-8 c).  The window loop has reused the
        // staging area: stage the canonical indices and factors again.
        float* io = reinterpret_cast<float*>(lds_raw + LY::sb);
        __syncthreads();
        {
            const int fi = row_s * 8 + tid;
            cf_idx[tid] = rt.canon[fi];
            cf_fac[tid] = kfactor(rt.kscale[fi]) * kVScale;
        }
#pragma unroll
        for (int T = 0; T < 4; ++T) {
            __syncthreads();
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int j = 16 * ct + li;
                    if (j < LY::IO) io[(w * 16 + 4 * g + r) * LY::IO + j] = S[T][ct][r];
                }
            __syncthreads();
#pragma unroll 4
            for (int i = 0; i < NIO; ++i) {
                const int idx = tid + 512 * i;
                if (idx < LY::io_rows * NCL) {
                    const int fr = idx % LY::io_rows, j = idx / LY::io_rows, kf = kf_of(T, fr);
                    const int F = cf_idx[kf];
                    if (F >= 0) state[(int64_t)gcol(j) * a.M_pad + F] = io[fr * LY::IO + j] / cf_fac[kf];
                }
            }
        }
        if (slice == 0) {
            const int64_t padn = a.M_pad - a.M;
            for (int64_t idx = tid; idx < NCL * padn; idx += 512)
                state[(int64_t)gcol((int)(idx / padn)) * a.M_pad + a.M + idx % padn] = 0.0f;
        }
    }
}

template <int D, int DV, int G, int NPC>
hipError_t launch_t(const PrefillSegArgs& a, const MfmaTables& m, hipStream_t st) {
    using LY = Layout<D, G == 0 ? 5 : 4>;
    static_assert(LY::bytes <= 160 * 1024, "LDS budget");
    RowPtrs rt{m.parent, m.weight, m.kscale, m.canon, m.wave_lblock};
    hipError_t e = hipFuncSetAttribute((const void*)scan_mfma_kernel<D, DV, G, NPC>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, LY::bytes);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((scan_mfma_kernel<D, DV, G, NPC>), dim3(a.nslices, a.BH * a.nsub), dim3(512), LY::bytes,
                       st, a, rt);
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
    const size_t bytes = nr * 4 + nr * 4 + nr * 8 * 4 + nr * 8 * 4 + nw * 4;
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
    m.parent = (const uint32_t*)put(r.parent.data(), nr * 4);
    m.weight = (const float*)put(r.weight.data(), nr * 4);
    m.kscale = (const float*)put(r.kscale.data(), nr * 8 * 4);
    m.canon = (const int32_t*)put(r.canon.data(), nr * 8 * 4);
    m.wave_lblock = (const int32_t*)put(r.wave_lblock.data(), nw * 4);
    m.d_rows = base;
    if (!m.parent || !m.weight || !m.kscale || !m.canon || !m.wave_lblock) {
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

namespace {
__global__ __launch_bounds__(kThreads) void state_prefix_kernel(float* __restrict__ states, const float* __restrict__ init,
                                                                float* __restrict__ final, int nsub, int64_t per_state) {
    const int64_t bh = blockIdx.y;
    const int64_t e = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    if (e >= per_state) return;
    float acc = init ? init[bh * per_state + e] : 0.0f;
    float* s = states + bh * nsub * per_state + e;
    for (int i = 0; i < nsub; ++i) {
        const float x = s[i * per_state];
        s[i * per_state] = acc;
        acc += x;
    }
    if (final) final[bh * per_state + e] = acc;
}
}  // namespace

hipError_t launch_state_prefix(float* states, const float* init, float* final, int BH, int nsub,
                               int64_t per_state, hipStream_t st) {
    dim3 grid((unsigned)((per_state + kThreads - 1) / kThreads), (unsigned)BH);
    hipLaunchKernelGGL(state_prefix_kernel, grid, dim3(kThreads), 0, st, states, init, final, nsub, per_state);
    return hipGetLastError();
}

int mfma_window(int d_K) { return d_K == 64 ? Layout<64, 5>::NSUB : Layout<128, 5>::NSUB; }

bool mfma_shape(bool bf16, int d_K, int d_V, int P, int L) {
    return bf16 && P >= 2 && P <= 5 && (d_V == 64 || d_V == 128) && (d_K == 64 || d_K == 128) && L == kL;
}

bool mfma_supported(const MfmaTables& m, bool bf16, int d_K, int d_V, int P, int L) {
    return m.ok && d_K == m.d_K && P == m.P && mfma_shape(bf16, d_K, d_V, P, L);
}

int mfma_slice_count(const HostTables& h) {
    MfmaHostRows r;
    if (!build_mfma_rows(h, r)) return 0;
    return r.nrows / kRowsPerSlice;
}

hipError_t launch_scan_mfma(const PrefillSegArgs& a, const MfmaTables& m, hipStream_t st) {
    return a.d_K == 128 ? launch_d<128>(a, m, st) : launch_d<64>(a, m, st);
}

}  // namespace sata
