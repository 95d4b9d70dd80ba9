// kern_scan_mfma.hip -- MFMA chunked prefill scan for gfx950 (fp16 operands, fp32 state).
//
// The inter-chunk half of the chunked prefill ([TA] "Feature maps and linear
// attention": the state recurrence, evaluated chunk by chunk):
//     readout   part[t][j] = sum_f qw_f phi_f(q_t) S[f][j]      (S before the window)
//     update    S[f][j]   += sum_t phi_f(k_t) u_t[j],   u_t = [v_t | 1]
// The readout is taken once per window of R tokens (256 at d_K = 64, 128 at d_K = 128)
// against the state before the window; the finalize adds the direct part of the window's
// earlier chunks.  The update runs per 128-token sub-chunk.  Both are dense contractions
// over tokens and a slice of the feature axis, run as v_mfma_f32_16x16x32_f16 with fp32
// accumulation:
//     readout  (16 tokens x 32 features) x (32 features x 16 columns)
//     update   (16 features x 32 tokens) x (32 tokens x 16 columns)
//
// Operands are fp16, built from the operand images of the prep kernels (kern_prep.hip):
// q' = q 2^-s_q, k' = k 2^-s_k, v' = v 2^-s_v with per-head powers of two that put each
// input's maximum in [1, 2).  gfx950 multiplies fp16 pairs in one VALU instruction (bf16 only
// one value at a time), and operand building competes with the matrix pipe for issue slots;
// the matrix rate of the two types is the same.  The scales are folded back exactly:
//   query operand  (W'_a q'_a) q'_l with W'_a = W_a 2^(p (s_q + s_k) - e_q), p the degree
//                  and e_q per head, so that every operand stays below 2^14;
//   state          S'' = c 2^(-p s_k) [S 2^-s_v | Z] in fp32 registers (c the key factor);
//   readout copy   S'' 2^-e_w in fp16, e_w per window from the slice's largest entry;
// so the readout accumulates (q~ . S) 2^-(e_q + e_w) (value columns also 2^-s_v), and each
// 16-token tile of the stored partials gets its own power-of-two scale.  No finite input
// overflows fp16 anywhere; precision is that of the fp16 operands (2^-11 relative).
//
// Work split.  The columns of [v | 1] are cut into groups of 64 value columns; group 0
// also carries the normaliser column (65 columns, 5 tiles of 16), the others 4 tiles.  One
// workgroup of 8 waves (two per SIMD, so that one wave's waits overlap the other's matrix
// work) owns one slice of 64 rows = 512 kernel features of one head for one column group,
// and walks all chunks of the segment in order.  Wave w owns rows 8w .. 8w+7: kernel
// features (parent a, l = 8b + e), e = 0..7, with one l-block b per wave (mfma_rows.cpp);
// its fp32 state never leaves the registers (4 update tiles x 5 column tiles x 4 = 80
// registers).  Feature tiles are never written to HBM: per contraction step the operands
// are built as
//     query side  q^(a, l)[t] = (W'_a q'_a[t]) * q'_l[t]
//     key side    k^(a, l)[t] = kpar_a[t] * k'_l[t] * c_(a,l)    (c: 0 / 1/(1+m) / 1)
// directly in the MFMA operand layout (q'_a, kpar_a: parent products).
//
// The readout is split by tokens: wave w computes R / 8 tokens of the window over all 512
// features of the slice, so the slice's partial readout leaves the registers straight to
// HBM with no exchange between waves.  Its B operand, the state packed to fp16 after the
// previous window's last update, is shared through LDS: the update's accumulator layout
// (lane = column, 4 rows each) over two tiles is a 32-deep B operand when the query operand
// uses the same feature order.
//
// Per window (the images arrive by direct-to-LDS loads, 1 KiB per wave instruction):
//     B1  q rows of the window landed; fp16 state copy written
//         readout, partial stores
//     B2  readout done (state copy and q rows free); tables of update 0 landed
//         load: tables of update 1 (over the state copy), next window's q rows
//         update 0
//     B3  update 0 done; tables of update 1 landed      (d_K = 64: two updates per window)
//         load: next window's tables of update 0
//         update 1
//     B4  updates done; per-wave state maxima posted
//         fp16 state copy of the next window
// so the barriers wait for LDS work only; every image load is issued a phase ahead.
#include "scan_mfma.h"

#include <hip/hip_runtime.h>

#include <type_traits>

namespace sata {

namespace {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4v __attribute__((ext_vector_type(4)));

constexpr int kWaves = kWavesPerSlice;      // 8 waves, 8 rows each
constexpr int kL = 64;                      // chunk length (partials, finalize)
constexpr int kLU = kImgLU;                 // tokens per state update

template <int D, int NCT>
struct Layout {
    static constexpr int L = kL;
    static constexpr int LU = kLU;
    static constexpr int R = img_window(D);          // readout window (tokens)
    static constexpr int NSUB = R / L;               // chunks per window
    static constexpr int NUPD = R / LU;              // updates per window
    static constexpr int TW = R / kWaves;            // readout tokens per wave (32 or 16)
    static constexpr int MTW = TW / 16;              // readout token tiles per wave
    static constexpr int KS = kRowsPerSlice / 4;     // readout K-steps (32 features each)
    static constexpr int XR = img_xr(D);             // q/k row: D coords, the constant 1, 7 zeros
    static constexpr int TS = img_ts();              // token-major row stride of the tables
    static constexpr int KTB = img_kt_bytes(D), VTB = img_vt_bytes(), TABB = KTB + VTB;
    static constexpr int QB = img_q_bytes(D);
    // LDS
    static constexpr int t1 = 0;                                    // update tables 1: keys, values
    static constexpr int sb = TABB;                                 // fp16 state: [4 ct][KS][64 lanes] x 16 B
    static constexpr int sb4 = sb + 4 * KS * 64 * 16;               // normaliser tile: [KS][4 g] x 16 B
    static constexpr int sb_end = sb4 + (NCT == 5 ? KS * 4 * 16 : 0);
    static constexpr int t2 = sb;                                   // update tables 2, over the state copy
    static constexpr int qt = sb_end;                               // the window's q rows [R][XR]
    static constexpr int ri = qt + QB;                              // [64 rows] readout row constants
    static constexpr int wmx = ri + kRowsPerSlice * 8;              // [8] per-wave state maxima
    static constexpr int bytes = wmx + kWaves * 4;
    // state load/store staging at the segment's ends (over the state copy)
    static constexpr int IO = 68;                                   // floats per feature row
    static constexpr int io_rows = kWaves * 16;                     // one tile per wave per phase
    static constexpr int cf = sb + io_rows * IO * 4;                // [512] canonical index, [512] factor
    static_assert(cf + kRowsPerSlice * 8 * 8 <= sb + 4 * KS * 64 * 16, "state staging size");
    static_assert(NUPD == 1 || TABB <= 4 * KS * 64 * 16, "second table buffer inside the state copy");
    // the second buffer is addressed from the first one's lane bases: its largest constant
    // offset must fit the 16-bit offset field of ds_read
    static_assert(NUPD == 1 || t2 - t1 + (3 * 16 * TS + 96) * 2 < 65536, "table offsets");
    static_assert(QB % 1024 == 0 && TABB % 1024 == 0 && KTB % 1024 == 0 && qt % 16 == 0 && ri % 16 == 0,
                  "whole DMA blocks, 16-byte alignment");
    static_assert(TW % 16 == 0 && L % TW == 0 && KS == 16 && R % LU == 0 && (NUPD == 1 || NUPD == 2), "tiling");
};

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

// Workgroup barrier for the window loop: this wave's LDS accesses have completed and
// at most VM of its vector-memory operations are still outstanding (63: no wait).
// Unlike __syncthreads() it does not wait for outstanding loads or stores unless VM asks
// for it (they complete in order on this architecture).
template <int VM>
__device__ inline void lds_barrier() {
    static_assert(VM >= 0 && VM <= 63, "vmcnt range");
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt((VM & 15) | (7 << 4) | (0 << 8) | ((VM >> 4) << 14));
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// Direct-to-LDS copy of NB KiB blocks: wave w moves blocks w, w + 8, ...; lane i fills
// bytes [16 i, 16 i + 16) of its block.  Source and destination are whole blocks.
template <int NB>
__device__ inline void dma_blocks(const uint16_t* src, unsigned char* dst, int w, int lane) {
    for (int blk = w; blk < NB; blk += kWaves)
        __builtin_amdgcn_global_load_lds((const void*)(src + blk * 512 + lane * 8),
                                         (void __attribute__((address_space(3)))*)(dst + blk * 1024), 16, 0, 0);
}
// the fewest blocks any wave moves in dma_blocks<NB> (for counted waits)
template <int NB>
constexpr int dma_min_per_wave() { return NB / kWaves; }

// DPP lane exchange of a float (CTRL is the DPP control word)
template <int CTRL>
__device__ inline float dpp_f(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xf, 0xf, false));
}
// largest value over a wave (non-negative inputs), in every lane: DPP within rows of 16
// lanes (quad swaps, then the half-row and row mirrors), then the four row results read
// out to scalars (no LDS round trip)
__device__ inline float wave_max(float x) {
    x = fmaxf(x, dpp_f<0xB1>(x));      // quad_perm [1,0,3,2]
    x = fmaxf(x, dpp_f<0x4E>(x));      // quad_perm [2,3,0,1]
    x = fmaxf(x, dpp_f<0x141>(x));     // row_half_mirror
    x = fmaxf(x, dpp_f<0x140>(x));     // row_mirror
    const int b = __float_as_int(x);
    return fmaxf(fmaxf(__int_as_float(__builtin_amdgcn_readlane(b, 0)), __int_as_float(__builtin_amdgcn_readlane(b, 16))),
                 fmaxf(__int_as_float(__builtin_amdgcn_readlane(b, 32)), __int_as_float(__builtin_amdgcn_readlane(b, 48))));
}

// floor(log2 x) of a positive normal float from its bits; clamped to [lo, hi]
__device__ inline int exp2_of(float x, int lo, int hi) {
    const int e = (int)((__float_as_uint(x) >> 23) & 0xffu) - 127;
    return e < lo ? lo : (e > hi ? hi : e);
}

struct RowPtrs {
    const uint32_t* parent;
    const float* weight;
    const float* kscale;
    const int32_t* canon;
    const int32_t* wave_lblock;
    const int8_t* degree;
    int wlog[8];
};

template <int D, int DV, int G, int NPC>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
void scan_mfma_kernel(PrefillSegArgs a, RowPtrs rt) {
    constexpr bool ONES = G == 0;            // group 0 carries the normaliser column
    constexpr int col0 = 64 * G;             // first value column of the group
    constexpr int NCT = ONES ? 5 : 4;        // column tiles of this group
    constexpr int NCL = ONES ? 65 : 64;      // live columns of this group
    constexpr int NG = DV / 64;              // column groups of the head
    using LY = Layout<D, NCT>;
    constexpr int L = kL, LU = LY::LU, TS = LY::TS, NSUB = LY::NSUB, TW = LY::TW;
    constexpr int XR = LY::XR, MTW = LY::MTW, KS = LY::KS, NUPD = LY::NUPD;
    constexpr int NB_Q = LY::QB / 1024;
    extern __shared__ __align__(16) unsigned char lds_raw[];
    f16x8* sb = reinterpret_cast<f16x8*>(lds_raw + LY::sb);
    f16x8* sb4 = reinterpret_cast<f16x8*>(lds_raw + LY::sb4);
    float* wmx = reinterpret_cast<float*>(lds_raw + LY::wmx);

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int g = lane >> 4, li = lane & 15;
    const int wu = __builtin_amdgcn_readfirstlane(w);        // the wave index, known uniform
    const int slice = blockIdx.x;
    const int64_t bh = blockIdx.y / a.nsub;
    const int sub = blockIdx.y % a.nsub;
    constexpr int d_V = DV;
    const int nch = a.c_end - a.c_begin;       // chunks of the partial buffer
    // the chunks this block scans: its sub-segment (the whole range when nsub = 1)
    const int cb = a.c_begin + sub * a.sub_chunks;
    const int ce = a.nsub > 1 && cb + a.sub_chunks < a.c_end ? cb + a.sub_chunks : a.c_end;
    const int row_s = slice * kRowsPerSlice;                 // first row of the slice
    const int lb_w = rt.wave_lblock[slice * kWaves + w];     // l-block of this wave's update rows
    // global column of local column j of this group (local 64 is the normaliser)
    auto gcol = [&](int j) { return (ONES && j == 64) ? d_V : col0 + j; };
    float* state = a.state ? a.state + (bh * a.nsub + sub) * (int64_t)(DV + 1) * a.M_pad : nullptr;
    // where the end state goes: this block's own slot, or (final_state) the final state from
    // the blocks of the last sub-segment alone
    float* sdst = a.final_state ? (sub == a.nsub - 1 ? a.final_state + bh * (int64_t)(DV + 1) * a.M_pad : nullptr)
                                : state;

    // per-head exponents of the input scales and of the query weights
    const int s_q = prep_scale_exp(a.maxbits[bh * 4 + 0]);
    const int s_k = prep_scale_exp(a.maxbits[bh * 4 + 1]);
    const int s_v = prep_scale_exp(a.maxbits[bh * 4 + 2]);
    int e_q = -1000;
    for (int p = 0; p < a.P; ++p) {
        const int e = rt.wlog[p] + p * (s_q + s_k + 1);
        e_q = e > e_q ? e : e_q;
    }
    e_q -= 14;

    // operand images of this head (windows and sub-chunks relative to the images' first)
    const uint16_t* qimg = a.qimg + bh * (int64_t)a.img_nwin * (LY::QB / 2);
    const uint16_t* kimg = a.kimg + bh * (int64_t)a.img_nsub * (LY::KTB / 2);
    const uint16_t* vimg = a.vimg + (bh * NG + G) * (int64_t)a.img_nsub * (LY::VTB / 2);
    auto dma_q = [&](int cw) {               // q rows of the window starting at chunk cw
        dma_blocks<NB_Q>(qimg + (int64_t)(cw / NSUB - a.img_w0) * (LY::QB / 2), lds_raw + LY::qt, wu, lane);
    };
    auto dma_tables = [&](int cu, int buf) {  // tables of the update sub-chunk starting at chunk cu
        const int64_t u = (int64_t)cu * L / LU - a.img_u0;
        unsigned char* dst = lds_raw + (buf == 0 ? LY::t1 : LY::t2);
        dma_blocks<LY::KTB / 1024>(kimg + u * (LY::KTB / 2), dst, wu, lane);
        dma_blocks<LY::VTB / 1024>(vimg + u * (LY::VTB / 2), dst + LY::KTB, wu, lane);
    };
    // the first window's q rows and first tables in flight while the state is set up
    if (!a.update_only) dma_q(cb);
    dma_tables(cb, 0);

    // readout constants of the slice's rows (K-step s covers rows 4 s .. 4 s + 3, lane group
    // g row 4 s + g), in LDS: the parent coordinates as byte offsets in a q row (10 bits
    // each) and the query weight W'_a (fp16 bits)
    if (tid < kRowsPerSlice) {
        const int row = row_s + tid;
        const uint32_t p3 = rt.parent[row];
        uint32_t o = 0;
#pragma unroll
        for (int e = 0; e < NPC; ++e) o |= (((p3 >> (10 * e)) & 1023u) * 2u) << (10 * e);
        const int p = rt.degree[row];
        const _Float16 wq = (_Float16)ldexpf(rt.weight[row], p * (s_q + s_k) - e_q);
        reinterpret_cast<uint2*>(lds_raw + LY::ri)[tid] = uint2{o, (uint32_t)__builtin_bit_cast(uint16_t, wq)};
    }
    // l-blocks of the slice's row octets (uniform)
    int lbg[KS / 2];
#pragma unroll
    for (int gi = 0; gi < KS / 2; ++gi) lbg[gi] = __builtin_amdgcn_readfirstlane(rt.wave_lblock[slice * kWaves + gi]);
    // key parents of this lane's update rows 8 w + 4 s + li / 4: byte offsets of their
    // coordinate rows in the key table (a missing parent is the constant coordinate d,
    // which is 1 for the tokens that exist and 0 past them)
    constexpr int NPR = NPC > 0 ? NPC : 1;
    uint32_t kpa[2][NPR];
#pragma unroll
    for (int s = 0; s < 2; ++s) {
        const uint32_t p3 = rt.parent[row_s + 8 * w + 4 * s + (li >> 2)];
#pragma unroll
        for (int e = 0; e < NPR; ++e)
            kpa[s][e] = lds_base(LY::t1 + (((p3 >> (10 * e)) & 1023u) * TS + 8 * g) * 2);
    }
    // key-side factors c (0 / 1/(1+m) / 1) of the 8 features of this lane's rows 8 w + 4 s + g,
    // in the order of its fp16 state copy (the update accumulates the plain products; the
    // factor enters once per window, with the copy)
    f16x8 cf8[2];
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
        for (int e = 0; e < 8; ++e) cf8[s][e] = (_Float16)rt.kscale[(row_s + 8 * w + 4 * s + g) * 8 + e];

    // Resident state slice S'', update-accumulator layout: lane (column 16 ct + li, g)
    // register r of tile T holds kernel feature (row 8 w + 4 (T / 2) + g, element 4 (T % 2) + r).
    f32x4v S[4][NCT];
#pragma unroll
    for (int T = 0; T < 4; ++T)
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) S[T][ct] = f32x4v{0.0f, 0.0f, 0.0f, 0.0f};

    // State I/O at the segment's ends goes through LDS, one update tile per wave at a time.
    // The slice's canonical feature index and the factor S'' / S per kernel feature are
    // staged in LDS first; consecutive threads then take consecutive kernel features of one
    // column (mostly consecutive canonical features: few cache lines per wave), and every
    // thread keeps several loads in flight.
    constexpr int NIO = (LY::io_rows * NCL + 511) / 512, IOB = 6;
    int32_t* cf_idx = reinterpret_cast<int32_t*>(lds_raw + LY::cf);
    float* cf_fac = reinterpret_cast<float*>(lds_raw + LY::cf) + kRowsPerSlice * 8;
    const float vfac = ldexpf(1.0f, -s_v);
    // S'' / S of local column j: the value scale (the normaliser has none)
    auto colfac = [&](int j) { return (ONES && j == 64) ? 1.0f : vfac; };
    auto stage_canon = [&]() {
        const int fi = row_s * 8 + tid;
        cf_idx[tid] = rt.canon[fi];
        cf_fac[tid] = ldexpf(1.0f, -(int)rt.degree[row_s + (tid >> 3)] * s_k);
    };
    // kernel feature (within the slice) of staging row fr of update tile T
    auto kf_of = [](int T, int fr) {
        const int ww = fr / 16, rho = fr % 16;
        return (8 * ww + 4 * (T >> 1) + (rho >> 2)) * 8 + 4 * (T & 1) + (rho & 3);
    };
    if (a.load_state) {
        stage_canon();
        float* io = reinterpret_cast<float*>(lds_raw + LY::sb);
#pragma unroll
        for (int T = 0; T < 4; ++T) {
            __syncthreads();
            for (int i0 = 0; i0 < NIO; i0 += IOB) {
                float vals[IOB];
#pragma unroll
                for (int i = 0; i < IOB; ++i) {
                    const int idx = tid + 512 * (i0 + i);
                    float x = 0.0f;
                    if (idx < LY::io_rows * NCL) {
                        const int j = idx / LY::io_rows, kf = kf_of(T, idx % LY::io_rows);
                        const int F = cf_idx[kf];
                        if (F >= 0) x = state[(int64_t)gcol(j) * a.M_pad + F] * (cf_fac[kf] * colfac(j));
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
    __syncthreads();                         // staging reads done before the area is reused

    // per-lane LDS bases of the contraction's operand tables (byte addresses); the second
    // table buffer is reached from the first one's bases by a constant offset
    constexpr uint32_t T2OFF = (uint32_t)(LY::t2 - LY::t1);
    const uint32_t a_sb = lds_base(LY::sb + lane * 16);                           // [ct][K-step][lane]
    const uint32_t a_sb4 = lds_base(LY::sb4 + g * 16);                            // [K-step][g]
    const uint32_t a_vt = lds_base(LY::t1 + LY::KTB + (li * TS + 8 * g) * 2);    // row 16 ct + li
    // B operand of the normaliser's tile: u = 1 in column 0 for every token (the key operand is
    // zero for tokens past the sequence)
    const _Float16 one_h = li == 0 ? (_Float16)1.0f : (_Float16)0.0f;
    const f16x8 ones_op = {one_h, one_h, one_h, one_h, one_h, one_h, one_h, one_h};
    const uint32_t a_kt = lds_base(LY::t1 + ((8 * lb_w + (li & 3)) * TS + 8 * g) * 2);
    const uint32_t a_q = lds_base(LY::qt + (TW * w + li) * XR * 2);               // token row, tile 0
    const uint32_t a_ri = lds_base(LY::ri + g * 8);                               // row 4 s + g

    // fp16 copy c S'' 2^-e_w of this wave's state for the readout (K-steps 2 w, 2 w + 1)
    auto store_sb = [&](int e_w) {
        const float f = ldexpf(1.0f, -e_w);
#pragma unroll
        for (int s = 0; s < 2; ++s)
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct) {
                const f32x4v lo = S[2 * s][ct] * f, hi = S[2 * s + 1][ct] * f;
                const f16x8 p = f16x8{(_Float16)lo[0], (_Float16)lo[1], (_Float16)lo[2], (_Float16)lo[3],
                                      (_Float16)hi[0], (_Float16)hi[1], (_Float16)hi[2], (_Float16)hi[3]} * cf8[s];
                if (ct < 4) sb[(ct * KS + 2 * w + s) * 64 + lane] = p;
                else if (li == 0) sb4[(2 * w + s) * 4 + g] = p;
            }
    };

    // update S'' += K^^T . [v' | 1] of this wave's rows over the sub-chunk in table buffer TB;
    // after each 32-token step, hook(kk) (other work to interleave with the matrix pipe)
    auto update = [&](auto TBc, auto hook) {
        constexpr uint32_t TO = decltype(TBc)::value ? T2OFF : 0u;
#pragma unroll
        for (int kk = 0; kk < LU / 32; ++kk) {
            f16x8 Vop[NCT], kreg[2];
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct)
                Vop[ct] = ct < 4 ? lds_at<f16x8>(lds_raw, a_vt, TO + (16 * ct * TS + 32 * kk) * 2) : ones_op;
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) kreg[hh] = lds_at<f16x8>(lds_raw, a_kt, TO + (4 * hh * TS + 32 * kk) * 2);
#pragma unroll
            for (int s = 0; s < 2; ++s) {
                // parent product of this lane's row for its 8 tokens
                f16x8 kp8 = lds_at<f16x8>(lds_raw, kpa[s][0], TO + 32 * kk * 2);
#pragma unroll
                for (int e = 1; e < NPR; ++e) kp8 = kp8 * lds_at<f16x8>(lds_raw, kpa[s][e], TO + 32 * kk * 2);
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const int T = 2 * s + h;
                    const f16x8 Au = kp8 * kreg[h];
#pragma unroll
                    for (int ct = 0; ct < NCT; ++ct)
                        S[T][ct] = __builtin_amdgcn_mfma_f32_16x16x32_f16(Au, Vop[ct], S[T][ct], 0, 0, 0);
                }
            }
            hook(kk);
        }
    };

    // largest |S''| over the slice: every wave posts its own, read after the next barrier
    auto post_max = [&]() {
        float m = 0.0f;
#pragma unroll
        for (int T = 0; T < 4; ++T)
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
                for (int r = 0; r < 4; ++r) m = fmaxf(m, fabsf(S[T][ct][r]));
        m = wave_max(m);
        if (lane == 0) wmx[w] = m;
    };
    auto slice_max = [&]() {
        float m = 0.0f;
#pragma unroll
        for (int i = 0; i < kWaves; ++i) m = fmaxf(m, wmx[i]);
        return m;
    };
    // exponent of the readout's fp16 state copy: c S'' 2^-e stays below 2^15 for |S''| <= bound
    auto copy_exp = [](float bound) { return bound > 0.0f ? exp2_of(bound, -100, 126) - 14 : 0; };
    // One window's updates add at most R 2^P to any |S''| (|k'|, |v'| < 2, products of P - 1
    // key coordinates), so the next copy's exponent is fixed from the state before the window
    // (measured during the readout, off the path between the updates and the next readout).
    constexpr float kGrowth = (float)LY::R * 32.0f;      // R 2^P for P <= 5

    // the fp16 state copy of the first window: exponent from the exact maximum
    int e_w = 0, e_next = 0;
    if (!a.update_only) {
        post_max();
        __syncthreads();
        e_w = copy_exp(slice_max());
        store_sb(e_w);
    }

    // Windows of NSUB chunks: one readout of the window's R tokens against the state
    // before the window, then the window's updates, LU tokens each.  The finalize adds
    // the direct part of the window's earlier chunks.
    for (int cw = cb; cw < ce; cw += NSUB) {
        const int nchw = ce - cw < NSUB ? ce - cw : NSUB;             // chunks of the window
        const bool next_w = cw + NSUB < ce;
        // B1: the window's q rows landed (only the next tables may still be in flight)
        lds_barrier<dma_min_per_wave<LY::KTB / 1024>() + dma_min_per_wave<LY::VTB / 1024>()>();
        f32x4v U[MTW][NCT];
        const int cs = (TW * w) / L;                                  // this wave's chunk in the window
        const bool stores = !a.update_only && cs < nchw;
        if (!a.update_only) {
            // ---- readout: window tokens TW w .. TW w + TW - 1 over the slice's K-steps ----
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
            // the state before this window, for the next copy's exponent (behind the MFMAs)
            if (next_w) post_max();
        }
        // B2: every readout is done (state copy and q rows free); the first update's tables
        // landed; every wave's state maximum is posted
        lds_barrier<0>();
        if (!a.update_only && next_w) e_next = copy_exp(slice_max() + kGrowth);
        const int cu1 = cw + LU / L;                                  // the window's second update sub-chunk
        const bool upd1 = NUPD == 2 && cu1 < cw + nchw;
        // the second update's tables and the next window's q rows are requested from inside
        // the first update (steps 0 and 2), behind its matrix work

        // Partials in HBM, per (chunk, slice), in the tiled layout (launch.h), written while
        // the first update runs: per 16-token tile a power-of-two scale from the tile's largest
        // value; a lane's accumulators of two adjacent column tiles as one 16-byte store of fp16
        // (one store instruction writes 1 KiB contiguously); the normaliser column in fp32,
        // [token]; the tile's scale.  This wave's tokens lie in one chunk.
        auto store_tile = [&](int m) {
            constexpr int NVP = d_V / 32;                       // value column-tile pairs of the head
            const int c = cw + cs;
            float* pp = a.partial + ((bh * nch + (c - a.c_begin)) * a.nslices + slice) * tiled_partial_floats(L, d_V);
            _Float16* ph = reinterpret_cast<_Float16*>(pp);
            const int mg = ((TW * w) % L) / 16 + m;             // token tile within the chunk
            float mx = 0.0f;
#pragma unroll
            for (int ct = 0; ct < 4; ++ct)
#pragma unroll
                for (int r = 0; r < 4; ++r) mx = fmaxf(mx, fabsf(U[m][ct][r]));
            mx = wave_max(mx);
            const int ex = mx > 0.0f ? exp2_of(mx, -110, 126) : 0;
            const float mul = ldexpf(1.0f, 14 - ex);
#pragma unroll
            for (int cp = 0; cp < 2; ++cp) {
                const f32x4v lo = U[m][2 * cp] * mul, hi = U[m][2 * cp + 1] * mul;
                const f16x8 h = {(_Float16)lo[0], (_Float16)lo[1], (_Float16)lo[2], (_Float16)lo[3],
                                 (_Float16)hi[0], (_Float16)hi[1], (_Float16)hi[2], (_Float16)hi[3]};
                *reinterpret_cast<f16x8*>(ph + ((mg * NVP + 2 * G + cp) * 64 + lane) * 8) = h;
            }
            if constexpr (ONES) {
                if (li == 0)
                    *reinterpret_cast<f32x4v*>(pp + L * d_V / 2 + 16 * mg + 4 * g) = U[m][NCT - 1] * ldexpf(1.0f, e_q + e_w);
            }
            if (lane == 0) pp[L * d_V / 2 + L + mg * NG + G] = mx > 0.0f ? ldexpf(1.0f, ex - 14 + e_q + e_w) : 0.0f;
        };
        update(std::integral_constant<bool, false>(), [&](int kk) {
            if (kk == 0 && upd1) dma_tables(cu1, 1);
            if (kk == 2 && next_w && !a.update_only) dma_q(cw + NSUB);
            // token tile m's stores after 32-token step 2 m + 1 of the first update
            if (stores && (kk & 1) && kk / 2 < MTW) store_tile(kk / 2);
        });
        if constexpr (MTW > LU / 64) {
            if (stores)
#pragma unroll
                for (int m = LU / 64; m < MTW; ++m) store_tile(m);
        }
        if constexpr (NUPD == 2) {
            if (upd1) {
                // B3: the first update is done (its tables are free); the second's landed:
                // only this wave's partial stores and the next window's q rows, both issued
                // after them, may be outstanding
                const bool q_out = next_w && !a.update_only;
                if (q_out && stores) lds_barrier<dma_min_per_wave<NB_Q>() + 2 * MTW>();
                else if (q_out) lds_barrier<dma_min_per_wave<NB_Q>()>();
                else if (stores) lds_barrier<2 * MTW>();
                else lds_barrier<0>();
                if (next_w) dma_tables(cw + NSUB, 0);
                update(std::integral_constant<bool, true>(), [](int) {});
            } else if (next_w) {
                lds_barrier<63>();
                dma_tables(cw + NSUB, 0);
            }
        }
        // B4: the window's updates are done (the state copy's area is free)
        lds_barrier<63>();
        if constexpr (NUPD == 1) {
            if (next_w) dma_tables(cw + NSUB, 0);
        }
        if (!a.update_only && next_w) {
            e_w = e_next;
            store_sb(e_w);
        }
    }
    __builtin_amdgcn_s_waitcnt(0);

    if (a.store_state && sdst) {
        // through LDS as for the load; S = S'' / factor.  The window loop has reused the
        // staging area: stage the canonical indices and factors again.
        float* io = reinterpret_cast<float*>(lds_raw + LY::sb);
        __syncthreads();
        stage_canon();
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
                    if (F >= 0) sdst[(int64_t)gcol(j) * a.M_pad + F] = io[fr * LY::IO + j] / (cf_fac[kf] * colfac(j));
                }
            }
        }
        if (slice == 0) {
            const int64_t padn = a.M_pad - a.M;
            for (int64_t idx = tid; idx < NCL * padn; idx += 512)
                sdst[(int64_t)gcol((int)(idx / padn)) * a.M_pad + a.M + idx % padn] = 0.0f;
        }
    }
}

template <int D, int DV, int G, int NPC>
hipError_t launch_t(const PrefillSegArgs& a, const MfmaTables& m, hipStream_t st) {
    using LY = Layout<D, G == 0 ? 5 : 4>;
    static_assert(LY::bytes <= 160 * 1024, "LDS budget");
    RowPtrs rt{m.parent, m.weight, m.kscale, m.canon, m.wave_lblock, m.degree, {0}};
    for (int p = 0; p < 8; ++p) rt.wlog[p] = m.wlog[p];
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
    const size_t bytes = nr * 4 + nr * 4 + nr * 8 * 4 + nr * 8 * 4 + nw * 4 + nr;
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
    m.degree = (const int8_t*)put(r.degree.data(), nr);
    for (int p = 0; p < 8; ++p) m.wlog[p] = r.wlog[p];
    m.d_rows = base;
    if (!m.parent || !m.weight || !m.kscale || !m.canon || !m.wave_lblock || !m.degree) {
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
__global__ __launch_bounds__(kThreads) void state_starts_kernel(const float* __restrict__ pieces,
                                                                const float* __restrict__ init,
                                                                float* __restrict__ starts, int nsub,
                                                                int pps, int64_t per_state) {
    const int64_t bh = blockIdx.y;
    const int64_t e = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    if (e >= per_state) return;
    float acc = init ? init[bh * per_state + e] : 0.0f;
    const float* p = pieces + bh * (int64_t)(nsub - 1) * pps * per_state + e;
    float* s = starts + bh * nsub * per_state + e;
    for (int i = 0; i < nsub; ++i) {
        s[i * per_state] = acc;
        if (i + 1 < nsub)
            for (int j = 0; j < pps; ++j) acc += p[(int64_t)(i * pps + j) * per_state];
    }
}
}  // namespace

hipError_t launch_state_starts(const float* pieces, const float* init, float* starts, int BH, int nsub,
                               int pieces_per_sub, int64_t per_state, hipStream_t st) {
    dim3 grid((unsigned)((per_state + kThreads - 1) / kThreads), (unsigned)BH);
    hipLaunchKernelGGL(state_starts_kernel, grid, dim3(kThreads), 0, st, pieces, init, starts, nsub,
                       pieces_per_sub, per_state);
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
