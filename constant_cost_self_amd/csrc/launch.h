// launch.h -- host-side launchers of the SATA kernels (internal to libsata).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "sata_common.h"

namespace sata {

struct DecodeArgs {
    float* state;
    const void* q;
    const void* k;
    const void* v;
    float* y;
    const uint32_t* fidx;
    const float* qw;
    float* partial;     // workspace: decode_partial_floats(BH, d_V, M_pad) floats
    int64_t M, M_pad;
    int BH, d_K, d_V, P, nblk;
    bool bf16;
    // pool form: batch entry b = bh / H uses state slot slots[b] of `pool` slots (device
    // array); NULL: entry bh uses state bh
    const int32_t* slots;
    int64_t pool;
    int H;
};

// Number of feature blocks per head of the decode kernel.
int decode_blocks(int64_t M_pad);
// Floats of decode workspace (per-wave partial readouts) for BH heads.
int64_t decode_partial_floats(int BH, int d_V, int64_t M_pad);
hipError_t launch_decode(const DecodeArgs& a, hipStream_t st);         // state RMW + partials
// Bytes of the fixed device scratch of the allocation-free decode step, and its device
// address on `device` (the current device; taken once per device, no allocation).
constexpr int64_t kNoAllocScratchBytes = 16LL << 20;
hipError_t noalloc_scratch(int device, float** ptr);
hipError_t launch_decode_reduce(const DecodeArgs& a, hipStream_t st);  // partials -> y

// The state in half precision (kern_state16.hip).  Compact layout of one head, each part
// starting on a multiple of 256 bytes:
//   header  int32 expo[P][d_V], float bound[P][d_V]
//   Z       fp32 [Mh]            the normaliser column
//   V       fp16 [d_V][Mh]       the value columns
// Feature rows are those of the fp32 state with degree block p moved to start at hoff[p] (a
// multiple of 64); rows past m_p of a block are zero.  Value entry (row r of degree p,
// column j) = V[j][hoff[p] + r] 2^expo[p][j]; bound[p][j] is the largest |entry| of that
// block when it was written.
struct State16Geom {
    int64_t M, M_pad;                 // fp32 layout
    int64_t Mh;                       // rows of the compact layout
    int64_t head_bytes, z_off, v_off; // compact layout of one head
    int64_t off[kMaxP], hoff[kMaxP], m[kMaxP];
    int d_K, d_V, P;
};
inline int64_t state16_header_bytes(int d_V, int P) { return ((int64_t)8 * P * d_V + 255) / 256 * 256; }
inline int64_t state16_head_bytes(int64_t Mh, int d_V, int P) {
    return (state16_header_bytes(d_V, P) + 4 * Mh + 2 * (int64_t)d_V * Mh + 255) / 256 * 256;
}

struct Decode16Args {
    uint8_t* state;                   // compact states (pool slots with `slots`)
    const void* q;
    const void* k;
    const void* v;
    float* y;
    const uint32_t* fidx_h;           // packed indices in compact row order [Mh]
    const float* qw_h;                // alpha_p C_p in compact row order [Mh]
    float* partial;                   // decode16_partial_floats(BH, d_V, P, Mh) floats: the partial
                                      // readouts, then the per-wave block maxima
    State16Geom g;
    int BH, nblk;
    bool bf16;
    const int32_t* slots;
    int64_t pool;
    int H;
};
int decode16_blocks(int64_t Mh);
int64_t decode16_partial_floats(int BH, int d_V, int P, int64_t Mh);
hipError_t launch_decode16(const Decode16Args& a, hipStream_t st);
hipError_t launch_decode16_reduce(const Decode16Args& a, hipStream_t st);
// fp32 states [count][d_V + 1][M_pad] <-> compact states [count][head_bytes]
hipError_t launch_state16_pack(const float* src, uint8_t* dst, const State16Geom& g, int count,
                               hipStream_t st);
hipError_t launch_state16_unpack(const uint8_t* src, float* dst, const State16Geom& g, int count,
                                 hipStream_t st);

// One segment [c_begin, c_end) of chunks of a chunked prefill.
struct PrefillSegArgs {
    const void* q;
    const void* k;
    const void* v;
    float* y;
    float* state;            // [BH][d_V+1][M_pad]; read if load_state, written if store_state
    float* partial;          // [BH][c_end-c_begin][nslices] blocks of slice partials: fp32
                             // [d_V+1][L]; with partial_tiled the matrix-core layout of
                             // tiled_partial_floats(L, d_V) floats (below)
    bool partial_tiled;
    float* den;              // nullable: the fp32 finalize writes D_T of every row here
    const uint32_t* fidx;    // packed feature indices [M_pad]
    const float* qw;         // alpha_p C_p [M_pad]
    const void* mfma_rows;   // slice tables of the MFMA scan (nullptr for the VALU scan)
    Alpha alpha;
    int64_t M, M_pad;
    int BH, n, d_K, d_V, P, L;
    int nslices, slice_feats; // slice decomposition of the feature axis
    int c_begin, c_end;
    int win;                 // chunks per readout window: chunk c's state readout is taken at the
                             // window's first chunk c_begin + win * floor((c - c_begin) / win)
    int load_state, store_state;
    bool bf16;
    // Two-level form (MFMA scan only): the chunks [c_begin, c_end) are cut into nsub
    // sub-segments of sub_chunks chunks (a multiple of win), scanned in parallel, each from
    // its own state: state holds [BH][nsub][d_V+1][M_pad].  nsub = 1: one segment, state
    // [BH][d_V+1][M_pad].  update_only: no readout and no partials, only the state updates.
    // final_state (two-level only, nullable): with store_state, the blocks of the last
    // sub-segment store their end state there ([BH][d_V+1][M_pad]) and the others store none.
    int nsub = 1, sub_chunks = 0;
    bool update_only = false;
    float* final_state = nullptr;
    // Matrix-core scan only: the fp16 operand images written by the prep kernels
    // (kern_prep.hip, layouts in scan_mfma.h) for windows [img_w0, img_w0 + img_nwin) and
    // 128-token update sub-chunks [img_u0, img_u0 + img_nsub) of every head, and the per-head
    // maxima of |q|, |k|, |v| (float bits, [BH][4]) that set their power-of-two scales.
    uint16_t* qimg = nullptr;
    uint16_t* kimg = nullptr;
    uint16_t* vimg = nullptr;
    int img_w0 = 0, img_nwin = 0, img_u0 = 0, img_nsub = 0;
    const uint32_t* maxbits = nullptr;
};

// Slice partials of the matrix-core scan, one block per (head, chunk, slice): the d_V value
// columns as fp16 in tile-pair order [token tile][pair of 16-column tiles][lane] x 16 bytes
// (lane (li, g): tokens 16 tile + 4 g .. + 3, halves 0-3 column 32 pair + li, halves 4-7
// column 32 pair + 16 + li), then the normaliser column as L fp32 values, then one fp32
// scale per 16-token tile: value column j of token t is (q~_t . S)_j = stored x scale[tile]
// x 2^s_v, with s_v the head's value scale (prep_scale_exp of its max |v|); the normaliser
// is stored as is.  Each tile's scale is a power of two chosen from the tile's largest
// value, so every finite partial fits fp16; there is one per tile and column group of 64
// ([tile][group]).
__host__ __device__ constexpr int64_t tiled_partial_floats(int L, int d_V) {
    return (int64_t)L * d_V / 2 + L + (L / 16) * (d_V / 64);
}

// Per-head power-of-two input scale of the matrix-core path: for a maximum |x| with float
// bits mb, the exponent s with max |x| 2^-s in [1, 2) (0 for an all-zero input), clamped.
__host__ __device__ inline int prep_scale_exp(uint32_t mb) {
    if (mb == 0u) return 0;
    int e = (int)((mb >> 23) & 0xffu) - 127;
    return e < -60 ? -60 : (e > 60 ? 60 : e);
}
// Prep kernels of the matrix-core scan (kern_prep.hip): the maxima, then the fp16 images.
hipError_t launch_prep_max(const PrefillSegArgs& a, uint32_t* maxbits, hipStream_t st);
hipError_t launch_prep_images(const PrefillSegArgs& a, int u_begin, int u_end, hipStream_t st);

// Two-level prefill: from the local states of the pieces of the first nsub - 1 sub-segments,
// pieces [BH][(nsub - 1) pieces_per_sub][per_state] in order, the state each of the nsub
// sub-segments starts from, starts [BH][nsub][per_state]: init ([BH][per_state], zero when
// null) plus the pieces before the sub-segment, added in order.
hipError_t launch_state_starts(const float* pieces, const float* init, float* starts, int BH, int nsub,
                               int pieces_per_sub, int64_t per_state, hipStream_t st);

// fp32 scan: slice_feats features per block, chosen by valu_slice_feats().
int valu_slice_feats(int d_K, int d_V, int L);
hipError_t launch_scan_valu(const PrefillSegArgs& a, hipStream_t st);

// Intra-chunk part + reduction of the slice partials + normalisation -> y.
int64_t finalize_lds_bytes(int d_K, int d_V, int L);
hipError_t launch_finalize(const PrefillSegArgs& a, hipStream_t st);
// The fp32 finalize whatever the input type (the backward's forward recompute); writes
// the normaliser D_T of every row to a.den when it is non-null.
hipError_t launch_finalize_fp32(const PrefillSegArgs& a, hipStream_t st);

// Backward of the chunked prefill, one segment [c_begin, c_end) of chunks.
struct BwdArgs {
    const void* q;
    const void* k;
    const void* v;
    const float* dy;         // [BH][n][d_V]
    const float* y;          // [BH][n][d_V] forward output
    const float* den;        // [BH][n] forward normaliser D_T
    const float* u;          // [BH][n][ucols]: dy / D, then -(dy . y) / D, then padding
    int ucols;               // d_V + 1 rounded up to a multiple of 4
    float* u_out;            // where bwd_u_kernel writes u (the same buffer)
    float* dq;
    float* dk;
    float* dv;
    float* state;            // S (dq pass) or R (dk, dv pass) carrier [BH][d_V+1][M_pad]
    float* part;             // dq or dk slice partials [BH][c_end-c_begin][nslices][L][d_K]
    float* part2;            // dv slice partials [BH][c_end-c_begin][nslices][L][d_V]
    const uint32_t* fidx;
    const float* qw;
    Alpha alpha;
    int64_t M, M_pad;
    int BH, n, d_K, d_V, P, L;
    int nslices, slice_feats;
    int c_begin, c_end;
    int load_state, store_state;
    bool bf16;
};
int bwd_slice_feats(int d_K, int d_V, int L);
int64_t bwd_fin_lds_bytes(int d_K, int d_V, int L);
hipError_t launch_bwd_u(const BwdArgs& a, hipStream_t st);
hipError_t launch_bwd_q(const BwdArgs& a, hipStream_t st);
hipError_t launch_bwd_kv(const BwdArgs& a, hipStream_t st);
hipError_t launch_bwd_fin(const BwdArgs& a, int mode, hipStream_t st);   // 0: dq; 1: dk, dv

}  // namespace sata
