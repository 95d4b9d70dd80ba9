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
hipError_t launch_decode_reduce(const DecodeArgs& a, hipStream_t st);  // partials -> y

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
    int nsub = 1, sub_chunks = 0;
    bool update_only = false;
};

// Slice partials of the matrix-core scan, one block per (head, chunk, slice): the d_V value
// columns as fp16 times kPartialScale, in tile-pair order [token tile][pair of 16-column
// tiles][lane] x 16 bytes (lane (li, g): tokens 16 tile + 4 g .. + 3, halves 0-3 column
// 32 pair + li, halves 4-7 column 32 pair + 16 + li), then the normaliser column as L fp32
// values.  The power-of-two scale keeps partials up to 65504 / kPartialScale in range.
constexpr float kPartialScale = 1.0f / 256.0f;
__host__ __device__ constexpr int64_t tiled_partial_floats(int L, int d_V) { return (int64_t)L * d_V / 2 + L; }

// Two-level prefill: replaces the nsub local states of every head, [BH][nsub][per_state],
// by the state each sub-segment starts from (exclusive prefix sums, starting from init, which
// is [BH][per_state] or zero when null), and writes the total to final when non-null (final
// may equal init).
hipError_t launch_state_prefix(float* states, const float* init, float* final, int BH, int nsub,
                               int64_t per_state, hipStream_t st);

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
