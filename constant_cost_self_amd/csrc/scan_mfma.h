// scan_mfma.h -- bf16 MFMA chunked prefill scan (internal to libsata).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <vector>

#include "launch.h"
#include "tables.h"

namespace sata {

// The MFMA scan works on "rows": a row is a parent monomial a (degree p-1) and an
// aligned block of 8 last indices l = 8b .. 8b+7; its 8 kernel features are the
// children (a, l).  Children with l below the parent's last index are not
// monomials of the basis (masked, weight 0).  The child with l equal to the
// parent's last index carries a multiplicity ratio.  Rows are grouped by l-block
// so that one wave's 16 rows share the same 8 last coordinates.
struct MfmaHostRows {
    int d_K = 0, P = 0;
    int nrows = 0;                       // multiple of kRowsPerSlice
    std::vector<uint32_t> parent;        // [nrows] 3 parent coordinates, 10 bits each (d_K = 1)
    std::vector<float> weight;           // [nrows] alpha_p C(a) p   (query side)
    std::vector<float> kscale;           // [nrows*8] key-side factor: 0 masked, 1/(m+1) diag, 1
    std::vector<int32_t> canon;          // [nrows*8] canonical feature index, -1 if none
    std::vector<int32_t> wave_lblock;    // [nrows/16] l-block of each wave
    std::vector<int8_t> degree;          // [nrows] degree p of the row's features
    int wlog[8] = {0};                   // per degree p: ceil(log2 max |weight|) over its rows
};

// fp16 operand images of the matrix-core scan, written by the prep kernels and copied as is
// into LDS (whole 1 KiB blocks per direct-to-LDS wave instruction):
//   q window image   [R][XR]: token rows q' = q 2^-s_q (d_K coordinates), then the constant
//                    slot (1, 0, ..., 0); R = 256 at d_K = 64, 128 at d_K = 128
//   key table        [XR][TS] per 128-token update sub-chunk: coordinate rows over tokens,
//                    k' = k 2^-s_k, then row d_K = 1 for the tokens that exist (0 past n),
//                    rows d_K + 1 .. d_K + 7 zero; 8 padding tokens per row
//   value table      [rows][TS] per sub-chunk and group of 64 value columns: v' = v 2^-s_v,
//                    then (group 0) the row of ones for the normaliser (0 past n)
constexpr int kImgLU = 128;
__host__ __device__ constexpr int img_pad1k(int b) { return (b + 1023) / 1024 * 1024; }
__host__ __device__ constexpr int img_xr(int d_K) { return d_K + 8; }
__host__ __device__ constexpr int img_ts() { return kImgLU + 8; }
__host__ __device__ constexpr int img_window(int d_K) { return d_K == 64 ? 256 : 128; }
__host__ __device__ constexpr int img_q_bytes(int d_K) { return img_window(d_K) * img_xr(d_K) * 2; }
__host__ __device__ constexpr int img_kt_bytes(int d_K) { return img_pad1k(img_xr(d_K) * img_ts() * 2); }
__host__ __device__ constexpr int img_vt_bytes() { return img_pad1k(65 * img_ts() * 2); }
// bytes of the images of one head for nwin windows and nsub sub-chunks
inline int64_t img_head_bytes(int d_K, int d_V, int64_t nwin, int64_t nsub) {
    return nwin * img_q_bytes(d_K) + nsub * img_kt_bytes(d_K) + nsub * (d_V / 64) * img_vt_bytes();
}

constexpr int kRowsPerWave = 8;
constexpr int kWavesPerSlice = 8;
constexpr int kRowsPerSlice = kRowsPerWave * kWavesPerSlice;   // 64 rows = 512 kernel features

bool build_mfma_rows(const HostTables& h, MfmaHostRows& r);

struct MfmaTables {
    int nslices = 0;
    int slice_feats = 0;                 // kernel features per slice (512)
    int d_K = 0, P = 0;
    void* d_rows = nullptr;              // one device allocation holding the arrays below
    const uint32_t* parent = nullptr;
    const float* weight = nullptr;
    const float* kscale = nullptr;
    const int32_t* canon = nullptr;
    const int32_t* wave_lblock = nullptr;
    const int8_t* degree = nullptr;
    int wlog[8] = {0};
    bool ok = false;
};

int build_mfma_tables(const HostTables& h, MfmaTables& m);
void free_mfma_tables(MfmaTables& m);
// Shapes the matrix-core scan serves (bf16 inputs, d_K and d_V in {64, 128}, 2 <= P <= 5,
// chunk 64), whatever the tables.
bool mfma_shape(bool bf16, int d_K, int d_V, int P, int L);
bool mfma_supported(const MfmaTables& m, bool bf16, int d_K, int d_V, int P, int L);
// Feature slices of the matrix-core scan for these host tables (0 if it does not apply).
int mfma_slice_count(const HostTables& h);
// Chunks per readout window of the MFMA scan (the finalize's direct part spans the window).
int mfma_window(int d_K);
hipError_t launch_scan_mfma(const PrefillSegArgs& a, const MfmaTables& m, hipStream_t st);

}  // namespace sata
