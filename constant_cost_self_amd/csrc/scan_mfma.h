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
};

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
