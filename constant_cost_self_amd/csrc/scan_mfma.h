// scan_mfma.h -- bf16 MFMA chunked prefill scan (internal to libsata).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "launch.h"
#include "tables.h"

namespace sata {

// Per-handle tables of the MFMA scan: the feature axis cut into slices, each
// slice laid out as rows of 8 features sharing a parent.
struct MfmaTables {
    int nslices = 0;
    int slice_feats = 0;
    void* d_rows = nullptr;
    bool ok = false;
};

int build_mfma_tables(const HostTables& h, MfmaTables& m);
void free_mfma_tables(MfmaTables& m);
bool mfma_supported(const MfmaTables& m, bool bf16, int d_K, int d_V, int P, int L);
hipError_t launch_scan_mfma(const PrefillSegArgs& a, const MfmaTables& m, hipStream_t st);

}  // namespace sata
