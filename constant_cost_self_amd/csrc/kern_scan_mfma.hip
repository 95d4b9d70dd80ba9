// kern_scan_mfma.hip -- bf16 MFMA chunked prefill scan (gfx950).
#include "scan_mfma.h"

namespace sata {

int build_mfma_tables(const HostTables&, MfmaTables& m) {
    m = MfmaTables();
    return 0;
}

void free_mfma_tables(MfmaTables& m) { m = MfmaTables(); }

bool mfma_supported(const MfmaTables& m, bool, int, int, int, int) { return m.ok; }

hipError_t launch_scan_mfma(const PrefillSegArgs&, const MfmaTables&, hipStream_t) {
    return hipErrorNotSupported;
}

}  // namespace sata
