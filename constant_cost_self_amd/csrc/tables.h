// tables.h -- host construction of the SATA feature tables (internal to libsata).
#pragma once

#include <stdint.h>

#include <vector>

namespace sata {

struct HostTables {
    int d_K = 0, P = 0;
    int64_t M = 0, M_pad = 0;
    std::vector<int64_t> m;                  // m_p, p = 0..P-1
    std::vector<int64_t> off;                // first feature of term p
    std::vector<std::vector<int32_t>> Mp;    // [p] -> [m_p][p]
    std::vector<std::vector<int32_t>> Cp;    // [p] -> [m_p]
    // Per feature f of the concatenated order (size M):
    std::vector<int32_t> parent;             // feature with the last index dropped (-1 for f = 0)
    std::vector<int32_t> last;               // last index (-1 for f = 0)
    std::vector<int8_t> degree;              // p
    std::vector<double> qweight;             // alpha_p C_p, fp64
    // Device-layout copies (size M_pad): packed indices, sentinel d_K; fp32 weights.
    std::vector<uint32_t> fidx;
    std::vector<float> qw;
    std::vector<double> alpha;               // alpha_p, fp64
    // Half-precision state order: degree block p starts at hoff[p], a multiple of 64, and
    // Mh = sum_p roundup(m_p, 64); fidx_h and qw_h are fidx and qw in that order (size Mh),
    // the rows past m_p of a block holding the sentinel indices and weight 0.
    int64_t Mh = 0;
    std::vector<int64_t> hoff;
    std::vector<uint32_t> fidx_h;
    std::vector<float> qw_h;
};

int64_t binom_i64(int64_t n, int64_t k);     // -1 on overflow
int64_t feature_dim(int d_K, int P);
int64_t state_stride(int d_K, int P);        // M rounded up to a multiple of 64
int64_t state16_stride(int d_K, int P);      // Mh of the half-precision state order
bool build_host_tables(int d_K, int P, HostTables& t);

}  // namespace sata
