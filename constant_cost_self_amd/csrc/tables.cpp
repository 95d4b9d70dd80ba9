// tables.cpp -- host construction of M_p, C_p and the derived per-feature tables.
//
// [TA] "The mathematical breakthrough of the Taylor approximation": only the
// unique monomials of q^{(x)p} are kept, the index tuples i1 <= ... <= ip, and
// there are binom(d_K + p - 1, p) of them.  [TA] "Feature maps and linear
// attention": C_p counts how often each one occurs in the full expansion, i.e.
// the multinomial coefficient p! / prod_i (count of i)!.  [TA] "Hardware
// optimisation path" points at the prefix hierarchy of the rows.
//
// Construction: the rows of M_p in lexicographic order are the rows of M_{p-1}
// in lexicographic order, each extended by every last index l >= its own last
// index.  So each feature records its parent (the row with the last index
// dropped) and that last index; kernels build phi_p = phi_{p-1}[parent] x_last.
#include "tables.h"

#include <cmath>

namespace sata {

int64_t binom_i64(int64_t n, int64_t k) {
    if (k < 0 || n < k) return 0;
    if (k > n - k) k = n - k;
    unsigned __int128 r = 1;
    for (int64_t i = 1; i <= k; ++i) {
        r = r * (unsigned __int128)(n - k + i) / (unsigned __int128)i;
        if (r > (unsigned __int128)INT64_MAX) return -1;
    }
    return (int64_t)r;
}

int64_t feature_dim(int d_K, int P) {
    if (d_K < 1 || P < 1) return -1;
    return binom_i64((int64_t)d_K + P - 1, P - 1);
}

int64_t state_stride(int d_K, int P) {
    const int64_t M = feature_dim(d_K, P);
    if (M < 0) return -1;
    return (M + 63) / 64 * 64;
}

int64_t state16_stride(int d_K, int P) {
    if (d_K < 1 || P < 1) return -1;
    int64_t total = 0;
    for (int p = 0; p < P; ++p) {
        const int64_t m = binom_i64((int64_t)d_K + p - 1, p);
        if (m < 0) return -1;
        total += (m + 63) / 64 * 64;
    }
    return total;
}

static int64_t multinomial(const int32_t* row, int p) {
    // p! / prod over runs of equal indices of (run length)!   (rows are sorted)
    int64_t num = 1;
    for (int s = 2; s <= p; ++s) num *= s;
    int64_t den = 1;
    int run = 1;
    for (int s = 1; s <= p; ++s) {
        if (s < p && row[s] == row[s - 1]) {
            ++run;
        } else {
            for (int r = 2; r <= run; ++r) den *= r;
            run = 1;
        }
    }
    return num / den;
}

bool build_host_tables(int d_K, int P, HostTables& t) {
    t = HostTables();
    if (d_K < 1 || d_K > 255 || P < 1 || P > 5) return false;
    t.d_K = d_K;
    t.P = P;
    t.m.resize(P);
    t.off.resize(P);
    t.Mp.resize(P);
    t.Cp.resize(P);
    t.alpha.resize(P);

    const double c = std::sqrt((double)d_K);
    for (int p = 0; p < P; ++p) {
        double fact = 1.0, cp = 1.0;
        for (int s = 1; s <= p; ++s) { fact *= s; cp *= c; }
        t.alpha[p] = 1.0 / (fact * cp);
    }

    // p = 0: one empty tuple, C_0 = 1.
    t.m[0] = 1;
    t.off[0] = 0;
    t.Cp[0] = {1};
    t.parent.push_back(-1);
    t.last.push_back(-1);
    t.degree.push_back(0);

    for (int p = 1; p < P; ++p) {
        const int64_t m_prev = t.m[p - 1];
        const std::vector<int32_t>& prev = t.Mp[p - 1];
        std::vector<int32_t>& cur = t.Mp[p];
        std::vector<int32_t>& cnt = t.Cp[p];
        t.off[p] = t.off[p - 1] + m_prev;
        std::vector<int32_t> row(p);
        for (int64_t r = 0; r < m_prev; ++r) {
            const int start = (p == 1) ? 0 : prev[r * (p - 1) + (p - 2)];
            for (int l = start; l < d_K; ++l) {
                for (int s = 0; s < p - 1; ++s) row[s] = prev[r * (p - 1) + s];
                row[p - 1] = l;
                cur.insert(cur.end(), row.begin(), row.end());
                cnt.push_back((int32_t)multinomial(row.data(), p));
                t.parent.push_back((int32_t)(t.off[p - 1] + r));
                t.last.push_back(l);
                t.degree.push_back((int8_t)p);
            }
        }
        t.m[p] = (int64_t)cnt.size();
    }
    t.M = t.off[P - 1] + t.m[P - 1];
    t.M_pad = (t.M + 63) / 64 * 64;

    // Per-feature query weight alpha_p C_p and packed gather indices.
    t.qweight.resize(t.M);
    t.fidx.assign(t.M_pad, 0);
    t.qw.assign(t.M_pad, 0.0f);
    uint32_t all_sentinel = 0;
    for (int s = 0; s < 4; ++s) all_sentinel |= (uint32_t)d_K << (8 * s);
    for (int p = 0; p < P; ++p) {
        for (int64_t r = 0; r < t.m[p]; ++r) {
            const int64_t f = t.off[p] + r;
            t.qweight[f] = t.alpha[p] * (double)t.Cp[p][r];
            t.qw[f] = (float)t.qweight[f];
            uint32_t packed = all_sentinel;
            for (int s = 0; s < p; ++s) {
                packed &= ~(0xffu << (8 * s));
                packed |= (uint32_t)t.Mp[p][r * p + s] << (8 * s);
            }
            t.fidx[f] = packed;
        }
    }
    for (int64_t f = t.M; f < t.M_pad; ++f) t.fidx[f] = all_sentinel;

    // the same rows with every degree block starting on a multiple of 64
    t.hoff.resize(P);
    t.Mh = 0;
    for (int p = 0; p < P; ++p) {
        t.hoff[p] = t.Mh;
        t.Mh += (t.m[p] + 63) / 64 * 64;
    }
    t.fidx_h.assign(t.Mh, all_sentinel);
    t.qw_h.assign(t.Mh, 0.0f);
    for (int p = 0; p < P; ++p) {
        for (int64_t r = 0; r < t.m[p]; ++r) {
            t.fidx_h[t.hoff[p] + r] = t.fidx[t.off[p] + r];
            t.qw_h[t.hoff[p] + r] = t.qw[t.off[p] + r];
        }
    }
    return (int64_t)t.M == feature_dim(d_K, P);
}

}  // namespace sata
