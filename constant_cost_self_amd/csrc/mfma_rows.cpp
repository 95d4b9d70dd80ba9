// mfma_rows.cpp -- host construction of the row tables of the MFMA prefill scan.
//
// The symmetric basis has a prefix hierarchy ([TA] "Hardware optimisation path":
// rows of M_p are non-decreasing, so monomials sharing a prefix can be computed
// together): every feature of degree p >= 1 is a parent of degree p-1 times one
// more coordinate l >= the parent's last index.  The MFMA scan computes
//     phi(a, l)(x) = phi_a(x) * x_l
// for a whole row of 8 children at once, with l running over an aligned block of
// 8 coordinates l = 8b .. 8b+7 that is the same for all rows of a wave, so the 8
// coordinates x_l live in registers and only the parent product varies by row.
//
// Weights ([TA] "Feature maps and linear attention": C_p counts each monomial in
// the full expansion).  For a child (a, l) of degree p, C(a, l) = C(a) p / (1+m),
// with m the multiplicity of l in a (m > 0 only for l = last index of a).  The
// query side carries alpha_p C(a) p, the same for the whole row; the key side
// carries the row element's factor 1/(1+m) (and 0 for the children l below the
// parent's last index, which are not monomials of the basis).  The state kept
// inside the scan is therefore S'[f] = S[f] / (1+m_f); it is converted back to
// the unweighted state when it is written out.
#include <algorithm>
#include <cmath>

#include "scan_mfma.h"

namespace sata {

bool build_mfma_rows(const HostTables& h, MfmaHostRows& r) {
    r = MfmaHostRows();
    const int d = h.d_K, P = h.P;
    if (d % 8 != 0 || d > 128 || P < 2 || P > 5) return false;
    r.d_K = d;
    r.P = P;
    const int nb = d / 8;                      // coordinate blocks; block nb holds the constant 1

    // first child of every parent feature
    std::vector<int64_t> first_child(h.M, -1);
    for (int64_t f = 1; f < h.M; ++f) {
        const int64_t a = h.parent[f];
        if (first_child[a] < 0) first_child[a] = f;
    }

    struct Row {
        int64_t a;       // parent feature (-1: the p = 0 row)
        int b;
    };
    std::vector<std::vector<Row>> partial(nb + 1), full(nb + 1);
    for (int64_t a = 0; a < h.M; ++a) {
        const int dp = h.degree[a];
        if (dp > P - 2) continue;
        const int start = dp == 0 ? 0 : h.last[a];
        for (int b = start / 8; b < nb; ++b) {
            const bool is_partial = dp >= 1 && start >= 8 * b;
            (is_partial ? partial[b] : full[b]).push_back(Row{a, b});
        }
    }
    full[nb].push_back(Row{-1, nb});

    const uint32_t sentinel = (uint32_t)d;     // coordinate d holds the constant 1
    auto push_dead = [&](int b) {
        r.parent.push_back(sentinel | (sentinel << 10) | (sentinel << 20));
        r.weight.push_back(0.0f);
        r.degree.push_back(0);
        for (int e = 0; e < 8; ++e) {
            r.kscale.push_back(0.0f);
            r.canon.push_back(-1);
        }
        (void)b;
    };

    for (int b = 0; b <= nb; ++b) {
        std::vector<Row> rows = partial[b];
        rows.insert(rows.end(), full[b].begin(), full[b].end());
        if (rows.empty()) continue;
        for (const Row& row : rows) {
            if (row.a < 0) {                    // phi_0 = 1: coordinate d, weight alpha_0
                r.parent.push_back(sentinel | (sentinel << 10) | (sentinel << 20));
                r.weight.push_back((float)h.alpha[0]);
                r.degree.push_back(0);
                for (int e = 0; e < 8; ++e) {
                    r.kscale.push_back(e == 0 ? 1.0f : 0.0f);
                    r.canon.push_back(e == 0 ? 0 : -1);
                }
                continue;
            }
            const int64_t a = row.a;
            const int dp = h.degree[a], p = dp + 1;
            const int32_t* coords = dp > 0 ? &h.Mp[dp][(a - h.off[dp]) * dp] : nullptr;
            uint32_t pc = 0;
            for (int s = 0; s < 3; ++s) {
                const uint32_t c = s < dp ? (uint32_t)coords[s] : sentinel;
                pc |= c << (10 * s);
            }
            r.parent.push_back(pc);
            const double Ca = (double)h.Cp[dp][a - h.off[dp]];
            r.weight.push_back((float)(h.alpha[p] * Ca * p));
            r.degree.push_back((int8_t)p);
            const int start = dp == 0 ? 0 : h.last[a];
            for (int e = 0; e < 8; ++e) {
                const int l = 8 * row.b + e;
                if (l < start) {
                    r.kscale.push_back(0.0f);
                    r.canon.push_back(-1);
                    continue;
                }
                int m = 0;
                for (int s = 0; s < dp; ++s) m += coords[s] == l;
                const int64_t F = first_child[a] + (l - start);
                if (F <= 0 || F >= h.M || h.parent[F] != a || h.last[F] != l) return false;
                r.kscale.push_back((float)(1.0 / (1.0 + m)));
                r.canon.push_back((int32_t)F);
            }
        }
        const int pad = (int)((kRowsPerWave - rows.size() % kRowsPerWave) % kRowsPerWave);
        for (int i = 0; i < pad; ++i) push_dead(b);
        for (size_t i = 0; i < (rows.size() + pad) / kRowsPerWave; ++i) r.wave_lblock.push_back(b);
    }
    while (r.wave_lblock.size() % kWavesPerSlice) {
        for (int i = 0; i < kRowsPerWave; ++i) push_dead(0);
        r.wave_lblock.push_back(0);
    }
    r.nrows = (int)r.parent.size();
    // per degree, the binary exponent bounding the rows' query weights: |w| <= 2^wlog[p]
    for (int p = 0; p < 8; ++p) r.wlog[p] = -126;
    for (int i = 0; i < r.nrows; ++i) {
        if (r.weight[i] == 0.0f) continue;
        int e = 0;
        const double m = std::frexp((double)std::fabs(r.weight[i]), &e);   // |w| = m 2^e, m in [0.5, 1)
        (void)m;
        if (e > r.wlog[r.degree[i]]) r.wlog[r.degree[i]] = e;
    }

    // every canonical feature must appear exactly once with a nonzero key factor
    std::vector<int> seen(h.M, 0);
    for (size_t i = 0; i < r.canon.size(); ++i)
        if (r.canon[i] >= 0) {
            if (r.kscale[i] == 0.0f) return false;
            seen[r.canon[i]] += 1;
        }
    for (int64_t f = 0; f < h.M; ++f)
        if (seen[f] != 1) return false;
    return r.nrows % kRowsPerSlice == 0;
}

}  // namespace sata
