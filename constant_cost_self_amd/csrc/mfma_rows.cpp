// mfma_rows.cpp -- host construction of the row tables of the MFMA prefill scan.
//
// Every feature of degree p >= 1 is a monomial x_{i1} ... x_{ip} of the symmetric basis
// ([TA] "The mathematical breakthrough of the Taylor approximation"), and it can be written
// as a parent monomial of degree p - 1 times one more coordinate l; the products x_i commute,
// so any one of the p indices can play l ([TA] "Hardware optimisation path" suggests
// computing monomials together through their shared parts).  The MFMA scan computes
//     phi(a, l)(x) = phi_a(x) * x_l
// for a whole row of 8 features at once: a parent a and l running over an aligned block of 8
// coordinates l = 8b .. 8b+7 that is the same for all rows of a wave, so the 8 coordinates
// x_l live in registers and only the parent product varies by row.
//
// Rows are chosen so that almost all of their 8 slots hold a monomial of the basis.  For a
// monomial m, let a block of coordinates that holds exactly one index of m be a singleton
// block.  If m has one, l is its index in the lowest singleton block and a = m - {l}: then
// every l' of that block gives a monomial a + {l'} whose lowest singleton block is the same,
// so the row (a, block) is full and claims exactly these 8 monomials.  Otherwise (every block
// of m holds two or more indices, e.g. all indices in one block) l is the largest index, and
// the row (a, block of l) holds the monomials a + {l'} with l' >= max(a); its lower slots are
// masked.  Each monomial of the basis belongs to exactly one row (checked when built).
//
// Weights ([TA] "Feature maps and linear attention": C_p counts each monomial in the full
// expansion).  For a child a + {l} of degree p, C(a + {l}) = C(a) p / (1+m), with m the
// multiplicity of l in a.  The query side carries alpha_p C(a) p, the same for the whole
// row; the key-side factor of the row element is 1/(1+m) (0 for masked slots).
#include <algorithm>
#include <array>
#include <cmath>
#include <unordered_map>

#include "scan_mfma.h"

namespace sata {

bool build_mfma_rows(const HostTables& h, MfmaHostRows& r) {
    r = MfmaHostRows();
    const int d = h.d_K, P = h.P;
    if (d % 8 != 0 || d > 128 || P < 2 || P > 5) return false;
    r.d_K = d;
    r.P = P;
    const int nb = d / 8;                      // coordinate blocks; block nb holds the constant 1
    const uint32_t sentinel = (uint32_t)d;     // coordinate d holds the constant 1

    // first child of every parent feature: canonical index of a sorted index tuple
    std::vector<int64_t> first_child(h.M, -1);
    for (int64_t f = 1; f < h.M; ++f) {
        const int64_t a = h.parent[f];
        if (first_child[a] < 0) first_child[a] = f;
    }
    auto canon = [&](const int* idx, int p) -> int64_t {
        int64_t f = 0;
        int last = 0;
        for (int s = 0; s < p; ++s) {
            if (first_child[f] < 0) return -1;
            f = first_child[f] + (idx[s] - last);
            last = idx[s];
        }
        return f;
    };

    struct Row {
        std::array<int, 3> par;  // parent indices, sorted, sentinel-padded
        int np, b;
        int32_t canon[8];
        float ks[8];
    };
    std::vector<Row> rows;
    std::unordered_map<uint64_t, int64_t> index;   // (parent, block) -> row
    auto key_of = [&](const int* par, int np, int b) {
        uint64_t k = (uint64_t)b;
        for (int s = 0; s < 3; ++s) k = (k << 8) | (uint64_t)(s < np ? par[s] : 255);
        return k;
    };

    for (int p = 1; p < P; ++p) {
        const std::vector<int32_t>& Mp = h.Mp[p];
        for (int64_t i = 0; i < h.m[p]; ++i) {
            const int32_t* m = &Mp[i * p];
            int cnt[16] = {0};
            for (int s = 0; s < p; ++s) cnt[m[s] / 8] += 1;
            int pos = -1;                                  // the index that plays l
            for (int s = 0; s < p && pos < 0; ++s)         // m sorted: lowest block first
                if (cnt[m[s] / 8] == 1) pos = s;
            const bool single = pos >= 0;
            if (!single) pos = p - 1;
            const int l = m[pos], b = l / 8;
            int par[3] = {0, 0, 0}, np = 0;
            for (int s = 0; s < p; ++s)
                if (s != pos) par[np++] = m[s];
            int mult = 0;
            for (int s = 0; s < np; ++s) mult += par[s] == l;
            const uint64_t key = key_of(par, np, b);
            auto it = index.find(key);
            int64_t ri;
            if (it == index.end()) {
                ri = (int64_t)rows.size();
                index.emplace(key, ri);
                Row row;
                row.np = np;
                row.b = b;
                for (int s = 0; s < 3; ++s) row.par[s] = s < np ? par[s] : (int)sentinel;
                for (int e = 0; e < 8; ++e) {
                    row.canon[e] = -1;
                    row.ks[e] = 0.0f;
                }
                rows.push_back(row);
            } else {
                ri = it->second;
            }
            Row& row = rows[ri];
            const int e = l - 8 * b;
            if (row.canon[e] >= 0) return false;            // two monomials in one slot
            const int64_t F = canon(m, p);
            if (F <= 0 || F >= h.M) return false;
            row.canon[e] = (int32_t)F;
            row.ks[e] = (float)(1.0 / (1.0 + mult));
        }
    }

    // multinomial coefficient of a sorted parent: (np)! / prod (run lengths)!
    auto multinomial = [](const std::array<int, 3>& par, int np) {
        double num = 1.0, den = 1.0;
        for (int s = 2; s <= np; ++s) num *= s;
        int run = 1;
        for (int s = 1; s <= np; ++s) {
            if (s < np && par[s] == par[s - 1]) {
                ++run;
            } else {
                for (int q = 2; q <= run; ++q) den *= q;
                run = 1;
            }
        }
        return num / den;
    };

    auto push_dead = [&]() {
        r.parent.push_back(sentinel | (sentinel << 10) | (sentinel << 20));
        r.weight.push_back(0.0f);
        r.degree.push_back(0);
        for (int e = 0; e < 8; ++e) {
            r.kscale.push_back(0.0f);
            r.canon.push_back(-1);
        }
    };
    // rows grouped by l-block (one wave's rows share it), in a fixed order within a block
    std::vector<std::vector<int64_t>> by_block(nb + 1);
    for (int64_t i = 0; i < (int64_t)rows.size(); ++i) by_block[rows[i].b].push_back(i);
    for (int b = 0; b <= nb; ++b) {
        std::vector<int64_t>& ids = by_block[b];
        std::sort(ids.begin(), ids.end(), [&](int64_t x, int64_t y) {
            const Row &u = rows[x], &v = rows[y];
            if (u.np != v.np) return u.np < v.np;
            return u.par < v.par;
        });
        int64_t count = (int64_t)ids.size() + (b == nb ? 1 : 0);
        if (count == 0) continue;
        if (b == nb) {                          // phi_0 = 1: coordinate d, weight alpha_0
            r.parent.push_back(sentinel | (sentinel << 10) | (sentinel << 20));
            r.weight.push_back((float)h.alpha[0]);
            r.degree.push_back(0);
            for (int e = 0; e < 8; ++e) {
                r.kscale.push_back(e == 0 ? 1.0f : 0.0f);
                r.canon.push_back(e == 0 ? 0 : -1);
            }
        }
        for (int64_t id : ids) {
            const Row& row = rows[id];
            const int p = row.np + 1;
            r.parent.push_back((uint32_t)row.par[0] | ((uint32_t)row.par[1] << 10) | ((uint32_t)row.par[2] << 20));
            r.weight.push_back((float)(h.alpha[p] * multinomial(row.par, row.np) * p));
            r.degree.push_back((int8_t)p);
            for (int e = 0; e < 8; ++e) {
                r.kscale.push_back(row.ks[e]);
                r.canon.push_back(row.canon[e]);
            }
        }
        const int64_t pad = (kRowsPerWave - count % kRowsPerWave) % kRowsPerWave;
        for (int64_t i = 0; i < pad; ++i) push_dead();
        for (int64_t i = 0; i < (count + pad) / kRowsPerWave; ++i) r.wave_lblock.push_back(b);
    }
    while (r.wave_lblock.size() % kWavesPerSlice) {
        for (int i = 0; i < kRowsPerWave; ++i) push_dead();
        r.wave_lblock.push_back(0);
    }
    r.nrows = (int)r.parent.size();
    // per degree, the binary exponent bounding the rows' query weights: |w| <= 2^wlog[p]
    for (int p = 0; p < 8; ++p) r.wlog[p] = -126;
    for (int i = 0; i < r.nrows; ++i) {
        if (r.weight[i] == 0.0f) continue;
        int e = 0;
        (void)std::frexp((double)std::fabs(r.weight[i]), &e);    // |w| = m 2^e, m in [0.5, 1)
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
