// Host half of libkvtc: configuration, the once-per-prefill fit (mean,
// covariance, symmetric eigensolver, rank, DP bit allocation, frozen ranges),
// the state-blob builder and the storage accounting.
//
// The method is the one of the KVTC cache module page
// (veloxquant_mlx.cache.kvtc_cache: module docstring "Design",
// _TensorKVTC.fit_prefill_from_pca / _requantize, KVTCKVCache.update_and_fetch)
// and, for the group-head mode, of the PALU cache API page
// (veloxquant_mlx.cache.palu_cache, "Design" and the palu_* parameters).
//
// Built with -ffp-contract=off: the DP compares sums of doubles and must
// evaluate them exactly in the order written.
#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdlib>
#include <cstring>
#include <functional>
#include <limits>
#include <new>
#include <queue>
#include <thread>
#include <vector>

#include "kvtc.h"
#include "kvtc_internal.h"

namespace kvtc {
namespace {

// ------------------------------------------------------------------ threads
int num_threads() {
    int t = static_cast<int>(std::thread::hardware_concurrency());
    if (const char *e = std::getenv("KVTC_THREADS")) t = std::atoi(e);
    else if (const char *o = std::getenv("OMP_NUM_THREADS")) t = std::min(t, std::atoi(o));
    return std::max(1, std::min(t, 64));
}

// Runs fn(i) for i in [0, n) on up to num_threads() threads.  Returns false if
// any call threw (the work of the others still completes).
bool parallel_for(int64_t n, const std::function<void(int64_t)> &fn) {
    std::atomic<int64_t> next{0};
    std::atomic<bool> ok{true};
    auto worker = [&] {
        for (;;) {
            int64_t i = next.fetch_add(1);
            if (i >= n) break;
            try {
                fn(i);
            } catch (...) {
                ok = false;
            }
        }
    };
    int64_t T = std::min<int64_t>(num_threads(), n);
    std::vector<std::thread> pool;
    for (int64_t t = 1; t < T; ++t) pool.emplace_back(worker);
    worker();
    for (auto &th : pool) th.join();
    return ok;
}

// ------------------------------------------------------------ fp16 rounding
// Nearest-even binary16 of a double, computed from the value (power-of-two
// scalings are exact, rint rounds half to even in the default mode).
uint16_t half_bits_rne(double x) {
    uint16_t sign = std::signbit(x) ? 0x8000u : 0u;
    double a = std::fabs(x);
    if (std::isnan(x)) return sign | 0x7E00u;
    if (a >= 65520.0) return sign | 0x7C00u;             // past the last finite midpoint
    if (a < 6.103515625e-05) {                            // below 2^-14: subnormal grid 2^-24
        double q = std::rint(std::ldexp(a, 24));
        return sign | static_cast<uint16_t>(q);           // q == 1024 is the smallest normal
    }
    int e;
    std::frexp(a, &e);                                    // a = m * 2^e, m in [0.5, 1)
    int ex = e - 1;                                       // a in [2^ex, 2^(ex+1))
    double q = std::rint(std::ldexp(a, 10 - ex));         // in [1024, 2048]
    if (q == 2048.0) {
        q = 1024.0;
        ++ex;
    }
    if (ex + 15 >= 31) return sign | 0x7C00u;
    return sign | static_cast<uint16_t>(((ex + 15) << 10) | (static_cast<int>(q) - 1024));
}

// Exact value of a binary16 bit pattern.
double half_value(uint16_t h) {
    const int e = (h >> 10) & 31, m = h & 1023;
    double v;
    if (e == 0) v = std::ldexp(static_cast<double>(m), -24);
    else if (e == 31) v = m ? std::numeric_limits<double>::quiet_NaN() : std::numeric_limits<double>::infinity();
    else v = std::ldexp(static_cast<double>(1024 + m), e - 25);
    return (h & 0x8000) ? -v : v;
}

// ---------------------------------------------------------- configuration
bool width_allowed(int b) { return b == 0 || b == 1 || b == 2 || b == 3 || b == 4 || b == 8; }

int32_t validate_config(const kvtc_config *c) {
    if (!c) return KVTC_E_ARG;
    if (c->mode != KVTC_MODE_DP && c->mode != KVTC_MODE_MIXED) return KVTC_E_CONFIG;
    if (c->head_dim <= 0 || c->head_dim % 64 != 0 || c->head_dim > 4096) return KVTC_E_CONFIG;
    if (c->heads_per_unit < 1) return KVTC_E_CONFIG;
    const int dg = c->head_dim * c->heads_per_unit;
    if (dg > 4096) return KVTC_E_CONFIG;
    if (c->rank < 0 || c->rank > dg) return KVTC_E_CONFIG;
    if (c->rank == 0 && !(c->energy_threshold > 0.0 && c->energy_threshold <= 1.0)) return KVTC_E_CONFIG;
    if (c->mode == KVTC_MODE_DP) {
        if (c->heads_per_unit != 1) return KVTC_E_CONFIG;
        if (c->bit_budget < 0) return KVTC_E_CONFIG;      // KVTCKVCache raises on budget < 0
        if (c->n_choices < 1 || c->n_choices > KVTC_MAX_CHOICES) return KVTC_E_CONFIG;
        for (int i = 0; i < c->n_choices; ++i)
            if (!width_allowed(c->choices[i])) return KVTC_E_CONFIG;
        if (!(c->beta > 0.0) || !std::isfinite(c->beta)) return KVTC_E_CONFIG;
    } else {
        if (!width_allowed(c->hi_bits) || !width_allowed(c->lo_bits) || c->hi_bits == 0 ||
            c->lo_bits == 0)
            return KVTC_E_CONFIG;
        if (c->group_size < 16 || c->group_size % 16 != 0) return KVTC_E_CONFIG;
        if (!(c->hi_fraction >= 0.0 && c->hi_fraction <= 1.0)) return KVTC_E_CONFIG;
    }
    return KVTC_OK;
}

// ------------------------------------------------------------ allocation
// Exact DP of the allocation (see kvtc_allocate_bits); returns false when no
// allocation fits the budget.
bool dp_allocate(const double *lam, int r, int budget, const std::vector<int> &choices_in,
                 double beta, uint8_t *bits) {
    std::vector<int> choices(choices_in);
    std::sort(choices.begin(), choices.end());
    choices.erase(std::unique(choices.begin(), choices.end()), choices.end());
    const double inf = std::numeric_limits<double>::infinity();
    // no allocation spends more than r * (widest choice) bits: columns past that
    // stay infinite, so clamping the table there changes neither the optimum
    // nor its tie-breaking, and bounds the work for any budget
    const int widest = choices.empty() ? 0 : choices.back();
    const int C = static_cast<int>(std::min<int64_t>(budget, static_cast<int64_t>(r) * widest)) + 1;
    std::vector<double> best(C, inf), nxt(C);
    std::vector<int8_t> pick(static_cast<size_t>(r) * C, -1);
    best[0] = 0.0;
    for (int i = 0; i < r; ++i) {
        std::fill(nxt.begin(), nxt.end(), inf);
        int8_t *arg = &pick[static_cast<size_t>(i) * C];
        for (int b : choices) {
            if (b >= C) continue;
            // distortion proxy: dropped -> lambda, b bits -> beta * lambda * 4^-b
            const double d = (b == 0) ? lam[i] : beta * lam[i] * std::ldexp(1.0, -2 * b);
            for (int c = b; c < C; ++c) {
                const double cand = best[c - b] + d;
                if (cand < nxt[c]) {
                    nxt[c] = cand;
                    arg[c] = static_cast<int8_t>(b);
                }
            }
        }
        best.swap(nxt);
    }
    int c_end = -1;
    double v_end = inf;
    for (int c = 0; c < C; ++c)
        if (best[c] < v_end) {
            v_end = best[c];
            c_end = c;
        }
    if (c_end < 0) return false;
    int c = c_end;
    for (int i = r - 1; i >= 0; --i) {
        int b = pick[static_cast<size_t>(i) * C + c];
        bits[i] = static_cast<uint8_t>(b);
        c -= b;
    }
    return c == 0;
}

int mixed_n_hi(int r, double hi_fraction, int group_size) {
    int n_hi = group_size * static_cast<int>(std::floor(hi_fraction * r / group_size + 0.5));
    return std::min(std::max(n_hi, 0), r);
}

int energy_rank(const double *lam, int n, double tau) {
    double total = 0.0;
    for (int i = 0; i < n; ++i) total += lam[i];
    if (total <= 0.0) return 1;
    double acc = 0.0;
    for (int k = 1; k <= n; ++k) {
        acc += lam[k - 1];
        if (acc >= tau * total) return k;
    }
    return n;
}

// ---------------------------------------------------------- eigensolver
// Symmetric eigendecomposition of the n x n row-major matrix A (destroyed):
// A = Q diag(w) Q^T.  Q^T is returned row-major in qt (row k = eigenvector of
// w[k]).  Householder tridiagonalisation with accumulated reflectors, then
// implicit symmetric QR steps with the Wilkinson shift on the tridiagonal
// (Golub and Van Loan, Matrix Computations, sections 8.3.1-8.3.3).
void sym_eig(std::vector<double> &A, int n, std::vector<double> &w, std::vector<double> &qt) {
    qt.assign(static_cast<size_t>(n) * n, 0.0);
    for (int i = 0; i < n; ++i) qt[static_cast<size_t>(i) * n + i] = 1.0;
    std::vector<double> v(n), p(n), z(n);
    auto a = [&](int i, int j) -> double & { return A[static_cast<size_t>(i) * n + j]; };
    for (int k = 0; k + 2 < n; ++k) {
        const int m = n - k - 1;                         // size of the trailing block
        double sigma = 0.0;
        for (int i = 0; i < m; ++i) sigma += a(k, k + 1 + i) * a(k, k + 1 + i);
        sigma = std::sqrt(sigma);
        if (sigma == 0.0) continue;
        const double x0 = a(k, k + 1);
        const double alpha = -std::copysign(sigma, x0);
        for (int i = 0; i < m; ++i) v[i] = a(k, k + 1 + i);
        v[0] -= alpha;
        double vn = 0.0;
        for (int i = 0; i < m; ++i) vn += v[i] * v[i];
        vn = std::sqrt(vn);
        if (vn == 0.0) continue;
        for (int i = 0; i < m; ++i) v[i] /= vn;
        // p = A_sub v, w = p - (v.p) v, A_sub -= 2 (v w^T + w v^T)
        double K = 0.0;
        for (int i = 0; i < m; ++i) {
            const double *row = &A[static_cast<size_t>(k + 1 + i) * n + k + 1];
            double s = 0.0;
            for (int j = 0; j < m; ++j) s += row[j] * v[j];
            p[i] = s;
            K += v[i] * s;
        }
        for (int i = 0; i < m; ++i) p[i] -= K * v[i];
        for (int i = 0; i < m; ++i) {
            double *row = &A[static_cast<size_t>(k + 1 + i) * n + k + 1];
            const double vi2 = 2.0 * v[i], pi2 = 2.0 * p[i];
            for (int j = 0; j < m; ++j) row[j] -= vi2 * p[j] + pi2 * v[j];
        }
        a(k, k + 1) = alpha;
        a(k + 1, k) = alpha;
        for (int i = 1; i < m; ++i) {
            a(k, k + 1 + i) = 0.0;
            a(k + 1 + i, k) = 0.0;
        }
        // accumulate Q <- Q H: rows k+1.. of Q^T get -2 v_j (v^T Q^T[k+1:, :])
        std::fill(z.begin(), z.end(), 0.0);
        for (int i = 0; i < m; ++i) {
            const double *row = &qt[static_cast<size_t>(k + 1 + i) * n];
            for (int j = 0; j < n; ++j) z[j] += v[i] * row[j];
        }
        for (int i = 0; i < m; ++i) {
            double *row = &qt[static_cast<size_t>(k + 1 + i) * n];
            const double f = 2.0 * v[i];
            for (int j = 0; j < n; ++j) row[j] -= f * z[j];
        }
    }
    std::vector<double> d(n), e(std::max(n - 1, 1), 0.0);
    double anorm = 0.0;
    for (int i = 0; i < n; ++i) {
        d[i] = a(i, i);
        if (i + 1 < n) e[i] = a(i, i + 1);
        anorm = std::max(anorm, std::fabs(d[i]) + (i + 1 < n ? std::fabs(e[i]) : 0.0) +
                                    (i > 0 ? std::fabs(e[i - 1]) : 0.0));
    }
    const double eps = std::numeric_limits<double>::epsilon();
    auto negligible = [&](int i) {
        return std::fabs(e[i]) <= eps * (std::fabs(d[i]) + std::fabs(d[i + 1])) ||
               std::fabs(e[i]) <= eps * eps * anorm;
    };
    int hi = n - 1;
    long iter = 0;
    const long max_iter = 64L * n + 64;
    while (hi > 0 && iter < max_iter) {
        if (negligible(hi - 1)) {
            e[hi - 1] = 0.0;
            --hi;
            continue;
        }
        int lo = hi - 1;
        while (lo > 0 && !negligible(lo - 1)) --lo;
        if (lo > 0) e[lo - 1] = 0.0;
        ++iter;
        const double dd = 0.5 * (d[hi - 1] - d[hi]);
        const double ee = e[hi - 1];
        const double denom = dd + std::copysign(std::hypot(dd, ee), dd);
        const double mu = d[hi] - ee * ee / denom;
        double x = d[lo] - mu, zb = e[lo];
        for (int k = lo; k < hi; ++k) {
            const double r = std::hypot(x, zb);
            const double c = (r == 0.0) ? 1.0 : x / r;
            const double s = (r == 0.0) ? 0.0 : zb / r;
            if (k > lo) e[k - 1] = r;
            const double aa = d[k], f = e[k], g = d[k + 1];
            d[k] = c * c * aa + 2.0 * c * s * f + s * s * g;
            d[k + 1] = s * s * aa - 2.0 * c * s * f + c * c * g;
            e[k] = (c * c - s * s) * f + c * s * (g - aa);
            if (k + 1 < hi) {
                const double bulge = s * e[k + 1];
                e[k + 1] = c * e[k + 1];
                x = e[k];
                zb = bulge;
            }
            double *rk = &qt[static_cast<size_t>(k) * n];
            double *rk1 = &qt[static_cast<size_t>(k + 1) * n];
            for (int j = 0; j < n; ++j) {
                const double q0 = rk[j], q1 = rk1[j];
                rk[j] = c * q0 + s * q1;
                rk1[j] = -s * q0 + c * q1;
            }
        }
    }
    w = d;
}

// ------------------------------------------------------------ unit fitting
struct UnitFit {
    std::vector<double> mean, lam;      // [dg]
    std::vector<double> vecs;           // [dg][dg] row k = eigenvector k (descending order)
    int rank = 0;
};

// Mean [dg] and 1/S covariance [dg][dg] of every unit's prefill rows.
struct Moments {
    explicit Moments(int64_t U) : mean(U), cov(U) {}
    std::vector<std::vector<double>> mean, cov;
};

struct FrozenParts;
// Fills qmin / qscale [U][rmax] (DP mode) from the frozen parts.
typedef std::function<int32_t(const FrozenParts &, std::vector<float> &, std::vector<float> &)> RangeFn;

// Reads unit u's prefill rows as float64, [S][dg], heads of the unit concatenated.
void load_unit_rows(const void *rows, int32_t dtype, int64_t B, int64_t H, int64_t S, int D, int hpu,
                    int64_t u, std::vector<double> &Y) {
    const int dg = D * hpu;
    const int64_t G = H / hpu;
    const int64_t b = u / G, g = u % G;
    Y.resize(static_cast<size_t>(S) * dg);
    for (int j = 0; j < hpu; ++j) {
        const int64_t h = g * hpu + j;
        const int64_t base = ((b * H + h) * S) * D;
        for (int64_t s = 0; s < S; ++s) {
            double *dst = &Y[static_cast<size_t>(s) * dg + static_cast<size_t>(j) * D];
            if (dtype == KVTC_F32) {
                const float *src = static_cast<const float *>(rows) + base + s * D;
                for (int d = 0; d < D; ++d) dst[d] = src[d];
            } else {
                const uint16_t *src = static_cast<const uint16_t *>(rows) + base + s * D;
                for (int d = 0; d < D; ++d) dst[d] = half_value(src[d]);
            }
        }
    }
}

// Mean and 1/S covariance of Y ([S][dg]); Y is centred in place.  Blocks of
// the upper triangle are accumulated with rank-4 updates.
void mean_cov(std::vector<double> &Y, int64_t S, int dg, std::vector<double> &mean,
              std::vector<double> &C, bool inner_parallel) {
    mean.assign(dg, 0.0);
    for (int64_t s = 0; s < S; ++s) {
        const double *y = &Y[static_cast<size_t>(s) * dg];
        for (int d = 0; d < dg; ++d) mean[d] += y[d];
    }
    for (int d = 0; d < dg; ++d) mean[d] /= static_cast<double>(S);
    for (int64_t s = 0; s < S; ++s) {
        double *y = &Y[static_cast<size_t>(s) * dg];
        for (int d = 0; d < dg; ++d) y[d] -= mean[d];
    }
    C.assign(static_cast<size_t>(dg) * dg, 0.0);
    constexpr int BS = 64;
    const int nb = (dg + BS - 1) / BS;
    std::vector<std::pair<int, int>> blocks;
    for (int bi = 0; bi < nb; ++bi)
        for (int bj = bi; bj < nb; ++bj) blocks.emplace_back(bi, bj);
    auto do_block = [&](int64_t t) {
        const int i0 = blocks[t].first * BS, j0 = blocks[t].second * BS;
        const int ni = std::min(BS, dg - i0), nj = std::min(BS, dg - j0);
        double acc[BS][BS] = {};
        int64_t s = 0;
        for (; s + 4 <= S; s += 4) {
            const double *y0 = &Y[static_cast<size_t>(s) * dg];
            const double *y1 = y0 + dg, *y2 = y1 + dg, *y3 = y2 + dg;
            for (int i = 0; i < ni; ++i) {
                const double a0 = y0[i0 + i], a1 = y1[i0 + i], a2 = y2[i0 + i], a3 = y3[i0 + i];
                double *row = acc[i];
                for (int j = 0; j < nj; ++j)
                    row[j] += a0 * y0[j0 + j] + a1 * y1[j0 + j] + a2 * y2[j0 + j] + a3 * y3[j0 + j];
            }
        }
        for (; s < S; ++s) {
            const double *y0 = &Y[static_cast<size_t>(s) * dg];
            for (int i = 0; i < ni; ++i)
                for (int j = 0; j < nj; ++j) acc[i][j] += y0[i0 + i] * y0[j0 + j];
        }
        for (int i = 0; i < ni; ++i)
            for (int j = 0; j < nj; ++j) {
                const double v = acc[i][j] / static_cast<double>(S);
                C[static_cast<size_t>(i0 + i) * dg + j0 + j] = v;
                C[static_cast<size_t>(j0 + j) * dg + i0 + i] = v;
            }
    };
    if (inner_parallel) {
        parallel_for(static_cast<int64_t>(blocks.size()), do_block);
    } else {
        for (size_t t = 0; t < blocks.size(); ++t) do_block(static_cast<int64_t>(t));
    }
}

// Eigenpairs sorted by descending eigenvalue, eigenvalues clamped at 0, each
// eigenvector signed so that its largest-magnitude entry (first on ties) is positive.
void eig_sorted(std::vector<double> &C, int dg, UnitFit &f) {
    std::vector<double> w, qt;
    sym_eig(C, dg, w, qt);
    std::vector<int> order(dg);
    for (int i = 0; i < dg; ++i) order[i] = i;
    std::stable_sort(order.begin(), order.end(), [&](int x, int y) { return w[x] > w[y]; });
    f.lam.resize(dg);
    f.vecs.resize(static_cast<size_t>(dg) * dg);
    for (int k = 0; k < dg; ++k) {
        f.lam[k] = std::max(w[order[k]], 0.0);
        const double *src = &qt[static_cast<size_t>(order[k]) * dg];
        int arg = 0;
        double big = -1.0;
        for (int d = 0; d < dg; ++d)
            if (std::fabs(src[d]) > big) {
                big = std::fabs(src[d]);
                arg = d;
            }
        const double sg = src[arg] < 0 ? -1.0 : 1.0;
        double *dst = &f.vecs[static_cast<size_t>(k) * dg];
        for (int d = 0; d < dg; ++d) dst[d] = sg * src[d];
    }
}

void range_from_minmax(double mn, double mx, int b, float *qmin, float *qscale);

// Frozen (min, scale) of every component with non-zero width, over the
// prefill latents (Y - mu32) . basis32 evaluated in float64.
void frozen_ranges(const std::vector<double> &Xraw, int64_t S, int dg, const float *mu32,
                   const float *basis32, int r, const uint8_t *bits, float *qmin, float *qscale,
                   bool inner_parallel) {
    std::vector<int> comps;
    for (int i = 0; i < r; ++i) {
        qmin[i] = 0.0f;
        qscale[i] = 0.0f;
        if (bits[i]) comps.push_back(i);
    }
    if (comps.empty()) return;
    const int nc = static_cast<int>(comps.size());
    const int64_t chunk = 512;
    const int64_t nchunks = (S + chunk - 1) / chunk;
    std::vector<double> lo(static_cast<size_t>(nchunks) * nc, std::numeric_limits<double>::infinity());
    std::vector<double> hi(static_cast<size_t>(nchunks) * nc, -std::numeric_limits<double>::infinity());
    std::vector<double> V(static_cast<size_t>(nc) * dg), mu(dg);
    for (int d = 0; d < dg; ++d) mu[d] = mu32[d];
    for (int c = 0; c < nc; ++c)
        for (int d = 0; d < dg; ++d)
            V[static_cast<size_t>(c) * dg + d] = basis32[static_cast<size_t>(comps[c]) * dg + d];
    auto do_chunk = [&](int64_t t) {
        std::vector<double> y(dg);
        double *l = &lo[static_cast<size_t>(t) * nc], *h = &hi[static_cast<size_t>(t) * nc];
        const int64_t s1 = std::min(S, (t + 1) * chunk);
        for (int64_t s = t * chunk; s < s1; ++s) {
            const double *x = &Xraw[static_cast<size_t>(s) * dg];
            for (int d = 0; d < dg; ++d) y[d] = x[d] - mu[d];
            for (int c = 0; c < nc; ++c) {
                const double *v = &V[static_cast<size_t>(c) * dg];
                double a0 = 0, a1 = 0, a2 = 0, a3 = 0;
                int d = 0;
                for (; d + 4 <= dg; d += 4) {
                    a0 += y[d] * v[d];
                    a1 += y[d + 1] * v[d + 1];
                    a2 += y[d + 2] * v[d + 2];
                    a3 += y[d + 3] * v[d + 3];
                }
                for (; d < dg; ++d) a0 += y[d] * v[d];
                const double val = (a0 + a1) + (a2 + a3);
                l[c] = std::min(l[c], val);
                h[c] = std::max(h[c], val);
            }
        }
    };
    if (inner_parallel) parallel_for(nchunks, do_chunk);
    else for (int64_t t = 0; t < nchunks; ++t) do_chunk(t);
    for (int c = 0; c < nc; ++c) {
        double mn = std::numeric_limits<double>::infinity(), mx = -mn;
        for (int64_t t = 0; t < nchunks; ++t) {
            mn = std::min(mn, lo[static_cast<size_t>(t) * nc + c]);
            mx = std::max(mx, hi[static_cast<size_t>(t) * nc + c]);
        }
        const int i = comps[c];
        range_from_minmax(mn, mx, bits[i], &qmin[i], &qscale[i]);
    }
}

// -------------------------------------------------------------- blob build
struct Layout {
    uint64_t off_unit, off_lambda, off_bits, off_qmin, off_qscale, off_mu, off_slot_comp,
        off_slot_bits, off_basis, off_qlo, off_qinv, off_w16, off_bias, off_kdesc, off_fslot, off_vdig, off_mv,
        total;
};

Layout plan_layout(int64_t U, int dg, int rmax, int kslots, int kfetch, bool digits) {
    Layout L{};
    uint64_t o = align_up(sizeof(kvtc_state_header), kSectionAlign);
    auto take = [&](uint64_t bytes) {
        uint64_t at = o;
        o = align_up(o + std::max<uint64_t>(bytes, 1), kSectionAlign);
        return at;
    };
    L.off_unit = take(U * sizeof(kvtc_unit_info));
    L.off_lambda = take(U * dg * sizeof(double));
    L.off_bits = take(U * rmax);
    L.off_qmin = take(U * rmax * sizeof(float));
    L.off_qscale = take(U * rmax * sizeof(float));
    L.off_mu = take(U * dg * sizeof(float));
    L.off_slot_comp = take(U * kslots * sizeof(int32_t));
    L.off_slot_bits = take(U * kslots * sizeof(uint32_t));
    L.off_basis = take(U * static_cast<uint64_t>(kslots) * dg * sizeof(float));
    L.off_qlo = take(U * kslots * sizeof(double));
    L.off_qinv = take(U * kslots * sizeof(double));
    L.off_w16 = take(U * static_cast<uint64_t>(kfetch) * dg * sizeof(uint16_t));
    L.off_bias = take(U * dg * sizeof(float));
    L.off_kdesc = take(U * static_cast<uint64_t>(kfetch / kKStep) * sizeof(uint32_t));
    L.off_fslot = take(U * static_cast<uint64_t>(kfetch) * sizeof(int32_t));
    if (digits) {
        L.off_vdig = take(U * 5 * static_cast<uint64_t>(kslots) * dg);
        L.off_mv = take(U * static_cast<uint64_t>(kslots) * sizeof(double));
    }
    L.total = o;
    return L;
}

// Builds the blob from per-unit frozen parts.  bits is ignored (recomputed)
// in mixed mode.  Returns a status; writes only when state_out is large enough.
int32_t build_blob(const kvtc_config *cfg, int64_t B, int64_t H, int32_t rmax, const int32_t *ranks,
                   const float *mu, const float *basis, const double *lambda, const uint8_t *bits_in,
                   const float *qmin, const float *qscale, int64_t s_prefill, void *state_out,
                   size_t *state_bytes) {
    const int hpu = cfg->heads_per_unit;
    const int dg = cfg->head_dim * hpu;
    const int64_t U = B * (H / hpu);
    std::vector<uint8_t> bits(static_cast<size_t>(U) * rmax, 0);
    std::vector<int> n_slots(U), row_bits(U);
    int n_hi = 0;
    for (int64_t u = 0; u < U; ++u) {
        const int r = ranks[u];
        if (r < 1 || r > rmax) return KVTC_E_ARG;
        uint8_t *bu = &bits[static_cast<size_t>(u) * rmax];
        if (cfg->mode == KVTC_MODE_DP) {
            for (int i = 0; i < r; ++i) {
                const int b = bits_in[static_cast<size_t>(u) * rmax + i];
                if (!width_allowed(b)) return KVTC_E_ARG;
                bu[i] = static_cast<uint8_t>(b);
            }
        } else {
            if (r != rmax) return KVTC_E_ARG;            // one stored rank for every group
            n_hi = mixed_n_hi(r, cfg->hi_fraction, cfg->group_size);
            for (int i = 0; i < r; ++i) bu[i] = static_cast<uint8_t>(i < n_hi ? cfg->hi_bits : cfg->lo_bits);
        }
        int ns = 0, rb = 0;
        for (int i = 0; i < r; ++i)
            if (bu[i]) {
                ++ns;
                rb += bu[i];
            }
        n_slots[u] = ns;
        row_bits[u] = rb;
    }
    int max_slots = 0, max_bits = 0;
    for (int64_t u = 0; u < U; ++u) {
        max_slots = std::max(max_slots, n_slots[u]);
        max_bits = std::max(max_bits, row_bits[u]);
    }
    if (max_bits > 0xFFFF) return KVTC_E_CONFIG;
    // fetch k-steps: every run of equal widths among the stored slots is padded
    // to a whole number of 16-slot k-steps, so each k-step has one width
    std::vector<int> n_ksteps(U, 0);
    for (int64_t u = 0; u < U; ++u) {
        const uint8_t *bu = &bits[static_cast<size_t>(u) * rmax];
        int run = 0, prev = -1, steps = 0;
        for (int i = 0; i < ranks[u]; ++i) {
            if (!bu[i]) continue;
            if (bu[i] != prev) {
                steps += (run + kKStep - 1) / kKStep;
                run = 0;
                prev = bu[i];
            }
            ++run;
        }
        steps += (run + kKStep - 1) / kKStep;
        n_ksteps[u] = steps;
    }
    int max_steps = 1;
    for (int64_t u = 0; u < U; ++u) max_steps = std::max(max_steps, n_ksteps[u]);
    const int kslots = std::max<int>(kSlotAlign, static_cast<int>(align_up(max_slots, kSlotAlign)));
    const int kfetch = kKStep * max_steps;
    // the int8 append's digit planes exist when every kept basis entry is at
    // most 1 in magnitude (always so for an orthonormal basis)
    bool digits = true;
    for (int64_t u = 0; u < U && digits; ++u)
        for (int i = 0; i < ranks[u] && digits; ++i) {
            const float *src = &basis[(static_cast<size_t>(u) * rmax + i) * dg];
            for (int d = 0; d < dg; ++d)
                if (!(std::fabs(src[d]) <= 1.0f)) {
                    digits = false;
                    break;
                }
        }
    const Layout L = plan_layout(U, dg, rmax, kslots, kfetch, digits);
    if (state_out == nullptr || *state_bytes < L.total) {
        *state_bytes = L.total;
        return state_out == nullptr ? KVTC_OK : KVTC_E_BUFSIZE;
    }
    *state_bytes = L.total;
    std::memset(state_out, 0, L.total);
    auto *h = static_cast<kvtc_state_header *>(state_out);
    h->magic = KVTC_MAGIC;
    h->version = KVTC_VERSION;
    h->mode = cfg->mode;
    h->head_dim = cfg->head_dim;
    h->heads_per_unit = hpu;
    h->dg = dg;
    h->batch = B;
    h->heads = H;
    h->units = U;
    h->rmax = rmax;
    h->kslots = kslots;
    h->row_stride = 4 * ((max_bits + 31) / 32);
    h->n_qgroups = cfg->mode == KVTC_MODE_MIXED ? (rmax + cfg->group_size - 1) / cfg->group_size : 0;
    h->group_size = cfg->group_size;
    h->hi_bits = cfg->hi_bits;
    h->lo_bits = cfg->lo_bits;
    h->n_hi = n_hi;
    h->bit_budget = cfg->bit_budget;
    h->n_choices = cfg->n_choices;
    for (int i = 0; i < KVTC_MAX_CHOICES; ++i) h->choices[i] = cfg->choices[i];
    h->beta = cfg->beta;
    h->energy_threshold = cfg->energy_threshold;
    h->rank_cfg = cfg->rank;
    h->kfetch = kfetch;
    h->s_prefill = s_prefill;
    h->off_unit = L.off_unit;
    h->off_lambda = L.off_lambda;
    h->off_bits = L.off_bits;
    h->off_qmin = L.off_qmin;
    h->off_qscale = L.off_qscale;
    h->off_mu = L.off_mu;
    h->off_slot_comp = L.off_slot_comp;
    h->off_slot_bits = L.off_slot_bits;
    h->off_basis = L.off_basis;
    h->off_qlo = L.off_qlo;
    h->off_qinv = L.off_qinv;
    h->off_w16 = L.off_w16;
    h->off_bias = L.off_bias;
    h->off_kdesc = L.off_kdesc;
    h->off_fslot = L.off_fslot;
    h->off_vdig = L.off_vdig;
    h->off_mv = L.off_mv;
    h->total_bytes = L.total;

    auto *ui = section_mut<kvtc_unit_info>(state_out, L.off_unit);
    auto *lam_o = section_mut<double>(state_out, L.off_lambda);
    auto *bits_o = section_mut<uint8_t>(state_out, L.off_bits);
    auto *qmin_o = section_mut<float>(state_out, L.off_qmin);
    auto *qscale_o = section_mut<float>(state_out, L.off_qscale);
    auto *mu_o = section_mut<float>(state_out, L.off_mu);
    auto *scomp = section_mut<int32_t>(state_out, L.off_slot_comp);
    auto *sbits = section_mut<uint32_t>(state_out, L.off_slot_bits);
    auto *sbasis = section_mut<float>(state_out, L.off_basis);
    auto *sqlo = section_mut<double>(state_out, L.off_qlo);
    auto *sqinv = section_mut<double>(state_out, L.off_qinv);
    auto *w16 = section_mut<uint16_t>(state_out, L.off_w16);
    auto *bias = section_mut<float>(state_out, L.off_bias);
    auto *kdesc = section_mut<uint32_t>(state_out, L.off_kdesc);
    auto *fslot = section_mut<int32_t>(state_out, L.off_fslot);
    auto *vdig = digits ? section_mut<int8_t>(state_out, L.off_vdig) : nullptr;
    auto *mv = digits ? section_mut<double>(state_out, L.off_mv) : nullptr;

    parallel_for(U, [&](int64_t u) {
        const int r = ranks[u];
        ui[u].rank = r;
        ui[u].n_slots = n_slots[u];
        ui[u].row_bits = row_bits[u];
        for (int d = 0; d < dg; ++d) {
            mu_o[u * dg + d] = mu[u * dg + d];
            lam_o[u * dg + d] = lambda ? lambda[u * dg + d] : 0.0;
        }
        const uint8_t *bu = &bits[static_cast<size_t>(u) * rmax];
        for (int kk = 0; kk < kfetch; ++kk) fslot[static_cast<size_t>(u) * kfetch + kk] = -1;
        std::vector<double> bacc(dg);
        for (int d = 0; d < dg; ++d) bacc[d] = mu[u * dg + d];
        int j = 0;
        uint32_t off = 0;
        int k = 0;               // next fetch slot (16-aligned at every width change)
        int prev_w = -1;
        int in_step = 0;
        for (int i = 0; i < rmax; ++i) {
            const size_t ci = static_cast<size_t>(u) * rmax + i;
            bits_o[ci] = bu[i];
            if (cfg->mode == KVTC_MODE_DP && i < r && bu[i]) {
                qmin_o[ci] = qmin[ci];
                qscale_o[ci] = qscale[ci];
            }
            if (i >= r || bu[i] == 0) continue;
            const size_t sj = static_cast<size_t>(u) * kslots + j;
            scomp[sj] = i;
            sbits[sj] = (off & kOffsetMask) | (static_cast<uint32_t>(bu[i]) << 24);
            const float *src = &basis[(static_cast<size_t>(u) * rmax + i) * dg];
            float *dst = &sbasis[sj * dg];
            for (int d = 0; d < dg; ++d) dst[d] = src[d];
            if (digits) {
                // rint(basis * 2^38) in five balanced base-256 digits, low digit first;
                // |basis| <= 1 keeps the top digit within [-64, 64].  The slot's offset
                // is mean . basis minus the constant the row digits leave out:
                // the int8 append forms a row's digits from X ^ 0x808080, whose bytes
                // as int8 sum to X - 0x808080 (X = x * 2^24).
                double m = 0.0;
                int64_t vsum = 0;
                for (int d = 0; d < dg; ++d) {
                    const int64_t vq = std::llrint(std::ldexp(static_cast<double>(src[d]), 38));
                    vsum += vq;
                    int64_t q = vq;
                    for (int k = 0; k < 5; ++k) {
                        const int64_t dk = static_cast<int8_t>(static_cast<uint8_t>(q & 0xFF));
                        vdig[((static_cast<size_t>(u) * 5 + k) * kslots + j) * dg + d] = static_cast<int8_t>(dk);
                        q = (q - dk) / 256;
                    }
                    m += static_cast<double>(mu[u * dg + d]) * static_cast<double>(src[d]);
                }
                mv[sj] = m - std::ldexp(static_cast<double>(vsum) * 8421504.0, -62);   // 8421504 = 0x808080
            }
            double wscale = 1.0;
            if (cfg->mode == KVTC_MODE_DP) {
                sqlo[sj] = static_cast<double>(qmin[ci]);
                sqinv[sj] = qscale[ci] > 0.0f ? 1.0 / static_cast<double>(qscale[ci]) : 0.0;
                wscale = static_cast<double>(qscale[ci]);
                for (int d = 0; d < dg; ++d) bacc[d] += static_cast<double>(qmin[ci]) * src[d];
            }
            if (bu[i] != prev_w || in_step == kKStep) {
                if (in_step) k = static_cast<int>(align_up(k, kKStep));
                const uint32_t qg = cfg->mode == KVTC_MODE_MIXED ? static_cast<uint32_t>(j / cfg->group_size) : 0u;
                kdesc[static_cast<size_t>(u) * (kfetch / kKStep) + k / kKStep] =
                    (off & 0xFFFFu) | (static_cast<uint32_t>(bu[i]) << 16) | (qg << 20);
                prev_w = bu[i];
                in_step = 0;
            }
            // position of this slot in the k-step: 4-bit halves arrive
            // nibble-interleaved, 2-bit k-steps in the byte-lane order
            int kk = k;
            if (bu[i] == 4) {
                const int e = in_step % 8;
                int p = 0;
                while (kNibbleOrder[p] != e) ++p;
                kk = k - e + p;
            } else if (bu[i] == 2) {
                kk = k - in_step + kTwoBitOrder[in_step];
            }
            for (int d = 0; d < dg; ++d)
                w16[(static_cast<size_t>(u) * dg + d) * kfetch + kk] =
                    half_bits_rne(wscale * static_cast<double>(src[d]));
            fslot[static_cast<size_t>(u) * kfetch + kk] = j;
            off += bu[i];
            ++k;
            ++in_step;
            ++j;
        }
        for (; j < kslots; ++j) scomp[static_cast<size_t>(u) * kslots + j] = -1;
        for (int d = 0; d < dg; ++d) bias[u * dg + d] = static_cast<float>(bacc[d]);
    });
    return KVTC_OK;
}

// ----------------------------------------------------------------- Huffman
// Total bits of an optimal prefix code for the given symbol counts: the sum of
// the internal-node weights of a Huffman tree (one bit each for a lone symbol).
uint64_t huffman_bits(const uint64_t *counts, int n) {
    std::priority_queue<uint64_t, std::vector<uint64_t>, std::greater<uint64_t>> q;
    for (int i = 0; i < n; ++i)
        if (counts[i]) q.push(counts[i]);
    if (q.empty()) return 0;
    if (q.size() == 1) return q.top();
    uint64_t total = 0;
    while (q.size() > 1) {
        const uint64_t a = q.top();
        q.pop();
        const uint64_t b = q.top();
        q.pop();
        total += a + b;
        q.push(a + b);
    }
    return total;
}

// ------------------------------------------------------------ fit core
// The fit after the per-unit moments, shared by the host and the device fits:
// eigenpairs, rank, fp32 mean and basis, DP allocation, ranges, blob.
struct FrozenParts {
    int rmax = 0;
    std::vector<int32_t> ranks;        // [U]
    std::vector<float> mu;             // [U][dg]
    std::vector<float> basis;          // [U][rmax][dg] row i = component i
    std::vector<double> lam;           // [U][dg]
    std::vector<uint8_t> bits;         // [U][rmax]
};

int32_t fit_from_moments(const kvtc_config *cfg, int64_t B, int64_t H, int64_t S, Moments &m, const RangeFn &ranges,
                         void *state_out, size_t *state_bytes) {
    const int hpu = cfg->heads_per_unit, dg = cfg->head_dim * hpu;
    const int64_t U = B * (H / hpu);
    std::vector<UnitFit> fits(U);
    if (!parallel_for(U, [&](int64_t u) {
            fits[u].mean = std::move(m.mean[u]);
            eig_sorted(m.cov[u], dg, fits[u]);
            std::vector<double>().swap(m.cov[u]);
        }))
        return KVTC_E_ARG;
    // rank per unit (mixed mode stores one rank for every group)
    FrozenParts fp;
    for (int64_t u = 0; u < U; ++u) {
        fits[u].rank = cfg->rank > 0 ? cfg->rank : energy_rank(fits[u].lam.data(), dg, cfg->energy_threshold);
        fp.rmax = std::max(fp.rmax, fits[u].rank);
    }
    if (cfg->mode == KVTC_MODE_MIXED)
        for (auto &f : fits) f.rank = fp.rmax;
    const int rmax = fp.rmax;
    fp.ranks.resize(U);
    fp.mu.resize(static_cast<size_t>(U) * dg);
    fp.basis.assign(static_cast<size_t>(U) * rmax * dg, 0.f);
    fp.lam.resize(static_cast<size_t>(U) * dg);
    fp.bits.assign(static_cast<size_t>(U) * rmax, 0);
    std::vector<int> choices(cfg->choices, cfg->choices + cfg->n_choices);
    std::atomic<bool> feasible{true};
    if (!parallel_for(U, [&](int64_t u) {
            const UnitFit &f = fits[u];
            const int r = f.rank;
            fp.ranks[u] = r;
            for (int d = 0; d < dg; ++d) {
                fp.mu[u * dg + d] = static_cast<float>(f.mean[d]);
                fp.lam[u * dg + d] = f.lam[d];
            }
            for (int i = 0; i < r; ++i)
                for (int d = 0; d < dg; ++d)
                    fp.basis[(static_cast<size_t>(u) * rmax + i) * dg + d] =
                        static_cast<float>(f.vecs[static_cast<size_t>(i) * dg + d]);
            if (cfg->mode == KVTC_MODE_DP &&
                !dp_allocate(f.lam.data(), r, cfg->bit_budget, choices, cfg->beta, &fp.bits[static_cast<size_t>(u) * rmax]))
                feasible = false;
        }))
        return KVTC_E_ARG;
    if (!feasible) return KVTC_E_CONFIG;
    std::vector<float> qmin(static_cast<size_t>(U) * rmax, 0.f), qscale(static_cast<size_t>(U) * rmax, 0.f);
    if (cfg->mode == KVTC_MODE_DP) {
        const int32_t st = ranges(fp, qmin, qscale);
        if (st != KVTC_OK) return st;
    }
    return build_blob(cfg, B, H, rmax, fp.ranks.data(), fp.mu.data(), fp.basis.data(), fp.lam.data(), fp.bits.data(),
                      qmin.data(), qscale.data(), S, state_out, state_bytes);
}

// (min, scale) of a component of width b from the float64 min and max of its
// latents, stored as fp32 (a constant component gets scale 0).
void range_from_minmax(double mn, double mx, int b, float *qmin, float *qscale) {
    *qmin = static_cast<float>(mn);
    *qscale = mx > mn ? static_cast<float>((mx - mn) / static_cast<double>((1 << b) - 1)) : 0.0f;
}

// ------------------------------------------------------------ entropy coding
// Code lengths of an optimal prefix code for counts[0..n) (the depths of a
// Huffman tree's leaves; 0 for absent symbols, 1 for a lone symbol).  Nodes
// merge lowest weight first, ties towards the lower node index (symbols are
// nodes 0..n-1, merged nodes n, n+1, ... in creation order).  Returns the
// longest length.
int huffman_code_lengths(const uint32_t *counts, int n, uint8_t *len) {
    std::fill(len, len + n, 0);
    typedef std::pair<uint64_t, int> Node;               // (weight, index)
    std::priority_queue<Node, std::vector<Node>, std::greater<Node>> q;
    for (int i = 0; i < n; ++i)
        if (counts[i]) q.push({counts[i], i});
    if (q.empty()) return 0;
    if (q.size() == 1) {
        len[q.top().second] = 1;
        return 1;
    }
    std::vector<int> parent(2 * n, -1);
    int next = n;
    while (q.size() > 1) {
        const Node a = q.top();
        q.pop();
        const Node b = q.top();
        q.pop();
        parent[a.second] = next;
        parent[b.second] = next;
        q.push({a.first + b.first, next++});
    }
    // depths: a merged node's parent was created after it, so walk from the root down
    std::vector<int> depth(next, 0);
    for (int v = next - 2; v >= n; --v) depth[v] = depth[parent[v]] + 1;
    int longest = 0;
    for (int i = 0; i < n; ++i)
        if (counts[i]) {
            const int d = depth[parent[i]] + 1;
            len[i] = static_cast<uint8_t>(std::min(d, 255));
            longest = std::max(longest, d);
        }
    return longest;
}

// The encoder's shape of a DP tensor over S rows: symbol position of each slot
// (prefix of 2^b in slot order), symbol positions per unit, chunks.
struct EntropyShape {
    std::vector<uint32_t> sym_off;     // [U][kslots]
    int nsym = 1, nchunks = 0;
};

EntropyShape entropy_shape(const kvtc_state_header *h, const void *blob, int64_t S) {
    EntropyShape e;
    const auto *ui = section<kvtc_unit_info>(blob, h->off_unit);
    const auto *sb = section<uint32_t>(blob, h->off_slot_bits);
    e.sym_off.assign(static_cast<size_t>(h->units) * h->kslots, 0);
    for (int64_t u = 0; u < h->units; ++u) {
        uint32_t o = 0;
        for (int j = 0; j < ui[u].n_slots; ++j) {
            e.sym_off[u * h->kslots + j] = o;
            o += 1u << (sb[u * h->kslots + j] >> 24);
        }
        e.nsym = std::max<int>(e.nsym, static_cast<int>(o));
    }
    e.nchunks = static_cast<int>((S + kEntropyChunk - 1) / kEntropyChunk);
    return e;
}

// Upper bound of the archive: the fixed-width parts of all units, whole words.
uint64_t entropy_archive_bound(const kvtc_state_header *h, const void *blob, int64_t S) {
    const auto *ui = section<kvtc_unit_info>(blob, h->off_unit);
    uint64_t b = 0;
    for (int64_t u = 0; u < h->units; ++u) b += (static_cast<uint64_t>(S) * ui[u].row_bits + 7) / 8;
    return align_up(b + 4, 4);
}

}  // namespace
}  // namespace kvtc

using namespace kvtc;

#ifndef KVTC_BUILD_ID
#define KVTC_BUILD_ID "0000000000000000"
#endif
// The hash of the sources the library was built from, behind a fixed marker so
// that a build script can read it from the file without loading the library.
static const char kBuildIdTag[] = "kvtc-build-id:" KVTC_BUILD_ID;

// =========================================================== C entry points
extern "C" {

const char *kvtc_build_id(void) { return kBuildIdTag + 14; }

void kvtc_config_default(kvtc_config *cfg, int32_t mode, int32_t head_dim) {
    if (!cfg) return;
    std::memset(cfg, 0, sizeof(*cfg));
    cfg->mode = mode;
    cfg->head_dim = head_dim;
    cfg->heads_per_unit = mode == KVTC_MODE_MIXED ? 8 : 1;
    cfg->rank = mode == KVTC_MODE_MIXED ? 0 : head_dim;
    cfg->energy_threshold = 0.90;
    cfg->bit_budget = 4 * head_dim;
    const int32_t ch[] = {0, 1, 2, 3, 4, 8};
    cfg->n_choices = 6;
    for (int i = 0; i < 6; ++i) cfg->choices[i] = ch[i];
    cfg->beta = 1.0;
    cfg->hi_bits = 4;
    cfg->lo_bits = 2;
    cfg->group_size = 32;
    cfg->hi_fraction = 0.25;
}

const char *kvtc_status_string(int32_t s) {
    switch (s) {
        case KVTC_OK: return "ok";
        case KVTC_E_CONFIG: return "invalid or infeasible configuration";
        case KVTC_E_SHAPE: return "shape, stride or alignment mismatch";
        case KVTC_E_DTYPE: return "unsupported dtype";
        case KVTC_E_CAPACITY: return "rows outside the store capacity";
        case KVTC_E_STATE: return "missing, unfitted or corrupt state";
        case KVTC_E_BUFSIZE: return "output buffer too small";
        case KVTC_E_DEVICE: return "HIP device error";
        case KVTC_E_ARG: return "invalid argument";
        default: return "unknown status";
    }
}

int32_t kvtc_allocate_bits(const double *lambda, int32_t r, int32_t budget, const int32_t *choices,
                           int32_t n_choices, double beta, uint8_t *bits_out) {
    if (!lambda || !choices || !bits_out || r < 1 || n_choices < 1 || n_choices > KVTC_MAX_CHOICES)
        return KVTC_E_ARG;
    if (budget < 0) return KVTC_E_CONFIG;
    std::vector<int> ch(choices, choices + n_choices);
    for (int b : ch)
        if (!width_allowed(b)) return KVTC_E_CONFIG;
    try {
        std::vector<uint8_t> tmp(r);
        if (!dp_allocate(lambda, r, budget, ch, beta, tmp.data())) return KVTC_E_CONFIG;
        std::memcpy(bits_out, tmp.data(), r);
    } catch (const std::bad_alloc &) {
        return KVTC_E_ARG;
    }
    return KVTC_OK;
}

int32_t kvtc_fit_host(const kvtc_config *cfg, const void *rows_host, int32_t dtype, int64_t B,
                      int64_t H, int64_t S, void *state_out, size_t *state_bytes) {
    int32_t st = validate_config(cfg);
    if (st != KVTC_OK) return st;
    if (!rows_host || !state_bytes) return KVTC_E_ARG;
    if (dtype != KVTC_F32 && dtype != KVTC_F16) return KVTC_E_DTYPE;
    if (B < 1 || H < 1 || H % cfg->heads_per_unit != 0) return KVTC_E_SHAPE;
    if (S < 2) return KVTC_E_CONFIG;                      // fit needs a prefill with S > 1
    const int hpu = cfg->heads_per_unit, D = cfg->head_dim, dg = D * hpu;
    const int64_t U = B * (H / hpu);
    try {
        // 1. mean and covariance per unit
        Moments m(U);
        if (U >= num_threads()) {
            if (!parallel_for(U, [&](int64_t u) {
                    std::vector<double> Y;
                    load_unit_rows(rows_host, dtype, B, H, S, D, hpu, u, Y);
                    mean_cov(Y, S, dg, m.mean[u], m.cov[u], false);
                }))
                return KVTC_E_ARG;
        } else {
            // few units: parallelise the covariance inside a unit
            for (int64_t u = 0; u < U; ++u) {
                std::vector<double> Y;
                load_unit_rows(rows_host, dtype, B, H, S, D, hpu, u, Y);
                mean_cov(Y, S, dg, m.mean[u], m.cov[u], true);
            }
        }
        // 2.-4. eigenpairs, rank, allocation; ranges over the prefill latents on the host
        const RangeFn ranges = [&](const FrozenParts &fp, std::vector<float> &qmin, std::vector<float> &qscale) {
            const bool inner = U < num_threads();
            auto one = [&](int64_t u) {
                std::vector<double> X;
                load_unit_rows(rows_host, dtype, B, H, S, D, hpu, u, X);
                frozen_ranges(X, S, dg, &fp.mu[u * dg], &fp.basis[static_cast<size_t>(u) * fp.rmax * dg], fp.ranks[u],
                              &fp.bits[static_cast<size_t>(u) * fp.rmax], &qmin[static_cast<size_t>(u) * fp.rmax],
                              &qscale[static_cast<size_t>(u) * fp.rmax], inner);
            };
            if (inner) {
                for (int64_t u = 0; u < U; ++u) one(u);
                return KVTC_OK;
            }
            return parallel_for(U, one) ? KVTC_OK : KVTC_E_ARG;
        };
        return fit_from_moments(cfg, B, H, S, m, ranges, state_out, state_bytes);
    } catch (const std::bad_alloc &) {
        return KVTC_E_ARG;
    }
}

int32_t kvtc_fit_bytes_bound(const kvtc_config *cfg, int64_t B, int64_t H, size_t *bytes) {
    int32_t st = validate_config(cfg);
    if (st != KVTC_OK) return st;
    if (!bytes) return KVTC_E_ARG;
    if (B < 1 || H < 1 || H % cfg->heads_per_unit != 0) return KVTC_E_SHAPE;
    const int dg = cfg->head_dim * cfg->heads_per_unit;
    const int64_t U = B * (H / cfg->heads_per_unit);
    const int rmax = cfg->rank > 0 ? cfg->rank : dg;
    const int kslots = std::max<int>(kSlotAlign, static_cast<int>(align_up(rmax, kSlotAlign)));
    // every run of equal widths is padded to whole k-steps: at most one run per
    // stored slot in DP mode, two runs (hi, lo) in mixed mode
    const int kfetch = cfg->mode == KVTC_MODE_MIXED ? kslots + 2 * kKStep : kKStep * kslots;
    *bytes = plan_layout(U, dg, rmax, kslots, kfetch, true).total;   // the bound includes the digit planes
    return KVTC_OK;
}

namespace {
// Slot capacity of the device fit's range pass: the configured rank (or the
// unit width) rounded up to 16; group-head tensors need no ranges.
int fit_device_kslots(const kvtc_config *cfg) {
    if (cfg->mode != KVTC_MODE_DP) return 0;
    const int dg = cfg->head_dim * cfg->heads_per_unit;
    return static_cast<int>(align_up(cfg->rank > 0 ? cfg->rank : dg, kSlotAlign));
}
}  // namespace

int32_t kvtc_fit_workspace(const kvtc_config *cfg, int64_t B, int64_t H, int64_t S, size_t *bytes) {
    int32_t st = validate_config(cfg);
    if (st != KVTC_OK) return st;
    if (!bytes) return KVTC_E_ARG;
    if (B < 1 || H < 1 || H % cfg->heads_per_unit != 0) return KVTC_E_SHAPE;
    if (S < 2) return KVTC_E_CONFIG;
    const int dg = cfg->head_dim * cfg->heads_per_unit;
    const int64_t U = B * (H / cfg->heads_per_unit);
    *bytes = fit_device_layout(U, dg, S, fit_device_kslots(cfg)).total;
    return KVTC_OK;
}

int32_t kvtc_fit_device(const kvtc_config *cfg, const void *rows_dev, int32_t dtype, const int64_t strides[4],
                        int64_t B, int64_t H, int64_t S, void *work_dev, size_t work_bytes, void *state_out,
                        size_t *state_bytes, void *hip_stream) {
    int32_t st = validate_config(cfg);
    if (st != KVTC_OK) return st;
    if (!rows_dev || !strides || !state_bytes) return KVTC_E_ARG;
    if (dtype != KVTC_F32 && dtype != KVTC_F16) return KVTC_E_DTYPE;
    if (B < 1 || H < 1 || H % cfg->heads_per_unit != 0) return KVTC_E_SHAPE;
    if (strides[3] != 1 || strides[0] < 0 || strides[1] < 0 || strides[2] < 0) return KVTC_E_SHAPE;
    if (S < 2) return KVTC_E_CONFIG;                      // fit needs a prefill with S > 1
    const int hpu = cfg->heads_per_unit, D = cfg->head_dim, dg = D * hpu;
    const int64_t U = B * (H / hpu);
    const int ks = fit_device_kslots(cfg);
    if (U > 65535 || ks > 256) return KVTC_E_SHAPE;
    const FitDeviceLayout L = fit_device_layout(U, dg, S, ks);
    if (!work_dev || work_bytes < L.total || reinterpret_cast<uintptr_t>(work_dev) % kSectionAlign)
        return KVTC_E_BUFSIZE;
    FitDeviceRows r{};
    r.rows = rows_dev;
    r.dtype = dtype;
    r.sb = strides[0];
    r.sh = strides[1];
    r.ss = strides[2];
    r.B = B;
    r.H = H;
    r.S = S;
    r.D = D;
    r.hpu = hpu;
    r.dg = dg;
    r.units = U;
    r.kslots = ks;
    r.work = work_dev;
    r.stream = hip_stream;
    try {
        // 1. mean and covariance per unit, on the device
        std::vector<double> mean(static_cast<size_t>(U) * dg), cov(static_cast<size_t>(U) * dg * dg);
        st = fit_device_moments(r, mean.data(), cov.data());
        if (st != KVTC_OK) return st;
        Moments m(U);
        if (!parallel_for(U, [&](int64_t u) {
                m.mean[u].assign(mean.begin() + u * dg, mean.begin() + (u + 1) * dg);
                m.cov[u].assign(cov.begin() + u * dg * dg, cov.begin() + (u + 1) * dg * dg);
            }))
            return KVTC_E_ARG;
        std::vector<double>().swap(cov);
        // 2.-4. eigenpairs, rank, allocation on the host; ranges over the prefill latents on the device
        const RangeFn ranges = [&](const FrozenParts &fp, std::vector<float> &qmin, std::vector<float> &qscale) {
            if (fp.rmax > ks) return KVTC_E_SHAPE;
            std::vector<float> bs(static_cast<size_t>(U) * ks * dg, 0.f);
            std::vector<int32_t> ns(U, 0);
            for (int64_t u = 0; u < U; ++u)
                for (int i = 0; i < fp.ranks[u]; ++i)
                    if (fp.bits[static_cast<size_t>(u) * fp.rmax + i]) {
                        std::memcpy(&bs[(static_cast<size_t>(u) * ks + ns[u]) * dg],
                                    &fp.basis[(static_cast<size_t>(u) * fp.rmax + i) * dg], dg * sizeof(float));
                        ++ns[u];
                    }
            std::vector<double> mn(static_cast<size_t>(U) * ks), mx(static_cast<size_t>(U) * ks);
            const int32_t s2 = fit_device_ranges(r, fp.mu.data(), bs.data(), ns.data(), mn.data(), mx.data());
            if (s2 != KVTC_OK) return s2;
            for (int64_t u = 0; u < U; ++u) {
                int j = 0;
                for (int i = 0; i < fp.ranks[u]; ++i) {
                    const size_t ci = static_cast<size_t>(u) * fp.rmax + i;
                    if (!fp.bits[ci]) continue;
                    const size_t sj = static_cast<size_t>(u) * ks + j++;
                    range_from_minmax(mn[sj], mx[sj], fp.bits[ci], &qmin[ci], &qscale[ci]);
                }
            }
            return KVTC_OK;
        };
        return fit_from_moments(cfg, B, H, S, m, ranges, state_out, state_bytes);
    } catch (const std::bad_alloc &) {
        return KVTC_E_ARG;
    }
}

// ------------------------------------------------------------ entropy-coded storage
int32_t kvtc_entropy_bytes(const void *state_host, int64_t S, size_t *work_bytes, size_t *archive_bytes,
                           size_t *index_bytes) {
    const kvtc_state_header *h = nullptr;
    int32_t st = check_state(state_host, &h);
    if (st != KVTC_OK) return st;
    if (h->mode != KVTC_MODE_DP) return KVTC_E_STATE;
    if (S < 0) return KVTC_E_ARG;
    try {
        const EntropyShape e = entropy_shape(h, state_host, S);
        if (work_bytes) *work_bytes = entropy_work_layout(h->units, h->kslots, e.nsym, e.nchunks).total;
        if (archive_bytes) *archive_bytes = entropy_archive_bound(h, state_host, S);
        if (index_bytes) *index_bytes = entropy_index_layout(h->units, h->kslots, e.nsym, e.nchunks).total;
    } catch (const std::bad_alloc &) {
        return KVTC_E_ARG;
    }
    return KVTC_OK;
}

int32_t kvtc_entropy_encode(const void *state_host, const void *state_dev, const void *codes_dev, int64_t capacity,
                            int64_t S, void *work_dev, size_t work_bytes, void *archive_dev, size_t archive_bytes,
                            void *index_host, size_t index_bytes, void *hip_stream) {
    const kvtc_state_header *h = nullptr;
    int32_t st = check_state(state_host, &h);
    if (st != KVTC_OK) return st;
    if (h->mode != KVTC_MODE_DP) return KVTC_E_STATE;
    if (!state_dev || !index_host) return KVTC_E_ARG;
    if (S < 0 || capacity < 0) return KVTC_E_ARG;
    if (S > capacity) return KVTC_E_CAPACITY;
    if (h->units > 65535) return KVTC_E_SHAPE;
    if (S > 0 && h->row_stride > 0 && (!codes_dev || reinterpret_cast<uintptr_t>(codes_dev) % 4)) return KVTC_E_ARG;
    try {
        const EntropyShape e = entropy_shape(h, state_host, S);
        const int64_t U = h->units;
        const int ks = h->kslots, nsym = e.nsym, nch = e.nchunks;
        const EntropyWorkLayout W = entropy_work_layout(U, ks, nsym, nch);
        const EntropyIndexLayout I = entropy_index_layout(U, ks, nsym, nch);
        const uint64_t bound = entropy_archive_bound(h, state_host, S);
        if (!work_dev || work_bytes < W.total || reinterpret_cast<uintptr_t>(work_dev) % kSectionAlign) return KVTC_E_BUFSIZE;
        if (!archive_dev || archive_bytes < bound || reinterpret_cast<uintptr_t>(archive_dev) % 4) return KVTC_E_BUFSIZE;
        if (index_bytes < I.total) return KVTC_E_BUFSIZE;
        const auto *ui = section<kvtc_unit_info>(state_host, h->off_unit);
        const auto *sbh = section<uint32_t>(state_host, h->off_slot_bits);
        const char *sd = static_cast<const char *>(state_dev);
        char *w = static_cast<char *>(work_dev);
        EntropyDevArgs a{};
        a.ui = reinterpret_cast<const kvtc_unit_info *>(sd + h->off_unit);
        a.sbits = reinterpret_cast<const uint32_t *>(sd + h->off_slot_bits);
        a.codes = static_cast<uint8_t *>(const_cast<void *>(codes_dev));
        a.capacity = capacity;
        a.S = S;
        a.units = U;
        a.kslots = ks;
        a.row_stride = h->row_stride;
        a.nsym = nsym;
        a.nchunks = nch;
        a.sym_off = reinterpret_cast<const uint32_t *>(w + W.sym_off);
        a.counts = reinterpret_cast<uint32_t *>(w + W.counts);
        a.enc_code = reinterpret_cast<const uint32_t *>(w + W.enc_code);
        a.enc_len = reinterpret_cast<const uint8_t *>(w + W.enc_len);
        a.unit = reinterpret_cast<const kvtc_entropy_unit *>(w + W.units);
        a.slot_pos = reinterpret_cast<const uint64_t *>(w + W.slot_pos);
        a.chunk_bits = reinterpret_cast<uint32_t *>(w + W.chunk_bits);
        a.chunk_pos = reinterpret_cast<uint64_t *>(w + W.chunk_pos);
        a.archive = static_cast<uint32_t *>(archive_dev);
        a.archive_words = archive_bytes / 4;
        a.stream = hip_stream;
        // 1. counts of every slot's codes over rows [0, S), on the device
        std::vector<uint32_t> counts(static_cast<size_t>(U) * nsym);
        if (fit_device_upload(w + W.sym_off, e.sym_off.data(), e.sym_off.size() * 4, hip_stream) != KVTC_OK)
            return KVTC_E_DEVICE;
        st = entropy_device_counts(a, counts.data());
        if (st != KVTC_OK) return st;
        // 2. code lengths, canonical codes and decode tables per slot; the unit forms
        std::memset(index_host, 0, I.total);
        auto *hdr = static_cast<kvtc_entropy_header *>(index_host);
        auto *units = section_mut<kvtc_entropy_unit>(index_host, I.off_unit);
        auto *dec = section_mut<kvtc_entropy_dec>(index_host, I.off_dec);
        auto *syms = section_mut<uint8_t>(index_host, I.off_syms);
        auto *chunk = section_mut<uint64_t>(index_host, I.off_chunk);
        std::vector<uint32_t> enc_code(static_cast<size_t>(U) * nsym, 0);
        std::vector<uint8_t> enc_len(static_cast<size_t>(U) * nsym, 0);
        std::vector<uint64_t> slot_bits(static_cast<size_t>(U) * ks, 0), slot_pos(static_cast<size_t>(U) * ks, 0);
        std::atomic<bool> too_long{false};
        if (!parallel_for(U, [&](int64_t u) {
                for (int j = 0; j < ui[u].n_slots; ++j) {
                    const int b = static_cast<int>(sbh[u * ks + j] >> 24), n = 1 << b;
                    const size_t so = static_cast<size_t>(u) * nsym + e.sym_off[u * ks + j];
                    const int longest = huffman_code_lengths(&counts[so], n, &enc_len[so]);
                    if (longest > KVTC_ENTROPY_MAX_LEN) {
                        too_long = true;
                        return;
                    }
                    kvtc_entropy_dec &d = dec[u * ks + j];
                    d.sym_off = e.sym_off[u * ks + j];
                    d.max_len = static_cast<uint32_t>(longest);
                    for (int k = 0; k < n; ++k) d.count[enc_len[so + k]] += enc_len[so + k] ? 1 : 0;
                    uint32_t code = 0, idx = 0;
                    for (int L = 1; L <= KVTC_ENTROPY_MAX_LEN; ++L) {
                        d.first[L] = code;
                        d.base[L] = static_cast<uint16_t>(idx);
                        code = (code + d.count[L]) << 1;
                        idx += d.count[L];
                    }
                    // symbols in (length, value) order take consecutive codes
                    std::vector<uint32_t> next(d.first, d.first + KVTC_ENTROPY_MAX_LEN + 1);
                    std::vector<uint16_t> put(d.base, d.base + KVTC_ENTROPY_MAX_LEN + 1);
                    uint64_t bits = 0;
                    for (int L = 1; L <= KVTC_ENTROPY_MAX_LEN; ++L)
                        for (int k = 0; k < n; ++k)
                            if (enc_len[so + k] == L) {
                                const uint32_t c = next[L]++;
                                syms[static_cast<size_t>(u) * nsym + d.sym_off + put[L]++] = static_cast<uint8_t>(k);
                                uint32_t rev = 0;                 // emitted most significant bit first
                                for (int t = 0; t < L; ++t) rev |= ((c >> t) & 1u) << (L - 1 - t);
                                enc_code[so + k] = rev;
                                bits += static_cast<uint64_t>(counts[so + k]) * L;
                            }
                    slot_bits[u * ks + j] = bits;
                }
            }))
            return KVTC_E_ARG;
        if (too_long) return KVTC_E_SHAPE;
        uint64_t off = 0, payload = 0, tables = 0;
        int64_t coded_units = 0;
        for (int64_t u = 0; u < U; ++u) {
            uint64_t hbits = 0, table = 0;
            for (int j = 0; j < ui[u].n_slots; ++j) {
                hbits += slot_bits[u * ks + j];
                table += 1ull << (sbh[u * ks + j] >> 24);
            }
            const uint64_t fixed = (static_cast<uint64_t>(S) * ui[u].row_bits + 7) / 8;
            const uint64_t coded_payload = (hbits + 7) / 8;
            kvtc_entropy_unit &un = units[u];
            un.offset = off;
            un.table_bytes = static_cast<uint32_t>(table);
            un.coded = coded_payload + table < fixed ? 1u : 0u;
            un.bytes = un.coded ? table + coded_payload : fixed;
            if (un.coded) {
                uint64_t p = 8 * (off + table);
                for (int j = 0; j < ui[u].n_slots; ++j) {
                    slot_pos[u * ks + j] = p;
                    p += slot_bits[u * ks + j];
                }
                payload += coded_payload;
                tables += table;
                ++coded_units;
            } else {
                payload += fixed;
            }
            off += un.bytes;
        }
        hdr->magic = KVTC_ENTROPY_MAGIC;
        hdr->version = KVTC_ENTROPY_VERSION;
        hdr->S = S;
        hdr->units = U;
        hdr->kslots = ks;
        hdr->chunk_rows = kEntropyChunk;
        hdr->nchunks = nch;
        hdr->nsym = nsym;
        hdr->archive_bytes = off;
        hdr->payload_bytes = payload;
        hdr->table_bytes = tables;
        hdr->units_coded = coded_units;
        hdr->off_unit = I.off_unit;
        hdr->off_dec = I.off_dec;
        hdr->off_syms = I.off_syms;
        hdr->off_chunk = I.off_chunk;
        hdr->total_bytes = I.total;
        // 3. the archive, on the device; the chunk positions come back into the index
        return entropy_device_encode(a, enc_code.data(), enc_len.data(), units, slot_pos.data(), chunk);
    } catch (const std::bad_alloc &) {
        return KVTC_E_ARG;
    }
}

int32_t kvtc_entropy_decode(const void *state_host, const void *state_dev, const void *index_host,
                            const void *index_dev, const void *archive_dev, void *codes_dev, int64_t capacity,
                            void *hip_stream) {
    const kvtc_state_header *h = nullptr;
    int32_t st = check_state(state_host, &h);
    if (st != KVTC_OK) return st;
    if (h->mode != KVTC_MODE_DP) return KVTC_E_STATE;
    if (!state_dev || !index_host || !index_dev || reinterpret_cast<uintptr_t>(index_dev) % 16) return KVTC_E_ARG;
    const auto *hdr = static_cast<const kvtc_entropy_header *>(index_host);
    if (hdr->magic != KVTC_ENTROPY_MAGIC || hdr->version != KVTC_ENTROPY_VERSION || hdr->units != h->units ||
        hdr->kslots != h->kslots || hdr->chunk_rows != kEntropyChunk || hdr->S < 0 ||
        hdr->nchunks != (hdr->S + kEntropyChunk - 1) / kEntropyChunk)
        return KVTC_E_STATE;
    try {
        const EntropyShape e = entropy_shape(h, state_host, hdr->S);
        const EntropyIndexLayout I = entropy_index_layout(h->units, h->kslots, e.nsym, e.nchunks);
        if (hdr->nsym != e.nsym || hdr->off_unit != I.off_unit || hdr->off_dec != I.off_dec ||
            hdr->off_syms != I.off_syms || hdr->off_chunk != I.off_chunk || hdr->total_bytes != I.total ||
            hdr->archive_bytes > entropy_archive_bound(h, state_host, hdr->S))
            return KVTC_E_STATE;
    } catch (const std::bad_alloc &) {
        return KVTC_E_ARG;
    }
    if (capacity < 0) return KVTC_E_ARG;
    if (hdr->S > capacity) return KVTC_E_CAPACITY;
    if (hdr->S == 0) return KVTC_OK;
    if (h->row_stride > 0 && (!codes_dev || reinterpret_cast<uintptr_t>(codes_dev) % 4)) return KVTC_E_ARG;
    if (!archive_dev || reinterpret_cast<uintptr_t>(archive_dev) % 4) return KVTC_E_ARG;
    if (h->units > 65535) return KVTC_E_SHAPE;
    const char *sd = static_cast<const char *>(state_dev);
    const char *ix = static_cast<const char *>(index_dev);
    EntropyDevArgs a{};
    a.ui = reinterpret_cast<const kvtc_unit_info *>(sd + h->off_unit);
    a.sbits = reinterpret_cast<const uint32_t *>(sd + h->off_slot_bits);
    a.codes = static_cast<uint8_t *>(codes_dev);
    a.capacity = capacity;
    a.S = hdr->S;
    a.units = h->units;
    a.kslots = h->kslots;
    a.row_stride = h->row_stride;
    a.nsym = hdr->nsym;
    a.nchunks = hdr->nchunks;
    a.unit = reinterpret_cast<const kvtc_entropy_unit *>(ix + hdr->off_unit);
    a.dec = reinterpret_cast<const kvtc_entropy_dec *>(ix + hdr->off_dec);
    a.syms = reinterpret_cast<const uint8_t *>(ix + hdr->off_syms);
    a.chunk_pos = reinterpret_cast<uint64_t *>(const_cast<char *>(ix + hdr->off_chunk));
    a.archive = static_cast<uint32_t *>(const_cast<void *>(archive_dev));
    a.archive_words = (hdr->archive_bytes + 3) / 4;
    a.stream = hip_stream;
    return entropy_device_decode(a);
}

int32_t kvtc_state_build(const kvtc_config *cfg, int64_t B, int64_t H, int32_t rmax,
                         const int32_t *ranks, const float *mu, const float *basis,
                         const double *lambda, const uint8_t *bits, const float *qmin,
                         const float *qscale, int64_t s_prefill, void *state_out,
                         size_t *state_bytes) {
    int32_t st = validate_config(cfg);
    if (st != KVTC_OK) return st;
    if (!ranks || !mu || !basis || !state_bytes) return KVTC_E_ARG;
    if (cfg->mode == KVTC_MODE_DP && (!bits || !qmin || !qscale)) return KVTC_E_ARG;
    if (B < 1 || H < 1 || H % cfg->heads_per_unit != 0) return KVTC_E_SHAPE;
    if (rmax < 1 || rmax > cfg->head_dim * cfg->heads_per_unit) return KVTC_E_CONFIG;
    try {
        return build_blob(cfg, B, H, rmax, ranks, mu, basis, lambda, bits, qmin, qscale, s_prefill,
                          state_out, state_bytes);
    } catch (const std::bad_alloc &) {
        return KVTC_E_ARG;
    }
}

int32_t kvtc_store_bytes(const void *state_host, int64_t capacity, size_t *codes_bytes,
                         size_t *params_bytes) {
    const kvtc_state_header *h = nullptr;
    int32_t st = check_state(state_host, &h);
    if (st != KVTC_OK) return st;
    if (capacity < 0) return KVTC_E_ARG;
    if (codes_bytes) *codes_bytes = static_cast<size_t>(h->units) * capacity * h->row_stride;
    if (params_bytes)
        *params_bytes = static_cast<size_t>(h->units) * capacity * h->n_qgroups * 4;
    return KVTC_OK;
}

int32_t kvtc_bytes(const void *state_host, const void *codes_host, const void *params_host,
                   int64_t capacity, int64_t S, kvtc_bytes_report *out) {
    const kvtc_state_header *h = nullptr;
    int32_t st = check_state(state_host, &h);
    if (st != KVTC_OK) return st;
    if (!out || (S > 0 && h->row_stride > 0 && !codes_host)) return KVTC_E_ARG;
    if (S < 0 || S > capacity) return KVTC_E_CAPACITY;
    (void)params_host;
    const int64_t U = h->units;
    const int dg = h->dg;
    const auto *ui = section<kvtc_unit_info>(state_host, h->off_unit);
    const auto *sbits = section<uint32_t>(state_host, h->off_slot_bits);
    const uint8_t *codes = static_cast<const uint8_t *>(codes_host);
    struct Per {
        uint64_t fixed, payload, table, side, basis, qp, coded;
    };
    std::vector<Per> per(U);
    try {
        bool ok = parallel_for(U, [&](int64_t u) {
            Per p{};
            const int ns = ui[u].n_slots, rb = ui[u].row_bits;
            p.fixed = (static_cast<uint64_t>(S) * rb + 7) / 8;
            if (h->mode == KVTC_MODE_DP) {
                p.basis = 2ull * (static_cast<uint64_t>(dg) * ns + dg);
                p.qp = 4ull * ns;
                uint64_t hb = 0, table = 0;
                std::vector<uint64_t> counts(256);
                for (int j = 0; j < ns; ++j) {
                    const uint32_t sb = sbits[static_cast<size_t>(u) * h->kslots + j];
                    const uint32_t off = sb & kOffsetMask, w = sb >> 24;
                    std::fill(counts.begin(), counts.end(), 0);
                    for (int64_t s = 0; s < S; ++s) {
                        const uint8_t *row = codes + (static_cast<size_t>(u) * capacity + s) * h->row_stride;
                        uint32_t c = 0;
                        for (uint32_t k = 0; k < w; ++k) {
                            const uint32_t bit = off + k;
                            c |= static_cast<uint32_t>((row[bit >> 3] >> (bit & 7)) & 1u) << k;
                        }
                        ++counts[c];
                    }
                    hb += huffman_bits(counts.data(), 1 << w);
                    table += 1ull << w;
                }
                const uint64_t payload = (hb + 7) / 8;
                if (payload + table < p.fixed) {
                    p.payload = payload;
                    p.table = table;
                    p.coded = 1;
                } else {
                    p.payload = p.fixed;
                }
            } else {
                p.basis = 4ull * (static_cast<uint64_t>(dg) * ui[u].rank + dg);
                p.qp = 4ull * static_cast<uint64_t>(S) * h->n_qgroups;
                p.payload = p.fixed;
            }
            per[u] = p;
        });
        if (!ok) return KVTC_E_ARG;
    } catch (const std::bad_alloc &) {
        return KVTC_E_ARG;
    }
    kvtc_bytes_report r{};
    for (int64_t u = 0; u < U; ++u) {
        const Per &p = per[u];
        r.fixed_payload += p.fixed;
        if (p.coded) {
            r.entropy_payload += p.payload;
            r.entropy_table += p.table;
            r.units_entropy_coded += 1;
        }
        r.stored_payload += p.payload;
        r.basis += p.basis;
        r.quant_params += p.qp;
        r.total += p.payload + p.table + p.basis + p.qp;
        r.pre_entropy += p.fixed + p.basis + p.qp;
        r.n_survived += ui[u].n_slots;
    }
    r.fp16_equiv = static_cast<uint64_t>(h->batch) * h->heads * S * h->head_dim * 2;
    r.device_store = static_cast<uint64_t>(U) * S * (h->row_stride + 4ull * h->n_qgroups);
    *out = r;
    return KVTC_OK;
}

}  // extern "C"
