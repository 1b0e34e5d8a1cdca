// Token-slicing plan of a token-level pipeline and its slice-latency model
// (host code).
//
// "TeraPipe: Token-Level Pipeline Parallelism for Training Large-Scale
// Language Models" (summary page), section 3, selecting the slicing scheme:
// the slice lengths l_1..l_M (sum L) are chosen by dynamic programming to
// minimise the forward-plus-backward latency of the pipeline; a slice's
// latency is its forward time without extra context plus a context overhead
// predicted by a linear model fitted on a subset of measured combinations.
//
// Latency of a plan over K stages whose every stage takes t_i for slice i:
// sum_i t_i + (K - 1) max_i t_i (the last slice leaves the last stage then).
// Search: for each candidate largest slice latency c (each distinct cost,
// increasing), the least sum of slice latencies with every slice <= c, by a
// prefix dynamic program; plan latency = that sum + (K - 1) c.  Since a
// plan's latency is at least K times its largest slice, candidates stop once
// K c reaches the best latency found.
#include <algorithm>
#include <cmath>
#include <limits>
#include <vector>

#include "tpshard.h"

// the library's error reporting (thread-local message) lives in api.cpp
extern "C" tp_status tp_internal_fail(tp_status s, const char *msg);

namespace {

tp_status set_error(tp_status s, const char *msg) { return tp_internal_fail(s, msg); }

}  // namespace

extern "C" {

tp_status tp_fit_context_model(int32_t n, const int32_t *len, const int32_t *offset, const double *ctx,
                               double coef[3]) {
    if (n < 3) return set_error(TP_EINVAL, "at least 3 samples are needed");
    if (!len || !offset || !ctx || !coef) return set_error(TP_EINVAL, "NULL argument");
    // normal equations of ctx ~ a_lo * l * o + a_o * o + a_1, with the
    // columns scaled to unit maximum for conditioning
    double scale[3] = {0, 0, 1};
    for (int i = 0; i < n; ++i) {
        if (len[i] <= 0 || offset[i] < 0 || !std::isfinite(ctx[i]))
            return set_error(TP_EINVAL, "samples need len > 0, offset >= 0 and finite times");
        scale[0] = std::max(scale[0], (double)len[i] * offset[i]);
        scale[1] = std::max(scale[1], (double)offset[i]);
    }
    if (scale[0] == 0 || scale[1] == 0) return set_error(TP_EINVAL, "the samples need some context (offset > 0)");
    double M[3][4] = {};
    for (int i = 0; i < n; ++i) {
        const double x[3] = {(double)len[i] * offset[i] / scale[0], (double)offset[i] / scale[1], 1.0};
        for (int r = 0; r < 3; ++r) {
            for (int c = 0; c < 3; ++c) M[r][c] += x[r] * x[c];
            M[r][3] += x[r] * ctx[i];
        }
    }
    // Gaussian elimination with partial pivoting
    for (int c = 0; c < 3; ++c) {
        int p = c;
        for (int r = c + 1; r < 3; ++r)
            if (std::fabs(M[r][c]) > std::fabs(M[p][c])) p = r;
        if (std::fabs(M[p][c]) < 1e-300) return set_error(TP_EINVAL, "the samples do not determine the model");
        for (int k = 0; k < 4; ++k) std::swap(M[c][k], M[p][k]);
        for (int r = 0; r < 3; ++r) {
            if (r == c) continue;
            const double f = M[r][c] / M[c][c];
            for (int k = c; k < 4; ++k) M[r][k] -= f * M[c][k];
        }
    }
    for (int r = 0; r < 3; ++r) coef[r] = M[r][3] / M[r][r] / scale[r];
    return TP_OK;
}

tp_status tp_slice_cost_table(int32_t units, int32_t granularity, const double *fwd, const double coef[3],
                              double *cost) {
    if (units < 1 || granularity < 1) return set_error(TP_EINVAL, "units and granularity must be positive");
    if (!fwd || !coef || !cost) return set_error(TP_EINVAL, "NULL argument");
    const int W = units + 1;
    for (int a = 0; a <= units; ++a)
        for (int b = 0; b <= units; ++b) {
            double v = std::numeric_limits<double>::infinity();
            if (a < b) {
                const double l = (double)(b - a) * granularity, o = (double)a * granularity;
                v = fwd[b - a];
                // the context term is a latency: a fitted line that
                // extrapolates below zero adds nothing
                if (a > 0) v += std::max(0.0, coef[0] * l * o + coef[1] * o + coef[2]);
            }
            cost[a * W + b] = v;
        }
    return TP_OK;
}

tp_status tp_plan_latency(int32_t units, const double *cost, int32_t stages, int32_t num_slices, const int32_t *ends,
                          double *latency) {
    if (units < 1 || units > 4096) return set_error(TP_EINVAL, "units must be in [1, 4096]");
    if (stages < 1) return set_error(TP_EINVAL, "stages must be positive");
    if (num_slices < 1) return set_error(TP_EINVAL, "a plan has at least one slice");
    if (!cost || !ends || !latency) return set_error(TP_EINVAL, "NULL argument");
    const int W = units + 1;
    double sum = 0.0, mx = 0.0;
    int a = 0;
    for (int i = 0; i < num_slices; ++i) {
        const int b = ends[i];
        if (b <= a || b > units) return set_error(TP_EINVAL, "slice ends must increase within [1, units]");
        const double t = cost[a * W + b];
        if (!(t >= 0) || std::isnan(t)) return set_error(TP_EINVAL, "slice costs must be >= 0 (or +inf)");
        sum += t;
        mx = std::max(mx, t);
        a = b;
    }
    if (a != units) return set_error(TP_EINVAL, "the last slice must end at units");
    *latency = sum + (double)(stages - 1) * mx;
    return TP_OK;
}

tp_status tp_slicing_plan(int32_t units, const double *cost, int32_t stages, int32_t *num_slices, int32_t *ends,
                          double *latency) {
    if (units < 1 || units > 4096) return set_error(TP_EINVAL, "units must be in [1, 4096]");
    if (stages < 1) return set_error(TP_EINVAL, "stages must be positive");
    if (!cost || !num_slices || !ends || !latency) return set_error(TP_EINVAL, "NULL argument");
    const int W = units + 1;
    std::vector<double> cands;
    cands.reserve((size_t)units * W / 2);
    for (int a = 0; a < units; ++a)
        for (int b = a + 1; b <= units; ++b) {
            const double c = cost[a * W + b];
            if (!(c >= 0) || std::isnan(c)) return set_error(TP_EINVAL, "slice costs must be >= 0 (or +inf)");
            if (std::isfinite(c)) cands.push_back(c);
        }
    std::sort(cands.begin(), cands.end());
    cands.erase(std::unique(cands.begin(), cands.end()), cands.end());
    double best_lat = std::numeric_limits<double>::infinity();
    std::vector<int> best_ends;
    std::vector<double> best(W);
    std::vector<int> arg(W);
    for (double c : cands) {
        if ((double)stages * c >= best_lat) break;
        std::fill(best.begin(), best.end(), std::numeric_limits<double>::infinity());
        std::fill(arg.begin(), arg.end(), -1);
        best[0] = 0.0;
        for (int b = 1; b <= units; ++b)
            for (int a = 0; a < b; ++a) {
                const double t = cost[a * W + b];
                if (t <= c && best[a] + t < best[b]) {
                    best[b] = best[a] + t;
                    arg[b] = a;
                }
            }
        if (!std::isfinite(best[units])) continue;
        const double lat = best[units] + (double)(stages - 1) * c;
        if (lat < best_lat) {
            best_lat = lat;
            best_ends.clear();
            for (int b = units; b > 0; b = arg[b]) best_ends.push_back(b);
            std::reverse(best_ends.begin(), best_ends.end());
        }
    }
    if (best_ends.empty()) return set_error(TP_EINVAL, "no plan has finite latency");
    *num_slices = (int32_t)best_ends.size();
    for (size_t i = 0; i < best_ends.size(); ++i) ends[i] = best_ends[i];
    *latency = best_lat;
    return TP_OK;
}

}  // extern "C"
