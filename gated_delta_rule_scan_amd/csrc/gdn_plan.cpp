// Checkpoint placement for sparse prefix caching, host only.
//
// "Sparse prefix caching for hybrid and recurrent LLM serving" §3 states the
// problem: a cached prefix of N tokens keeps exact states at M positions
// 1 <= c_1 < ... < c_M <= N; a request that matches the prefix to depth d
// resumes from the deepest c_j <= d (none: the zero state, c_0 = 0) and
// recomputes d - c_j tokens.  With depths d ~ p on 0..N the expected
// recomputation is
//     R(p, C) = sum_d p(d) (d - max({0} u {c_i <= d})),
// which is the page's R(p, g) written with the positions c_i = sum_{j<=i} g_j
// instead of the gaps g (the gaps sum to N + 1, the last one ending at the
// sentinel N + 1).  Its §4 gives
//  - Theorem 1: for uniform p on 1..N the optimal gaps differ by at most one;
//    gdn_balanced_checkpoints builds such a set, c_i = floor(i (N+1) / (M+1));
//  - Theorem 2: for any p an O(N M) dynamic programme over the last
//    checkpoint, made linear per level by the convex hull trick.
//
// The programme.  With P0(x) = sum_{d<x} p(d) and P1(x) = sum_{d<x} d p(d), a
// gap that starts at checkpoint a and ends before the next boundary b costs
//     cost(a, b) = sum_{d=a}^{b-1} p(d) (d - a) = P1(b) - P1(a) - a (P0(b) - P0(a)).
// F_0(b) = cost(0, b); F_k(b) = min_{k <= a < b} F_{k-1}(a) + cost(a, b) is the
// least cost of depths 0..b-1 with k checkpoints, the k-th at a; the answer is
// F_M(N + 1).  Expanding cost(a, b),
//     F_k(b) = P1(b) + min_a [ y_a - a P0(b) ],  y_a = F_{k-1}(a) - P1(a) + a P0(a),
// a minimum over lines of slope -a evaluated at x = P0(b).  Lines arrive in
// order of decreasing slope (a grows with b) and the queries x = P0(b) never
// decrease (p >= 0), so a deque of the lower envelope answers each level in
// O(N) total.
#include <cmath>
#include <cstdint>
#include <vector>

#include "../../include/gdnreplay.h"
#include "gdn_error.h"

#define GDN_API extern "C" __attribute__((visibility("default")))

namespace {

// p must be finite and non-negative on 0..N.
bool valid_distribution(const double *p, int64_t N) {
    for (int64_t d = 0; d <= N; ++d)
        if (!(p[d] >= 0.0) || !std::isfinite(p[d])) return false;
    return true;
}

// Largest prefix and argmin table (entries) the planner keeps.
constexpr int64_t kMaxTable = int64_t(1) << 28;

}  // namespace

GDN_API double gdn_expected_recompute(const double *p, int64_t N, const int64_t *pos, int32_t M) {
    if (!p || N < 0 || M < 0 || (M > 0 && !pos) || !valid_distribution(p, N)) return -1.0;
    for (int32_t i = 0; i < M; ++i)
        if (pos[i] < 1 || pos[i] > N || (i > 0 && pos[i] <= pos[i - 1])) return -1.0;
    double r = 0.0;
    int64_t last = 0;  // deepest checkpoint at or before d (c_0 = 0)
    int32_t j = 0;
    for (int64_t d = 0; d <= N; ++d) {
        while (j < M && pos[j] <= d) last = pos[j++];
        r += p[d] * (double)(d - last);
    }
    return r;
}

GDN_API int32_t gdn_balanced_checkpoints(int64_t N, int32_t M, int64_t *pos_out) {
    if (N < 0 || M < 0 || M > N || (M > 0 && !pos_out)) return -1;
    // c_i = floor(i (N + 1) / (M + 1)): gaps floor/ceil of (N + 1) / (M + 1)
    for (int32_t i = 1; i <= M; ++i) {
        const __int128 num = (__int128)i * (N + 1);
        pos_out[i - 1] = (int64_t)(num / (M + 1));
    }
    return 0;
}

GDN_API gdn_status gdn_plan_checkpoints(const double *p, int64_t N, int32_t M, int64_t *pos_out,
                                        double *cost_out) {
    if (!p) return gdn::host_fail(GDN_ERR_INVALID_ARGUMENT, "p is NULL");
    if (N < 1) return gdn::host_fail(GDN_ERR_INVALID_ARGUMENT, "N = %lld must be >= 1", (long long)N);
    if (N + 2 > kMaxTable)
        return gdn::host_fail(GDN_ERR_UNSUPPORTED, "N = %lld exceeds the planner's limit %lld", (long long)N,
                              (long long)(kMaxTable - 2));
    if (M < 0 || M > N)
        return gdn::host_fail(GDN_ERR_INVALID_ARGUMENT, "M = %d must lie in 0..N (N = %lld)", M, (long long)N);
    if (M > 0 && !pos_out) return gdn::host_fail(GDN_ERR_INVALID_ARGUMENT, "pos_out is NULL");
    if (!valid_distribution(p, N))
        return gdn::host_fail(GDN_ERR_INVALID_ARGUMENT, "p must be finite and non-negative on 0..N");
    if ((int64_t)M * (N + 2) > kMaxTable)
        return gdn::host_fail(GDN_ERR_UNSUPPORTED, "M (N + 2) = %lld exceeds the planner's table limit %lld",
                              (long long)M * (N + 2), (long long)kMaxTable);

    const int64_t E = N + 1;  // boundaries b run over 1..E; E is the sentinel after depth N
    std::vector<double> P0(E + 1, 0.0), P1(E + 1, 0.0);
    for (int64_t d = 0; d <= N; ++d) {
        P0[d + 1] = P0[d] + p[d];
        P1[d + 1] = P1[d] + (double)d * p[d];
    }
    auto cost = [&](int64_t a, int64_t b) { return (P1[b] - P1[a]) - (double)a * (P0[b] - P0[a]); };

    std::vector<double> prev(E + 1), cur(E + 1);
    for (int64_t b = 1; b <= E; ++b) prev[b] = cost(0, b);
    // arg[k-1][b]: position of the k-th checkpoint in the best F_k(b)
    std::vector<int32_t> arg((size_t)M * (E + 1), 0);
    std::vector<int64_t> hull((size_t)E + 1);
    std::vector<double> hy((size_t)E + 1);

    for (int32_t k = 1; k <= M; ++k) {
        // lines a = k .. E-1, slope -a, intercept y_a; queries b = k+1 .. E
        int64_t head = 0, tail = 0;
        int32_t *argk = &arg[(size_t)(k - 1) * (E + 1)];
        auto y_of = [&](int64_t a) { return prev[a] - P1[a] + (double)a * P0[a]; };
        for (int64_t b = k + 1; b <= E; ++b) {
            // add the line of a = b - 1 (smallest slope so far)
            const int64_t a = b - 1;
            const double ya = y_of(a);
            // drop the last hull line while it is nowhere below both neighbours
            while (tail - head >= 2) {
                const int64_t a1 = hull[tail - 2], a2 = hull[tail - 1];
                const long double y1 = hy[tail - 2], y2 = hy[tail - 1];
                // line 2 is useless if the intersection of 1 and 3 lies at or
                // left of that of 1 and 2 (slopes -a1 > -a2 > -a)
                const long double lhs = ((long double)ya - y1) * (long double)(a2 - a1);
                const long double rhs = (y2 - y1) * (long double)(a - a1);
                if (lhs <= rhs) --tail;
                else break;
            }
            hull[tail] = a;
            hy[tail] = ya;
            ++tail;
            // query x = P0(b); the envelope's minimum moves right as x grows
            const double x = P0[b];
            while (tail - head >= 2 && hy[head + 1] - (double)hull[head + 1] * x <= hy[head] - (double)hull[head] * x)
                ++head;
            cur[b] = P1[b] + hy[head] - (double)hull[head] * x;
            argk[b] = (int32_t)hull[head];
        }
        prev.swap(cur);
    }

    // backtrack from the sentinel
    int64_t b = E;
    for (int32_t k = M; k >= 1; --k) {
        const int64_t a = arg[(size_t)(k - 1) * (E + 1) + b];
        pos_out[k - 1] = a;
        b = a;
    }
    if (cost_out) *cost_out = prev[E];
    return GDN_OK;
}
