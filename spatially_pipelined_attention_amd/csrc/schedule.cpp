// The execution model's timing and allocation search on the host: equation
// 1 (segment-to-stage binding), equations 4-5 (max-plus makespan of the
// augmented task DAG), the counts behind equation 7, and the pairwise-line
// allocation refinement of section 4.2 (Algorithm 2) of the SubGPU Pipelining
// paper. The tuner uses the same refinement with measured iteration times as
// the objective.
#include <string.h>

#include <algorithm>
#include <limits>
#include <vector>

#include "host.h"

using namespace spa;

static int64_t binom(int64_t n, int64_t k) {
  if (k < 0 || k > n) return 0;
  k = std::min(k, n - k);
  __int128 r = 1;
  for (int64_t i = 1; i <= k; ++i) {
    r = r * (n - k + i) / i;
    if (r > (__int128)std::numeric_limits<int64_t>::max()) return -1;
  }
  return (int64_t)r;
}

extern "C" {

int32_t spa_sched_binding(int32_t k, int32_t K, int32_t w) { return (w == 1 && k == K) ? 1 : k; }

spa_status spa_sched_makespan(int32_t n_regions, int32_t n_micro, int32_t K, int32_t w, const double* tau,
                              double* makespan, double* start_out, double* end_out) {
  if (n_regions < 1 || n_micro < 1 || K < 1 || (w != 0 && w != 1) || !tau || !makespan)
    return fail(SPA_EINVAL, "bad argument");
  if (w == 1 && K < 2) return fail(SPA_EINVAL, "boundary reuse needs K >= 2");
  const size_t n = (size_t)n_regions * n_micro * K;
  std::vector<double> C(n, 0.0);
  std::vector<long long> last_on_stage(K + 1, -1);
  double T = 0.0;
  // dispatch order: region, then microbatch, then segment (topological)
  for (int l = 0; l < n_regions; ++l)
    for (int mu = 0; mu < n_micro; ++mu)
      for (int k = 1; k <= K; ++k) {
        const size_t i = ((size_t)l * n_micro + mu) * K + (k - 1);
        double a = 0.0;
        if (k > 1) a = std::max(a, C[i - 1]);
        else if (l > 0) a = std::max(a, C[(((size_t)(l - 1) * n_micro + mu) * K) + (K - 1)]);
        const int st = spa_sched_binding(k, K, w);
        if (last_on_stage[st] >= 0) a = std::max(a, C[(size_t)last_on_stage[st]]);
        C[i] = a + tau[i];
        last_on_stage[st] = (long long)i;
        if (start_out) start_out[i] = a;
        if (end_out) end_out[i] = C[i];
        T = std::max(T, C[i]);
      }
  *makespan = T;
  return SPA_OK;
}

spa_status spa_sched_counts(int32_t n_ops, int32_t n_stages, int32_t n_units, int32_t quantum, int64_t* cut_choices,
                            int64_t* allocations) {
  if (n_ops < 1 || n_stages < 1 || n_units < 1 || quantum < 1) return fail(SPA_EINVAL, "bad argument");
  if (cut_choices) *cut_choices = binom(n_ops - 1, n_stages - 1) + binom(n_ops - 1, n_stages);
  if (allocations) {
    if (n_units % quantum) *allocations = 0;
    else *allocations = binom(n_units / quantum - 1, n_stages - 1);
  }
  return SPA_OK;
}

spa_status spa_refine_allocation(int32_t n_stages, int32_t total, int32_t quantum, int32_t p_min, int32_t* p,
                                 spa_objective_fn objective, void* user, int32_t pass_limit, double* best,
                                 int32_t* n_evals) {
  if (n_stages < 1 || total < 1 || quantum < 1 || !p || !objective) return fail(SPA_EINVAL, "bad argument");
  auto feasible = [&](const std::vector<int32_t>& x) {
    long long s = 0;
    for (int32_t v : x) {
      if (v < p_min || v < quantum || v % quantum) return false;
      s += v;
    }
    return s == total;
  };
  std::vector<int32_t> cur(p, p + n_stages);
  if (!feasible(cur)) return fail(SPA_EINVAL, "initial allocation is infeasible");
  int evals = 0;
  auto F = [&](const std::vector<int32_t>& x) {
    ++evals;
    return objective(x.data(), n_stages, user);
  };
  auto move = [&](const std::vector<int32_t>& x, int d, int r, int z) {
    std::vector<int32_t> y = x;
    y[d] -= z * quantum;
    y[r] += z * quantum;
    return y;
  };
  double t = F(cur);
  for (int pass = 0; pass_limit <= 0 || pass < pass_limit; ++pass) {
    // best legal one-quantum transfer (ties: lowest donor, then receiver)
    bool any = false;
    double t_line = 0.0;
    int bd = -1, br = -1;
    for (int d = 0; d < n_stages; ++d)
      for (int r = 0; r < n_stages; ++r) {
        if (d == r) continue;
        std::vector<int32_t> c = move(cur, d, r, 1);
        if (!feasible(c)) continue;
        double v = F(c);
        if (!any || v < t_line) {
          any = true;
          t_line = v;
          bd = d;
          br = r;
        }
      }
    if (!any || t_line >= t) break;
    // line search along donor -> receiver: grow the step on improvement, halve otherwise
    int z = 1, h = 1;
    while (h > 0) {
      std::vector<int32_t> c = move(cur, bd, br, z + h);
      if (feasible(c)) {
        double v = F(c);
        if (v < t_line) {
          z += h;
          t_line = v;
          h *= 2;
          continue;
        }
      }
      h /= 2;
    }
    cur = move(cur, bd, br, z);
    t = t_line;
  }
  memcpy(p, cur.data(), sizeof(int32_t) * n_stages);
  if (best) *best = t;
  if (n_evals) *n_evals = evals;
  return SPA_OK;
}

}  // extern "C"
