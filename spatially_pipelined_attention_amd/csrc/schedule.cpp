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

// Section 4.2's allocation refinement: a local search over CU allocations in
// which each pass picks the best one-quantum transfer between an ordered
// (donor, receiver) pair of stages, and, if it improves on the current
// allocation, follows that direction with a doubling/halving step to the best
// transfer size. It ends when no legal pairwise move improves, or after the
// pass limit.
namespace {

struct Probe {
  int donor = -1, receiver = -1;
  double value = 0.0;
};

struct AllocSearch {
  int n, total, quantum, p_min;
  spa_objective_fn fn;
  void* user;
  int evals = 0;
  double last_line_value = 0.0;

  bool legal(const std::vector<int32_t>& x) const {
    long long sum = 0;
    for (int32_t v : x) {
      if (v < p_min || v < quantum || v % quantum) return false;
      sum += v;
    }
    return sum == total;
  }
  double cost(const std::vector<int32_t>& x) {
    ++evals;
    return fn(x.data(), n, user);
  }
  std::vector<int32_t> shifted(const std::vector<int32_t>& x, int d, int r, int quanta) const {
    std::vector<int32_t> y = x;
    y[d] -= quanta * quantum;
    y[r] += quanta * quantum;
    return y;
  }
  // the best legal one-quantum transfer (ties to the lowest donor, then receiver)
  Probe best_probe(const std::vector<int32_t>& x) {
    Probe b;
    for (int d = 0; d < n; ++d)
      for (int r = 0; r < n; ++r) {
        if (d == r) continue;
        const std::vector<int32_t> c = shifted(x, d, r, 1);
        if (!legal(c)) continue;
        const double v = cost(c);
        if (b.donor < 0 || v < b.value) b = Probe{d, r, v};
      }
    return b;
  }
  // transfer size along the probe's direction: a trial at z + step that
  // improves is taken and the step doubles; otherwise the step halves
  int gallop(const std::vector<int32_t>& x, const Probe& pr) {
    int z = 1;
    double v_best = pr.value;
    for (int step = 1; step > 0;) {
      const std::vector<int32_t> c = shifted(x, pr.donor, pr.receiver, z + step);
      double v = 0.0;
      const bool better = legal(c) && (v = cost(c)) < v_best;
      if (better) {
        z += step;
        v_best = v;
        step *= 2;
      } else {
        step /= 2;
      }
    }
    last_line_value = v_best;
    return z;
  }
};

}  // namespace

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
  AllocSearch S{n_stages, total, quantum, p_min, objective, user};
  std::vector<int32_t> cur(p, p + n_stages);
  if (!S.legal(cur)) return fail(SPA_EINVAL, "initial allocation is infeasible");
  double value = S.cost(cur);
  for (int pass = 0; pass_limit <= 0 || pass < pass_limit; ++pass) {
    const Probe pr = S.best_probe(cur);
    if (pr.donor < 0 || !(pr.value < value)) break;   // converged: no improving pairwise move
    const int z = S.gallop(cur, pr);
    cur = S.shifted(cur, pr.donor, pr.receiver, z);
    value = S.last_line_value;
  }
  memcpy(p, cur.data(), sizeof(int32_t) * n_stages);
  if (best) *best = value;
  if (n_evals) *n_evals = S.evals;
  return SPA_OK;
}

}  // extern "C"
