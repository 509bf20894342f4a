// Static tree optimiser (host code).
//
// P2 ("[vLLM] Medusa"), the paper-results section: on top of tree attention
// (~1.9x) an optimised tree configuration brings ~2.2x; P1 ("Medusa 심층
// 아키텍처"), section on the tree-size trade-off: the topology (usually 32-64
// nodes) is to be chosen by profiling for the model and the GPU.
//
// Model: the candidate of rank r from head d is the target's next token with
// probability p[d][r], independently of the ranks above it on the path (a
// per-depth, per-rank acceptance table, e.g. measured by profiling).  A node
// n = (r_1, .., r_d) is then accepted with probability P(n) = prod_i p[i][r_i]
// and, by linearity, a tree accepts sum_{n != root} P(n) nodes per step on
// average.  P(child) <= P(parent), so the best set of T - 1 non-root nodes
// is simply the T - 1 most probable tuples (prefix-closed by construction);
// a best-first search over the tuples yields them in order.  Ties: smaller
// depth first, then the lexicographically smaller tuple (the same rule the
// cost-ordered topology uses, which this reproduces for p[d][r] =
// 2^-(r+1)).  Nodes are numbered breadth-first by (depth, tuple).
#include <algorithm>
#include <cmath>
#include <queue>
#include <vector>

#include "internal.h"

using namespace medusa;

namespace {

struct Cand {
  double p;
  std::vector<int> t;  // rank tuple
};

// a ranks ahead of b in the selection order
bool ahead(const Cand& a, const Cand& b) {
  if (a.p != b.p) return a.p > b.p;
  if (a.t.size() != b.t.size()) return a.t.size() < b.t.size();
  return a.t < b.t;
}

struct Behind {
  bool operator()(const Cand& a, const Cand& b) const { return ahead(b, a); }
};

}  // namespace

extern "C" int medusa_tree_optimize(const double* p_accept, int K, int kmax_in,
                                    const int32_t* k_per_depth, int T, int32_t* parent_out,
                                    int32_t* rank_out, double* expected_out) {
  clear_error();
  MEDUSA_CHECK_ARG(p_accept && k_per_depth && parent_out && rank_out, "pointer arguments must be non-NULL");
  MEDUSA_CHECK_ARG(K >= 1 && K <= MEDUSA_MAX_HEADS, "K=%d outside 1..%d", K, MEDUSA_MAX_HEADS);
  MEDUSA_CHECK_ARG(T >= 1 && T <= MEDUSA_MAX_TREE_NODES, "T=%d outside 1..%d", T, MEDUSA_MAX_TREE_NODES);
  long long total = 0, level = 1;
  for (int d = 0; d < K; ++d) {
    MEDUSA_CHECK_ARG(k_per_depth[d] >= 1 && k_per_depth[d] <= MEDUSA_MAX_TOPK && k_per_depth[d] <= kmax_in,
                     "k_per_depth[%d]=%d outside 1..min(%d, kmax_in=%d)", d, k_per_depth[d], MEDUSA_MAX_TOPK,
                     kmax_in);
    for (int r = 0; r < k_per_depth[d]; ++r) {
      const double p = p_accept[static_cast<int64_t>(d) * kmax_in + r];
      MEDUSA_CHECK_ARG(p >= 0.0 && p <= 1.0, "p_accept[%d][%d]=%g outside [0, 1]", d, r, p);
    }
    level = std::min(level * k_per_depth[d], 1ll << 40);
    total = std::min(total + level, 1ll << 40);
  }
  MEDUSA_CHECK_ARG(T - 1 <= total, "T=%d exceeds the %lld nodes of the full tree", T, total + 1);

  std::priority_queue<Cand, std::vector<Cand>, Behind> frontier;
  for (int r = 0; r < k_per_depth[0]; ++r) frontier.push({p_accept[r], {r}});
  std::vector<Cand> kept;
  double expected = 0.0;
  while (static_cast<int>(kept.size()) < T - 1) {
    Cand c = frontier.top();
    frontier.pop();
    const int d = static_cast<int>(c.t.size());
    if (d < K)
      for (int r = 0; r < k_per_depth[d]; ++r) {
        Cand ch{c.p * p_accept[static_cast<int64_t>(d) * kmax_in + r], c.t};
        ch.t.push_back(r);
        frontier.push(std::move(ch));
      }
    kept.push_back(std::move(c));
  }
  for (const Cand& c : kept) expected += c.p;
  // breadth-first numbering by (depth, tuple)
  std::sort(kept.begin(), kept.end(), [](const Cand& a, const Cand& b) {
    if (a.t.size() != b.t.size()) return a.t.size() < b.t.size();
    return a.t < b.t;
  });
  parent_out[0] = -1;
  rank_out[0] = 0;
  for (size_t n = 0; n < kept.size(); ++n) {
    const std::vector<int>& t = kept[n].t;
    int par = 0;
    if (t.size() > 1) {
      const std::vector<int> pre(t.begin(), t.end() - 1);
      // the parent was kept (prefix-closed) and sits earlier in the order
      const auto it = std::lower_bound(kept.begin(), kept.begin() + n, pre, [](const Cand& a, const std::vector<int>& v) {
        if (a.t.size() != v.size()) return a.t.size() < v.size();
        return a.t < v;
      });
      par = static_cast<int>(it - kept.begin()) + 1;
    }
    parent_out[n + 1] = par;
    rank_out[n + 1] = t.back();
  }
  if (expected_out) *expected_out = expected;
  return MEDUSA_OK;
}
