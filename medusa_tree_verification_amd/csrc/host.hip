// Host side of the library: error text, version, and the static tree
// (validation, ancestor bitmask, child lists, upload).
//
// The tree follows P1 ("Medusa 심층 아키텍처"), section "트리 어텐션 ... 고정 트리
// 토폴로지와 2차원 어텐션 마스크": token i may see tree token j iff j is an
// ancestor of i or i itself.  As in P1's sketch code, each node's row is its
// parent's row plus its own bit; that needs parents numbered before children,
// which the validation enforces.
#include <algorithm>
#include <cstring>
#include <string>

#include "internal.h"

namespace medusa {

static thread_local std::string g_error;

void set_error(const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_error = buf;
}

void clear_error() { g_error.clear(); }

int check_launch(const char* what) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) {
    set_error("launch of %s failed: %s", what, hipGetErrorString(e));
    return MEDUSA_EHIP;
  }
  return MEDUSA_OK;
}

int current_device() {
  int d = -1;
  hipError_t e = hipGetDevice(&d);
  if (e != hipSuccess) {
    set_error("hipGetDevice failed: %s", hipGetErrorString(e));
    return -1;
  }
  return d;
}

int check_tree(const medusa_tree_t* tree) {
  if (!tree) {
    set_error("tree is NULL");
    return MEDUSA_EINVAL;
  }
  int d = current_device();
  if (d < 0) return MEDUSA_EHIP;
  if (d != tree->device) {
    set_error("tree was created on device %d but device %d is current", tree->device, d);
    return MEDUSA_EINVAL;
  }
  return MEDUSA_OK;
}

// Validation and host-side construction shared by build_host and create.
static int build_tree(const int32_t* parent, const int32_t* rank, int T, const int32_t* kpd,
                      int K, medusa_tree& t) {
  MEDUSA_CHECK_ARG(parent && rank && kpd, "parent, rank and k_per_depth must be non-NULL");
  MEDUSA_CHECK_ARG(T >= 1 && T <= MEDUSA_MAX_TREE_NODES, "T=%d outside 1..%d", T,
                   MEDUSA_MAX_TREE_NODES);
  MEDUSA_CHECK_ARG(K >= 1 && K <= MEDUSA_MAX_HEADS, "K=%d outside 1..%d", K, MEDUSA_MAX_HEADS);
  for (int d = 0; d < K; ++d)
    MEDUSA_CHECK_ARG(kpd[d] >= 1 && kpd[d] <= MEDUSA_MAX_TOPK,
                     "k_per_depth[%d]=%d outside 1..%d", d, kpd[d], MEDUSA_MAX_TOPK);
  MEDUSA_CHECK_ARG(parent[0] == -1, "node 0 must be the root (parent[0]=%d, expected -1)",
                   parent[0]);
  t.T = T;
  t.K = K;
  t.W = (T + 63) / 64;
  t.parent.assign(parent, parent + T);
  t.rank.assign(rank, rank + T);
  t.rank[0] = 0;
  t.kpd.assign(kpd, kpd + K);
  t.depth.assign(T, 0);
  t.kmax = *std::max_element(kpd, kpd + K);
  t.max_depth = 0;
  std::vector<uint64_t> used(T, 0);  // rank slots taken among each node's children (k <= 32)
  for (int n = 1; n < T; ++n) {
    int p = parent[n];
    MEDUSA_CHECK_ARG(p >= 0 && p < n, "parent[%d]=%d is not an earlier node", n, p);
    int d = t.depth[p] + 1;
    MEDUSA_CHECK_ARG(d <= K, "node %d has depth %d > K=%d", n, d, K);
    MEDUSA_CHECK_ARG(rank[n] >= 0 && rank[n] < kpd[d - 1],
                     "rank[%d]=%d outside head %d's top-%d", n, rank[n], d, kpd[d - 1]);
    uint64_t bit = 1ull << rank[n];
    MEDUSA_CHECK_ARG(!(used[p] & bit), "two children of node %d share rank %d", p, rank[n]);
    used[p] |= bit;
    t.depth[n] = d;
    t.max_depth = std::max(t.max_depth, d);
  }
  // ancestor bitmask: own bit plus the parent's row
  t.mask.assign(static_cast<size_t>(T) * t.W, 0);
  for (int n = 0; n < T; ++n) {
    uint64_t* row = &t.mask[static_cast<size_t>(n) * t.W];
    if (n > 0) {
      const uint64_t* prow = &t.mask[static_cast<size_t>(parent[n]) * t.W];
      for (int w = 0; w < t.W; ++w) row[w] = prow[w];
    }
    row[n / 64] |= 1ull << (n % 64);
  }
  // children in rank order (CSR)
  std::vector<std::vector<int32_t>> kids(T);
  for (int n = 1; n < T; ++n) kids[parent[n]].push_back(n);
  t.child_start.assign(T + 1, 0);
  t.child_list.clear();
  for (int u = 0; u < T; ++u) {
    std::sort(kids[u].begin(), kids[u].end(),
              [&](int a, int b) { return rank[a] < rank[b]; });
    t.child_start[u] = static_cast<int32_t>(t.child_list.size());
    t.child_list.insert(t.child_list.end(), kids[u].begin(), kids[u].end());
  }
  t.child_start[T] = static_cast<int32_t>(t.child_list.size());
  return MEDUSA_OK;
}

}  // namespace medusa

using namespace medusa;

extern "C" {

const char* medusa_last_error(void) { return g_error.c_str(); }

const char* medusa_version(void) { return "medusa-amd 0.1 gfx950"; }

int medusa_tree_build_host(const int32_t* parent, const int32_t* rank, int T,
                           const int32_t* k_per_depth, int K, uint64_t* mask_out,
                           int32_t* depth_out) {
  clear_error();
  medusa_tree t;
  int rc = build_tree(parent, rank, T, k_per_depth, K, t);
  if (rc != MEDUSA_OK) return rc;
  if (mask_out) std::memcpy(mask_out, t.mask.data(), t.mask.size() * sizeof(uint64_t));
  if (depth_out) std::memcpy(depth_out, t.depth.data(), t.depth.size() * sizeof(int32_t));
  return MEDUSA_OK;
}

int medusa_tree_create(const int32_t* parent, const int32_t* rank, int T,
                       const int32_t* k_per_depth, int K, medusa_tree_t** out) {
  clear_error();
  MEDUSA_CHECK_ARG(out != nullptr, "out is NULL");
  *out = nullptr;
  medusa_tree* t = new medusa_tree();
  int rc = build_tree(parent, rank, T, k_per_depth, K, *t);
  if (rc != MEDUSA_OK) {
    delete t;
    return rc;
  }
  t->device = current_device();
  if (t->device < 0) {
    delete t;
    return MEDUSA_EHIP;
  }
  // blob layout: mask (8-byte words) first, then the int32 arrays
  const size_t n_mask = t->mask.size();
  const size_t n_i32 = static_cast<size_t>(T) * 3 + (T + 1) + t->child_list.size() + K;
  const size_t bytes = n_mask * 8 + n_i32 * 4 + 16;
  std::vector<uint8_t> host(bytes, 0);
  size_t off = 0;
  auto put = [&](const void* src, size_t nbytes) {
    size_t at = off;
    if (nbytes) std::memcpy(host.data() + off, src, nbytes);
    off += nbytes;
    return at;
  };
  size_t o_mask = put(t->mask.data(), n_mask * 8);
  size_t o_parent = put(t->parent.data(), T * 4);
  size_t o_rank = put(t->rank.data(), T * 4);
  size_t o_depth = put(t->depth.data(), T * 4);
  size_t o_cs = put(t->child_start.data(), (T + 1) * 4);
  size_t o_cl = put(t->child_list.data(), t->child_list.size() * 4);
  size_t o_kpd = put(t->kpd.data(), K * 4);
  hipError_t e = hipMalloc(&t->blob, bytes);
  if (e == hipSuccess) e = hipMemcpy(t->blob, host.data(), bytes, hipMemcpyHostToDevice);
  if (e != hipSuccess) {
    set_error("tree upload failed: %s", hipGetErrorString(e));
    if (t->blob) (void)hipFree(t->blob);
    delete t;
    return MEDUSA_EHIP;
  }
  uint8_t* b = static_cast<uint8_t*>(t->blob);
  t->d_mask = reinterpret_cast<const uint64_t*>(b + o_mask);
  t->d_parent = reinterpret_cast<const int32_t*>(b + o_parent);
  t->d_rank = reinterpret_cast<const int32_t*>(b + o_rank);
  t->d_depth = reinterpret_cast<const int32_t*>(b + o_depth);
  t->d_child_start = reinterpret_cast<const int32_t*>(b + o_cs);
  t->d_child_list = reinterpret_cast<const int32_t*>(b + o_cl);
  t->d_kpd = reinterpret_cast<const int32_t*>(b + o_kpd);
  *out = t;
  return MEDUSA_OK;
}

void medusa_tree_destroy(medusa_tree_t* tree) {
  if (!tree) return;
  if (tree->blob) (void)hipFree(tree->blob);
  delete tree;
}

int medusa_tree_mask(const medusa_tree_t* tree, uint64_t* host_out) {
  clear_error();
  MEDUSA_CHECK_ARG(tree && host_out, "tree and host_out must be non-NULL");
  std::memcpy(host_out, tree->mask.data(), tree->mask.size() * sizeof(uint64_t));
  return MEDUSA_OK;
}

int medusa_tree_info(const medusa_tree_t* tree, int32_t* T, int32_t* K, int32_t* W,
                     int32_t* max_depth, int32_t* kmax) {
  clear_error();
  MEDUSA_CHECK_ARG(tree != nullptr, "tree is NULL");
  if (T) *T = tree->T;
  if (K) *K = tree->K;
  if (W) *W = tree->W;
  if (max_depth) *max_depth = tree->max_depth;
  if (kmax) *kmax = tree->kmax;
  return MEDUSA_OK;
}

}  // extern "C"
