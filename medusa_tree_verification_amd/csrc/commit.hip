// Commit of an accepted path: KV rollback/compaction and the next step's
// root and context length.
//
// P3 ("Speculative Decoding(투기적 디코딩) 원리와 가속 아키텍처"), the pipeline of
// its architecture section ends with rollback and the confirmed correction
// token, and its section 5 (Case 2) checks K-token verification with early
// rejection and rollback; P4 ("추측 디코딩과 긴 컨텍스트"), section 1.3: the
// matched drafts are kept and everything after the first mismatch is
// discarded.  With the tree tokens' K/V in cache slots ctx .. ctx+T-1 (slot
// ctx + n for tree node n, the root at ctx), keeping the accepted path means
// moving the K/V of its node at depth d from slot ctx + node to slot ctx + d,
// d = 1 .. accept_len; the other tree slots are dropped simply by the new
// context length ctx + accept_len + 1 (the correction / bonus token becomes
// the next root, whose K/V the next step computes at the new ctx).
//
// One workgroup per (layer, sequence, K/V head): the accepted rows (at most
// K of them) are read into registers first and written afterwards, because
// a row's source slot can be another row's destination.
#include "internal.h"

using namespace medusa;

namespace {

constexpr int CT = 64;  // one wave per (layer, sequence, head): a 256-thread shape measured 6x slower

struct CommitArgs {
  char* k;
  char* v;
  int64_t layer_bytes;  // bytes between layers of one cache
  int L, B, Hkv, S_cap, T, K;
  int row_bytes;        // D * element size (multiple of 16)
  const int32_t* acc_len;
  const int32_t* nodes;   // [B][K+1]
  const int32_t* tokens;  // [B][K+1]
  const int32_t* ctx;     // [B]
  int32_t* ctx_next;      // [B]
  int32_t* root_next;     // [B]
};

__global__ __launch_bounds__(CT) void commit_kernel(CommitArgs a) {
  const int id = blockIdx.x;
  const int kvh = id % a.Hkv;
  const int b = (id / a.Hkv) % a.B;
  const int layer = id / (a.Hkv * a.B);
  int ctx = a.ctx[b];
  ctx = ctx < 0 ? 0 : (ctx > a.S_cap - a.T ? a.S_cap - a.T : ctx);
  int len = a.acc_len[b];
  len = len < 0 ? 0 : (len > a.K ? a.K : len);
  const int32_t* nodes = a.nodes + static_cast<int64_t>(b) * (a.K + 1);
  if (layer == 0 && kvh == 0 && threadIdx.x == 0) {
    a.ctx_next[b] = ctx + len + 1;
    a.root_next[b] = a.tokens[static_cast<int64_t>(b) * (a.K + 1) + len];
  }
  // rows d = 1 .. len, chunks of 16 bytes: thread t takes (d, chunk) pairs
  const int chunks = a.row_bytes / 16;
  const int64_t head_off =
      static_cast<int64_t>(layer) * a.layer_bytes + (static_cast<int64_t>(b) * a.Hkv + kvh) * a.S_cap * a.row_bytes;
  constexpr int MAX_CHUNKS = 512 / 16;  // a row is at most 512 bytes
  constexpr int PER = (2 * MEDUSA_MAX_HEADS * MAX_CHUNKS + CT - 1) / CT;  // (K/V, row, chunk) per thread
  uint4 buf[PER];
  const int work = 2 * len * chunks;
#pragma unroll
  for (int u = 0; u < PER; ++u) {
    const int w = threadIdx.x + u * CT;
    if (w < work) {
      const int kv = w / (len * chunks), rest = w % (len * chunks);
      const int d = 1 + rest / chunks, c = rest % chunks;
      int node = nodes[d];
      node = node < 0 ? 0 : (node >= a.T ? a.T - 1 : node);
      const char* src = (kv ? a.v : a.k) + head_off + static_cast<int64_t>(ctx + node) * a.row_bytes + c * 16;
      buf[u] = *reinterpret_cast<const uint4*>(src);
    }
  }
  __syncthreads();
#pragma unroll
  for (int u = 0; u < PER; ++u) {
    const int w = threadIdx.x + u * CT;
    if (w < work) {
      const int kv = w / (len * chunks), rest = w % (len * chunks);
      const int d = 1 + rest / chunks, c = rest % chunks;
      char* dst = (kv ? a.v : a.k) + head_off + static_cast<int64_t>(ctx + d) * a.row_bytes + c * 16;
      *reinterpret_cast<uint4*>(dst) = buf[u];
    }
  }
}

}  // namespace

extern "C" int medusa_commit_accepted(void* k_cache, void* v_cache, int64_t layer_stride, int L,
                                      const int32_t* accept_len, const int32_t* out_nodes,
                                      const int32_t* out_tokens, const int32_t* ctx_len,
                                      int32_t* ctx_next, int32_t* root_next,
                                      const medusa_tree_t* tree, int B, int Hkv, int D, int S_cap,
                                      medusa_dtype_t dt, hipStream_t stream) {
  clear_error();
  int rc = check_tree(tree);
  if (rc) return rc;
  MEDUSA_CHECK_ARG(k_cache && v_cache && accept_len && out_nodes && out_tokens && ctx_len && ctx_next &&
                       root_next,
                   "all pointer arguments must be non-NULL");
  MEDUSA_CHECK_ARG(dt == MEDUSA_F32 || dt == MEDUSA_BF16, "unknown dtype %d", static_cast<int>(dt));
  const int esize = dt == MEDUSA_F32 ? 4 : 2;
  MEDUSA_CHECK_ARG(L >= 1 && B >= 1 && Hkv >= 1, "L=%d, B=%d, Hkv=%d must be >= 1", L, B, Hkv);
  MEDUSA_CHECK_ARG(D >= 1 && (D * esize) % 16 == 0 && D * esize <= 512,
                   "D=%d: a cache row must be a multiple of 16 bytes and at most 512", D);
  MEDUSA_CHECK_ARG(S_cap >= tree->T, "S_cap=%d smaller than the tree (T=%d)", S_cap, tree->T);
  const int64_t head_elems = static_cast<int64_t>(B) * Hkv * S_cap * D;
  MEDUSA_CHECK_ARG(L == 1 || layer_stride >= head_elems,
                   "layer_stride=%lld smaller than one layer's cache (%lld elements)",
                   static_cast<long long>(layer_stride), static_cast<long long>(head_elems));
  MEDUSA_CHECK_ARG(aligned16(k_cache) && aligned16(v_cache) && (layer_stride * esize) % 16 == 0,
                   "caches must be 16-byte aligned (layer stride included)");
  MEDUSA_CHECK_ARG(static_cast<int64_t>(L) * B * Hkv < (1ll << 31), "too many (layer, sequence, head) rows");
  CommitArgs a{};
  a.k = static_cast<char*>(k_cache);
  a.v = static_cast<char*>(v_cache);
  a.layer_bytes = layer_stride * esize;
  a.L = L;
  a.B = B;
  a.Hkv = Hkv;
  a.S_cap = S_cap;
  a.T = tree->T;
  a.K = tree->K;
  a.row_bytes = D * esize;
  a.acc_len = accept_len;
  a.nodes = out_nodes;
  a.tokens = out_tokens;
  a.ctx = ctx_len;
  a.ctx_next = ctx_next;
  a.root_next = root_next;
  hipLaunchKernelGGL(commit_kernel, dim3(static_cast<unsigned>(L * B * Hkv)), dim3(CT), 0, stream, a);
  return check_launch("commit of the accepted path");
}
