// Per-head top-k and candidate tree tokens.
//
// P1 ("Medusa 심층 아키텍처"), section "소스코드 레벨 구조 분석": every head keeps
// the indices of its k largest logits (generate_candidates); P2 ("[vLLM]
// Medusa"), section "propose()", is the k = 1 case.  P1, section "트리 어텐션
// ... 고정 트리 토폴로지": the fixed topology combines head d's candidates at
// depth d, so node n carries candidate rank(n) of head depth(n), and sits
// depth(n) positions after the cached context.
//
// Order: larger logit first; equal logits by smaller index (-0 and +0 are
// equal).  Comparing (value, index) pairs this way is a total order, so the
// result is unique and bit-exact.
//
// Two kernels spread every logit row over many CUs:
//   1. one wave per (sequence, head, chunk of CW columns): each lane sorts its
//      8 (logit, column) pairs under that order; the chunk's top-kmax is then
//      popped from the 64 lane lists by kmax wave-wide arg-max rounds and
//      written as a sorted (logit, column) list;
//   2. one wave per (sequence, head): with at most 64 chunks each lane's
//      chunk list already is its sorted list (more chunks are merged into
//      per-lane lists by sorted insertion, in column order); k_d arg-max
//      rounds pop the head's candidates, and the same wave writes them, the
//      tree tokens of the nodes at depth head+1, and (head 0) the root and
//      every position.
// The chunk lists live in the caller's workspace.
#include "internal.h"

using namespace medusa;
using namespace medusa::dev;

namespace {

constexpr int CW = 512;  // columns per chunk (8 per lane)

struct CandArgs {
  const float* logits;  // [B][K][V]
  int K, V, kmax, T, nchunks;
  const int32_t* kpd;    // [K]
  const int32_t* depth;  // [T]
  const int32_t* rank;   // [T]
  const int32_t* root;   // [B]
  const int32_t* ctx;    // [B]
  float* cv;             // [B][K][nchunks][kmax] chunk lists
  int32_t* ci;
  int32_t* topk;         // [B][K][kmax]
  int32_t* tree_tokens;  // [B][T]
  int32_t* pos;          // [B][T]
  int rows;              // B * K
};

// the lane holding the popped winner drops it from its list
template <int KM>
__device__ __forceinline__ void list_pop_if(float (&tv)[KM], int (&ti)[KM], float bv, int bi) {
  if (tv[0] == bv && ti[0] == bi) {
#pragma unroll
    for (int q = 0; q + 1 < KM; ++q) {
      tv[q] = tv[q + 1];
      ti[q] = ti[q + 1];
    }
    tv[KM - 1] = -INFINITY;
    ti[KM - 1] = 0x7fffffff;
  }
}

template <int KM>
__device__ __forceinline__ void list_init(float (&tv)[KM], int (&ti)[KM]) {
#pragma unroll
  for (int s = 0; s < KM; ++s) {
    tv[s] = -INFINITY;
    ti[s] = 0x7fffffff;
  }
}

template <int KM>
__global__ __launch_bounds__(256) void cand_chunks(CandArgs a) {
  const int lane = threadIdx.x & 63;
  const int w = blockIdx.x * 4 + (threadIdx.x >> 6);  // = row * nchunks + chunk
  if (w >= a.rows * a.nchunks) return;                // whole wave, no barrier
  const int row = w / a.nchunks, chunk = w % a.nchunks;
  const float* x = a.logits + static_cast<int64_t>(row) * a.V;
  const int c0 = chunk * CW;
  float v[CW / 64];
#pragma unroll
  for (int i = 0; i < CW / 64; ++i) {  // every load in flight before any compare
    const int c = c0 + 64 * i + lane;
    v[i] = c < a.V ? x[c] : -INFINITY;
  }
  // the lane's 8 (logit, column) pairs sorted by a 19-comparator odd-even
  // merge network under the total order (columns past V sort last as
  // padding); the lane list keeps the first min(KM, 8) -- a lane cannot hold
  // more than kmax <= KM of the chunk's top-kmax
  static_assert(CW / 64 == 8, "the sorting network takes 8 values per lane");
  float sv[8];
  int si[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int c = c0 + 64 * i + lane;
    sv[i] = c < a.V ? v[i] : -INFINITY;
    si[i] = c < a.V ? c : 0x7fffffff;
  }
  auto cmpx = [&](int i, int j) __attribute__((always_inline)) {  // (i, j) in order afterwards
    const bool sw = sv[j] > sv[i] || (sv[j] == sv[i] && si[j] < si[i]);
    const float fv = sw ? sv[j] : sv[i], bv = sw ? sv[i] : sv[j];
    const int fi = sw ? si[j] : si[i], bi = sw ? si[i] : si[j];
    sv[i] = fv; sv[j] = bv; si[i] = fi; si[j] = bi;
  };
  cmpx(0, 1); cmpx(2, 3); cmpx(4, 5); cmpx(6, 7);
  cmpx(0, 2); cmpx(1, 3); cmpx(4, 6); cmpx(5, 7);
  cmpx(1, 2); cmpx(5, 6);
  cmpx(0, 4); cmpx(1, 5); cmpx(2, 6); cmpx(3, 7);
  cmpx(2, 4); cmpx(3, 5);
  cmpx(1, 2); cmpx(3, 4); cmpx(5, 6);
  float tv[KM];
  int ti[KM];
  list_init<KM>(tv, ti);
#pragma unroll
  for (int i = 0; i < (KM < 8 ? KM : 8); ++i) {
    tv[i] = sv[i];
    ti[i] = si[i];
  }
  const int64_t base = (static_cast<int64_t>(row) * a.nchunks + chunk) * a.kmax;
  for (int s = 0; s < a.kmax; ++s) {
    float bv = tv[0];
    int bi = ti[0];
    wave_best(bv, bi);
    if (lane == 0) {
      a.cv[base + s] = bv;
      a.ci[base + s] = bi;
    }
    list_pop_if<KM>(tv, ti, bv, bi);
  }
}

template <int KM>
__global__ __launch_bounds__(256) void cand_merge_tree(CandArgs a) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);  // = b * K + d
  if (row >= a.rows) return;                              // whole wave, no barrier
  const int b = row / a.K, d = row % a.K;
  // the first 64 nodes' depth and rank, the context length and the root are
  // loaded now and used after the pops
  const int dn0 = lane < a.T ? a.depth[lane] : -1;
  const int rn0 = lane < a.T ? a.rank[lane] : 0;
  const int ctx_b = a.ctx[b];
  const int root_b = a.root[b];
  const int kd = a.kpd[d];
  float tv[KM];
  int ti[KM];
  list_init<KM>(tv, ti);
  const float* cv = a.cv + static_cast<int64_t>(row) * a.nchunks * a.kmax;
  const int32_t* ci = a.ci + static_cast<int64_t>(row) * a.nchunks * a.kmax;
  if (a.nchunks <= 64) {
    // one chunk list per lane, already sorted: it is the lane's list
    if (lane < a.nchunks) {
#pragma unroll
      for (int s = 0; s < KM; ++s) {
        if (s < a.kmax) {
          tv[s] = cv[lane * a.kmax + s];
          ti[s] = ci[lane * a.kmax + s];
        }
      }
    }
  } else {
    for (int l = lane; l < a.nchunks; l += 64) {
      float xv[KM];
      int xi[KM];
#pragma unroll
      for (int s = 0; s < KM; ++s) {  // the whole chunk list in flight at once
        xv[s] = s < a.kmax ? cv[l * a.kmax + s] : -INFINITY;
        xi[s] = s < a.kmax ? ci[l * a.kmax + s] : 0x7fffffff;
      }
      // a sorted list: once an entry stays out, every later one does too
#pragma unroll
      for (int s = 0; s < KM; ++s)
        if (xv[s] > tv[KM - 1]) list_insert<KM>(tv, ti, xv[s], xi[s]);
    }
  }
  // k_d arg-max rounds; lane s keeps the head's candidate of rank s
  int mine = -1;
  for (int s = 0; s < kd; ++s) {
    float bv = tv[0];
    int bi = ti[0];
    wave_best(bv, bi);
    mine = lane == s ? bi : mine;
    list_pop_if<KM>(tv, ti, bv, bi);
  }
  if (lane < a.kmax) a.topk[static_cast<int64_t>(row) * a.kmax + lane] = mine;  // -1 past k_d
  // nodes at depth d+1 carry the candidate of their rank
  int32_t* tok = a.tree_tokens + static_cast<int64_t>(b) * a.T;
  for (int n0 = 0; n0 < a.T; n0 += 64) {
    const int n = n0 + lane;
    const int dn = n0 == 0 ? dn0 : (n < a.T ? a.depth[n] : -1);
    const int rn = n0 == 0 ? rn0 : (n < a.T ? a.rank[n] : 0);
    const int t = __shfl(mine, dn == d + 1 ? rn : 0);
    if (dn == d + 1) tok[n] = t;
  }
  if (d == 0) {
    for (int n = lane; n < a.T; n += 64) {
      a.pos[static_cast<int64_t>(b) * a.T + n] = ctx_b + (n < 64 ? dn0 : a.depth[n]);
      if (n == 0) tok[0] = root_b;
    }
  }
}

int km_for(int kmax) { return kmax <= 4 ? 4 : kmax <= 8 ? 8 : kmax <= 12 ? 12 : kmax <= 16 ? 16 : 32; }

size_t cand_ws_bytes(int B, int V, const medusa_tree_t* tree, int* nchunks) {
  const int nc = (V + CW - 1) / CW;
  if (nchunks) *nchunks = nc;
  const size_t one = round_up(static_cast<size_t>(B) * tree->K * nc * tree->kmax * 4, 256);
  return 2 * one;
}

template <int KM>
int launch_cand(const CandArgs& a, hipStream_t s) {
  const int64_t chunks = static_cast<int64_t>(a.rows) * a.nchunks;
  hipLaunchKernelGGL(cand_chunks<KM>, dim3(static_cast<unsigned>((chunks + 3) / 4)), dim3(256), 0, s, a);
  int rc = check_launch("top-k chunks");
  if (rc) return rc;
  hipLaunchKernelGGL(cand_merge_tree<KM>, dim3(static_cast<unsigned>((a.rows + 3) / 4)), dim3(256), 0, s, a);
  return check_launch("top-k merge / tree tokens");
}

}  // namespace

extern "C" size_t medusa_tree_candidates_workspace_size(int B, int V, const medusa_tree_t* tree) {
  if (!tree || B < 1 || V < 1) return 0;
  return cand_ws_bytes(B, V, tree, nullptr);
}

extern "C" int medusa_tree_candidates(const float* head_logits, const int32_t* root,
                                      const int32_t* ctx_len, const medusa_tree_t* tree, int B,
                                      int V, int32_t* topk_idx, int32_t* tree_tokens, int32_t* pos,
                                      void* ws, size_t ws_bytes, hipStream_t stream) {
  clear_error();
  int rc = check_tree(tree);
  if (rc) return rc;
  MEDUSA_CHECK_ARG(head_logits && root && ctx_len && topk_idx && tree_tokens && pos,
                   "all tensor arguments must be non-NULL");
  MEDUSA_CHECK_ARG(B >= 1 && V >= 1, "B=%d and V=%d must be >= 1", B, V);
  for (int d = 0; d < tree->K; ++d)
    MEDUSA_CHECK_ARG(tree->kpd[d] <= V, "head %d keeps %d candidates but V=%d", d + 1,
                     tree->kpd[d], V);
  MEDUSA_CHECK_ARG(static_cast<int64_t>(B) * tree->K * V < (1ll << 31), "B*K*V too large");
  CandArgs a{};
  const size_t need = cand_ws_bytes(B, V, tree, &a.nchunks);
  if (!ws || ws_bytes < need || !aligned256(ws)) {
    set_error("candidates workspace: need %zu bytes, 256-byte aligned (got %zu at %p)", need, ws_bytes, ws);
    return MEDUSA_EWORKSPACE;
  }
  a.logits = head_logits;
  a.K = tree->K;
  a.V = V;
  a.kmax = tree->kmax;
  a.T = tree->T;
  a.kpd = tree->d_kpd;
  a.depth = tree->d_depth;
  a.rank = tree->d_rank;
  a.root = root;
  a.ctx = ctx_len;
  a.cv = static_cast<float*>(ws);
  a.ci = reinterpret_cast<int32_t*>(static_cast<char*>(ws) + need / 2);
  a.topk = topk_idx;
  a.tree_tokens = tree_tokens;
  a.pos = pos;
  a.rows = B * tree->K;
  switch (km_for(tree->kmax)) {
    case 4: return launch_cand<4>(a, stream);
    case 8: return launch_cand<8>(a, stream);
    case 12: return launch_cand<12>(a, stream);
    case 16: return launch_cand<16>(a, stream);
    default: return launch_cand<32>(a, stream);
  }
}
