// Per-head top-k and candidate tree tokens.
//
// P1 ("Medusa 심층 아키텍처"), section "소스코드 레벨 구조 분석": every head keeps
// the indices of its k largest logits (generate_candidates); P2 ("[vLLM]
// Medusa"), section "propose()", is the k = 1 case.  P1, section "트리 어텐션
// ... 고정 트리 토폴로지": the fixed topology combines head d's candidates at
// depth d, so node n carries candidate rank(n) of head depth(n), and sits
// depth(n) positions after the cached context.
//
// Order: larger logit first; equal logits by smaller index (a total order,
// so the result is unique and bit-exact).
//
// One workgroup per (head, sequence).  Every thread scans a strided share of
// the vocabulary and keeps its own sorted top-KM list in registers (an
// element enters only if it beats the current last entry, so the common case
// is one compare).  The lists are then merged k_d times: each round a
// block-wide arg-max over the list heads picks the next winner, whose owner
// pops it.  The same workgroup writes the tree tokens of the nodes at depth
// head+1 (and the root, for head 0).
#include "internal.h"

using namespace medusa;

namespace {

// (v, i) beats (w, j) in the output order
__device__ __forceinline__ bool beats(float v, int i, float w, int j) {
  return v > w || (v == w && static_cast<unsigned>(i) < static_cast<unsigned>(j));
}

struct CandArgs {
  const float* logits;  // [B][K][V]
  int K, V, kmax, T;
  const int32_t* kpd;    // [K]
  const int32_t* depth;  // [T]
  const int32_t* rank;   // [T]
  const int32_t* root;   // [B]
  const int32_t* ctx;    // [B]
  int32_t* topk;         // [B][K][kmax]
  int32_t* tree_tokens;  // [B][T]
  int32_t* pos;          // [B][T]
};

constexpr int THREADS = 256;

template <int KM>
__global__ __launch_bounds__(THREADS) void topk_tree_kernel(CandArgs a) {
  const int head = blockIdx.x;
  const int b = blockIdx.y;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const float* x = a.logits + (static_cast<int64_t>(b) * a.K + head) * a.V;
  const int kd = a.kpd[head];

  float lv[KM];
  int li[KM];
#pragma unroll
  for (int j = 0; j < KM; ++j) {
    lv[j] = -INFINITY;
    li[j] = -1;
  }
  auto insert = [&](float v, int i) {
    if (!beats(v, i, lv[KM - 1], li[KM - 1])) return;
    float cv = v;
    int ci = i;
#pragma unroll
    for (int j = 0; j < KM; ++j) {
      bool bt = beats(cv, ci, lv[j], li[j]);
      float tv = lv[j];
      int ti = li[j];
      lv[j] = bt ? cv : tv;
      li[j] = bt ? ci : ti;
      cv = bt ? tv : cv;
      ci = bt ? ti : ci;
    }
  };
  // strided scan, 8 loads in flight per thread
  int v0 = tid;
  for (; v0 + 7 * THREADS < a.V; v0 += 8 * THREADS) {
    float buf[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) buf[u] = x[v0 + u * THREADS];
#pragma unroll
    for (int u = 0; u < 8; ++u) insert(buf[u], v0 + u * THREADS);
  }
  for (; v0 < a.V; v0 += THREADS) insert(x[v0], v0);

  __shared__ float s_wv[4];
  __shared__ int s_wi[4];
  __shared__ int s_top[MEDUSA_MAX_TOPK];
  for (int round = 0; round < kd; ++round) {
    float bv = lv[0];
    int bi = li[0];
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      float ov = __shfl_xor(bv, off, 64);
      int oi = __shfl_xor(bi, off, 64);
      if (beats(ov, oi, bv, bi)) {
        bv = ov;
        bi = oi;
      }
    }
    if (lane == 0) {
      s_wv[wave] = bv;
      s_wi[wave] = bi;
    }
    __syncthreads();
    float wv = s_wv[0];
    int wi = s_wi[0];
#pragma unroll
    for (int w = 1; w < THREADS / 64; ++w)
      if (beats(s_wv[w], s_wi[w], wv, wi)) {
        wv = s_wv[w];
        wi = s_wi[w];
      }
    if (tid == 0) s_top[round] = wi;
    // the owner of the winner pops its list head (indices are unique)
    if (wi >= 0 && li[0] == wi) {
#pragma unroll
      for (int j = 0; j < KM - 1; ++j) {
        lv[j] = lv[j + 1];
        li[j] = li[j + 1];
      }
      lv[KM - 1] = -INFINITY;
      li[KM - 1] = -1;
    }
    __syncthreads();  // s_wv/s_wi reused next round; s_top complete after the loop
  }
  int32_t* out = a.topk + (static_cast<int64_t>(b) * a.K + head) * a.kmax;
  for (int j = tid; j < a.kmax; j += THREADS) out[j] = j < kd ? s_top[j] : -1;

  // tree tokens of the nodes this head feeds
  const int c = a.ctx[b];
  for (int n = tid; n < a.T; n += THREADS) {
    const int d = a.depth[n];
    if (n == 0) {
      if (head == 0) {
        a.tree_tokens[static_cast<int64_t>(b) * a.T] = a.root[b];
        a.pos[static_cast<int64_t>(b) * a.T] = c;
      }
    } else if (d == head + 1) {
      a.tree_tokens[static_cast<int64_t>(b) * a.T + n] = s_top[a.rank[n]];
      a.pos[static_cast<int64_t>(b) * a.T + n] = c + d;
    }
  }
}

}  // namespace

extern "C" int medusa_tree_candidates(const float* head_logits, const int32_t* root,
                                      const int32_t* ctx_len, const medusa_tree_t* tree, int B,
                                      int V, int32_t* topk_idx, int32_t* tree_tokens, int32_t* pos,
                                      hipStream_t stream) {
  clear_error();
  int rc = check_tree(tree);
  if (rc) return rc;
  MEDUSA_CHECK_ARG(head_logits && root && ctx_len && topk_idx && tree_tokens && pos,
                   "all tensor arguments must be non-NULL");
  MEDUSA_CHECK_ARG(B >= 1 && V >= 1, "B=%d and V=%d must be >= 1", B, V);
  for (int d = 0; d < tree->K; ++d)
    MEDUSA_CHECK_ARG(tree->kpd[d] <= V, "head %d keeps %d candidates but V=%d", d + 1,
                     tree->kpd[d], V);
  CandArgs a{};
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
  a.topk = topk_idx;
  a.tree_tokens = tree_tokens;
  a.pos = pos;
  dim3 grid(tree->K, B);
  const int km = tree->kmax;
  if (km <= 4)
    hipLaunchKernelGGL(topk_tree_kernel<4>, grid, dim3(THREADS), 0, stream, a);
  else if (km <= 8)
    hipLaunchKernelGGL(topk_tree_kernel<8>, grid, dim3(THREADS), 0, stream, a);
  else if (km <= 16)
    hipLaunchKernelGGL(topk_tree_kernel<16>, grid, dim3(THREADS), 0, stream, a);
  else
    hipLaunchKernelGGL(topk_tree_kernel<32>, grid, dim3(THREADS), 0, stream, a);
  return check_launch("top-k / tree tokens");
}
