// Per-head top-k and candidate tree tokens.
//
// P1 ("Medusa 심층 아키텍처"), section "소스코드 레벨 구조 분석": every head keeps
// the indices of its k largest logits (generate_candidates); P2 ("[vLLM]
// Medusa"), section "propose()", is the k = 1 case.  P1, section "트리 어텐션
// ... 고정 트리 토폴로지": the fixed topology combines head d's candidates at
// depth d, so node n carries candidate rank(n) of head depth(n), and sits
// depth(n) positions after the cached context.
//
// Order: larger logit first; equal logits by smaller index.  Comparing
// (value, index) pairs this way is a total order, so the result is unique
// and bit-exact.
//
// One workgroup of 1024 threads per (head, sequence), three phases:
//   1. every thread takes the best of its strided share of the row (kept in
//      registers when the row has at most 32 values per thread);
//   2. the k-th best of the 1024 per-thread bests is a threshold: the k
//      threads whose best beats or equals it hold k distinct entries at or
//      above it, so every true top-k entry is at or above it too.  It is
//      found by k wave arg-max rounds per wave, then k rounds over the
//      waves' survivors;
//   3. entries at or above the threshold (at most k per contributing thread,
//      i.e. at most k * values-per-thread) are collected in LDS and the exact
//      top-k is selected from them by k more arg-max rounds.
// The same workgroup then writes the tree tokens and positions of the nodes
// at depth head+1 (and the root, for head 0).
#include "internal.h"

using namespace medusa;

namespace {

constexpr int THREADS = 1024;
constexpr int WAVES = THREADS / 64;
constexpr int REG_VALUES = 32;            // values per thread kept in registers
constexpr int MAX_CAND = 4096;            // LDS candidate capacity
constexpr unsigned NONE = 0xffffffffu;    // index of an empty / removed slot

// (v, i) beats (w, j) in the output order
__device__ __forceinline__ bool beats(float v, unsigned i, float w, unsigned j) {
  return v > w || (v == w && i < j);
}

__device__ __forceinline__ void wave_argmax(float& v, unsigned& i) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    const float ov = __shfl_xor(v, off, 64);
    const unsigned oi = __shfl_xor(i, off, 64);
    if (beats(ov, oi, v, i)) {
      v = ov;
      i = oi;
    }
  }
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

// k rounds of wave arg-max over per-lane slot arrays (slots kept in LDS).
// cv/ci: the lane's slots are cand_v[base + lane + 64*s], s < per_lane.
// Returns in lanes r < kd the r-th best (value, index); removes winners.
__device__ void wave_select(float* cand_v, unsigned* cand_i, int n, int kd, float& out_v,
                            unsigned& out_i) {
  const int lane = threadIdx.x & 63;
  // lane-local best slot
  auto local_best = [&](float& bv, unsigned& bi, int& bs) {
    bv = -INFINITY;
    bi = NONE;
    bs = -1;
    for (int s = lane; s < n; s += 64) {
      if (beats(cand_v[s], cand_i[s], bv, bi)) {
        bv = cand_v[s];
        bi = cand_i[s];
        bs = s;
      }
    }
  };
  float bv;
  unsigned bi;
  int bs;
  local_best(bv, bi, bs);
  out_v = -INFINITY;
  out_i = NONE;
  for (int r = 0; r < kd; ++r) {
    float wv = bv;
    unsigned wi = bi;
    wave_argmax(wv, wi);
    if (lane == r) {
      out_v = wv;
      out_i = wi;
    }
    if (wi != NONE && bi == wi) {  // owner removes the winner and rescans its slots
      cand_v[bs] = -INFINITY;
      cand_i[bs] = NONE;
      local_best(bv, bi, bs);
    }
  }
}

template <bool REG>
__global__ __launch_bounds__(THREADS) void topk_tree_kernel(CandArgs a) {
  const int head = blockIdx.x;
  const int b = blockIdx.y;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const float* x = a.logits + (static_cast<int64_t>(b) * a.K + head) * a.V;
  const int kd = a.kpd[head];

  __shared__ float s_v[MAX_CAND];
  __shared__ unsigned s_i[MAX_CAND];
  __shared__ int s_n;
  __shared__ float s_thv;
  __shared__ unsigned s_thi;
  __shared__ int s_top[MEDUSA_MAX_TOPK];

  // ---- 1. per-thread best ----
  float vals[REG ? REG_VALUES : 1];
  float bv = -INFINITY;
  unsigned bi = NONE;
  if (REG) {
#pragma unroll
    for (int j = 0; j < REG_VALUES; ++j) {
      const int v = tid + j * THREADS;
      vals[j] = v < a.V ? x[v] : -INFINITY;
    }
#pragma unroll
    for (int j = 0; j < REG_VALUES; ++j) {
      const unsigned v = tid + j * THREADS;
      if (v < static_cast<unsigned>(a.V) && beats(vals[j], v, bv, bi)) {
        bv = vals[j];
        bi = v;
      }
    }
  } else {
    for (int v = tid; v < a.V; v += THREADS) {
      const float y = x[v];
      if (beats(y, v, bv, bi)) {
        bv = y;
        bi = v;
      }
    }
  }

  // ---- 2. threshold = k-th best of the per-thread bests ----
  {
    float cv = bv;
    unsigned ci = bi;
    float keep_v = -INFINITY;
    unsigned keep_i = NONE;
    for (int r = 0; r < kd; ++r) {  // wave-level: one slot per lane
      float wv = cv;
      unsigned wi = ci;
      wave_argmax(wv, wi);
      if (lane == r) {
        keep_v = wv;
        keep_i = wi;
      }
      if (wi != NONE && ci == wi) {
        cv = -INFINITY;
        ci = NONE;
      }
    }
    if (lane < kd) {
      s_v[wave * kd + lane] = keep_v;
      s_i[wave * kd + lane] = keep_i;
    }
  }
  __syncthreads();
  if (wave == 0) {
    float ov;
    unsigned oi;
    wave_select(s_v, s_i, WAVES * kd, kd, ov, oi);
    if (lane == kd - 1) {
      s_thv = ov;
      s_thi = oi;
    }
    if (lane == 0) s_n = 0;
  }
  __syncthreads();
  const float thv = s_thv;
  const unsigned thi = s_thi;

  // ---- 3. collect entries at or above the threshold, select exactly ----
  auto offer = [&](float y, unsigned v) {
    if (v == thi || beats(y, v, thv, thi)) {
      const int slot = atomicAdd(&s_n, 1);
      if (slot < MAX_CAND) {
        s_v[slot] = y;
        s_i[slot] = v;
      }
    }
  };
  if (REG) {
#pragma unroll
    for (int j = 0; j < REG_VALUES; ++j) {
      const unsigned v = tid + j * THREADS;
      if (v < static_cast<unsigned>(a.V)) offer(vals[j], v);
    }
  } else {
    for (int v = tid; v < a.V; v += THREADS) offer(x[v], v);
  }
  __syncthreads();
  if (wave == 0) {
    const int n = min(s_n, MAX_CAND);
    float ov;
    unsigned oi;
    wave_select(s_v, s_i, n, kd, ov, oi);
    if (lane < kd) s_top[lane] = static_cast<int>(oi);
  }
  __syncthreads();

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
  // the candidate list holds at most k * ceil(V / 1024) entries
  const long long per_thread = (static_cast<long long>(V) + THREADS - 1) / THREADS;
  if (per_thread * tree->kmax > MAX_CAND) {
    set_error("top-%d over V=%d exceeds the candidate buffer (%d)", tree->kmax, V, MAX_CAND);
    return MEDUSA_EUNSUPPORTED;
  }
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
  if (V <= THREADS * REG_VALUES)
    hipLaunchKernelGGL(topk_tree_kernel<true>, grid, dim3(THREADS), 0, stream, a);
  else
    hipLaunchKernelGGL(topk_tree_kernel<false>, grid, dim3(THREADS), 0, stream, a);
  return check_launch("top-k / tree tokens");
}
