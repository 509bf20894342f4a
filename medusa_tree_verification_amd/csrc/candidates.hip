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
// One workgroup of 1024 threads per (head, sequence), radix select:
//   1. each logit becomes an order-preserving 32-bit key (larger logit ->
//      larger key; -0 is keyed as +0);
//   2. the k-th largest key K* is found digit by digit (11, 11 and 10 bits):
//      an LDS histogram of the keys that match the digits found so far, then
//      a scan from the top bucket down finds the bucket holding the k-th;
//   3. every key above K* is a winner; when more keys equal K* than are still
//      needed, the smallest indices among them are found the same way (a
//      radix select on the index);
//   4. the k winners are ranked by (value, index) inside one wave.
// The same workgroup then writes the tree tokens and positions of the nodes
// at depth head+1 (and the root, for head 0).
#include "internal.h"

using namespace medusa;

namespace {

constexpr int THREADS = 1024;
constexpr int WAVES = THREADS / 64;
constexpr int REG_VALUES = 32;  // values per thread kept in registers
constexpr int BINS = 2048;      // histogram buckets (11-bit digits)

__device__ __forceinline__ uint32_t order_key(float y) {
  uint32_t u = __float_as_uint(y == 0.f ? 0.f : y);  // -0 keyed as +0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
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

struct Shared {
  int hist[BINS];
  int wave_sum[WAVES];
  int found_bin, found_before;  // bucket of the target rank, count above it
  int n_win;
  uint32_t win_key[MEDUSA_MAX_TOPK];
  uint32_t win_idx[MEDUSA_MAX_TOPK];
  int top[MEDUSA_MAX_TOPK];
};

// Given the histogram of one digit, find the bucket that holds the element
// of rank `want` (1-based) counting from the top bucket (descending = true)
// or from the bottom one.  Writes found_bin / found_before.
__device__ void find_bucket(Shared& sh, int want, bool descending) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // thread t owns ordered positions 2t and 2t+1
  const int b0 = descending ? BINS - 1 - 2 * tid : 2 * tid;
  const int b1 = descending ? b0 - 1 : b0 + 1;
  const int h0 = sh.hist[b0], h1 = sh.hist[b1];
  int x = h0 + h1;  // inclusive scan over threads in position order
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(x, off, 64);
    if (lane >= off) x += y;
  }
  if (lane == 63) sh.wave_sum[wave] = x;
  __syncthreads();
  int before = 0;
  for (int w = 0; w < wave; ++w) before += sh.wave_sum[w];
  const int incl = before + x;
  const int excl = incl - h0 - h1;
  if (excl < want && want <= incl) {
    if (want <= excl + h0) {
      sh.found_bin = b0;
      sh.found_before = excl;
    } else {
      sh.found_bin = b1;
      sh.found_before = excl + h0;
    }
  }
  __syncthreads();
}

template <bool REG>
__global__ __launch_bounds__(THREADS) void topk_tree_kernel(CandArgs a) {
  const int head = blockIdx.x;
  const int b = blockIdx.y;
  const int tid = threadIdx.x;
  const float* x = a.logits + (static_cast<int64_t>(b) * a.K + head) * a.V;
  const int kd = a.kpd[head];
  __shared__ Shared sh;

  // ---- 1. keys ----
  uint32_t keys[REG ? REG_VALUES : 1];
  if (REG) {
#pragma unroll
    for (int j = 0; j < REG_VALUES; ++j) {
      const int v = tid + j * THREADS;
      keys[j] = v < a.V ? order_key(x[v]) : 0u;  // key 0 is below every logit's key
    }
  }
  // visit every (key, index) of the row (registers or a strided re-read)
  auto for_each = [&](auto&& f) __attribute__((always_inline)) {
    if (REG) {
#pragma unroll
      for (int j = 0; j < REG_VALUES; ++j) {
        const int v = tid + j * THREADS;
        if (v < a.V) f(keys[j], static_cast<uint32_t>(v));
      }
    } else {
      for (int v = tid; v < a.V; v += THREADS) f(order_key(x[v]), static_cast<uint32_t>(v));
    }
  };

  // ---- 2. K* = the kd-th largest key, one digit at a time ----
  uint32_t prefix = 0, pmask = 0;
  int want = kd;  // rank of K* among the keys matching the prefix
  const int shifts[3] = {21, 10, 0};
  const uint32_t widths[3] = {0x7FFu, 0x7FFu, 0x3FFu};
  for (int p = 0; p < 3; ++p) {
    for (int i = tid; i < BINS; i += THREADS) sh.hist[i] = 0;
    __syncthreads();
    for_each([&](uint32_t k, uint32_t) {
      if ((k & pmask) == prefix) atomicAdd(&sh.hist[(k >> shifts[p]) & widths[p]], 1);
    });
    __syncthreads();
    find_bucket(sh, want, true);
    want -= sh.found_before;
    prefix |= static_cast<uint32_t>(sh.found_bin) << shifts[p];
    pmask |= widths[p] << shifts[p];
    __syncthreads();  // everyone has read found_* before the next pass rewrites it
  }
  const uint32_t kstar = prefix;
  const int equal = sh.hist[kstar & 0x3FFu];  // keys equal to K* (last digit's bucket)
  // keys above K*: kd - want of them; ties needed: want (1 <= want <= equal)

  // ---- 3. winners: keys above K*, then the `want` smallest tied indices ----
  uint32_t imax = 0xFFFFFFFFu;  // take tied indices <= imax
  if (want < equal) {
    // radix select of the want-th smallest index among keys == K* (2 digits)
    uint32_t ip = 0, im = 0;
    int w2 = want;
    const int ishift[2] = {11, 0};
    for (int p = 0; p < 2; ++p) {
      __syncthreads();
      for (int i = tid; i < BINS; i += THREADS) sh.hist[i] = 0;
      __syncthreads();
      for_each([&](uint32_t k, uint32_t v) {
        if (k == kstar && (v & im) == ip) atomicAdd(&sh.hist[(v >> ishift[p]) & 0x7FFu], 1);
      });
      __syncthreads();
      find_bucket(sh, w2, false);
      w2 -= sh.found_before;
      ip |= static_cast<uint32_t>(sh.found_bin) << ishift[p];
      im |= 0x7FFu << ishift[p];
    }
    imax = ip;
  }
  if (tid == 0) sh.n_win = 0;
  __syncthreads();
  for_each([&](uint32_t k, uint32_t v) {
    if (k > kstar || (k == kstar && v <= imax)) {
      const int slot = atomicAdd(&sh.n_win, 1);
      if (slot < MEDUSA_MAX_TOPK) {
        sh.win_key[slot] = k;
        sh.win_idx[slot] = v;
      }
    }
  });
  __syncthreads();

  // ---- 4. rank the kd winners by (value desc, index asc) ----
  if (tid < kd) {
    const uint32_t k = sh.win_key[tid], v = sh.win_idx[tid];
    int r = 0;
    for (int j = 0; j < kd; ++j) {
      const uint32_t kj = sh.win_key[j], vj = sh.win_idx[j];
      r += (kj > k || (kj == k && vj < v)) ? 1 : 0;
    }
    sh.top[r] = static_cast<int>(v);
  }
  __syncthreads();

  int32_t* out = a.topk + (static_cast<int64_t>(b) * a.K + head) * a.kmax;
  for (int j = tid; j < a.kmax; j += THREADS) out[j] = j < kd ? sh.top[j] : -1;

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
      a.tree_tokens[static_cast<int64_t>(b) * a.T + n] = sh.top[a.rank[n]];
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
  // indices are radix-selected in two 11-bit digits
  MEDUSA_CHECK_ARG(V <= (1 << 22), "V=%d above 4194304", V);
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
