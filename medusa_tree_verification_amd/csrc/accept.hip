// Path acceptance: greedy match or rejection sampling over the static tree.
//
// Greedy follows P3 ("Speculative Decoding(투기적 디코딩) 원리와 가속 아키텍처"),
// section 5 (greedy check): drafts are compared with the target's argmax and
// the first mismatch is replaced by it; P4 ("추측 디코딩과 긴 컨텍스트"), section
// 1.3: everything after the first mismatch is dropped and, when every draft
// matches, the target's next prediction is a free extra token.
//
// Rejection sampling follows P1 ("Medusa 심층 아키텍처"), section "수학적 무손실
// 보장: 기각 샘플링": a draft x is accepted iff r < min(1, p(x)/q(x)); after a
// rejection the target distribution is replaced by the residual
// max(0, p - q) / sum(max(0, p - q)); P3, section 2, proves the emitted token
// is distributed as p when the draft is a sample from q.  On the tree the
// children of the current node are tried in rank order (the residual carries
// over from one sibling to the next), an accepted child becomes the current
// node, and the walk ends with one token drawn from the current p by inverse
// CDF.  That guarantee needs drafts drawn from q; a tree filled by top-k
// (deterministic drafts) does not give samples from q, so on such trees the
// output is not exactly distributed as p.  The kernel still computes exactly
// the rule above, which is what its parity with the reference walk checks.
//
// Greedy: one workgroup per (node, sequence) takes the target's argmax of
// that node (first maximum), then the last workgroup of the sequence walks
// the tree.  Rejection sampling: the walk is sequential by nature, so one
// workgroup per sequence walks; for vocabularies up to 32768 entries the
// root's p and every depth's q are first computed in parallel over (row,
// sequence) and the walk keeps p in registers, otherwise each step is a
// block-wide pass over the vocabulary in the workspace.  Probabilities are
// fp64 so that the accept/reject decisions and the sampled token agree with
// an fp64 reference except in ties at the 1e-12 level.
#include "internal.h"

using namespace medusa;

namespace {

__device__ __forceinline__ bool beats(float v, int i, float w, int j) {
  return v > w || (v == w && static_cast<unsigned>(i) < static_cast<unsigned>(j));
}

struct AcceptArgs {
  const float* base;   // [B][T][V]
  const float* head;   // [B][K][V]
  const int32_t* toks; // [B][T]
  const float* ua;     // [B][T]
  const float* us;     // [B][T]
  const int32_t* child_start;
  const int32_t* child_list;
  const int32_t* depth;
  int T, V, K, Kp1, max_depth;
  float tau;
  int32_t* acc_len;
  int32_t* out_tokens;
  int32_t* out_nodes;
  double* pbuf;        // [B][V]       (rejection)
  double* qbuf;        // [B][max_depth + 1][V] (rejection, V <= RT * 32): row 0 the root's p, row d q_d
  int32_t* argmax;     // [B][T]       (greedy)
};

// ---------------------------------------------------------------------------
// greedy: the target's argmax of every tree node in parallel (one workgroup
// per node and sequence, the whole row in flight at once), then a second
// launch walks each sequence's tree over those argmaxes (a second launch
// costs less than publishing the argmaxes device-wide from every workgroup).
// ---------------------------------------------------------------------------
constexpr int GT = 1024;

__global__ __launch_bounds__(GT) void accept_greedy_kernel(AcceptArgs a) {
  const int n = blockIdx.x;
  const int b = blockIdx.y;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  __shared__ float s_v[GT / 64];
  __shared__ int s_i[GT / 64];
  const float* row = a.base + (static_cast<int64_t>(b) * a.T + n) * a.V;
  float bv = -INFINITY;
  int bi = -1;
  if ((a.V & 3) == 0 && (reinterpret_cast<uintptr_t>(row) & 15) == 0) {
    const float4* r4 = reinterpret_cast<const float4*>(row);
    const int n4 = a.V >> 2;
    int v = tid;
    for (; v + 7 * GT < n4; v += 8 * GT) {
      float4 buf[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) buf[k] = r4[v + k * GT];
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const int i0 = 4 * (v + k * GT);
        if (beats(buf[k].x, i0, bv, bi)) { bv = buf[k].x; bi = i0; }
        if (beats(buf[k].y, i0 + 1, bv, bi)) { bv = buf[k].y; bi = i0 + 1; }
        if (beats(buf[k].z, i0 + 2, bv, bi)) { bv = buf[k].z; bi = i0 + 2; }
        if (beats(buf[k].w, i0 + 3, bv, bi)) { bv = buf[k].w; bi = i0 + 3; }
      }
    }
    for (; v < n4; v += GT) {
      const float4 f = r4[v];
      const int i0 = 4 * v;
      if (beats(f.x, i0, bv, bi)) { bv = f.x; bi = i0; }
      if (beats(f.y, i0 + 1, bv, bi)) { bv = f.y; bi = i0 + 1; }
      if (beats(f.z, i0 + 2, bv, bi)) { bv = f.z; bi = i0 + 2; }
      if (beats(f.w, i0 + 3, bv, bi)) { bv = f.w; bi = i0 + 3; }
    }
  } else {
    for (int v = tid; v < a.V; v += GT)
      if (beats(row[v], v, bv, bi)) {
        bv = row[v];
        bi = v;
      }
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    const float ov = __shfl_xor(bv, off, 64);
    const int oi = __shfl_xor(bi, off, 64);
    if (beats(ov, oi, bv, bi)) {
      bv = ov;
      bi = oi;
    }
  }
  if (lane == 0) {
    s_v[wave] = bv;
    s_i[wave] = bi;
  }
  __syncthreads();
  if (tid == 0) {
    float wv = s_v[0];
    int wi = s_i[0];
    for (int w = 1; w < GT / 64; ++w)
      if (beats(s_v[w], s_i[w], wv, wi)) {
        wv = s_v[w];
        wi = s_i[w];
      }
    a.argmax[static_cast<int64_t>(b) * a.T + n] = wi;
  }
}

// The walk, one workgroup per sequence: every node's argmax and token and
// the child lists go to LDS in one parallel round trip, then one thread
// walks the tree there.
constexpr int GW = 256;  // >= MEDUSA_MAX_TREE_NODES + 1

__global__ __launch_bounds__(GW) void accept_greedy_walk(AcceptArgs a) {
  const int b = blockIdx.x;
  const int tid = threadIdx.x;
  __shared__ int32_t s_am[MEDUSA_MAX_TREE_NODES], s_tk[MEDUSA_MAX_TREE_NODES];
  __shared__ int32_t s_cs[MEDUSA_MAX_TREE_NODES + 1], s_cl[MEDUSA_MAX_TREE_NODES];
  const int32_t* am = a.argmax + static_cast<int64_t>(b) * a.T;
  const int32_t* tk = a.toks + static_cast<int64_t>(b) * a.T;
  for (int i = tid; i <= a.T; i += GW) {
    if (i < a.T) {
      s_am[i] = am[i];
      s_tk[i] = tk[i];
    }
    s_cs[i] = a.child_start[i];
    if (i < a.T - 1) s_cl[i] = a.child_list[i];
  }
  __syncthreads();
  if (tid != 0) return;
  int32_t* onodes = a.out_nodes + static_cast<int64_t>(b) * a.Kp1;
  int32_t* otoks = a.out_tokens + static_cast<int64_t>(b) * a.Kp1;
  int u = 0, len = 0;
  while (true) {
    onodes[len] = u;
    const int t = s_am[u];
    int nxt = -1;
    for (int ci = s_cs[u]; ci < s_cs[u + 1]; ++ci) {
      const int c = s_cl[ci];
      if (s_tk[c] == t) {
        nxt = c;
        break;
      }
    }
    if (nxt < 0 || len >= a.max_depth) {
      otoks[len] = t;
      break;
    }
    otoks[len] = s_tk[nxt];
    ++len;
    u = nxt;
  }
  a.acc_len[b] = len;
  for (int j = len + 1; j < a.Kp1; ++j) {
    otoks[j] = -1;
    onodes[j] = -1;
  }
}

// ---------------------------------------------------------------------------
// rejection sampling (fp64)
// ---------------------------------------------------------------------------
constexpr int RT = 1024;
constexpr int RW = RT / 64;

__device__ double block_sum(double x, double* sh) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off, 64);
  __syncthreads();
  if (lane == 0) sh[wave] = x;
  __syncthreads();
  double s = 0.0;
  for (int w = 0; w < RW; ++w) s += sh[w];  // same order in every thread
  return s;
}

__device__ double block_max(double x, double* sh) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x = fmax(x, __shfl_xor(x, off, 64));
  __syncthreads();
  if (lane == 0) sh[wave] = x;
  __syncthreads();
  double m = sh[0];
  for (int w = 1; w < RW; ++w) m = fmax(m, sh[w]);
  return m;
}

__device__ int block_min_int(int x, int* sh) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x = min(x, __shfl_xor(x, off, 64));
  __syncthreads();
  if (lane == 0) sh[wave] = x;
  __syncthreads();
  int m = sh[0];
  for (int w = 1; w < RW; ++w) m = min(m, sh[w]);
  return m;
}

__device__ int block_max_int(int x, int* sh) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x = max(x, __shfl_xor(x, off, 64));
  __syncthreads();
  if (lane == 0) sh[wave] = x;
  __syncthreads();
  int m = sh[0];
  for (int w = 1; w < RW; ++w) m = max(m, sh[w]);
  return m;
}

// p <- softmax(z / tau), fp64, written to p[0..V)
__device__ void softmax_into(const float* z, double tau, int V, double* p, double* shd) {
  double mx = -INFINITY;
  for (int v = threadIdx.x; v < V; v += RT) mx = fmax(mx, static_cast<double>(z[v]) / tau);
  mx = block_max(mx, shd);
  double s = 0.0;
  for (int v = threadIdx.x; v < V; v += RT) {
    const double e = exp(static_cast<double>(z[v]) / tau - mx);
    p[v] = e;
    s += e;
  }
  const double Z = block_sum(s, shd);
  for (int v = threadIdx.x; v < V; v += RT) p[v] = p[v] / Z;
  __syncthreads();
}

// Draw the final token from p by inverse CDF with u_sample[b][u] (chunked
// prefix sums in thread order) and finish the sequence's outputs.
__device__ void sample_tail(const AcceptArgs& a, int b, int u, int len, const double* p, int* shi,
                            int32_t* otoks, int32_t* onodes) {
  const int V = a.V;
  const int tid = threadIdx.x;
  const int C = (V + RT - 1) / RT;
  const int v0 = tid * C;
  const int v1 = min(V, v0 + C);
  double local = 0.0;
  for (int v = v0; v < v1; ++v) local += p[v];
  // exclusive scan of the per-thread sums (wave scan, then wave totals)
  const int lane = tid & 63, wave = tid >> 6;
  double incl = local;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const double o = __shfl_up(incl, off, 64);
    if (lane >= off) incl += o;
  }
  __shared__ double s_wsum[RW];
  if (lane == 63) s_wsum[wave] = incl;
  __syncthreads();
  double wave_off = 0.0, total = 0.0;
  for (int w = 0; w < RW; ++w) {
    if (w < wave) wave_off += s_wsum[w];
    total += s_wsum[w];
  }
  const double thr = static_cast<double>(a.us[static_cast<int64_t>(b) * a.T + u]) * total;
  double run = wave_off + incl - local;
  int hit = 0x7fffffff, lastpos = -1;
  for (int v = v0; v < v1; ++v) {
    run += p[v];
    if (run > thr) {
      hit = v;
      break;
    }
  }
  for (int v = v0; v < v1; ++v)
    if (p[v] > 0.0) lastpos = v;
  hit = block_min_int(hit, shi);
  lastpos = block_max_int(lastpos, shi);
  if (tid == 0) {
    const int y = (hit != 0x7fffffff) ? hit : lastpos;
    otoks[len] = y;
    a.acc_len[b] = len;
    for (int j = len + 1; j < a.Kp1; ++j) {
      otoks[j] = -1;
      onodes[j] = -1;
    }
  }
}

__global__ __launch_bounds__(RT) void accept_reject_kernel(AcceptArgs a) {
  const int b = blockIdx.x;
  const int tid = threadIdx.x;
  __shared__ double shd[RW];
  __shared__ int shi[RW];
  __shared__ double s_mq[MEDUSA_MAX_HEADS + 1], s_zq[MEDUSA_MAX_HEADS + 1];
  const double tau = static_cast<double>(a.tau);
  const int V = a.V;
  double* p = a.pbuf + static_cast<int64_t>(b) * V;
  const float* hb = a.head + static_cast<int64_t>(b) * a.K * V;
  const int32_t* tk = a.toks + static_cast<int64_t>(b) * a.T;

  // q_d = softmax(head[d-1] / tau): keep its max and normaliser per depth
  for (int d = 1; d <= a.max_depth; ++d) {
    const float* h = hb + static_cast<int64_t>(d - 1) * V;
    double mx = -INFINITY;
    for (int v = tid; v < V; v += RT) mx = fmax(mx, static_cast<double>(h[v]) / tau);
    mx = block_max(mx, shd);
    double s = 0.0;
    for (int v = tid; v < V; v += RT) s += exp(static_cast<double>(h[v]) / tau - mx);
    s = block_sum(s, shd);
    if (tid == 0) {
      s_mq[d] = mx;
      s_zq[d] = s;
    }
  }
  __syncthreads();

  softmax_into(a.base + static_cast<int64_t>(b) * a.T * V, tau, V, p, shd);
  int u = 0, len = 0;
  int32_t* onodes = a.out_nodes + static_cast<int64_t>(b) * a.Kp1;
  int32_t* otoks = a.out_tokens + static_cast<int64_t>(b) * a.Kp1;
  if (tid == 0) onodes[0] = 0;
  while (true) {
    int accepted = -1;
    for (int ci = a.child_start[u]; ci < a.child_start[u + 1]; ++ci) {
      const int c = a.child_list[ci];
      const int d = a.depth[c];
      const int x = min(max(tk[c], 0), V - 1);  // a token outside the vocabulary is clamped
      const float* h = hb + static_cast<int64_t>(d - 1) * V;
      const double mq = s_mq[d], zq = s_zq[d];
      const double qx = exp(static_cast<double>(h[x]) / tau - mq) / zq;
      const double px = p[x];
      const double alpha = (qx == 0.0) ? 1.0 : fmin(1.0, px / qx);
      if (static_cast<double>(a.ua[static_cast<int64_t>(b) * a.T + c]) < alpha) {
        accepted = c;
        break;
      }
      // residual max(0, p - q_d), renormalised
      double s = 0.0;
      for (int v = tid; v < V; v += RT) {
        const double q = exp(static_cast<double>(h[v]) / tau - mq) / zq;
        const double r = fmax(0.0, p[v] - q);
        p[v] = r;
        s += r;
      }
      const double Z = block_sum(s, shd);
      if (Z > 0.0)
        for (int v = tid; v < V; v += RT) p[v] = p[v] / Z;
      __syncthreads();
    }
    if (accepted < 0) break;
    if (tid == 0) {
      otoks[len] = min(max(tk[accepted], 0), V - 1);
      onodes[len + 1] = accepted;
    }
    ++len;
    u = accepted;
    softmax_into(a.base + (static_cast<int64_t>(b) * a.T + u) * V, tau, V, p, shd);
  }

  sample_tail(a, b, u, len, p, shi, otoks, onodes);
}

// ---- rejection sampling with the distributions in registers (V <= RT * PER) ----
// The formulas of accept_reject_kernel, per thread in the same order (thread
// t owns v = t + RT * i), except that each division by tau or by a row sum
// is a multiplication by its reciprocal (one rounding apart: fp64 values
// agree to an ulp, decisions agree except at ties of that size).
// First, in parallel over (row, sequence): the root's p = softmax(base / tau)
// and each depth's q_d = softmax(head[d-1] / tau), fp64, into qbuf.  Then one
// workgroup per sequence walks the tree with p in registers: p(x) comes from
// its owner thread, q from qbuf, and a rejection's residual and
// renormalisation never leave the registers, nor does the final
// inverse-CDF draw.  Rows are read and written through buffer
// descriptors that end at the row's end (element i of a thread at the scalar
// offset RT * i): past V a load reads 0 and a store is dropped, so padded
// elements add exact zeros to the sums and need no guard there.
constexpr int RSRC_WORD3 = 0x00020000;  // raw buffer, 32-bit data format
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ __amdgpu_buffer_rsrc_t row_rsrc(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, bytes, RSRC_WORD3);
}
__device__ __forceinline__ double ld_f64(__amdgpu_buffer_rsrc_t r, int voff, int soff) {
  return __builtin_bit_cast(double, __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, 0));
}
__device__ __forceinline__ float ld_f32(__amdgpu_buffer_rsrc_t r, int voff, int soff) {
  return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, 0));
}
__device__ __forceinline__ void st_f64(double x, __amdgpu_buffer_rsrc_t r, int voff, int soff) {
  __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, x), r, voff, soff, 0);
}

// p = softmax(z / tau) of one row into registers (the arithmetic of
// softmax_into, per thread in the same order); z is read twice in batches
template <int PER>
__device__ __forceinline__ void softmax_regs(const float* z, double inv_tau, int V, int nv, double (&pr)[PER],
                                             double* shd) {
  const int tid = threadIdx.x;
  const __amdgpu_buffer_rsrc_t rz = row_rsrc(z, V * 4);
  constexpr int ZB = PER < 16 ? PER : 16;
  double mx = -INFINITY;
#pragma unroll
  for (int h = 0; h < PER; h += ZB) {
    float zv[ZB];
#pragma unroll
    for (int j = 0; j < ZB; ++j) zv[j] = ld_f32(rz, tid * 4, RT * 4 * (h + j));
#pragma unroll
    for (int j = 0; j < ZB; ++j)
      if (h + j < nv) mx = fmax(mx, static_cast<double>(zv[j]) * inv_tau);
  }
  mx = block_max(mx, shd);
  double s = 0.0;
#pragma unroll
  for (int h = 0; h < PER; h += ZB) {
    float zv[ZB];
#pragma unroll
    for (int j = 0; j < ZB; ++j) zv[j] = ld_f32(rz, tid * 4, RT * 4 * (h + j));
#pragma unroll
    for (int j = 0; j < ZB; ++j) {
      pr[h + j] = 0.0;
      if (h + j < nv) {
        pr[h + j] = exp(static_cast<double>(zv[j]) * inv_tau - mx);
        s += pr[h + j];
      }
    }
  }
  const double inv_z = 1.0 / block_sum(s, shd);
#pragma unroll
  for (int i = 0; i < PER; ++i) pr[i] *= inv_z;
}

template <int PER>
__global__ __launch_bounds__(RT) void accept_rows_kernel(AcceptArgs a) {
  const int d = blockIdx.x, b = blockIdx.y;
  const int tid = threadIdx.x;
  __shared__ double shd[RW];
  const int V = a.V;
  const int nv = tid < V ? (V - tid + RT - 1) / RT : 0;  // this thread's elements below V
  const float* z = d == 0 ? a.base + static_cast<int64_t>(b) * a.T * V
                          : a.head + (static_cast<int64_t>(b) * a.K + d - 1) * V;
  double pr[PER];
  softmax_regs<PER>(z, 1.0 / static_cast<double>(a.tau), V, nv, pr, shd);
  const __amdgpu_buffer_rsrc_t ro =
      row_rsrc(a.qbuf + (static_cast<int64_t>(b) * (a.max_depth + 1) + d) * V, V * 8);
#pragma unroll
  for (int i = 0; i < PER; ++i) st_f64(pr[i], ro, tid * 8, RT * 8 * i);
}

template <int PER>
__global__ __launch_bounds__(RT) void accept_walk_kernel(AcceptArgs a) {
  const int b = blockIdx.x;
  const int tid = threadIdx.x;
  __shared__ double shd[RW];
  __shared__ int shi[RW];
  __shared__ double s_px;
  const double inv_tau = 1.0 / static_cast<double>(a.tau);
  const int V = a.V;
  const int nv = tid < V ? (V - tid + RT - 1) / RT : 0;
  const double* qb = a.qbuf + static_cast<int64_t>(b) * (a.max_depth + 1) * V;
  const int32_t* tk = a.toks + static_cast<int64_t>(b) * a.T;
  double pr[PER];  // p[tid + RT * i]; 0 past V
  {
    const __amdgpu_buffer_rsrc_t r0 = row_rsrc(qb, V * 8);
#pragma unroll
    for (int i = 0; i < PER; ++i) pr[i] = ld_f64(r0, tid * 8, RT * 8 * i);
  }
  int u = 0, len = 0;
  int32_t* onodes = a.out_nodes + static_cast<int64_t>(b) * a.Kp1;
  int32_t* otoks = a.out_tokens + static_cast<int64_t>(b) * a.Kp1;
  if (tid == 0) onodes[0] = 0;
  while (true) {
    int accepted = -1;
    // the walk is the same in every thread: node, depth and token are uniform
    const int c_end = __builtin_amdgcn_readfirstlane(a.child_start[u + 1]);
    for (int ci = __builtin_amdgcn_readfirstlane(a.child_start[u]); ci < c_end; ++ci) {
      const int c = __builtin_amdgcn_readfirstlane(a.child_list[ci]);
      const int d = __builtin_amdgcn_readfirstlane(a.depth[c]);
      const int x = __builtin_amdgcn_readfirstlane(min(max(tk[c], 0), V - 1));  // clamped to the vocabulary
      const double* q = qb + static_cast<int64_t>(d) * V;
      const double qx = q[x];
      if (tid == x % RT) {
        double px = 0.0;
#pragma unroll
        for (int i = 0; i < PER; ++i)
          if (i == x / RT) px = pr[i];
        s_px = px;
      }
      __syncthreads();
      const double px = s_px;
      __syncthreads();  // every thread has read s_px before it is written again
      const double alpha = (qx == 0.0) ? 1.0 : fmin(1.0, px / qx);
      const bool take = static_cast<double>(a.ua[static_cast<int64_t>(b) * a.T + c]) < alpha;
      if (__builtin_amdgcn_readfirstlane(static_cast<int>(take))) {  // the same in every thread
        accepted = c;
        break;
      }
      // residual max(0, p - q_d), renormalised; q in batches of 16
      const __amdgpu_buffer_rsrc_t rq = row_rsrc(q, V * 8);
      constexpr int QB = PER < 16 ? PER : 16;
      double s = 0.0;
#pragma unroll
      for (int h = 0; h < PER; h += QB) {
        double qv[QB];
#pragma unroll
        for (int j = 0; j < QB; ++j) qv[j] = ld_f64(rq, tid * 8, RT * 8 * (h + j));
#pragma unroll
        for (int j = 0; j < QB; ++j) {
          const double r = fmax(0.0, pr[h + j] - qv[j]);  // 0 past V
          pr[h + j] = r;
          s += r;
        }
      }
      const double Z = block_sum(s, shd);
      if (Z > 0.0) {
        const double inv_z = 1.0 / Z;
#pragma unroll
        for (int i = 0; i < PER; ++i) pr[i] *= inv_z;
      }
    }
    if (accepted < 0) break;
    if (tid == 0) {
      otoks[len] = min(max(tk[accepted], 0), V - 1);
      onodes[len + 1] = accepted;
    }
    ++len;
    u = __builtin_amdgcn_readfirstlane(accepted);
    softmax_regs<PER>(a.base + (static_cast<int64_t>(b) * a.T + u) * V, inv_tau, V, nv, pr, shd);
  }
  // Inverse CDF from the registers: the smallest v with cumsum(p)[v] >
  // u_sample * sum(p), else the last v with p > 0.  The vocabulary is taken
  // in groups of 8 rows (8192 entries) staged through LDS in v order; thread
  // t sums entries 8t .. 8t+7 of the group, an exclusive block scan gives
  // each thread the sum before them, and the first group that crosses the
  // threshold ends the search.
  double tsum = 0.0;
  int lastpos = -1;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    tsum += pr[i];
    if (pr[i] > 0.0) lastpos = tid + RT * i;
  }
  const double total = block_sum(tsum, shd);
  lastpos = block_max_int(lastpos, shi);
  const double thr = static_cast<double>(a.us[static_cast<int64_t>(b) * a.T + u]) * total;
  __shared__ double s_grp[8 * RT];
  __shared__ double s_wsum[RW];
  const int lane = tid & 63, wave = tid >> 6;
  double before_grp = 0.0;  // cumsum before the group (the same in every thread)
  int hit = 0x7fffffff;
#pragma unroll
  for (int g = 0; g < PER; g += 8) {
    __syncthreads();  // the previous group's reads are done
#pragma unroll
    for (int j = 0; j < 8; ++j) s_grp[j * RT + tid] = pr[g + j];  // entry v - RT*g
    __syncthreads();
    double loc = 0.0;
#pragma unroll
    for (int k = 0; k < 8; ++k) loc += s_grp[8 * tid + k];
    double incl = loc;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const double o = __shfl_up(incl, off, 64);
      if (lane >= off) incl += o;
    }
    if (lane == 63) s_wsum[wave] = incl;
    __syncthreads();
    double wave_off = 0.0, gtot = 0.0;
    for (int w = 0; w < RW; ++w) {
      if (w < wave) wave_off += s_wsum[w];
      gtot += s_wsum[w];
    }
    double run = before_grp + wave_off + incl - loc;
    int h = 0x7fffffff;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      run += s_grp[8 * tid + k];
      if (run > thr && h == 0x7fffffff) h = RT * g + 8 * tid + k;
    }
    hit = block_min_int(h, shi);
    if (hit != 0x7fffffff) break;
    before_grp += gtot;
  }
  if (tid == 0) {
    otoks[len] = (hit != 0x7fffffff) ? hit : lastpos;
    a.acc_len[b] = len;
    for (int j = len + 1; j < a.Kp1; ++j) {
      otoks[j] = -1;
      onodes[j] = -1;
    }
  }
}

// elements per thread of the register-resident rejection path (0: V too
// large, the vocabulary stays in the workspace)
int reject_per(int V) { return V <= RT * 8 ? 8 : V <= RT * 16 ? 16 : V <= RT * 32 ? 32 : 0; }

template <int PER>
int launch_reject_regs(const AcceptArgs& a, int B, hipStream_t stream) {
  hipLaunchKernelGGL((accept_rows_kernel<PER>), dim3(a.max_depth + 1, B), dim3(RT), 0, stream, a);
  int rc = check_launch("rejection-sampling rows (root p, q per depth)");
  if (rc) return rc;
  hipLaunchKernelGGL((accept_walk_kernel<PER>), dim3(B), dim3(RT), 0, stream, a);
  return check_launch("rejection-sampling acceptance");
}

}  // namespace

extern "C" size_t medusa_accept_workspace_size(int B, int V, const medusa_tree_t* tree,
                                               float temperature) {
  if (B < 1 || V < 1 || !tree) return 0;
  if (temperature == 0.f)
    return round_up(static_cast<size_t>(B) * tree->T * 4, 256);
  size_t n = round_up(static_cast<size_t>(B) * V * sizeof(double), 256);
  if (reject_per(V)) n += round_up(static_cast<size_t>(B) * (tree->max_depth + 1) * V * sizeof(double), 256);
  return n;
}

extern "C" int medusa_accept_paths(const float* base_logits, const float* head_logits,
                                   const int32_t* tree_tokens, const medusa_tree_t* tree,
                                   const float* u_accept, const float* u_sample, float temperature,
                                   int B, int V, int32_t* accept_len, int32_t* out_tokens,
                                   int32_t* out_nodes, void* ws, size_t ws_bytes,
                                   hipStream_t stream) {
  clear_error();
  int rc = check_tree(tree);
  if (rc) return rc;
  MEDUSA_CHECK_ARG(base_logits && tree_tokens && accept_len && out_tokens && out_nodes,
                   "base_logits, tree_tokens and the outputs must be non-NULL");
  MEDUSA_CHECK_ARG(B >= 1 && V >= 1, "B=%d and V=%d must be >= 1", B, V);
  MEDUSA_CHECK_ARG(temperature >= 0.f && temperature < 1e30f,
                   "temperature=%g must be >= 0 and finite", static_cast<double>(temperature));
  AcceptArgs a{};
  a.base = base_logits;
  a.head = head_logits;
  a.toks = tree_tokens;
  a.ua = u_accept;
  a.us = u_sample;
  a.child_start = tree->d_child_start;
  a.child_list = tree->d_child_list;
  a.depth = tree->d_depth;
  a.T = tree->T;
  a.V = V;
  a.K = tree->K;
  a.Kp1 = tree->K + 1;
  a.max_depth = tree->max_depth;
  a.tau = temperature;
  a.acc_len = accept_len;
  a.out_tokens = out_tokens;
  a.out_nodes = out_nodes;
  if (temperature != 0.f)
    MEDUSA_CHECK_ARG(head_logits && u_accept && u_sample,
                     "rejection sampling needs head_logits, u_accept and u_sample");
  const size_t need = medusa_accept_workspace_size(B, V, tree, temperature);
  if (!ws || ws_bytes < need || !aligned256(ws)) {
    set_error("acceptance workspace: need %zu bytes, 256-byte aligned (got %zu at %p)", need,
              ws_bytes, ws);
    return MEDUSA_EWORKSPACE;
  }
  if (temperature == 0.f) {
    a.argmax = static_cast<int32_t*>(ws);
    hipLaunchKernelGGL(accept_greedy_kernel, dim3(tree->T, B), dim3(GT), 0, stream, a);
    int rc = check_launch("greedy acceptance (argmax)");
    if (rc) return rc;
    hipLaunchKernelGGL(accept_greedy_walk, dim3(B), dim3(GW), 0, stream, a);
    return check_launch("greedy acceptance (walk)");
  }
  a.pbuf = static_cast<double*>(ws);
  switch (reject_per(V)) {
    case 8:
    case 16:
    case 32:
      a.qbuf = reinterpret_cast<double*>(static_cast<char*>(ws) +
                                         round_up(static_cast<size_t>(B) * V * sizeof(double), 256));
      if (reject_per(V) == 8) return launch_reject_regs<8>(a, B, stream);
      if (reject_per(V) == 16) return launch_reject_regs<16>(a, B, stream);
      return launch_reject_regs<32>(a, B, stream);
    default:
      hipLaunchKernelGGL(accept_reject_kernel, dim3(B), dim3(RT), 0, stream, a);
      return check_launch("rejection-sampling acceptance");
  }
}
