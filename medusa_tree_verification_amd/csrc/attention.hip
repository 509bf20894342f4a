// Tree-masked attention of one layer (split-KV flash decode).
//
// P1 ("Medusa 심층 아키텍처"), section "트리 어텐션 ... 2차원 어텐션 마스크": the T
// tree tokens are verified in one attention pass; tree token i sees the whole
// cached context and, among the tree tokens, only its ancestors and itself.
// P4 ("추측 디코딩과 긴 컨텍스트"), section 3.3: attention over separate key
// blocks can be merged exactly by tracking the running max and exp-sum (the
// online softmax), which is what lets the key range be cut into splits and
// waves here and merged afterwards.
//
// bf16 design (gfx950, D = 128)
//   Work item: one workgroup (4 waves) per (sequence b, K/V head, query chunk,
//   key split).  All T*G query rows of a K/V head (G = Hq/Hkv; row r = node
//   r/G, query head r%G) are handled by the same workgroup, so every K/V byte
//   of the split is read from HBM once.  The 4 waves are QG query groups x KS
//   key sub-splits; a wave owns QTW tiles of 16 query rows and every KS-th
//   32-key block of the split.
//   Scores: S^T = K Q^T on v_mfma_f32_16x16x32_bf16, K as the A operand read
//   straight from HBM (lane l: key l%16, 64 contiguous bytes of d), Q as B
//   kept in registers for the whole kernel.  The d order is permuted the same
//   way in both operands.  Result layout: lane l holds query l%16 and 4
//   consecutive keys, so every lane's softmax state (max, sum, rescale) is
//   its own query's.
//   Values: O^T += V^T P^T.  The MFMA wants 8 consecutive keys of one d per
//   lane, V is stored [key][d], so each wave transposes its V block through a
//   private LDS tile: rows = d, 4-key granules of 8 bytes, rows padded to 72
//   bytes and granules XOR-swizzled by (d/16)%8, which keeps both the
//   transposing 8-byte writes and the 8-byte operand reads free of bank
//   conflicts.  P^T comes straight from the score registers (converted to
//   bf16) because the key order of the MFMA k-slots is chosen to match them.
//   Mask: context keys are always visible; tree key j is visible to node i
//   iff bit j of node i's ancestor bitmask is set (rows staged in LDS).  Only
//   blocks that reach past the context evaluate it.
//   exp2 with log2(e) folded into the scale; fp32 scores, sums and outputs.
//   Partials of a split (unnormalised O, max, sum) go to the workspace and a
//   second kernel merges the splits in a fixed order (deterministic).
//   Workgroups are numbered so that all splits of one (b, K/V head) land on
//   the same XCD (dispatch assigns workgroup i to XCD i % 8).
#include <cstdlib>

#include "internal.h"

using namespace medusa;
using namespace medusa::dev;

namespace {

constexpr int D = 128;
constexpr int KB = 32;                 // keys per block
constexpr int VROWB = 72;              // bytes per V^T row in LDS (64 + 8 pad)
constexpr int VT_BYTES = D * VROWB;    // one wave's V^T tile
constexpr float LOG2E = 1.4426950408889634f;

struct AttnArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const int32_t* ctx;
  const uint64_t* mask;  // [T][W]
  int W, B, T, Hq, Hkv, G, S_cap;
  int QR, QRpad, QC, NS, chunk;
  int tasks, per_xcd;
  float scale_log2;
  uint16_t* out;
  float* part_o;   // [NS][B*Hkv][QRpad][D]
  float* part_ml;  // [NS][B*Hkv][QRpad][2]
  int mask_bytes;  // LDS bytes reserved for the mask rows
};

__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__device__ __forceinline__ float wave_max_16_32(float x) {
  x = fmaxf(x, __shfl_xor(x, 16, 64));
  x = fmaxf(x, __shfl_xor(x, 32, 64));
  return x;
}

__device__ __forceinline__ uint4 ldg16(const uint16_t* p) {
  return *reinterpret_cast<const uint4*>(p);
}

template <int QTW>
struct KVRegs {
  uint4 k[2][4];  // [16-key subtile][d step]
  uint4 v[2][4];  // [quad half][key in quad]
};

template <int QTW, int QG, int KS>
__global__ __launch_bounds__(256) void tree_attn_bf16(AttnArgs a) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  const int id = blockIdx.x;
  const int task = (id & 7) * a.per_xcd + (id >> 3);
  if (task >= a.tasks) return;  // whole workgroup leaves before any barrier
  const int split = task % a.NS;
  const int rest = task / a.NS;
  const int qc = rest % a.QC;
  const int bh = rest / a.QC;
  const int b = bh / a.Hkv;
  const int kvh = bh % a.Hkv;

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int qg = wave / KS;
  const int ks = wave % KS;
  const int l16 = lane & 15;
  const int grp = lane >> 4;

  uint64_t* smask = reinterpret_cast<uint64_t*>(smem);
  float* sml = reinterpret_cast<float*>(smem + a.mask_bytes);           // [4][QTW*16][2]
  char* sbig = smem + a.mask_bytes + 4 * QTW * 16 * 2 * 4;               // V^T tiles / merge
  for (int i = threadIdx.x; i < a.T * a.W; i += 256) smask[i] = a.mask[i];
  __syncthreads();

  int ctx = a.ctx[b];
  ctx = ctx < 0 ? 0 : (ctx > a.S_cap - a.T ? a.S_cap - a.T : ctx);
  const int S = ctx + a.T;
  const int k_begin = split * a.chunk;
  const int k_end = (split == a.NS - 1) ? S : min(S, k_begin + a.chunk);

  // ---- Q fragments (B operand of S^T = K Q^T) ----
  const int row_base = (qc * QG + qg) * QTW * 16;
  uint4 qf[QTW][4];
  int qnode[QTW];
#pragma unroll
  for (int t = 0; t < QTW; ++t) {
    const int r = row_base + t * 16 + l16;
    const bool ok = r < a.QR;
    const int node = ok ? r / a.G : 0;
    const int gq = ok ? r % a.G : 0;
    qnode[t] = node;
    const uint16_t* qp =
        a.q + ((static_cast<int64_t>(b) * a.T + node) * a.Hq + kvh * a.G + gq) * D + grp * 32;
#pragma unroll
    for (int s = 0; s < 4; ++s) qf[t][s] = ok ? ldg16(qp + 8 * s) : make_uint4(0, 0, 0, 0);
  }

  f32x4 o[QTW][8];
  float m_run[QTW], l_run[QTW];
#pragma unroll
  for (int t = 0; t < QTW; ++t) {
    m_run[t] = -INFINITY;
    l_run[t] = 0.f;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) o[t][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  const uint16_t* kbase = a.k + static_cast<int64_t>(bh) * a.S_cap * D;
  const uint16_t* vbase = a.v + static_cast<int64_t>(bh) * a.S_cap * D;
  char* vt = sbig + wave * VT_BYTES;

  auto load_kv = [&](KVRegs<QTW>& r, int kb) {
#pragma unroll
    for (int st = 0; st < 2; ++st) {
      const int key = kb + st * 16 + l16;
      const bool ok = key < k_end;
      const uint16_t* p = kbase + static_cast<int64_t>(ok ? key : 0) * D + grp * 32;
#pragma unroll
      for (int s = 0; s < 4; ++s) r.k[st][s] = ok ? ldg16(p + 8 * s) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int h = 0; h < 2; ++h) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int key = kb + 4 * (grp + 4 * h) + i;
        const bool ok = key < k_end;
        const uint16_t* p = vbase + static_cast<int64_t>(ok ? key : 0) * D + 8 * l16;
        r.v[h][i] = ok ? ldg16(p) : make_uint4(0, 0, 0, 0);
      }
    }
  };

  auto compute = [&](const KVRegs<QTW>& r, int kb) {
    // V block -> transposed, swizzled LDS tile
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int q = grp + 4 * h;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int d = 8 * l16 + e;
        uint32_t w0, w1;
        const uint32_t a0 = reinterpret_cast<const uint32_t*>(&r.v[h][0])[e >> 1];
        const uint32_t a1 = reinterpret_cast<const uint32_t*>(&r.v[h][1])[e >> 1];
        const uint32_t a2 = reinterpret_cast<const uint32_t*>(&r.v[h][2])[e >> 1];
        const uint32_t a3 = reinterpret_cast<const uint32_t*>(&r.v[h][3])[e >> 1];
        if ((e & 1) == 0) {
          w0 = (a0 & 0xffffu) | (a1 << 16);
          w1 = (a2 & 0xffffu) | (a3 << 16);
        } else {
          w0 = (a0 >> 16) | (a1 & 0xffff0000u);
          w1 = (a2 >> 16) | (a3 & 0xffff0000u);
        }
        const int gp = q ^ ((d >> 4) & 7);
        *reinterpret_cast<uint2*>(vt + d * VROWB + gp * 8) = make_uint2(w0, w1);
      }
    }
    // scores S^T = K Q^T for 2 subtiles x QTW query tiles
    f32x4 sc[2][QTW];
#pragma unroll
    for (int st = 0; st < 2; ++st) {
#pragma unroll
      for (int t = 0; t < QTW; ++t) {
        f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < 4; ++s)
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(r.k[st][s]), as_bf16x8(qf[t][s]),
                                                        acc, 0, 0, 0);
        sc[st][t] = acc * a.scale_log2;
      }
    }
    // mask (only blocks reaching past the context or the end of the split)
    if (kb + KB > ctx || kb + KB > k_end) {
#pragma unroll
      for (int st = 0; st < 2; ++st) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int key = kb + st * 16 + 4 * grp + e;
          const int j = key - ctx;
#pragma unroll
          for (int t = 0; t < QTW; ++t) {
            bool vis = key < k_end;
            if (vis && j >= 0) {
              const uint64_t wd = smask[qnode[t] * a.W + (j >> 6)];
              vis = (wd >> (j & 63)) & 1ull;
            }
            if (!vis) sc[st][t][e] = -INFINITY;
          }
        }
      }
    }
    // online softmax per query (lane-local state; max shared across the 4 lane groups)
    bf16x8 pb[QTW];
#pragma unroll
    for (int t = 0; t < QTW; ++t) {
      float bm = fmaxf(fmaxf(fmaxf(sc[0][t][0], sc[0][t][1]), fmaxf(sc[0][t][2], sc[0][t][3])),
                       fmaxf(fmaxf(sc[1][t][0], sc[1][t][1]), fmaxf(sc[1][t][2], sc[1][t][3])));
      bm = wave_max_16_32(bm);
      const float mnew = fmaxf(m_run[t], bm);
      const float muse = (mnew == -INFINITY) ? 0.f : mnew;
      const float alpha = __builtin_amdgcn_exp2f(m_run[t] - muse);
      m_run[t] = mnew;
      float ps = 0.f;
#pragma unroll
      for (int st = 0; st < 2; ++st) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float p = __builtin_amdgcn_exp2f(sc[st][t][e] - muse);
          ps += p;
          pb[t][st * 4 + e] = static_cast<__bf16>(p);
        }
      }
      l_run[t] = l_run[t] * alpha + ps;
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) o[t][dt] *= alpha;
    }
    wave_lds_sync();
    // O^T += V^T P^T
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
      const int d = dt * 16 + l16;
      const char* rowp = vt + d * VROWB;
      const uint2 lo = *reinterpret_cast<const uint2*>(rowp + ((grp ^ (dt & 7)) * 8));
      const uint2 hi = *reinterpret_cast<const uint2*>(rowp + (((grp + 4) ^ (dt & 7)) * 8));
      const bf16x8 va = as_bf16x8(make_uint4(lo.x, lo.y, hi.x, hi.y));
#pragma unroll
      for (int t = 0; t < QTW; ++t)
        o[t][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, pb[t], o[t][dt], 0, 0, 0);
    }
    wave_lds_sync();
  };

  // ---- main loop: register double buffer over this wave's blocks ----
  const int stride = KS * KB;
  int kb = k_begin + ks * KB;
  if (kb < k_end) {
    KVRegs<QTW> ra, rb;
    load_kv(ra, kb);
    while (true) {
      const int kb1 = kb + stride;
      if (kb1 < k_end) load_kv(rb, kb1);
      compute(ra, kb);
      if (kb1 >= k_end) break;
      const int kb2 = kb1 + stride;
      if (kb2 < k_end) load_kv(ra, kb2);
      compute(rb, kb1);
      if (kb2 >= k_end) break;
      kb = kb2;
    }
  }

  // full per-query sums (each lane group holds a quarter of the keys)
#pragma unroll
  for (int t = 0; t < QTW; ++t) {
    l_run[t] += __shfl_xor(l_run[t], 16, 64);
    l_run[t] += __shfl_xor(l_run[t], 32, 64);
  }

  // ---- merge the KS key sub-splits of each query group ----
  if (KS > 1) {
    if (grp == 0) {
#pragma unroll
      for (int t = 0; t < QTW; ++t) {
        sml[(wave * QTW * 16 + t * 16 + l16) * 2 + 0] = m_run[t];
        sml[(wave * QTW * 16 + t * 16 + l16) * 2 + 1] = l_run[t];
      }
    }
    __syncthreads();  // also: every wave has finished with its V^T tile
#pragma unroll
    for (int t = 0; t < QTW; ++t) {
      float M = -INFINITY;
#pragma unroll
      for (int w = 0; w < KS; ++w)
        M = fmaxf(M, sml[((qg * KS + w) * QTW * 16 + t * 16 + l16) * 2 + 0]);
      const float muse = (M == -INFINITY) ? 0.f : M;
      float L = 0.f;
#pragma unroll
      for (int w = 0; w < KS; ++w) {
        const int idx = ((qg * KS + w) * QTW * 16 + t * 16 + l16) * 2;
        L += sml[idx + 1] * __builtin_amdgcn_exp2f(sml[idx] - muse);
      }
      const float f = __builtin_amdgcn_exp2f(m_run[t] - muse);
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) o[t][dt] *= f;
      m_run[t] = M;
      l_run[t] = L;
    }
    // waves ks >= 1 hand their O to wave ks == 0 of the same query group
    f32x4* slot = reinterpret_cast<f32x4*>(sbig);
    const int per_wave = QTW * 8 * 64;  // f32x4 entries
    if (ks > 0) {
      f32x4* dst = slot + (qg * (KS - 1) + (ks - 1)) * per_wave;
#pragma unroll
      for (int t = 0; t < QTW; ++t)
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) dst[(t * 8 + dt) * 64 + lane] = o[t][dt];
    }
    __syncthreads();
    if (ks > 0) return;  // no barriers follow
    for (int w = 1; w < KS; ++w) {
      const f32x4* src = slot + (qg * (KS - 1) + (w - 1)) * per_wave;
#pragma unroll
      for (int t = 0; t < QTW; ++t)
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) o[t][dt] += src[(t * 8 + dt) * 64 + lane];
    }
  }

  // ---- write: final output (one split) or the split's partial ----
  const int BH = a.B * a.Hkv;
#pragma unroll
  for (int t = 0; t < QTW; ++t) {
    const int r = row_base + t * 16 + l16;
    if (r >= a.QR) continue;
    if (a.NS == 1) {
      const float inv = 1.0f / l_run[t];
      const int node = r / a.G, gq = r % a.G;
      uint16_t* op = a.out + ((static_cast<int64_t>(b) * a.T + node) * a.Hq + kvh * a.G + gq) * D;
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) {
        const int d = dt * 16 + 4 * grp;
        const uint32_t lo = f32_to_bf16_bits(o[t][dt][0] * inv) | (f32_to_bf16_bits(o[t][dt][1] * inv) << 16);
        const uint32_t hi = f32_to_bf16_bits(o[t][dt][2] * inv) | (f32_to_bf16_bits(o[t][dt][3] * inv) << 16);
        *reinterpret_cast<uint2*>(op + d) = make_uint2(lo, hi);
      }
    } else {
      const int64_t prow = (static_cast<int64_t>(split) * BH + bh) * a.QRpad + r;
      float* po = a.part_o + prow * D;
#pragma unroll
      for (int dt = 0; dt < 8; ++dt)
        *reinterpret_cast<f32x4*>(po + dt * 16 + 4 * grp) = o[t][dt];
      if (grp == 0) {
        a.part_ml[prow * 2 + 0] = m_run[t];
        a.part_ml[prow * 2 + 1] = l_run[t];
      }
    }
  }
}

// Merge the NS split partials of every query row, in split order.
// grid: ceil(BH*QR / 4); block 256 (one wave per row, 2 d-values per lane)
__global__ __launch_bounds__(256) void merge_splits(AttnArgs a) {
  const int lane = threadIdx.x & 63;
  const int BH = a.B * a.Hkv;
  const int64_t gr = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (gr >= static_cast<int64_t>(BH) * a.QR) return;
  const int bh = static_cast<int>(gr / a.QR);
  const int r = static_cast<int>(gr % a.QR);
  float M = -INFINITY;
  for (int s = 0; s < a.NS; ++s)
    M = fmaxf(M, a.part_ml[((static_cast<int64_t>(s) * BH + bh) * a.QRpad + r) * 2]);
  const float muse = (M == -INFINITY) ? 0.f : M;
  float L = 0.f, o0 = 0.f, o1 = 0.f;
  for (int s = 0; s < a.NS; ++s) {
    const int64_t prow = (static_cast<int64_t>(s) * BH + bh) * a.QRpad + r;
    const float w = __builtin_amdgcn_exp2f(a.part_ml[prow * 2] - muse);
    L += a.part_ml[prow * 2 + 1] * w;
    const float2 v = *reinterpret_cast<const float2*>(a.part_o + prow * D + 2 * lane);
    o0 += v.x * w;
    o1 += v.y * w;
  }
  const float inv = 1.0f / L;
  const int b = bh / a.Hkv, kvh = bh % a.Hkv;
  const int node = r / a.G, gq = r % a.G;
  uint16_t* op = a.out + ((static_cast<int64_t>(b) * a.T + node) * a.Hq + kvh * a.G + gq) * D + 2 * lane;
  *reinterpret_cast<uint32_t*>(op) = f32_to_bf16_bits(o0 * inv) | (f32_to_bf16_bits(o1 * inv) << 16);
}

// ---- fp32 path: one wave per (b, node, query head), keys in sequence ----
struct AttnF32Args {
  const float* q;
  const float* k;
  const float* v;
  const int32_t* ctx;
  const uint64_t* mask;
  int W, B, T, Hq, Hkv, G, S_cap, Dd;
  float scale;
  float* out;
};

__global__ __launch_bounds__(256) void tree_attn_f32(AttnF32Args a) {
  const int lane = threadIdx.x & 63;
  const int64_t row = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (row >= static_cast<int64_t>(a.B) * a.T * a.Hq) return;
  const int h = static_cast<int>(row % a.Hq);
  const int i = static_cast<int>((row / a.Hq) % a.T);
  const int b = static_cast<int>(row / (static_cast<int64_t>(a.Hq) * a.T));
  const int kvh = h / a.G;
  int ctx = a.ctx[b];
  ctx = ctx < 0 ? 0 : (ctx > a.S_cap - a.T ? a.S_cap - a.T : ctx);
  const float* qp = a.q + row * a.Dd;
  const float q0 = lane < a.Dd ? qp[lane] : 0.f;
  const float q1 = lane + 64 < a.Dd ? qp[lane + 64] : 0.f;
  const float* kb = a.k + (static_cast<int64_t>(b) * a.Hkv + kvh) * a.S_cap * a.Dd;
  const float* vb = a.v + (static_cast<int64_t>(b) * a.Hkv + kvh) * a.S_cap * a.Dd;
  const uint64_t* mrow = a.mask + static_cast<int64_t>(i) * a.W;
  float m = -INFINITY, l = 0.f, o0 = 0.f, o1 = 0.f;
  const int S = ctx + a.T;
  for (int key = 0; key < S; ++key) {
    if (key >= ctx) {
      const int j = key - ctx;
      if (!((mrow[j >> 6] >> (j & 63)) & 1ull)) continue;
    }
    const float* kr = kb + static_cast<int64_t>(key) * a.Dd;
    float s = 0.f;
    if (lane < a.Dd) s = q0 * kr[lane];
    if (lane + 64 < a.Dd) s = fmaf(q1, kr[lane + 64], s);
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) s += __shfl_xor(s, off, 64);
    s *= a.scale;
    const float mnew = fmaxf(m, s);
    const float alpha = expf(m - mnew);
    const float p = expf(s - mnew);
    const float* vr = vb + static_cast<int64_t>(key) * a.Dd;
    l = l * alpha + p;
    o0 = o0 * alpha + (lane < a.Dd ? p * vr[lane] : 0.f);
    o1 = o1 * alpha + (lane + 64 < a.Dd ? p * vr[lane + 64] : 0.f);
    m = mnew;
  }
  float* op = a.out + row * a.Dd;
  if (lane < a.Dd) op[lane] = o0 / l;
  if (lane + 64 < a.Dd) op[lane + 64] = o1 / l;
}

// ---- launch planning -------------------------------------------------------
struct Plan {
  int G, QR, NQT, QTW, QG, KS, QC, QRpad, NS, chunk;
  size_t ws_bytes;
  int lds_bytes;
};

int env_int(const char* name, int dflt) {
  const char* s = std::getenv(name);
  return s ? std::atoi(s) : dflt;
}

Plan make_plan(int B, int Hq, int Hkv, int ctx_max, int T, int W) {
  Plan p{};
  p.G = Hq / Hkv;
  p.QR = T * p.G;
  p.NQT = (p.QR + 15) / 16;
  // A wave keeps at most 3 query tiles (48 rows) of state in registers; more
  // query tiles go to more waves of the workgroup (QG groups sharing each K/V
  // block) and then to more workgroups (QC chunks).
  if (p.NQT <= 3) {
    p.QTW = p.NQT;
    p.QG = 1;
  } else if (p.NQT <= 6) {
    p.QG = 2;
    p.QTW = (p.NQT + 1) / 2;
  } else {
    p.QG = 4;
    const int qc = (p.NQT + 11) / 12;
    p.QTW = (p.NQT + 4 * qc - 1) / (4 * qc);
  }
  p.KS = 4 / p.QG;
  p.QC = (p.NQT + p.QG * p.QTW - 1) / (p.QG * p.QTW);
  p.QRpad = p.NQT * 16;
  const int Smax = ctx_max + T;
  const int base = B * Hkv * p.QC;
  int ns = env_int("MEDUSA_ATTN_SPLITS", 0);
  if (ns <= 0) {
    ns = (512 + base - 1) / base;          // about two workgroups per CU
    const int max_ns = (Smax + 2 * p.KS * KB - 1) / (2 * p.KS * KB);  // >= 2 blocks per wave
    if (ns > max_ns) ns = max_ns;
    if (ns < 1) ns = 1;
  }
  int chunk = (Smax + ns - 1) / ns;
  chunk = (chunk + KB - 1) / KB * KB;
  p.chunk = chunk;
  p.NS = (Smax + chunk - 1) / chunk;
  if (p.NS < 1) p.NS = 1;
  p.ws_bytes = p.NS > 1 ? round_up(static_cast<size_t>(p.NS) * B * Hkv * p.QRpad * (D + 2) * 4, 256)
                        : 0;
  const int mask_bytes = static_cast<int>(round_up(static_cast<size_t>(T) * W * 8, 16));
  const int ml_bytes = 4 * p.QTW * 16 * 2 * 4;
  const int vt = 4 * VT_BYTES;
  const int merge = p.KS > 1 ? p.QG * (p.KS - 1) * p.QTW * 8 * 64 * 16 : 0;
  p.lds_bytes = mask_bytes + ml_bytes + (vt > merge ? vt : merge);
  return p;
}

template <int QTW, int QG, int KS>
void launch_cfg(const AttnArgs& a, int grid, int lds, hipStream_t s) {
  hipLaunchKernelGGL((tree_attn_bf16<QTW, QG, KS>), dim3(grid), dim3(256), lds, s, a);
}

bool launch_bf16(const Plan& p, const AttnArgs& a, int grid, hipStream_t s) {
#define MEDUSA_CASE(QTW_, QG_, KS_)                                                \
  if (p.QTW == QTW_ && p.QG == QG_ && p.KS == KS_) {                               \
    static bool attr_set = false;                                                  \
    if (!attr_set) {                                                               \
      (void)hipFuncSetAttribute(                                                   \
          reinterpret_cast<const void*>(&tree_attn_bf16<QTW_, QG_, KS_>),          \
          hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);                 \
      attr_set = true;                                                             \
    }                                                                              \
    launch_cfg<QTW_, QG_, KS_>(a, grid, p.lds_bytes, s);                           \
    return true;                                                                   \
  }
  MEDUSA_CASE(1, 1, 4)
  MEDUSA_CASE(2, 1, 4)
  MEDUSA_CASE(3, 1, 4)
  MEDUSA_CASE(2, 2, 2)
  MEDUSA_CASE(3, 2, 2)
  MEDUSA_CASE(2, 4, 1)
  MEDUSA_CASE(3, 4, 1)
#undef MEDUSA_CASE
  return false;
}

}  // namespace

extern "C" size_t medusa_tree_attention_workspace_size(int B, int Hq, int Hkv, int D_, int ctx_max,
                                                       const medusa_tree_t* tree,
                                                       medusa_dtype_t dt) {
  if (!tree || B < 1 || Hkv < 1 || Hq < Hkv || Hq % Hkv || ctx_max < 0) return 0;
  if (dt != MEDUSA_BF16 || D_ != D) return 0;
  return make_plan(B, Hq, Hkv, ctx_max, tree->T, tree->W).ws_bytes;
}

extern "C" int medusa_tree_attention(const void* q, const void* k_cache, const void* v_cache,
                                     const int32_t* ctx_len, int ctx_max, const medusa_tree_t* tree,
                                     int B, int Hq, int Hkv, int D_, int S_cap, float scale,
                                     medusa_dtype_t dt, void* out, void* ws, size_t ws_bytes,
                                     hipStream_t stream) {
  clear_error();
  int rc = check_tree(tree);
  if (rc) return rc;
  MEDUSA_CHECK_ARG(q && k_cache && v_cache && ctx_len && out, "tensor arguments must be non-NULL");
  MEDUSA_CHECK_ARG(B >= 1 && Hkv >= 1 && Hq >= Hkv && Hq % Hkv == 0,
                   "need B >= 1 and Hq (%d) a positive multiple of Hkv (%d)", Hq, Hkv);
  MEDUSA_CHECK_ARG(ctx_max >= 0 && S_cap >= ctx_max + tree->T,
                   "S_cap=%d must hold ctx_max=%d plus the T=%d tree tokens", S_cap, ctx_max, tree->T);
  MEDUSA_CHECK_ARG(scale > 0.f && scale < 1e30f, "scale=%g must be positive and finite",
                   static_cast<double>(scale));
  MEDUSA_CHECK_ARG(aligned16(q) && aligned16(k_cache) && aligned16(v_cache) && aligned16(out),
                   "tensor pointers must be 16-byte aligned");
  if (dt == MEDUSA_F32) {
    if (D_ < 1 || D_ > 128 || D_ % 4) {
      set_error("f32 tree attention supports D in 1..128 with D %% 4 == 0 (D=%d)", D_);
      return MEDUSA_EUNSUPPORTED;
    }
    AttnF32Args f{};
    f.q = static_cast<const float*>(q);
    f.k = static_cast<const float*>(k_cache);
    f.v = static_cast<const float*>(v_cache);
    f.ctx = ctx_len;
    f.mask = tree->d_mask;
    f.W = tree->W;
    f.B = B;
    f.T = tree->T;
    f.Hq = Hq;
    f.Hkv = Hkv;
    f.G = Hq / Hkv;
    f.S_cap = S_cap;
    f.Dd = D_;
    f.scale = scale;
    f.out = static_cast<float*>(out);
    const int64_t rows = static_cast<int64_t>(B) * tree->T * Hq;
    hipLaunchKernelGGL(tree_attn_f32, dim3(static_cast<unsigned>((rows + 3) / 4)), dim3(256), 0,
                       stream, f);
    return check_launch("tree attention (f32)");
  }
  MEDUSA_CHECK_ARG(dt == MEDUSA_BF16, "unknown dtype %d", static_cast<int>(dt));
  if (D_ != D) {
    set_error("bf16 tree attention supports D = 128 (got D=%d)", D_);
    return MEDUSA_EUNSUPPORTED;
  }
  const Plan p = make_plan(B, Hq, Hkv, ctx_max, tree->T, tree->W);
  if (p.NS > 1 && (!ws || ws_bytes < p.ws_bytes || !aligned256(ws))) {
    set_error("tree attention workspace: need %zu bytes, 256-byte aligned (got %zu at %p)",
              p.ws_bytes, ws_bytes, ws);
    return MEDUSA_EWORKSPACE;
  }
  if (p.lds_bytes > 160 * 1024) {
    set_error("tree attention needs %d bytes of LDS (T=%d too large)", p.lds_bytes, tree->T);
    return MEDUSA_EUNSUPPORTED;
  }
  AttnArgs a{};
  a.q = static_cast<const uint16_t*>(q);
  a.k = static_cast<const uint16_t*>(k_cache);
  a.v = static_cast<const uint16_t*>(v_cache);
  a.ctx = ctx_len;
  a.mask = tree->d_mask;
  a.W = tree->W;
  a.B = B;
  a.T = tree->T;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.G = p.G;
  a.S_cap = S_cap;
  a.QR = p.QR;
  a.QRpad = p.QRpad;
  a.QC = p.QC;
  a.NS = p.NS;
  a.chunk = p.chunk;
  a.tasks = B * Hkv * p.QC * p.NS;
  a.per_xcd = (a.tasks + 7) / 8;
  a.scale_log2 = scale * LOG2E;
  a.out = static_cast<uint16_t*>(out);
  a.part_o = p.NS > 1 ? static_cast<float*>(ws) : nullptr;
  a.part_ml = p.NS > 1 ? reinterpret_cast<float*>(static_cast<char*>(ws) +
                                                  static_cast<size_t>(p.NS) * B * Hkv * p.QRpad * D * 4)
                       : nullptr;
  a.mask_bytes = static_cast<int>(round_up(static_cast<size_t>(tree->T) * tree->W * 8, 16));
  if (!launch_bf16(p, a, 8 * a.per_xcd, stream)) {
    set_error("no tree attention kernel for QTW=%d QG=%d KS=%d", p.QTW, p.QG, p.KS);
    return MEDUSA_EUNSUPPORTED;
  }
  rc = check_launch("tree attention (bf16)");
  if (rc || p.NS == 1) return rc;
  const int64_t rows = static_cast<int64_t>(B) * Hkv * p.QR;
  hipLaunchKernelGGL(merge_splits, dim3(static_cast<unsigned>((rows + 3) / 4)), dim3(256), 0, stream, a);
  return check_launch("tree attention split merge");
}
