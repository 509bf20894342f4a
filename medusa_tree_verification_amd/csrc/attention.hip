// Tree-masked attention of one layer (split-KV flash decode).
//
// P1 ("Medusa 심층 아키텍처"), section "트리 어텐션 ... 2차원 어텐션 마스크": the T
// tree tokens are verified in one attention pass; tree token i sees the whole
// cached context and, among the tree tokens, only its ancestors and itself.
// P4 ("추측 디코딩과 긴 컨텍스트"), section 3.3: attention over separate key
// blocks can be merged exactly by tracking the running max and exp-sum (the
// online softmax), which is what lets the key range be cut into splits and
// merged afterwards.
//
// bf16 design (gfx950, D = 128)
//   Work item: one workgroup (4 waves) per (sequence b, K/V head, query chunk,
//   key split).  All T*G query rows of a K/V head (G = Hq/Hkv; row r = node
//   r/G, query head r%G) go through the same pass over its keys, so every K/V
//   byte of the split is read from HBM once.  The query tiles (16 rows) of
//   the chunk are dealt round-robin to the 4 waves; every wave consumes every
//   32-key block.
//   Staging: the workgroup streams its key range in 32-key blocks (16 KB of
//   K and V).  Each thread loads 64 bytes of every block into registers,
//   three blocks ahead of use, then writes them to a ring of LDS slots: half
//   the threads store K rows with their 16-byte chunks XOR-swizzled by key
//   (conflict-free MFMA operand reads), the other half hold 4 keys x 8 d of V
//   and store them transposed (rows = d, 4-key granules of 8 bytes, rows
//   padded to 72 bytes, granules swizzled by (d/16)%8) -- the layout the
//   P.V product needs.  One barrier per block; a slot is rewritten only
//   after every wave has passed the barrier that follows its last use.
//   Scores: S^T = K Q^T on v_mfma_f32_16x16x32_bf16 (K rows as the A
//   operand, Q rows, staged once in LDS, as B; the d order is permuted the
//   same way in both).  Lane l then holds query l%16 and 4 keys, so every
//   lane's softmax state (max, sum, rescale) is its own query's.
//   Values: O^T += V^T P^T; P^T comes straight from the score registers
//   (packed to bf16) because the key order of the MFMA k-slots is chosen to
//   match them.
//   Mask: context keys are always visible; tree key j is visible to node i
//   iff bit j of node i's ancestor bitmask is set (rows staged in LDS); only
//   blocks that reach past the context evaluate it.
//   exp2 with log2(e) folded into the scale; fp32 scores, sums and outputs.
//   Splits: each workgroup writes its partial (unnormalised O, max, sum); a
//   second kernel merges the splits of every row in split order (fixed
//   order: deterministic).  Workgroups are numbered so that all splits of one
//   (b, K/V head) land on the same XCD (dispatch assigns workgroup i to XCD
//   i % 8), which keeps their partials in one L2.
#include <cmath>
#include <cstdlib>

#include "internal.h"

using namespace medusa;
using namespace medusa::dev;

namespace {

constexpr int D = 128;
constexpr int KB = 64;                  // keys per staged block
constexpr int HALF = 32;                // keys per compute half (one P.V MFMA k-step)
constexpr int VROWB = 72;               // bytes per V^T row (64 + 8 pad)
constexpr int VT_BYTES = D * VROWB;     // one 32-key V^T tile: 9216
constexpr int KROWB = D * 2;            // 256 bytes per K row
constexpr int K_BYTES = KB * KROWB;     // 16384
constexpr int SLOT_BYTES = K_BYTES + 2 * VT_BYTES;
constexpr int QROW_CHUNKS = D / 8;      // 16-byte chunks per Q / K row
constexpr int PREFETCH = 2;             // blocks in flight per workgroup (= LDS slots)
constexpr int RSRC_WORD3 = 0x00020000;  // raw buffer, 32-bit data format
constexpr float LOG2E = 1.4426950408889634f;

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

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
  int lds_mask, lds_q, lds_ring;  // dynamic LDS layout (byte offsets)
};

__device__ __forceinline__ float wave_max_16_32(float x) {
  x = fmaxf(x, __shfl_xor(x, 16, 64));
  x = fmaxf(x, __shfl_xor(x, 32, 64));
  return x;
}

__device__ __forceinline__ uint4 ldg16(const uint16_t* p) {
  return *reinterpret_cast<const uint4*>(p);
}

__device__ __forceinline__ uint4 bload16(__amdgpu_buffer_rsrc_t r, int byte_off) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, 0));
}

__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  const bf16x2 v = {static_cast<__bf16>(lo), static_cast<__bf16>(hi)};
  return __builtin_bit_cast(uint32_t, v);
}

struct Stage {
  uint4 k[4];  // 64 bytes of one K row
  uint4 v[4];  // 4 keys x 8 d of V
};

template <int QTW>
__global__ __launch_bounds__(256) void tree_attn_bf16(AttnArgs a) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  const int id = blockIdx.x;
  const int task = (id & 7) * a.per_xcd + (id >> 3);
  if (task >= a.tasks) return;  // whole workgroup leaves before any barrier
  const int split = task % a.NS;
  const int rest = task / a.NS;  // = bh * QC + qc
  const int qc = rest % a.QC;
  const int bh = rest / a.QC;
  const int b = bh / a.Hkv;
  const int kvh = bh % a.Hkv;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l16 = lane & 15;
  const int grp = lane >> 4;

  int ctx = a.ctx[b];
  ctx = ctx < 0 ? 0 : (ctx > a.S_cap - a.T ? a.S_cap - a.T : ctx);
  const int S = ctx + a.T;
  const int k_begin = split * a.chunk;
  const int k_end = (split == a.NS - 1) ? S : min(S, k_begin + a.chunk);
  const int nblk = k_end > k_begin ? (k_end - k_begin + KB - 1) / KB : 0;

  // K/V of this (b, head) as buffer resources limited to the split's end:
  // reads of keys >= k_end return zeros (never the unused cache slots)
  const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(a.k + static_cast<int64_t>(bh) * a.S_cap * D), 0, k_end * KROWB, RSRC_WORD3);
  const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(a.v + static_cast<int64_t>(bh) * a.S_cap * D), 0, k_end * KROWB, RSRC_WORD3);

  // staging roles (every thread): K row tid/4, 16-byte chunks 4*(tid%4)..+3;
  // V keys 4*(tid/16)..+3 at d-octet tid%16
  const int k_row = tid >> 2, k_ch = (tid & 3) * 4;
  const int v_quad = tid >> 4, v_oct = tid & 15;
  auto gload = [&](Stage& st, int blk) __attribute__((always_inline)) {
    const int kb = k_begin + blk * KB;
    const int ko = (kb + k_row) * KROWB + k_ch * 16;
#pragma unroll
    for (int i = 0; i < 4; ++i) st.k[i] = bload16(rk, ko + 16 * i);
#pragma unroll
    for (int i = 0; i < 4; ++i) st.v[i] = bload16(rv, (kb + 4 * v_quad + i) * KROWB + v_oct * 16);
  };
  auto lds_put = [&](const Stage& st, char* slot) __attribute__((always_inline)) {
    uint4* row = reinterpret_cast<uint4*>(slot + k_row * KROWB);
#pragma unroll
    for (int i = 0; i < 4; ++i) row[(k_ch + i) ^ (k_row & 15)] = st.k[i];
    // V: 4 keys x 8 d -> 8 granules (4 keys of one d) of this half's V^T tile
    char* vt = slot + K_BYTES + (v_quad >> 3) * VT_BYTES;
    const int qd = v_quad & 7;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int d = 8 * v_oct + e;
      const uint32_t a0 = reinterpret_cast<const uint32_t*>(&st.v[0])[e >> 1];
      const uint32_t a1 = reinterpret_cast<const uint32_t*>(&st.v[1])[e >> 1];
      const uint32_t a2 = reinterpret_cast<const uint32_t*>(&st.v[2])[e >> 1];
      const uint32_t a3 = reinterpret_cast<const uint32_t*>(&st.v[3])[e >> 1];
      uint32_t w0, w1;
      if ((e & 1) == 0) {
        w0 = (a0 & 0xffffu) | (a1 << 16);
        w1 = (a2 & 0xffffu) | (a3 << 16);
      } else {
        w0 = (a0 >> 16) | (a1 & 0xffff0000u);
        w1 = (a2 >> 16) | (a3 & 0xffff0000u);
      }
      *reinterpret_cast<uint2*>(vt + d * VROWB + ((qd ^ ((d >> 4) & 7)) * 8)) = make_uint2(w0, w1);
    }
  };

  // ---- prologue: Q rows and mask rows first, then the first blocks ----
  constexpr int ROWS_WG = 4 * QTW * 16;
  constexpr int Q_PER_THREAD = ROWS_WG * QROW_CHUNKS / 256;  // 4 * QTW
  const int row0 = qc * ROWS_WG;
  uint4 qv[Q_PER_THREAD];
#pragma unroll
  for (int u = 0; u < Q_PER_THREAD; ++u) {
    const int idx = tid + 256 * u;
    const int rr = idx / QROW_CHUNKS, ch = idx % QROW_CHUNKS;
    const int r = min(row0 + rr, a.QR - 1);
    const int node = r / a.G, gq = r % a.G;
    qv[u] = ldg16(a.q + ((static_cast<int64_t>(b) * a.T + node) * a.Hq + kvh * a.G + gq) * D + ch * 8);
  }
  const int nmask = a.T * a.W;
  uint64_t mv[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) mv[u] = (tid + 256 * u < nmask) ? a.mask[tid + 256 * u] : 0ull;
  Stage s0, s1;
  if (nblk > 0) gload(s0, 0);
  if (nblk > 1) gload(s1, 1);
  uint4* sq = reinterpret_cast<uint4*>(smem + a.lds_q);
#pragma unroll
  for (int u = 0; u < Q_PER_THREAD; ++u) {
    const int idx = tid + 256 * u;
    const int rr = idx / QROW_CHUNKS, ch = idx % QROW_CHUNKS;
    sq[rr * QROW_CHUNKS + (ch ^ (rr & 15))] = (row0 + rr < a.QR) ? qv[u] : make_uint4(0, 0, 0, 0);
  }
  uint64_t* smask = reinterpret_cast<uint64_t*>(smem + a.lds_mask);
#pragma unroll
  for (int u = 0; u < 4; ++u)
    if (tid + 256 * u < nmask) smask[tid + 256 * u] = mv[u];

  // this wave's query tiles: wave, wave + 4, ...
  int qnode[QTW];
#pragma unroll
  for (int t = 0; t < QTW; ++t) {
    const int r = row0 + (wave + 4 * t) * 16 + l16;
    qnode[t] = r < a.QR ? r / a.G : 0;
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
  char* ring = smem + a.lds_ring;

  // one 32-key half of a staged block
  auto compute_half = [&](const char* slot, int h, int kb) __attribute__((always_inline)) {
    bf16x8 kf[2][4];
#pragma unroll
    for (int st = 0; st < 2; ++st) {
      const uint4* row = reinterpret_cast<const uint4*>(slot + (h * HALF + st * 16 + l16) * KROWB);
#pragma unroll
      for (int s = 0; s < 4; ++s) kf[st][s] = as_bf16x8(row[(grp * 4 + s) ^ l16]);
    }
    f32x4 sc[2][QTW];
#pragma unroll
    for (int t = 0; t < QTW; ++t) {
      const uint4* qrow = sq + ((wave + 4 * t) * 16 + l16) * QROW_CHUNKS;
      f32x4 acc0 = f32x4{0.f, 0.f, 0.f, 0.f};
      f32x4 acc1 = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const bf16x8 qf = as_bf16x8(qrow[(grp * 4 + s) ^ l16]);
        acc0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[0][s], qf, acc0, 0, 0, 0);
        acc1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[1][s], qf, acc1, 0, 0, 0);
      }
      sc[0][t] = acc0 * a.scale_log2;
      sc[1][t] = acc1 * a.scale_log2;
    }
    if (kb + HALF > ctx || kb + HALF > k_end) {  // the tree region or the split's end
#pragma unroll
      for (int st = 0; st < 2; ++st) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int key = kb + st * 16 + 4 * grp + e;
          const int jj = key - ctx;
#pragma unroll
          for (int t = 0; t < QTW; ++t) {
            bool vis = key < k_end;
            if (vis && jj >= 0) vis = (smask[qnode[t] * a.W + (jj >> 6)] >> (jj & 63)) & 1ull;
            if (!vis) sc[st][t][e] = -INFINITY;
          }
        }
      }
    }
    uint4 pb[QTW];
#pragma unroll
    for (int t = 0; t < QTW; ++t) {
      float bm = fmaxf(fmaxf(fmaxf(sc[0][t][0], sc[0][t][1]), fmaxf(sc[0][t][2], sc[0][t][3])),
                       fmaxf(fmaxf(sc[1][t][0], sc[1][t][1]), fmaxf(sc[1][t][2], sc[1][t][3])));
      bm = wave_max_16_32(bm);
      const float mnew = fmaxf(m_run[t], bm);
      const float muse = (mnew == -INFINITY) ? 0.f : mnew;
      const float alpha = __builtin_amdgcn_exp2f(m_run[t] - muse);
      m_run[t] = mnew;
      float p[8];
#pragma unroll
      for (int st = 0; st < 2; ++st)
#pragma unroll
        for (int e = 0; e < 4; ++e) p[st * 4 + e] = __builtin_amdgcn_exp2f(sc[st][t][e] - muse);
      l_run[t] = l_run[t] * alpha + ((p[0] + p[1]) + (p[2] + p[3])) + ((p[4] + p[5]) + (p[6] + p[7]));
      pb[t] = make_uint4(pack_bf16(p[0], p[1]), pack_bf16(p[2], p[3]), pack_bf16(p[4], p[5]),
                         pack_bf16(p[6], p[7]));
      if (__builtin_amdgcn_ballot_w64(alpha != 1.0f)) {  // some query's max moved
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) o[t][dt] *= alpha;
      }
    }
    const char* vt = slot + K_BYTES + h * VT_BYTES;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
      const char* rowp = vt + (dt * 16 + l16) * VROWB;
      const uint2 lo = *reinterpret_cast<const uint2*>(rowp + ((grp ^ (dt & 7)) * 8));
      const uint2 hi = *reinterpret_cast<const uint2*>(rowp + (((grp + 4) ^ (dt & 7)) * 8));
      const bf16x8 va = as_bf16x8(make_uint4(lo.x, lo.y, hi.x, hi.y));
#pragma unroll
      for (int t = 0; t < QTW; ++t)
        o[t][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, as_bf16x8(pb[t]), o[t][dt], 0, 0, 0);
    }
  };

  // Pipeline: block 0 is staged before the loop; step i computes block i from
  // its slot while staging block i+1 into the other slot and refilling that
  // register buffer with block i+1+PREFETCH; one barrier per step.  A slot is
  // rewritten only after the barrier that follows its last reader.
  if (nblk > 0) {
    lds_put(s0, ring);
    if (PREFETCH < nblk) gload(s0, PREFETCH);
  }
  __syncthreads();
  auto step = [&](int blk, Stage& next, int si_cur, int si_next) __attribute__((always_inline)) {
    const char* cur = ring + si_cur * SLOT_BYTES;
    const int kb = k_begin + blk * KB;
    compute_half(cur, 0, kb);
    if (kb + HALF < k_end) compute_half(cur, 1, kb + HALF);
    if (blk + 1 < nblk) {
      lds_put(next, ring + si_next * SLOT_BYTES);
      if (blk + 1 + PREFETCH < nblk) gload(next, blk + 1 + PREFETCH);
    }
    __syncthreads();
  };
  int blk = 0;
  for (; blk + 2 <= nblk; blk += 2) {
    step(blk, s1, 0, 1);
    step(blk + 1, s0, 1, 0);
  }
  if (blk < nblk) step(blk, s1, 0, 1);

  // full per-query sums (each lane group holds a quarter of the keys)
#pragma unroll
  for (int t = 0; t < QTW; ++t) {
    l_run[t] += __shfl_xor(l_run[t], 16, 64);
    l_run[t] += __shfl_xor(l_run[t], 32, 64);
  }

  // ---- one split: the output; several: this split's partial ----
  const int BH = a.B * a.Hkv;
#pragma unroll
  for (int t = 0; t < QTW; ++t) {
    const int r = row0 + (wave + 4 * t) * 16 + l16;
    if (r >= a.QR) continue;
    if (a.NS == 1) {
      const float inv = 1.0f / l_run[t];
      const int node = r / a.G, gq = r % a.G;
      uint16_t* op = a.out + ((static_cast<int64_t>(b) * a.T + node) * a.Hq + kvh * a.G + gq) * D;
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) {
        const f32x4 v = o[t][dt] * inv;
        *reinterpret_cast<uint2*>(op + dt * 16 + 4 * grp) =
            make_uint2(pack_bf16(v[0], v[1]), pack_bf16(v[2], v[3]));
      }
    } else {
      const int64_t prow = (static_cast<int64_t>(split) * BH + bh) * a.QRpad + r;
      float* po = a.part_o + prow * D;
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) *reinterpret_cast<f32x4*>(po + dt * 16 + 4 * grp) = o[t][dt];
      if (grp == 0) *reinterpret_cast<float2*>(a.part_ml + prow * 2) = make_float2(m_run[t], l_run[t]);
    }
  }
}

// Merge the NS split partials of every query row, in split order (NS <= 64).
// One wave per row, 2 consecutive d per lane; every split's (max, sum) and
// output values are requested before any arithmetic (one round trip).
__global__ __launch_bounds__(256) void merge_splits(AttnArgs a) {
  const int lane = threadIdx.x & 63;
  const int BH = a.B * a.Hkv;
  const int64_t gr = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (gr >= static_cast<int64_t>(BH) * a.QR) return;
  const int bh = static_cast<int>(gr / a.QR);
  const int r = static_cast<int>(gr % a.QR);
  const int64_t stride = static_cast<int64_t>(BH) * a.QRpad;  // rows between splits
  const int64_t row = static_cast<int64_t>(bh) * a.QRpad + r;
  const int ns = a.NS;
  float2 ml = make_float2(-INFINITY, 0.f);
  if (lane < ns) ml = *reinterpret_cast<const float2*>(a.part_ml + (lane * stride + row) * 2);
  float2 ov[16];
#pragma unroll
  for (int u = 0; u < 16; ++u)
    ov[u] = (u < ns) ? *reinterpret_cast<const float2*>(a.part_o + (u * stride + row) * D + 2 * lane)
                     : make_float2(0.f, 0.f);
  float M = ml.x;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) M = fmaxf(M, __shfl_xor(M, off, 64));
  const float muse = (M == -INFINITY) ? 0.f : M;
  const float w = __builtin_amdgcn_exp2f(ml.x - muse);  // lane s: weight of split s
  float L = ml.y * w;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) L += __shfl_xor(L, off, 64);
  float o0 = 0.f, o1 = 0.f;
#pragma unroll
  for (int u = 0; u < 16; ++u) {
    const float wu = __shfl(w, u, 64);
    o0 = fmaf(ov[u].x, wu, o0);
    o1 = fmaf(ov[u].y, wu, o1);
  }
  for (int s = 16; s < ns; ++s) {
    const float2 v = *reinterpret_cast<const float2*>(a.part_o + (s * stride + row) * D + 2 * lane);
    const float wu = __shfl(w, s, 64);
    o0 = fmaf(v.x, wu, o0);
    o1 = fmaf(v.y, wu, o1);
  }
  const float inv = 1.0f / L;
  const int b = bh / a.Hkv, kvh = bh % a.Hkv;
  const int node = r / a.G, gq = r % a.G;
  uint16_t* op = a.out + ((static_cast<int64_t>(b) * a.T + node) * a.Hq + kvh * a.G + gq) * D + 2 * lane;
  *reinterpret_cast<uint32_t*>(op) = pack_bf16(o0 * inv, o1 * inv);
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
  int G, QR, NQT, QTW, QC, QRpad, NS, chunk;
  size_t ws_bytes, off_ml;
  int lds_bytes, lds_mask, lds_q, lds_ring;
};

int env_int(const char* name, int dflt) {
  const char* s = std::getenv(name);
  return s ? std::atoi(s) : dflt;
}

int cu_count() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (!cached[dev]) {
    hipDeviceProp_t prop;
    cached[dev] = (hipGetDeviceProperties(&prop, dev) == hipSuccess && prop.multiProcessorCount > 0)
                      ? prop.multiProcessorCount
                      : 256;
  }
  return cached[dev];
}

const void* kernel_for(int qtw) {
  switch (qtw) {
    case 1: return reinterpret_cast<const void*>(&tree_attn_bf16<1>);
    case 2: return reinterpret_cast<const void*>(&tree_attn_bf16<2>);
    case 3: return reinterpret_cast<const void*>(&tree_attn_bf16<3>);
    default: return reinterpret_cast<const void*>(&tree_attn_bf16<4>);
  }
}

// workgroups of this configuration one CU runs at once (1 if unknown)
int occupancy(int qtw, int lds) {
  static int cache[5][8] = {{0}};
  const int bucket = lds / (20 * 1024);
  if (bucket < 8 && cache[qtw][bucket]) return cache[qtw][bucket];
  int n = 0;
  if (lds > 64 * 1024)
    (void)hipFuncSetAttribute(kernel_for(qtw), hipFuncAttributeMaxDynamicSharedMemorySize, lds);
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, kernel_for(qtw), 256, lds) != hipSuccess || n < 1) {
    (void)hipGetLastError();
    n = 1;
  }
  if (bucket < 8) cache[qtw][bucket] = n;
  return n;
}

Plan make_plan(int B, int Hq, int Hkv, int ctx_max, int T, int W) {
  Plan p{};
  p.G = Hq / Hkv;
  p.QR = T * p.G;
  p.NQT = (p.QR + 15) / 16;
  p.QTW = (p.NQT + 3) / 4;
  if (p.QTW > 4) p.QTW = 4;
  p.QC = (p.NQT + 4 * p.QTW - 1) / (4 * p.QTW);
  p.QRpad = p.NQT * 16;
  p.lds_mask = 0;
  p.lds_q = static_cast<int>(round_up(static_cast<size_t>(T) * W * 8, 16));
  p.lds_ring = p.lds_q + 4 * p.QTW * 16 * D * 2;
  p.lds_bytes = p.lds_ring + PREFETCH * SLOT_BYTES;
  const int Smax = ctx_max + T;
  const int base = B * Hkv * p.QC;
  int ns = env_int("MEDUSA_ATTN_SPLITS", 0);
  if (ns <= 0) {
    // pick the split count minimising rounds x (fixed cost + keys per split),
    // counting the workgroups all CUs hold at once
    const int slots = cu_count() * occupancy(p.QTW, p.lds_bytes);
    const double fixed_keys = 96.0;  // per-workgroup latency, in key-times
    double best = 1e300;
    ns = 1;
    const int max_ns = (Smax + KB - 1) / KB;  // >= one staged block per split
    for (int n = 1; n <= max_ns && n <= 64; ++n) {
      const int rounds = (base * n + slots - 1) / slots;
      const double t = rounds * (fixed_keys + std::ceil(static_cast<double>(Smax) / n));
      if (t < best * 0.999) {
        best = t;
        ns = n;
      }
    }
  }
  if (ns > 64) ns = 64;  // the merge keeps one split per lane
  int chunk = (Smax + ns - 1) / ns;
  chunk = (chunk + KB - 1) / KB * KB;
  p.chunk = chunk;
  p.NS = (Smax + chunk - 1) / chunk;
  if (p.NS < 1) p.NS = 1;
  if (p.NS > 1) {
    const size_t rows = static_cast<size_t>(p.NS) * B * Hkv * p.QRpad;
    p.off_ml = round_up(rows * D * 4, 256);
    p.ws_bytes = p.off_ml + round_up(rows * 2 * 4, 256);
  }
  return p;
}

template <int QTW>
int launch_cfg(const AttnArgs& a, int grid, int lds, hipStream_t s) {
  if (lds > 64 * 1024) {
    // above 64 KiB the dynamic LDS size must be allowed explicitly
    static int allowed = 0;
    if (lds > allowed) {
      hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&tree_attn_bf16<QTW>),
                                         hipFuncAttributeMaxDynamicSharedMemorySize, lds);
      if (e != hipSuccess) {
        (void)hipGetLastError();
        set_error("cannot allow %d bytes of dynamic LDS for tree attention: %s", lds,
                  hipGetErrorString(e));
        return MEDUSA_EUNSUPPORTED;
      }
      allowed = lds;
    }
  }
  hipLaunchKernelGGL((tree_attn_bf16<QTW>), dim3(grid), dim3(256), lds, s, a);
  return check_launch("tree attention (bf16)");
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
  if (p.NS > 1) {
    char* w = static_cast<char*>(ws);
    a.part_o = reinterpret_cast<float*>(w);
    a.part_ml = reinterpret_cast<float*>(w + p.off_ml);
  }
  a.lds_mask = p.lds_mask;
  a.lds_q = p.lds_q;
  a.lds_ring = p.lds_ring;
  const int grid = 8 * a.per_xcd;
  switch (p.QTW) {
    case 1: rc = launch_cfg<1>(a, grid, p.lds_bytes, stream); break;
    case 2: rc = launch_cfg<2>(a, grid, p.lds_bytes, stream); break;
    case 3: rc = launch_cfg<3>(a, grid, p.lds_bytes, stream); break;
    default: rc = launch_cfg<4>(a, grid, p.lds_bytes, stream); break;
  }
  if (rc || p.NS == 1) return rc;
  const int64_t rows = static_cast<int64_t>(B) * Hkv * p.QR;
  hipLaunchKernelGGL(merge_splits, dim3(static_cast<unsigned>((rows + 3) / 4)), dim3(256), 0, stream, a);
  return check_launch("tree attention split merge");
}
