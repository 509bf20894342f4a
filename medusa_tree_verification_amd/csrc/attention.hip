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
//   Work item: one workgroup per (sequence b, K/V head, query chunk, key
//   split).  All T*G query rows of a K/V head (G = Hq/Hkv; row r = node r/G,
//   query head r%G) go through the same pass over its keys, so every K/V byte
//   of the split is read from HBM once.  The workgroup has 12 waves in two
//   roles that meet at one barrier per 64-key block:
//   - 4 staging waves stream the split's K/V through buffer loads into
//     registers, NREG blocks ahead of use, and write each block into one of
//     three LDS slots: K rows of 256 bytes with their 16-byte chunks
//     XOR-swizzled by the row; V transposed (rows = d, 128 bytes) with the 8
//     keys a lane feeds to one P.V MFMA k-step in one 16-byte granule,
//     granules XOR-swizzled by a function of d.  Memory stalls of these
//     waves do not hold up the arithmetic.
//   LDS banks (gfx950, measured with the bank-conflict counter): a 16-byte
//   read is served in 4 passes of 16 lanes over 64 four-byte banks, lanes
//   {0-3, 12-15, 20-27} (and the same +32) sharing a pass, the others the
//   other; a 16-byte write in 8 passes of 8 consecutive lanes over 32 banks.
//   Both swizzles make every read and write of the kernel conflict-free
//   under that rule.
//   - 8 compute waves: wave w takes query tiles (16 rows) w%4, w%4 + 4, ...
//     and the 32-key half w/4 of every block, keeping its own online-softmax
//     state; the two halves are merged through LDS at the end (fixed order).
//   Scores: S^T = K Q^T on v_mfma_f32_16x16x32_bf16 (K rows as the A
//   operand, Q rows as B -- in registers for one tile per wave, else staged
//   in LDS; the d order is permuted the same way in both).  Lane l then holds
//   query l%16 and 8 keys of the half, so every lane's softmax state (max,
//   sum, rescale) is its own query's; the max over the lane rows uses the
//   gfx950 permlane swaps (no LDS round trip).
//   Values: O^T += V^T P^T; P^T comes straight from the score registers
//   (packed to bf16) because the key order of the staged V^T granules is
//   chosen to match them.
//   Mask: context keys are always visible; tree key j is visible to node i
//   iff bit j of node i's ancestor bitmask is set (rows staged in LDS); only
//   halves that reach past the context or the split evaluate it.
//   exp2 with log2(e) folded into the scale; fp32 scores, sums and outputs.
//   Splits: each workgroup writes its partial (its output normalised by its
//   own sum, in bf16, and the max and sum in fp32); a second kernel merges
//   the splits of every row in split order (fixed order: deterministic).  Workgroups are numbered so that all splits of one
//   (b, K/V head) land on the same XCD (dispatch assigns workgroup i to XCD
//   i % 8), which keeps their partials in one L2.
#include <cmath>
#include <cstdlib>
#include <mutex>
#include <type_traits>

#include "internal.h"

using namespace medusa;
using namespace medusa::dev;

namespace {

constexpr int D = 128;
constexpr int KB = 64;                      // keys per block (one wave's unit of work)
constexpr int GROWB = D * 2;                // bytes per K/V row in HBM
constexpr int KROWB = GROWB;                // K (and staged Q) row in LDS: 256
constexpr int K_TILE = KB * KROWB;          // 16384
constexpr int VROWB = KB * 2;               // V^T row (one d, 64 keys) in LDS: 128
constexpr int V_TILE = D * VROWB;           // 16384
constexpr int BLK_BYTES = K_TILE + V_TILE;  // 32768

// K / staged Q tile: 16-byte chunk c of row r lives at r * 256 + 16 * (c ^ (r & 15)).
__device__ __forceinline__ int kq_off(int r, int c) { return r * KROWB + 16 * (c ^ (r & 15)); }
// V^T tile: granule G (8 keys) of row d lives at d * 128 + 16 * (G ^ vswz(d)),
// vswz(d) = rot3((d >> 3) & 7) ^ 4 * (bit 1 of d ^ bit 2 of d), rot3 rotating
// 3 bits left by one.
__device__ __forceinline__ constexpr int rot3(int x) { return ((x << 1) | (x >> 2)) & 7; }
constexpr int NSLOT = 3;                    // LDS slots (blocks staged at once)
constexpr int NREG = 2;                     // blocks in flight in staging registers
constexpr int MERGE_BYTES = 8 * 64 * 16 + 64 * 8;  // one wave-tile's O, max and sum
constexpr int MAX_SPLITS = 64;
// exponents may exceed the reference by up to this much (log2 units), so
// unnormalised probabilities stay <= 256
constexpr float RESCALE_SLACK = 8.0f;
constexpr int LDS_MAX = 160 * 1024;         // LDS of one CU
constexpr int RSRC_WORD3 = 0x00020000;      // raw buffer, 32-bit data format
constexpr float LOG2E = 1.4426950408889634f;

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

struct AttnArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const int32_t* ctx;
  const uint64_t* mask;  // [T][W]
  int W, B, T, Hq, Hkv, G, S_cap;
  int L;                                       // layers in this call
  int64_t q_lstride, kv_lstride, out_lstride;  // elements between layers
  int QR, QRpad, QC, NS, chunk;
  int tasks, per_xcd;
  float scale_log2;
  uint16_t* out;
  uint16_t* part_o;  // [NS][B*Hkv][QRpad][D] bf16, normalised (O / sum)
  float* part_ml;    // [B*Hkv][QRpad][NS][2] fp32 (max, sum): a row's splits side by side
  int lds_mask, lds_q, lds_ring;  // dynamic LDS layout (byte offsets)
};

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

__device__ __forceinline__ uint32_t word(const uint4& v, int i) {
  return i == 0 ? v.x : i == 1 ? v.y : i == 2 ? v.z : v.w;
}

// max / sum over the 4 lane rows (lanes l%16 + 16r) of a wave
__device__ __forceinline__ float rows_max(float x) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
  r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float rows_sum(float x) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

template <int QTW>
__global__ __launch_bounds__(768) void tree_attn_bf16(AttnArgs a) {
  constexpr bool QREG = QTW == 1;  // Q fragments in registers, else in LDS
  constexpr int ROWS_WG = 4 * QTW * 16;
  extern __shared__ __attribute__((aligned(16))) char smem[];
  const int id = blockIdx.x;
  const int task = (id & 7) * a.per_xcd + (id >> 3);
  if (task >= a.tasks) return;  // whole workgroup leaves before any barrier
  const int split = task % a.NS;
  const int rest = task / a.NS;  // = lbh * QC + qc
  const int qc = rest % a.QC;
  const int lbh = rest / a.QC;   // = layer * B * Hkv + bh
  const int bh = lbh % (a.B * a.Hkv);
  const int layer = lbh / (a.B * a.Hkv);
  const int b = bh / a.Hkv;
  const int kvh = bh % a.Hkv;
  const uint16_t* qL = a.q + layer * a.q_lstride;
  uint16_t* outL = a.out + layer * a.out_lstride;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const bool computes = wave < 8;  // waves 0-7 compute, waves 8-11 stage K/V
  const int qw = wave & 3;         // query-tile lane of a compute wave
  const int half = (wave >> 2) & 1;  // the 32-key half of every block it computes
  const int l16 = lane & 15;
  const int grp = lane >> 4;

  const int k_begin = split * a.chunk;
  // the sequence's bounds; each role reads ctx_len only after issuing its
  // first loads, which do not depend on it
  int ctx = 0, k_end = 0, nblk = 0;
  auto read_ctx = [&]() __attribute__((always_inline)) {
    ctx = a.ctx[b];
    ctx = ctx < 0 ? 0 : (ctx > a.S_cap - a.T ? a.S_cap - a.T : ctx);
    const int S = ctx + a.T;
    k_end = (split == a.NS - 1) ? S : min(S, k_begin + a.chunk);
    nblk = k_end > k_begin ? (k_end - k_begin + KB - 1) / KB : 0;
  };

  // ---- staging roles: waves 8-9 load K rows, waves 10-11 V ----
  const bool k_role = wave < 10;
  const int rt = tid - (k_role ? 512 : 640);  // 0..127 within the role
  const uint16_t* gbase =
      (k_role ? a.k : a.v) + layer * a.kv_lstride + static_cast<int64_t>(bh) * a.S_cap * D;
  int goff[8];   // byte offsets of this thread's 8 loads within a block
  int krow0;     // key of load 0 within its block (load i: krow0 + kstep * i, V: see below)
  int lds_w;     // this thread's LDS store offset within a slot (K: even loads)
  int lds_w_odd; // K: odd loads (their row is 8 further, which flips bit 3 of the swizzle)
  if (k_role) {
    // load i: key row rt/16 + 8i, 16-byte chunk rt%16
    const int r = rt >> 4, c = rt & 15;
    const int base = r * GROWB + c * 16;
#pragma unroll
    for (int i = 0; i < 8; ++i) goff[i] = base + 8 * i * GROWB;
    krow0 = r;
    lds_w = kq_off(r, c);
    lds_w_odd = kq_off(r + 8, c) - 8 * KROWB;
  } else {
    // d-octet o of the 8 keys {4g..4g+3, 16+4g..16+4g+3} of half h: row
    // d = 8o + dd of V^T, granule 4h + g
    const int o = rt & 15, g = (rt >> 4) & 3, h = rt >> 6;
    const int base = (h * 32 + 4 * g) * GROWB + o * 16;
#pragma unroll
    for (int i = 0; i < 8; ++i) goff[i] = base + (i < 4 ? i : 12 + i) * GROWB;
    krow0 = h * 32 + 4 * g;
    lds_w = K_TILE + 8 * o * VROWB + 16 * ((h * 4 + g) ^ rot3(o & 7));
    lds_w_odd = 0;
  }
  // A block's loads go through a buffer resource that ends where the split
  // can end at most (the next split's start, or the cache's end), a bound
  // that does not depend on the context length: the first loads leave before
  // ctx_len has arrived.  Rows of keys >= k_end (unused cache slots) are
  // zeroed before they reach LDS, so nothing past the sequence can enter the
  // products; keys past the bound read as zeros.
  const int spec_end = (split == a.NS - 1) ? a.S_cap : min(a.S_cap, k_begin + a.chunk);
  auto gload = [&](uint4 (&x)[8], int blk) __attribute__((always_inline)) {
    const int kb = k_begin + blk * KB;
    const int nrec = (spec_end - kb) * GROWB;
    const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(gbase + static_cast<int64_t>(kb) * D), 0, nrec > 0 ? nrec : 0,
        RSRC_WORD3);
#pragma unroll
    for (int i = 0; i < 8; ++i) x[i] = bload16(r, goff[i]);
  };
  auto lds_put = [&](const uint4 (&xin)[8], char* slot, int blk) __attribute__((always_inline)) {
    uint4 x[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) x[i] = xin[i];
    const int lim = k_end - (k_begin + blk * KB);  // keys of this block below k_end
    if (lim < KB) {  // the block reaches past the sequence (or the split)
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int key = krow0 + (k_role ? 8 * i : (i < 4 ? i : 12 + i));
        if (key >= lim) x[i] = make_uint4(0, 0, 0, 0);
      }
    }
    if (k_role) {
#pragma unroll
      for (int i = 0; i < 8; ++i)
        *reinterpret_cast<uint4*>(slot + 8 * i * KROWB + ((i & 1) ? lds_w_odd : lds_w)) = x[i];
    } else {
      // row d = 8o + dd of V^T: element dd of each of the 8 keys, in k-slot order
#pragma unroll
      for (int dd = 0; dd < 8; ++dd) {
        const uint32_t sel = (dd & 1) ? 0x07060302u : 0x05040100u;
        uint4 w;
        w.x = __builtin_amdgcn_perm(word(x[1], dd >> 1), word(x[0], dd >> 1), sel);
        w.y = __builtin_amdgcn_perm(word(x[3], dd >> 1), word(x[2], dd >> 1), sel);
        w.z = __builtin_amdgcn_perm(word(x[5], dd >> 1), word(x[4], dd >> 1), sel);
        w.w = __builtin_amdgcn_perm(word(x[7], dd >> 1), word(x[6], dd >> 1), sel);
        // vswz(8o + dd) = rot3(o & 7) ^ 4 * (bit 1 of dd ^ bit 2 of dd)
        *reinterpret_cast<uint4*>(slot + (lds_w ^ ((((dd >> 1) ^ (dd >> 2)) & 1) ? 64 : 0)) + dd * VROWB) = w;
      }
    }
  };

  char* ring = smem + a.lds_ring;

  // ---- staging waves: stream K/V into the LDS ring, one block per barrier ----
  // Every global load here is issued unconditionally (a block past the
  // split's end reads zeros through its empty buffer resource), and this
  // path never joins the compute waves' code, so the loads in flight are the
  // same on every path and each wait covers exactly the block it needs.
  // Pipeline: while the compute waves work on block i (and the second-half
  // waves finish block i-1) from their LDS slots, these waves write block
  // i+1 (from registers) into the third slot, the one block i-2 held, and
  // refill those registers with block i+1+NREG.  A slot is rewritten only
  // after the barrier that follows its last reader.  Both roles pass the
  // same number of barriers.
  if (!computes) {
    uint4 R[NREG][8];  // blocks loaded but not yet in LDS
#pragma unroll
    for (int j = 0; j < NREG; ++j) {
      gload(R[j], j);
      __builtin_amdgcn_sched_barrier(0);  // keep the blocks' loads in order
    }
    read_ctx();
    if (nblk > 0) lds_put(R[0], ring, 0);
    gload(R[0], NREG);
    __syncthreads();
    int ws = 1;  // slot of block blk + j + 1
    for (int blk = 0; blk < nblk; blk += NREG) {
#pragma unroll
      for (int j = 0; j < NREG; ++j) {
        if (blk + j + 1 < nblk) lds_put(R[(j + 1) % NREG], ring + ws * BLK_BYTES, blk + j + 1);
        ws = ws == NSLOT - 1 ? 0 : ws + 1;
        gload(R[(j + 1) % NREG], blk + j + 1 + NREG);
        __syncthreads();
      }
    }
    __syncthreads();  // the second-half waves' last P.V
    __syncthreads();  // the compute waves' merge of the two key halves
    return;
  }

  // ---- compute waves ----
  // Q and the mask rows (the staging waves' only
  // global loads are K/V)
  const int row0 = qc * ROWS_WG;
  auto q_ptr = [&](int r, int ch) __attribute__((always_inline)) {
    const int node = r / a.G, gq = r % a.G;
    return qL + ((static_cast<int64_t>(b) * a.T + node) * a.Hq + kvh * a.G + gq) * D + ch * 8;
  };
  bf16x8 qf[QREG ? 4 : 1];
  uint64_t* smask = reinterpret_cast<uint64_t*>(smem + a.lds_mask);
  {
    if constexpr (QREG) {
      const int r = min(row0 + qw * 16 + l16, a.QR - 1);
#pragma unroll
      for (int s = 0; s < 4; ++s) qf[s] = as_bf16x8(ldg16(q_ptr(r, 4 * s + grp)));
    } else {
      constexpr int Q_PER_THREAD = ROWS_WG * 16 / 512;
#pragma unroll
      for (int u = 0; u < Q_PER_THREAD; ++u) {
        const int idx = tid + 512 * u;
        const uint4 v = ldg16(q_ptr(min(row0 + idx / 16, a.QR - 1), idx % 16));
        *reinterpret_cast<uint4*>(smem + a.lds_q + kq_off(idx / 16, idx % 16)) =
            (row0 + idx / 16 < a.QR) ? v : make_uint4(0, 0, 0, 0);
      }
    }
    const int nmask = a.T * a.W;  // <= 1024
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const uint64_t mv = a.mask[min(tid + 512 * u, nmask - 1)];
      if (tid + 512 * u < nmask) smask[tid + 512 * u] = mv;
    }
  }
  __builtin_amdgcn_sched_barrier(0);
  read_ctx();
  const uint32_t* smask32 = reinterpret_cast<const uint32_t*>(smask);

  // compute-wave state: this wave's query tiles qw, qw + 4, ...
  int qnode[QTW];
#pragma unroll
  for (int t = 0; t < QTW; ++t) {
    const int r = row0 + (qw + 4 * t) * 16 + l16;
    qnode[t] = r < a.QR ? r / a.G : 0;
  }
  f32x4 o[QTW][8];
  // per query: m_run the largest scaled score seen when the reference last
  // moved (-inf before any visible key), mu the reference the exponents use
  // (m_run, or 0 while m_run is -inf), l_run the sum of exp2(s - mu) and o
  // the matching weighted sum of values
  float m_run[QTW], mu[QTW], l_run[QTW];
#pragma unroll
  for (int t = 0; t < QTW; ++t) {
    m_run[t] = -INFINITY;
    mu[t] = 0.f;
    l_run[t] = 0.f;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) o[t][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  // k-step s feeds lane group grp the 16-byte d-chunk 4s + grp of its K and
  // Q rows (a permutation of d shared by both operands); chunk 4s + grp of
  // row r (r % 16 = l16) sits at 16 * ((4s + grp) ^ l16) = kx0 ^ 64s
  const int kx0 = 16 * (grp ^ l16);
  const char* sq = smem + a.lds_q + l16 * KROWB;
  // V^T: row dt*16 + l16, granule 4*half + grp at
  // (vbase ^ 16 * rot3(2dt & 7)) + dt * 16 * VROWB
  const int vbase = K_TILE + l16 * VROWB +
                    16 * ((4 * half + grp) ^ rot3(l16 >> 3) ^ (4 * (((l16 >> 1) ^ (l16 >> 2)) & 1)));

  // scores and probabilities of this wave's 32-key half of a 64-key block
  // (keys kh .. kh+31), packed as the P.V operand
  auto qk_softmax = [&](const char* blk, int kh, uint4 (&pb)[QTW]) __attribute__((always_inline)) {
    f32x4 sc[QTW][2];
    const char* kr = blk + (half * 32 + l16) * KROWB;
#pragma unroll
    for (int st = 0; st < 2; ++st) {
      bf16x8 kf[4];
#pragma unroll
      for (int s = 0; s < 4; ++s)
        kf[s] = as_bf16x8(*reinterpret_cast<const uint4*>(kr + st * 16 * KROWB + (kx0 ^ (64 * s))));
#pragma unroll
      for (int t = 0; t < QTW; ++t) {
        f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          bf16x8 q;
          if constexpr (QREG) q = qf[s];
          else q = as_bf16x8(*reinterpret_cast<const uint4*>(sq + (qw + 4 * t) * 16 * KROWB + (kx0 ^ (64 * s))));
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[s], q, acc, 0, 0, 0);
        }
        sc[t][st] = acc;
      }
    }
    if (kh + 32 > ctx || kh + 32 > k_end) {  // the tree region or the split's end
#pragma unroll
      for (int st = 0; st < 2; ++st) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int key = kh + st * 16 + 4 * grp + e;
          const int jj = key - ctx;
          const int jc = jj < 0 ? 0 : (jj >= a.T ? a.T - 1 : jj);
#pragma unroll
          for (int t = 0; t < QTW; ++t) {
            const uint32_t wv = smask32[qnode[t] * 2 * a.W + (jc >> 5)];
            const bool vis = key < k_end && (jj < 0 || ((wv >> (jc & 31)) & 1u));
            if (!vis) sc[t][st][e] = -INFINITY;
          }
        }
      }
    }
    // the reference mu moves only when a score passes it by more than
    // RESCALE_SLACK (log2 units): then, and only then, the block max is
    // reduced over the 4 lane rows and the state rescaled
    float lm[QTW];
    bool over = false;
#pragma unroll
    for (int t = 0; t < QTW; ++t) {
      lm[t] = fmaxf(fmaxf(fmaxf(sc[t][0][0], sc[t][0][1]), fmaxf(sc[t][0][2], sc[t][0][3])),
                    fmaxf(fmaxf(sc[t][1][0], sc[t][1][1]), fmaxf(sc[t][1][2], sc[t][1][3])));
      over |= lm[t] * a.scale_log2 > m_run[t] + RESCALE_SLACK;
    }
    if (__builtin_amdgcn_ballot_w64(over)) {
#pragma unroll
      for (int t = 0; t < QTW; ++t) {
        const float mnew = fmaxf(m_run[t], rows_max(lm[t]) * a.scale_log2);
        const float mu_new = (mnew == -INFINITY) ? 0.f : mnew;
        const float alpha = __builtin_amdgcn_exp2f(m_run[t] - mu_new);  // 0 before any key
        m_run[t] = mnew;
        mu[t] = mu_new;
        l_run[t] *= alpha;
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) o[t][dt] *= alpha;
      }
    }
#pragma unroll
    for (int t = 0; t < QTW; ++t) {
      float p[2][4];
#pragma unroll
      for (int st = 0; st < 2; ++st)
#pragma unroll
        for (int e = 0; e < 4; ++e) p[st][e] = __builtin_amdgcn_exp2f(fmaf(sc[t][st][e], a.scale_log2, -mu[t]));
      l_run[t] += ((p[0][0] + p[0][1]) + (p[0][2] + p[0][3])) + ((p[1][0] + p[1][1]) + (p[1][2] + p[1][3]));
      pb[t] = make_uint4(pack_bf16(p[0][0], p[0][1]), pack_bf16(p[0][2], p[0][3]), pack_bf16(p[1][0], p[1][1]),
                         pack_bf16(p[1][2], p[1][3]));
    }
  };
  // O^T += V^T P^T over the same 32 keys
  auto pv = [&](const char* blk, const uint4 (&pb)[QTW]) __attribute__((always_inline)) {
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
      const bf16x8 va = as_bf16x8(*reinterpret_cast<const uint4*>(
          blk + (vbase ^ (16 * rot3((2 * dt) & 7))) + dt * 16 * VROWB));
#pragma unroll
      for (int t = 0; t < QTW; ++t)
        o[t][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, as_bf16x8(pb[t]), o[t][dt], 0, 0, 0);
    }
  };

  // The first-half waves finish each block in its own interval; the
  // second-half waves run one stage behind on P.V (block i-1's P.V, then
  // block i's scores), so on every SIMD one wave's softmax overlaps the
  // other's MFMAs.  Block i-1 stays in its slot through interval i: three
  // slots, the third being written by the staging waves.
  auto block_loop = [&](auto skew_tag) __attribute__((always_inline)) {
    constexpr bool SKEW = decltype(skew_tag)::value;
    uint4 pb_prev[QTW];
    const char* slot_prev = ring;
    bool have_prev = false;
    int rs = 0;  // slot of block blk + j
    for (int blk = 0; blk < nblk; blk += NREG) {
#pragma unroll
      for (int j = 0; j < NREG; ++j) {
        const char* slot = ring + rs * BLK_BYTES;
        rs = rs == NSLOT - 1 ? 0 : rs + 1;
        const int kh = k_begin + (blk + j) * KB + 32 * half;
        const bool live = blk + j < nblk && kh < k_end;
        if constexpr (!SKEW) {
          if (live) {
            uint4 pb[QTW];
            qk_softmax(slot, kh, pb);
            pv(slot, pb);
          }
        } else {
          if (have_prev) pv(slot_prev, pb_prev);
          have_prev = live;
          if (live) {
            qk_softmax(slot, kh, pb_prev);
            slot_prev = slot;
          }
        }
        __syncthreads();
      }
    }
    if constexpr (SKEW) {
      if (have_prev) pv(slot_prev, pb_prev);
    }
  };
  __syncthreads();
  if (half == 0) block_loop(std::false_type{});
  else block_loop(std::true_type{});
  __syncthreads();  // no wave reads the ring past this point

  // full per-query sums (each lane row holds a quarter of the keys)
#pragma unroll
  for (int t = 0; t < QTW; ++t) l_run[t] = rows_sum(l_run[t]);

  // the second-half waves hand their state to the first-half waves through
  // LDS (Q and the ring are free after the loop's last barrier)
  auto region = [&](int t) __attribute__((always_inline)) {
    return smem + a.lds_q + (qw * QTW + t) * MERGE_BYTES;
  };
  if (half == 1) {
#pragma unroll
    for (int t = 0; t < QTW; ++t) {
      char* r = region(t);
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) reinterpret_cast<f32x4*>(r)[dt * 64 + lane] = o[t][dt];
      reinterpret_cast<float2*>(r + 8 * 64 * 16)[lane] = make_float2(m_run[t], l_run[t]);
    }
  }
  __syncthreads();
  if (half == 1) return;
#pragma unroll
  for (int t = 0; t < QTW; ++t) {
    const char* r = region(t);
    const float2 ml = reinterpret_cast<const float2*>(r + 8 * 64 * 16)[lane];
    const float M = fmaxf(m_run[t], ml.x);
    const float muse = (M == -INFINITY) ? 0.f : M;
    const float a0 = __builtin_amdgcn_exp2f(m_run[t] - muse);
    const float a1 = __builtin_amdgcn_exp2f(ml.x - muse);
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) o[t][dt] = o[t][dt] * a0 + reinterpret_cast<const f32x4*>(r)[dt * 64 + lane] * a1;
    l_run[t] = l_run[t] * a0 + ml.y * a1;
    m_run[t] = M;
  }

  // ---- one split: the output; several: this split's partial ----
  const int BH = a.B * a.Hkv;
#pragma unroll
  for (int t = 0; t < QTW; ++t) {
    const int r = row0 + (qw + 4 * t) * 16 + l16;
    if (r >= a.QR) continue;
    if (a.NS == 1) {
      const float inv = 1.0f / l_run[t];
      const int node = r / a.G, gq = r % a.G;
      uint16_t* op = outL + ((static_cast<int64_t>(b) * a.T + node) * a.Hq + kvh * a.G + gq) * D;
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) {
        const f32x4 v = o[t][dt] * inv;
        *reinterpret_cast<uint2*>(op + dt * 16 + 4 * grp) =
            make_uint2(pack_bf16(v[0], v[1]), pack_bf16(v[2], v[3]));
      }
    } else {
      // the split's output normalised by its own sum (bf16), with its max and
      // sum in fp32; a split that saw no key has sum 0 and writes zeros
      const int64_t prow = (static_cast<int64_t>(split) * a.L * BH + lbh) * a.QRpad + r;
      uint16_t* po = a.part_o + prow * D;
      const float inv = l_run[t] > 0.f ? 1.0f / l_run[t] : 0.f;
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) {
        const f32x4 v = o[t][dt] * inv;
        *reinterpret_cast<uint2*>(po + dt * 16 + 4 * grp) = make_uint2(pack_bf16(v[0], v[1]), pack_bf16(v[2], v[3]));
      }
      if (grp == 0)
        *reinterpret_cast<float2*>(a.part_ml + ((static_cast<int64_t>(lbh) * a.QRpad + r) * a.NS + split) * 2) =
            make_float2(m_run[t], l_run[t]);
    }
  }
}

// Merge the NS split partials of every query row, in split order (NS <= 64):
// out = sum_s w_s l_s O_s / sum_s w_s l_s with w_s = exp2(m_s - max_s m_s) and
// O_s the split's normalised output.  Two rows per wave, 32 lanes per row,
// 4 consecutive d per lane; every split's (max, sum) and output values are
// requested before any arithmetic (one round trip).
__global__ __launch_bounds__(64) void merge_splits(AttnArgs a) {
  const int lane = threadIdx.x & 31;  // lane within the row's half-wave
  const int BH = a.B * a.Hkv;
  const int64_t gr = static_cast<int64_t>(blockIdx.x) * 2 + (threadIdx.x >> 5);
  const bool live = gr < static_cast<int64_t>(a.L) * BH * a.QR;  // both halves reach the shuffles
  const int64_t grc = live ? gr : 0;
  const int lbh = static_cast<int>(grc / a.QR);  // = layer * B * Hkv + bh
  const int bh = lbh % BH, layer = lbh / BH;
  const int r = static_cast<int>(grc % a.QR);
  const int64_t stride = static_cast<int64_t>(a.L) * BH * a.QRpad;  // rows between splits
  const int64_t row = static_cast<int64_t>(lbh) * a.QRpad + r;
  const int ns = a.NS;
  // lane s holds splits s and s + 32
  float2 ml0 = make_float2(-INFINITY, 0.f), ml1 = make_float2(-INFINITY, 0.f);
  if (lane < ns) ml0 = *reinterpret_cast<const float2*>(a.part_ml + (row * ns + lane) * 2);
  if (lane + 32 < ns) ml1 = *reinterpret_cast<const float2*>(a.part_ml + (row * ns + lane + 32) * 2);
  uint2 ov[16];
#pragma unroll
  for (int u = 0; u < 16; ++u)
    ov[u] = (u < ns) ? *reinterpret_cast<const uint2*>(a.part_o + (u * stride + row) * D + 4 * lane)
                     : make_uint2(0, 0);
  float M = fmaxf(ml0.x, ml1.x);
#pragma unroll
  for (int off = 16; off >= 1; off >>= 1) M = fmaxf(M, __shfl_xor(M, off, 32));
  const float muse = (M == -INFINITY) ? 0.f : M;
  const float w0 = __builtin_amdgcn_exp2f(ml0.x - muse) * ml0.y;  // weight of split lane
  const float w1 = __builtin_amdgcn_exp2f(ml1.x - muse) * ml1.y;  // weight of split lane + 32
  float L = w0 + w1;
#pragma unroll
  for (int off = 16; off >= 1; off >>= 1) L += __shfl_xor(L, off, 32);
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
  auto add = [&](uint2 v, float wu) __attribute__((always_inline)) {
    acc[0] = fmaf(bf16_bits_to_f32(v.x & 0xffffu), wu, acc[0]);
    acc[1] = fmaf(bf16_bits_to_f32(v.x >> 16), wu, acc[1]);
    acc[2] = fmaf(bf16_bits_to_f32(v.y & 0xffffu), wu, acc[2]);
    acc[3] = fmaf(bf16_bits_to_f32(v.y >> 16), wu, acc[3]);
  };
#pragma unroll
  for (int u = 0; u < 16; ++u) add(ov[u], __shfl(w0, u, 32));
  for (int s_ = 16; s_ < ns; ++s_) {
    const uint2 v = *reinterpret_cast<const uint2*>(a.part_o + (s_ * stride + row) * D + 4 * lane);
    add(v, s_ < 32 ? __shfl(w0, s_, 32) : __shfl(w1, s_ - 32, 32));
  }
  if (!live) return;
  const float inv = 1.0f / L;
  const int b = bh / a.Hkv, kvh = bh % a.Hkv;
  const int node = r / a.G, gq = r % a.G;
  uint16_t* op = a.out + layer * a.out_lstride +
                 ((static_cast<int64_t>(b) * a.T + node) * a.Hq + kvh * a.G + gq) * D + 4 * lane;
  *reinterpret_cast<uint2*>(op) = make_uint2(pack_bf16(acc[0] * inv, acc[1] * inv), pack_bf16(acc[2] * inv, acc[3] * inv));
}

// The same merge with 16-byte pieces: four rows per wave, 16 lanes per row,
// 8 consecutive d per lane (NS <= 64: lane s holds splits s, s + 16, ...).
__global__ __launch_bounds__(64) void merge_splits16(AttnArgs a) {
  const int lane = threadIdx.x & 15;  // lane within the row's 16
  const int BH = a.B * a.Hkv;
  const int64_t gr = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 4);
  const bool live = gr < static_cast<int64_t>(a.L) * BH * a.QR;  // every row group reaches the shuffles
  const int64_t grc = live ? gr : 0;
  const int lbh = static_cast<int>(grc / a.QR);
  const int bh = lbh % BH, layer = lbh / BH;
  const int r = static_cast<int>(grc % a.QR);
  const int64_t stride = static_cast<int64_t>(a.L) * BH * a.QRpad;
  const int64_t row = static_cast<int64_t>(lbh) * a.QRpad + r;
  const int ns = a.NS;
  float2 ml[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int sp = lane + 16 * q;
    ml[q] = sp < ns ? *reinterpret_cast<const float2*>(a.part_ml + (row * ns + sp) * 2) : make_float2(-INFINITY, 0.f);
  }
  uint4 ov[16];
#pragma unroll
  for (int u = 0; u < 16; ++u)
    ov[u] = (u < ns) ? *reinterpret_cast<const uint4*>(a.part_o + (u * stride + row) * D + 8 * lane)
                     : make_uint4(0, 0, 0, 0);
  float M = fmaxf(fmaxf(ml[0].x, ml[1].x), fmaxf(ml[2].x, ml[3].x));
#pragma unroll
  for (int off = 8; off >= 1; off >>= 1) M = fmaxf(M, __shfl_xor(M, off, 16));
  const float muse = (M == -INFINITY) ? 0.f : M;
  float w[4], L = 0.f;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    w[q] = __builtin_amdgcn_exp2f(ml[q].x - muse) * ml[q].y;
    L += w[q];
  }
#pragma unroll
  for (int off = 8; off >= 1; off >>= 1) L += __shfl_xor(L, off, 16);
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  auto add = [&](uint4 v, float wu) __attribute__((always_inline)) {
    const uint32_t p[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      acc[2 * e] = fmaf(bf16_bits_to_f32(p[e] & 0xffffu), wu, acc[2 * e]);
      acc[2 * e + 1] = fmaf(bf16_bits_to_f32(p[e] >> 16), wu, acc[2 * e + 1]);
    }
  };
#pragma unroll
  for (int u = 0; u < 16; ++u)
    if (u < ns) add(ov[u], __shfl(w[0], u, 16));
  for (int s_ = 16; s_ < ns; ++s_) {
    const uint4 v = *reinterpret_cast<const uint4*>(a.part_o + (s_ * stride + row) * D + 8 * lane);
    const float ws = s_ < 32 ? w[1] : (s_ < 48 ? w[2] : w[3]);
    add(v, __shfl(ws, s_ & 15, 16));
  }
  if (!live) return;
  const float inv = 1.0f / L;
  const int b = bh / a.Hkv, kvh = bh % a.Hkv;
  const int node = r / a.G, gq = r % a.G;
  uint16_t* op = a.out + layer * a.out_lstride +
                 ((static_cast<int64_t>(b) * a.T + node) * a.Hq + kvh * a.G + gq) * D + 8 * lane;
  *reinterpret_cast<uint4*>(op) = make_uint4(pack_bf16(acc[0] * inv, acc[1] * inv), pack_bf16(acc[2] * inv, acc[3] * inv),
                                             pack_bf16(acc[4] * inv, acc[5] * inv), pack_bf16(acc[6] * inv, acc[7] * inv));
}

// ---- grouped-query shapes: every query row of a K/V head in one workgroup ----
// For more than 128 query rows per K/V head (T * G, e.g. 64 nodes x 4 query
// heads) the rows no longer fit the two-role kernel above without a second
// workgroup staging the same K/V.  Here one workgroup of 8 waves takes all of
// them (up to 256): wave w owns query tiles 2w and 2w + 1 (32 rows, Q in
// registers) and every key of the split, so each K/V byte is staged into LDS
// once and read from LDS once per wave.  There are no staging waves: every
// wave writes its share of a 64-key block (8 K rows and 8 V rows) straight
// from HBM into LDS with buffer loads (`buffer_load_dwordx4 ... lds`: lane i
// of a load lands at the load's LDS base + 16 i, so each lane fetches the
// chunk that belongs at its place under the swizzle), two blocks ahead, into
// a ring of four slot arrays.  Each slot is a separate LDS object, so the
// compiler's wait before a read covers only the loads into that slot.  Both
// K and V stay key-major (rows of 256 bytes); P.V reads V through gfx950's
// transposing LDS read (ds_read_b64_tr_b16: within 16 lanes, lanes 4r..4r+3
// supply row r and lane i receives element i of the four rows), two reads
// per MFMA giving a lane the 8 keys of one d that its P^T operand holds.
// Swizzles (16-byte chunk c of row r at position c ^ f(r)): K f(r) = r & 15
// (the conflict-free K layout of the kernel above); V f(r) = 2 * ((r & 3) |
// 4 * (bit 2 of r ^ bit 3 of r)), under which the 32 lanes of either half of
// a transposing read cover the 64 banks once (also for halves made of lane
// groups {0, 2} and {1, 3}), checked on the host over every read.
// One barrier per block; a block is taken as two 32-key halves, pipelined
// within each wave so that MFMAs and the softmax's vector work are
// independent neighbours, interleaved one MFMA to three vector instructions
// (see the loop).  Each query's running sum of probabilities comes from one
// more MFMA per tile and half (a ones operand against P^T), which sums the
// same bf16 values P.V uses and takes the additions off the vector unit.
// Four slots, loads two blocks ahead.
// The loads' buffer resources end at the split's end, so keys past the
// sequence read as zeros (never NaN into P.V) and are masked in the scores.
constexpr int GQ_WAVES = 8;
constexpr int GQ_TILES = 2;                      // query tiles per wave
constexpr int GQ_ROWS = GQ_WAVES * GQ_TILES * 16;  // 256 query rows per workgroup
constexpr int GQ_SLOT = 2 * KB * GROWB;          // one block: K rows, then V rows
constexpr int GQ_AHEAD = 2;                      // blocks loaded ahead of use
constexpr int GQ_MASK_WORDS = 1024;              // T * W <= 1024 (T <= 256)

__device__ __forceinline__ int gq_vswz(int r) {
  return 2 * ((r & 3) | ((((r >> 2) ^ (r >> 3)) & 1) << 2));
}

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
typedef __attribute__((address_space(3))) void* gq_lds_ptr;

__device__ __forceinline__ uint2 lds_read_tr(const char* p) {
  const i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p));
  return __builtin_bit_cast(uint2, v);
}

__global__ __launch_bounds__(512) void tree_attn_gqa(AttnArgs a) {
  __shared__ __attribute__((aligned(16))) char s0[GQ_SLOT], s1[GQ_SLOT], s2[GQ_SLOT], s3[GQ_SLOT];
  __shared__ uint64_t smask[GQ_MASK_WORDS];
  __shared__ int s_redo;
  const int id = blockIdx.x;
  const int task = (id & 7) * a.per_xcd + (id >> 3);
  if (task >= a.tasks) return;  // whole workgroup leaves before any barrier
  const int split = task % a.NS;
  const int rest = task / a.NS;  // = lbh * QC + qc
  const int qc = rest % a.QC;
  const int lbh = rest / a.QC;   // = layer * B * Hkv + bh
  const int bh = lbh % (a.B * a.Hkv);
  const int layer = lbh / (a.B * a.Hkv);
  const int b = bh / a.Hkv;
  const int kvh = bh % a.Hkv;
  const uint16_t* qL = a.q + layer * a.q_lstride;
  uint16_t* outL = a.out + layer * a.out_lstride;

  const int tid = threadIdx.x;
  if (tid == 0) s_redo = 0;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l16 = lane & 15;
  const int grp = lane >> 4;

  int ctx = a.ctx[b];
  ctx = ctx < 0 ? 0 : (ctx > a.S_cap - a.T ? a.S_cap - a.T : ctx);
  const int S = ctx + a.T;
  const int k_begin = split * a.chunk;
  const int k_end = (split == a.NS - 1) ? S : min(S, k_begin + a.chunk);
  const int nblk = k_end > k_begin ? (k_end - k_begin + KB - 1) / KB : 0;

  // Q fragments (tile t, k-step s: d-chunk 4s + grp of row l16) and mask rows
  const int row0 = qc * GQ_ROWS + wave * GQ_TILES * 16;
  auto q_ptr = [&](int r, int ch) __attribute__((always_inline)) {
    const int node = r / a.G, gq = r % a.G;
    return qL + ((static_cast<int64_t>(b) * a.T + node) * a.Hq + kvh * a.G + gq) * D + ch * 8;
  };
  bf16x8 qf[GQ_TILES][4];
  int qnode[GQ_TILES];
#pragma unroll
  for (int t = 0; t < GQ_TILES; ++t) {
    const int r = row0 + t * 16 + l16;
    qnode[t] = r < a.QR ? r / a.G : 0;
    const int rc = min(r, a.QR - 1);
#pragma unroll
    for (int s = 0; s < 4; ++s) qf[t][s] = as_bf16x8(ldg16(q_ptr(rc, 4 * s + grp)));
  }
  const int nmask = a.T * a.W;
  uint64_t mv[2];
#pragma unroll
  for (int u = 0; u < 2; ++u) mv[u] = a.mask[min(tid + 512 * u, nmask - 1)];
  // Q and mask loads first: the mask's wait below then leaves the K/V loads in flight
  __builtin_amdgcn_sched_barrier(0);

  // this wave's share of every block: K rows and V rows 8w .. 8w + 7, as two
  // loads of 4 rows each; lane i fills row i / 16 of a load at position i % 16
  const uint16_t* kbase = a.k + layer * a.kv_lstride + static_cast<int64_t>(bh) * a.S_cap * D;
  const uint16_t* vbase_g = a.v + layer * a.kv_lstride + static_cast<int64_t>(bh) * a.S_cap * D;
  int koff[2], voff[2];
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int r = 8 * wave + 4 * q + (lane >> 4), p = lane & 15;
    koff[q] = r * GROWB + 16 * (p ^ (r & 15));
    voff[q] = r * GROWB + 16 * (p ^ gq_vswz(r));
  }
  auto gload = [&](char* slot, int blk) __attribute__((always_inline)) {
    const int kb = k_begin + blk * KB;
    const int nrec = (k_end - kb) * GROWB;
    const int64_t eoff = static_cast<int64_t>(kb) * D;
    const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(kbase + eoff), 0, nrec > 0 ? nrec : 0, RSRC_WORD3);
    const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(vbase_g + eoff), 0, nrec > 0 ? nrec : 0, RSRC_WORD3);
#pragma unroll
    for (int q = 0; q < 2; ++q)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (gq_lds_ptr)(slot + (8 * wave + 4 * q) * GROWB), 16,
                                               koff[q], 0, 0, 0);
#pragma unroll
    for (int q = 0; q < 2; ++q)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (gq_lds_ptr)(slot + K_TILE + (8 * wave + 4 * q) * GROWB),
                                               16, voff[q], 0, 0, 0);
  };
  gload(s0, 0);
  gload(s1, 1);
#pragma unroll
  for (int u = 0; u < 2; ++u)
    if (tid + 512 * u < nmask) smask[tid + 512 * u] = mv[u];
  const uint32_t* smask32 = reinterpret_cast<const uint32_t*>(smask);

  f32x4 o[GQ_TILES][8];
  // lsum[t]: every element holds the running sum of the query's probabilities
  // (as bf16, the values P.V uses), accumulated by an MFMA against ones
  f32x4 lsum[GQ_TILES];
  float m_run[GQ_TILES], mu[GQ_TILES];
  auto reset = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int t = 0; t < GQ_TILES; ++t) {
      m_run[t] = -INFINITY;
      mu[t] = 0.f;
      lsum[t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) o[t][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
  };
  reset();
  const bf16x8 ones = as_bf16x8(make_uint4(0x3f803f80u, 0x3f803f80u, 0x3f803f80u, 0x3f803f80u));
  // K row kt * 16 + l16, chunk 4s + grp sits at kx0 ^ 64 s in the row
  const int kx0 = 16 * (grp ^ l16);
  // transposing V reads: row 32h + 16 s2 + 4 grp + (l16 >> 2), the 8 bytes of
  // d = 16 dt + 4 (l16 & 3); the row's swizzle depends on its low 4 bits only
  const int vr = 4 * grp + (l16 >> 2);
  const int vx0 = K_TILE + vr * GROWB + 16 * (((l16 >> 1) & 1) ^ gq_vswz(vr)) + 8 * (l16 & 1);

  // Scores of one 32-key half (keys kh .. kh + 31): the MFMAs, then the mask.
  auto qk_mma = [&](const char* blk, int h, f32x4 (&sc)[GQ_TILES][2]) __attribute__((always_inline)) {
#pragma unroll
    for (int st = 0; st < 2; ++st) {
      const char* kr = blk + ((2 * h + st) * 16 + l16) * GROWB;
      bf16x8 kf[4];
#pragma unroll
      for (int s = 0; s < 4; ++s) kf[s] = as_bf16x8(*reinterpret_cast<const uint4*>(kr + (kx0 ^ (64 * s))));
#pragma unroll
      for (int t = 0; t < GQ_TILES; ++t) {
        f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < 4; ++s) acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[s], qf[t][s], acc, 0, 0, 0);
        sc[t][st] = acc;
      }
    }
  };
  auto qk_mask = [&](int kh, f32x4 (&sc)[GQ_TILES][2]) __attribute__((always_inline)) {
    if (kh + 32 > ctx || kh + 32 > k_end) {  // the tree region or the split's end
#pragma unroll
      for (int st = 0; st < 2; ++st) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int key = kh + st * 16 + 4 * grp + e;
          const int jj = key - ctx;
          const int jc = jj < 0 ? 0 : (jj >= a.T ? a.T - 1 : jj);
#pragma unroll
          for (int t = 0; t < GQ_TILES; ++t) {
            const uint32_t wv = smask32[qnode[t] * 2 * a.W + (jc >> 5)];
            const bool vis = key < k_end && (jj < 0 || ((wv >> (jc & 31)) & 1u));
            if (!vis) sc[t][st][e] = -INFINITY;
          }
        }
      }
    }
  };
  // The softmax of a half in two parts.  pre(): the reference max with
  // slack, as in the kernel above; when it moves, the state is rescaled --
  // o, the running sum and, if a half's P^T is still waiting for its P.V
  // (pending), that P^T too, so that it matches the new reference.
  // expo(): the probabilities against the current reference, P^T packed for
  // P.V in pb[t].
  auto pre = [&](const f32x4 (&sc)[GQ_TILES][2], uint4* pending) __attribute__((always_inline)) {
    float lm[GQ_TILES];
    bool over = false;
#pragma unroll
    for (int t = 0; t < GQ_TILES; ++t) {
      lm[t] = fmaxf(__builtin_fmaxf(__builtin_fmaxf(sc[t][0][0], sc[t][0][1]), sc[t][0][2]),
                    __builtin_fmaxf(__builtin_fmaxf(sc[t][0][3], sc[t][1][0]), sc[t][1][1]));
      lm[t] = fmaxf(lm[t], fmaxf(sc[t][1][2], sc[t][1][3]));
      over |= lm[t] * a.scale_log2 > m_run[t] + RESCALE_SLACK;
    }
    if (__builtin_amdgcn_ballot_w64(over)) {
#pragma unroll
      for (int t = 0; t < GQ_TILES; ++t) {
        const float mnew = fmaxf(m_run[t], rows_max(lm[t]) * a.scale_log2);
        const float mu_new = (mnew == -INFINITY) ? 0.f : mnew;
        const float alpha = __builtin_amdgcn_exp2f(m_run[t] - mu_new);
        m_run[t] = mnew;
        mu[t] = mu_new;
        lsum[t] *= alpha;
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) o[t][dt] *= alpha;
        if (pending) {
          uint4& w = pending[t];
          auto sc2 = [&](uint32_t x) {
            return pack_bf16(bf16_bits_to_f32(x & 0xffffu) * alpha, bf16_bits_to_f32(x >> 16) * alpha);
          };
          w = make_uint4(sc2(w.x), sc2(w.y), sc2(w.z), sc2(w.w));
        }
      }
    }
  };
  auto expo = [&](const f32x4 (&sc)[GQ_TILES][2], uint4 (&pb)[GQ_TILES]) __attribute__((always_inline)) {
#pragma unroll
    for (int t = 0; t < GQ_TILES; ++t) {
      float p[2][4];
#pragma unroll
      for (int st = 0; st < 2; ++st)
#pragma unroll
        for (int e = 0; e < 4; ++e) p[st][e] = __builtin_amdgcn_exp2f(fmaf(sc[t][st][e], a.scale_log2, -mu[t]));
      pb[t] = make_uint4(pack_bf16(p[0][0], p[0][1]), pack_bf16(p[0][2], p[0][3]), pack_bf16(p[1][0], p[1][1]),
                         pack_bf16(p[1][2], p[1][3]));
    }
  };
  // O^T += V^T P^T over the half's 32 keys.  All 16 transposing reads of the
  // half are issued before the first MFMA uses them, so their latencies
  // overlap (read one pair, wait, multiply left each wave with eight
  // LDS round trips in a row).
  auto pv = [&](const char* blk, int h, const uint4 (&pb)[GQ_TILES]) __attribute__((always_inline)) {
    uint2 lo[8], hi[8];
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
      const char* vp = blk + (vx0 ^ (32 * dt)) + 32 * h * GROWB;
      lo[dt] = lds_read_tr(vp);
      hi[dt] = lds_read_tr(vp + 16 * GROWB);
    }
#pragma unroll
    for (int t = 0; t < GQ_TILES; ++t)
      lsum[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones, as_bf16x8(pb[t]), lsum[t], 0, 0, 0);
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
      const bf16x8 va = as_bf16x8(make_uint4(lo[dt].x, lo[dt].y, hi[dt].x, hi[dt].y));
#pragma unroll
      for (int t = 0; t < GQ_TILES; ++t)
        o[t][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, as_bf16x8(pb[t]), o[t][dt], 0, 0, 0);
    }
  };

  // One block per interval: wait for this wave's loads of the block (the
  // next block's 4 loads may still fly), pass the barrier, load two blocks
  // ahead into the slot nobody reads any more, then compute the block as a
  // short software pipeline whose MFMA and VALU parts are independent: the
  // second half's scores next to the first half's exponentials, the first
  // half's P.V next to the second half's exponentials.  A rescale at the
  // second half also rescales the first half's waiting P^T.  With checks
  // off the block's probabilities are taken against the reference as it
  // stands, however far its scores rise above it (see the pass below).
  auto step = [&](char* cur, char* ahead, int i, bool checks) __attribute__((always_inline)) {
    __builtin_amdgcn_s_waitcnt(0x0074);  // vmcnt(4) lgkmcnt(0)
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    gload(ahead, i + GQ_AHEAD);  // past the split: an empty resource, zeros, never read
    if (i < nblk) {
      const int kb0 = k_begin + i * KB;
      f32x4 sc0[GQ_TILES][2], sc1[GQ_TILES][2];
      uint4 pb0[GQ_TILES], pb1[GQ_TILES];
      qk_mma(cur, 0, sc0);
      qk_mask(kb0, sc0);
      if (checks) pre(sc0, nullptr);
      // second half's scores (16 MFMAs) beside the first half's exponentials
      qk_mma(cur, 1, sc1);
      expo(sc0, pb0);
#pragma unroll
      for (int g = 0; g < 16; ++g) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);
      }
      qk_mask(kb0 + 32, sc1);
      if (checks) pre(sc1, pb0);
      // first half's P.V (18 MFMAs) beside the second half's exponentials
      pv(cur, 0, pb0);
      expo(sc1, pb1);
#pragma unroll
      for (int g = 0; g < 18; ++g) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 1);
        __builtin_amdgcn_sched_group_barrier(0x002, 3, 1);
      }
      pv(cur, 1, pb1);
    }
  };
  // First pass: the reference max is checked in the split's first block
  // only and then held, which takes the per-half maxima and their vote off
  // the vector unit.  Softmax does not depend on the reference, so the
  // result is the same wherever the probabilities stay in range.  They do
  // unless a later key's score exceeds the first block's maximum by a wide
  // margin: the pass is kept if every live row's running sum is at most 2^64
  // and its output accumulators are finite (then no probability, sum or
  // product overflowed, and the merge's weights exp2(m - M) l keep their
  // range), and if it saw a key in the first block (else its reference is a
  // placeholder that later probabilities could underflow against).  If any
  // wave fails, the workgroup computes the split again checking every half,
  // the reference then following the running maximum within RESCALE_SLACK.
  bool exact = false;
  for (;;) {
    for (int i = 0; i < nblk; i += 4) {
      step(s0, s2, i, exact || i == 0);
      step(s1, s3, i + 1, exact);
      step(s2, s0, i + 2, exact);
      step(s3, s1, i + 3, exact);
    }
    __builtin_amdgcn_s_waitcnt(0x0070);  // every load (also those past the split) has landed
    __syncthreads();
    if (exact) break;
    bool bad = false;
#pragma unroll
    for (int t = 0; t < GQ_TILES; ++t) {
      float mag = 0.f;  // inf and NaN carry through the sum
#pragma unroll
      for (int dt = 0; dt < 8; ++dt)
#pragma unroll
        for (int e = 0; e < 4; ++e) mag += fabsf(o[t][dt][e]);
      const bool live = row0 + t * 16 + l16 < a.QR;  // padding rows repeat a row under the root's mask
      bad |= live && (!(lsum[t][0] <= 0x1p64f) || !(mag <= 3.0e38f) || (nblk > 0 && m_run[t] == -INFINITY));
    }
    if (__builtin_amdgcn_ballot_w64(bad)) s_redo = 1;
    __syncthreads();
    if (!s_redo) break;
    exact = true;
    reset();
    gload(s0, 0);
    gload(s1, 1);
  }

  float l_run[GQ_TILES];
#pragma unroll
  for (int t = 0; t < GQ_TILES; ++t) l_run[t] = lsum[t][0];

  const int BH = a.B * a.Hkv;
#pragma unroll
  for (int t = 0; t < GQ_TILES; ++t) {
    const int r = row0 + t * 16 + l16;
    if (r >= a.QR) continue;
    if (a.NS == 1) {
      const float inv = 1.0f / l_run[t];
      const int node = r / a.G, gq = r % a.G;
      uint16_t* op = outL + ((static_cast<int64_t>(b) * a.T + node) * a.Hq + kvh * a.G + gq) * D;
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) {
        const f32x4 v = o[t][dt] * inv;
        *reinterpret_cast<uint2*>(op + dt * 16 + 4 * grp) =
            make_uint2(pack_bf16(v[0], v[1]), pack_bf16(v[2], v[3]));
      }
    } else {
      const int64_t prow = (static_cast<int64_t>(split) * a.L * BH + lbh) * a.QRpad + r;
      uint16_t* po = a.part_o + prow * D;
      const float inv = l_run[t] > 0.f ? 1.0f / l_run[t] : 0.f;
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) {
        const f32x4 v = o[t][dt] * inv;
        *reinterpret_cast<uint2*>(po + dt * 16 + 4 * grp) = make_uint2(pack_bf16(v[0], v[1]), pack_bf16(v[2], v[3]));
      }
      if (grp == 0)
        *reinterpret_cast<float2*>(a.part_ml + ((static_cast<int64_t>(lbh) * a.QRpad + r) * a.NS + split) * 2) =
            make_float2(m_run[t], l_run[t]);
    }
  }
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
  bool gqa;  // more than 128 query rows per K/V head: tree_attn_gqa
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
    default: return reinterpret_cast<const void*>(&tree_attn_bf16<2>);
  }
}

// Above 64 KiB the dynamic LDS size must be allowed for each kernel (the
// attribute must not exceed what the kernel can use, so it is set to the
// largest size asked for so far).
int allow_lds(int qtw, int lds) {
  static int allowed[4] = {0};
  if (lds <= 64 * 1024 || lds <= allowed[qtw]) return MEDUSA_OK;
  const hipError_t e = hipFuncSetAttribute(kernel_for(qtw), hipFuncAttributeMaxDynamicSharedMemorySize, lds);
  if (e != hipSuccess) {
    (void)hipGetLastError();
    set_error("cannot allow %d bytes of dynamic LDS for tree attention: %s", lds, hipGetErrorString(e));
    return MEDUSA_EUNSUPPORTED;
  }
  allowed[qtw] = lds;
  return MEDUSA_OK;
}

// workgroups of this configuration one CU runs at once (1 if unknown)
int occupancy(int qtw, int lds) {
  static int cache[4][9] = {{0}};
  const int bucket = lds / (20 * 1024);
  if (bucket < 9 && cache[qtw][bucket]) return cache[qtw][bucket];
  int n = 0;
  if (allow_lds(qtw, lds) != MEDUSA_OK ||
      hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, kernel_for(qtw), 768, lds) != hipSuccess || n < 1) {
    (void)hipGetLastError();
    n = 1;
  }
  if (bucket < 9) cache[qtw][bucket] = n;
  return n;
}

int occupancy_gqa() {
  static int n = 0;
  if (!n) {
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, reinterpret_cast<const void*>(&tree_attn_gqa), 512,
                                                     0) != hipSuccess || n < 1) {
      (void)hipGetLastError();
      n = 1;
    }
  }
  return n;
}

Plan make_plan(int B, int Hq, int Hkv, int ctx_max, int T, int W) {
  Plan p{};
  p.G = Hq / Hkv;
  p.QR = T * p.G;
  p.NQT = (p.QR + 15) / 16;
  p.QRpad = p.NQT * 16;
  p.gqa = p.NQT > 8;
  if (p.gqa) {
    // 256 query rows per workgroup, 2 tiles per wave, static LDS
    p.QC = (p.NQT + 15) / 16;
    p.QTW = GQ_TILES;
    p.lds_bytes = 0;
  } else {
    // at most 2 query tiles per compute wave (more would spill registers)
    p.QC = (p.NQT + 7) / 8;
    p.QTW = (p.NQT + 4 * p.QC - 1) / (4 * p.QC);
    p.lds_mask = 0;
    p.lds_q = static_cast<int>(round_up(static_cast<size_t>(T) * W * 8, 16));
    p.lds_ring = p.lds_q + (p.QTW == 1 ? 0 : 4 * p.QTW * 16 * KROWB);
    p.lds_bytes = p.lds_ring + NSLOT * BLK_BYTES;
  }
  const int Smax = ctx_max + T;
  const int base = B * Hkv * p.QC;
  int ns = env_int("MEDUSA_ATTN_SPLITS", 0);
  if (ns <= 0) {
    // the most splits whose workgroups all run in one round of the
    // resident slots (a second, partly filled round costs more than longer
    // splits do, and fewer splits leave CUs idle); at least one block each
    const int slots = cu_count() * (p.gqa ? occupancy_gqa() : occupancy(p.QTW, p.lds_bytes));
    const int max_ns = (Smax + KB - 1) / KB;
    ns = slots / (base > 0 ? base : 1);
    if (ns > max_ns) ns = max_ns;
    if (ns < 1) ns = 1;
  }
  if (ns > MAX_SPLITS) ns = MAX_SPLITS;
  int chunk = (Smax + ns - 1) / ns;
  chunk = (chunk + KB - 1) / KB * KB;
  p.chunk = chunk;
  p.NS = (Smax + chunk - 1) / chunk;
  if (p.NS < 1) p.NS = 1;
  if (p.NS > 1) {
    const size_t rows = static_cast<size_t>(p.NS) * B * Hkv * p.QRpad;
    p.off_ml = round_up(rows * D * 2, 256);
    p.ws_bytes = p.off_ml + round_up(rows * 2 * 4, 256);
  }
  return p;
}

template <int QTW>
int launch_cfg(const AttnArgs& a, int grid, int lds, hipStream_t s) {
  const int rc = allow_lds(QTW, lds);
  if (rc) return rc;
  hipLaunchKernelGGL((tree_attn_bf16<QTW>), dim3(grid), dim3(768), lds, s, a);
  return check_launch("tree attention (bf16)");
}

}  // namespace

namespace {

// one or several layers (layer l at base + l * stride elements)
int attention_launch(const void* q, const void* k_cache, const void* v_cache, int64_t q_lstride,
                     int64_t kv_lstride, int64_t out_lstride, int L, const int32_t* ctx_len,
                     int ctx_max, const medusa_tree_t* tree, int B, int Hq, int Hkv, int D_,
                     int S_cap, float scale, medusa_dtype_t dt, void* out, void* ws,
                     size_t ws_bytes, hipStream_t stream) {
  int rc = check_tree(tree);
  if (rc) return rc;
  MEDUSA_CHECK_ARG(L >= 1, "L=%d must be >= 1", L);
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
    for (int l = 0; l < L; ++l) {  // small configurations: one launch per layer
      f.q = static_cast<const float*>(q) + l * q_lstride;
      f.k = static_cast<const float*>(k_cache) + l * kv_lstride;
      f.v = static_cast<const float*>(v_cache) + l * kv_lstride;
      f.out = static_cast<float*>(out) + l * out_lstride;
      hipLaunchKernelGGL(tree_attn_f32, dim3(static_cast<unsigned>((rows + 3) / 4)), dim3(256), 0,
                         stream, f);
      rc = check_launch("tree attention (f32)");
      if (rc) return rc;
    }
    return MEDUSA_OK;
  }
  MEDUSA_CHECK_ARG(dt == MEDUSA_BF16, "unknown dtype %d", static_cast<int>(dt));
  if (D_ != D) {
    set_error("bf16 tree attention supports D = 128 (got D=%d)", D_);
    return MEDUSA_EUNSUPPORTED;
  }
  MEDUSA_CHECK_ARG(S_cap < (1 << 23), "S_cap=%d too large (K/V byte offsets are 32-bit)", S_cap);
  const Plan p = make_plan(L * B, Hq, Hkv, ctx_max, tree->T, tree->W);
  if (p.NS > 1 && (!ws || ws_bytes < p.ws_bytes || !aligned256(ws))) {
    set_error("tree attention workspace: need %zu bytes, 256-byte aligned (got %zu at %p)",
              p.ws_bytes, ws_bytes, ws);
    return MEDUSA_EWORKSPACE;
  }
  if (p.lds_bytes > LDS_MAX) {
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
  a.L = L;
  a.q_lstride = q_lstride;
  a.kv_lstride = kv_lstride;
  a.out_lstride = out_lstride;
  a.QR = p.QR;
  a.QRpad = p.QRpad;
  a.QC = p.QC;
  a.NS = p.NS;
  a.chunk = p.chunk;
  // both grids must stay within 2^32 work-items (768 per attention
  // workgroup, 32 per merged row)
  const int64_t tasks = static_cast<int64_t>(L) * B * Hkv * p.QC * p.NS;
  const int64_t merge_rows = static_cast<int64_t>(L) * B * Hkv * p.QR;
  if ((tasks + 7) / 8 * 8 * 768 >= (1ll << 32) || (p.NS > 1 && merge_rows * 32 >= (1ll << 32))) {
    set_error("tree attention grid too large (L*B*Hkv=%lld, %d splits)",
              static_cast<long long>(L) * B * Hkv, p.NS);
    return MEDUSA_EUNSUPPORTED;
  }
  a.tasks = static_cast<int>(tasks);
  a.per_xcd = (a.tasks + 7) / 8;
  a.scale_log2 = scale * LOG2E;
  a.out = static_cast<uint16_t*>(out);
  if (p.NS > 1) {
    char* w = static_cast<char*>(ws);
    a.part_o = reinterpret_cast<uint16_t*>(w);
    a.part_ml = reinterpret_cast<float*>(w + p.off_ml);
  }
  a.lds_mask = p.lds_mask;
  a.lds_q = p.lds_q;
  a.lds_ring = p.lds_ring;
  const int grid = 8 * a.per_xcd;
  if (p.gqa) {
    hipLaunchKernelGGL(tree_attn_gqa, dim3(grid), dim3(512), 0, stream, a);
    rc = check_launch("tree attention (bf16, grouped queries)");
  } else {
    switch (p.QTW) {
      case 1: rc = launch_cfg<1>(a, grid, p.lds_bytes, stream); break;
      default: rc = launch_cfg<2>(a, grid, p.lds_bytes, stream); break;
    }
  }
  if (rc || p.NS == 1) return rc;
  const int64_t rows = static_cast<int64_t>(L) * B * Hkv * p.QR;
  // one wave per workgroup (measured faster than 4 or 16 waves); with 4096
  // rows or more, four rows per wave in 16-byte pieces (zephyr7b-shaped: a
  // layer's call ~4.5 us shorter), below that two rows per wave in 8-byte
  // pieces (more waves for few rows)
  if (rows >= 4096)
    hipLaunchKernelGGL(merge_splits16, dim3(static_cast<unsigned>((rows + 3) / 4)), dim3(64), 0, stream, a);
  else
    hipLaunchKernelGGL(merge_splits, dim3(static_cast<unsigned>((rows + 1) / 2)), dim3(64), 0, stream, a);
  return check_launch("tree attention split merge");
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
  return attention_launch(q, k_cache, v_cache, 0, 0, 0, 1, ctx_len, ctx_max, tree, B, Hq, Hkv, D_,
                          S_cap, scale, dt, out, ws, ws_bytes, stream);
}

extern "C" size_t medusa_tree_attention_layers_workspace_size(int L, int B, int Hq, int Hkv, int D_,
                                                              int ctx_max, const medusa_tree_t* tree,
                                                              medusa_dtype_t dt) {
  if (L < 1 || B < 1 || static_cast<int64_t>(L) * B >= (1ll << 31)) return 0;
  return medusa_tree_attention_workspace_size(L * B, Hq, Hkv, D_, ctx_max, tree, dt);
}

extern "C" int medusa_tree_attention_layers(const void* q, const void* k_cache, const void* v_cache,
                                            int64_t q_layer_stride, int64_t kv_layer_stride,
                                            int64_t out_layer_stride, int L, const int32_t* ctx_len,
                                            int ctx_max, const medusa_tree_t* tree, int B, int Hq,
                                            int Hkv, int D_, int S_cap, float scale,
                                            medusa_dtype_t dt, void* out, void* ws, size_t ws_bytes,
                                            hipStream_t stream) {
  clear_error();
  MEDUSA_CHECK_ARG(L >= 1 && static_cast<int64_t>(L) * B * Hkv < (1ll << 28), "L=%d out of range", L);
  const int esize = dt == MEDUSA_F32 ? 4 : 2;
  const int64_t q_elems = static_cast<int64_t>(B) * (tree ? tree->T : 0) * Hq * D_;
  const int64_t kv_elems = static_cast<int64_t>(B) * Hkv * S_cap * D_;
  MEDUSA_CHECK_ARG(L == 1 || (q_layer_stride >= q_elems && out_layer_stride >= q_elems &&
                              kv_layer_stride >= kv_elems),
                   "layer strides (%lld, %lld, %lld) smaller than one layer",
                   static_cast<long long>(q_layer_stride), static_cast<long long>(kv_layer_stride),
                   static_cast<long long>(out_layer_stride));
  MEDUSA_CHECK_ARG((q_layer_stride * esize) % 16 == 0 && (kv_layer_stride * esize) % 16 == 0 &&
                       (out_layer_stride * esize) % 16 == 0,
                   "layer strides must keep 16-byte alignment");
  return attention_launch(q, k_cache, v_cache, q_layer_stride, kv_layer_stride, out_layer_stride, L,
                          ctx_len, ctx_max, tree, B, Hq, Hkv, D_, S_cap, scale, dt, out, ws,
                          ws_bytes, stream);
}

// ---- the no-allocation variant of medusa_tree_attention ---------------------
// For callers that cannot allocate device memory (code under HIP graph
// capture, tight serving loops, harnesses that forbid allocation): the split
// partials live in a fixed array of this library's module instead of a
// caller's workspace.  Each GPU the library runs on holds its own copy until
// the process ends; the host-side name is only a stand-in, so its device
// address is taken once per device with hipGetSymbolAddress (with that device
// current) and that address is what the kernels receive.  Every call on a
// GPU shares that GPU's array: calls that overlap on one GPU (e.g. on two
// streams) race.  Nothing in it needs clearing: every partial a merge reads
// is written by the same call first.
static __device__ __align__(256) char scratch[MEDUSA_ATTENTION_SCRATCH_BYTES];

namespace {

std::mutex scratch_mutex;
void* scratch_ptr[64] = {nullptr};

int scratch_for_current_device(void** out) {
  int dev = 0;
  const hipError_t e0 = hipGetDevice(&dev);
  if (e0 != hipSuccess || dev < 0 || dev >= 64) {
    (void)hipGetLastError();
    set_error("no usable current device for the attention scratch (device %d)", dev);
    return MEDUSA_EHIP;
  }
  std::lock_guard<std::mutex> lock(scratch_mutex);
  if (!scratch_ptr[dev]) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) {
      (void)hipGetLastError();
      set_error("hipGetSymbolAddress of the attention scratch failed on device %d: %s", dev,
                hipGetErrorString(e));
      return MEDUSA_EHIP;
    }
    scratch_ptr[dev] = p;
  }
  *out = scratch_ptr[dev];
  return MEDUSA_OK;
}

}  // namespace

extern "C" int medusa_tree_attention_noalloc(const void* q, const void* k_cache, const void* v_cache,
                                             const int32_t* ctx_len, int ctx_max,
                                             const medusa_tree_t* tree, int B, int Hq, int Hkv,
                                             int D_, int S_cap, float scale, medusa_dtype_t dt,
                                             void* out, hipStream_t stream) {
  clear_error();
  // host-only sizing first: invalid arguments give 0 here and are reported
  // by the launch below
  const size_t need = medusa_tree_attention_workspace_size(B, Hq, Hkv, D_, ctx_max, tree, dt);
  if (need > MEDUSA_ATTENTION_SCRATCH_BYTES) {
    set_error("tree attention needs %zu bytes of split partials; the no-allocation call's scratch "
              "holds %zu (use medusa_tree_attention with a workspace)",
              need, static_cast<size_t>(MEDUSA_ATTENTION_SCRATCH_BYTES));
    return MEDUSA_EWORKSPACE;
  }
  void* ws = nullptr;
  if (need > 0) {
    const int rc = scratch_for_current_device(&ws);
    if (rc) return rc;
  }
  return attention_launch(q, k_cache, v_cache, 0, 0, 0, 1, ctx_len, ctx_max, tree, B, Hq, Hkv, D_,
                          S_cap, scale, dt, out, ws, ws ? MEDUSA_ATTENTION_SCRATCH_BYTES : 0, stream);
}
