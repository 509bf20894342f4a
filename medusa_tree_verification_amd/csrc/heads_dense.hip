// Dense-variant Medusa heads: the K heads on the hidden state of every tree
// token at once (M = B*T rows) as tiled MFMA GEMMs, with each head's top-k
// taken from the vocab projection's output tiles.
//
// P1 ("Medusa 심층 아키텍처"), section "Medusa의 핵심 철학 ... 잔차 블록을 포함한
// Medusa 헤드 구조": head k maps a hidden state h to r = SiLU(W1_k h) + h and
// then to logits W_lm,k r; its section "소스코드 레벨 구조 분석" keeps every
// head's top-k logits as that head's candidates.  Run on all B*T tree rows,
// the heads leave the next step's candidates in place for whichever node is
// accepted.
//
// bf16 design (gfx950)
//   C[m][n] = sum_k X[m][k] W[n][k], X the activations [M][Kd] and W the
//   weights [N][Kd], both k-contiguous.  v_mfma_f32_16x16x32_bf16 takes 16
//   weight rows as A and 16 activation rows as B, so a lane's accumulator
//   holds one activation row and 4 consecutive output columns.
//   Workgroup: BM activation rows (64 or 128) x 128 output columns, 4 waves
//   in a 2 x 2 arrangement of (BM/2) x 64 wave tiles, k-steps of 64.  Both
//   tiles of a k-step go global -> registers two steps ahead (buffer loads
//   whose descriptors end at the matrices' ends, every load issued
//   unconditionally so each wait covers exactly its step) -> LDS (two
//   buffers, one barrier per step).  LDS rows are 128 bytes, 16-byte chunk c
//   of row r at 16 * (c ^ ((r >> 1) & 7)): the MFMA operand reads (lane group
//   g of k-step s reads chunk 4s + g of its row) and the staging writes are
//   free of bank conflicts under the gfx950 rule (16-byte reads in lane
//   groups {0-3, 12-15, 20-27} and +32, 16-byte writes in groups of 8
//   consecutive lanes).
//   Workgroups are numbered so that the row tiles of one weight tile run on
//   one XCD (dispatch gives workgroup i to XCD i % 8): the weight tile is
//   read from HBM once and served to the others from that XCD's L2.
//   Residual-block epilogue: bf16(SiLU(acc) + h).  Vocab-projection
//   epilogue: the fp32 tile goes to LDS; each row's 128 columns are scanned
//   in column order by 256/BM threads, each keeping a sorted list of its
//   largest values (a value enters only if strictly larger, so equal logits
//   keep the lower column first); the lists of a row are merged and the
//   row's top-kmax (logit, column) pairs written as that tile's candidates.
//   A second kernel merges every row's tile candidates into each head's
//   top-k.  The fp32 logits reach HBM only when the caller asks for them.
#include <cfloat>

#include "internal.h"

using namespace medusa;
using namespace medusa::dev;

namespace {

constexpr int BN = 128;               // output columns per workgroup
constexpr int BK = 64;                // k per step
constexpr int TROW = BK * 2;          // bytes per staged row
constexpr int RSRC_WORD3 = 0x00020000;

enum { EPI_RESID = 1, EPI_TOPK = 2 };

__device__ __forceinline__ int toff(int r, int c) { return r * TROW + 16 * (c ^ ((r >> 1) & 7)); }

__device__ __forceinline__ uint4 bload16(__amdgpu_buffer_rsrc_t r, int byte_off) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, 0));
}

struct DenseArgs {
  const uint16_t* x;  // head h's activations: x + h * x_hstride, [M][Kd]
  int64_t x_hstride;
  const uint16_t* w;  // head h's weights: w + h * w_hstride, [N][Kd]
  int64_t w_hstride;
  int M, N, Kd;
  int mtiles, ntiles, tasks, per_xcd;
  // residual block
  const uint16_t* hid;  // [M][Kd], N == Kd
  uint16_t* r_out;      // [heads][M][N]
  // vocab projection
  int K;                // heads (for the [M][K][...] layouts)
  int kmax;
  float* cand_v;        // [M][K][ntiles][kmax]
  int32_t* cand_i;
  float* logits;        // optional [M][K][N]
};

// KG k-groups of 4 waves: group q takes k-steps q, q + KG, ... with its own
// LDS buffers, and the groups' sums meet in LDS before the epilogue, so a
// workgroup keeps KG times the loads in flight (the residual block at small M
// has one workgroup per CU and is bound by the bytes on their way).
template <int BM, int EPI, int KM, int BNT = BN, int KG = 1>
__global__ __launch_bounds__(256 * KG) void dense_gemm_bf16(DenseArgs a) {
  static_assert(BNT == BN || EPI == EPI_RESID, "the top-k epilogue takes 128-column tiles");
  static_assert(KG == 1 || EPI == EPI_RESID, "k-groups only in front of the residual epilogue");
  constexpr int MT = BM / 32;         // 16-row activation tiles per wave
  constexpr int NJ = BNT / 32;        // 16-column output tiles per wave
  constexpr int XCH = BM * 8 / 256;   // 16-byte X chunks per thread per step
  constexpr int WCH = BNT * 8 / 256;  // 16-byte W chunks per thread per step
  constexpr int CH = XCH + WCH;
  constexpr int XT = BM * TROW;       // X tile bytes (W tile follows)
  constexpr int STAGE = (BM + BNT) * TROW;
  extern __shared__ __attribute__((aligned(16))) char smem[];

  const int id = blockIdx.x;
  const int task = (id & 7) * a.per_xcd + (id >> 3);
  if (task >= a.tasks) return;  // the whole workgroup leaves before any barrier
  const int mt = task % a.mtiles;
  const int rest = task / a.mtiles;
  const int nt = rest % a.ntiles;
  const int head = rest / a.ntiles;
  const int m0 = mt * BM, n0 = nt * BNT;
  if (m0 >= a.M || n0 >= a.N) return;  // no tile past the matrices (whole workgroup, no barrier yet)

  const int tid = threadIdx.x & 255;
  const int kg = KG == 1 ? 0 : __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) >> 8);
  char* const sm = smem + kg * 2 * STAGE;  // this k-group's two buffers
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wr = wave >> 1, wc = wave & 1;
  const int l16 = lane & 15, g = lane >> 4;

  const uint16_t* xb = a.x + head * a.x_hstride + static_cast<int64_t>(m0) * a.Kd;
  const uint16_t* wb = a.w + head * a.w_hstride + static_cast<int64_t>(n0) * a.Kd;
  const int xrows = min(BM, a.M - m0), wrows = min(BNT, a.N - n0);
  const __amdgpu_buffer_rsrc_t rx =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(xb), 0, xrows * a.Kd * 2, RSRC_WORD3);
  const __amdgpu_buffer_rsrc_t rw =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(wb), 0, wrows * a.Kd * 2, RSRC_WORD3);

  // this thread's chunks c = tid + 256u of each tile: row c / 8, chunk c % 8
  int goff[CH], loff[CH];
#pragma unroll
  for (int u = 0; u < CH; ++u) {
    const bool isx = u < XCH;
    const int c = tid + 256 * (isx ? u : u - XCH);
    goff[u] = (c >> 3) * a.Kd * 2 + (c & 7) * 16;
    loff[u] = (isx ? 0 : XT) + toff(c >> 3, c & 7);
  }
  auto gload = [&](uint4 (&R)[CH], int ks) __attribute__((always_inline)) {
    const int kb = (ks * KG + kg) * TROW;  // this group's ks-th k-step
#pragma unroll
    for (int u = 0; u < CH; ++u) R[u] = bload16(u < XCH ? rx : rw, goff[u] + kb);
  };
  auto lput = [&](const uint4 (&R)[CH], char* st) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < CH; ++u) *reinterpret_cast<uint4*>(st + loff[u]) = R[u];
  };

  f32x4 acc[MT][NJ];
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  // operand rows: W wc*(BNT/2) + 16j + l16, X wr*(BM/2) + 16i + l16; chunk 4s + g
  const int sw = (l16 >> 1) & 7;
  const int cx0 = 16 * (g ^ sw), cx1 = 16 * ((4 + g) ^ sw);
  const int wrow = XT + (wc * (BNT / 2) + l16) * TROW;
  const int xrow = (wr * (BM / 2) + l16) * TROW;
  auto compute = [&](const char* st) __attribute__((always_inline)) {
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const int cx = s ? cx1 : cx0;
      bf16x8 wf[NJ], xf[MT];
#pragma unroll
      for (int j = 0; j < NJ; ++j) wf[j] = as_bf16x8(*reinterpret_cast<const uint4*>(st + wrow + j * 16 * TROW + cx));
#pragma unroll
      for (int i = 0; i < MT; ++i) xf[i] = as_bf16x8(*reinterpret_cast<const uint4*>(st + xrow + i * 16 * TROW + cx));
#pragma unroll
      for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int j = 0; j < NJ; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wf[j], xf[i], acc[i][j], 0, 0, 0);
    }
  };

  // Pipeline: block b is in registers R[b & 1] until it is written to LDS
  // buffer b & 1 during step b - 1; a group's step count is even, so the
  // unrolled pair of steps keeps every register index a constant.  Loads of
  // blocks past the end read zeros or bytes of the next row and are never
  // used.
  const int nk = a.Kd / BK / KG;
  uint4 R[2][CH];
  gload(R[0], 0);
  __builtin_amdgcn_sched_barrier(0);
  gload(R[1], 1);
  __builtin_amdgcn_sched_barrier(0);
  lput(R[0], sm);
  gload(R[0], 2);
  __syncthreads();
  for (int ks = 0; ks < nk; ks += 2) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      compute(sm + j * STAGE);
      lput(R[(j + 1) & 1], sm + ((j + 1) & 1) * STAGE);
      gload(R[(j + 1) & 1], ks + j + 3);
      __syncthreads();
    }
  }
  if constexpr (KG == 2) {
    // the second group's sums into its own buffers (the loop's last barrier
    // ended every read of them), then added by the first group in k-group
    // order; the second group leaves (no barrier follows in its epilogue)
    static_assert(MT * NJ * 256 * 16 <= 2 * STAGE, "k-group sums exceed the group's buffers");
    if (kg == 1) {
#pragma unroll
      for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int j = 0; j < NJ; ++j) *reinterpret_cast<f32x4*>(sm + ((i * NJ + j) * 256 + tid) * 16) = acc[i][j];
    }
    __syncthreads();
    if (kg == 1) return;
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
      for (int j = 0; j < NJ; ++j)
        acc[i][j] += *reinterpret_cast<const f32x4*>(smem + 2 * STAGE + ((i * NJ + j) * 256 + tid) * 16);
  }

  if constexpr (EPI == EPI_RESID) {
    // r[head][m][n] = bf16(SiLU(acc) + h[m][n]), 4 consecutive n per lane
#pragma unroll
    for (int i = 0; i < MT; ++i) {
      const int m = m0 + wr * (BM / 2) + 16 * i + l16;
      if (m >= a.M) continue;
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        const int n = n0 + wc * (BNT / 2) + 16 * j + 4 * g;
        if (n >= a.N) continue;  // N % 4 == 0: all 4 columns are in range
        const uint2 hv = *reinterpret_cast<const uint2*>(a.hid + static_cast<int64_t>(m) * a.Kd + n);
        float o[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float y = acc[i][j][e];
          const uint32_t hb = (e & 1) ? ((e < 2 ? hv.x : hv.y) >> 16) : ((e < 2 ? hv.x : hv.y) & 0xffffu);
          o[e] = y / (1.0f + expf(-y)) + bf16_bits_to_f32(hb);
        }
        uint16_t* dst = a.r_out + (static_cast<int64_t>(head) * a.M + m) * a.N + n;
        *reinterpret_cast<uint2*>(dst) =
            make_uint2(f32_to_bf16_bits(o[0]) | (f32_to_bf16_bits(o[1]) << 16),
                       f32_to_bf16_bits(o[2]) | (f32_to_bf16_bits(o[3]) << 16));
      }
    }
  } else {
    // the fp32 tile in LDS: column granule q (4 columns) of row r at
    // r * 512 + 16 * (q ^ (r & 7)); the loop's last barrier freed the buffers
    float* tile = reinterpret_cast<float*>(smem);
    auto tgran = [](int r, int q) { return r * 128 + 4 * (q ^ (r & 7)); };  // in floats
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        *reinterpret_cast<f32x4*>(tile + tgran(wr * (BM / 2) + 16 * i + l16, wc * 16 + 4 * j + g)) = acc[i][j];
    __syncthreads();
    if (a.logits) {  // rows of the tile to logits[m][head][n0 ..], 8 rows per pass
#pragma unroll
      for (int p = 0; p < BM / 8; ++p) {
        const int r = p * 8 + (tid >> 5), q = tid & 31;
        const int m = m0 + r, n = n0 + 4 * q;
        if (m < a.M && n < a.N)
          *reinterpret_cast<f32x4*>(a.logits + (static_cast<int64_t>(m) * a.K + head) * a.N + n) =
              *reinterpret_cast<const f32x4*>(tile + tgran(r, q));
      }
    }
    constexpr int TPR = 256 / BM;   // threads per row
    constexpr int CPT = BN / TPR;   // columns per thread
    const int r = tid / TPR, part = tid % TPR;
    float tv[KM];
    int ti[KM];
#pragma unroll
    for (int s = 0; s < KM; ++s) {
      tv[s] = -INFINITY;
      ti[s] = 0x7fffffff;
    }
#pragma unroll 4
    for (int q = 0; q < CPT / 4; ++q) {
      const int qq = part * (CPT / 4) + q;
      const f32x4 v = *reinterpret_cast<const f32x4*>(tile + tgran(r, qq));
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int n = n0 + 4 * qq + e;
        if (v[e] > tv[KM - 1] && n < a.N) list_insert<KM>(tv, ti, v[e], n);
      }
    }
    __syncthreads();  // every thread is done with the tile
    // the row's other threads hand their lists over (each covers later
    // columns than the one before it, so merging in order keeps ties right)
    float* lv = tile;
    int* li = reinterpret_cast<int*>(tile + 256 * KM);
    if (part) {
#pragma unroll
      for (int s = 0; s < KM; ++s) {
        lv[tid * KM + s] = tv[s];
        li[tid * KM + s] = ti[s];
      }
    }
    __syncthreads();
    if (part == 0) {
      for (int o = 1; o < TPR; ++o) {
        for (int s = 0; s < KM; ++s) {
          const float x = lv[(tid + o) * KM + s];
          if (!(x > tv[KM - 1])) break;  // the list is sorted: nothing after it enters either
          list_insert<KM>(tv, ti, x, li[(tid + o) * KM + s]);
        }
      }
      const int m = m0 + r;
      if (m < a.M) {
        const int64_t base = ((static_cast<int64_t>(m) * a.K + head) * a.ntiles + nt) * a.kmax;
#pragma unroll
        for (int s = 0; s < KM; ++s) {
          if (s < a.kmax) {
            a.cand_v[base + s] = tv[s];
            a.cand_i[base + s] = ti[s];
          }
        }
      }
    }
  }
}

// ---- large-M tiles: 256 x 256, direct-to-LDS loads -----------------------
// For M > 128 (e.g. zephyr7b-shaped, M = 512) a workgroup of 8 waves takes
// 256 activation rows x 256 output columns (wave tile 64 x 128), halving the
// L2 -> LDS bytes per FLOP of the 128 x 128 tile.  Each 32-wide k-step's two
// tiles (64-byte rows, chunk c of row r at 16 * (c ^ 2 * bit2(r))) are
// written straight into LDS by buffer loads (`buffer_load_dwordx4 ... lds`:
// lane i of a wave's load lands at the wave's LDS base + 16 i, so each lane
// fetches the chunk that belongs at its position) into a ring of four stage
// buffers, four steps ahead of their MFMAs.  The MFMA operands go LDS ->
// registers one step ahead (two register sets), so the MFMAs of a step run
// on fragments already in registers while the next step's are read: with
// two waves per SIMD meeting at every barrier, an LDS round trip between the
// barrier and the first MFMA left the matrix cores idle for most of the
// step.  The buffers are separate LDS objects so that the compiler's wait
// for the loads into one does not cover the others.
constexpr int B2M = 256, B2N = 256, B2K = 32;
constexpr int B2ROW = B2K * 2;               // 64 bytes per staged row
constexpr int B2X = B2M * B2ROW;             // X tile bytes; the W tile follows
constexpr int B2STAGE = (B2M + B2N) * B2ROW; // 32 KiB
typedef __attribute__((address_space(3))) void* lds_ptr_t;

__device__ __forceinline__ int b2swz(int r) { return ((r >> 2) & 1) << 1; }

template <int EPI, int KM>
__global__ __launch_bounds__(512) void dense_gemm_big(DenseArgs a) {
  __shared__ __attribute__((aligned(16))) char st0[B2STAGE], st1[B2STAGE], st2[B2STAGE], st3[B2STAGE];
  const int id = blockIdx.x;
  const int task = (id & 7) * a.per_xcd + (id >> 3);
  if (task >= a.tasks) return;  // the whole workgroup leaves before any barrier
  const int mt = task % a.mtiles;
  const int rest = task / a.mtiles;
  const int nt = rest % a.ntiles;
  const int head = rest / a.ntiles;
  const int m0 = mt * B2M, n0 = nt * B2N;
  if (m0 >= a.M || n0 >= a.N) return;  // no tile past the matrices (whole workgroup, no barrier yet)

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave & 3, wn = wave >> 2;  // 64-row quarter, 128-column half
  const int l16 = lane & 15, g = lane >> 4;

  const uint16_t* xb = a.x + head * a.x_hstride + static_cast<int64_t>(m0) * a.Kd;
  const uint16_t* wb = a.w + head * a.w_hstride + static_cast<int64_t>(n0) * a.Kd;
  const int xrows = min(B2M, a.M - m0), wrows = min(B2N, a.N - n0);
  const __amdgpu_buffer_rsrc_t rx =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(xb), 0, xrows * a.Kd * 2, RSRC_WORD3);
  const __amdgpu_buffer_rsrc_t rw =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(wb), 0, wrows * a.Kd * 2, RSRC_WORD3);

  // this wave's loads: 16-row blocks 2*wave and 2*wave + 1 of each tile;
  // lane i fills row i/4 of the block at position i%4 with chunk
  // (i%4) ^ swizzle(row).  Rows past the matrices' ends are left as they
  // are: they only feed outputs that are never written.
  int goff[2];
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int row = 16 * (2 * wave + q) + (lane >> 2);
    goff[q] = row * a.Kd * 2 + 16 * ((lane & 3) ^ b2swz(row));
  }
  auto dma = [&](char* st, int ks) __attribute__((always_inline)) {
    const int kb = ks * B2ROW;
#pragma unroll
    for (int q = 0; q < 2; ++q)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rx, (lds_ptr_t)(st + (2 * wave + q) * 1024), 16, goff[q] + kb, 0, 0, 0);
#pragma unroll
    for (int q = 0; q < 2; ++q)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rw, (lds_ptr_t)(st + B2X + (2 * wave + q) * 1024), 16, goff[q] + kb, 0, 0, 0);
  };

  f32x4 acc[4][8];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int cx = 16 * (g ^ b2swz(l16));
  const int xrow = (wm * 64 + l16) * B2ROW + cx;
  const int wrow = B2X + (wn * 128 + l16) * B2ROW + cx;
  // operand fragments of one k-step: [0, 4) X rows, [4, 12) W rows
  auto read = [&](bf16x8 (&f)[12], const char* st) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < 4; ++i) f[i] = as_bf16x8(*reinterpret_cast<const uint4*>(st + xrow + i * 16 * B2ROW));
#pragma unroll
    for (int j = 0; j < 8; ++j) f[4 + j] = as_bf16x8(*reinterpret_cast<const uint4*>(st + wrow + j * 16 * B2ROW));
  };
  auto mma = [&](const bf16x8 (&f)[12]) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(f[4 + j], f[i], acc[i][j], 0, 0, 0);
  };
  // Step k multiplies the fragments read during step k - 1 while it reads
  // step k + 1's, so the barrier is never followed by an LDS round trip
  // before the first MFMA.  At its top a wave waits for its own loads of
  // step k + 1 (s_waitcnt vmcnt(8) lgkmcnt(0): steps k + 2 and k + 3 may
  // still fly) and for its reads of step k's buffer; after the barrier every
  // wave's step k + 1 bytes are in LDS and nobody reads step k's buffer any
  // more, so the loads of step k + 4 go there.
  auto step = [&](const bf16x8 (&cur)[12], bf16x8 (&nxt)[12], const char* rd, char* buf, int ks)
      __attribute__((always_inline)) {
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(0x0078);
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    dma(buf, ks + 4);  // past the end: bytes of the next row or zeros, never used
    read(nxt, rd);     // past the end (last step): in-bounds LDS, never used
    mma(cur);
    // one LDS read between pairs of MFMAs, the loads up front
    __builtin_amdgcn_sched_group_barrier(0x020, 4, 0);
#pragma unroll
    for (int r = 0; r < 12; ++r) {
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);
  };
  const int nk = a.Kd / B2K;  // a multiple of 4
  bf16x8 f0[12], f1[12];
  dma(st0, 0);
  dma(st1, 1);
  dma(st2, 2);
  dma(st3, 3);
  __builtin_amdgcn_s_waitcnt(0x007c);  // vmcnt(12): this wave's loads of step 0 are in
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);
  read(f0, st0);
  for (int ks = 0; ks < nk; ks += 4) {
    step(f0, f1, st1, st0, ks);
    step(f1, f0, st2, st1, ks + 1);
    step(f0, f1, st3, st2, ks + 2);
    step(f1, f0, st0, st3, ks + 3);
  }
  // every load (also those past the end) has landed before LDS is reused
  __builtin_amdgcn_s_waitcnt(0x0070);
  __syncthreads();

  if constexpr (EPI == EPI_RESID) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = m0 + wm * 64 + 16 * i + l16;
      if (m >= a.M) continue;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int n = n0 + wn * 128 + 16 * j + 4 * g;
        if (n >= a.N) continue;
        const uint2 hv = *reinterpret_cast<const uint2*>(a.hid + static_cast<int64_t>(m) * a.Kd + n);
        float o[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float y = acc[i][j][e];
          const uint32_t hw = e < 2 ? hv.x : hv.y;
          o[e] = y / (1.0f + expf(-y)) + bf16_bits_to_f32((e & 1) ? (hw >> 16) : (hw & 0xffffu));
        }
        uint16_t* dst = a.r_out + (static_cast<int64_t>(head) * a.M + m) * a.N + n;
        *reinterpret_cast<uint2*>(dst) =
            make_uint2(f32_to_bf16_bits(o[0]) | (f32_to_bf16_bits(o[1]) << 16),
                       f32_to_bf16_bits(o[2]) | (f32_to_bf16_bits(o[3]) << 16));
      }
    }
  } else {
    // ---- the tile's per-row top-kmax, from the accumulators ---------------
    // Local row r = wm*64 + 16i + l16 is held by 8 lanes, slot sl = wn*4 + g
    // (lanes l16 + 16g of waves (wm, 0) and (wm, 1)); each holds, in
    // acc[i][j], columns wn*128 + 16j + 4g + e: 8 granules of 4 columns.
    //  1. every lane: its 8 granule maxima and the 3 largest of them
    //  2. a thread per row: T = the kmax-th largest of the row's 24 such
    //     maxima.  They are maxima of 24 distinct granules, so at least kmax
    //     values of the row reach T: every value of the row's top kmax does
    //  3. every lane appends its granules whose maximum reaches T to its
    //     row's list (an LDS counter per row)
    //  4. a thread per row moves the values >= T of those granules to the
    //     front of the same bytes and 5. ranks them into its list (larger
    //     value first, equal values by lower column, whatever order the
    //     granules arrived in).
    // On normally distributed logits a row keeps about kmax + 1 values.  A
    // row with more than FT_CAP granules reaching T (many equal logits)
    // sends the whole tile to the general epilogue further down.
    constexpr int FT_CAP = 24;                  // granules per row
    constexpr int FT_META = FT_CAP * 1024;      // granule index bytes
    constexpr int FT_COL = FT_META + FT_CAP * 64;  // column bytes of the kept values
    constexpr int FT_TAIL = B2STAGE - 512;      // the rows' thresholds, then their counters
    static_assert(FT_COL + FT_CAP * 256 <= FT_TAIL, "row lists exceed a stage buffer");
    // rows 64b .. 64b + 63 live in stage buffer b, slot-major (lanes of
    // consecutive rows touch consecutive 16-byte chunks): granule slot s of
    // row r at s * 1024 + (r & 63) * 16, its index byte at
    // FT_META + s * 64 + (r & 63), column byte of kept value k at
    // FT_COL + (k / 4) * 256 + (r & 63) * 4 + k % 4
    auto buf = [&](int b) __attribute__((always_inline)) {
      return b == 0 ? st0 : b == 1 ? st1 : b == 2 ? st2 : st3;
    };
    auto s_thr = [&](int r) __attribute__((always_inline)) -> float& {
      return *reinterpret_cast<float*>(buf(r >> 6) + FT_TAIL + (r & 63) * 4);
    };
    auto s_cnt = [&](int r) __attribute__((always_inline)) -> int& {
      return *reinterpret_cast<int*>(buf(r >> 6) + FT_TAIL + 256 + (r & 63) * 4);
    };
    __shared__ int s_over;
    if (a.logits) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int m = m0 + wm * 64 + 16 * i + l16;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int n = n0 + wn * 128 + 16 * j + 4 * g;
          if (m < a.M && n < a.N)
            *reinterpret_cast<f32x4*>(a.logits + (static_cast<int64_t>(m) * a.K + head) * a.N + n) = acc[i][j];
        }
      }
    }
    if (n0 + B2N > a.N) {  // columns past the vocabulary take no part
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j)
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (n0 + wn * 128 + 16 * j + 4 * g + e >= a.N) acc[i][j][e] = -INFINITY;
    }
    // 1.
    char* const wbuf = buf(wm);
    const int sl = wn * 4 + g;
    float gm[4][8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float t1 = -INFINITY, t2 = -INFINITY, t3 = -INFINITY;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const f32x4 v = acc[i][j];
        float x = fmaxf(fmaxf(v[0], v[1]), fmaxf(v[2], v[3]));
        x = x > -INFINITY ? x : -INFINITY;  // an all-NaN granule counts as empty
        gm[i][j] = x;
        t3 = fmaxf(t3, fminf(t2, x));
        t2 = fmaxf(t2, fminf(t1, x));
        t1 = fmaxf(t1, x);
      }
      *reinterpret_cast<f32x4*>(wbuf + sl * 1024 + (16 * i + l16) * 16) = f32x4{t1, t2, t3, -INFINITY};
    }
    if (tid < B2M) s_cnt(tid) = 0;
    if (tid == 0) s_over = 0;
    __syncthreads();
    // 2. (threads 0..255 are waves 0..3: row tid sits in buffer `wave`)
    if (tid < B2M) {
      const char* rb = buf(wave) + (tid & 63) * 16;
      float tl[KM];  // descending
#pragma unroll
      for (int s2 = 0; s2 < KM; ++s2) tl[s2] = -INFINITY;
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const f32x4 v = *reinterpret_cast<const f32x4*>(rb + q * 1024);
#pragma unroll
        for (int c = 0; c < 3; ++c) {
          const float x = v[c];
#pragma unroll
          for (int s2 = KM - 1; s2 > 0; --s2) tl[s2] = __builtin_amdgcn_fmed3f(tl[s2 - 1], tl[s2], x);
          tl[0] = fmaxf(tl[0], x);
        }
      }
      float th = -INFINITY;
#pragma unroll
      for (int s2 = 0; s2 < KM; ++s2) th = s2 == a.kmax - 1 ? tl[s2] : th;
      s_thr(tid) = fmaxf(th, -FLT_MAX);  // -inf logits (masked columns) never qualify
    }
    __syncthreads();
    // 3.
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int rl = 16 * i + l16;
      const float th = s_thr(wm * 64 + rl);
      int n = 0;
#pragma unroll
      for (int j = 0; j < 8; ++j) n += gm[i][j] >= th ? 1 : 0;
      int k = 0;
      if (n) k = atomicAdd(&s_cnt(wm * 64 + rl), n);
      if (k + n > FT_CAP) s_over = 1;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        if (gm[i][j] >= th) {
          if (k < FT_CAP) {
            *reinterpret_cast<f32x4*>(wbuf + k * 1024 + rl * 16) = acc[i][j];
            wbuf[FT_META + k * 64 + rl] = static_cast<char>(wn * 32 + 4 * j + g);
          }
          ++k;
        }
      }
    }
    __syncthreads();
    if (!s_over) {
      if (tid < B2M) {
        char* rb = buf(wave);
        const int rl = tid & 63;
        const float th = s_thr(tid);
        const int ng = s_cnt(tid);
        // 4. four granules a round, their reads issued together.  Kept value
        //    k goes to word k % 4 of granule slot k / 4, which is at most the
        //    last slot read; its column byte to byte k % 4 of word k / 4 of
        //    the column area.  Every value is written and the count moves on
        //    only for a kept one, so the next write replaces a dropped value.
        int k = 0;
        for (int s = 0; s < ng; s += 4) {
          f32x4 v[4];
          int q[4];
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            const int su = min(s + u, ng - 1);
            v[u] = *reinterpret_cast<const f32x4*>(rb + su * 1024 + rl * 16);
            q[u] = static_cast<unsigned char>(rb[FT_META + su * 64 + rl]);
          }
#pragma unroll
          for (int u = 0; u < 4; ++u) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              *reinterpret_cast<float*>(rb + (k >> 2) * 1024 + rl * 16 + 4 * (k & 3)) = v[u][e];
              rb[FT_COL + (k >> 2) * 256 + rl * 4 + (k & 3)] = static_cast<char>(4 * q[u] + e);
              k += (s + u < ng && v[u][e] >= th) ? 1 : 0;
            }
          }
        }
        // 5. 64-bit keys: the value's bits in unsigned order above the
        //    complemented column, so one unsigned compare ranks larger values
        //    first and equal values by lower column (-0 taken as +0); key 0
        //    is below every kept value
        uint64_t tk[KM];
#pragma unroll
        for (int s2 = 0; s2 < KM; ++s2) tk[s2] = 0;
        for (int c = 0; c < k; c += 4) {
          const f32x4 x4 = *reinterpret_cast<const f32x4*>(rb + (c >> 2) * 1024 + rl * 16);
          const uint32_t c4 = *reinterpret_cast<const uint32_t*>(rb + FT_COL + (c >> 2) * 256 + rl * 4);
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            const uint32_t bits = __float_as_uint(x4[u] + 0.0f);
            const uint32_t ord = (bits & 0x80000000u) ? ~bits : (bits | 0x80000000u);
            const uint32_t col = static_cast<uint32_t>(n0) + ((c4 >> (8 * u)) & 0xffu);
            uint64_t key = (static_cast<uint64_t>(ord) << 32) | static_cast<uint32_t>(~col);
            if (c + u < k && key > tk[KM - 1]) {
#pragma unroll
              for (int s2 = 0; s2 < KM; ++s2) {  // keys are distinct: no tie to break
                const bool take = key > tk[s2];
                const uint64_t o = tk[s2];
                tk[s2] = take ? key : o;
                key = take ? o : key;
              }
            }
          }
        }
        float tv[KM];
        int ti[KM];
#pragma unroll
        for (int s2 = 0; s2 < KM; ++s2) {
          const uint32_t ord = static_cast<uint32_t>(tk[s2] >> 32);
          const uint32_t bits = (ord & 0x80000000u) ? (ord & 0x7fffffffu) : ~ord;
          tv[s2] = tk[s2] ? __uint_as_float(bits) : -INFINITY;
          ti[s2] = tk[s2] ? static_cast<int>(~static_cast<uint32_t>(tk[s2])) : 0x7fffffff;
        }
        const int m = m0 + tid;
        if (m < a.M) {
          const int64_t base = ((static_cast<int64_t>(m) * a.K + head) * a.ntiles + nt) * a.kmax;
#pragma unroll
          for (int s2 = 0; s2 < KM; ++s2) {
            if (s2 < a.kmax) {
              a.cand_v[base + s2] = tv[s2];
              a.cand_i[base + s2] = ti[s2];
            }
          }
        }
      }
      return;
    }

    // ---- general epilogue (a row with many equal logits) -------------------
    // two passes of 128 rows; rows 32a .. 32a + 31 of a pass sit in stage
    // buffer a, column granule q (4 columns) of local row r at
    // (r % 32) * 1024 + 16 * (q ^ (r & 7))
    auto cell = [&](int r, int q) __attribute__((always_inline)) {
      const int b = r >> 5;
      char* base = b == 0 ? st0 : b == 1 ? st1 : b == 2 ? st2 : st3;
      return reinterpret_cast<float*>(base + (r & 31) * 1024 + 16 * (q ^ (r & 7)));
    };
#pragma unroll
    for (int pass = 0; pass < 2; ++pass) {
      if ((wm >> 1) == pass) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 8; ++j)
            *reinterpret_cast<f32x4*>(cell((wm & 1) * 64 + 16 * i + l16, wn * 32 + 4 * j + g)) = acc[i][j];
      }
      __syncthreads();
      if (a.logits) {  // 4 rows per pass of the 512 threads
        for (int rr = 0; rr < 128; rr += 8) {
          const int r = rr + (tid >> 6), q = tid & 63;
          const int m = m0 + pass * 128 + r, n = n0 + 4 * q;
          if (m < a.M && n < a.N)
            *reinterpret_cast<f32x4*>(a.logits + (static_cast<int64_t>(m) * a.K + head) * a.N + n) =
                *reinterpret_cast<const f32x4*>(cell(r, q));
        }
      }
      // 4 adjacent lanes per row, 64 columns each.  The row's bound: each
      // lane's c-th largest 8-column maximum (c = ceil(kmax / 4) <= 3), then
      // the smallest over the row's 4 lanes.  At least 4c >= kmax values of
      // the row reach it, so no value below it is among the row's kmax
      // largest; only values at or above it go through the sorted insertion
      // (most lanes hold a handful), taken in column order.
      const int r = tid >> 2, part = tid & 3;
      float g1 = -INFINITY, g2 = -INFINITY, g3 = -INFINITY;  // largest granule maxima, descending
#pragma unroll
      for (int gi = 0; gi < 8; ++gi) {
        const int qq = part * 16 + 2 * gi;
        const f32x4 v0 = *reinterpret_cast<const f32x4*>(cell(r, qq));
        const f32x4 v1 = *reinterpret_cast<const f32x4*>(cell(r, qq + 1));
        const int nb = n0 + 4 * qq;
        float gm = -INFINITY;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          gm = fmaxf(gm, nb + e < a.N ? v0[e] : -INFINITY);
          gm = fmaxf(gm, nb + 4 + e < a.N ? v1[e] : -INFINITY);
        }
        const float t1 = fmaxf(g1, gm), r1 = fminf(g1, gm);
        const float t2 = fmaxf(g2, r1), r2 = fminf(g2, r1);
        g3 = fmaxf(g3, r2);
        g2 = t2;
        g1 = t1;
      }
      const int c = (a.kmax + 3) >> 2;
      float th = c == 1 ? g1 : (c == 2 ? g2 : g3);
      th = fminf(th, __shfl_xor(th, 1));
      th = fminf(th, __shfl_xor(th, 2));
      uint32_t cand[2] = {0u, 0u};  // bit 4q + e: column 4(part*16 + q) + e reaches the bound
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        const f32x4 v = *reinterpret_cast<const f32x4*>(cell(r, part * 16 + q));
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int n = n0 + 4 * (part * 16 + q) + e;
          if (v[e] >= th && n < a.N) cand[q >> 3] |= 1u << (4 * (q & 7) + e);
        }
      }
      float tv[KM];
      int ti[KM];
#pragma unroll
      for (int s2 = 0; s2 < KM; ++s2) {
        tv[s2] = -INFINITY;
        ti[s2] = 0x7fffffff;
      }
      while (__builtin_amdgcn_ballot_w64((cand[0] | cand[1]) != 0u)) {
        if (cand[0] | cand[1]) {
          const int i = cand[0] ? __builtin_ctz(cand[0]) : 32 + __builtin_ctz(cand[1]);
          if (cand[0]) cand[0] &= cand[0] - 1u;
          else cand[1] &= cand[1] - 1u;
          const int qq = part * 16 + (i >> 2);
          const float x = cell(r, qq)[i & 3];
          if (x > tv[KM - 1]) list_insert<KM>(tv, ti, x, n0 + 4 * qq + (i & 3));
        }
      }
      // merge with the lanes of the same row (xor 1, then xor 2): the list
      // of the lower part goes first, so equal logits keep the lower column
#pragma unroll
      for (int sh = 1; sh <= 2; sh <<= 1) {
        float pv[KM];
        int pi[KM];
#pragma unroll
        for (int s2 = 0; s2 < KM; ++s2) {
          pv[s2] = __shfl_xor(tv[s2], sh);
          pi[s2] = __shfl_xor(ti[s2], sh);
        }
        if (part & sh) {  // this lane holds the later columns: start from the partner's list
#pragma unroll
          for (int s2 = 0; s2 < KM; ++s2) {
            const float t0 = tv[s2];
            const int i0 = ti[s2];
            tv[s2] = pv[s2];
            ti[s2] = pi[s2];
            pv[s2] = t0;
            pi[s2] = i0;
          }
        }
#pragma unroll
        for (int s2 = 0; s2 < KM; ++s2) {
          if (pv[s2] > tv[KM - 1]) list_insert<KM>(tv, ti, pv[s2], pi[s2]);
        }
      }
      const int m = m0 + pass * 128 + r;
      if (part == 0 && m < a.M) {
        const int64_t base = ((static_cast<int64_t>(m) * a.K + head) * a.ntiles + nt) * a.kmax;
#pragma unroll
        for (int s2 = 0; s2 < KM; ++s2) {
          if (s2 < a.kmax) {
            a.cand_v[base + s2] = tv[s2];
            a.cand_i[base + s2] = ti[s2];
          }
        }
      }
      __syncthreads();  // the next pass rewrites the buffers
    }
  }
}

// ---- final merge: each (row, head) keeps its k_d best candidates ----------
// One wave per (row m, head d).  Lanes take lists (tile candidates, sorted)
// or strided elements of a logits row into their own sorted lists; then k_d
// rounds of a wave-wide arg-max over the lanes' list heads (larger value, or
// equal value and lower index) pop the winners in order.
struct MergeArgs {
  const float* v;      // LISTS: [M][K][nlist][kmax]; ROW: [M][K][N]
  const int32_t* ix;   // LISTS only
  int M, K, nlist, kmax, N;
  const int32_t* kpd;  // [K] candidates kept by head d
  int32_t* out_idx;    // [M][K][kmax_out]
  float* out_val;      // optional, same layout
  int kmax_out;
};

template <int KM, bool LISTS>
__global__ __launch_bounds__(256) void dense_topk_merge(MergeArgs a) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);  // = m * K + d
  if (row >= a.M * a.K) return;  // whole wave: no barrier below
  const int d = row % a.K;
  float tv[KM];
  int ti[KM];
#pragma unroll
  for (int s = 0; s < KM; ++s) {
    tv[s] = -INFINITY;
    ti[s] = 0x7fffffff;
  }
  if constexpr (LISTS) {
    const float* v = a.v + static_cast<int64_t>(row) * a.nlist * a.kmax;
    const int32_t* ix = a.ix + static_cast<int64_t>(row) * a.nlist * a.kmax;
    // each list whole in registers, the next one's loads issued before this
    // one is inserted; a sorted list: once an entry stays out, so do the rest
    float xv[2][KM];
    int xi[2][KM];
    auto load = [&](int l, float (&dv)[KM], int (&di)[KM]) __attribute__((always_inline)) {
#pragma unroll
      for (int s = 0; s < KM; ++s) {
        const bool in = l < a.nlist && s < a.kmax;
        dv[s] = in ? v[l * a.kmax + s] : -INFINITY;
        di[s] = in ? ix[l * a.kmax + s] : 0x7fffffff;
      }
    };
    auto absorb = [&](const float (&dv)[KM], const int (&di)[KM]) __attribute__((always_inline)) {
#pragma unroll
      for (int s = 0; s < KM; ++s)
        if (dv[s] > tv[KM - 1]) list_insert<KM>(tv, ti, dv[s], di[s]);
    };
    load(lane, xv[0], xi[0]);
    for (int l = lane; l < a.nlist; l += 128) {
      load(l + 64, xv[1], xi[1]);
      absorb(xv[0], xi[0]);
      load(l + 128, xv[0], xi[0]);
      absorb(xv[1], xi[1]);
    }
  } else {
    const float* v = a.v + static_cast<int64_t>(row) * a.N;
    for (int n = lane; n < a.N; n += 64) {
      const float x = v[n];
      if (x > tv[KM - 1]) list_insert<KM>(tv, ti, x, n);
    }
  }
  const int kd = a.kpd[d];
  int32_t* oi = a.out_idx + static_cast<int64_t>(row) * a.kmax_out;
  float* ov = a.out_val ? a.out_val + static_cast<int64_t>(row) * a.kmax_out : nullptr;
  for (int s = 0; s < a.kmax_out; ++s) {
    float bv = tv[0];
    int bi = ti[0];
    wave_best(bv, bi);
    if (s < kd) {
      if (lane == 0) {
        oi[s] = bi;
        if (ov) ov[s] = bv;
      }
      // the lane holding the winner drops it from its list
      if (ti[0] == bi && tv[0] == bv) {
#pragma unroll
        for (int q = 0; q + 1 < KM; ++q) {
          tv[q] = tv[q + 1];
          ti[q] = ti[q + 1];
        }
        tv[KM - 1] = -INFINITY;
        ti[KM - 1] = 0x7fffffff;
      }
    } else if (lane == 0) {
      oi[s] = -1;
      if (ov) ov[s] = 0.f;
    }
  }
}

// ---- final merge of sorted tile lists: a tournament -------------------------
// One wave per (row m, head d).  The pair's tile lists (each sorted: larger
// logit first, equal logits by lower column) are copied to LDS; lane L
// follows lists L, L + 64, ... with a cursor each.  Every round takes the
// wave-wide arg-max of the lanes' best list heads (ties to the lower index),
// and only the winning list moves on, so a round costs one arg-max and one
// LDS read rather than insertions into every lane's list.
constexpr int TOURNEY_LPL = 4;  // lists per lane: up to 256 lists
__global__ __launch_bounds__(256) void dense_topk_tourney(MergeArgs a) {
  extern __shared__ __attribute__((aligned(16))) char tl_lds[];
  const int row = blockIdx.x;  // = m * K + d; the grid is M * K
  const int lane = threadIdx.x & 63;
  const int n = a.nlist * a.kmax;
  float* sv = reinterpret_cast<float*>(tl_lds);
  int* si = reinterpret_cast<int*>(tl_lds + ((n * 4 + 15) & ~15));
  const float* v = a.v + static_cast<int64_t>(row) * n;
  const int32_t* ix = a.ix + static_cast<int64_t>(row) * n;
  // All four waves stage the lists, 16 loads per lane in flight at once (the
  // lists were just written by workgroups on other XCDs, so every read is a
  // trip to memory): one round trip up to 4096 entries; then one wave
  // takes the tournament
  constexpr int U = 16;
  for (int e0 = 0; e0 < n; e0 += 256 * U) {
    float xv[U];
    int xi[U];
#pragma unroll
    for (int q = 0; q < U; ++q) {
      const int e = e0 + static_cast<int>(threadIdx.x) + 256 * q;
      xv[q] = e < n ? v[e] : 0.f;
      xi[q] = e < n ? ix[e] : 0;
    }
#pragma unroll
    for (int q = 0; q < U; ++q) {
      const int e = e0 + static_cast<int>(threadIdx.x) + 256 * q;
      if (e < n) {
        sv[e] = xv[q];
        si[e] = xi[q];
      }
    }
  }
  __syncthreads();
  if (threadIdx.x >= 64) return;  // one wave takes the tournament
  float hv[TOURNEY_LPL];
  int hi[TOURNEY_LPL], cur[TOURNEY_LPL];
#pragma unroll
  for (int u = 0; u < TOURNEY_LPL; ++u) {
    const int l = lane + 64 * u;
    const bool in = l < a.nlist;
    const int e = in ? l * a.kmax : 0;  // every read in range
    cur[u] = 0;
    hv[u] = in ? sv[e] : -INFINITY;
    hi[u] = in ? si[e] : 0x7fffffff;
  }
  const int kd = a.kpd[row % a.K];
  int32_t* oi = a.out_idx + static_cast<int64_t>(row) * a.kmax_out;
  float* ov = a.out_val ? a.out_val + static_cast<int64_t>(row) * a.kmax_out : nullptr;
  for (int s = 0; s < a.kmax_out; ++s) {
    if (s >= kd) {
      if (lane == 0) {
        oi[s] = -1;
        if (ov) ov[s] = 0.f;
      }
      continue;
    }
    float bv = hv[0];
    int bi = hi[0];
#pragma unroll
    for (int u = 1; u < TOURNEY_LPL; ++u) best_of(bv, bi, hv[u], hi[u]);
    wave_best(bv, bi);
    if (lane == 0) {
      oi[s] = bi;
      if (ov) ov[s] = bv;
    }
#pragma unroll
    for (int u = 0; u < TOURNEY_LPL; ++u) {
      if (hv[u] == bv && hi[u] == bi) {  // indices are distinct: one list moves on
        const int l = lane + 64 * u;
        const bool more = l < a.nlist && ++cur[u] < a.kmax;
        const int e = more ? l * a.kmax + cur[u] : 0;
        hv[u] = more ? sv[e] : -INFINITY;
        hi[u] = more ? si[e] : 0x7fffffff;
      }
    }
  }
}

// ---- fp32: plain VALU products (small configurations) ---------------------
struct DenseF32Args {
  const float* x;  // [M][H] hidden, or r [K][M][H]
  int64_t x_hstride;
  const float* w;  // [K][N][H]
  int64_t w_hstride;
  int M, N, H, K;
  const float* hid;  // residual: [M][H]
  float* out;        // residual: r [K][M][N]; logits: [M][K][N]
  bool resid;
};

__global__ __launch_bounds__(256) void dense_f32(DenseF32Args a) {
  const int64_t t = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  const int64_t total = static_cast<int64_t>(a.K) * a.M * a.N;
  if (t >= total) return;
  const int n = static_cast<int>(t % a.N);
  const int m = static_cast<int>((t / a.N) % a.M);
  const int h = static_cast<int>(t / (static_cast<int64_t>(a.N) * a.M));
  const float* x = a.x + h * a.x_hstride + static_cast<int64_t>(m) * a.H;
  const float* w = a.w + h * a.w_hstride + static_cast<int64_t>(n) * a.H;
  float acc = 0.f;
  for (int k = 0; k < a.H; ++k) acc = fmaf(w[k], x[k], acc);
  if (a.resid) {
    a.out[(static_cast<int64_t>(h) * a.M + m) * a.N + n] =
        acc / (1.0f + expf(-acc)) + a.hid[static_cast<int64_t>(m) * a.H + n];
  } else {
    a.out[(static_cast<int64_t>(m) * a.K + h) * a.N + n] = acc;
  }
}

// ---- host -------------------------------------------------------------------
int km_for(int kmax) { return kmax <= 4 ? 4 : kmax <= 8 ? 8 : kmax <= 12 ? 12 : kmax <= 16 ? 16 : 32; }

struct DensePlan {
  int BM, mtiles, ntiles, KM;
  bool big;  // 256 x 256 tiles with direct-to-LDS loads
  size_t r_bytes, cand_off, cand_v_bytes, cand_i_off, ws_bytes;
};

DensePlan dense_plan(int M, int H, int V, int K, int kmax, medusa_dtype_t dt) {
  DensePlan p{};
  p.KM = km_for(kmax);
  if (dt == MEDUSA_BF16) {
    // 256 x 256 tiles for large M; their epilogue keeps the accumulators of
    // the second row half live while the first is ranked, which leaves room
    // for lists of up to 12 entries without spilling
    p.big = M > 128 && p.KM <= 12;
    p.BM = p.big ? B2M : M <= 64 ? 64 : 128;
    p.mtiles = (M + p.BM - 1) / p.BM;
    p.ntiles = (V + (p.big ? B2N : BN) - 1) / (p.big ? B2N : BN);
    p.r_bytes = round_up(static_cast<size_t>(K) * M * H * 2, 256);
    p.cand_off = p.r_bytes;
    p.cand_v_bytes = round_up(static_cast<size_t>(M) * K * p.ntiles * kmax * 4, 256);
    p.cand_i_off = p.cand_off + p.cand_v_bytes;
    p.ws_bytes = p.cand_i_off + p.cand_v_bytes;
  } else {
    p.r_bytes = round_up(static_cast<size_t>(K) * M * H * 4, 256);
    p.cand_off = p.r_bytes;  // logits [M][K][V] fp32
    p.ws_bytes = p.cand_off + round_up(static_cast<size_t>(M) * K * V * 4, 256);
  }
  return p;
}

// LDS: the two staging buffers, then (vocab projection) the fp32 tile and
// the per-thread candidate lists, each reusing the same bytes
template <int BM, int EPI, int KM, int BNT = BN>
constexpr int dense_lds() {
  constexpr int stage = 2 * (BM + BNT) * TROW;
  constexpr int tile = EPI == EPI_TOPK ? BM * BN * 4 : 0;
  constexpr int lists = EPI == EPI_TOPK ? 2 * 256 * KM * 4 : 0;
  return stage > tile ? (stage > lists ? stage : lists) : (tile > lists ? tile : lists);
}

template <int BM, int EPI, int KM, int BNT = BN, int KG = 1>
int launch_gemm(const DenseArgs& a, hipStream_t s, const char* what) {
  constexpr int lds = KG * dense_lds<BM, EPI, KM, BNT>();
  static_assert(lds <= 64 * 1024, "dense heads LDS above the default limit");
  const int grid = 8 * a.per_xcd;
  hipLaunchKernelGGL((dense_gemm_bf16<BM, EPI, KM, BNT, KG>), dim3(grid), dim3(256 * KG), lds, s, a);
  return check_launch(what);
}

template <int BM, int KM>
int launch_topk_gemm(const DenseArgs& a, hipStream_t s) {
  return launch_gemm<BM, EPI_TOPK, KM>(a, s, "dense heads vocab projection");
}

int launch_topk_bm(const DenseArgs& a, int BM, int KM, hipStream_t s) {
#define MEDUSA_DENSE_KM(BMv)                                   \
  switch (KM) {                                                \
    case 4: return launch_topk_gemm<BMv, 4>(a, s);             \
    case 8: return launch_topk_gemm<BMv, 8>(a, s);             \
    case 12: return launch_topk_gemm<BMv, 12>(a, s);           \
    case 16: return launch_topk_gemm<BMv, 16>(a, s);           \
    default: return launch_topk_gemm<BMv, 32>(a, s);           \
  }
  if (BM == 64) {
    MEDUSA_DENSE_KM(64)
  }
  MEDUSA_DENSE_KM(128)
#undef MEDUSA_DENSE_KM
}

template <int EPI, int KM>
int launch_big(const DenseArgs& a, hipStream_t s, const char* what) {
  hipLaunchKernelGGL((dense_gemm_big<EPI, KM>), dim3(8 * a.per_xcd), dim3(512), 0, s, a);
  return check_launch(what);
}

int launch_topk_big(const DenseArgs& a, int KM, hipStream_t s) {
  const char* what = "dense heads vocab projection (256 x 256 tiles)";
  switch (KM) {  // the plan keeps KM <= 12 here
    case 4: return launch_big<EPI_TOPK, 4>(a, s, what);
    case 8: return launch_big<EPI_TOPK, 8>(a, s, what);
    default: return launch_big<EPI_TOPK, 12>(a, s, what);
  }
}

size_t tourney_lds(const MergeArgs& a) {
  const size_t n = static_cast<size_t>(a.nlist) * a.kmax;
  return round_up(n * 4, 16) + n * 4;
}

template <bool LISTS>
int launch_merge(const MergeArgs& a, int KM, hipStream_t s) {
  if (LISTS && a.nlist <= 64 * TOURNEY_LPL && tourney_lds(a) <= 64 * 1024) {
    const dim3 grid(static_cast<unsigned>(static_cast<int64_t>(a.M) * a.K));
    hipLaunchKernelGGL(dense_topk_tourney, grid, dim3(256), tourney_lds(a), s, a);
    return check_launch("dense heads top-k merge");
  }
  const dim3 grid(static_cast<unsigned>((static_cast<int64_t>(a.M) * a.K + 3) / 4));
  switch (KM) {
    case 4: hipLaunchKernelGGL((dense_topk_merge<4, LISTS>), grid, dim3(256), 0, s, a); break;
    case 8: hipLaunchKernelGGL((dense_topk_merge<8, LISTS>), grid, dim3(256), 0, s, a); break;
    case 12: hipLaunchKernelGGL((dense_topk_merge<12, LISTS>), grid, dim3(256), 0, s, a); break;
    case 16: hipLaunchKernelGGL((dense_topk_merge<16, LISTS>), grid, dim3(256), 0, s, a); break;
    default: hipLaunchKernelGGL((dense_topk_merge<32, LISTS>), grid, dim3(256), 0, s, a); break;
  }
  return check_launch("dense heads top-k merge");
}

}  // namespace

extern "C" size_t medusa_heads_dense_workspace_size(int M, int H, int V, int K,
                                                    const medusa_tree_t* tree, medusa_dtype_t dt) {
  if (!tree || M < 1 || H < 1 || V < 1 || K < 1) return 0;
  if (dt != MEDUSA_F32 && dt != MEDUSA_BF16) return 0;
  return dense_plan(M, H, V, K, tree->kmax, dt).ws_bytes;
}

extern "C" int medusa_heads_dense(const void* hidden, const void* w1, int64_t w1_head_stride,
                                  const void* wlm, int64_t wlm_head_stride, int M, int H, int V,
                                  int K, const medusa_tree_t* tree, medusa_dtype_t dt,
                                  int32_t* topk_idx, float* topk_val, float* logits, void* ws,
                                  size_t ws_bytes, hipStream_t stream) {
  clear_error();
  int rc = check_tree(tree);
  if (rc) return rc;
  MEDUSA_CHECK_ARG(hidden && w1 && wlm && topk_idx, "hidden, w1, wlm and topk_idx must be non-NULL");
  MEDUSA_CHECK_ARG(M >= 1 && H >= 1, "M=%d, H=%d must be >= 1", M, H);
  MEDUSA_CHECK_ARG(K == tree->K, "K=%d must equal the tree's head count %d", K, tree->K);
  MEDUSA_CHECK_ARG(V >= tree->kmax, "V=%d smaller than the largest top-k %d", V, tree->kmax);
  MEDUSA_CHECK_ARG(dt == MEDUSA_F32 || dt == MEDUSA_BF16, "unknown dtype %d", static_cast<int>(dt));
  MEDUSA_CHECK_ARG(K == 1 || w1_head_stride >= static_cast<int64_t>(H) * H,
                   "w1_head_stride=%lld smaller than H*H", static_cast<long long>(w1_head_stride));
  MEDUSA_CHECK_ARG(wlm_head_stride == 0 || wlm_head_stride >= static_cast<int64_t>(V) * H,
                   "wlm_head_stride=%lld must be 0 (shared) or >= V*H",
                   static_cast<long long>(wlm_head_stride));
  MEDUSA_CHECK_ARG(aligned16(hidden) && aligned16(w1) && aligned16(wlm) && aligned16(topk_idx) &&
                       aligned16(topk_val) && aligned16(logits),
                   "pointers must be 16-byte aligned");
  const DensePlan p = dense_plan(M, H, V, K, tree->kmax, dt);
  if (!ws || ws_bytes < p.ws_bytes || !aligned256(ws)) {
    set_error("dense heads workspace: need %zu bytes, 256-byte aligned (got %zu at %p)", p.ws_bytes,
              ws_bytes, ws);
    return MEDUSA_EWORKSPACE;
  }
  char* w = static_cast<char*>(ws);
  MergeArgs mg{};
  mg.M = M;
  mg.K = K;
  mg.kmax = tree->kmax;
  mg.kpd = tree->d_kpd;
  mg.out_idx = topk_idx;
  mg.out_val = topk_val;
  mg.kmax_out = tree->kmax;
  if (dt == MEDUSA_F32) {
    DenseF32Args f{};
    f.x = static_cast<const float*>(hidden);
    f.x_hstride = 0;
    f.w = static_cast<const float*>(w1);
    f.w_hstride = w1_head_stride;
    f.M = M;
    f.N = H;
    f.H = H;
    f.K = K;
    f.hid = static_cast<const float*>(hidden);
    f.out = reinterpret_cast<float*>(w);
    f.resid = true;
    int64_t total = static_cast<int64_t>(K) * M * H;
    hipLaunchKernelGGL(dense_f32, dim3(static_cast<unsigned>((total + 255) / 256)), dim3(256), 0, stream, f);
    if ((rc = check_launch("dense heads residual block (f32)"))) return rc;
    float* lg = logits ? logits : reinterpret_cast<float*>(w + p.cand_off);
    f.x = reinterpret_cast<const float*>(w);
    f.x_hstride = static_cast<int64_t>(M) * H;
    f.w = static_cast<const float*>(wlm);
    f.w_hstride = wlm_head_stride;
    f.N = V;
    f.out = lg;
    f.resid = false;
    total = static_cast<int64_t>(K) * M * V;
    hipLaunchKernelGGL(dense_f32, dim3(static_cast<unsigned>((total + 255) / 256)), dim3(256), 0, stream, f);
    if ((rc = check_launch("dense heads vocab projection (f32)"))) return rc;
    mg.v = lg;
    mg.N = V;
    return launch_merge<false>(mg, p.KM, stream);
  }
  MEDUSA_CHECK_ARG(H % 128 == 0, "bf16 dense heads need H %% 128 == 0 (H=%d)", H);
  MEDUSA_CHECK_ARG(V % 4 == 0, "bf16 dense heads need V %% 4 == 0 (V=%d)", V);
  MEDUSA_CHECK_ARG(w1_head_stride % 8 == 0 && wlm_head_stride % 8 == 0,
                   "bf16 head strides must be multiples of 8 elements");
  MEDUSA_CHECK_ARG(static_cast<int64_t>(BN) * H * 2 < (1ll << 31) && static_cast<int64_t>(p.BM) * H * 2 < (1ll << 31),
                   "H=%d too large (tile byte offsets are 32-bit)", H);
  DenseArgs a{};
  a.M = M;
  a.Kd = H;
  a.K = K;
  a.kmax = tree->kmax;
  a.mtiles = p.mtiles;
  // stage 1: r = bf16(SiLU(W1 h) + h) for every head, into the workspace
  a.x = static_cast<const uint16_t*>(hidden);
  a.x_hstride = 0;
  a.w = static_cast<const uint16_t*>(w1);
  a.w_hstride = w1_head_stride;
  a.N = H;
  // (64-column tiles on the small-tile path: at H = 4096 the 128-column ones
  // give too few workgroups to fill the chip)
  constexpr int RBN = 64;
  a.ntiles = p.big ? (H + B2N - 1) / B2N : (H + RBN - 1) / RBN;
  a.tasks = p.mtiles * a.ntiles * K;
  // 256 x 256 tiles only while they make at least 128 workgroups: at
  // vicuna13b-shaped (M = 256, 100 of them) 128 x 64 tiles are faster (dense
  // heads 714 -> 688 us), at zephyr7b-shaped (M = 512, 160) slower (759 -> 781)
  const bool big_resid = p.big && a.tasks >= 128;
  if (p.big && !big_resid) {
    a.mtiles = (M + 127) / 128;
    a.ntiles = (H + RBN - 1) / RBN;
    a.tasks = a.mtiles * a.ntiles * K;
  }
  a.per_xcd = (a.tasks + 7) / 8;
  a.hid = static_cast<const uint16_t*>(hidden);
  a.r_out = reinterpret_cast<uint16_t*>(w);
  if (big_resid) rc = launch_big<EPI_RESID, 4>(a, stream, "dense heads residual block (256 x 256 tiles)");
  else if (p.big) rc = launch_gemm<128, EPI_RESID, 4, RBN>(a, stream, "dense heads residual block");
  else if (p.BM == 64 && (H / BK) % 4 == 0)  // two k-groups: each an even number of k-steps
    rc = launch_gemm<64, EPI_RESID, 4, RBN, 2>(a, stream, "dense heads residual block");
  else if (p.BM == 64) rc = launch_gemm<64, EPI_RESID, 4, RBN>(a, stream, "dense heads residual block");
  else rc = launch_gemm<128, EPI_RESID, 4, RBN>(a, stream, "dense heads residual block");
  if (rc) return rc;
  // stage 2: logits tiles of every head and their per-tile top-kmax
  a.mtiles = p.mtiles;
  DenseArgs b = a;
  b.x = reinterpret_cast<const uint16_t*>(w);
  b.x_hstride = static_cast<int64_t>(M) * H;
  b.w = static_cast<const uint16_t*>(wlm);
  b.w_hstride = wlm_head_stride;
  b.N = V;
  b.ntiles = p.ntiles;
  b.tasks = p.mtiles * p.ntiles * K;
  b.per_xcd = (b.tasks + 7) / 8;
  b.cand_v = reinterpret_cast<float*>(w + p.cand_off);
  b.cand_i = reinterpret_cast<int32_t*>(w + p.cand_i_off);
  b.logits = logits;
  rc = p.big ? launch_topk_big(b, p.KM, stream) : launch_topk_bm(b, p.BM, p.KM, stream);
  if (rc) return rc;
  mg.v = b.cand_v;
  mg.ix = b.cand_i;
  mg.nlist = p.ntiles;
  return launch_merge<true>(mg, p.KM, stream);
}
