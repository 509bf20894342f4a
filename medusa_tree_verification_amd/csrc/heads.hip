// Medusa heads: r = SiLU(W1 h) + h, logits = W_lm r.
//
// P1 ("Medusa 심층 아키텍처"), section "Medusa의 핵심 철학 ... 잔차 블록을 포함한
// Medusa 헤드 구조" gives the two equations; its sketch code fixes bias-free
// [out, in] projections and the residual add.  Both projections are weight
// streams with a handful of activation rows (M = batch), so each is a
// "skinny" product Y[n][r] = sum_k W[r][k] X[n][k] whose cost is reading W
// from HBM once.
//
// bf16 design (gfx950): one workgroup owns 16 consecutive weight rows; its 4
// waves split the k range (wave w streams chunks w, w+4, ...) and add their
// partial sums through LDS in wave order at the end (deterministic).  A chunk
// is 8 (one column tile) or 4 MFMA k-steps of 32 elements: lane l (row l%16,
// group q = l/16) loads the 8 elements at 8q + 32j of k-step j, so one load
// instruction covers 64 contiguous bytes of each of the 16 rows and the
// lane's elements sit exactly in the k-slots v_mfma_f32_16x16x32_bf16 wants
// (weights as the A operand, activation rows as B, up to 16 columns per tile,
// zero-padded).  The activation rows are staged once per workgroup in LDS
// when they fit, so the vector memory pipe carries only weights.  Two chunks
// are kept in flight per wave (register double buffer).  The MFMA work is far
// below the matrix-core peak; the point is that it costs almost no VALU issue
// slots, so the waves spend their time keeping loads in flight.
#include "internal.h"

using namespace medusa;
using namespace medusa::dev;

namespace {

enum { EPI_RESID = 1, EPI_LOGITS = 2 };

__host__ __device__ constexpr int round_up16(int x) { return (x + 15) & ~15; }

struct GemmArgs {
  const uint16_t* W;  // group g: W + g*w_gstride, [R][Kd]
  int64_t w_gstride;
  const uint16_t* X;  // group g: X + g*x_gstride, [N][Kd]
  int64_t x_gstride;
  int R, Kd, N;
  // EPI_RESID: out_r[g*N*R + n*R + r] = bf16(silu(acc) + hid[n*R + r])
  const uint16_t* hid;
  uint16_t* out_r;
  // EPI_LOGITS: logits[(n % M)*stride_m + (g + n / M)*V + r] = acc
  float* logits;
  int M;
  int64_t stride_m;
  int V;
};

template <int CH>
struct Chunk {
  uint4 v[CH];
};

// piece j of a lane's chunk: 8 elements at p + 32*j (lane group q = l/16 starts
// at 8q, so one load instruction covers 64 contiguous bytes of each of the 16
// rows); avail = elements of the row from p onward
template <int CH>
__device__ __forceinline__ void load_chunk(Chunk<CH>& c, const uint16_t* p, int avail) {
#pragma unroll
  for (int j = 0; j < CH; ++j) {
    if (32 * j + 8 <= avail)
      c.v[j] = *reinterpret_cast<const uint4*>(p + 32 * j);
    else
      c.v[j] = make_uint4(0, 0, 0, 0);
  }
}

template <int RT, int NT, int CH>
__device__ __forceinline__ void mfma_chunk(f32x4 (&acc)[RT][NT], const Chunk<CH> (&w)[RT],
                                           const Chunk<CH> (&x)[NT]) {
#pragma unroll
  for (int j = 0; j < CH; ++j) {
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
      for (int t = 0; t < NT; ++t)
        acc[rt][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(w[rt].v[j]), as_bf16x8(x[t].v[j]),
                                                              acc[rt][t], 0, 0, 0);
  }
}

constexpr int XPAD = 8;              // LDS row padding of the staged activations (elements)
constexpr int XLDS_MAX = 64 * 1024;  // largest activation block staged in LDS (more costs occupancy)

// grid: (ceil(R/(16 RT)), G, passes); block: 256 (4 waves on the same 16 RT
// rows).  RT = 2 when the activation rows come from L2 (too large to stage):
// each of their loads then serves 32 weight rows instead of 16.
template <int NT, int EPI, bool XLDS, int RT = 1>
__global__ __launch_bounds__(256) void skinny_gemm_bf16(GemmArgs a) {
  constexpr int CH = (NT == 1 && RT == 1) ? 8 : 4;  // MFMA k-steps (16-byte loads per lane) per chunk
  constexpr int STEP = 32 * CH;                     // elements per chunk
  extern __shared__ __attribute__((aligned(16))) char smem[];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int g = blockIdx.y;
  const int n0 = blockIdx.z * NT * 16;
  const int row0 = blockIdx.x * 16 * RT;
  const int nl = min(NT * 16, a.N - n0);  // activation rows of this pass
  const int kq = (lane >> 4) * 8;
  const uint16_t* wp[RT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const int rl = min(row0 + 16 * rt + (lane & 15), a.R - 1);
    wp[rt] = a.W + g * a.w_gstride + static_cast<int64_t>(rl) * a.Kd + kq;
  }
  const uint16_t* xg = a.X + g * a.x_gstride + static_cast<int64_t>(n0) * a.Kd;
  const int xrow = a.Kd + XPAD;
  uint16_t* sx = reinterpret_cast<uint16_t*>(smem);
  if constexpr (XLDS) {
    // stage the activation rows n0 .. n0+nl-1 (16-byte pieces, Kd % 8 == 0)
    const int pieces = nl * (a.Kd / 8);
    for (int i = threadIdx.x; i < pieces; i += 256) {
      const int n = i / (a.Kd / 8), k = (i % (a.Kd / 8)) * 8;
      *reinterpret_cast<uint4*>(sx + n * xrow + k) =
          *reinterpret_cast<const uint4*>(xg + static_cast<int64_t>(n) * a.Kd + k);
    }
    __syncthreads();
  }
  int xo[NT];  // this lane's activation row (offset), -1 beyond N
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const int n = t * 16 + (lane & 15);
    xo[t] = n < nl ? (XLDS ? n * xrow : n * a.Kd) + kq : -1;
  }
  f32x4 acc[RT][NT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt)
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[rt][t] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int nchunks = (a.Kd + STEP - 1) / STEP;
  Chunk<CH> wa[RT], wb[RT], xa[NT], xb[NT];
  auto load = [&](Chunk<CH>(&w)[RT], Chunk<CH>(&x)[NT], int c) __attribute__((always_inline)) {
    const int avail = a.Kd - c * STEP - kq;
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) load_chunk<CH>(w[rt], wp[rt] + static_cast<int64_t>(c) * STEP, avail);
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      if (xo[t] < 0) {
#pragma unroll
        for (int j = 0; j < CH; ++j) x[t].v[j] = make_uint4(0, 0, 0, 0);
      } else if constexpr (XLDS) {
#pragma unroll
        for (int j = 0; j < CH; ++j)
          x[t].v[j] = (32 * j + 8 <= avail) ? *reinterpret_cast<const uint4*>(sx + xo[t] + c * STEP + 32 * j)
                                            : make_uint4(0, 0, 0, 0);
      } else {
        load_chunk<CH>(x[t], xg + xo[t] + static_cast<int64_t>(c) * STEP, avail);
      }
    }
  };
  // this wave's chunks: wave, wave + 4, ...
  int c = wave;
  if (c < nchunks) load(wa, xa, c);
  for (; c + 4 < nchunks; c += 8) {
    load(wb, xb, c + 4);
    mfma_chunk<RT, NT, CH>(acc, wa, xa);
    if (c + 8 < nchunks) load(wa, xa, c + 8);
    mfma_chunk<RT, NT, CH>(acc, wb, xb);
  }
  if (c < nchunks) mfma_chunk<RT, NT, CH>(acc, wa, xa);

  // waves 1-3 hand their partial sums to wave 0 (added in wave order)
  f32x4* red = reinterpret_cast<f32x4*>(smem + (XLDS ? round_up16(nl * xrow * 2) : 0));
  if (wave > 0) {
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
      for (int t = 0; t < NT; ++t) red[(((wave - 1) * RT + rt) * NT + t) * 64 + lane] = acc[rt][t];
  }
  __syncthreads();
  if (wave > 0) return;
#pragma unroll
  for (int w = 0; w < 3; ++w)
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
      for (int t = 0; t < NT; ++t) acc[rt][t] += red[((w * RT + rt) * NT + t) * 64 + lane];

  // C layout: lane holds column (lane & 15) and rows 4*(lane >> 4) + e of
  // each 16-row tile
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const int rbase = row0 + 16 * rt + 4 * (lane >> 4);
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const int n = n0 + t * 16 + (lane & 15);
      if (n >= a.N) continue;
      if (EPI == EPI_RESID) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          int r = rbase + e;
          if (r >= a.R) break;
          float y = acc[rt][t][e];
          float s = y / (1.0f + expf(-y));
          float h = bf16_bits_to_f32(a.hid[static_cast<int64_t>(n) * a.R + r]);
          a.out_r[static_cast<int64_t>(g) * a.N * a.R + static_cast<int64_t>(n) * a.R + r] =
              static_cast<uint16_t>(f32_to_bf16_bits(s + h));
        }
      } else {
        float* dst = a.logits + static_cast<int64_t>(n % a.M) * a.stride_m +
                     static_cast<int64_t>(g + n / a.M) * a.V + rbase;
        if (rbase + 3 < a.R && (reinterpret_cast<uintptr_t>(dst) & 15) == 0) {
          *reinterpret_cast<float4*>(dst) =
              make_float4(acc[rt][t][0], acc[rt][t][1], acc[rt][t][2], acc[rt][t][3]);
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (rbase + e < a.R) dst[e] = acc[rt][t][e];
        }
      }
    }
  }
}

// ---- fp32 path (small configurations): one wave per output row ----------
struct GemvF32Args {
  const float* W;
  int64_t w_gstride;
  const float* X;
  int64_t x_gstride;
  int R, Kd, N;
  const float* hid;
  float* out_r;
  float* logits;
  int M;
  int64_t stride_m;
  int V;
};

// grid: (ceil(R/4), G, ceil(N/16)); block 256
template <int EPI>
__global__ __launch_bounds__(256) void gemv_f32(GemvF32Args a) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int g = blockIdx.y;
  const int n0 = blockIdx.z * 16;
  if (row >= a.R) return;
  const float* w = a.W + g * a.w_gstride + static_cast<int64_t>(row) * a.Kd;
  const float* x = a.X + g * a.x_gstride;
  float acc[16];
#pragma unroll
  for (int j = 0; j < 16; ++j) acc[j] = 0.f;
  for (int k = lane; k < a.Kd; k += 64) {
    float wk = w[k];
#pragma unroll
    for (int j = 0; j < 16; ++j)
      if (n0 + j < a.N) acc[j] = fmaf(wk, x[static_cast<int64_t>(n0 + j) * a.Kd + k], acc[j]);
  }
#pragma unroll
  for (int j = 0; j < 16; ++j) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) acc[j] += __shfl_xor(acc[j], off, 64);
  }
  if (lane < 16) {
    const int n = n0 + lane;
    float y = 0.f;
#pragma unroll
    for (int j = 0; j < 16; ++j)
      if (j == lane) y = acc[j];
    if (n < a.N) {
      if (EPI == EPI_RESID) {
        float s = y / (1.0f + expf(-y));
        a.out_r[static_cast<int64_t>(g) * a.N * a.R + static_cast<int64_t>(n) * a.R + row] =
            s + a.hid[static_cast<int64_t>(n) * a.R + row];
      } else {
        a.logits[static_cast<int64_t>(n % a.M) * a.stride_m +
                 static_cast<int64_t>(g + n / a.M) * a.V + row] = y;
      }
    }
  }
}

template <int NT, int EPI>
int launch_nt(const GemmArgs& a, int G, hipStream_t s) {
  const dim3 grid((a.R + 15) / 16, G, (a.N + NT * 16 - 1) / (NT * 16));
  const int nl = a.N < NT * 16 ? a.N : NT * 16;
  const int xbytes = static_cast<int>(round_up(static_cast<size_t>(nl) * (a.Kd + XPAD) * 2, 16));
  const int red = 3 * NT * 64 * 16;
  if (xbytes <= XLDS_MAX) {
    const int lds = xbytes + red;
    if (lds > 64 * 1024) {
      static int allowed = 0;
      if (lds > allowed) {
        if (hipFuncSetAttribute(reinterpret_cast<const void*>(&skinny_gemm_bf16<NT, EPI, true>),
                                hipFuncAttributeMaxDynamicSharedMemorySize, lds) != hipSuccess) {
          (void)hipGetLastError();
          set_error("cannot allow %d bytes of dynamic LDS for the heads GEMM", lds);
          return MEDUSA_EUNSUPPORTED;
        }
        allowed = lds;
      }
    }
    hipLaunchKernelGGL((skinny_gemm_bf16<NT, EPI, true>), grid, dim3(256), lds, s, a);
  } else if constexpr (NT <= 2) {
    // activation rows from L2: two 16-row weight tiles per workgroup (with
    // more column tiles the registers would not hold two)
    const dim3 grid2((a.R + 31) / 32, G, grid.z);
    hipLaunchKernelGGL((skinny_gemm_bf16<NT, EPI, false, 2>), grid2, dim3(256), 2 * red, s, a);
  } else {
    hipLaunchKernelGGL((skinny_gemm_bf16<NT, EPI, false>), grid, dim3(256), red, s, a);
  }
  return check_launch(EPI == EPI_RESID ? "heads residual block (bf16)" : "heads vocab projection (bf16)");
}

template <int EPI>
int launch_bf16(const GemmArgs& a, int G, hipStream_t s) {
  int nt = (a.N + 15) / 16;
  if (nt > 4) nt = 4;
  switch (nt) {
    case 1: return launch_nt<1, EPI>(a, G, s);
    case 2: return launch_nt<2, EPI>(a, G, s);
    case 3: return launch_nt<3, EPI>(a, G, s);
    default: return launch_nt<4, EPI>(a, G, s);
  }
}

template <int EPI>
int launch_f32(const GemvF32Args& a, int G, hipStream_t s) {
  dim3 grid((a.R + 3) / 4, G, (a.N + 15) / 16);
  hipLaunchKernelGGL((gemv_f32<EPI>), grid, dim3(256), 0, s, a);
  return check_launch(EPI == EPI_RESID ? "heads residual block (f32)" : "heads vocab projection (f32)");
}

}  // namespace

extern "C" size_t medusa_heads_workspace_size(int M, int H, int K, medusa_dtype_t dt) {
  if (M <= 0 || H <= 0 || K <= 0) return 0;
  size_t e = (dt == MEDUSA_F32) ? 4 : 2;
  return round_up(static_cast<size_t>(K) * M * H * e, 256);
}

extern "C" int medusa_heads(const void* hidden, const void* w1, int64_t w1_head_stride,
                            const void* wlm, int64_t wlm_head_stride, int M, int H, int V, int K,
                            medusa_dtype_t dt, float* logits, void* ws, size_t ws_bytes,
                            hipStream_t stream) {
  clear_error();
  MEDUSA_CHECK_ARG(hidden && w1 && wlm && logits, "hidden, w1, wlm and logits must be non-NULL");
  MEDUSA_CHECK_ARG(M >= 1 && H >= 1 && V >= 1, "M=%d, H=%d, V=%d must be >= 1", M, H, V);
  MEDUSA_CHECK_ARG(K >= 1 && K <= MEDUSA_MAX_HEADS, "K=%d outside 1..%d", K, MEDUSA_MAX_HEADS);
  MEDUSA_CHECK_ARG(dt == MEDUSA_F32 || dt == MEDUSA_BF16, "unknown dtype %d", static_cast<int>(dt));
  MEDUSA_CHECK_ARG(K == 1 || w1_head_stride >= static_cast<int64_t>(H) * H,
                   "w1_head_stride=%lld smaller than H*H", static_cast<long long>(w1_head_stride));
  MEDUSA_CHECK_ARG(wlm_head_stride == 0 || wlm_head_stride >= static_cast<int64_t>(V) * H,
                   "wlm_head_stride=%lld must be 0 (shared) or >= V*H",
                   static_cast<long long>(wlm_head_stride));
  if (dt == MEDUSA_BF16) {
    MEDUSA_CHECK_ARG(H % 8 == 0, "bf16 heads need H %% 8 == 0 (H=%d)", H);
    MEDUSA_CHECK_ARG(w1_head_stride % 8 == 0 && wlm_head_stride % 8 == 0,
                     "bf16 head strides must be multiples of 8 elements");
  }
  MEDUSA_CHECK_ARG(aligned16(hidden) && aligned16(w1) && aligned16(wlm) && aligned16(logits),
                   "tensor pointers must be 16-byte aligned");
  const size_t need = medusa_heads_workspace_size(M, H, K, dt);
  if (!ws || ws_bytes < need || !aligned256(ws)) {
    set_error("heads workspace: need %zu bytes, 256-byte aligned (got %zu at %p)", need, ws_bytes, ws);
    return MEDUSA_EWORKSPACE;
  }
  const bool shared = wlm_head_stride == 0;
  if (dt == MEDUSA_BF16) {
    GemmArgs a{};
    // stage 1: per head, rows = H, X = hidden shared by all heads
    a.W = static_cast<const uint16_t*>(w1);
    a.w_gstride = w1_head_stride;
    a.X = static_cast<const uint16_t*>(hidden);
    a.x_gstride = 0;
    a.R = H;
    a.Kd = H;
    a.N = M;
    a.hid = static_cast<const uint16_t*>(hidden);
    a.out_r = static_cast<uint16_t*>(ws);
    int rc = launch_bf16<EPI_RESID>(a, K, stream);
    if (rc) return rc;
    // stage 2: vocab projection of r
    GemmArgs b{};
    b.W = static_cast<const uint16_t*>(wlm);
    b.w_gstride = wlm_head_stride;
    b.X = static_cast<const uint16_t*>(ws);
    b.R = V;
    b.Kd = H;
    b.logits = logits;
    b.M = M;
    b.stride_m = static_cast<int64_t>(K) * V;
    b.V = V;
    if (shared) {
      b.x_gstride = 0;
      b.N = K * M;  // columns k*M + m: every head's r against the one matrix
      return launch_bf16<EPI_LOGITS>(b, 1, stream);
    }
    b.x_gstride = static_cast<int64_t>(M) * H;
    b.N = M;
    return launch_bf16<EPI_LOGITS>(b, K, stream);
  }
  GemvF32Args a{};
  a.W = static_cast<const float*>(w1);
  a.w_gstride = w1_head_stride;
  a.X = static_cast<const float*>(hidden);
  a.x_gstride = 0;
  a.R = H;
  a.Kd = H;
  a.N = M;
  a.hid = static_cast<const float*>(hidden);
  a.out_r = static_cast<float*>(ws);
  int rc = launch_f32<EPI_RESID>(a, K, stream);
  if (rc) return rc;
  GemvF32Args b{};
  b.W = static_cast<const float*>(wlm);
  b.w_gstride = wlm_head_stride;
  b.X = static_cast<const float*>(ws);
  b.R = V;
  b.Kd = H;
  b.logits = logits;
  b.M = M;
  b.stride_m = static_cast<int64_t>(K) * V;
  b.V = V;
  if (shared) {
    b.x_gstride = 0;
    b.N = K * M;
    return launch_f32<EPI_LOGITS>(b, 1, stream);
  }
  b.x_gstride = static_cast<int64_t>(M) * H;
  b.N = M;
  return launch_f32<EPI_LOGITS>(b, K, stream);
}
