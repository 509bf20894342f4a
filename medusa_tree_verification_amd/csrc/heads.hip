// Medusa heads: r = SiLU(W1 h) + h, logits = W_lm r.
//
// P1 ("Medusa 심층 아키텍처"), section "Medusa의 핵심 철학 ... 잔차 블록을 포함한
// Medusa 헤드 구조" gives the two equations; its sketch code fixes bias-free
// [out, in] projections and the residual add.  Both projections are weight
// streams with a handful of activation rows (M = batch), so each is a
// "skinny" product Y[n][r] = sum_k W[r][k] X[n][k] whose cost is reading W
// from HBM once.
//
// bf16 design (gfx950): one wave owns 16 consecutive weight rows and streams
// them along k in 128-byte-per-lane chunks (lane l reads row l%16 at k-slice
// (l/16)*64 .. +64, so every wave load instruction covers 16 rows x 512
// contiguous bytes).  The products run on v_mfma_f32_16x16x32_bf16 with the
// weights as the A operand (16 rows) and the activation rows as B (up to 16
// columns per tile, zero-padded).  The k order inside a chunk is permuted
// identically for A and B, which leaves the dot products unchanged and lets
// each lane consume its contiguous 128 bytes as 8 MFMA k-steps.  Two chunks
// are kept in flight per wave (register double buffer).  The MFMA work is
// far below the matrix-core peak; the point is that it costs almost no VALU
// issue slots, so the wave spends its time keeping loads in flight.
#include "internal.h"

using namespace medusa;
using namespace medusa::dev;

namespace {

enum { EPI_RESID = 1, EPI_LOGITS = 2 };

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

template <int CH>
__device__ __forceinline__ void load_chunk(Chunk<CH>& c, const uint16_t* p, int avail) {
  // avail: elements of this lane's slice that lie inside the row (>= 8*CH means all)
#pragma unroll
  for (int j = 0; j < CH; ++j) {
    if (8 * j + 8 <= avail)
      c.v[j] = *reinterpret_cast<const uint4*>(p + 8 * j);
    else
      c.v[j] = make_uint4(0, 0, 0, 0);
  }
}

template <int NT, int CH>
__device__ __forceinline__ void mfma_chunk(f32x4 (&acc)[NT], const Chunk<CH>& w,
                                           const Chunk<CH> (&x)[NT]) {
#pragma unroll
  for (int j = 0; j < CH; ++j) {
#pragma unroll
    for (int t = 0; t < NT; ++t)
      acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(w.v[j]), as_bf16x8(x[t].v[j]),
                                                        acc[t], 0, 0, 0);
  }
}

// grid: (ceil(R/64), G, passes); block: 256 (4 waves x 16 rows)
template <int NT, int EPI>
__global__ __launch_bounds__(256) void skinny_gemm_bf16(GemmArgs a) {
  constexpr int CH = (NT == 1) ? 8 : 4;  // 16-byte loads per lane per chunk
  constexpr int SLICE = 8 * CH;          // elements per lane per chunk
  constexpr int STEP = 4 * SLICE;        // elements per chunk (4 lane groups)
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int g = blockIdx.y;
  const int n0 = blockIdx.z * NT * 16;
  const int row0 = blockIdx.x * 64 + wave * 16;
  if (row0 >= a.R) return;  // no block-level synchronisation in this kernel
  const int rl = min(row0 + (lane & 15), a.R - 1);
  const int kq = (lane >> 4) * SLICE;
  const uint16_t* wp = a.W + g * a.w_gstride + static_cast<int64_t>(rl) * a.Kd + kq;
  const uint16_t* xp[NT];
  bool xv[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    int n = n0 + t * 16 + (lane & 15);
    xv[t] = n < a.N;
    xp[t] = a.X + g * a.x_gstride + static_cast<int64_t>(xv[t] ? n : 0) * a.Kd + kq;
  }
  f32x4 acc[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int nchunks = (a.Kd + STEP - 1) / STEP;
  Chunk<CH> wa, wb, xa[NT], xb[NT];
  auto load = [&](Chunk<CH>& w, Chunk<CH>(&x)[NT], int c) {
    int avail = a.Kd - c * STEP - kq;
    load_chunk<CH>(w, wp + static_cast<int64_t>(c) * STEP, avail);
#pragma unroll
    for (int t = 0; t < NT; ++t)
      load_chunk<CH>(x[t], xp[t] + static_cast<int64_t>(c) * STEP, xv[t] ? avail : 0);
  };
  load(wa, xa, 0);
  int c = 0;
  for (; c + 2 <= nchunks; c += 2) {
    load(wb, xb, c + 1);
    mfma_chunk<NT, CH>(acc, wa, xa);
    if (c + 2 < nchunks) load(wa, xa, c + 2);
    mfma_chunk<NT, CH>(acc, wb, xb);
  }
  if (c < nchunks) mfma_chunk<NT, CH>(acc, wa, xa);

  // C layout: lane holds column (lane & 15) and rows 4*(lane >> 4) + e
  const int rbase = row0 + 4 * (lane >> 4);
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const int n = n0 + t * 16 + (lane & 15);
    if (n >= a.N) continue;
    if (EPI == EPI_RESID) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        int r = rbase + e;
        if (r >= a.R) break;
        float y = acc[t][e];
        float s = y / (1.0f + expf(-y));
        float h = bf16_bits_to_f32(a.hid[static_cast<int64_t>(n) * a.R + r]);
        a.out_r[static_cast<int64_t>(g) * a.N * a.R + static_cast<int64_t>(n) * a.R + r] =
            static_cast<uint16_t>(f32_to_bf16_bits(s + h));
      }
    } else {
      float* dst = a.logits + static_cast<int64_t>(n % a.M) * a.stride_m +
                   static_cast<int64_t>(g + n / a.M) * a.V + rbase;
      if (rbase + 3 < a.R && (reinterpret_cast<uintptr_t>(dst) & 15) == 0) {
        *reinterpret_cast<float4*>(dst) = make_float4(acc[t][0], acc[t][1], acc[t][2], acc[t][3]);
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (rbase + e < a.R) dst[e] = acc[t][e];
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

template <int EPI>
int launch_bf16(const GemmArgs& a, int G, hipStream_t s) {
  int nt = (a.N + 15) / 16;
  if (nt > 4) nt = 4;
  dim3 grid((a.R + 63) / 64, G, (a.N + nt * 16 - 1) / (nt * 16));
  switch (nt) {
    case 1: hipLaunchKernelGGL((skinny_gemm_bf16<1, EPI>), grid, dim3(256), 0, s, a); break;
    case 2: hipLaunchKernelGGL((skinny_gemm_bf16<2, EPI>), grid, dim3(256), 0, s, a); break;
    case 3: hipLaunchKernelGGL((skinny_gemm_bf16<3, EPI>), grid, dim3(256), 0, s, a); break;
    default: hipLaunchKernelGGL((skinny_gemm_bf16<4, EPI>), grid, dim3(256), 0, s, a); break;
  }
  return check_launch(EPI == EPI_RESID ? "heads residual block (bf16)" : "heads vocab projection (bf16)");
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
