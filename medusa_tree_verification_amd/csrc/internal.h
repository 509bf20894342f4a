// Internal declarations shared by the library's translation units.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <vector>

#include "medusa.h"

namespace medusa {

// ---- errors --------------------------------------------------------------
void set_error(const char* fmt, ...) __attribute__((format(printf, 1, 2)));
void clear_error();

#define MEDUSA_CHECK_ARG(cond, ...)          \
  do {                                       \
    if (!(cond)) {                           \
      ::medusa::set_error(__VA_ARGS__);      \
      return MEDUSA_EINVAL;                  \
    }                                        \
  } while (0)

#define MEDUSA_HIP_TRY(expr)                                                    \
  do {                                                                          \
    hipError_t e_ = (expr);                                                     \
    if (e_ != hipSuccess) {                                                     \
      ::medusa::set_error("%s failed: %s", #expr, hipGetErrorString(e_));       \
      return MEDUSA_EHIP;                                                       \
    }                                                                           \
  } while (0)

// after a kernel launch
int check_launch(const char* what);

// current device id, or -1 with the error set
int current_device();

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }
inline bool aligned256(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 255) == 0; }

inline size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

}  // namespace medusa

// ---- the static tree -----------------------------------------------------
// Device arrays live in one allocation; all are int32 except the mask.
struct medusa_tree {
  int T = 0, K = 0, W = 0, max_depth = 0, kmax = 0;
  int device = -1;
  std::vector<int32_t> parent, rank, depth, kpd;
  std::vector<int32_t> child_start;  // [T+1] CSR offsets into child_list
  std::vector<int32_t> child_list;   // [T-1] children of each node, rank order
  std::vector<uint64_t> mask;        // [T][W]
  void* blob = nullptr;
  const uint64_t* d_mask = nullptr;
  const int32_t* d_parent = nullptr;
  const int32_t* d_rank = nullptr;
  const int32_t* d_depth = nullptr;
  const int32_t* d_child_start = nullptr;
  const int32_t* d_child_list = nullptr;
  const int32_t* d_kpd = nullptr;
};

namespace medusa {
// Checks that the tree exists and belongs to the current device.
int check_tree(const medusa_tree_t* tree);
}  // namespace medusa

// ---- device helpers ------------------------------------------------------
namespace medusa {
namespace dev {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

// fp32 -> bf16 bits, round to nearest even (finite inputs; NaN kept quiet)
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7f800000u) == 0x7f800000u && (u & 0x007fffffu)) return (u >> 16) | 0x40u;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8, v); }

// Sorted insertion into a KM-entry list (descending value; an entry enters
// only at a place whose value it strictly exceeds, so among equal values the
// one inserted first stays first, and -0 equals +0): the new pair takes the
// first place it beats and every entry from there on moves down exactly one
// place (a displaced entry is not compared again: it may equal the next one).
// Wave-wide arg-max of (value, index) pairs (larger value, then lower index),
// left in every lane.  All on the vector ALU: DPP quad permutes pair lanes
// that differ in bit 0 and bit 1, the half-row and row mirrors then pair
// uniform groups of 4 and 8, and the 16- and 32-lane swaps finish across rows.
__device__ __forceinline__ void best_of(float& bv, int& bi, float ov, int oi) {
  const bool take = ov > bv || (ov == bv && oi < bi);
  bv = take ? ov : bv;
  bi = take ? oi : bi;
}

template <int CTRL>
__device__ __forceinline__ void best_dpp(float& bv, int& bi) {
  const float ov = __uint_as_float(__builtin_amdgcn_update_dpp(0u, __float_as_uint(bv), CTRL, 0xf, 0xf, false));
  const int oi = __builtin_amdgcn_update_dpp(0, bi, CTRL, 0xf, 0xf, false);
  best_of(bv, bi, ov, oi);
}

__device__ __forceinline__ void wave_best(float& bv, int& bi) {
  best_dpp<0xB1>(bv, bi);   // quad_perm [1,0,3,2]
  best_dpp<0x4E>(bv, bi);   // quad_perm [2,3,0,1]
  best_dpp<0x141>(bv, bi);  // row_half_mirror
  best_dpp<0x140>(bv, bi);  // row_mirror
  {
    // rows 0<->1 and 2<->3: both halves of the swap carry one candidate each
    const auto v = __builtin_amdgcn_permlane16_swap(__float_as_uint(bv), __float_as_uint(bv), false, false);
    const auto i = __builtin_amdgcn_permlane16_swap(static_cast<unsigned>(bi), static_cast<unsigned>(bi), false, false);
    float av = __uint_as_float(v[0]);
    int ai = static_cast<int>(i[0]);
    best_of(av, ai, __uint_as_float(v[1]), static_cast<int>(i[1]));
    bv = av;
    bi = ai;
  }
  {
    const auto v = __builtin_amdgcn_permlane32_swap(__float_as_uint(bv), __float_as_uint(bv), false, false);
    const auto i = __builtin_amdgcn_permlane32_swap(static_cast<unsigned>(bi), static_cast<unsigned>(bi), false, false);
    float av = __uint_as_float(v[0]);
    int ai = static_cast<int>(i[0]);
    best_of(av, ai, __uint_as_float(v[1]), static_cast<int>(i[1]));
    bv = av;
    bi = ai;
  }
}

template <int KM>
__device__ __forceinline__ void list_insert(float (&tv)[KM], int (&ti)[KM], float x, int xi) {
  bool shifting = false;
#pragma unroll
  for (int s = 0; s < KM; ++s) {
    const bool take = shifting || x > tv[s];
    shifting = take;
    const float ov = tv[s];
    const int oi = ti[s];
    tv[s] = take ? x : ov;
    ti[s] = take ? xi : oi;
    x = take ? ov : x;
    xi = take ? oi : xi;
  }
}

}  // namespace dev
}  // namespace medusa
