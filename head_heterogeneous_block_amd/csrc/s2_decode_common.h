// Shared pieces of the decode kernels: 16-byte vector loads as floats and
// cross-lane sums and maxima inside a wavefront.
#pragma once

#include <type_traits>

#include "s2_internal.h"

namespace s2 {
namespace decode_detail {

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

template <typename T>
struct Vec;
template <>
struct Vec<__bf16> {
  static constexpr int N = 8;
  __device__ static void to_float(const u32x4 &v, float *f) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[2 * i] = __uint_as_float(v[i] << 16);
      f[2 * i + 1] = __uint_as_float(v[i] & 0xffff0000u);
    }
  }
};
template <>
struct Vec<float> {
  static constexpr int N = 4;
  __device__ static void to_float(const u32x4 &v, float *f) {
#pragma unroll
    for (int i = 0; i < 4; ++i) f[i] = __uint_as_float(v[i]);
  }
};

constexpr int kThreads = 256;

// Cross-lane sums and maxima without LDS: DPP moves inside a 16-lane row
// (quad swaps, 8- and 16-lane mirrors) and the gfx950 row swaps across rows.
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xf, 0xf, false));
}
constexpr int kQuadXor1 = 0xb1;     // quad_perm [1,0,3,2]
constexpr int kQuadXor2 = 0x4e;     // quad_perm [2,3,0,1]
constexpr int kHalfMirror = 0x141;  // lane i <-> 7-i within 8 lanes
constexpr int kMirror = 0x140;      // lane i <-> 15-i within 16 lanes
__device__ __forceinline__ float swap16_sum(float x) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float swap32_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float swap16_max(float x) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return nan_max(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float swap32_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return nan_max(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
// sum over the N lanes of each aligned group of N (N = 1, 2, 4, ... 64); every lane gets it
template <int N>
__device__ __forceinline__ float group_sum(float x) {
  if constexpr (N >= 2) x += dpp<kQuadXor1>(x);
  if constexpr (N >= 4) x += dpp<kQuadXor2>(x);
  if constexpr (N >= 8) x += dpp<kHalfMirror>(x);
  if constexpr (N >= 16) x += dpp<kMirror>(x);
  if constexpr (N >= 32) x = swap16_sum(x);
  if constexpr (N >= 64) x = swap32_sum(x);
  return x;
}
// combine across the 64/N groups of a wave (lanes at distance N, 2N, ...)
template <int N>
__device__ __forceinline__ float across_groups_max(float x) {
  if constexpr (N <= 8) {
    for (int off = N; off < 16; off <<= 1) x = nan_max(x, __shfl_xor(x, off));
  }
  if constexpr (N <= 16) x = swap16_max(x);
  if constexpr (N <= 32) x = swap32_max(x);
  return x;
}
template <int N>
__device__ __forceinline__ float across_groups_sum(float x) {
  if constexpr (N <= 8) {
    for (int off = N; off < 16; off <<= 1) x += __shfl_xor(x, off);
  }
  if constexpr (N <= 16) x = swap16_sum(x);
  if constexpr (N <= 32) x = swap32_sum(x);
  return x;
}

}  // namespace decode_detail
}  // namespace s2
