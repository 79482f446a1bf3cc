// gdn_mfma_util.h -- small device helpers shared by the matrix-core window
// kernels (gdn_window_mfma.hip, gdn_kda_mfma.hip): vector types, the two
// MFMA forms they use, the bf16 hi/lo split, DPP row shifts, lane reads and
// the kernel-argument byte tables.
//
// MFMA layouts (wave64):
//   v_mfma_f32_16x16x32_bf16: lane l holds A[l%16][8(l/16) + e] and
//     B[8(l/16) + e][l%16] (e = 0..7);
//   v_mfma_f32_16x16x4_f32:   lane l holds A[l%16][l/16] and B[l/16][l%16];
//   both: D[4(l/16) + e][l%16], e = 0..3.
#pragma once
#include <hip/hip_runtime.h>

#include <cstdint>

#include "gdn_window_common.h"

namespace gdn {
namespace wm {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kBufWord3 = 0x00020000;  // raw buffer resource, 32-bit data
constexpr int kNT = 2;                 // nontemporal cache policy

__device__ __forceinline__ f32x4 mma_bf16(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(
      __builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mma_f32(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ float lo_f(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float hi_f(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Eight consecutive entries of a staged row, widened to f32 (exact).
__device__ __forceinline__ void row8(const uint16_t* p, float (&x)[8]) {
  const u32x4 w = *reinterpret_cast<const u32x4*>(p);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[2 * i] = lo_f(w[i]);
    x[2 * i + 1] = hi_f(w[i]);
  }
}
__device__ __forceinline__ void row8(const float* p, float (&x)[8]) {
  const f32x4 a = reinterpret_cast<const f32x4*>(p)[0];
  const f32x4 b = reinterpret_cast<const f32x4*>(p)[1];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[i] = a[i];
    x[4 + i] = b[i];
  }
}
// Two f32 values as packed bf16 pairs: hi = bf16(x), lo = bf16(x - hi), both
// rounded to nearest even.
__device__ __forceinline__ void split2(float a, float b, uint32_t& hi,
                                       uint32_t& lo) {
  const f32x2 x = {a, b};
  hi = __builtin_bit_cast(uint32_t, __builtin_convertvector(x, bf16x2));
  const f32x2 r = {a - lo_f(hi), b - hi_f(hi)};
  lo = __builtin_bit_cast(uint32_t, __builtin_convertvector(r, bf16x2));
}

// LDS written by some lanes of a wave and read by others of the same wave.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Entry i of a per-lane byte table in the kernel arguments, through a
// scalar load of the dword that holds it (i is uniform).  A by-value kernel
// argument lives in the kernel-argument segment (the constant address
// space), so its address converts back to that space.
__device__ __forceinline__ int table_byte(const LaneTable& t, int i) {
  typedef const __attribute__((address_space(4))) uint32_t cword;
  i = __builtin_amdgcn_readfirstlane(i);
  const uint32_t w = ((cword*)(const void*)t.v)[i >> 2];
  return (int)((w >> (8 * (i & 3))) & 0xffu);
}

__device__ __forceinline__ float lane_value(float x, int t) {  // t uniform
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), t));
}
// x from the lane CTRL selects within the 16-lane row (a DPP row shift);
// lanes whose source lies outside the row get `id`.
template <int CTRL>
__device__ __forceinline__ float row_shift(float x, float id) {
  return __int_as_float(__builtin_amdgcn_update_dpp(
      __float_as_int(id), __float_as_int(x), CTRL, 0xf, 0xf, false));
}
template <int CTRL>
__device__ __forceinline__ int row_shift_int(int x, int id) {
  return __builtin_amdgcn_update_dpp(id, x, CTRL, 0xf, 0xf, false);
}
__device__ __forceinline__ int lane_int(int x, int t) {  // t uniform
  return __builtin_amdgcn_readlane(x, t);
}
// Parent of cell i of a draft-tree table (-1 for a root), read like
// table_byte.
__device__ __forceinline__ int tree_parent(const TreeTable& t, int i) {
  typedef const __attribute__((address_space(4))) uint32_t cword;
  i = __builtin_amdgcn_readfirstlane(i);
  const uint32_t w = ((cword*)(const void*)t.v)[i >> 2];
  const int p = (int)((w >> (8 * (i & 3))) & 0xffu);
  return p == kNoParent ? -1 : p;
}
__device__ __forceinline__ int tree_parent(const NoTable&, int) { return -1; }

}  // namespace wm
}  // namespace gdn
