// Wavefront-wide reductions and prefix sums of 32-bit integers on the DPP
// (data-parallel primitives) and permlane paths of gfx950, instead of
// ds_bpermute: within a row of 16 lanes by row rotations and quad
// permutations, across the four rows by v_permlane16/32_swap (reductions) or
// row broadcasts (prefix sums).  Every control operand is a literal.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace v41 {

// Row reduction step helpers: the value of the lane `n` places further round
// the row of 16 (row_ror:n), or of the quad lane given by a permutation.
__device__ __forceinline__ uint32_t dpp_ror8(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x128, 0xF, 0xF, false);
}
__device__ __forceinline__ uint32_t dpp_ror4(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x124, 0xF, 0xF, false);
}
__device__ __forceinline__ uint32_t dpp_quad_swap2(uint32_t v) {  // quad_perm [2,3,0,1]
  return (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x4E, 0xF, 0xF, false);
}
__device__ __forceinline__ uint32_t dpp_quad_swap1(uint32_t v) {  // quad_perm [1,0,3,2]
  return (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0xB1, 0xF, 0xF, false);
}

// Combine each lane with its counterpart in the other rows (rows 0..3 of 16
// lanes): after both swaps every lane sees all four rows' values of its
// position in the row.
__device__ __forceinline__ uint32_t rows_max(uint32_t v) {
  const auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);
  v = max(r[0], r[1]);
  const auto t = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  return max(t[0], t[1]);
}
__device__ __forceinline__ uint32_t rows_min(uint32_t v) {
  const auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);
  v = min(r[0], r[1]);
  const auto t = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  return min(t[0], t[1]);
}
__device__ __forceinline__ uint32_t rows_sum(uint32_t v) {
  const auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);
  v = r[0] + r[1];
  const auto t = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  return t[0] + t[1];
}

// The wavefront's maximum / minimum / sum, in every lane.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = max(v, dpp_ror8(v));
  v = max(v, dpp_ror4(v));
  v = max(v, dpp_quad_swap2(v));
  v = max(v, dpp_quad_swap1(v));
  return rows_max(v);
}
__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) {
  v = min(v, dpp_ror8(v));
  v = min(v, dpp_ror4(v));
  v = min(v, dpp_quad_swap2(v));
  v = min(v, dpp_quad_swap1(v));
  return rows_min(v);
}
__device__ __forceinline__ uint32_t wave_sum_u32(uint32_t v) {
  v += dpp_ror8(v);
  v += dpp_ror4(v);
  v += dpp_quad_swap2(v);
  v += dpp_quad_swap1(v);
  return rows_sum(v);
}

// Inclusive prefix sum over the 64 lanes (lane i gets v_0 + .. + v_i):
// sums of four within the row (row_shr 1..3, zero past the row start), then
// row_shr 4 and 8 on the upper banks, then the row totals carried by
// row_bcast:15 (into rows 1 and 3) and row_bcast:31 (into rows 2 and 3).
__device__ __forceinline__ uint32_t wave_incl_scan_u32(uint32_t a) {
  uint32_t x = a;
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)a, 0x111, 0xF, 0xF, true);
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)a, 0x112, 0xF, 0xF, true);
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)a, 0x113, 0xF, 0xF, true);
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x114, 0xF, 0xE, true);
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x118, 0xF, 0xC, true);
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x142, 0xA, 0xF, false);
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x143, 0xC, 0xF, false);
  return x;
}

}  // namespace v41
