// fp8 round trip of bf16 values, shared by the kernels that end in the FP8(W)
// step (act_quant_inplace / pow2_ceil contracts of the "deepseek_v41_ref::attn"
// rustdoc).  Every step is exact in binary32 except the single round to the
// nearest OCP E4M3FN value, which is a round-to-nearest-even to an integer on
// the grid quantum of the value's binade.
#pragma once

#include "v41_common.h"

namespace v41 {

// Scale of a 32-value block from the largest |x| bf16 bit pattern of the block:
// s = 2^ceil(log2(max(amax, 1e-4) / 448)) taken from the IEEE fields of the
// binary32 quotient, and its exact inverse.
__device__ __forceinline__ void fp8_block_scale(uint32_t amax_bits, float& s, float& inv_s) {
  const float amax = fmaxf(bf16_bits_to_f32(amax_bits), 1e-4f);
  const float ratio = __fdiv_rn(amax, 448.0f);
  const uint32_t rb = __float_as_uint(ratio);
  const uint32_t ef = ((rb >> 23) & 0xFFu) + ((rb & 0x7FFFFFu) != 0u ? 1u : 0u);
  s = __uint_as_float(ef << 23);
  inv_s = __uint_as_float((254u - ef) << 23);
}

// One bf16 value through e4m3 at scale s: x / s clamped to +-448, rounded to
// the E4M3FN grid (quantum 2^(E-3) in [2^E, 2^(E+1)), 2^-9 below 2^-6, sign of
// zero kept), times s; the result lies on the bf16 grid.
__device__ __forceinline__ uint32_t fp8_round_one(uint32_t xb, float inv_s, float s) {
  float x = bf16_bits_to_f32(xb);
  float y = x * inv_s;
  y = fminf(fmaxf(y, -448.0f), 448.0f);
  float a = fabsf(y);
  int E = (int)((__float_as_uint(a) >> 23) & 0xFFu) - 127;
  int qe = (a < 0.015625f) ? -9 : E - 3;
  float inv_q = __uint_as_float((uint32_t)(127 - qe) << 23);
  float q = __uint_as_float((uint32_t)(127 + qe) << 23);
  float r = __builtin_rintf(a * inv_q) * q;
  r = __builtin_copysignf(r, y);
  float o = r * s;
  return __float_as_uint(o) >> 16;
}

// Largest |x| bit pattern of the 8 bf16 values of one lane (|x| patterns of
// finite values compare like the magnitudes).
__device__ __forceinline__ uint32_t chunk_amax_bits(u32x4 v) {
  uint32_t m = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    m = max(m, v[i] & 0x7FFFu);
    m = max(m, (v[i] >> 16) & 0x7FFFu);
  }
  return m;
}

// The fp8 round trip of a lane's 8 values whose block (this lane and the three
// others of its aligned lane quad) has the scale s.
__device__ __forceinline__ u32x4 fp8_round_chunk(u32x4 v, float inv_s, float s) {
  u32x4 o;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    uint32_t lo = fp8_round_one(v[i] & 0xFFFFu, inv_s, s);
    uint32_t hi = fp8_round_one(v[i] >> 16, inv_s, s);
    o[i] = lo | (hi << 16);
  }
  return o;
}

// Block amax over the aligned quad of lanes that own one 32-value block.
__device__ __forceinline__ uint32_t quad_max(uint32_t m) {
  // quad_perm [1,0,3,2] then [2,3,0,1] on the DPP path
  m = max(m, (uint32_t)__builtin_amdgcn_update_dpp((int)m, (int)m, 0xB1, 0xF, 0xF, false));
  m = max(m, (uint32_t)__builtin_amdgcn_update_dpp((int)m, (int)m, 0x4E, 0xF, 0xF, false));
  return m;
}

}  // namespace v41
