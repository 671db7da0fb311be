// fp8 round trip of kv rows (act_quant_inplace / pow2_ceil contracts of the
// "deepseek_v41_ref::attn" rustdoc; the FP8(W) step of the "Compressed sparse
// attention" page), for gfx950.
//
// Layout: one lane owns 8 consecutive bf16 (16 bytes) of a row, so the four
// lanes 4i..4i+3 of a wavefront own one 32-value block.  The block amax is two
// xor-shuffles inside the lane quad; the power-of-two scale comes from the
// IEEE exponent and fraction fields of amax/448; the e4m3 rounding is done in
// f32 on the grid quantum of each value's binade (exact: every step is a
// multiply by a power of two or a round-to-nearest-even to an integer).
// Loads and stores are 16 bytes per lane and fully coalesced along a row.
#include "v41_common.h"

namespace v41 {
namespace {

constexpr int kThreads = 256;

__device__ __forceinline__ uint32_t round_one(uint32_t xb, float inv_s, float s) {
  float x = bf16_bits_to_f32(xb);
  float y = x * inv_s;                       // exact: inv_s is 2^-k
  y = fminf(fmaxf(y, -448.0f), 448.0f);
  float a = fabsf(y);
  // binade of a: E = floor(log2 a); quantum 2^(E-3), or 2^-9 below 2^-6
  int E = (int)((__float_as_uint(a) >> 23) & 0xFFu) - 127;
  int qe = (a < 0.015625f) ? -9 : E - 3;
  float inv_q = __uint_as_float((uint32_t)(127 - qe) << 23);
  float q = __uint_as_float((uint32_t)(127 + qe) << 23);
  float r = __builtin_rintf(a * inv_q) * q;  // RNE on the grid, exact
  r = __builtin_copysignf(r, y);
  float o = r * s;                           // exact, or +-inf at 2^128
  return __float_as_uint(o) >> 16;           // o is on the bf16 grid
}

__global__ __launch_bounds__(kThreads) void fp8_round_rows_kernel(
    const uint16_t* __restrict__ in, int64_t in_ld, uint16_t* out, int64_t out_ld,
    int32_t rows, int32_t chunks_per_row, int32_t row_len, uint16_t* ring,
    int32_t ring_slots, int64_t first_pos, int32_t ring_first_row) {
  // the C ABI keeps rows * chunks_per_row below 2^31
  const int32_t total = rows * chunks_per_row;
  const int32_t stride = (int32_t)gridDim.x * kThreads;
  for (int32_t g = (int32_t)blockIdx.x * kThreads + (int32_t)threadIdx.x;
       g - (int32_t)(threadIdx.x & 3) < total; g += stride) {
    // total is a multiple of 4, so the four lanes of a block agree on `live`
    const bool live = g < total;
    const int32_t r = live ? g / chunks_per_row : 0;
    const int32_t c = live ? g - r * chunks_per_row : 0;
    u32x4 v = {0u, 0u, 0u, 0u};
    if (live) v = *reinterpret_cast<const u32x4*>(in + (int64_t)r * in_ld + c * 8);
    // |x| bit patterns compare like magnitudes for finite values
    uint32_t m = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      m = max(m, v[i] & 0x7FFFu);
      m = max(m, (v[i] >> 16) & 0x7FFFu);
    }
    m = max(m, (uint32_t)__shfl_xor((int)m, 1));
    m = max(m, (uint32_t)__shfl_xor((int)m, 2));
    float amax = fmaxf(bf16_bits_to_f32(m), 1e-4f);
    float ratio = __fdiv_rn(amax, 448.0f);
    uint32_t rb = __float_as_uint(ratio);
    uint32_t ef = ((rb >> 23) & 0xFFu) + ((rb & 0x7FFFFFu) != 0u ? 1u : 0u);
    float s = __uint_as_float(ef << 23);             // pow2_ceil(amax / 448)
    float inv_s = __uint_as_float((254u - ef) << 23);
    u32x4 o;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      uint32_t lo = round_one(v[i] & 0xFFFFu, inv_s, s);
      uint32_t hi = round_one(v[i] >> 16, inv_s, s);
      o[i] = lo | (hi << 16);
    }
    if (live) {
      *reinterpret_cast<u32x4*>(out + (int64_t)r * out_ld + c * 8) = o;
      if (ring != nullptr && r >= ring_first_row) {
        const int64_t slot = (first_pos + r) % ring_slots;
        *reinterpret_cast<u32x4*>(ring + slot * row_len + c * 8) = o;
      }
    }
  }
}

}  // namespace

hipError_t launch_fp8_round_rows(const uint16_t* in, int64_t in_ld, uint16_t* out,
                                 int64_t out_ld, int64_t rows, int32_t row_len,
                                 uint16_t* ring, int32_t ring_slots, int64_t first_pos,
                                 hipStream_t s) {
  if (rows == 0) return hipSuccess;
  const int32_t cpr = row_len / 8;
  const int64_t total = rows * cpr;
  int64_t blocks = (total + kThreads - 1) / kThreads;
  if (blocks > 65536) blocks = 65536;
  const int64_t ring_first = ring ? (rows > ring_slots ? rows - ring_slots : 0) : rows;
  hipLaunchKernelGGL(fp8_round_rows_kernel, dim3((unsigned)blocks), dim3(kThreads), 0, s,
                     in, in_ld, out, out_ld, (int32_t)rows, cpr, row_len, ring, ring_slots,
                     first_pos, (int32_t)ring_first);
  return hipGetLastError();
}

}  // namespace v41
