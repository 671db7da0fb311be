// fp8 round trip of kv rows (act_quant_inplace / pow2_ceil contracts of the
// "deepseek_v41_ref::attn" rustdoc; the FP8(W) step of the "Compressed sparse
// attention" page), for gfx950.
//
// Layout: one lane owns 8 consecutive bf16 (16 bytes) of a row, so the four
// lanes 4i..4i+3 of a wavefront own one 32-value block.  The block amax is two
// xor-shuffles inside the lane quad; the scale and the e4m3 rounding are the
// exact binary32 steps of v41_fp8_math.h.
// Loads and stores are 16 bytes per lane and fully coalesced along a row.
#include "v41_common.h"
#include "v41_fp8_math.h"

namespace v41 {
namespace {

constexpr int kThreads = 256;

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
    const uint32_t m = quad_max(chunk_amax_bits(v));
    float s, inv_s;
    fp8_block_scale(m, s, inv_s);
    const u32x4 o = fp8_round_chunk(v, inv_s, s);
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
