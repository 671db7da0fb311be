// Launchers of the rotary-embedding kernels (v41_rope.hip); arguments are
// validated by the C ABI layer before a launcher runs.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace v41 {

struct RopeRowsArgs {
  const uint16_t* in;
  int64_t in_ld;
  uint16_t* out;
  int64_t out_ld;
  int32_t batch, n_tokens, rows_per_pos;
  int32_t row_len, rope_dim;
  const float* table;
  int64_t table_rows;
  const int32_t* pos;
  int64_t start_pos;
  bool inverse;
  bool fp8;
  uint16_t* ring;
  int32_t ring_slots;
  int64_t ring_bs;
};

// The front of a decode step (q tails rotated in place, kv rows through the
// rotation and fp8 into their ring slots, window indices), positions on the
// device.  table NULL: no rotation.
struct DecodeFrontArgs {
  uint16_t* q;
  const uint16_t* kv;
  uint16_t* ring;
  int64_t ring_bs;
  int32_t* idx;
  int64_t idx_ld;
  const int32_t* pos;
  const float* table;
  int64_t table_rows;
  int32_t batch, n_heads, row_len, window, rope_dim;
};

hipError_t launch_decode_front(const DecodeFrontArgs& a, hipStream_t s);

hipError_t launch_rope_table(double theta, int32_t rope_dim, int64_t n_pos, float* table,
                             hipStream_t s);
hipError_t launch_rope_rows(const RopeRowsArgs& a, hipStream_t s);

}  // namespace v41
