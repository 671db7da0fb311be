// Internal device helpers and launcher declarations of libv41 (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace v41 {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t h) {
  return __uint_as_float(h << 16);
}

// binary32 -> bf16 bits, round to nearest even (NaN kept quiet).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return 0x7FC0u;
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) {
  return __builtin_bit_cast(bf16x8, v);
}

// D[16x16] += A[16x32] * B[32x16] on the matrix cores, bf16 in, f32 out.
// Lane l holds A[l%16][k(l/16, 0..7)], B[k(l/16, 0..7)][l%16] and
// D[4*(l/16) + i][l%16]; the k mapping is the same for A and B.
__device__ __forceinline__ f32x4 mfma16x16x32(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// ---------------------------------------------------------------- launchers
// Each returns a hipError_t from the launch; arguments are validated by the
// C ABI layer before any launcher runs.

hipError_t launch_fp8_round_rows(const uint16_t* in, int64_t in_ld, uint16_t* out,
                                 int64_t out_ld, int64_t rows, int32_t row_len,
                                 uint16_t* ring, int32_t ring_slots, int64_t first_pos,
                                 hipStream_t s);

hipError_t launch_window_idx(int64_t start_pos, int32_t n_tokens, int32_t window,
                             int32_t cols, int32_t batch, int32_t* idx, int64_t idx_ld,
                             int64_t idx_bs, hipStream_t s);

hipError_t launch_indexer_scores(const uint16_t* qI, const uint16_t* kI, int64_t kI_bs,
                                 const float* w, const uint8_t* cand, int32_t cand_width,
                                 int32_t cand_block, int32_t batch, int32_t n_tokens,
                                 int64_t start_pos, const int32_t* pos, int32_t ratio,
                                 int32_t n_heads, int32_t head_dim, int64_t n_rows,
                                 float* scores, int64_t scores_ld, hipStream_t s);

hipError_t launch_topk_select(const float* scores, int64_t n_sel_rows, int64_t n_cols,
                              int64_t scores_ld, int32_t k, int32_t offset, int32_t* idx,
                              int64_t idx_ld, hipStream_t s);

hipError_t launch_candidate_blocks(const float* scores, int64_t n_sel_rows, int64_t n_cols,
                                   int64_t scores_ld, int32_t cand_block, int32_t topk_blocks,
                                   uint8_t* cand, int64_t cand_ld, hipStream_t s);

struct AttnArgs {
  const uint16_t* q;
  const uint16_t* rows_a;
  int64_t rows_a_len, a_bs;
  const uint16_t* rows_b;
  int64_t rows_b_len, b_bs;
  const int32_t* idx;
  int32_t width;
  int64_t idx_ld;
  const float* sink;
  float scale;
  int32_t batch, n_tokens, n_heads, head_dim;
  uint16_t* out;
  void* workspace;
  int64_t workspace_bytes;
};

hipError_t launch_probe_hbm_read(const void* buf, int64_t bytes, int32_t nontemporal,
                                 uint32_t* sink, hipStream_t s);
hipError_t launch_probe_mfma(int32_t workgroups, int32_t iters, float* sink, hipStream_t s);

int attn_preferred_splits(int32_t queries, int32_t n_heads, int32_t width);
int64_t attn_workspace_bytes(int32_t queries, int32_t n_heads, int32_t head_dim,
                             int32_t splits);
hipError_t launch_sparse_attn_sink(const AttnArgs& a, hipStream_t s);

}  // namespace v41
