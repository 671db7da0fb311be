// The front of a decode step, shared by its own kernel (v41_rope.hip) and the
// indexer launch that carries it as extra workgroups (v41_indexer.hip): the
// rotation of q tails in place, the new kv rows through the rotation and the
// fp8 round trip into their ring slots, and the window indices of the ring.
#pragma once

#include "v41_common.h"
#include "v41_fp8_math.h"
#include "v41_rope.h"

namespace v41 {

// Four complex pairs (x0 + i x1) times (c + i s), binary32 products and sums
// each rounded on its own (no contraction into fused multiply-adds), results
// rounded to bf16.
// t0, t1: the four (cos, sin) table entries of the pairs.
__device__ __forceinline__ u32x4 rotate_chunk(u32x4 v, f32x4 t0, f32x4 t1, float sgn) {
#pragma clang fp contract(off)
  const float cs[8] = {t0[0], t0[1], t0[2], t0[3], t1[0], t1[1], t1[2], t1[3]};
  u32x4 o;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float c = cs[2 * i];
    const float s = cs[2 * i + 1] * sgn;
    const float x0 = bf16_bits_to_f32(v[i] & 0xFFFFu);
    const float x1 = bf16_bits_to_f32(v[i] >> 16);
    const float a = x0 * c;
    const float b = x1 * s;
    const float e = x0 * s;
    const float f = x1 * c;
    const float re = a - b;
    const float im = e + f;
    o[i] = f32_to_bf16_bits(re) | (f32_to_bf16_bits(im) << 16);
  }
  return o;
}

// The same with the entries read from the table at tp.
__device__ __forceinline__ u32x4 rotate_chunk(u32x4 v, const float* tp, float sgn) {
  return rotate_chunk(v, *reinterpret_cast<const f32x4*>(tp),
                      *reinterpret_cast<const f32x4*>(tp + 4), sgn);
}

// The front of a decode step in one launch, three kinds of workgroups told
// apart by blockIdx (each kind a contiguous range, so a workgroup's branch is
// uniform): [q tails rotated in place | new kv rows (rotated when a table is
// given) through fp8 into ring slot pos[b] mod W | the ring's window indices,
// oldest first].  Every position is read on the device.  A sequence whose
// position is negative (or, with a table, past its end) writes no kv row and
// gets an all -1 window; its q is not rotated.
struct FrontParams {
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
  int32_t q_blocks, kv_blocks;
};

// Workgroup blk (of 256 threads) of the front work.
__device__ __forceinline__ void decode_front_block(const FrontParams& p, int32_t blk) {
  constexpr int kThreads = 256;
  const int32_t half = p.rope_dim / 2;
  const int32_t rot0 = (p.row_len - p.rope_dim) / 8;
  if (blk < p.q_blocks) {
    // q: rope_dim / 8 chunks per head row
    const int32_t chunks = p.rope_dim / 8;
    const int32_t g = blk * kThreads + (int32_t)threadIdx.x;
    if (g < p.batch * p.n_heads * chunks) {
      const int32_t r = g / chunks;
      const int32_t c = rot0 + (g - r * chunks);
      const int32_t b = r / p.n_heads;
      const int64_t ps = p.pos[b];
      if (ps >= 0 && ps < p.table_rows) {
        uint16_t* at = p.q + (int64_t)r * p.row_len + c * 8;
        const u32x4 v = *reinterpret_cast<const u32x4*>(at);
        *reinterpret_cast<u32x4*>(at) =
            rotate_chunk(v, p.table + (ps * half + (c - rot0) * 4) * 2, 1.0f);
      }
    }
    return;
  }
  blk -= p.q_blocks;
  if (blk < p.kv_blocks) {
    // kv: row_len / 8 chunks per row, a multiple of 4, so a lane quad
    // (one fp8 block) shares its row and position
    const int32_t cpr = p.row_len / 8;
    const int32_t g = blk * kThreads + (int32_t)threadIdx.x;
    const bool in_range = g < p.batch * cpr;
    const int32_t b = in_range ? g / cpr : 0;
    const int32_t c = in_range ? g - b * cpr : 0;
    const int64_t ps = p.pos[b];
    const bool live = in_range && ps >= 0 && (p.table == nullptr || ps < p.table_rows);
    u32x4 v = {0u, 0u, 0u, 0u};
    if (live) {
      v = *reinterpret_cast<const u32x4*>(p.kv + (int64_t)b * p.row_len + c * 8);
      if (p.table != nullptr && c >= rot0)
        v = rotate_chunk(v, p.table + (ps * half + (c - rot0) * 4) * 2, 1.0f);
    }
    const uint32_t m = quad_max(chunk_amax_bits(v));
    float s, inv_s;
    fp8_block_scale(m, s, inv_s);
    v = fp8_round_chunk(v, inv_s, s);
    if (live) {
      const int64_t slot = ps % p.window;
      *reinterpret_cast<u32x4*>(p.ring + b * p.ring_bs + slot * p.row_len + c * 8) = v;
    }
    return;
  }
  blk -= p.kv_blocks;
  // window indices: the whole ring oldest first once it has wrapped, else
  // slots 0 .. pos then -1
  const int32_t g = blk * kThreads + (int32_t)threadIdx.x;
  if (g < p.batch * p.window) {
    const int32_t b = g / p.window;
    const int32_t c = g - b * p.window;
    const int64_t ps = p.pos[b];
    const bool live = ps >= 0 && (p.table == nullptr || ps < p.table_rows);
    int32_t v = -1;
    if (live) {
      if (ps >= p.window - 1) v = (int32_t)((ps + 1 + c) % p.window);
      else v = (c <= ps) ? c : -1;
    }
    p.idx[(int64_t)b * p.idx_ld + c] = v;
  }
}


// Device parameters and workgroup count of the front work of a decode step.
inline int32_t make_front_params(const DecodeFrontArgs& a, FrontParams& p) {
  p.q = a.q;
  p.kv = a.kv;
  p.ring = a.ring;
  p.ring_bs = a.ring_bs;
  p.idx = a.idx;
  p.idx_ld = a.idx_ld;
  p.pos = a.pos;
  p.table = a.table;
  p.table_rows = a.table_rows;
  p.batch = a.batch;
  p.n_heads = a.n_heads;
  p.row_len = a.row_len;
  p.window = a.window;
  p.rope_dim = a.table != nullptr ? a.rope_dim : 0;
  const int64_t q_lanes =
      a.table != nullptr ? (int64_t)a.batch * a.n_heads * (a.rope_dim / 8) : 0;
  const int64_t kv_lanes = (int64_t)a.batch * (a.row_len / 8);
  const int64_t w_lanes = (int64_t)a.batch * a.window;
  p.q_blocks = (int32_t)((q_lanes + 255) / 256);
  p.kv_blocks = (int32_t)((kv_lanes + 255) / 256);
  const int64_t w_blocks = (w_lanes + 255) / 256;
  return (int32_t)(p.q_blocks + p.kv_blocks + w_blocks);
}

// The indexer scores of a decode step with its front work as extra
// workgroups of the same launch (front_args NULL: the scores alone).
hipError_t launch_indexer_scores_front(const uint16_t* qI, const uint16_t* kI, int64_t kI_bs,
                                       const float* w, const uint8_t* cand, int32_t cand_width,
                                       int32_t cand_block, int32_t batch, int32_t n_tokens,
                                       int64_t start_pos, const int32_t* pos, int32_t ratio,
                                       int32_t n_heads, int32_t head_dim, int64_t n_rows,
                                       float* scores, int64_t scores_ld,
                                       const DecodeFrontArgs* front_args, hipStream_t s);

}  // namespace v41
