// Rotary position embedding for gfx950: the ratio-0 table (freqs_cis of the
// "deepseek_v41_ref::attn" rustdoc) and the rotation of the last rope_dim
// values of rows (apply_rotary there; R_t and R_t^-1 in "All 25 steps" of the
// "Compressed sparse attention" page), alone for queries and for the inverse
// on the attention output, or followed by the fp8 round trip and the ring
// write for window keys (W_{t,448:} <- R_t w^n; W <- FP8(W)).
//
// Layout: one lane owns 8 consecutive bf16 of a row (16 bytes, coalesced
// along the row), i.e. 4 adjacent complex pairs, and reads their 4 (cos, sin)
// table entries as two 16-byte loads.  With fp8 the four lanes of an aligned
// quad own one 32-value block, as in the plain fp8 kernel.  A rotation alone,
// in place, touches only the chunks of the rotated part.
#include "v41_common.h"
#include "v41_fp8_math.h"
#include "v41_rope.h"
#include "v41_front.h"

namespace v41 {
namespace {

constexpr int kThreads = 256;

struct RopeParams {
  const uint16_t* in;
  int64_t in_ld;
  uint16_t* out;  // NULL only with fp8 and a ring
  int64_t out_ld;
  int32_t n_tokens, rows_per_pos;
  int32_t row_len, rope_dim;
  const float* table;
  int64_t table_rows;
  const int32_t* pos;  // device [batch] or NULL (then start_pos)
  int64_t start_pos;
  float sin_sign;      // +1 forward, -1 inverse (negated angle)
  uint16_t* ring;
  int32_t ring_slots;
  int64_t ring_bs;
  int32_t ring_first_tok;
  int32_t rows;        // batch * n_tokens * rows_per_pos
  int32_t chunks;      // 8-value chunks handled per row
  int32_t chunk0;      // first handled chunk of a row
};

template <bool kFp8>
__global__ __launch_bounds__(kThreads) void rope_rows_kernel(RopeParams p) {
  const int32_t total = p.rows * p.chunks;  // below 2^31 (checked by the C ABI)
  const int32_t stride = (int32_t)gridDim.x * kThreads;
  const int32_t rot0 = (p.row_len - p.rope_dim) / 8;  // first rotated chunk
  const int32_t half = p.rope_dim / 2;
  const int32_t per_seq = p.n_tokens * p.rows_per_pos;
  for (int32_t g = (int32_t)blockIdx.x * kThreads + (int32_t)threadIdx.x;
       kFp8 ? (g - (int32_t)(threadIdx.x & 3) < total) : (g < total); g += stride) {
    // with fp8 every row has a multiple of 4 chunks, so a lane quad shares
    // its row, its position and `live`
    const bool in_range = g < total;
    const int32_t r = in_range ? g / p.chunks : 0;
    const int32_t c = p.chunk0 + (in_range ? g - r * p.chunks : 0);
    const int32_t b = r / per_seq;
    const int32_t t = (r - b * per_seq) / p.rows_per_pos;
    const int64_t base = (p.pos != nullptr) ? (int64_t)p.pos[b] : p.start_pos;
    const int64_t ps = base + t;
    const bool live = in_range && ps >= 0 && ps < p.table_rows;
    u32x4 v = {0u, 0u, 0u, 0u};
    if (live) {
      v = *reinterpret_cast<const u32x4*>(p.in + (int64_t)r * p.in_ld + c * 8);
      if (c >= rot0) {
        const int32_t j0 = (c - rot0) * 4;
        v = rotate_chunk(v, p.table + (ps * half + j0) * 2, p.sin_sign);
      }
    }
    if constexpr (kFp8) {
      const uint32_t m = quad_max(chunk_amax_bits(v));
      float s, inv_s;
      fp8_block_scale(m, s, inv_s);
      v = fp8_round_chunk(v, inv_s, s);
      if (live) {
        if (p.out != nullptr)
          *reinterpret_cast<u32x4*>(p.out + (int64_t)r * p.out_ld + c * 8) = v;
        if (p.ring != nullptr && t >= p.ring_first_tok) {
          const int64_t slot = ps % p.ring_slots;
          *reinterpret_cast<u32x4*>(p.ring + b * p.ring_bs + slot * p.row_len + c * 8) = v;
        }
      }
    } else {
      if (live) *reinterpret_cast<u32x4*>(p.out + (int64_t)r * p.out_ld + c * 8) = v;
    }
  }
}

// Table entry (p, i): cos and sin of p * theta^(-2i/rope_dim), evaluated in
// binary64 and rounded once to binary32.
__global__ __launch_bounds__(kThreads) void rope_table_kernel(double theta, int32_t rope_dim,
                                                              int64_t n, float* table) {
  const int32_t half = rope_dim / 2;
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  for (int64_t g = (int64_t)blockIdx.x * kThreads + threadIdx.x; g < n; g += stride) {
    const int64_t p = g / half;
    const int32_t i = (int32_t)(g - p * half);
    const double freq = pow(theta, -(double)(2 * i) / (double)rope_dim);
    const double ang = (double)p * freq;
    double sn, cn;
    sincos(ang, &sn, &cn);
    float2 e;
    e.x = (float)cn;
    e.y = (float)sn;
    reinterpret_cast<float2*>(table)[g] = e;
  }
}

__global__ __launch_bounds__(256) void decode_front_kernel(FrontParams p) {
  decode_front_block(p, (int32_t)blockIdx.x);
}

unsigned grid_for(int64_t lanes, int64_t cap) {
  int64_t blocks = (lanes + kThreads - 1) / kThreads;
  if (blocks > cap) blocks = cap;
  if (blocks < 1) blocks = 1;
  return (unsigned)blocks;
}

}  // namespace

hipError_t launch_rope_table(double theta, int32_t rope_dim, int64_t n_pos, float* table,
                             hipStream_t s) {
  const int64_t n = n_pos * (rope_dim / 2);
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(rope_table_kernel, dim3(grid_for(n, 16384)), dim3(kThreads), 0, s, theta,
                     rope_dim, n, table);
  return hipGetLastError();
}

hipError_t launch_rope_rows(const RopeRowsArgs& a, hipStream_t s) {
  const int64_t rows = (int64_t)a.batch * a.n_tokens * a.rows_per_pos;
  if (rows == 0) return hipSuccess;
  RopeParams p;
  p.in = a.in;
  p.in_ld = a.in_ld;
  p.out = a.out;
  p.out_ld = a.out_ld;
  p.n_tokens = a.n_tokens;
  p.rows_per_pos = a.rows_per_pos;
  p.row_len = a.row_len;
  p.rope_dim = a.rope_dim;
  p.table = a.table;
  p.table_rows = a.table_rows;
  p.pos = a.pos;
  p.start_pos = a.start_pos;
  p.sin_sign = a.inverse ? -1.0f : 1.0f;
  p.ring = a.ring;
  p.ring_slots = a.ring_slots;
  p.ring_bs = a.ring_bs;
  p.ring_first_tok = a.ring ? (a.n_tokens > a.ring_slots ? a.n_tokens - a.ring_slots : 0)
                            : a.n_tokens;
  p.rows = (int32_t)rows;
  // a rotation alone, in place, leaves the values before the rotated part as
  // they are and touches only its chunks
  const bool rotated_only = !a.fp8 && a.out == a.in && a.out_ld == a.in_ld;
  p.chunks = rotated_only ? a.rope_dim / 8 : a.row_len / 8;
  p.chunk0 = rotated_only ? (a.row_len - a.rope_dim) / 8 : 0;
  const unsigned grid = grid_for(rows * p.chunks, 65536);
  if (a.fp8)
    hipLaunchKernelGGL(rope_rows_kernel<true>, dim3(grid), dim3(kThreads), 0, s, p);
  else
    hipLaunchKernelGGL(rope_rows_kernel<false>, dim3(grid), dim3(kThreads), 0, s, p);
  return hipGetLastError();
}

}  // namespace v41

namespace v41 {

hipError_t launch_decode_front(const DecodeFrontArgs& a, hipStream_t s) {
  if (a.batch == 0) return hipSuccess;
  FrontParams p;
  const int32_t grid = make_front_params(a, p);
  hipLaunchKernelGGL(decode_front_kernel, dim3((unsigned)grid), dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace v41
