// Sparse attention with the sink over [window rows ; selected compressed rows]
// ("Compressed sparse attention" page, "All 25 steps": G_t = Y[J_t],
// S = Q G / sqrt(d), A = exp S / (exp s_h + sum exp S), O = sum A G; the
// sparse_attn contract of the "deepseek_v41_ref::attn" rustdoc), for gfx950.
//
// One latent row is key and value for every head, so a workgroup takes a
// query and 64 of its heads (16 per wavefront) and streams the query's valid
// rows through LDS in tiles of 32:
//  * the idx row is compacted first (entries outside the two row sources are
//    dropped), so -1 padding costs neither loads nor matrix-core time;
//  * gather: rows go from HBM straight into LDS with global_load_lds_dwordx4
//    (one 1 KB row per wavefront instruction, row address in scalar
//    registers), into a double buffer one tile ahead of the tile in use;
//    16-byte chunks are xor-swizzled by row so the reads below hit distinct
//    LDS banks;
//  * S^T = G Q^T on the matrix cores (v_mfma_f32_16x16x32_bf16): A operand =
//    16 rows x 32 dims read with ds_read_b128, B operand = the wave's query
//    fragments held in registers;
//  * online softmax in f32 on the log2 scale; the reference max starts at the
//    sink (which enters only the final denominator) and is moved lazily;
//  * O^T += G^T P^T: the A operand (16 dims x 32 rows) comes from the same
//    row-major tile through two ds_read_b64_tr_b16 transposing loads, and the
//    B operand is the probabilities exactly as the S^T accumulator left them
//    in the lane (the transposing loads fetch the rows in that order), rounded
//    to bf16.
// Decode has few queries: a query's rows are then split over several
// workgroups, each writing an f32 partial (max, sum, O), and a combine kernel
// merges them.
#include "v41_common.h"

namespace v41 {
namespace {

constexpr int kThreads = 256;
constexpr int kTile = 32;
constexpr int kHeadsPerBlock = 64;
constexpr int kMaxWidth = 2048;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kRescaleLog2 = 8.0f;  // probabilities stay below 2^8 before a rescale

typedef __attribute__((address_space(3))) void lds_void;

struct Params {
  const uint16_t* q;
  const uint16_t* rows_a;
  int64_t rows_a_len, a_bs;
  const uint16_t* rows_b;
  int64_t rows_b_len, b_bs;
  const int32_t* idx;
  int32_t width;
  int64_t idx_ld;
  const float* sink;
  float scale_log2;
  int32_t n_tokens, n_heads;
  uint16_t* out;
  float* part_o;   // [q][split][head][D]
  float* part_ml;  // [q][split][head][2]
  int32_t splits;
};

// LDS placement of a 32-row tile.  A wavefront load instruction fills one
// 1 KB block (RPI rows of D values); blocks are padded by 32 bytes.  For
// D = 512 the 16-byte chunk c of row r sits at chunk c ^ ((r >> 3) & 1).
template <int D>
struct Tile {
  static constexpr int LPR = D / 8;      // 16-byte chunks per row
  static constexpr int RPI = 64 / LPR;   // rows per load instruction
  static constexpr int kBlkBytes = 1024 + 32;
  static constexpr int kBlocks = kTile / RPI;
  static constexpr int kBufBytes = kBlocks * kBlkBytes;
  static __device__ __forceinline__ int row_off(int r) {
    return (r / RPI) * kBlkBytes + (r % RPI) * (2 * D);
  }
  static __device__ __forceinline__ int swz(int r) { return D == 512 ? ((r >> 3) & 1) : 0; }
};

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Eight ds_read_b64_tr_b16 (four 16-dim M-tiles, rows of slots 0..3 and
// 4..7) and a wait for them.  Written as one asm block so the compiler does
// not make these LDS reads wait for the direct-to-LDS loads of the next tile,
// which target the other buffer.
__device__ __forceinline__ void tr_load4(u32x2 (&t)[8], uint32_t lo, uint32_t hi) {
  asm volatile(
      "ds_read_b64_tr_b16 %0, %8\n\t"
      "ds_read_b64_tr_b16 %1, %9\n\t"
      "ds_read_b64_tr_b16 %2, %8 offset:32\n\t"
      "ds_read_b64_tr_b16 %3, %9 offset:32\n\t"
      "ds_read_b64_tr_b16 %4, %8 offset:64\n\t"
      "ds_read_b64_tr_b16 %5, %9 offset:64\n\t"
      "ds_read_b64_tr_b16 %6, %8 offset:96\n\t"
      "ds_read_b64_tr_b16 %7, %9 offset:96\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(t[0]), "=&v"(t[1]), "=&v"(t[2]), "=&v"(t[3]), "=&v"(t[4]), "=&v"(t[5]),
        "=&v"(t[6]),
        "=&v"(t[7])
      : "v"(lo), "v"(hi)
      : "memory");
}

__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

template <int D>
__global__ __launch_bounds__(kThreads, 2) void attn_kernel(Params p) {
  using TL = Tile<D>;
  constexpr int KS = D / 32;  // QK K-steps
  constexpr int MT = D / 16;  // PV M-tiles (dims)
  __shared__ __attribute__((aligned(16))) uint8_t tiles[2 * TL::kBufBytes];
  __shared__ int32_t list[kMaxWidth];
  __shared__ uint32_t wave_cnt[kThreads / kWave];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int r16 = lane & 15;
  const int g = lane >> 4;
  const int64_t qi = blockIdx.x / p.splits;
  const int split = (int)(blockIdx.x - qi * p.splits);
  const int64_t b = qi / p.n_tokens;
  const int head = blockIdx.y * kHeadsPerBlock + 16 * wave + r16;
  const bool head_ok = head < p.n_heads;
  const int64_t total_rows = p.rows_a_len + p.rows_b_len;

  // ---- compact the idx row: each wave takes a contiguous quarter
  const int32_t* irow = p.idx + qi * p.idx_ld;
  {
    const int per_wave = ((p.width + 4 * kWave - 1) / (4 * kWave)) * kWave;
    const int w0 = wave * per_wave;
    int w1 = w0 + per_wave;
    if (w1 > p.width) w1 = p.width;
    uint32_t cnt = 0;
    for (int i0 = w0; i0 < w1; i0 += kWave) {
      const int i = i0 + lane;
      const int32_t ix = (i < w1) ? irow[i] : -1;
      const bool ok = ix >= 0 && (int64_t)ix < total_rows;
      cnt += __popcll(__ballot(ok));
    }
    if (lane == 0) wave_cnt[wave] = cnt;
    __syncthreads();
    uint32_t base = 0;
    for (int w = 0; w < wave; ++w) base += wave_cnt[w];
    for (int i0 = w0; i0 < w1; i0 += kWave) {
      const int i = i0 + lane;
      const int32_t ix = (i < w1) ? irow[i] : -1;
      const bool ok = ix >= 0 && (int64_t)ix < total_rows;
      const unsigned long long bal = __ballot(ok);
      const uint32_t before = __popcll(bal & ((1ull << lane) - 1ull));
      if (ok) list[base + before] = ix;
      base += __popcll(bal);
    }
  }
  __syncthreads();
  uint32_t n_valid = 0;
  for (int w = 0; w < kThreads / kWave; ++w) n_valid += wave_cnt[w];
  const int n_tiles = (int)((n_valid + kTile - 1) / kTile);
  const int tps = (n_tiles + p.splits - 1) / p.splits;
  const int t_begin = split * tps;
  const int t_end = (t_begin + tps < n_tiles) ? t_begin + tps : n_tiles;

  // ---- gather of one tile into LDS buffer `buf` (rows past n_valid repeat
  // the first valid row: finite data whose probability is 0)
  const uint16_t* a_base = p.rows_a + b * p.a_bs;
  const uint16_t* b_base = p.rows_b + b * p.b_bs;
  auto gather = [&](int tile, int buf) {
    const int base_pos = tile * kTile;
#pragma unroll
    for (int bk = wave; bk < TL::kBlocks; bk += kThreads / kWave) {
      const int r = bk * TL::RPI + lane / TL::LPR;
      const int c = (lane % TL::LPR) ^ TL::swz(r);
      int pos = base_pos + r;
      if ((uint32_t)pos >= n_valid) pos = 0;
      int64_t ix = list[pos];
      if (TL::RPI == 1) ix = __builtin_amdgcn_readfirstlane((int)ix);
      const uint16_t* src = (ix < p.rows_a_len) ? a_base + ix * D
                                                : b_base + (ix - p.rows_a_len) * D;
      __builtin_amdgcn_global_load_lds(
          src + 8 * c, (lds_void*)(size_t)(tiles + buf * TL::kBufBytes + bk * TL::kBlkBytes),
          16, 0, 0);
    }
  };

  // ---- query fragments (B operand of S^T = G Q^T): head r16, dims 32kk+8g..
  bf16x8 qf[KS];
  {
    const uint16_t* qp = p.q + (qi * p.n_heads + (head_ok ? head : 0)) * D + 8 * g;
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) {
      u32x4 v = {0u, 0u, 0u, 0u};
      if (head_ok) v = *reinterpret_cast<const u32x4*>(qp + 32 * kk);
      qf[kk] = as_bf16x8(v);
    }
  }
  const float sink2 = head_ok ? p.sink[head] * kLog2e : 0.0f;
  const float kNegInf = -__builtin_huge_valf();
  float m2 = sink2;  // reference max on the log2 scale
  float l_part = 0.0f;
  f32x4 acc_o[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) acc_o[mt] = (f32x4){0.f, 0.f, 0.f, 0.f};

  // per-lane LDS byte offsets inside a tile buffer
  //  QK: row 16mt + r16, chunk 4kk + g (swizzled)
  int qk_off[2];
#pragma unroll
  for (int mt = 0; mt < 2; ++mt) {
    const int r = 16 * mt + r16;
    qk_off[mt] = TL::row_off(r) + 16 * (g ^ TL::swz(r));
  }
  //  PV transposing loads: lane (g, a, bb) reads 8 bytes of row 4g + a (first)
  //  and 16 + 4g + a (second) at dims 16mt + 4bb
  const int ta = (lane >> 2) & 3, tb = lane & 3;
  const int r_lo = 4 * g + ta, r_hi = 16 + 4 * g + ta;
  const int tr_lo = TL::row_off(r_lo) + 16 * ((tb >> 1) ^ TL::swz(r_lo)) + 8 * (tb & 1);
  const int tr_hi = TL::row_off(r_hi) + 16 * ((tb >> 1) ^ TL::swz(r_hi)) + 8 * (tb & 1);

  if (t_begin < t_end) gather(t_begin, 0);
  for (int tile = t_begin; tile < t_end; ++tile) {
    const int buf = (tile - t_begin) & 1;
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    lds_barrier();
    if (tile + 1 < t_end) gather(tile + 1, buf ^ 1);
    const uint8_t* tb_base = tiles + buf * TL::kBufBytes;

    // S^T tile: rows 16mt + 4g + i, head r16
    f32x4 sacc[2] = {(f32x4){0.f, 0.f, 0.f, 0.f}, (f32x4){0.f, 0.f, 0.f, 0.f}};
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) {
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) {
        const u32x4 a = *reinterpret_cast<const u32x4*>(tb_base + qk_off[mt] + 64 * kk);
        sacc[mt] = mfma16x16x32(as_bf16x8(a), qf[kk], sacc[mt]);
      }
    }
    // online softmax on the log2 scale
    const int tbase = tile * kTile;
    float sv[8];
    float mx = kNegInf;
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const int r = (s < 4) ? 4 * g + s : 16 + 4 * g + (s - 4);
      float v = sacc[s >> 2][s & 3] * p.scale_log2;
      if ((uint32_t)(tbase + r) >= n_valid) v = kNegInf;
      sv[s] = v;
      mx = fmaxf(mx, v);
    }
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    // lazy rescale: the reference moves only when a score exceeds it by more
    // than 2^8 (O and l share the reference, so O / l is unchanged); the
    // branch is uniform across the wavefront
    if (__any(mx > m2 + kRescaleLog2)) {
      const float m_new = fmaxf(m2, mx);
      const float alpha = (m_new == m2) ? 1.0f : exp2f(m2 - m_new);
      m2 = m_new;
      l_part *= alpha;
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) acc_o[mt] *= alpha;
    }
    bf16x8 pf;
    float psum = 0.0f;
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const float pv = (sv[s] == kNegInf) ? 0.0f : __builtin_amdgcn_exp2f(sv[s] - m2);
      psum += pv;
      pf[s] = (__bf16)pv;
    }
    l_part += psum;
    // O^T += G^T P^T, four M-tiles per batch of transposing loads
    const uint32_t lds_lo = (uint32_t)(size_t)(tb_base + tr_lo);
    const uint32_t lds_hi = (uint32_t)(size_t)(tb_base + tr_hi);
#pragma unroll
    for (int mt0 = 0; mt0 < MT; mt0 += 4) {
      u32x2 t[8];
      tr_load4(t, lds_lo + 32 * mt0, lds_hi + 32 * mt0);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const u32x4 a = {t[2 * j][0], t[2 * j][1], t[2 * j + 1][0], t[2 * j + 1][1]};
        acc_o[mt0 + j] = mfma16x16x32(as_bf16x8(a), pf, acc_o[mt0 + j]);
      }
    }
  }

  // ---- epilogue: lane holds O^T[dims 16mt + 4g + i][head r16]
  float l_tot = l_part;
  l_tot += __shfl_xor(l_tot, 16);
  l_tot += __shfl_xor(l_tot, 32);
  if (!head_ok) return;
  if (p.splits == 1) {
    const float sink_term = (sink2 == kNegInf) ? 0.0f : exp2f(sink2 - m2);
    const float den = l_tot + sink_term;
    const float inv = den > 0.0f ? 1.0f / den : 0.0f;
    uint16_t* op = p.out + (qi * p.n_heads + head) * D + 4 * g;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const uint32_t lo = f32_to_bf16_bits(acc_o[mt][0] * inv) |
                          (f32_to_bf16_bits(acc_o[mt][1] * inv) << 16);
      const uint32_t hi = f32_to_bf16_bits(acc_o[mt][2] * inv) |
                          (f32_to_bf16_bits(acc_o[mt][3] * inv) << 16);
      uint2 v;
      v.x = lo;
      v.y = hi;
      *reinterpret_cast<uint2*>(op + 16 * mt) = v;
    }
  } else {
    const int64_t slot = (qi * p.splits + split) * p.n_heads + head;
    float* po = p.part_o + slot * D + 4 * g;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) *reinterpret_cast<f32x4*>(po + 16 * mt) = acc_o[mt];
    if (g == 0) {
      p.part_ml[2 * slot] = m2;
      p.part_ml[2 * slot + 1] = l_tot;
    }
  }
}

// Merge the row splits of each (query, head): M = max_s m_s,
// den = sum_s l_s 2^(m_s - M) + 2^(sink - M), o = sum_s O_s 2^(m_s - M) / den.
template <int D>
__global__ __launch_bounds__(256) void attn_combine_kernel(const float* __restrict__ part_o,
                                                           const float* __restrict__ part_ml,
                                                           const float* __restrict__ sink,
                                                           int32_t n_heads, int32_t splits,
                                                           uint16_t* __restrict__ out) {
  constexpr int Q4 = D / 4;
  const int64_t qi = blockIdx.x;
  const int e = blockIdx.y * 256 + threadIdx.x;  // (head, 4-dim group)
  if (e >= n_heads * Q4) return;
  const int h = e / Q4;
  const int d4 = e - h * Q4;
  const float kNegInf = -__builtin_huge_valf();
  const float sink2 = sink[h] * kLog2e;
  float M = sink2;
  for (int s = 0; s < splits; ++s)
    M = fmaxf(M, part_ml[2 * ((qi * splits + s) * n_heads + h)]);
  float den = (sink2 == kNegInf) ? 0.0f : exp2f(sink2 - M);
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int s = 0; s < splits; ++s) {
    const int64_t slot = (qi * splits + s) * n_heads + h;
    const float ms = part_ml[2 * slot];
    const float wgt = (ms == kNegInf) ? 0.0f : exp2f(ms - M);
    den += part_ml[2 * slot + 1] * wgt;
    const f32x4 v = *reinterpret_cast<const f32x4*>(part_o + slot * D + 4 * d4);
    acc += v * wgt;
  }
  const float inv = den > 0.0f ? 1.0f / den : 0.0f;
  uint2 o;
  o.x = f32_to_bf16_bits(acc[0] * inv) | (f32_to_bf16_bits(acc[1] * inv) << 16);
  o.y = f32_to_bf16_bits(acc[2] * inv) | (f32_to_bf16_bits(acc[3] * inv) << 16);
  *reinterpret_cast<uint2*>(out + (qi * n_heads + h) * D + 4 * d4) = o;
}

template <int D>
hipError_t launch_d(const AttnArgs& a, int splits, hipStream_t s) {
  const int64_t nq = (int64_t)a.batch * a.n_tokens;
  Params p;
  p.q = a.q;
  p.rows_a = a.rows_a;
  p.rows_a_len = a.rows_a_len;
  p.a_bs = a.a_bs;
  p.rows_b = a.rows_b;
  p.rows_b_len = a.rows_b ? a.rows_b_len : 0;
  p.b_bs = a.b_bs;
  p.idx = a.idx;
  p.width = a.width;
  p.idx_ld = a.idx_ld;
  p.sink = a.sink;
  p.scale_log2 = a.scale * kLog2e;
  p.n_tokens = a.n_tokens;
  p.n_heads = a.n_heads;
  p.out = a.out;
  p.splits = splits;
  p.part_o = nullptr;
  p.part_ml = nullptr;
  if (splits > 1) {
    p.part_o = reinterpret_cast<float*>(a.workspace);
    p.part_ml = p.part_o + nq * splits * a.n_heads * (int64_t)D;
  }
  const dim3 grid((unsigned)(nq * splits), (unsigned)((a.n_heads + kHeadsPerBlock - 1) /
                                                      kHeadsPerBlock));
  hipLaunchKernelGGL((attn_kernel<D>), grid, dim3(kThreads), 0, s, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || splits == 1) return e;
  const int per_q = a.n_heads * (D / 4);
  const dim3 cgrid((unsigned)nq, (unsigned)((per_q + 255) / 256));
  hipLaunchKernelGGL((attn_combine_kernel<D>), cgrid, dim3(256), 0, s, p.part_o, p.part_ml,
                     a.sink, a.n_heads, splits, a.out);
  return hipGetLastError();
}

}  // namespace

int attn_preferred_splits(int32_t queries, int32_t n_heads, int32_t width) {
  // Aim for ~256 workgroups (one per compute unit) when there are few queries,
  // keeping at least 4 tiles of rows per split.
  const int64_t hg = (n_heads + kHeadsPerBlock - 1) / kHeadsPerBlock;
  const int64_t wgs = (int64_t)queries * hg;
  if (wgs >= 256) return 1;
  int64_t s = (256 + wgs - 1) / wgs;
  const int64_t max_s = width / (4 * kTile);
  if (s > max_s) s = max_s;
  if (s < 1) s = 1;
  if (s > 64) s = 64;
  return (int)s;
}

int64_t attn_workspace_bytes(int32_t queries, int32_t n_heads, int32_t head_dim,
                             int32_t splits) {
  if (splits <= 1) return 0;
  const int64_t slots = (int64_t)queries * splits * n_heads;
  return slots * head_dim * 4 + slots * 2 * 4;
}

hipError_t launch_sparse_attn_sink(const AttnArgs& a, hipStream_t s) {
  const int64_t nq = (int64_t)a.batch * a.n_tokens;
  if (nq == 0) return hipSuccess;
  int splits = attn_preferred_splits((int32_t)nq, a.n_heads, a.width);
  while (splits > 1 &&
         (a.workspace == nullptr ||
          attn_workspace_bytes((int32_t)nq, a.n_heads, a.head_dim, splits) > a.workspace_bytes))
    --splits;
  switch (a.head_dim) {
    case 64: return launch_d<64>(a, splits, s);
    case 128: return launch_d<128>(a, splits, s);
    case 256: return launch_d<256>(a, splits, s);
    default: return launch_d<512>(a, splits, s);
  }
}

}  // namespace v41
