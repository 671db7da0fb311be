// Sparse attention with the sink over [window rows ; selected compressed rows]
// ("Compressed sparse attention" page, "All 25 steps": G_t = Y[J_t],
// S = Q G / sqrt(d), A = exp S / (exp s_h + sum exp S), O = sum A G; the
// sparse_attn contract of the "deepseek_v41_ref::attn" rustdoc), for gfx950.
//
// Two forms share the row handling below.  The wide form (many queries, e.g.
// a prefill chunk) is described here; the narrow form (few queries, decode)
// follows its own comment further down.
//
// One latent row is key and value for every head, so a wide workgroup takes
// a query and 64 of its heads (16 per wavefront) and streams the query's
// valid rows through LDS in tiles of 32:
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
//    in the lane (the transposing loads fetch the rows in that order), as a
//    pair of bf16 terms (high part and remainder, two products per operand
//    read), so P enters the product with about 16 significant bits.
// When even the narrow grid does not cover the compute units, a query's rows
// are split over several workgroups, each writing an f32 partial (max, sum,
// O), and a combine kernel merges them.
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

// LDS placement of a tile of ROWS rows.  A wavefront load instruction fills
// one 1 KB block (RPI rows of D values); blocks are padded by 32 bytes, so
// rows r .. r+3 start 32 bytes apart mod 128.  For D = 512 the 16-byte chunk
// c of row r sits at chunk c ^ (bit 2 of r ^ bit 3 of r): the 8 (16) lanes
// an LDS cycle serves when 16 consecutive rows touch one chunk index then
// hit 8 (16) distinct 16-byte bank groups, and the transposing reads (4 rows
// of 32 bytes per 16 lanes, rows 4k .. 4k+3) share one permutation.
template <int D, int ROWS>
struct Tile {
  static constexpr int LPR = D / 8;      // 16-byte chunks per row
  static constexpr int RPI = 64 / LPR;   // rows per load instruction
  static constexpr int kBlkBytes = 1024 + 32;
  static constexpr int kBlocks = ROWS / RPI;
  static constexpr int kBufBytes = kBlocks * kBlkBytes;
  static __device__ __forceinline__ int row_off(int r) {
    return (r / RPI) * kBlkBytes + (r % RPI) * (2 * D);
  }
  static __device__ __forceinline__ int swz(int r) {
    return D == 512 ? (((r >> 2) ^ (r >> 3)) & 1) : 0;
  }
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

// The same for N = 1, 2 or 4 M-tiles.
template <int N>
__device__ __forceinline__ void tr_load(u32x2 (&t)[2 * N], uint32_t lo, uint32_t hi) {
  if constexpr (N == 4) {
    tr_load4(t, lo, hi);
  } else if constexpr (N == 2) {
    asm volatile(
        "ds_read_b64_tr_b16 %0, %4\n\t"
        "ds_read_b64_tr_b16 %1, %5\n\t"
        "ds_read_b64_tr_b16 %2, %4 offset:32\n\t"
        "ds_read_b64_tr_b16 %3, %5 offset:32\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(t[0]), "=&v"(t[1]), "=&v"(t[2]), "=&v"(t[3])
        : "v"(lo), "v"(hi)
        : "memory");
  } else {
    asm volatile(
        "ds_read_b64_tr_b16 %0, %2\n\t"
        "ds_read_b64_tr_b16 %1, %3\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(t[0]), "=&v"(t[1])
        : "v"(lo), "v"(hi)
        : "memory");
  }
}

__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Compacts the usable entries of an idx row (0 <= ix < total_rows, in their
// order) into list and returns how many there are.  Every thread of the
// workgroup (kW wavefronts) calls it; each wavefront scans a contiguous share
// of the row.
struct NoHook {
  __device__ __forceinline__ void operator()() const {}
};

// mid() runs between the two barriers (every wavefront has passed the first,
// none the second).
template <int kW, class Mid = NoHook>
__device__ __forceinline__ uint32_t compact_idx(const int32_t* __restrict__ irow, int width,
                                                int64_t total_rows, int32_t* list,
                                                uint32_t* wave_cnt, int wave, int lane,
                                                Mid mid = Mid()) {
  const int per_wave = ((width + kW * kWave - 1) / (kW * kWave)) * kWave;
  const int w0 = wave * per_wave;
  int w1 = w0 + per_wave;
  if (w1 > width) w1 = width;
  uint32_t cnt = 0;
  for (int i0 = w0; i0 < w1; i0 += kWave) {
    const int i = i0 + lane;
    const int32_t ix = (i < w1) ? irow[i] : -1;
    const bool ok = ix >= 0 && (int64_t)ix < total_rows;
    cnt += __popcll(__ballot(ok));
  }
  if (lane == 0) wave_cnt[wave] = cnt;
  __syncthreads();
  mid();
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
  __syncthreads();
  uint32_t n_valid = 0;
  for (int w = 0; w < kW; ++w) n_valid += wave_cnt[w];
  return n_valid;
}

// One 32-row tile of the wide form into the LDS buffer dst: rows
// base_pos .. base_pos+31 of the compacted list (rows past n_valid repeat the
// first valid row: finite data whose probability is 0).  For D = 512 each
// wavefront's eight row indices come from one LDS read and go to the row
// loads by readlane.  (A function template rather than a lambda: the host
// pass drops kernels whose lambdas hold discarded constexpr branches.)
// 16 bytes per lane from src into LDS at dst + 16 lane (global_load_lds_dwordx4).
__device__ __forceinline__ void dma16(const uint16_t* src, uint8_t* dst) {
  __builtin_amdgcn_global_load_lds(src, (lds_void*)(size_t)dst, 16, 0, 0);
}

__device__ __forceinline__ int lane_value(int v, int j) { return __builtin_amdgcn_readlane(v, j); }

template <int D>
__device__ __forceinline__ void wide_gather(uint8_t* dst, int base_pos, const int32_t* list,
                                            uint32_t n_valid, int wave, int lane,
                                            const uint16_t* a_base, const uint16_t* b_base,
                                            int64_t rows_a_len) {
  using TL = Tile<D, kTile>;
  constexpr int kW = kThreads / kWave;
  if constexpr (TL::RPI == 1) {
    constexpr int kPer = TL::kBlocks / kW;
    int pos = base_pos + wave + kW * (lane % kPer);
    if ((uint32_t)pos >= n_valid) pos = 0;
    const int32_t my_ix = list[pos];
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      const int bk = wave + kW * j;
      const int64_t ix = lane_value(my_ix, j);
      const uint16_t* src = (ix < rows_a_len) ? a_base + ix * D : b_base + (ix - rows_a_len) * D;
      dma16(src + 8 * (lane ^ TL::swz(bk)), dst + bk * TL::kBlkBytes);
    }
  } else {
#pragma unroll
    for (int bk = wave; bk < TL::kBlocks; bk += kW) {
      const int r = bk * TL::RPI + lane / TL::LPR;
      const int c = (lane % TL::LPR) ^ TL::swz(r);
      int pos = base_pos + r;
      if ((uint32_t)pos >= n_valid) pos = 0;
      const int64_t ix = list[pos];
      const uint16_t* src = (ix < rows_a_len) ? a_base + ix * D : b_base + (ix - rows_a_len) * D;
      dma16(src + 8 * c, dst + bk * TL::kBlkBytes);
    }
  }
}

template <int N>
__device__ __forceinline__ void wait_vm() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// NS: LDS ring depth in tiles (NS - 1 tiles in flight ahead of the one in use).
// Maximum / sum over the four lanes 16 apart (the k-groups of an MFMA
// operand), on the permlane swaps.
__device__ __forceinline__ float group_max(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false,
                                                  false);
  v = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
  const auto t = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false,
                                                  false);
  return fmaxf(__uint_as_float(t[0]), __uint_as_float(t[1]));
}
__device__ __forceinline__ float group_sum(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false,
                                                  false);
  v = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  const auto t = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false,
                                                  false);
  return __uint_as_float(t[0]) + __uint_as_float(t[1]);
}

template <int D, int NS>
__global__ __launch_bounds__(kThreads, NS == 2 ? 2 : 1) void attn_kernel(Params p) {
  using TL = Tile<D, kTile>;
  constexpr int KS = D / 32;  // QK K-steps
  constexpr int MT = D / 16;  // PV M-tiles (dims)
  constexpr int kPerWave = TL::kBlocks / (kThreads / kWave);  // loads per tile and wavefront
  static_assert(NS >= 2 && NS <= 4, "ring depth");
  __shared__ __attribute__((aligned(16))) uint8_t tiles[NS * TL::kBufBytes];
  __shared__ int32_t list[kMaxWidth];
  __shared__ uint32_t wave_cnt[kThreads / kWave];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int r16 = lane & 15;
  const int g = lane >> 4;
  // queries in reverse order: in a chunk the later tokens see more rows, so
  // the longest workgroups start first and the short ones fill the tail
  const int64_t unit = (int64_t)(gridDim.x - 1 - blockIdx.x);
  const int64_t qi = unit / p.splits;
  const int split = (int)(unit - qi * p.splits);
  const int64_t b = qi / p.n_tokens;
  const int head = blockIdx.y * kHeadsPerBlock + 16 * wave + r16;
  const bool head_ok = head < p.n_heads;
  // the sink goes out with the first loads (read where it is first needed,
  // after the prologue's waits, it cost a memory latency of its own)
  const float sink_in = p.sink[head_ok ? head : 0];  // zeroed below past n_heads
  const int64_t total_rows = p.rows_a_len + p.rows_b_len;

  // ---- query fragments (B operand of S^T = G Q^T): head r16, dims 32kk+8g..
  // requested before the idx row, so the two latencies overlap.  For D = 512
  // each wavefront pulls its 16 head rows (16 KB, contiguous) into its part
  // of the idle tile buffers with 1 KB direct-to-LDS loads and reads the
  // fragments back between the compaction's barriers (whose second barrier
  // then frees the buffers for the gather); 16-byte register loads spread
  // over 16 head rows measured slow.
  constexpr int kQStride = 2 * D + 16;  // padded rows: the fragment reads spread over banks
  bf16x8 qf[KS];
  uint32_t n_valid;
  if constexpr (D == 512) {
    static_assert(kHeadsPerBlock * kQStride <= NS * TL::kBufBytes, "query staging");
    const int hbase = blockIdx.y * kHeadsPerBlock;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int h = 16 * wave + j;
      const int hh = (hbase + h < p.n_heads) ? hbase + h : 0;  // finite rows past n_heads
      dma16(p.q + (qi * p.n_heads + hh) * D + 8 * lane, tiles + h * kQStride);
    }
    n_valid = compact_idx<kThreads / kWave>(
        p.idx + qi * p.idx_ld, p.width, total_rows, list, wave_cnt, wave, lane, [&]() {
          wait_vm<0>();
          const uint8_t* const qrow = tiles + (16 * wave + r16) * kQStride + 16 * g;
#pragma unroll
          for (int kk = 0; kk < KS; ++kk)
            qf[kk] = as_bf16x8(*reinterpret_cast<const u32x4*>(qrow + 64 * kk));
        });
  } else {
    const uint16_t* qp = p.q + (qi * p.n_heads + (head_ok ? head : 0)) * D + 8 * g;
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) {
      u32x4 v = {0u, 0u, 0u, 0u};
      if (head_ok) v = *reinterpret_cast<const u32x4*>(qp + 32 * kk);
      qf[kk] = as_bf16x8(v);
    }
    n_valid = compact_idx<kThreads / kWave>(p.idx + qi * p.idx_ld, p.width, total_rows, list,
                                            wave_cnt, wave, lane);
  }
  const int n_tiles = (int)((n_valid + kTile - 1) / kTile);
  const int tps = (n_tiles + p.splits - 1) / p.splits;
  const int t_begin = split * tps;
  const int t_end = (t_begin + tps < n_tiles) ? t_begin + tps : n_tiles;

  const uint16_t* a_base = p.rows_a + b * p.a_bs;
  const uint16_t* b_base = p.rows_b + b * p.b_bs;
  const float sink2 = head_ok ? sink_in * kLog2e : 0.0f;
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

  // the query loads land before the ring's loads go out, so the waits below
  // count ring loads only (each empty asm makes the compiler wait here)
#pragma unroll
  for (int kk = 0; kk < KS; ++kk) asm volatile("" : "+v"(qf[kk]));
  asm volatile("" ::"v"(sink2));
  const int nt = t_end > t_begin ? t_end - t_begin : 0;
#pragma unroll
  for (int st = 0; st < NS - 1; ++st)
    if (st < nt)
      wide_gather<D>(tiles + st * TL::kBufBytes, (t_begin + st) * kTile, list, n_valid, wave,
                     lane, a_base, b_base, p.rows_a_len);
  for (int k = 0; k < nt; ++k) {
    const int tile = t_begin + k;
    const int buf = k % NS;
    // tiles issued after this one: min(NS - 2, nt - 1 - k)
    const int ahead = (nt - 1 - k < NS - 2) ? nt - 1 - k : NS - 2;
    if (ahead <= 0) wait_vm<0>();
    else if (ahead == 1) wait_vm<kPerWave>();
    else wait_vm<2 * kPerWave>();
    lds_barrier();
    if (k + NS - 1 < nt)
      wide_gather<D>(tiles + ((k + NS - 1) % NS) * TL::kBufBytes, (tile + NS - 1) * kTile, list,
                     n_valid, wave, lane, a_base, b_base, p.rows_a_len);
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
    mx = group_max(mx);
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
    // probabilities as a bf16 pair (high part and remainder): P enters the
    // product with about 16 significant bits
    bf16x8 pf, pr;
    float psum = 0.0f;
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const float pv = (sv[s] == kNegInf) ? 0.0f : __builtin_amdgcn_exp2f(sv[s] - m2);
      psum += pv;
      const __bf16 h = (__bf16)pv;
      pf[s] = h;
      pr[s] = (__bf16)(pv - (float)h);
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
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const u32x4 a = {t[2 * j][0], t[2 * j][1], t[2 * j + 1][0], t[2 * j + 1][1]};
        acc_o[mt0 + j] = mfma16x16x32(as_bf16x8(a), pr, acc_o[mt0 + j]);
      }
    }
  }

  // ---- epilogue: lane holds O^T[dims 16mt + 4g + i][head r16]
  float l_tot = l_part;
  l_tot = group_sum(l_tot);
  if constexpr (D == 512) {
    if (p.splits == 1) {
      // the 64 heads' bf16 rows go through the (now idle) tile buffers and
      // leave as the query's contiguous output block, 16 bytes per lane
      // (8-byte stores spread over 16 head rows measured slow); rows are
      // padded by 16 bytes so the 16 head rows of a store hit distinct banks
      constexpr int kOStride = 2 * D + 16;
      static_assert(kHeadsPerBlock * kOStride <= NS * TL::kBufBytes, "output staging");
      const float sink_term = (sink2 == kNegInf) ? 0.0f : exp2f(sink2 - m2);
      const float den = l_tot + sink_term;
      const float inv = den > 0.0f ? 1.0f / den : 0.0f;
      lds_barrier();  // every wavefront is done with the last tile
      uint8_t* const orow = tiles + (16 * wave + r16) * kOStride + 8 * g;
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        uint2 v;
        v.x = f32_to_bf16_bits(acc_o[mt][0] * inv) | (f32_to_bf16_bits(acc_o[mt][1] * inv) << 16);
        v.y = f32_to_bf16_bits(acc_o[mt][2] * inv) | (f32_to_bf16_bits(acc_o[mt][3] * inv) << 16);
        *reinterpret_cast<uint2*>(orow + 32 * mt) = v;
      }
      lds_barrier();
      const int hbase = blockIdx.y * kHeadsPerBlock;
      const int nh = (p.n_heads - hbase < kHeadsPerBlock) ? p.n_heads - hbase : kHeadsPerBlock;
      uint16_t* const qout = p.out + (qi * p.n_heads + hbase) * D;
      constexpr int kCPR = D / 8;  // 16-byte chunks per head row
      for (int e = tid; e < nh * kCPR; e += kThreads) {
        const int h = e / kCPR, c = e - h * kCPR;
        *reinterpret_cast<u32x4*>(qout + h * D + 8 * c) =
            *reinterpret_cast<const u32x4*>(tiles + h * kOStride + 16 * c);
      }
      return;
    }
  }
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

// ---------------------------------------------------------------- narrow form
// Few queries (decode): a workgroup takes one query, 16 heads and the query's
// rows (or one split of them), so a query spreads over several compute units
// without partial results.  The workgroups of one row set sit 8 apart in the
// grid (one XCD under round-robin dispatch) and share its rows in that L2.
// Eight wavefronts (two per SIMD, so one hides the other's latencies) each
// work alone on every eighth 16-row tile, with their own online softmax, and
// are merged at the end:
//  * the 16 heads' queries sit in LDS and feed the QK B operand;
//  * a tile's rows are loaded one tile ahead into registers.  For D = 512 a
//    load instruction fetches one whole 1 KB row (a lane per 16-byte chunk):
//    loads laid out as the QK operand (16 rows x 64 bytes per instruction)
//    were measured 2.3x slower on this gather;
//  * the rows go to the wavefront's own LDS slot, come back in the QK A
//    layout (ds_read_b128; for D < 512 they are loaded in that layout and
//    used from registers) and come back transposed (ds_read_b64_tr_b16) as
//    the A operand of O^T += G^T P^T, all D dims;
//  * QK: 16 rows x 16 heads over four independent accumulators; the S
//    accumulator is laid out as the B operand of a 16-row PV product, so
//    the probabilities never leave the lane.  They enter as a bf16 pair
//    (high part and remainder) stacked on K of one 16x16x32 product whose A
//    operand holds the transposed rows twice: O^T += [G^T G^T] [P_hi; P_lo].
//    On this chip a 16x16x16 product takes as long as a 16x16x32 one, so the
//    pair costs no more than a single bf16 P;
//  * head maxima and sums across the lane groups use permlane swaps;
//  * no barrier inside the loop; at the end the eight (max, sum, O) are
//    merged through LDS, half of the dims at a time.
constexpr int kWaveRows = 16;
constexpr int kNarrowHeads = 16;
constexpr int kNarrowThreads = 512;

// One 16x16x32 product sums a_lane[s] * b_lane'[s] over the four lane
// groups and the eight slots s, pairing the operands' slots one to one
// (whatever k each names).  With the four values of a repeated in slots 4-7
// and b = {four high parts, four remainders}, c += a * (b_hi + b_lo) over
// the 16 rows of a 16x16x16 product.
__device__ __forceinline__ f32x4 mfma_pair(u32x2 a, u32x4 b, f32x4 c) {
  const u32x4 aa = {a[0], a[1], a[0], a[1]};
  return mfma16x16x32(as_bf16x8(aa), as_bf16x8(b), c);
}

// Eight ds_read_b64_tr_b16 at 32-byte steps (eight 16-dim M-tiles of one
// 16-row K block) and a wait for them.
__device__ __forceinline__ void tr_load8(u32x2 (&t)[8], uint32_t a) {
  asm volatile(
      "ds_read_b64_tr_b16 %0, %8\n\t"
      "ds_read_b64_tr_b16 %1, %8 offset:32\n\t"
      "ds_read_b64_tr_b16 %2, %8 offset:64\n\t"
      "ds_read_b64_tr_b16 %3, %8 offset:96\n\t"
      "ds_read_b64_tr_b16 %4, %8 offset:128\n\t"
      "ds_read_b64_tr_b16 %5, %8 offset:160\n\t"
      "ds_read_b64_tr_b16 %6, %8 offset:192\n\t"
      "ds_read_b64_tr_b16 %7, %8 offset:224\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(t[0]), "=&v"(t[1]), "=&v"(t[2]), "=&v"(t[3]), "=&v"(t[4]), "=&v"(t[5]),
        "=&v"(t[6]), "=&v"(t[7])
      : "v"(a)
      : "memory");
}

__device__ __forceinline__ void tr_load4_1(u32x2 (&t)[4], uint32_t a) {
  asm volatile(
      "ds_read_b64_tr_b16 %0, %4\n\t"
      "ds_read_b64_tr_b16 %1, %4 offset:32\n\t"
      "ds_read_b64_tr_b16 %2, %4 offset:64\n\t"
      "ds_read_b64_tr_b16 %3, %4 offset:96\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(t[0]), "=&v"(t[1]), "=&v"(t[2]), "=&v"(t[3])
      : "v"(a)
      : "memory");
}

// A wavefront's 16-row LDS slot: rows 2D + 32 bytes apart (rows r .. r+3 at
// distinct 32-byte bank groups mod 128); 16-byte chunk c of row r at chunk
// c ^ (bit 2 of r ^ bit 3 of r), so the row stores (8 or 16 rows, one chunk
// index per LDS cycle) and the transposing reads (rows 4k .. 4k+3, 32 bytes
// each, per 16 lanes) are both free of bank conflicts.
template <int D>
struct WaveSlot {
  static constexpr int kStride = 2 * D + 32;
  static constexpr int kBytes = kWaveRows * kStride;
  static __device__ __forceinline__ int swz(int r) { return ((r >> 2) ^ (r >> 3)) & 1; }
};

template <int D>
__global__ __launch_bounds__(kNarrowThreads, 1) void attn_narrow_kernel(Params p,
                                                                        int32_t head_groups,
                                                                        int64_t n_units) {
  using WS = WaveSlot<D>;
  constexpr int kW = kNarrowThreads / kWave;
  constexpr int KS = D / 32;     // QK K-steps (16-byte chunks per lane and row)
  constexpr int DT = D / 16;     // PV M-tiles (all dims)
  constexpr int kHalfDT = DT / 2;
  constexpr int kQStride = 2 * D + 16;  // bytes per head row of the query tile
  static_assert(kW * kHalfDT * kWave * 16 <= kW * WS::kBytes, "merge area");
  static_assert(D != 512 || KS == kWaveRows, "one register per tile row");
  __shared__ __attribute__((aligned(16))) uint8_t slots[kW * WS::kBytes];
  __shared__ __attribute__((aligned(16))) uint8_t qs[kNarrowHeads * kQStride];
  __shared__ int32_t ixs[kMaxWidth];  // the idx row, entries outside the sources as -1
  __shared__ float xm[kW][kNarrowHeads];
  __shared__ float xl[kW][kNarrowHeads];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r16 = lane & 15;
  const int g = lane >> 4;
  const int grp = blockIdx.x >> 3;
  const int hg = grp % head_groups;
  const int64_t unit = (int64_t)(grp / head_groups) * 8 + (blockIdx.x & 7);
  if (unit >= n_units) return;  // whole workgroup
  const int64_t qi = unit / p.splits;
  const int split = (int)(unit - qi * p.splits);
  const int64_t b = qi / p.n_tokens;
  const int head = hg * kNarrowHeads + r16;
  const bool head_ok = head < p.n_heads;
  const int64_t total_rows = p.rows_a_len + p.rows_b_len;

  // Tiles are 16 consecutive entries of the idx row itself (no compaction):
  // an entry outside the two sources loads row 0 and gets probability 0.
  const int n_tiles = total_rows > 0 ? (p.width + kWaveRows - 1) / kWaveRows : 0;
  const int tps = (n_tiles + p.splits - 1) / p.splits;
  const int t_begin = split * tps;
  const int t_end = (t_begin + tps < n_tiles) ? t_begin + tps : n_tiles;
  const int nt = t_end > t_begin ? t_end - t_begin : 0;
  const int32_t* const irow = p.idx + qi * p.idx_ld;
  // wavefront w takes tiles w, w + 8, ... (handing tiles out through an LDS
  // counter measured 2% slower with this prologue)

  // ---- a lane's share of a tile: entry r16 of the tile.  Returns the tile's
  // 16-bit validity mask (bit r: entry r names a row).
  const uint16_t* a_base = p.rows_a + b * p.a_bs;
  const uint16_t* b_base = p.rows_b + b * p.b_bs;
  //  D = 512: rb[j] = row j of the tile, lane l holding its chunk l ^ swz(j)
  //  (the slot position of chunk l); otherwise rb[kk] = chunk 4kk + g of row r16
  auto load = [&](int32_t raw, u32x4 (&rb)[KS]) -> uint32_t {
    const bool ok = raw >= 0 && (int64_t)raw < total_rows;
    const uint32_t vm = (uint32_t)__ballot(ok) & 0xFFFFu;
    const int32_t my_ix = ok ? raw : 0;
    if constexpr (D == 512) {
#pragma unroll
      for (int j = 0; j < kWaveRows; ++j) {
        const int64_t ix = __builtin_amdgcn_readlane(my_ix, j);
        const uint16_t* src =
            (ix < p.rows_a_len) ? a_base + ix * D : b_base + (ix - p.rows_a_len) * D;
        rb[j] = *reinterpret_cast<const u32x4*>(src + 8 * (lane ^ WS::swz(j)));
      }
    } else {
      const int64_t ix = my_ix;
      const uint16_t* src =
          ((ix < p.rows_a_len) ? a_base + ix * D : b_base + (ix - p.rows_a_len) * D) + 8 * g;
#pragma unroll
      for (int kk = 0; kk < KS; ++kk) rb[kk] = *reinterpret_cast<const u32x4*>(src + 32 * kk);
    }
    return vm;
  };
  auto entry = [&](int tile) -> int {  // this lane's position in the idx row
    return (t_begin + tile) * kWaveRows + r16;
  };

  // ---- prologue: the first tile's entries, the idx row and the 16 heads'
  // queries (zero rows past n_heads) are all requested before anything waits,
  // then the first tile's rows go out; one barrier publishes the LDS copies
  int cur = wave;
  int32_t raw0 = -1;
  if (cur < nt && entry(cur) < p.width) raw0 = irow[entry(cur)];
  constexpr int kIxPer = kMaxWidth / kNarrowThreads;
  int32_t iv[kIxPer];
#pragma unroll
  for (int j = 0; j < kIxPer; ++j) {
    const int i = tid + j * kNarrowThreads;
    iv[j] = (i < p.width) ? irow[i] : -1;
  }
  constexpr int CPR = D / 8;
  constexpr int kQPer = (kNarrowHeads * CPR + kNarrowThreads - 1) / kNarrowThreads;
  u32x4 qv[kQPer];
  const uint16_t* q0 = p.q + (qi * p.n_heads + hg * kNarrowHeads) * D;
#pragma unroll
  for (int j = 0; j < kQPer; ++j) {
    const int e = tid + j * kNarrowThreads;
    const int h = e / CPR, c = e % CPR;
    qv[j] = (u32x4){0u, 0u, 0u, 0u};
    if (e < kNarrowHeads * CPR && hg * kNarrowHeads + h < p.n_heads)
      qv[j] = *reinterpret_cast<const u32x4*>(q0 + h * D + 8 * c);
  }
  u32x4 rb[KS];
  uint32_t vm_cur = 0u;
  if (cur < nt) vm_cur = load(raw0, rb);
#pragma unroll
  for (int j = 0; j < kQPer; ++j) {
    const int e = tid + j * kNarrowThreads;
    const int h = e / CPR, c = e % CPR;
    if (e < kNarrowHeads * CPR) *reinterpret_cast<u32x4*>(qs + h * kQStride + 16 * c) = qv[j];
  }
#pragma unroll
  for (int j = 0; j < kIxPer; ++j) {
    const int i = tid + j * kNarrowThreads;
    if (i < p.width) ixs[i] = (iv[j] >= 0 && (int64_t)iv[j] < total_rows) ? iv[j] : -1;
  }
  __syncthreads();

  const float sink2 = head_ok ? p.sink[head] * kLog2e : 0.0f;
  const float kNegInf = -__builtin_huge_valf();
  float m2 = sink2;  // this wavefront's reference max on the log2 scale
  float l_part = 0.0f;
  f32x4 acc_o[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) acc_o[dt] = (f32x4){0.f, 0.f, 0.f, 0.f};

  uint8_t* const slot = slots + wave * WS::kBytes;
  const int st_off = r16 * WS::kStride + 16 * (g ^ WS::swz(r16));  // + 64 kk
  const uint8_t* const q_frag = qs + r16 * kQStride + 16 * g;      // + 64 kk
  //  transposing loads: lane (g, j, q) reads 8 bytes of row 4g + j at dims 4q..
  const int tj = (lane >> 2) & 3, tq = lane & 3;
  const int tr_row = 4 * g + tj;
  const uint32_t tr_addr = (uint32_t)(size_t)(lds_void*)(size_t)(
      slot + tr_row * WS::kStride + 16 * ((tq >> 1) ^ WS::swz(tr_row)) + 8 * (tq & 1));

  while (cur < nt) {
    const int nxt = cur + kW;
    uint32_t vm_nxt = 0u;
    // S^T: rows 4g + e of the tile, head r16
    f32x4 sa[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) sa[c] = (f32x4){0.f, 0.f, 0.f, 0.f};
    if constexpr (D == 512) {
      // rows to the slot, the next tile's loads out, then QK from the slot
#pragma unroll
      for (int j = 0; j < kWaveRows; ++j)
        *reinterpret_cast<u32x4*>(slot + j * WS::kStride + 16 * lane) = rb[j];
      if (nxt < nt) vm_nxt = load(entry(nxt) < p.width ? ixs[entry(nxt)] : -1, rb);
#pragma unroll
      for (int kk = 0; kk < KS; ++kk) {
        const u32x4 qv = *reinterpret_cast<const u32x4*>(q_frag + 64 * kk);
        const u32x4 av = *reinterpret_cast<const u32x4*>(slot + st_off + 64 * kk);
        sa[kk & 3] = mfma16x16x32(as_bf16x8(av), as_bf16x8(qv), sa[kk & 3]);
      }
    } else {
#pragma unroll
      for (int kk = 0; kk < KS; ++kk) {
        const u32x4 qv = *reinterpret_cast<const u32x4*>(q_frag + 64 * kk);
        sa[kk & 3] = mfma16x16x32(as_bf16x8(rb[kk]), as_bf16x8(qv), sa[kk & 3]);
      }
#pragma unroll
      for (int kk = 0; kk < KS; ++kk) *reinterpret_cast<u32x4*>(slot + st_off + 64 * kk) = rb[kk];
      if (nxt < nt) vm_nxt = load(entry(nxt) < p.width ? ixs[entry(nxt)] : -1, rb);
    }
    const f32x4 sacc = (sa[0] + sa[1]) + (sa[2] + sa[3]);

    float sv[4];
    float mx = kNegInf;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      float v = sacc[e] * p.scale_log2;
      if (!((vm_cur >> (4 * g + e)) & 1u)) v = kNegInf;
      sv[e] = v;
      mx = fmaxf(mx, v);
    }
    mx = group_max(mx);
    if (__any(mx > m2 + kRescaleLog2)) {
      const float m_new = fmaxf(m2, mx);
      const float alpha = (m_new == m2) ? 1.0f : exp2f(m2 - m_new);
      m2 = m_new;
      l_part *= alpha;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) acc_o[dt] *= alpha;
    }
    // probabilities as a bf16 pair (high part pk and remainder pl)
    u32x2 pk, pl;
#pragma unroll
    for (int e = 0; e < 4; e += 2) {
      const float p0 = (sv[e] == kNegInf) ? 0.0f : __builtin_amdgcn_exp2f(sv[e] - m2);
      const float p1 = (sv[e + 1] == kNegInf) ? 0.0f : __builtin_amdgcn_exp2f(sv[e + 1] - m2);
      l_part += p0 + p1;
      const __bf16 b0 = (__bf16)p0, b1 = (__bf16)p1;
      const __bf16 c0 = (__bf16)(p0 - (float)b0), c1 = (__bf16)(p1 - (float)b1);
      pk[e / 2] = (uint32_t)__builtin_bit_cast(uint16_t, b0) |
                  ((uint32_t)__builtin_bit_cast(uint16_t, b1) << 16);
      pl[e / 2] = (uint32_t)__builtin_bit_cast(uint16_t, c0) |
                  ((uint32_t)__builtin_bit_cast(uint16_t, c1) << 16);
    }
    // O^T[dims][head] += G^T[dims][16 rows] (P_hi + P_lo)^T[16 rows][head]
    const u32x4 pp = {pk[0], pk[1], pl[0], pl[1]};
    if constexpr (DT >= 8) {
#pragma unroll
      for (int d0 = 0; d0 < DT; d0 += 8) {
        u32x2 t[8];
        tr_load8(t, tr_addr + 32 * d0);
#pragma unroll
        for (int j = 0; j < 8; ++j) acc_o[d0 + j] = mfma_pair(t[j], pp, acc_o[d0 + j]);
      }
    } else {
      u32x2 t[4];
      tr_load4_1(t, tr_addr);
#pragma unroll
      for (int j = 0; j < DT; ++j) acc_o[j] = mfma_pair(t[j], pp, acc_o[j]);
    }
    cur = nxt;
    vm_cur = vm_nxt;
  }

  // ---- merge the wavefronts: M = max m_w, O = sum 2^(m_w - M) O_w,
  // l = sum 2^(m_w - M) l_w.  Each wavefront's half of O goes, unscaled,
  // into its own slot (free once its last tile is done), so the first half
  // is written before the barrier, while other wavefronts still work.
  const float l_w = group_sum(l_part);
  if (g == 0) {
    xm[wave][r16] = m2;
    xl[wave][r16] = l_w;
  }
  static_assert(kHalfDT * kWave * 16 <= WS::kBytes, "half of O fits a slot");
  // [wave slot][half dim-tile][lane]
  auto merge_at = [&](int w, int j) -> f32x4* {
    return reinterpret_cast<f32x4*>(slots + w * WS::kBytes) + j * kWave + lane;
  };
#pragma unroll
  for (int j = 0; j < kHalfDT; ++j) *merge_at(wave, j) = acc_o[j];
  lds_barrier();
  float M = kNegInf;
#pragma unroll
  for (int w = 0; w < kW; ++w) M = fmaxf(M, xm[w][r16]);
  float l_tot = 0.0f;
  float wt[kW];  // 2^(m_w - M) of head r16, 0 for a wavefront without rows
#pragma unroll
  for (int w = 0; w < kW; ++w) {
    const float mw = xm[w][r16];
    wt[w] = (mw == kNegInf) ? 0.0f : exp2f(mw - M);
    l_tot += xl[w][r16] * wt[w];
  }
  const float sink_term = (sink2 == kNegInf) ? 0.0f : exp2f(sink2 - M);
  const float den = l_tot + sink_term;
  const float inv = den > 0.0f ? 1.0f / den : 0.0f;
  constexpr int kPerWave = kHalfDT / kW;  // dim-tiles each wavefront finishes per half
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    if (h == 1) {
#pragma unroll
      for (int j = 0; j < kHalfDT; ++j) *merge_at(wave, j) = acc_o[kHalfDT + j];
      lds_barrier();
    }
    if (kPerWave > 0 || wave < kHalfDT) {
      const int j0 = kPerWave > 0 ? wave * kPerWave : wave;
      const int jn = kPerWave > 0 ? kPerWave : 1;
      for (int jj = 0; jj < jn; ++jj) {
        const int j = j0 + jj;
        f32x4 o = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int w = 0; w < kW; ++w) o += *merge_at(w, j) * wt[w];
        const int dim = 16 * (h * kHalfDT + j) + 4 * g;  // lane: dims dim .. dim+3, head r16
        if (!head_ok) continue;
        if (p.splits == 1) {
          uint2 v;
          v.x = f32_to_bf16_bits(o[0] * inv) | (f32_to_bf16_bits(o[1] * inv) << 16);
          v.y = f32_to_bf16_bits(o[2] * inv) | (f32_to_bf16_bits(o[3] * inv) << 16);
          *reinterpret_cast<uint2*>(p.out + (qi * p.n_heads + head) * D + dim) = v;
        } else {
          const int64_t slot_i = (qi * p.splits + split) * p.n_heads + head;
          *reinterpret_cast<f32x4*>(p.part_o + slot_i * D + dim) = o;
        }
      }
    }
    if (h == 0) lds_barrier();  // every wavefront has read the first half
  }
  if (p.splits > 1 && head_ok && wave == 0 && g == 0) {
    const int64_t slot_i = (qi * p.splits + split) * p.n_heads + head;
    p.part_ml[2 * slot_i] = M;
    p.part_ml[2 * slot_i + 1] = l_tot;
  }
}

// ---------------------------------------------------------------- round form
// The narrow form for D = 512 without the final merge: a workgroup (query,
// 16 heads, eight wavefronts) takes the query's rows in rounds of 128 (eight
// 16-row tiles, tile r * 8 + w to wavefront w).  In a round each wavefront
//  * stores its tile (loaded two rounds ahead into registers, a 1 KB row per
//    load instruction) into its LDS slot and sends the loads of round + 2;
//  * computes S^T (16 rows x 16 heads) from the slot and the query tile and
//    writes it, scaled to the log2 domain, into a shared [head][row] array;
// then, after a barrier, every wavefront reads the round's 128 scores of the
// 16 heads, takes the same running maximum and probabilities (identical
// arithmetic in every wavefront, so they agree exactly), and computes
// O^T += G^T P^T for its own 64 of the 512 dims over the 128 rows, on
// v_mfma_f32_16x16x32_bf16 (32 rows per K-step: transposing reads of two
// tiles), with P as a pair of bf16 terms (high part and remainder).  Each
// wavefront ends with the finished output of its dims.
constexpr int kRoundTiles = 8;
constexpr int kRoundRows = kRoundTiles * kWaveRows;
constexpr int kSxStride = kRoundRows + 4;  // floats per head row (bank spread)

__global__ __launch_bounds__(kNarrowThreads, 1) void attn_round_kernel(Params p,
                                                                       int32_t head_groups,
                                                                       int64_t n_units) {
  constexpr int D = 512;
  using WS = WaveSlot<D>;
  constexpr int kW = kNarrowThreads / kWave;
  static_assert(kW == kRoundTiles, "one tile per wavefront and round");
  constexpr int KS = D / 32;                 // QK K-steps (one per tile row register)
  constexpr int kQStride = 2 * D + 16;
  constexpr int kDimsPerWave = D / kW;       // 64
  constexpr int DT = kDimsPerWave / 16;      // 4 output dim-tiles per wavefront
  static_assert(KS == kWaveRows, "one register per tile row");
  __shared__ __attribute__((aligned(16))) uint8_t slots[kW * WS::kBytes];
  __shared__ __attribute__((aligned(16))) uint8_t qs[kNarrowHeads * kQStride];
  __shared__ __attribute__((aligned(16))) float sx[kNarrowHeads * kSxStride];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r16 = lane & 15;
  const int g = lane >> 4;
  const int grp = blockIdx.x >> 3;
  const int hg = grp % head_groups;
  const int64_t unit = (int64_t)(grp / head_groups) * 8 + (blockIdx.x & 7);
  if (unit >= n_units) return;  // whole workgroup
  const int64_t qi = unit / p.splits;
  const int split = (int)(unit - qi * p.splits);
  const int64_t b = qi / p.n_tokens;
  const int head = hg * kNarrowHeads + r16;
  const bool head_ok = head < p.n_heads;
  // the sink goes out with the first loads (read where it is first needed,
  // after the prologue's waits, it cost a memory latency of its own)
  const float sink_in = p.sink[head_ok ? head : 0];  // zeroed below past n_heads
  const int64_t total_rows = p.rows_a_len + p.rows_b_len;

  // tiles are 16 consecutive entries of the idx row (an entry outside the
  // two sources loads row 0 and is masked); the split's tiles run in rounds
  const int n_tiles = total_rows > 0 ? (p.width + kWaveRows - 1) / kWaveRows : 0;
  const int tps = (n_tiles + p.splits - 1) / p.splits;
  const int t_begin = split * tps;
  const int t_end = (t_begin + tps < n_tiles) ? t_begin + tps : n_tiles;
  const int nt = t_end > t_begin ? t_end - t_begin : 0;
  const int n_rounds = (nt + kRoundTiles - 1) / kRoundTiles;
  const int32_t* const irow = p.idx + qi * p.idx_ld;
  const uint16_t* a_base = p.rows_a + b * p.a_bs;
  const uint16_t* b_base = p.rows_b + b * p.b_bs;

  // this lane's idx entry (row r16) of round r's tile; -1 past the split
  auto entry = [&](int r) -> int32_t {
    const int tile = r * kRoundTiles + wave;
    const int pos = (t_begin + tile) * kWaveRows + r16;
    return (tile < nt && pos < p.width) ? irow[pos] : -1;
  };
  // rb[j] = row j of the tile, lane l holding its chunk l ^ swz(j); returns
  // the 16-bit validity mask
  auto load = [&](int32_t raw, u32x4 (&rb)[KS]) -> uint32_t {
    const bool ok = raw >= 0 && (int64_t)raw < total_rows;
    const uint32_t vm = (uint32_t)__ballot(ok) & 0xFFFFu;
    const int32_t my_ix = ok ? raw : 0;
#pragma unroll
    for (int j = 0; j < kWaveRows; ++j) {
      const int64_t ix = __builtin_amdgcn_readlane(my_ix, j);
      const uint16_t* src =
          (ix < p.rows_a_len) ? a_base + ix * D : b_base + (ix - p.rows_a_len) * D;
      rb[j] = *reinterpret_cast<const u32x4*>(src + 8 * (lane ^ WS::swz(j)));
    }
    return vm;
  };

  // ---- prologue: entries of rounds 0 .. 2, the queries, the rows of rounds
  // 0 and 1 (two rounds of rows stay in flight in registers)
  const int32_t ent0 = n_rounds > 0 ? entry(0) : -1;
  const int32_t ent1 = n_rounds > 1 ? entry(1) : -1;
  int32_t ent_a = n_rounds > 2 ? entry(2) : -1;  // next entries for buffer a
  int32_t ent_b = -1;                            // ... and for buffer b
  constexpr int CPR = D / 8;
  constexpr int kQPer = (kNarrowHeads * CPR + kNarrowThreads - 1) / kNarrowThreads;
  u32x4 qv[kQPer];
  const uint16_t* q0 = p.q + (qi * p.n_heads + hg * kNarrowHeads) * D;
#pragma unroll
  for (int j = 0; j < kQPer; ++j) {
    const int e = tid + j * kNarrowThreads;
    const int h = e / CPR, c = e % CPR;
    qv[j] = (u32x4){0u, 0u, 0u, 0u};
    if (e < kNarrowHeads * CPR && hg * kNarrowHeads + h < p.n_heads)
      qv[j] = *reinterpret_cast<const u32x4*>(q0 + h * D + 8 * c);
  }
  u32x4 rb_a[KS], rb_b[KS];
  uint32_t vm_a = 0u, vm_b = 0u;
  if (n_rounds > 0) vm_a = load(ent0, rb_a);
  if (n_rounds > 1) vm_b = load(ent1, rb_b);
#pragma unroll
  for (int j = 0; j < kQPer; ++j) {
    const int e = tid + j * kNarrowThreads;
    const int h = e / CPR, c = e % CPR;
    if (e < kNarrowHeads * CPR) *reinterpret_cast<u32x4*>(qs + h * kQStride + 16 * c) = qv[j];
  }

  const float sink2 = head_ok ? sink_in * kLog2e : 0.0f;
  const float kNegInf = -__builtin_huge_valf();
  float m2 = sink2;  // running reference max on the log2 scale (same in every wavefront)
  float l_part = 0.0f;
  f32x4 acc[DT];
#pragma unroll
  for (int d = 0; d < DT; ++d) acc[d] = (f32x4){0.f, 0.f, 0.f, 0.f};

  uint8_t* const slot = slots + wave * WS::kBytes;
  const int st_off = r16 * WS::kStride + 16 * (g ^ WS::swz(r16));  // + 64 kk
  const uint8_t* const q_frag = qs + r16 * kQStride + 16 * g;      // + 64 kk
  //  transposing loads: lane (g, j, q) reads 8 bytes of row 4g + j at dims
  //  4q .. (+ 32 bytes per 16-dim tile) of a slot
  const int tj = (lane >> 2) & 3, tq = lane & 3;
  const int tr_row = 4 * g + tj;
  const uint32_t tr0 = (uint32_t)(size_t)(lds_void*)(size_t)(
      slots + tr_row * WS::kStride + 16 * ((tq >> 1) ^ WS::swz(tr_row)) + 8 * (tq & 1) +
      32 * (wave * DT));
  float* const sx_w = sx + r16 * kSxStride + wave * kWaveRows + 4 * g;  // S^T rows 4g..

  // one round from the rows in rb (validity vm); rb then takes the rows of
  // round r + 2 (entry ent), and ent the entry of round r + 4
  auto round = [&](int r, u32x4 (&rb)[KS], uint32_t& vm, int32_t& ent) {
    // slots and the score array are free once every wavefront finished the
    // previous round (the first barrier also publishes the query tile)
    lds_barrier();
#pragma unroll
    for (int j = 0; j < kWaveRows; ++j)
      *reinterpret_cast<u32x4*>(slot + j * WS::kStride + 16 * lane) = rb[j];
    const uint32_t vm_cur = vm;
    if (r + 2 < n_rounds) {
      vm = load(ent, rb);
      ent = (r + 4 < n_rounds) ? entry(r + 4) : -1;
    }
    // S^T: rows 4g + e of this wavefront's tile, head r16
    f32x4 sa[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) sa[c] = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) {
      const u32x4 qq = *reinterpret_cast<const u32x4*>(q_frag + 64 * kk);
      const u32x4 av = *reinterpret_cast<const u32x4*>(slot + st_off + 64 * kk);
      sa[kk & 3] = mfma16x16x32(as_bf16x8(av), as_bf16x8(qq), sa[kk & 3]);
    }
    const f32x4 sacc = (sa[0] + sa[1]) + (sa[2] + sa[3]);
    f32x4 sv;
#pragma unroll
    for (int e = 0; e < 4; ++e)
      sv[e] = ((vm_cur >> (4 * g + e)) & 1u) ? sacc[e] * p.scale_log2 : kNegInf;
    *reinterpret_cast<f32x4*>(sx_w) = sv;
    lds_barrier();

    // the round's 128 scores of head r16: this lane's K-step values are
    // rows 32ks + 4g + e (e < 4) and 32ks + 16 + 4g + e, the order of the
    // transposing reads of tiles 2ks and 2ks + 1
    f32x4 s_lo[4], s_hi[4];
    const float* const sx_h = sx + r16 * kSxStride + 4 * g;
    float mx = kNegInf;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      s_lo[ks] = *reinterpret_cast<const f32x4*>(sx_h + 32 * ks);
      s_hi[ks] = *reinterpret_cast<const f32x4*>(sx_h + 32 * ks + 16);
#pragma unroll
      for (int e = 0; e < 4; ++e) mx = fmaxf(mx, fmaxf(s_lo[ks][e], s_hi[ks][e]));
    }
    mx = group_max(mx);
    if (mx > m2 + kRescaleLog2) {  // the same decision in every lane of a head
      const float alpha = exp2f(m2 - mx);
      m2 = mx;
      l_part *= alpha;
#pragma unroll
      for (int d = 0; d < DT; ++d) acc[d] *= alpha;
    }
    // probabilities as a bf16 pair (high part and remainder), so P enters
    // the product with about 16 significant bits
    bf16x8 pf[4], pr[4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float p0 = (s_lo[ks][e] == kNegInf) ? 0.0f : __builtin_amdgcn_exp2f(s_lo[ks][e] - m2);
        const float p1 = (s_hi[ks][e] == kNegInf) ? 0.0f : __builtin_amdgcn_exp2f(s_hi[ks][e] - m2);
        l_part += p0 + p1;
        const __bf16 h0 = (__bf16)p0, h1 = (__bf16)p1;
        pf[ks][e] = h0;
        pf[ks][4 + e] = h1;
        pr[ks][e] = (__bf16)(p0 - (float)h0);
        pr[ks][4 + e] = (__bf16)(p1 - (float)h1);
      }
    }
    // O^T[this wavefront's dims][head] += G^T[dims][32 rows] P^T[32 rows][head]
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      u32x2 t[8];
      tr_load4(t, tr0 + (2 * ks) * WS::kBytes, tr0 + (2 * ks + 1) * WS::kBytes);
#pragma unroll
      for (int d = 0; d < DT; ++d) {
        const u32x4 a = {t[2 * d][0], t[2 * d][1], t[2 * d + 1][0], t[2 * d + 1][1]};
        acc[d] = mfma16x16x32(as_bf16x8(a), pf[ks], acc[d]);
        acc[d] = mfma16x16x32(as_bf16x8(a), pr[ks], acc[d]);
      }
    }
  };
  // entries: buffer a loads rounds 0, 2, 4, ..; buffer b rounds 1, 3, 5, ..
  if (n_rounds > 3) ent_b = entry(3);
  for (int r = 0; r < n_rounds; r += 2) {
    round(r, rb_a, vm_a, ent_a);
    if (r + 1 < n_rounds) round(r + 1, rb_b, vm_b, ent_b);
  }

  // ---- epilogue: lane holds O^T[dims 64 wave + 16d + 4g + i][head r16]
  const float l_tot = group_sum(l_part);
  if (!head_ok) return;
  if (p.splits == 1) {
    const float sink_term = (sink2 == kNegInf) ? 0.0f : exp2f(sink2 - m2);
    const float den = l_tot + sink_term;
    const float inv = den > 0.0f ? 1.0f / den : 0.0f;
    uint16_t* op = p.out + (qi * p.n_heads + head) * D + kDimsPerWave * wave + 4 * g;
#pragma unroll
    for (int d = 0; d < DT; ++d) {
      uint2 v;
      v.x = f32_to_bf16_bits(acc[d][0] * inv) | (f32_to_bf16_bits(acc[d][1] * inv) << 16);
      v.y = f32_to_bf16_bits(acc[d][2] * inv) | (f32_to_bf16_bits(acc[d][3] * inv) << 16);
      *reinterpret_cast<uint2*>(op + 16 * d) = v;
    }
  } else {
    const int64_t slot_i = (qi * p.splits + split) * p.n_heads + head;
    float* po = p.part_o + slot_i * D + kDimsPerWave * wave + 4 * g;
#pragma unroll
    for (int d = 0; d < DT; ++d) *reinterpret_cast<f32x4*>(po + 16 * d) = acc[d];
    if (wave == 0 && g == 0) {
      p.part_ml[2 * slot_i] = m2;
      p.part_ml[2 * slot_i + 1] = l_tot;
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
  // splits in chunks of kChunk: a chunk's loads are all issued before any
  // returns, then its maximum updates the running one (a single chunk gives
  // exactly the two-pass form: M over the sink and every split first)
  constexpr int kChunk = 8;
  float2 ml[kChunk];
  f32x4 v[kChunk];
  auto load_chunk = [&](int s0) {
#pragma unroll
    for (int i = 0; i < kChunk; ++i) {
      ml[i] = make_float2(kNegInf, 0.0f);
      v[i] = (f32x4){0.f, 0.f, 0.f, 0.f};
      if (s0 + i < splits) {
        const int64_t slot = (qi * splits + s0 + i) * n_heads + h;
        ml[i] = *reinterpret_cast<const float2*>(part_ml + 2 * slot);
        v[i] = *reinterpret_cast<const f32x4*>(part_o + slot * D + 4 * d4);
      }
    }
  };
  // the first chunk's loads go out before the sink's, so that one memory
  // latency covers them all (read first, the sink was waited for alone)
  load_chunk(0);
  const float sink2 = sink[h] * kLog2e;
  float M = sink2;
  float den = (sink2 == kNegInf) ? 0.0f : 1.0f;  // 2^(sink - M) at M = sink
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int s0 = 0; s0 < splits; s0 += kChunk) {
    if (s0 > 0) load_chunk(s0);
    float Mc = M;
#pragma unroll
    for (int i = 0; i < kChunk; ++i) Mc = fmaxf(Mc, ml[i].x);
    if (Mc > M) {
      const float a = (M == kNegInf) ? 0.0f : exp2f(M - Mc);
      den *= a;
      acc *= a;
      M = Mc;
    }
#pragma unroll
    for (int i = 0; i < kChunk; ++i) {
      const float wgt = (ml[i].x == kNegInf) ? 0.0f : exp2f(ml[i].x - M);
      den += ml[i].y * wgt;
      acc += v[i] * wgt;
    }
  }
  const float inv = den > 0.0f ? 1.0f / den : 0.0f;
  uint2 o;
  o.x = f32_to_bf16_bits(acc[0] * inv) | (f32_to_bf16_bits(acc[1] * inv) << 16);
  o.y = f32_to_bf16_bits(acc[2] * inv) | (f32_to_bf16_bits(acc[3] * inv) << 16);
  *reinterpret_cast<uint2*>(out + (qi * n_heads + h) * D + 4 * d4) = o;
}

// The narrow form serves shapes whose wide grid (one workgroup per query and
// 64 heads) would not cover the compute units.
bool attn_narrow(int64_t queries, int32_t n_heads) {
  return queries * ((n_heads + kHeadsPerBlock - 1) / kHeadsPerBlock) < 256;
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
  if (attn_narrow(nq, a.n_heads)) {
    const int32_t hg = (a.n_heads + kNarrowHeads - 1) / kNarrowHeads;
    const int64_t units = nq * splits;
    const int64_t blocks = 8 * hg * ((units + 7) / 8);
    if (blocks > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
    // a workgroup whose rows fit one round (at most 8 tiles) takes the round
    // form: no final merge; with more rounds its two barriers per round cost
    // more than the merge saves (measured), so the wavefronts work alone
    const int64_t tiles = (a.width + kWaveRows - 1) / kWaveRows;
    const bool one_round = (tiles + splits - 1) / splits <= kRoundTiles;
    if (D == 512 && one_round)
      hipLaunchKernelGGL(attn_round_kernel, dim3((unsigned)blocks), dim3(kNarrowThreads), 0, s,
                         p, hg, units);
    else
      hipLaunchKernelGGL((attn_narrow_kernel<D>), dim3((unsigned)blocks), dim3(kNarrowThreads),
                         0, s, p, hg, units);
  } else {
    // two workgroups per CU with a two-tile ring each (a four-tile ring with
    // one workgroup per CU measured slower on row-split decode shapes)
    const dim3 grid((unsigned)(nq * splits), (unsigned)((a.n_heads + kHeadsPerBlock - 1) /
                                                        kHeadsPerBlock));
    hipLaunchKernelGGL((attn_kernel<D, 2>), grid, dim3(kThreads), 0, s, p);
  }
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
  // keeping at least 2 narrow tiles (4 wide ones) of rows per split.
  const bool narrow = attn_narrow(queries, n_heads);
  const int64_t per_wg = narrow ? kNarrowHeads : kHeadsPerBlock;
  const int64_t hg = (n_heads + per_wg - 1) / per_wg;
  const int64_t wgs = (int64_t)queries * hg;
  if (wgs >= 256) return 1;
  int64_t s = (256 + wgs - 1) / wgs;
  const int64_t max_s = narrow ? width / (8 * kWaveRows) : width / (4 * kTile);
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
