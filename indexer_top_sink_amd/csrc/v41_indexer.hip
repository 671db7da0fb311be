// Indexer score S[q, j] = sum_h w[q, h] * ReLU(qI[q, h, :] . kI[j, :]) over the
// visible compressed positions ("Compressed sparse attention" page, "All 25
// steps", S^I and I_t), for gfx950.
//
// The contraction is qI[heads x DI] x kI^T[DI x 16 positions] on the matrix
// cores (v_mfma_f32_16x16x32_bf16): the heads are the M side (16 per tile, up
// to 4 tiles), 16 positions the N side, DI the K side.
//
// A workgroup of four wavefronts owns one query and a share of its positions.
// The query's qI (at most 64 x 128 bf16) and weights go through LDS once per
// workgroup and then sit in registers.  The positions are cut into 16-key
// blocks dealt round-robin to the query's wavefronts, so neighbouring
// wavefronts stream neighbouring 4 KB blocks.  Each wavefront keeps a private
// ring of kStages blocks in LDS, filled by global_load_lds_dwordx4: every
// instruction moves 1 KB of contiguous key bytes (the access pattern HBM
// streams best), and the lanes permute 16-byte chunks within each key row so
// that the MFMA operand reads from LDS hit distinct banks.  The wavefront
// waits on the oldest block with an explicit vmcnt, reads it, refills the slot
// with the block kStages ahead, and multiplies.
//
// The epilogue applies ReLU and the weights in f32, sums the 4 heads a lane
// holds per tile, then across the 4 lane groups with two xor-shuffles.  Keys
// past the causal bound are never loaded and score -inf.  With a candidate
// mask, a wavefront first finds which of its blocks hold an unmasked visible
// position (64 blocks at a time, one lane per block reading the block's mask
// bytes into a 16-bit keep mask, the live ones listed by a ballot): the
// others score -inf without a key load or a matrix product, and the stream
// runs over the live blocks with their keep masks in a register (no memory
// access of the mask inside the stream, so no wait on it there).
#include "v41_common.h"
#include "v41_front.h"

namespace v41 {
namespace {

typedef __attribute__((address_space(3))) void lds_void;

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;
constexpr int kStages = 2;

template <int DI>
struct KeyTile {
  static constexpr int KS = DI / 32;         // MFMA k-steps = 1 KB loads per block
  static constexpr int CPR = DI / 8;         // 16-byte chunks in a key row
  static constexpr int kBytes = 16 * DI * 2; // one 16-key block
  // Chunk c of row r sits in slot c ^ swz(r) of that row.  Rows 256 bytes
  // apart (or two or four to 256 bytes) get different permutations, so the
  // 16 rows a ds_read_b128 touches spread over all banks.
  static __device__ __forceinline__ int swz(int r) { return (r / (16 / CPR)) & (CPR - 1); }
};

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// KS ds_read_b128 and a wait for them, as one asm block: the compiler neither
// reorders the uses above the wait nor makes these reads wait for the
// direct-to-LDS loads still in flight into the other ring slots.
template <int KS>
__device__ __forceinline__ void lds_read_ks(u32x4 (&o)[KS], const uint32_t (&a)[KS], uint32_t base) {
  if constexpr (KS == 4) {
    asm volatile(
        "ds_read_b128 %0, %4\n\t"
        "ds_read_b128 %1, %5\n\t"
        "ds_read_b128 %2, %6\n\t"
        "ds_read_b128 %3, %7\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(o[0]), "=&v"(o[1]), "=&v"(o[2]), "=&v"(o[3])
        : "v"(a[0] + base), "v"(a[1] + base), "v"(a[2] + base), "v"(a[3] + base)
        : "memory");
  } else if constexpr (KS == 2) {
    asm volatile(
        "ds_read_b128 %0, %2\n\t"
        "ds_read_b128 %1, %3\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(o[0]), "=&v"(o[1])
        : "v"(a[0] + base), "v"(a[1] + base)
        : "memory");
  } else {
    asm volatile(
        "ds_read_b128 %0, %1\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(o[0])
        : "v"(a[0] + base)
        : "memory");
  }
}

// One 16-key block, rows j0 .. j0+15, into a ring slot: KS loads of 1 KB
// each (LDS byte 1024 c + 16 lane of the slot).  Rows at or past live_end
// reload row j0 (j0 < live_end keeps every address inside the keys).
template <int DI, int AUX>
__device__ __forceinline__ void issue_block(const uint16_t* kb, int j0, int live_end, int lane,
                                            uint8_t* slot) {
  using KT = KeyTile<DI>;
#pragma unroll
  for (int c = 0; c < KT::KS; ++c) {
    const int s = 64 * c + lane;
    const int r = s / KT::CPR;
    const int pos = s % KT::CPR;
    int j = j0 + r;
    if (j >= live_end) j = j0;
    const uint16_t* src = kb + (int64_t)j * DI + 8 * (pos ^ KT::swz(r));
    lds_void* dst = (lds_void*)(size_t)(slot + 1024 * c);
    // the cache-policy operand must be a literal for the host pass
    if constexpr (AUX == 2) __builtin_amdgcn_global_load_lds(src, dst, 16, 0, 2);
    else __builtin_amdgcn_global_load_lds(src, dst, 16, 0, 0);
  }
}

// F bit 0: keys streamed past the caches (a decode step); bit 1: a
// candidate mask is given (the two prologue orders below are then separate
// kernels, so the compiler never joins their loads in flight).
template <int DI, int HT, int F>
__global__ __launch_bounds__(kThreads, 2) void indexer_kernel(
    const uint16_t* __restrict__ qI, const uint16_t* __restrict__ kI, int64_t kI_bs,
    const float* __restrict__ w, const uint8_t* __restrict__ cand_in, int32_t cand_width,
    int32_t cand_block, int32_t n_tokens, int64_t start_pos, const int32_t* __restrict__ pos,
    int32_t ratio, int32_t n_heads, int32_t n_rows, float* __restrict__ scores,
    int64_t scores_ld, int32_t blocks_per_query, FrontParams front, int32_t score_blocks) {
  // workgroups past the score grid carry a decode step's front work
  if ((int32_t)blockIdx.x >= score_blocks) {
    decode_front_block(front, (int32_t)blockIdx.x - score_blocks);
    return;
  }
  using KT = KeyTile<DI>;
  constexpr int KS = KT::KS;
  constexpr int kQBytes = 16 * HT * DI * 2;
  constexpr int kRingBytes = kStages * KT::kBytes;
  constexpr int kAux = (F & 1) ? 2 : 0;  // no reuse expected
  const uint8_t* __restrict__ const cand = (F & 2) ? cand_in : nullptr;
  __shared__ __attribute__((aligned(16))) uint8_t smem[kQBytes + 64 * 4 + kWaves * kRingBytes];
  __shared__ int32_t wlist[kWaves][kWave];   // live block lists
  __shared__ uint32_t wkeep[kWaves][kWave];  // and their 16-bit keep masks
  uint8_t* const qs = smem;
  float* const ws = reinterpret_cast<float*>(smem + kQBytes);

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r16 = lane & 15;
  const int g = lane >> 4;
  // Decode (one token per sequence, a multiple of 8 queries): the
  // workgroups of query q sit on XCD q mod 8 (dispatch is round-robin over
  // the 8 XCDs), where the top-k and the attention of that query run, so
  // they read its scores from that XCD's L2.  Otherwise queries go in
  // reverse order: in a chunk the later tokens see more keys, so the longest
  // workgroups start first and the short ones fill the tail.
  int32_t unit;
  if (n_tokens == 1 && (score_blocks / blocks_per_query) % 8 == 0) {
    const int32_t xcd = (int32_t)blockIdx.x & 7, j = (int32_t)blockIdx.x >> 3;
    unit = (8 * (j / blocks_per_query) + xcd) * blocks_per_query + j % blocks_per_query;
  } else {
    unit = score_blocks - 1 - (int32_t)blockIdx.x;
  }
  const int64_t q = unit / blocks_per_query;
  const int wpq = blocks_per_query * kWaves;
  const int part = (int)(unit - q * blocks_per_query) * kWaves + wave;
  const int64_t b = q / n_tokens;
  const int64_t t = q - b * n_tokens;
  // position of the token: the call's start_pos, or read on the device
  const int64_t base = pos != nullptr ? (int64_t)pos[b] : start_pos;
  int64_t vis = (base + t + 1) / ratio;
  vis = vis < 0 ? 0 : vis;
  const int live_end = (int)(vis < n_rows ? vis : n_rows);
  const int nbt = (n_rows + 15) / 16;     // 16-key blocks in the row
  const int nbv = (live_end + 15) / 16;   // ... with a visible key
  const int nw = part < nbv ? (nbv - 1 - part) / wpq + 1 : 0;  // this wavefront's visible blocks

  float* __restrict__ srow = scores + q * scores_ld;
  const float kNegInf = -__builtin_huge_valf();

  uint8_t* const ring = smem + kQBytes + 64 * 4 + wave * kRingBytes;
  const uint16_t* __restrict__ kb = kI + b * kI_bs;

  // ---- this wavefront's blocks part + i wpq, i < nw, taken 64 at a time:
  // with a mask, the live ones of a chunk are listed (lane l holds the
  // l-th), the masked ones score -inf here
  auto chunk_list = [&](int c0, int& n_live, uint32_t& keep) -> int32_t {
    const int cn = nw - c0 < kWave ? nw - c0 : kWave;
    keep = 0xFFFFu;  // without a mask: every position (the causal bound is checked apart)
    if (cand == nullptr) {
      n_live = cn;
      return c0 + lane;
    }
    uint32_t km = 0u;  // bit p: position j0 + p is visible and unmasked
    if (lane < cn) {
      const int j0 = (part + (c0 + lane) * wpq) * 16;
      const int j1 = j0 + 16 < live_end ? j0 + 16 : live_end;
      for (int cb = j0 / cand_block; cb <= (j1 - 1) / cand_block; ++cb) {
        if (cand[q * cand_width + cb] != 0) {
          const int a = cb * cand_block > j0 ? cb * cand_block : j0;
          const int e = (cb + 1) * cand_block < j1 ? (cb + 1) * cand_block : j1;
          km |= ((1u << (e - a)) - 1u) << (a - j0);
        }
      }
    }
    const bool live = km != 0u;
    const unsigned long long lm = __ballot(live);
    n_live = __popcll(lm);
    // masked blocks: -inf for their 16 positions
    for (unsigned long long dm = __ballot(lane < cn && !live); dm != 0ull; dm &= dm - 1ull) {
      const int j = (part + (c0 + __builtin_ctzll(dm)) * wpq) * 16 + lane;
      if (lane < 16 && j < n_rows) srow[j] = -__builtin_huge_valf();
    }
    // lane l: the index and keep mask of the l-th live block (through
    // per-wavefront lists)
    if (live) {
      const int rank = __popcll(lm & ((1ull << lane) - 1ull));
      wlist[wave][rank] = c0 + lane;
      wkeep[wave][rank] = km;
    }
    __builtin_amdgcn_wave_barrier();
    keep = lane < n_live ? wkeep[wave][lane] : 0u;
    return lane < n_live ? wlist[wave][lane] : 0;
  };
  // ---- the query's qI and weights into registers, the first kStages live
  // blocks in flight, then the query through LDS.  With a candidate mask the
  // qI loads go first, so that their latency overlaps the mask reads of the
  // block list (prefill chunk 23.8 -> 20.3 us); without one the key stream
  // is the critical path and its first blocks go first.  The two orders are
  // separate kernels (F bit 1): joined in one, the compiler made the
  // keys-first path wait for every load in flight before its query loads
  // (decode64 24.4 -> 23.7 us once split)
  constexpr int kQPer = (16 * HT * KT::CPR + kThreads - 1) / kThreads;
  u32x4 qv[kQPer];
  float wv = 0.0f;
  const uint16_t* qrow = qI + q * n_heads * DI;
  auto load_query = [&]() {
#pragma unroll
    for (int j = 0; j < kQPer; ++j) {
      const int e = (int)threadIdx.x + j * kThreads;
      const int h = e / KT::CPR;
      const int c = e % KT::CPR;
      qv[j] = (u32x4){0u, 0u, 0u, 0u};
      if (e < 16 * HT * KT::CPR && h < n_heads)
        qv[j] = *reinterpret_cast<const u32x4*>(qrow + h * DI + 8 * c);
    }
    if (threadIdx.x < 64 && (int)threadIdx.x < n_heads) wv = w[q * n_heads + threadIdx.x];
  };
  int n_live0 = 0;
  uint32_t keep0 = 0u;
  int32_t list0 = 0;
  auto issue_first = [&]() {
#pragma unroll
    for (int s = 0; s < kStages; ++s)
      if (s < n_live0)
        issue_block<DI, kAux>(kb, (part + __builtin_amdgcn_readlane(list0, s) * wpq) * 16,
                              live_end, lane, ring + s * KT::kBytes);
  };
  if constexpr ((F & 2) != 0) {
    load_query();
    if (nw > 0) list0 = chunk_list(0, n_live0, keep0);
    issue_first();
  } else {
    if (nw > 0) list0 = chunk_list(0, n_live0, keep0);
    issue_first();
    load_query();
  }
#pragma unroll
  for (int j = 0; j < kQPer; ++j) {
    const int e = (int)threadIdx.x + j * kThreads;
    const int h = e / KT::CPR;
    const int c = e % KT::CPR;
    if (e < 16 * HT * KT::CPR)
      *reinterpret_cast<u32x4*>(qs + h * 2 * DI + 16 * (c ^ KT::swz(h))) = qv[j];
  }
  if (threadIdx.x < 64) ws[threadIdx.x] = wv;
  lds_barrier();

  // lane offsets of its k-step operands in a block (row r16, chunks g + 4kk)
  uint32_t off[KS];
#pragma unroll
  for (int kk = 0; kk < KS; ++kk)
    off[kk] = (uint32_t)(r16 * 2 * DI + 16 * ((g + 4 * kk) ^ KT::swz(r16)));
  const uint32_t ring_lds = (uint32_t)(size_t)(lds_void*)(size_t)ring;
  const uint32_t qs_lds = (uint32_t)(size_t)(lds_void*)(size_t)qs;

  bf16x8 afr[HT][KS];
  float wh[HT][4];
#pragma unroll
  for (int ht = 0; ht < HT; ++ht) {
    u32x4 v[KS];
    lds_read_ks<KS>(v, off, qs_lds + ht * 16 * 2 * DI);
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) afr[ht][kk] = as_bf16x8(v[kk]);
    u32x4 wv;
    const uint32_t wa = (uint32_t)(size_t)(lds_void*)(size_t)(ws + 16 * ht + 4 * g);
    asm volatile("ds_read_b128 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=&v"(wv) : "v"(wa) : "memory");
#pragma unroll
    for (int i = 0; i < 4; ++i) wh[ht][i] = __uint_as_float(wv[i]);
  }

  // ---- invisible blocks of this wavefront: -inf
  for (int blk = part + nw * wpq; blk < nbt; blk += wpq) {
    const int j = blk * 16 + lane;
    if (lane < 16 && j < n_rows) srow[j] = kNegInf;
  }

  // ---- the stream, over the live blocks of each chunk
  int32_t list = list0;
  uint32_t keepv = keep0;
  int n_live = n_live0;
  for (int c0 = 0; c0 < nw; c0 += kWave) {
    if (c0 > 0) {
      list = chunk_list(c0, n_live, keepv);
#pragma unroll
      for (int s = 0; s < kStages; ++s)
        if (s < n_live)
          issue_block<DI, kAux>(kb, (part + __builtin_amdgcn_readlane(list, s) * wpq) * 16,
                                live_end, lane, ring + s * KT::kBytes);
    }
    for (int i0 = 0; i0 < n_live; i0 += kStages) {
#pragma unroll
      for (int s = 0; s < kStages; ++s) {
        const int i = i0 + s;
        if (i < n_live) {
          if (i + kStages - 1 < n_live) wait_vmcnt<KS * (kStages - 1)>();
          else wait_vmcnt<0>();
          u32x4 kf[KS];
          lds_read_ks<KS>(kf, off, ring_lds + s * KT::kBytes);
          const int blk = part + __builtin_amdgcn_readlane(list, i) * wpq;
          const uint32_t keep = (__builtin_amdgcn_readlane(keepv, i) >> r16) & 1u;
          if (i + kStages < n_live)
            issue_block<DI, kAux>(
                kb, (part + __builtin_amdgcn_readlane(list, i + kStages) * wpq) * 16, live_end,
                lane, ring + s * KT::kBytes);
          f32x4 acc[HT];
#pragma unroll
          for (int ht = 0; ht < HT; ++ht) acc[ht] = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int kk = 0; kk < KS; ++kk) {
            const bf16x8 bk = as_bf16x8(kf[kk]);
#pragma unroll
            for (int ht = 0; ht < HT; ++ht) acc[ht] = mfma16x16x32(afr[ht][kk], bk, acc[ht]);
          }
          float sum = 0.0f;
#pragma unroll
          for (int ht = 0; ht < HT; ++ht)
#pragma unroll
            for (int e = 0; e < 4; ++e) sum += wh[ht][e] * fmaxf(acc[ht][e], 0.0f);
          {
            // the four k-groups' partial sums of the key (lanes 16 and 32
            // apart), on the permlane swaps
            const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(sum),
                                                            __float_as_uint(sum), false, false);
            sum = __uint_as_float(r[0]) + __uint_as_float(r[1]);
            const auto t = __builtin_amdgcn_permlane32_swap(__float_as_uint(sum),
                                                            __float_as_uint(sum), false, false);
            sum = __uint_as_float(t[0]) + __uint_as_float(t[1]);
          }
          const int j = blk * 16 + r16;
          if (g == 0 && j < n_rows) srow[j] = (j < live_end && keep != 0u) ? sum : kNegInf;
        }
      }
    }
  }
}

template <int DI, int F>
hipError_t dispatch_heads(int ht, dim3 grid, hipStream_t s, const uint16_t* qI,
                          const uint16_t* kI, int64_t kI_bs, const float* w,
                          const uint8_t* cand, int32_t cand_width, int32_t cand_block,
                          int32_t n_tokens, int64_t start_pos, const int32_t* pos,
                          int32_t ratio, int32_t n_heads, int32_t n_rows, float* scores,
                          int64_t scores_ld, int32_t bpq, const FrontParams& front,
                          int32_t score_blocks) {
#define V41_IDX_LAUNCH(HT_)                                                                   \
  hipLaunchKernelGGL((indexer_kernel<DI, HT_, F>), grid, dim3(kThreads), 0, s, qI, kI,       \
                     kI_bs, w, cand, cand_width, cand_block, n_tokens, start_pos, pos,       \
                     ratio, n_heads, n_rows, scores, scores_ld, bpq, front, score_blocks)
  switch (ht) {
    case 1: V41_IDX_LAUNCH(1); break;
    case 2: V41_IDX_LAUNCH(2); break;
    case 3: V41_IDX_LAUNCH(3); break;
    default: V41_IDX_LAUNCH(4); break;
  }
#undef V41_IDX_LAUNCH
  return hipGetLastError();
}

template <int DI>
hipError_t dispatch_nt(bool nt, int ht, dim3 grid, hipStream_t s, const uint16_t* qI,
                       const uint16_t* kI, int64_t kI_bs, const float* w, const uint8_t* cand,
                       int32_t cand_width, int32_t cand_block, int32_t n_tokens,
                       int64_t start_pos, const int32_t* pos, int32_t ratio, int32_t n_heads,
                       int32_t n_rows, float* scores, int64_t scores_ld, int32_t bpq,
                       const FrontParams& front, int32_t score_blocks) {
#define V41_IDX_FLAGS(F_)                                                                     \
  return dispatch_heads<DI, F_>(ht, grid, s, qI, kI, kI_bs, w, cand, cand_width, cand_block, \
                                n_tokens, start_pos, pos, ratio, n_heads, n_rows, scores,    \
                                scores_ld, bpq, front, score_blocks)
  switch ((nt ? 1 : 0) | (cand != nullptr ? 2 : 0)) {
    case 1: V41_IDX_FLAGS(1);
    case 2: V41_IDX_FLAGS(2);
    case 3: V41_IDX_FLAGS(3);
    default: V41_IDX_FLAGS(0);
  }
#undef V41_IDX_FLAGS
}

}  // namespace

hipError_t launch_indexer_scores_front(const uint16_t* qI, const uint16_t* kI, int64_t kI_bs,
                                       const float* w, const uint8_t* cand, int32_t cand_width,
                                       int32_t cand_block, int32_t batch, int32_t n_tokens,
                                       int64_t start_pos, const int32_t* pos, int32_t ratio,
                                       int32_t n_heads, int32_t head_dim, int64_t n_rows,
                                       float* scores, int64_t scores_ld,
                                       const DecodeFrontArgs* front_args, hipStream_t s) {
  const int64_t nq = (int64_t)batch * n_tokens;
  FrontParams front{};
  const int32_t front_blocks =
      (front_args != nullptr && front_args->batch > 0) ? make_front_params(*front_args, front) : 0;
  if (nq == 0 || n_rows == 0) {
    if (front_blocks == 0) return hipSuccess;
    // nothing to score: the front work alone
    return launch_decode_front(*front_args, s);
  }
  // Workgroups per query: about 512 over the whole grid (2 per CU; up to 3
  // fit in LDS), the best measured for decode at 16 and 64 sequences (with
  // the XCD placement: 256 clearly slower, 384 and 768 slightly), but at
  // least two 16-key blocks for each wavefront.
  const int64_t nbt = (n_rows + 15) / 16;
  int64_t bpq = (512 + nq / 2) / nq;
  const int64_t bpq_max = nbt / (2 * kWaves);
  if (bpq > bpq_max) bpq = bpq_max;
  if (bpq < 1) bpq = 1;
  if (nq * bpq + front_blocks > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
  const int32_t score_blocks = (int32_t)(nq * bpq);
  const dim3 grid((unsigned)(score_blocks + front_blocks));
  const int ht = (n_heads + 15) / 16;
  // a key serves one query at a decode step: stream it past the caches
  const bool nt = n_tokens == 1;
  const int32_t rows = (int32_t)n_rows;
  switch (head_dim) {
    case 32:
      return dispatch_nt<32>(nt, ht, grid, s, qI, kI, kI_bs, w, cand, cand_width, cand_block,
                             n_tokens, start_pos, pos, ratio, n_heads, rows, scores, scores_ld,
                             (int32_t)bpq, front, score_blocks);
    case 64:
      return dispatch_nt<64>(nt, ht, grid, s, qI, kI, kI_bs, w, cand, cand_width, cand_block,
                             n_tokens, start_pos, pos, ratio, n_heads, rows, scores, scores_ld,
                             (int32_t)bpq, front, score_blocks);
    default:
      return dispatch_nt<128>(nt, ht, grid, s, qI, kI, kI_bs, w, cand, cand_width, cand_block,
                              n_tokens, start_pos, pos, ratio, n_heads, rows, scores, scores_ld,
                              (int32_t)bpq, front, score_blocks);
  }
}

hipError_t launch_indexer_scores(const uint16_t* qI, const uint16_t* kI, int64_t kI_bs,
                                 const float* w, const uint8_t* cand, int32_t cand_width,
                                 int32_t cand_block, int32_t batch, int32_t n_tokens,
                                 int64_t start_pos, const int32_t* pos, int32_t ratio,
                                 int32_t n_heads, int32_t head_dim, int64_t n_rows,
                                 float* scores, int64_t scores_ld, hipStream_t s) {
  return launch_indexer_scores_front(qI, kI, kI_bs, w, cand, cand_width, cand_block, batch,
                                     n_tokens, start_pos, pos, ratio, n_heads, head_dim, n_rows,
                                     scores, scores_ld, nullptr, s);
}

}  // namespace v41
