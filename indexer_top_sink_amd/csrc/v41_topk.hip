// Index top-k of a score row (I_t = top_k over the visible positions, the
// "Compressed sparse attention" page, "All 25 steps"; selection offset past
// the window rows with -1 for an absent entry, "attn_v41.rs" module
// documentation), for gfx950.
//
// One workgroup per score row.  Scores map to order-preserving u32 keys
// (-0 folded onto +0; -inf and NaN become key 0 = not selectable) and are
// staged in LDS when the row fits.  A radix select (4 passes of 8 bits, MSB
// first) finds the k-th largest key T and how many keys equal to T must be
// taken; the histograms are replicated 8 ways across lanes so that clustered
// keys (scores share their exponent bits) do not serialise on one LDS word.
// Every thread then owns a contiguous range of positions: it counts its keys
// above T and equal to T, a block-wide scan turns the counts into output
// slots, and the threshold group is filled from the lowest positions.  A
// bitonic sort in LDS puts the m selected (key, position) pairs in
// (score desc, position asc) order, and the row is written with the offset,
// padded with -1 up to k.
#include "v41_common.h"

namespace v41 {
namespace {

constexpr int kMaxK = 2048;
constexpr int kHistCopies = 8;

__device__ __forceinline__ uint32_t score_key(float s) {
  uint32_t u = __float_as_uint(s);
  if (s != s || u == 0xFF800000u) return 0u;  // NaN, -inf: not selectable
  if (u == 0x80000000u) u = 0u;               // -0 == +0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Exclusive scan of one value per thread over the block; also returns the
// total.  Uses `scratch` (one word per wavefront) and two barriers.
template <int NT>
__device__ __forceinline__ uint32_t block_excl_scan(uint32_t v, uint32_t* scratch,
                                                    uint32_t& total) {
  constexpr int NW = NT / kWave;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  uint32_t incl = v;
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    uint32_t o = __shfl_up(incl, off);
    if (lane >= off) incl += o;
  }
  if (lane == kWave - 1) scratch[wave] = incl;
  __syncthreads();
  uint32_t base = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    uint32_t x = scratch[w];
    base += (w < wave) ? x : 0u;
    tot += x;
  }
  __syncthreads();
  total = tot;
  return base + incl - v;
}

template <int NT, int CAP>
__global__ __launch_bounds__(NT) void topk_kernel(const float* __restrict__ scores,
                                                  int32_t n_cols, int64_t scores_ld, int32_t k,
                                                  int32_t offset, int32_t* __restrict__ idx,
                                                  int64_t idx_ld) {
  __shared__ uint32_t keys[CAP > 0 ? CAP : 1];
  __shared__ uint32_t hist[kHistCopies][256];
  __shared__ uint32_t hsum[256];
  __shared__ unsigned long long sel[kMaxK];
  __shared__ uint32_t scratch[NT / kWave];
  __shared__ uint32_t sh_digit, sh_above;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int64_t row = blockIdx.x;
  const float* __restrict__ srow = scores + row * scores_ld;
  int32_t* __restrict__ orow = idx + row * idx_ld;
  const bool staged = n_cols <= CAP;

  auto key_at = [&](int32_t j) -> uint32_t {
    return staged ? keys[j] : score_key(srow[j]);
  };

  // 1. keys and the count of selectable positions
  uint32_t nv_t = 0;
  for (int32_t j = tid; j < n_cols; j += NT) {
    const uint32_t kk = score_key(srow[j]);
    if (staged) keys[j] = kk;
    nv_t += kk != 0u;
  }
  uint32_t nv;
  (void)block_excl_scan<NT>(nv_t, scratch, nv);
  const uint32_t m = nv < (uint32_t)k ? nv : (uint32_t)k;

  // 2. threshold key T and how many keys equal to T to take.  With no more
  // valid positions than k, T = 0 and every valid key (> 0) is taken.
  uint32_t T = 0u, need = 0u;
  if (nv > (uint32_t)k) {
    uint32_t prefix = 0u, pmask = 0u, need_r = m;
    for (int pass = 0; pass < 4; ++pass) {
      const int shift = 24 - 8 * pass;
      for (int i = tid; i < kHistCopies * 256; i += NT) (&hist[0][0])[i] = 0u;
      __syncthreads();
      uint32_t* myhist = hist[lane % kHistCopies];
      for (int32_t j = tid; j < n_cols; j += NT) {
        const uint32_t kk = key_at(j);
        if (kk != 0u && (kk & pmask) == prefix) atomicAdd(&myhist[(kk >> shift) & 255u], 1u);
      }
      __syncthreads();
      for (int b = tid; b < 256; b += NT) {
        uint32_t s = 0;
#pragma unroll
        for (int c = 0; c < kHistCopies; ++c) s += hist[c][b];
        hsum[b] = s;
      }
      __syncthreads();
      if (tid < kWave) {
        // lane l owns bins 255-4l .. 252-4l; scan them from the top
        const uint32_t c0 = hsum[255 - 4 * lane], c1 = hsum[254 - 4 * lane];
        const uint32_t c2 = hsum[253 - 4 * lane], c3 = hsum[252 - 4 * lane];
        const uint32_t s = c0 + c1 + c2 + c3;
        uint32_t incl = s;
#pragma unroll
        for (int off = 1; off < kWave; off <<= 1) {
          uint32_t o = __shfl_up(incl, off);
          if (lane >= off) incl += o;
        }
        const uint32_t excl = incl - s;
        if (excl < need_r && need_r <= incl) {
          uint32_t cum = excl, d;
          if (need_r <= cum + c0) {
            d = 255 - 4 * lane;
          } else if (cum += c0, need_r <= cum + c1) {
            d = 254 - 4 * lane;
          } else if (cum += c1, need_r <= cum + c2) {
            d = 253 - 4 * lane;
          } else {
            cum += c2;
            d = 252 - 4 * lane;
          }
          sh_digit = d;
          sh_above = cum;
        }
      }
      __syncthreads();
      prefix |= sh_digit << shift;
      pmask |= 255u << shift;
      need_r -= sh_above;
      __syncthreads();
    }
    T = prefix;
    need = need_r;
  }
  const uint32_t n_gt = m - need;

  // 3. contiguous range per thread: count, scan, emit
  const int32_t C = (n_cols + NT - 1) / NT;
  const int32_t lo = tid * C;
  const int32_t hi = lo + C < n_cols ? lo + C : n_cols;
  uint32_t cgt = 0, ceq = 0;
  // rotated start spreads the lanes of a wavefront over the LDS banks
  int32_t rot = (C > 0) ? tid % C : 0;
  for (int32_t i = 0; i < C; ++i) {
    const int32_t j = lo + rot;
    rot = (rot + 1 == C) ? 0 : rot + 1;
    if (j < hi) {
      const uint32_t kk = key_at(j);
      cgt += kk > T;
      ceq += (need != 0u) && (kk == T);
    }
  }
  uint32_t tot_gt, tot_eq;
  uint32_t at_gt = block_excl_scan<NT>(cgt, scratch, tot_gt);
  uint32_t at_eq = block_excl_scan<NT>(ceq, scratch, tot_eq);
  for (int32_t j = lo; j < hi; ++j) {
    const uint32_t kk = key_at(j);
    const unsigned long long comp =
        ((unsigned long long)kk << 32) | (unsigned long long)(0xFFFFFFFFu - (uint32_t)j);
    if (kk > T) {
      sel[at_gt++] = comp;
    } else if (need != 0u && kk == T && at_eq < need) {
      sel[n_gt + at_eq] = comp;
      ++at_eq;
    }
  }

  // 4. bitonic sort of sel[0 .. P) descending, P = next power of two >= m.
  // Pair i of a stage is handled by thread i mod NT, so a wavefront owns the
  // 128-element chunks of its pairs; stages whose stride stays inside a chunk
  // (<= 64) need only the in-order LDS accesses of one wavefront, and a block
  // barrier is placed only next to stages that cross chunks.
  uint32_t P = 1;
  while (P < m) P <<= 1;
  for (uint32_t i = m + tid; i < P; i += NT) sel[i] = 0ull;
  __syncthreads();
  uint32_t prev_stride = 0;
  for (uint32_t size = 2; size <= P; size <<= 1) {
    for (uint32_t stride = size >> 1; stride > 0; stride >>= 1) {
      if (stride >= 128 || prev_stride >= 128)
        __syncthreads();
      else
        __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
      prev_stride = stride;
      for (uint32_t i = tid; i < P / 2; i += NT) {
        const uint32_t a = 2 * i - (i & (stride - 1));
        const uint32_t b = a + stride;
        const unsigned long long x = sel[a], y = sel[b];
        const bool desc = (a & size) == 0;
        if (desc ? (x < y) : (x > y)) {
          sel[a] = y;
          sel[b] = x;
        }
      }
    }
  }
  __syncthreads();

  // 5. positions + offset, then -1
  for (int32_t i = tid; i < k; i += NT) {
    int32_t v = -1;
    if ((uint32_t)i < m) v = (int32_t)(0xFFFFFFFFu - (uint32_t)(sel[i] & 0xFFFFFFFFull)) + offset;
    orow[i] = v;
  }
}

}  // namespace

hipError_t launch_topk_select(const float* scores, int64_t n_sel_rows, int64_t n_cols,
                              int64_t scores_ld, int32_t k, int32_t offset, int32_t* idx,
                              int64_t idx_ld, hipStream_t s) {
  if (n_sel_rows == 0) return hipSuccess;
  const dim3 grid((unsigned)n_sel_rows);
  const int32_t nc = (int32_t)n_cols;  // the ABI bounds n_cols below 2^31
  if (n_cols <= 4096) {
    hipLaunchKernelGGL((topk_kernel<256, 4096>), grid, dim3(256), 0, s, scores, nc,
                       scores_ld, k, offset, idx, idx_ld);
  } else if (n_cols <= 32768) {
    hipLaunchKernelGGL((topk_kernel<1024, 32768>), grid, dim3(1024), 0, s, scores, nc,
                       scores_ld, k, offset, idx, idx_ld);
  } else {
    hipLaunchKernelGGL((topk_kernel<1024, 0>), grid, dim3(1024), 0, s, scores, nc,
                       scores_ld, k, offset, idx, idx_ld);
  }
  return hipGetLastError();
}

}  // namespace v41
