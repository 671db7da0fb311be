// Index top-k of a score row (I_t = top_k over the visible positions, the
// "Compressed sparse attention" page, "All 25 steps"; selection offset past
// the window rows with -1 for an absent entry, "attn_v41.rs" module
// documentation), for gfx950.
//
// One workgroup per score row; thread t owns the contiguous positions
// [t*KPT, (t+1)*KPT) and keeps their keys in registers (rows longer than
// 32768 re-read them from memory instead).  Scores map to order-preserving
// u32 keys (-0 folded onto +0; -inf and NaN become key 0 = not selectable).
//  1. count of valid keys and their min / max (wavefront reductions, one
//     barrier);
//  2. radix select of the k-th largest key T: digits of 8 bits of
//     (key - min), starting at the top bit of (max - min), so the first pass
//     already spreads over the bins; the LDS histogram is replicated across
//     lanes (2 to 8 copies by keys per thread) so that equal digits do not
//     serialise on one word; two
//     histograms alternate so clearing the next one overlaps the counting,
//     and the first wavefront sums the copies while it scans (two barriers
//     per pass).  The passes stop as soon as the bin holding the k-th key is
//     taken whole (then no tie inside it needs breaking): with distinct
//     scores that is usually after two passes;
//  3. the selection is {key > T} plus the first `need` positions with key == T
//     (ties to the lower position); one block-wide exclusive scan of packed
//     (greater, equal) counts gives each thread its output slots, and the
//     positions are written in ascending order, then -1 up to k.
// The candidate-block selection runs the same select over per-block maxima
// and writes a byte mask instead of positions.
#include <float.h>

#include "v41_common.h"
#include "v41_wave.h"

namespace v41 {
namespace {

constexpr int kHistCopies = 8;
constexpr int kHistStride = 257;

__device__ __forceinline__ uint32_t score_key(float s) {
  uint32_t u = __float_as_uint(s);
  if (s != s || u == 0xFF800000u) return 0u;  // NaN, -inf: not selectable
  if (u == 0x80000000u) u = 0u;               // -0 == +0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

template <int NT, int HC = kHistCopies>
struct TopkShared {
  static constexpr int kCopies = HC;
  // alternate passes (the idle one is cleared); copy c of bin b at
  // c * kHistStride + b, so the copies of one bin sit in distinct banks
  uint32_t hist[2][HC * kHistStride];
  uint32_t red[3][NT / kWave];
  uint32_t digit, above, bin;
};

// Capacity of the sampled select's candidate buffer (keys and positions).
constexpr int kCandCap = 4096;

// Exclusive scan of one value per thread over the block (two barriers; the
// last scan of a kernel skips the second, which only protects sh.red for a
// later use).
template <int NT, bool kLast = false, int HC>
__device__ __forceinline__ uint32_t block_excl_scan(uint32_t v, TopkShared<NT, HC>& sh) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint32_t incl = wave_incl_scan_u32(v);
  if (lane == kWave - 1) sh.red[0][wave] = incl;
  __syncthreads();
  uint32_t base = 0;
  for (int w = 0; w < wave; ++w) base += sh.red[0][w];
  if constexpr (!kLast) __syncthreads();
  return base + incl - v;
}

// The same, also returning the block total.
template <int NT, int HC>
__device__ __forceinline__ uint32_t block_excl_scan_tot(uint32_t v, TopkShared<NT, HC>& sh,
                                                        uint32_t& total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint32_t incl = wave_incl_scan_u32(v);
  if (lane == kWave - 1) sh.red[0][wave] = incl;
  __syncthreads();
  uint32_t base = 0, tot = 0;
  for (int w = 0; w < NT / kWave; ++w) {
    const uint32_t c = sh.red[0][w];
    base += (w < wave) ? c : 0u;
    tot += c;
  }
  __syncthreads();
  total = tot;
  return base + incl - v;
}

// Count, min and max of the valid keys over the block (two barriers; with
// kTrail false the caller orders any later write of sh.red itself).
template <int NT, bool kTrail = true, int HC>
__device__ __forceinline__ void block_stats(uint32_t nv, uint32_t kmin, uint32_t kmax,
                                            TopkShared<NT, HC>& sh, uint32_t& o_nv,
                                            uint32_t& o_min, uint32_t& o_max) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  nv = wave_sum_u32(nv);
  kmin = wave_min_u32(kmin);
  kmax = wave_max_u32(kmax);
  if (lane == 0) {
    sh.red[0][wave] = nv;
    sh.red[1][wave] = kmin;
    sh.red[2][wave] = kmax;
  }
  __syncthreads();
  o_nv = 0;
  o_min = 0xFFFFFFFFu;
  o_max = 0;
  for (int w = 0; w < NT / kWave; ++w) {
    o_nv += sh.red[0][w];
    o_min = min(o_min, sh.red[1][w]);
    o_max = max(o_max, sh.red[2][w]);
  }
  if constexpr (kTrail) __syncthreads();
}

// Radix select over d = key - kmin of the valid keys: returns T (a key) and
// `need`, the number of keys equal to T that belong to the top m.
// for_keys(f) calls f(key) for every key the thread owns.
template <int NT, class ForKeys, bool kPreCleared = false, int HC>
__device__ __forceinline__ void radix_select(ForKeys for_keys, uint32_t m, uint32_t kmin,
                                             uint32_t kmax, TopkShared<NT, HC>& sh, uint32_t& T,
                                             uint32_t& need) {
  const int tid = threadIdx.x, lane = tid & 63;
  const uint32_t range = kmax - kmin;
  if (range == 0u) {
    // without the clearing barrier this is the caller's only barrier between
    // its statistics and its next use of sh.red
    if constexpr (kPreCleared) __syncthreads();
    T = kmax;
    need = m;
    return;
  }
  const int top = 31 - __clz(range);
  int shift = top > 7 ? top - 7 : 0;
  uint32_t prefix = 0u, pmask = 0u, need_r = m;
  if constexpr (!kPreCleared) {
    for (int i = tid; i < HC * kHistStride; i += NT) sh.hist[0][i] = 0u;
    __syncthreads();
  }
  for (int pass = 0;; ++pass) {
    uint32_t* const hist = sh.hist[pass & 1];
    // the other copy was last read before the previous pass's final barrier
    for (int i = tid; i < HC * kHistStride; i += NT) sh.hist[(pass + 1) & 1][i] = 0u;
    uint32_t* const myhist = hist + (lane % HC) * kHistStride;
    // a run of equal digits among the thread's keys (its positions are
    // contiguous, so tied scores form runs) costs one atomic
    uint32_t run_bin = 0u, run_cnt = 0u;
    for_keys([&](uint32_t key) {
      if (key != 0u) {
        const uint32_t d = key - kmin;
        if ((d & pmask) == prefix) {
          const uint32_t bin = (d >> shift) & 255u;
          if (run_cnt != 0u && bin != run_bin) {
            atomicAdd(&myhist[run_bin], run_cnt);
            run_cnt = 0u;
          }
          run_bin = bin;
          ++run_cnt;
        }
      }
    });
    if (run_cnt != 0u) atomicAdd(&myhist[run_bin], run_cnt);
    __syncthreads();
    if (tid < kWave) {
      // lane l owns bins 255-4l .. 252-4l (summed over the copies); find the
      // bin holding the need_r-th largest digit, scanning from the top
      uint32_t c[4] = {0u, 0u, 0u, 0u};
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int cp = 0; cp < HC; ++cp) c[j] += hist[cp * kHistStride + 255 - 4 * lane - j];
      const uint32_t s = c[0] + c[1] + c[2] + c[3];
      const uint32_t incl = wave_incl_scan_u32(s);
      const uint32_t excl = incl - s;
      if (excl < need_r && need_r <= incl) {
        uint32_t cum = excl;
        int j = 0;
        while (j < 3 && need_r > cum + c[j]) cum += c[j++];
        sh.digit = 255 - 4 * lane - j;
        sh.above = cum;
        sh.bin = c[j];
      }
    }
    __syncthreads();
    prefix |= sh.digit << shift;
    pmask |= 255u << shift;
    need_r -= sh.above;
    if (need_r == sh.bin) {
      // the whole bin is taken: the selection is every valid key with
      // d >= prefix, and no tie inside the bin needs breaking
      T = kmin + prefix - 1u;
      need = 0u;
      return;
    }
    if (shift == 0) break;
    // the last window may overlap decided bits; they are fixed by the prefix
    shift = shift > 8 ? shift - 8 : 0;
  }
  T = kmin + prefix;
  need = need_r;
}

// Keys in registers: KPT contiguous positions per thread (n_cols <= NT * KPT,
// KPT <= 16).
template <int NT, int KPT>
__global__ __launch_bounds__(NT) void topk_reg_kernel(const float* __restrict__ scores,
                                                      int32_t n_cols, int64_t scores_ld,
                                                      int32_t k, int32_t offset,
                                                      int32_t* __restrict__ idx,
                                                      int64_t idx_ld) {
  static_assert(KPT <= 16, "rows of 32 keys per thread take topk_long_kernel");
  // histogram copies: fewer copies make the bin scan cheaper, more spread
  // the atomics of many keys per thread (measured: 2 best at 8 keys per
  // thread)
  __shared__ TopkShared<NT, (KPT <= 8 ? 2 : 4)> sh;
  const int tid = threadIdx.x;
  const int64_t row = blockIdx.x;
  const float* __restrict__ srow = scores + row * scores_ld;
  int32_t* __restrict__ orow = idx + row * idx_ld;
  const int32_t lo = tid * KPT;

  uint32_t key[KPT];
  const bool vec = (KPT % 4 == 0) && ((reinterpret_cast<uintptr_t>(srow + lo) & 15u) == 0) &&
                   (lo + KPT <= n_cols);
  if (vec) {
#pragma unroll
    for (int v = 0; v < KPT / 4; ++v) {
      const float4 f = *reinterpret_cast<const float4*>(srow + lo + 4 * v);
      key[4 * v + 0] = score_key(f.x);
      key[4 * v + 1] = score_key(f.y);
      key[4 * v + 2] = score_key(f.z);
      key[4 * v + 3] = score_key(f.w);
    }
  } else {
#pragma unroll
    for (int i = 0; i < KPT; ++i) key[i] = (lo + i < n_cols) ? score_key(srow[lo + i]) : 0u;
  }
  uint32_t nv_t = 0, kmin_t = 0xFFFFFFFFu, kmax_t = 0u;
#pragma unroll
  for (int i = 0; i < KPT; ++i) {
    if (key[i] != 0u) {
      ++nv_t;
      kmin_t = min(kmin_t, key[i]);
      kmax_t = max(kmax_t, key[i]);
    }
  }
  uint32_t nv, kmin, kmax;
  // the first radix histogram is cleared before the statistics' barrier,
  // which then also publishes it; the select (or, when every valid key is
  // taken, one barrier) follows the statistics before anything rewrites
  // sh.red
  for (int i = tid; i < sh.kCopies * kHistStride; i += NT) sh.hist[0][i] = 0u;
  block_stats<NT, false>(nv_t, kmin_t, kmax_t, sh, nv, kmin, kmax);
  const uint32_t m = nv < (uint32_t)k ? nv : (uint32_t)k;
  uint32_t T = 0u, need = 0u;
  if (nv <= (uint32_t)k) {
    __syncthreads();
  } else {
    auto all_keys = [&](auto f) {
#pragma unroll
      for (int i = 0; i < KPT; ++i) f(key[i]);
    };
    radix_select<NT, decltype(all_keys), true>(all_keys, m, kmin, kmax, sh, T, need);
  }

  uint32_t cg = 0, ce = 0;
#pragma unroll
  for (int i = 0; i < KPT; ++i) {
    cg += key[i] > T;
    ce += (need != 0u) && (key[i] == T);
  }
  // n_cols <= 4096 * 4, so both counts fit 16 bits
  const uint32_t excl = block_excl_scan<NT, true>((cg << 16) | ce, sh);
  const uint32_t base_e = excl & 0xFFFFu;
  uint32_t pos = (excl >> 16) + (base_e < need ? base_e : need);
  uint32_t er = base_e;
#pragma unroll
  for (int i = 0; i < KPT; ++i) {
    if (key[i] > T) {
      orow[pos++] = lo + i + offset;
    } else if (need != 0u && key[i] == T) {
      if (er < need) orow[pos++] = lo + i + offset;
      ++er;
    }
  }
  for (int32_t i = (int32_t)m + tid; i < k; i += NT) orow[i] = -1;
}

// Rows of 8193..32768 scores, 32 per thread.  The whole row is taken in one
// step per wavefront: wavefront w reads its 64 * 32 contiguous scores with
// consecutive lanes on consecutive 16-byte pieces (whole cache lines per
// instruction; lanes reading their own 128-byte runs touched 64 lines per
// instruction), all loads issued before the first is used, parks them in its
// own LDS region and reads back lane l's 32 contiguous scores (16-byte
// chunks swizzled, so 16 lanes' reads fall on distinct banks); the staged
// row stays there for the candidates' scores.  The per-score
// passes then run on the scores as floats: with -inf and NaN excluded and
// -0 == +0, the float order is the key order, so a comparison costs one
// instruction where building the key took eight (one workgroup does all of
// a row's arithmetic, so instructions per score set its time).
//  1. valid count (wavefront ballots), the row's largest score, and the
//     sample (key[0] of every thread: one score per 32) count and minimum,
//     one block reduction;
//  2. sampled threshold: a radix select over the sample picks T0, a key
//     that about r * nv / n_s scores reach, r set a few standard deviations
//     above the m * n_s / nv samples expected among the top m;
//  3. one pass counts the scores above and at T0 and writes the positions of
//     those above it (from a bit mask per lane) into the wavefront's region
//     of a candidate buffer; then with G above T0 and E equal:
//     - G <= m <= G + E: T0 is the m-th key; the counts give the output
//       slots directly;
//     - G > m (and every wavefront's candidates fit its region): an exact
//       select among the candidates;
//     - otherwise the full select over the keys.
template <int NT, int KPT>
__global__ __launch_bounds__(NT) void topk_long_kernel(const float* __restrict__ scores,
                                                       int32_t n_cols, int64_t scores_ld,
                                                       int32_t k, int32_t offset,
                                                       int32_t* __restrict__ idx,
                                                       int64_t idx_ld) {
  static_assert(KPT == 32, "one staged row of 32 scores per thread");
  constexpr int kNW = NT / kWave;
  constexpr uint32_t kWaveCap = kCandCap / kNW;
  // the staged row stays in LDS to the end (the candidates are kept as
  // positions and read their scores from it): wavefront w's 2048 scores at
  // [w * 2048, + 2048), lane l's 32 as eight 16-byte chunks, chunk c at
  // l * 8 + (c ^ ((l >> 1) & 7)) so that 16 lanes reading chunk c fall on
  // distinct banks
  constexpr int kStageBytes = NT * KPT * 4;
  static_assert(KPT == 32, "the chunk swizzle assumes 8 chunks per lane");
  __shared__ TopkShared<NT, 4> sh;
  // the staged row, then the candidates' positions
  __shared__ __attribute__((aligned(16))) uint8_t raw[kStageBytes + kCandCap * 4];
  const float* const stage = reinterpret_cast<const float*>(raw);
  uint32_t* const cand = reinterpret_cast<uint32_t*>(raw + kStageBytes);
  // LDS float index of row position p (p < NT * KPT)
  auto staged_at = [](uint32_t p) {
    const uint32_t w = p >> 11, q = p & 2047u, l = q >> 5, c = (q >> 2) & 7u;
    return (w << 11) + ((l * 8u + (c ^ ((l >> 1) & 7u))) << 2) + (q & 3u);
  };
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid >> 6;
  const int64_t row = blockIdx.x;
  const float* __restrict__ srow = scores + row * scores_ld;
  int32_t* __restrict__ orow = idx + row * idx_ld;
  const int32_t lo = tid * KPT;

  float f[KPT];
  {
    constexpr int V = KPT / 4;
    const int32_t wbase = wave * 64 * KPT;
    float* const ws = reinterpret_cast<float*>(raw) + wave * 64 * KPT;
    float4 g[V];
    if (((reinterpret_cast<uintptr_t>(srow) & 15u) == 0) && wbase + 64 * KPT <= n_cols) {
#pragma unroll
      for (int v = 0; v < V; ++v)
        g[v] = *reinterpret_cast<const float4*>(srow + wbase + v * 256 + lane * 4);
    } else {
#pragma unroll
      for (int v = 0; v < V; ++v) {
        const int32_t p = wbase + v * 256 + lane * 4;
        g[v].x = p + 0 < n_cols ? srow[p + 0] : -INFINITY;
        g[v].y = p + 1 < n_cols ? srow[p + 1] : -INFINITY;
        g[v].z = p + 2 < n_cols ? srow[p + 2] : -INFINITY;
        g[v].w = p + 3 < n_cols ? srow[p + 3] : -INFINITY;
      }
    }
#pragma unroll
    for (int v = 0; v < V; ++v) {
      const int q = v * 256 + lane * 4;
      const int l = q / KPT, c = (q % KPT) / 4;
      *reinterpret_cast<float4*>(ws + (l * 8 + (c ^ ((l >> 1) & 7))) * 4) = g[v];
    }
    // the read-back takes other lanes' writes: a wavefront's LDS operations
    // are performed in order, so only the compiler must keep them in order
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
    for (int v = 0; v < V; ++v) {
      const float4 h =
          *reinterpret_cast<const float4*>(ws + (lane * 8 + (v ^ ((lane >> 1) & 7))) * 4);
      f[4 * v + 0] = h.x;
      f[4 * v + 1] = h.y;
      f[4 * v + 2] = h.z;
      f[4 * v + 3] = h.w;
    }
  }

  // 1. statistics (f >= -FLT_MAX is false for NaN and -inf, the unselectable
  // scores; the comparison-select maximum skips them too).  The ballot's
  // predicate is written as >= -FLT_MAX: the equivalent f > -inf becomes an
  // ordered not-equal that the ballot lowering turns into the unordered
  // v_cmp_neq_f32, true for NaN.
  uint32_t nvw = 0;
  float mf = -INFINITY;
#pragma unroll
  for (int i = 0; i < KPT; ++i) {
    nvw += (uint32_t)__popcll(__ballot(f[i] >= -FLT_MAX));
    mf = f[i] > mf ? f[i] : mf;
  }
  const uint32_t key0 = score_key(f[0]);
  // the sample select's histogram is cleared before the statistics'
  // barrier, which publishes it
  for (int i = tid; i < sh.kCopies * kHistStride; i += NT) sh.hist[0][i] = 0u;
  // valid count (<= 32768) in the high half, valid samples (<= NT) in the low
  uint32_t nvp, kmin_s, kmax;
  block_stats<NT, true>(((lane == 0 ? nvw : 0u) << 16) | (key0 != 0u ? 1u : 0u),
                        key0 != 0u ? key0 : 0xFFFFFFFFu, score_key(mf), sh, nvp, kmin_s, kmax);
  const uint32_t nv = nvp >> 16, n_s = nvp & 0xFFFFu;
  const uint32_t m = nv < (uint32_t)k ? nv : (uint32_t)k;

  if (nv > (uint32_t)k && n_s > 0u) {
    const float expct = (float)m * (float)n_s / (float)nv;
    const uint32_t r = (uint32_t)ceilf(expct + 3.0f * sqrtf(expct) + 8.0f);
    if (r < n_s) {
      // 2. T0 from the sample (its own minimum bounds it from below)
      uint32_t Ts = 0u, need_s = 0u;
      auto sample = [&](auto g) { g(key0); };
      radix_select<NT, decltype(sample), true>(sample, r, kmin_s, kmax, sh, Ts, need_s);
      const uint32_t T0 = need_s != 0u ? Ts : Ts + 1u;
      // T0 as scores: key > T0 <=> f > t_gt and key == T0 <=> f == t_eq.
      // Key 0x7FFFFFFF (that of -0, which counts as +0) is no score's key:
      // above it lies every score >= -0, i.e. above the negative score
      // closest to zero, and nothing equals it.
      float t_gt, t_eq;
      if (T0 == 0x7FFFFFFFu) {
        t_gt = __uint_as_float(0x80000001u);
        t_eq = __uint_as_float(0x7FC00000u);
      } else {
        t_gt = __uint_as_float((T0 & 0x80000000u) ? (T0 ^ 0x80000000u) : ~T0);
        t_eq = t_gt;
      }
      // 3. one pass counts the scores above T0 and writes them to the
      // wavefront's region of the candidate buffer (in position order, when
      // they fit); wavefront totals go to sh.red[1], which nothing rewrites
      // later, and one barrier publishes both.  The scores equal to T0 are
      // counted in the same pass when T0 is a sample key (need_s != 0, ties
      // at T0 likely: the row may end there), otherwise only if the
      // candidates cannot settle the row.
      const bool with_eq = need_s != 0u;
      uint32_t gm = 0, ce0 = 0;  // bit i: f[i] above T0
#pragma unroll
      for (int i = 0; i < KPT; ++i) gm |= (f[i] > t_gt ? 1u : 0u) << i;
      const uint32_t cg0 = (uint32_t)__popc(gm);
      if (with_eq) {
#pragma unroll
        for (int i = 0; i < KPT; ++i) ce0 += f[i] == t_eq;
      }
      // n_cols <= 32768, so both counts fit 16 bits
      const uint32_t pk = (cg0 << 16) | ce0;
      const uint32_t incl = wave_incl_scan_u32(pk);
      const uint32_t wtot = (uint32_t)__builtin_amdgcn_readlane((int)incl, kWave - 1) >> 16;
      if (wtot <= kWaveCap) {
        uint32_t at = (uint32_t)wave * kWaveCap + ((incl - pk) >> 16);
        for (uint32_t mm = gm; mm != 0u; mm &= mm - 1u) cand[at++] = (uint32_t)lo + __builtin_ctz(mm);
      }
      if (lane == kWave - 1) sh.red[1][wave] = incl;
      __syncthreads();
      uint32_t below = 0, tot = 0, wmax = 0;
#pragma unroll
      for (int w = 0; w < kNW; ++w) {
        const uint32_t c = sh.red[1][w];
        below += (w < wave) ? c : 0u;
        tot += c;
        wmax = max(wmax, c >> 16);
      }
      const uint32_t G = tot >> 16;
      if (G <= m) {
        uint32_t excl = below + incl - pk;
        if (!with_eq) {
#pragma unroll
          for (int i = 0; i < KPT; ++i) ce0 += f[i] == t_eq;
          excl = block_excl_scan_tot<NT>((cg0 << 16) | ce0, sh, tot);
        }
        const uint32_t E = tot & 0xFFFFu;
        if (m <= G + E) {
          // T0 is the m-th key: the G scores above it and the first m - G
          // at it
          const uint32_t need0 = m - G;
          const uint32_t base_e = excl & 0xFFFFu;
          uint32_t pos = (excl >> 16) + (base_e < need0 ? base_e : need0);
          uint32_t er = base_e;
#pragma unroll
          for (int i = 0; i < KPT; ++i) {
            if (f[i] > t_gt) {
              orow[pos++] = lo + i + offset;
            } else if (need0 != 0u && f[i] == t_eq) {
              if (er < need0) orow[pos++] = lo + i + offset;
              ++er;
            }
          }
          for (int32_t i = (int32_t)m + tid; i < k; i += NT) orow[i] = -1;
          return;
        }
      } else if (wmax <= kWaveCap) {
        // the top m lie among the candidates; wavefront w's sit at
        // [w * kWaveCap, + its count), in position order.  Each wavefront's
        // lanes take its own region's (lane + 64 s), so slots past the count
        // cost nothing once a whole wavefront has none.
        constexpr int SPT = kWaveCap / kWave;
        const uint32_t cw = sh.red[1][wave] >> 16;
        uint32_t ckr[SPT];
#pragma unroll
        for (int j = 0; j < SPT; ++j) {
          const uint32_t o = (uint32_t)(lane + j * kWave);
          ckr[j] = o < cw ? score_key(stage[staged_at(cand[wave * kWaveCap + o])]) : 0u;
        }
        uint32_t Tc = 0u, need_c = 0u;
        radix_select<NT>(
            [&](auto g) {
#pragma unroll
              for (int j = 0; j < SPT; ++j)
                if ((uint32_t)(lane + j * kWave) < cw) g(ckr[j]);
            },
            m, T0 + 1u, kmax, sh, Tc, need_c);
        // output: thread t takes CPT consecutive slots (one wavefront's
        // region holds all of them), so slot order is position order
        constexpr int CPT = kCandCap / NT;
        const uint32_t c0 = (uint32_t)tid * CPT;
        const uint32_t cw0 = sh.red[1][c0 / kWaveCap] >> 16;
        uint32_t ck[CPT];
        uint32_t cg = 0, ce = 0;
#pragma unroll
        for (int i = 0; i < CPT; ++i) {
          ck[i] = ((c0 + i) % kWaveCap < cw0) ? score_key(stage[staged_at(cand[c0 + i])]) : 0u;
          cg += ck[i] > Tc;
          ce += (need_c != 0u) && (ck[i] == Tc);
        }
        const uint32_t excl = block_excl_scan<NT, true>((cg << 16) | ce, sh);
        const uint32_t base_e = excl & 0xFFFFu;
        uint32_t pos = (excl >> 16) + (base_e < need_c ? base_e : need_c);
        uint32_t er = base_e;
#pragma unroll
        for (int i = 0; i < CPT; ++i) {
          if (ck[i] > Tc) {
            orow[pos++] = (int32_t)cand[c0 + i] + offset;
          } else if (need_c != 0u && ck[i] == Tc) {
            if (er < need_c) orow[pos++] = (int32_t)cand[c0 + i] + offset;
            ++er;
          }
        }
        for (int32_t i = (int32_t)m + tid; i < k; i += NT) orow[i] = -1;
        return;
      }
    }
  }

  // the full select over the keys (every valid score taken when nv <= k);
  // the barrier orders the reads of sh.red above before its next writes
  __syncthreads();
  uint32_t key[KPT];
  uint32_t kmin_t = 0xFFFFFFFFu;
#pragma unroll
  for (int i = 0; i < KPT; ++i) {
    key[i] = score_key(f[i]);
    if (key[i] != 0u) kmin_t = min(kmin_t, key[i]);
  }
  uint32_t T = 0u, need = 0u;
  if (nv > (uint32_t)k) {
    uint32_t unused_n, kmin, unused_max;
    block_stats<NT, true>(0u, kmin_t, 0u, sh, unused_n, kmin, unused_max);
    radix_select<NT>(
        [&](auto g) {
#pragma unroll
          for (int i = 0; i < KPT; ++i) g(key[i]);
        },
        m, kmin, kmax, sh, T, need);
  }
  uint32_t cg = 0, ce = 0;
#pragma unroll
  for (int i = 0; i < KPT; ++i) {
    cg += key[i] > T;
    ce += (need != 0u) && (key[i] == T);
  }
  // n_cols <= 32768, so both counts fit 16 bits
  const uint32_t excl = block_excl_scan<NT, true>((cg << 16) | ce, sh);
  const uint32_t base_e = excl & 0xFFFFu;
  uint32_t pos = (excl >> 16) + (base_e < need ? base_e : need);
  uint32_t er = base_e;
#pragma unroll
  for (int i = 0; i < KPT; ++i) {
    if (key[i] > T) {
      orow[pos++] = lo + i + offset;
    } else if (need != 0u && key[i] == T) {
      if (er < need) orow[pos++] = lo + i + offset;
      ++er;
    }
  }
  for (int32_t i = (int32_t)m + tid; i < k; i += NT) orow[i] = -1;
}

// Short rows (at most 64 * KPL scores, used for KPL = 8): one wavefront per
// row, four rows per workgroup, the whole select inside the wavefront: lane
// l owns positions [l*KPL, (l+1)*KPL); count, min and max by wavefront
// reductions; the radix
// passes count into the wavefront's own LDS histogram (a run of equal digits
// costs one atomic), and lane l reads bins 255-4l .. 252-4l and scans; the
// output slots come from one wavefront scan.  No workgroup barrier: LDS
// operations of one wavefront take effect in order.
constexpr int kWaveRowsPerBlock = 4;

template <int KPL>
__global__ __launch_bounds__(kWave * kWaveRowsPerBlock) void topk_wave_kernel(
    const float* __restrict__ scores, int64_t n_rows, int32_t n_cols, int64_t scores_ld,
    int32_t k, int32_t offset, int32_t* __restrict__ idx, int64_t idx_ld) {
  __shared__ uint32_t hist_all[kWaveRowsPerBlock][256];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int64_t row = (int64_t)blockIdx.x * kWaveRowsPerBlock + wave;
  if (row >= n_rows) return;  // whole wavefront; no barrier follows
  uint32_t* const hist = hist_all[wave];
  const float* __restrict__ srow = scores + row * scores_ld;
  int32_t* __restrict__ orow = idx + row * idx_ld;
  const int32_t lo = lane * KPL;

  uint32_t key[KPL];
  const bool vec = ((reinterpret_cast<uintptr_t>(srow + lo) & 15u) == 0) && (lo + KPL <= n_cols);
  if (vec) {
#pragma unroll
    for (int v = 0; v < KPL / 4; ++v) {
      const float4 f = *reinterpret_cast<const float4*>(srow + lo + 4 * v);
      key[4 * v + 0] = score_key(f.x);
      key[4 * v + 1] = score_key(f.y);
      key[4 * v + 2] = score_key(f.z);
      key[4 * v + 3] = score_key(f.w);
    }
  } else {
#pragma unroll
    for (int i = 0; i < KPL; ++i) key[i] = (lo + i < n_cols) ? score_key(srow[lo + i]) : 0u;
  }
  uint32_t nv = 0, kmin = 0xFFFFFFFFu, kmax = 0u;
#pragma unroll
  for (int i = 0; i < KPL; ++i) {
    if (key[i] != 0u) {
      ++nv;
      kmin = min(kmin, key[i]);
      kmax = max(kmax, key[i]);
    }
  }
  nv = wave_sum_u32(nv);
  kmin = wave_min_u32(kmin);
  kmax = wave_max_u32(kmax);
  const uint32_t m = nv < (uint32_t)k ? nv : (uint32_t)k;

  uint32_t T = 0u, need = 0u;
  if (nv > (uint32_t)k) {
    const uint32_t range = kmax - kmin;
    if (range == 0u) {
      T = kmax;
      need = m;
    } else {
      const int top = 31 - __clz(range);
      int shift = top > 7 ? top - 7 : 0;
      uint32_t prefix = 0u, pmask = 0u, need_r = m;
      bool decided = false;
      for (;;) {
#pragma unroll
        for (int j = 0; j < 4; ++j) hist[4 * lane + j] = 0u;
        uint32_t run_bin = 0u, run_cnt = 0u;
#pragma unroll
        for (int i = 0; i < KPL; ++i) {
          const uint32_t kk = key[i];
          if (kk != 0u) {
            const uint32_t d = kk - kmin;
            if ((d & pmask) == prefix) {
              const uint32_t bin = (d >> shift) & 255u;
              if (run_cnt != 0u && bin != run_bin) {
                atomicAdd(&hist[run_bin], run_cnt);
                run_cnt = 0u;
              }
              run_bin = bin;
              ++run_cnt;
            }
          }
        }
        if (run_cnt != 0u) atomicAdd(&hist[run_bin], run_cnt);
        // lane l: bins 255-4l .. 252-4l, scanned from the top
        uint32_t c[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) c[j] = hist[255 - 4 * lane - j];
        const uint32_t sum4 = c[0] + c[1] + c[2] + c[3];
        const uint32_t incl = wave_incl_scan_u32(sum4);
        const uint32_t excl = incl - sum4;
        const bool mine = excl < need_r && need_r <= incl;
        uint32_t pick = 0u, above = 0u, binc = 0u;  // digit, keys above, bin count
        if (mine) {
          uint32_t cum = excl;
          int j = 0;
          while (j < 3 && need_r > cum + c[j]) cum += c[j++];
          pick = 255u - 4u * (uint32_t)lane - (uint32_t)j;
          above = cum;
          binc = c[j];
        }
        const unsigned long long who = __ballot(mine);
        const int src = (int)__builtin_ctzll(who);
        const uint32_t digit = __builtin_amdgcn_readlane(pick, src);
        above = __builtin_amdgcn_readlane(above, src);
        binc = __builtin_amdgcn_readlane(binc, src);
        prefix |= digit << shift;
        pmask |= 255u << shift;
        need_r -= above;
        if (need_r == binc) {
          T = kmin + prefix - 1u;
          need = 0u;
          decided = true;
          break;
        }
        if (shift == 0) break;
        shift = shift > 8 ? shift - 8 : 0;
      }
      if (!decided) {
        T = kmin + prefix;
        need = need_r;
      }
    }
  }

  uint32_t cg = 0, ce = 0;
#pragma unroll
  for (int i = 0; i < KPL; ++i) {
    cg += key[i] > T;
    ce += (need != 0u) && (key[i] == T);
  }
  // row length <= 64 * KPL <= 4096: both counts fit 16 bits
  const uint32_t packed = (cg << 16) | ce;
  const uint32_t excl = wave_incl_scan_u32(packed) - packed;
  const uint32_t base_e = excl & 0xFFFFu;
  uint32_t pos = (excl >> 16) + (base_e < need ? base_e : need);
  uint32_t er = base_e;
#pragma unroll
  for (int i = 0; i < KPL; ++i) {
    if (key[i] > T) {
      orow[pos++] = lo + i + offset;
    } else if (need != 0u && key[i] == T) {
      if (er < need) orow[pos++] = lo + i + offset;
      ++er;
    }
  }
  for (int32_t i = (int32_t)m + lane; i < k; i += kWave) orow[i] = -1;
}

// Long rows: each thread owns a contiguous range and re-reads its scores.
template <int NT, int HC>
__device__ __forceinline__ void mem_select(const float* __restrict__ srow, int32_t n_cols,
                                           int32_t k, int32_t offset,
                                           int32_t* __restrict__ orow, TopkShared<NT, HC>& sh) {
  const int tid = threadIdx.x;
  const int32_t C = (n_cols + NT - 1) / NT;
  const int32_t lo = tid * C;
  const int32_t hi = lo + C < n_cols ? lo + C : n_cols;
  // the counting passes read the row strided (coalesced; their order does
  // not matter) with eight loads in flight per thread, the output pass in
  // contiguous ranges
  constexpr int U = 8;
  auto for_keys = [&](auto f) {
    for (int32_t j0 = tid; j0 < n_cols; j0 += NT * U) {
      float v[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int32_t j = j0 + u * NT;
        v[u] = j < n_cols ? srow[j] : -__builtin_huge_valf();
      }
#pragma unroll
      for (int u = 0; u < U; ++u) f(score_key(v[u]));
    }
  };

  uint32_t nv_t = 0, kmin_t = 0xFFFFFFFFu, kmax_t = 0u;
  for_keys([&](uint32_t key) {
    if (key != 0u) {
      ++nv_t;
      kmin_t = min(kmin_t, key);
      kmax_t = max(kmax_t, key);
    }
  });
  uint32_t nv, kmin, kmax;
  block_stats<NT>(nv_t, kmin_t, kmax_t, sh, nv, kmin, kmax);
  const uint32_t m = nv < (uint32_t)k ? nv : (uint32_t)k;
  uint32_t T = 0u, need = 0u;
  if (nv > (uint32_t)k) radix_select<NT>(for_keys, m, kmin, kmax, sh, T, need);

  uint32_t cg = 0, ce = 0;
  for (int32_t j0 = lo; j0 < hi; j0 += U) {
    float v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = j0 + u < hi ? srow[j0 + u] : -__builtin_huge_valf();
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const uint32_t key = score_key(v[u]);
      cg += key > T;
      ce += (need != 0u) && (key == T);
    }
  }
  // counts can exceed 16 bits here: two scans
  const uint32_t base_g = block_excl_scan<NT>(cg, sh);
  const uint32_t base_e = block_excl_scan<NT>(ce, sh);
  uint32_t pos = base_g + (base_e < need ? base_e : need);
  uint32_t er = base_e;
  for (int32_t j0 = lo; j0 < hi; j0 += U) {
    float v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = j0 + u < hi ? srow[j0 + u] : -__builtin_huge_valf();
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const uint32_t key = score_key(v[u]);
      if (key > T) {
        orow[pos++] = j0 + u + offset;
      } else if (need != 0u && key == T) {
        if (er < need) orow[pos++] = j0 + u + offset;
        ++er;
      }
    }
  }
  for (int32_t i = (int32_t)m + tid; i < k; i += NT) orow[i] = -1;
}

template <int NT>
__global__ __launch_bounds__(NT) void topk_mem_kernel(const float* __restrict__ scores,
                                                      int32_t n_cols, int64_t scores_ld,
                                                      int32_t k, int32_t offset,
                                                      int32_t* __restrict__ idx,
                                                      int64_t idx_ld) {
  __shared__ TopkShared<NT> sh;
  const int64_t row = blockIdx.x;
  mem_select<NT>(scores + row * scores_ld, n_cols, k, offset, idx + row * idx_ld, sh);
}

// Candidate blocks of a score row: block b covers positions [b*cb, (b+1)*cb);
// its key is the largest key of its positions (key 0, not selectable, when
// none is valid).  The topk_blocks best block keys are chosen exactly as the
// index top-k chooses positions (same radix select, ties to the lower block)
// and written as a byte mask over the ceil(n_cols / cb) blocks.  Thread t owns
// the KPT contiguous blocks [t*KPT, (t+1)*KPT).
// CB > 0 fixes the block size at compile time (16-byte loads, all issued
// before the maxima are taken); CB == 0 reads a runtime block size one score
// at a time.
template <int NT, int KPT, int CB>
__global__ __launch_bounds__(NT) void cand_reg_kernel(const float* __restrict__ scores,
                                                      int32_t n_cols, int64_t scores_ld,
                                                      int32_t cb_rt, int32_t k,
                                                      uint8_t* __restrict__ cand,
                                                      int64_t cand_ld) {
  __shared__ TopkShared<NT> sh;
  const int tid = threadIdx.x;
  const int64_t row = blockIdx.x;
  const float* __restrict__ srow = scores + row * scores_ld;
  uint8_t* __restrict__ crow = cand + row * cand_ld;
  const int32_t cb = CB > 0 ? CB : cb_rt;
  const int32_t nb = (n_cols + cb - 1) / cb;
  const int32_t b0 = tid * KPT;

  uint32_t key[KPT];
  if constexpr (CB > 0) {
    // whole blocks of this thread lie inside the row and start 16-byte aligned
    const bool vec = ((reinterpret_cast<uintptr_t>(srow) & 15u) == 0) &&
                     (b0 + KPT) * CB <= n_cols;
    if (vec) {
      float4 f[KPT][CB / 4];
#pragma unroll
      for (int i = 0; i < KPT; ++i)
#pragma unroll
        for (int v = 0; v < CB / 4; ++v)
          f[i][v] = *reinterpret_cast<const float4*>(srow + (b0 + i) * CB + 4 * v);
#pragma unroll
      for (int i = 0; i < KPT; ++i) {
        uint32_t m = 0u;
#pragma unroll
        for (int v = 0; v < CB / 4; ++v) {
          m = max(m, score_key(f[i][v].x));
          m = max(m, score_key(f[i][v].y));
          m = max(m, score_key(f[i][v].z));
          m = max(m, score_key(f[i][v].w));
        }
        key[i] = m;
      }
    } else {
#pragma unroll
      for (int i = 0; i < KPT; ++i) {
        uint32_t m = 0u;
        const int32_t j0 = (b0 + i) * CB;
#pragma unroll
        for (int j = 0; j < CB; ++j)
          if (j0 + j < n_cols) m = max(m, score_key(srow[j0 + j]));
        key[i] = m;
      }
    }
  } else {
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
      uint32_t m = 0u;
      if (b0 + i < nb) {
        const int32_t j0 = (b0 + i) * cb;
        const int32_t j1 = j0 + cb < n_cols ? j0 + cb : n_cols;
        for (int32_t j = j0; j < j1; ++j) m = max(m, score_key(srow[j]));
      }
      key[i] = m;
    }
  }
  uint32_t nv_t = 0, kmin_t = 0xFFFFFFFFu, kmax_t = 0u;
#pragma unroll
  for (int i = 0; i < KPT; ++i) {
    if (key[i] != 0u) {
      ++nv_t;
      kmin_t = min(kmin_t, key[i]);
      kmax_t = max(kmax_t, key[i]);
    }
  }
  uint32_t nv, kmin, kmax;
  block_stats<NT>(nv_t, kmin_t, kmax_t, sh, nv, kmin, kmax);
  const uint32_t m = nv < (uint32_t)k ? nv : (uint32_t)k;
  uint32_t T = 0u, need = 0u;
  if (nv > (uint32_t)k) {
    radix_select<NT>(
        [&](auto f) {
#pragma unroll
          for (int i = 0; i < KPT; ++i) f(key[i]);
        },
        m, kmin, kmax, sh, T, need);
  }
  uint32_t ce = 0;
#pragma unroll
  for (int i = 0; i < KPT; ++i) ce += (need != 0u) && (key[i] == T);
  uint32_t er = block_excl_scan<NT>(ce, sh);
#pragma unroll
  for (int i = 0; i < KPT; ++i) {
    uint8_t take = 0;
    if (key[i] > T) {
      take = 1;
    } else if (need != 0u && key[i] == T) {
      take = er < need ? 1 : 0;
      ++er;
    }
    if (b0 + i < nb) crow[b0 + i] = take;
  }
}

}  // namespace

hipError_t launch_candidate_blocks(const float* scores, int64_t n_sel_rows, int64_t n_cols,
                                   int64_t scores_ld, int32_t cand_block, int32_t topk_blocks,
                                   uint8_t* cand, int64_t cand_ld, hipStream_t s) {
  if (n_sel_rows == 0) return hipSuccess;
  const dim3 grid((unsigned)n_sel_rows);
  const int64_t nb = (n_cols + cand_block - 1) / cand_block;
  const int32_t nc = (int32_t)n_cols;  // the ABI bounds the block count
#define V41_CAND(NT_, KPT_, CB_)                                                              \
  hipLaunchKernelGGL((cand_reg_kernel<NT_, KPT_, CB_>), grid, dim3(NT_), 0, s, scores, nc,   \
                     scores_ld, cand_block, topk_blocks, cand, cand_ld)
  if (cand_block == 8) {
    // the configured block size
    if (nb <= 256 * 4) V41_CAND(256, 4, 8);
    else if (nb <= 1024 * 4) V41_CAND(1024, 4, 8);
    else if (nb <= 1024 * 16) V41_CAND(1024, 16, 0);
    else V41_CAND(1024, 32, 0);
  } else {
    if (nb <= 256 * 4) V41_CAND(256, 4, 0);
    else if (nb <= 1024 * 4) V41_CAND(1024, 4, 0);
    else if (nb <= 1024 * 16) V41_CAND(1024, 16, 0);
    else V41_CAND(1024, 32, 0);
  }
#undef V41_CAND
  return hipGetLastError();
}

hipError_t launch_topk_select(const float* scores, int64_t n_sel_rows, int64_t n_cols,
                              int64_t scores_ld, int32_t k, int32_t offset, int32_t* idx,
                              int64_t idx_ld, hipStream_t s) {
  if (n_sel_rows == 0) return hipSuccess;
  const dim3 grid((unsigned)n_sel_rows);
  const int32_t nc = (int32_t)n_cols;  // the ABI bounds n_cols below 2^31
#define V41_TOPK_REG(NT_, KPT_)                                                            \
  hipLaunchKernelGGL((topk_reg_kernel<NT_, KPT_>), grid, dim3(NT_), 0, s, scores, nc,      \
                     scores_ld, k, offset, idx, idx_ld)
  if (n_cols <= 64 * 8) {
    // short rows: one wavefront each (with 16 keys per lane a 1024-score row
    // measured slower than 256 threads, 5.8 against 4.7 us)
    const dim3 wgrid((unsigned)((n_sel_rows + kWaveRowsPerBlock - 1) / kWaveRowsPerBlock));
    hipLaunchKernelGGL((topk_wave_kernel<8>), wgrid, dim3(kWave * kWaveRowsPerBlock), 0, s,
                       scores, n_sel_rows, nc, scores_ld, k, offset, idx, idx_ld);
  } else if (n_cols <= 256 * 4) {
    V41_TOPK_REG(256, 4);
  } else if (n_cols <= 256 * 8) {
    V41_TOPK_REG(256, 8);
  } else if (n_cols <= 256 * 16) {
    V41_TOPK_REG(256, 16);
  } else if (n_cols <= 1024 * 8) {
    V41_TOPK_REG(1024, 8);
  } else if (n_cols <= 1024 * 32) {
    hipLaunchKernelGGL((topk_long_kernel<1024, 32>), grid, dim3(1024), 0, s, scores, nc,
                       scores_ld, k, offset, idx, idx_ld);
  } else {
    hipLaunchKernelGGL((topk_mem_kernel<1024>), grid, dim3(1024), 0, s, scores, nc, scores_ld,
                       k, offset, idx, idx_ld);
  }
#undef V41_TOPK_REG
  return hipGetLastError();
}

}  // namespace v41
