// Indexer score S[q, j] = sum_h w[q, h] * ReLU(qI[q, h, :] . kI[j, :]) over the
// visible compressed positions ("Compressed sparse attention" page, "All 25
// steps", S^I and I_t), for gfx950.
//
// The contraction is qI[heads x DI] x kI^T[DI x 16 positions] on the matrix
// cores (v_mfma_f32_16x16x32_bf16): the heads are the M side (16 per tile, up
// to 4 tiles), 16 positions the N side, DI the K side.  One wavefront owns a
// query and a run of positions: its qI fragments and weights stay in
// registers, and it streams the index keys straight from HBM into MFMA B
// operands (each lane loads 16 contiguous bytes of one key; the 16-lane groups
// of a load cover 16 keys x 64 bytes), one 16-key block ahead of the block it
// multiplies.  The epilogue applies ReLU and the weights in f32, sums the 4
// heads a lane holds per tile, then across the 4 lane groups with two
// xor-shuffles.  Keys past the causal bound or in a masked candidate block are
// never loaded; their scores are -inf.
#include "v41_common.h"

namespace v41 {
namespace {

constexpr int kWavesPerBlock = 4;

template <int DI, int HT>
__global__ __launch_bounds__(256) void indexer_kernel(
    const uint16_t* __restrict__ qI, const uint16_t* __restrict__ kI, int64_t kI_bs,
    const float* __restrict__ w, const uint8_t* __restrict__ cand, int32_t cand_width,
    int32_t cand_block, int32_t n_tokens, int64_t n_queries, int64_t start_pos,
    int32_t ratio, int32_t n_heads, int64_t n_rows, float* __restrict__ scores,
    int64_t scores_ld, int32_t rows_per_wave, int32_t waves_per_query) {
  constexpr int KS = DI / 32;
  const int lane = threadIdx.x & 63;
  const int64_t wv = (int64_t)blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6);
  const int64_t q = wv / waves_per_query;
  if (q >= n_queries) return;
  const int64_t part = wv - q * waves_per_query;
  const int64_t b = q / n_tokens;
  const int64_t t = q - b * n_tokens;
  int64_t n_vis = (start_pos + t + 1) / ratio;
  if (n_vis > n_rows) n_vis = n_rows;
  const int64_t j_begin = part * rows_per_wave;
  int64_t j_end = j_begin + rows_per_wave;
  if (j_end > n_rows) j_end = n_rows;
  if (j_begin >= j_end) return;
  const int64_t live_end = j_end < n_vis ? j_end : n_vis;

  float* __restrict__ srow = scores + q * scores_ld;
  const float kNegInf = -__builtin_huge_valf();
  for (int64_t j = (j_begin > live_end ? j_begin : live_end) + lane; j < j_end; j += kWave)
    srow[j] = kNegInf;
  if (j_begin >= live_end) return;

  const int r16 = lane & 15;
  const int g = lane >> 4;

  bf16x8 afr[HT][KS];
  float wh[HT][4];
#pragma unroll
  for (int ht = 0; ht < HT; ++ht) {
    const int h = 16 * ht + r16;
    const uint16_t* qp = qI + (q * n_heads + h) * DI + 8 * g;
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) {
      u32x4 v = {0u, 0u, 0u, 0u};
      if (h < n_heads) v = *reinterpret_cast<const u32x4*>(qp + 32 * kk);
      afr[ht][kk] = as_bf16x8(v);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int hh = 16 * ht + 4 * g + i;
      wh[ht][i] = hh < n_heads ? w[q * n_heads + hh] : 0.0f;
    }
  }

  const uint16_t* __restrict__ kb = kI + b * kI_bs + 8 * g;
  const uint8_t* __restrict__ crow = cand ? cand + q * cand_width : nullptr;

  // positions stay below 2^31 (checked by the C ABI), so 32-bit division
  auto allowed = [&](int64_t j) -> bool {
    return j < live_end && (crow == nullptr || crow[(uint32_t)j / (uint32_t)cand_block] != 0);
  };
  auto load_block = [&](int64_t j0, u32x4 (&buf)[KS]) {
    const int64_t j = j0 + r16;
    const bool ok = allowed(j);
    const uint16_t* p = kb + (ok ? j : j0) * DI;
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) {
      u32x4 v = {0u, 0u, 0u, 0u};
      if (ok) v = *reinterpret_cast<const u32x4*>(p + 32 * kk);
      buf[kk] = v;
    }
  };

  u32x4 cur[KS], nxt[KS];
  load_block(j_begin, cur);
  for (int64_t j0 = j_begin; j0 < live_end; j0 += 16) {
    const int64_t jn = j0 + 16;
    if (jn < live_end) load_block(jn, nxt);
    f32x4 acc[HT];
#pragma unroll
    for (int ht = 0; ht < HT; ++ht) acc[ht] = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) {
      const bf16x8 bk = as_bf16x8(cur[kk]);
#pragma unroll
      for (int ht = 0; ht < HT; ++ht) acc[ht] = mfma16x16x32(afr[ht][kk], bk, acc[ht]);
    }
    float part_sum = 0.0f;
#pragma unroll
    for (int ht = 0; ht < HT; ++ht)
#pragma unroll
      for (int i = 0; i < 4; ++i) part_sum += wh[ht][i] * fmaxf(acc[ht][i], 0.0f);
    part_sum += __shfl_xor(part_sum, 16);
    part_sum += __shfl_xor(part_sum, 32);
    const int64_t j = j0 + r16;
    if (g == 0 && j < live_end) srow[j] = allowed(j) ? part_sum : kNegInf;
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) cur[kk] = nxt[kk];
  }
}

template <int DI>
hipError_t dispatch_heads(int ht, dim3 grid, hipStream_t s, const uint16_t* qI,
                          const uint16_t* kI, int64_t kI_bs, const float* w,
                          const uint8_t* cand, int32_t cand_width, int32_t cand_block,
                          int32_t n_tokens, int64_t nq, int64_t start_pos, int32_t ratio,
                          int32_t n_heads, int64_t n_rows, float* scores, int64_t scores_ld,
                          int32_t rpw, int32_t wpq) {
#define V41_IDX_LAUNCH(HT_)                                                                  \
  hipLaunchKernelGGL((indexer_kernel<DI, HT_>), grid, dim3(256), 0, s, qI, kI, kI_bs, w,    \
                     cand, cand_width, cand_block, n_tokens, nq, start_pos, ratio, n_heads, \
                     n_rows, scores, scores_ld, rpw, wpq)
  switch (ht) {
    case 1: V41_IDX_LAUNCH(1); break;
    case 2: V41_IDX_LAUNCH(2); break;
    case 3: V41_IDX_LAUNCH(3); break;
    default: V41_IDX_LAUNCH(4); break;
  }
#undef V41_IDX_LAUNCH
  return hipGetLastError();
}

}  // namespace

hipError_t launch_indexer_scores(const uint16_t* qI, const uint16_t* kI, int64_t kI_bs,
                                 const float* w, const uint8_t* cand, int32_t cand_width,
                                 int32_t cand_block, int32_t batch, int32_t n_tokens,
                                 int64_t start_pos, int32_t ratio, int32_t n_heads,
                                 int32_t head_dim, int64_t n_rows, float* scores,
                                 int64_t scores_ld, hipStream_t s) {
  const int64_t nq = (int64_t)batch * n_tokens;
  if (nq == 0 || n_rows == 0) return hipSuccess;
  // Rows per wavefront: enough wavefronts to keep HBM busy (~2k), at most 256
  // keys (64 KB at DI = 128) per wavefront so its qI fragments stay amortised.
  int64_t rpw = (nq * n_rows + 2047) / 2048;
  rpw = (rpw + 15) / 16 * 16;
  if (rpw < 32) rpw = 32;
  if (rpw > 256) rpw = 256;
  const int64_t wpq = (n_rows + rpw - 1) / rpw;
  const int64_t waves = nq * wpq;
  const int64_t blocks = (waves + kWavesPerBlock - 1) / kWavesPerBlock;
  const int ht = (n_heads + 15) / 16;
  const dim3 grid((unsigned)blocks);
  switch (head_dim) {
    case 32:
      return dispatch_heads<32>(ht, grid, s, qI, kI, kI_bs, w, cand, cand_width, cand_block,
                                n_tokens, nq, start_pos, ratio, n_heads, n_rows, scores,
                                scores_ld, (int32_t)rpw, (int32_t)wpq);
    case 64:
      return dispatch_heads<64>(ht, grid, s, qI, kI, kI_bs, w, cand, cand_width, cand_block,
                                n_tokens, nq, start_pos, ratio, n_heads, n_rows, scores,
                                scores_ld, (int32_t)rpw, (int32_t)wpq);
    default:
      return dispatch_heads<128>(ht, grid, s, qI, kI, kI_bs, w, cand, cand_width, cand_block,
                                 n_tokens, nq, start_pos, ratio, n_heads, n_rows, scores,
                                 scores_ld, (int32_t)rpw, (int32_t)wpq);
  }
}

}  // namespace v41
