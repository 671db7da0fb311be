// Window selection (window_topk_idxs contract of the "deepseek_v41_ref::attn"
// rustdoc; J^w_t of the "Compressed sparse attention" page), for gfx950.
// One thread per output entry; the layout is the same for every sequence of
// the batch.
#include "v41_common.h"

namespace v41 {
namespace {

__global__ __launch_bounds__(256) void window_idx_kernel(int64_t start_pos, int32_t n_tokens,
                                                         int32_t window, int32_t cols,
                                                         int32_t batch, int32_t* idx,
                                                         int64_t idx_ld, int64_t idx_bs) {
  // the C ABI keeps batch * n_tokens * cols below 2^31
  const int32_t per_seq = n_tokens * cols;
  const int32_t total = per_seq * batch;
  for (int32_t e = (int32_t)(blockIdx.x * blockDim.x + threadIdx.x); e < total;
       e += (int32_t)(gridDim.x * blockDim.x)) {
    const int32_t b = e / per_seq;
    const int32_t rem = e - b * per_seq;
    const int32_t t = rem / cols;
    const int32_t c = rem - t * cols;
    int32_t v;
    if (start_pos == 0) {
      // causal band of the chunk: rows max(0, t-window+1) .. t, then -1
      const int32_t lo = t - window + 1 > 0 ? t - window + 1 : 0;
      v = (lo + c <= t) ? lo + c : -1;
    } else if (start_pos >= window - 1) {
      // full ring, oldest first: the token start_pos - window + 1 + c
      v = (int32_t)((start_pos + 1 + c) % window);
    } else {
      v = (c <= start_pos) ? c : -1;
    }
    idx[(int64_t)b * idx_bs + (int64_t)t * idx_ld + c] = v;
  }
}

}  // namespace

hipError_t launch_window_idx(int64_t start_pos, int32_t n_tokens, int32_t window,
                             int32_t cols, int32_t batch, int32_t* idx, int64_t idx_ld,
                             int64_t idx_bs, hipStream_t s) {
  const int64_t total = (int64_t)batch * n_tokens * cols;
  if (total == 0) return hipSuccess;
  int64_t blocks = (total + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(window_idx_kernel, dim3((unsigned)blocks), dim3(256), 0, s, start_pos,
                     n_tokens, window, cols, batch, idx, idx_ld, idx_bs);
  return hipGetLastError();
}

}  // namespace v41
