// C ABI of libv41: argument validation on the host, the gfx950 device check,
// the thread-local last-error message, then one launcher per call.  The
// contracts (and the passages of the pages they come from) are in
// include/v41.h.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>

#include "../../include/v41.h"
#include "v41_common.h"
#include "v41_rope.h"
#include "v41_gemm.h"
#include "v41_front.h"

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return code;
}

// 0 = unknown, 1 = gfx950, 2 = other device
std::atomic<int> g_dev_kind[64];

int check_device() {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(V41_EHIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= 64) return fail(V41_EDEVICE, "device ordinal %d out of range", dev);
  int kind = g_dev_kind[dev].load(std::memory_order_relaxed);
  if (kind == 0) {
    hipDeviceProp_t prop;
    e = hipGetDeviceProperties(&prop, dev);
    if (e != hipSuccess)
      return fail(V41_EHIP, "hipGetDeviceProperties: %s", hipGetErrorString(e));
    kind = (std::strncmp(prop.gcnArchName, "gfx950", 6) == 0) ? 1 : 2;
    g_dev_kind[dev].store(kind, std::memory_order_relaxed);
    if (kind == 2)
      return fail(V41_EDEVICE, "device %d is %s, this library is built for gfx950", dev,
                  prop.gcnArchName);
  }
  if (kind == 2) return fail(V41_EDEVICE, "device %d is not a gfx950", dev);
  return V41_OK;
}

int launched(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(V41_EHIP, "%s launch: %s", what, hipGetErrorString(e));
  g_err[0] = '\0';
  return V41_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

}  // namespace

extern "C" {

const char* v41_last_error(void) { return g_err; }

int v41_abi_version(void) { return 8; }

int v41_fp8_round_rows(const v41_bf16* in, int64_t in_ld, v41_bf16* out, int64_t out_ld,
                       int64_t rows, int32_t row_len, v41_bf16* ring, int32_t ring_slots,
                       int64_t first_pos, v41_stream stream) {
  if (rows < 0) return fail(V41_EINVAL, "fp8_round_rows: rows < 0");
  if (row_len <= 0 || row_len % V41_FP8_BLOCK != 0)
    return fail(V41_EINVAL, "fp8_round_rows: row_len %d is not a positive multiple of %d",
                row_len, V41_FP8_BLOCK);
  if (in_ld < row_len || out_ld < row_len || in_ld % 8 != 0 || out_ld % 8 != 0)
    return fail(V41_EINVAL, "fp8_round_rows: in_ld/out_ld must be >= row_len and multiples of 8");
  if (rows > 0 && (in == nullptr || out == nullptr))
    return fail(V41_EINVAL, "fp8_round_rows: NULL in/out");
  if (!aligned16(in) || !aligned16(out) || !aligned16(ring))
    return fail(V41_EINVAL, "fp8_round_rows: pointers must be 16-byte aligned");
  if (ring != nullptr && ring_slots <= 0)
    return fail(V41_EINVAL, "fp8_round_rows: ring given with ring_slots <= 0");
  if (ring != nullptr && first_pos < 0)
    return fail(V41_EINVAL, "fp8_round_rows: first_pos < 0");
  if (rows * (int64_t)(row_len / 8) >= 0x7FFFFFFFLL)
    return fail(V41_EINVAL, "fp8_round_rows: rows * row_len / 8 must stay below 2^31");
  int rc = check_device();
  if (rc) return rc;
  return launched(v41::launch_fp8_round_rows(in, in_ld, out, out_ld, rows, row_len, ring,
                                             ring_slots, first_pos, (hipStream_t)stream),
                  "fp8_round_rows");
}

int v41_window_idx(int64_t start_pos, int32_t n_tokens, int32_t window, int32_t batch,
                   int32_t* idx, int64_t idx_ld, int64_t idx_bs, int32_t* cols_out,
                   v41_stream stream) {
  if (start_pos < 0 || n_tokens < 0 || window <= 0 || batch < 0)
    return fail(V41_EINVAL, "window_idx: negative start_pos/n_tokens/batch or window <= 0");
  if (start_pos > 0 && n_tokens != 1)
    return fail(V41_EINVAL, "window_idx: a decode call (start_pos > 0) takes one token, got %d",
                n_tokens);
  const int32_t cols = (start_pos == 0) ? (n_tokens < window ? n_tokens : window) : window;
  if (idx_ld < cols) return fail(V41_EINVAL, "window_idx: idx_ld %lld < cols %d",
                                 (long long)idx_ld, cols);
  if (batch > 1 && idx_bs < (int64_t)n_tokens * idx_ld)
    return fail(V41_EINVAL, "window_idx: idx_bs too small");
  if ((int64_t)batch * n_tokens * cols >= 0x7FFFFFFFLL)
    return fail(V41_EINVAL, "window_idx: batch * n_tokens * cols must stay below 2^31");
  if (idx == nullptr && (int64_t)batch * n_tokens * cols > 0)
    return fail(V41_EINVAL, "window_idx: NULL idx");
  if (cols_out) *cols_out = cols;
  int rc = check_device();
  if (rc) return rc;
  return launched(v41::launch_window_idx(start_pos, n_tokens, window, cols, batch, idx, idx_ld,
                                         idx_bs, (hipStream_t)stream),
                  "window_idx");
}

int v41_indexer_scores(const v41_bf16* qI, const v41_bf16* kI, int64_t kI_bs, const float* w,
                       const uint8_t* cand, int32_t cand_width, int32_t cand_block,
                       int32_t batch, int32_t n_tokens, int64_t start_pos, int32_t ratio,
                       int32_t n_heads, int32_t head_dim, int64_t n_rows, float* scores,
                       int64_t scores_ld, v41_stream stream) {
  if (batch < 0 || n_tokens < 0 || n_rows < 0 || start_pos < 0)
    return fail(V41_EINVAL, "indexer_scores: negative batch/n_tokens/n_rows/start_pos");
  if (ratio < 1) return fail(V41_EINVAL, "indexer_scores: ratio %d < 1", ratio);
  if (n_heads < 1 || n_heads > V41_MAX_INDEX_HEADS)
    return fail(V41_EINVAL, "indexer_scores: n_heads %d outside 1..%d", n_heads,
                V41_MAX_INDEX_HEADS);
  if (head_dim != 32 && head_dim != 64 && head_dim != 128)
    return fail(V41_EINVAL, "indexer_scores: head_dim %d not in {32, 64, 128}", head_dim);
  if (start_pos > 0 && n_tokens != 1)
    return fail(V41_EINVAL, "indexer_scores: a decode call (start_pos > 0) takes one token");
  if (scores_ld < n_rows) return fail(V41_EINVAL, "indexer_scores: scores_ld < n_rows");
  if (n_rows >= 0x7FFFFFFFLL) return fail(V41_EINVAL, "indexer_scores: n_rows must stay below 2^31");
  if (batch > 1 && kI_bs < n_rows * head_dim)
    return fail(V41_EINVAL, "indexer_scores: kI_bs < n_rows * head_dim");
  if (kI_bs % 8 != 0) return fail(V41_EINVAL, "indexer_scores: kI_bs must be a multiple of 8");
  const bool work = (int64_t)batch * n_tokens > 0 && n_rows > 0;
  if (work && (qI == nullptr || kI == nullptr || w == nullptr || scores == nullptr))
    return fail(V41_EINVAL, "indexer_scores: NULL qI/kI/w/scores (kI NULL means no latent "
                            "index-key cache has been published)");
  if (cand != nullptr && (cand_block < 1 || (int64_t)cand_width * cand_block < n_rows))
    return fail(V41_EINVAL, "indexer_scores: candidate mask needs cand_block >= 1 and "
                            "cand_width * cand_block >= n_rows");
  if (!aligned16(qI) || !aligned16(kI))
    return fail(V41_EINVAL, "indexer_scores: qI and kI must be 16-byte aligned");
  int rc = check_device();
  if (rc) return rc;
  return launched(v41::launch_indexer_scores(qI, kI, kI_bs, w, cand, cand_width, cand_block,
                                             batch, n_tokens, start_pos, nullptr, ratio,
                                             n_heads, head_dim, n_rows, scores, scores_ld,
                                             (hipStream_t)stream),
                  "indexer_scores");
}

int v41_topk_select(const float* scores, int64_t n_sel_rows, int64_t n_cols, int64_t scores_ld,
                    int32_t k, int32_t offset, int32_t* idx, int64_t idx_ld,
                    v41_stream stream) {
  if (n_sel_rows < 0 || n_cols < 0) return fail(V41_EINVAL, "topk_select: negative size");
  if (k < 1 || k > V41_MAX_WIDTH)
    return fail(V41_EINVAL, "topk_select: k %d outside 1..%d", k, V41_MAX_WIDTH);
  if (scores_ld < n_cols) return fail(V41_EINVAL, "topk_select: scores_ld < n_cols");
  if (idx_ld < k) return fail(V41_EINVAL, "topk_select: idx_ld < k");
  if (n_cols >= 0x7FFFFFFFLL) return fail(V41_EINVAL, "topk_select: n_cols too large");
  if (n_sel_rows > 0 && (idx == nullptr || (scores == nullptr && n_cols > 0)))
    return fail(V41_EINVAL, "topk_select: NULL scores/idx");
  if (offset < 0 || (int64_t)offset + n_cols > 0x7FFFFFFFLL)
    return fail(V41_EINVAL, "topk_select: offset out of range");
  int rc = check_device();
  if (rc) return rc;
  return launched(v41::launch_topk_select(scores, n_sel_rows, n_cols, scores_ld, k, offset, idx,
                                          idx_ld, (hipStream_t)stream),
                  "topk_select");
}

int64_t v41_sparse_attn_workspace_bytes(int32_t batch, int32_t n_tokens, int32_t n_heads,
                                        int32_t head_dim, int32_t width) {
  if (batch <= 0 || n_tokens <= 0 || n_heads <= 0 || width <= 0) return 0;
  const int32_t nq = batch * n_tokens;
  return v41::attn_workspace_bytes(nq, n_heads, head_dim,
                                   v41::attn_preferred_splits(nq, n_heads, width));
}

}  // extern "C"

namespace {

// The device array behind v41_sparse_attn_sink_noalloc.  In host code its
// name stands for a host-side shadow, not a device address: kernels get the
// address hipGetSymbolAddress returns for the current device.
__device__ __align__(256) uint8_t scratch[V41_NOALLOC_SCRATCH_BYTES];

std::mutex g_scratch_mu;
void* g_scratch_ptr[64];  // per device ordinal, set on the first call there

// This device's address of `scratch` (the device is current and checked).
int scratch_address(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(V41_EHIP, "hipGetDevice: %s", hipGetErrorString(e));
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || p == nullptr)
      return fail(V41_EHIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev,
                  hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return V41_OK;
}

// Checks and launch shared by the two attention entry points.  With
// `noalloc`, the workspace arguments are ignored and the device scratch array
// serves instead.
int sparse_attn_call(const v41_bf16* q, const v41_bf16* rows_a, int64_t rows_a_len,
                     int64_t a_bs, const v41_bf16* rows_b, int64_t rows_b_len, int64_t b_bs,
                     const int32_t* idx, int32_t width, int64_t idx_ld, const float* sink,
                     float scale, int32_t batch, int32_t n_tokens, int32_t n_heads,
                     int32_t head_dim, v41_bf16* out, void* workspace, int64_t workspace_bytes,
                     bool noalloc, v41_stream stream) {
  if (batch < 0 || n_tokens < 0 || rows_a_len < 0 || rows_b_len < 0)
    return fail(V41_EINVAL, "sparse_attn_sink: negative size");
  if (n_heads < 1) return fail(V41_EINVAL, "sparse_attn_sink: n_heads < 1");
  if (head_dim != 64 && head_dim != 128 && head_dim != 256 && head_dim != 512)
    return fail(V41_EINVAL, "sparse_attn_sink: head_dim %d not in {64, 128, 256, 512}",
                head_dim);
  if (width < 0 || width > V41_MAX_WIDTH)
    return fail(V41_EINVAL, "sparse_attn_sink: width %d outside 0..%d (the selection limit)",
                width, V41_MAX_WIDTH);
  if (idx_ld < width) return fail(V41_EINVAL, "sparse_attn_sink: idx_ld < width");
  if (rows_b == nullptr && rows_b_len > 0)
    return fail(V41_EINVAL, "sparse_attn_sink: rows_b is NULL but rows_b_len = %lld (no "
                            "latent cache published)",
                (long long)rows_b_len);
  if (rows_a_len + rows_b_len > 0x7FFFFFFFLL)
    return fail(V41_EINVAL, "sparse_attn_sink: too many rows for int32 indices");
  if (batch > 1 && (a_bs < rows_a_len * head_dim || (rows_b_len > 0 && b_bs < rows_b_len * head_dim)))
    return fail(V41_EINVAL, "sparse_attn_sink: a_bs/b_bs smaller than one sequence's rows");
  if (a_bs % 8 != 0 || b_bs % 8 != 0)
    return fail(V41_EINVAL, "sparse_attn_sink: a_bs/b_bs must be multiples of 8");
  const int64_t nq = (int64_t)batch * n_tokens;
  if (nq > 0x7FFFFFFFLL) return fail(V41_EINVAL, "sparse_attn_sink: too many queries");
  if (nq > 0 && (q == nullptr || out == nullptr || sink == nullptr ||
                 (width > 0 && idx == nullptr) || (rows_a == nullptr && rows_a_len > 0)))
    return fail(V41_EINVAL, "sparse_attn_sink: NULL q/out/sink/idx/rows_a");
  if (!aligned16(q) || !aligned16(rows_a) || !aligned16(rows_b) || !aligned16(out) ||
      !aligned16(workspace))
    return fail(V41_EINVAL, "sparse_attn_sink: q/rows/out/workspace must be 16-byte aligned");
  if (workspace_bytes < 0) return fail(V41_EINVAL, "sparse_attn_sink: workspace_bytes < 0");
  int rc = check_device();
  if (rc) return rc;
  if (noalloc) {
    // exactly the split the workspace-taking call prefers for this shape
    const int64_t need = (nq > 0 && width > 0)
                             ? v41::attn_workspace_bytes(
                                   (int32_t)nq, n_heads, head_dim,
                                   v41::attn_preferred_splits((int32_t)nq, n_heads, width))
                             : 0;
    if (need > V41_NOALLOC_SCRATCH_BYTES)
      return fail(V41_EINVAL,
                  "sparse_attn_sink_noalloc: this shape needs %lld bytes of scratch, more "
                  "than the static %lld; call v41_sparse_attn_sink with a workspace",
                  (long long)need, (long long)V41_NOALLOC_SCRATCH_BYTES);
    workspace = nullptr;
    workspace_bytes = 0;
    if (need > 0) {
      rc = scratch_address(&workspace);
      if (rc) return rc;
      workspace_bytes = need;
    }
  }
  v41::AttnArgs a;
  a.q = q;
  a.rows_a = rows_a;
  a.rows_a_len = rows_a_len;
  a.a_bs = a_bs;
  a.rows_b = rows_b;
  a.rows_b_len = rows_b_len;
  a.b_bs = b_bs;
  a.idx = idx;
  a.width = width;
  a.idx_ld = idx_ld;
  a.sink = sink;
  a.scale = scale;
  a.batch = batch;
  a.n_tokens = n_tokens;
  a.n_heads = n_heads;
  a.head_dim = head_dim;
  a.out = out;
  a.workspace = workspace;
  a.workspace_bytes = workspace ? workspace_bytes : 0;
  return launched(v41::launch_sparse_attn_sink(a, (hipStream_t)stream),
                  noalloc ? "sparse_attn_sink_noalloc" : "sparse_attn_sink");
}

}  // namespace

extern "C" {

int v41_sparse_attn_sink(const v41_bf16* q, const v41_bf16* rows_a, int64_t rows_a_len,
                         int64_t a_bs, const v41_bf16* rows_b, int64_t rows_b_len, int64_t b_bs,
                         const int32_t* idx, int32_t width, int64_t idx_ld, const float* sink,
                         float scale, int32_t batch, int32_t n_tokens, int32_t n_heads,
                         int32_t head_dim, v41_bf16* out, void* workspace,
                         int64_t workspace_bytes, v41_stream stream) {
  return sparse_attn_call(q, rows_a, rows_a_len, a_bs, rows_b, rows_b_len, b_bs, idx, width,
                          idx_ld, sink, scale, batch, n_tokens, n_heads, head_dim, out,
                          workspace, workspace_bytes, false, stream);
}

int v41_sparse_attn_sink_noalloc(const v41_bf16* q, const v41_bf16* rows_a, int64_t rows_a_len,
                                 int64_t a_bs, const v41_bf16* rows_b, int64_t rows_b_len,
                                 int64_t b_bs, const int32_t* idx, int32_t width,
                                 int64_t idx_ld, const float* sink, float scale, int32_t batch,
                                 int32_t n_tokens, int32_t n_heads, int32_t head_dim,
                                 v41_bf16* out, v41_stream stream) {
  return sparse_attn_call(q, rows_a, rows_a_len, a_bs, rows_b, rows_b_len, b_bs, idx, width,
                          idx_ld, sink, scale, batch, n_tokens, n_heads, head_dim, out, nullptr,
                          0, true, stream);
}

int v41_rope_table(double theta, int32_t rope_dim, int64_t n_pos, float* table,
                   v41_stream stream) {
  if (!(theta > 0.0) || !(theta < 1e300))
    return fail(V41_EINVAL, "rope_table: theta must be positive and finite");
  if (rope_dim <= 0 || rope_dim % 2 != 0)
    return fail(V41_EINVAL, "rope_table: rope_dim %d is not a positive even number", rope_dim);
  if (n_pos < 0) return fail(V41_EINVAL, "rope_table: n_pos < 0");
  if (n_pos > 0 && table == nullptr) return fail(V41_EINVAL, "rope_table: NULL table");
  if ((reinterpret_cast<uintptr_t>(table) & 7u) != 0)
    return fail(V41_EINVAL, "rope_table: table must be 8-byte aligned");
  if (n_pos > (int64_t)1 << 40) return fail(V41_EINVAL, "rope_table: n_pos too large");
  int rc = check_device();
  if (rc) return rc;
  return launched(v41::launch_rope_table(theta, rope_dim, n_pos, table, (hipStream_t)stream),
                  "rope_table");
}

namespace {

// Checks shared by the two rotation entry points.
int check_rope_rows(const char* who, const v41_bf16* in, int64_t in_ld, const v41_bf16* out,
                    int64_t out_ld, int32_t batch, int32_t n_tokens, int32_t rows_per_pos,
                    int32_t row_len, int32_t rope_dim, const float* table, int64_t table_rows,
                    const int32_t* pos, int64_t start_pos, int32_t row_quantum) {
  if (batch < 0 || n_tokens < 0) return fail(V41_EINVAL, "%s: negative batch/n_tokens", who);
  if (rows_per_pos < 1) return fail(V41_EINVAL, "%s: rows_per_pos < 1", who);
  if (row_len <= 0 || row_len % row_quantum != 0)
    return fail(V41_EINVAL, "%s: row_len %d is not a positive multiple of %d", who, row_len,
                row_quantum);
  if (rope_dim <= 0 || rope_dim % 8 != 0 || rope_dim > row_len)
    return fail(V41_EINVAL, "%s: rope_dim %d must be a positive multiple of 8, at most row_len",
                who, rope_dim);
  if (in_ld < row_len || in_ld % 8 != 0 || (out != nullptr && (out_ld < row_len ||
                                                               out_ld % 8 != 0)))
    return fail(V41_EINVAL, "%s: in_ld/out_ld must be >= row_len and multiples of 8", who);
  const int64_t rows = (int64_t)batch * n_tokens * rows_per_pos;
  if (rows * (row_len / 8) >= 0x7FFFFFFFLL)
    return fail(V41_EINVAL, "%s: rows * row_len / 8 must stay below 2^31", who);
  if (rows > 0 && (in == nullptr || table == nullptr))
    return fail(V41_EINVAL, "%s: NULL in or table", who);
  if (!aligned16(in) || !aligned16(out) || !aligned16(table) || !aligned16(pos))
    return fail(V41_EINVAL, "%s: pointers must be 16-byte aligned", who);
  if (table_rows < 1) return fail(V41_EINVAL, "%s: table_rows < 1", who);
  if (pos == nullptr && (start_pos < 0 || start_pos + n_tokens > table_rows))
    return fail(V41_EINVAL, "%s: positions %lld .. %lld outside the table's %lld rows", who,
                (long long)start_pos, (long long)(start_pos + n_tokens - 1),
                (long long)table_rows);
  if (in != nullptr && out != nullptr && in != out) {
    // distinct buffers must not overlap (in place means the same pointer)
    const char* a0 = reinterpret_cast<const char*>(in);
    const char* b0 = reinterpret_cast<const char*>(out);
    const int64_t span_in = ((rows - 1) * in_ld + row_len) * 2;
    const int64_t span_out = ((rows - 1) * out_ld + row_len) * 2;
    if (rows > 0 && a0 < b0 + span_out && b0 < a0 + span_in)
      return fail(V41_EINVAL, "%s: in and out overlap without being the same buffer", who);
  }
  if (in != nullptr && in == out && in_ld != out_ld)
    return fail(V41_EINVAL, "%s: in place needs in_ld == out_ld", who);
  return V41_OK;
}

}  // namespace

int v41_rope_rows(const v41_bf16* in, int64_t in_ld, v41_bf16* out, int64_t out_ld,
                  int32_t batch, int32_t n_tokens, int32_t rows_per_pos, int32_t row_len,
                  int32_t rope_dim, const float* table, int64_t table_rows, const int32_t* pos,
                  int64_t start_pos, int32_t inverse, v41_stream stream) {
  const int64_t rows = (int64_t)batch * n_tokens * rows_per_pos;
  if (rows > 0 && out == nullptr) return fail(V41_EINVAL, "rope_rows: NULL out");
  int rc = check_rope_rows("rope_rows", in, in_ld, out, out_ld, batch, n_tokens, rows_per_pos,
                           row_len, rope_dim, table, table_rows, pos, start_pos, 8);
  if (rc) return rc;
  rc = check_device();
  if (rc) return rc;
  v41::RopeRowsArgs a{in, in_ld, out, out_ld, batch, n_tokens, rows_per_pos, row_len,
                      rope_dim, table, table_rows, pos, start_pos, inverse != 0, false,
                      nullptr, 0, 0};
  return launched(v41::launch_rope_rows(a, (hipStream_t)stream), "rope_rows");
}

int v41_rope_fp8_rows(const v41_bf16* in, int64_t in_ld, v41_bf16* out, int64_t out_ld,
                      int32_t batch, int32_t n_tokens, int32_t row_len, int32_t rope_dim,
                      const float* table, int64_t table_rows, const int32_t* pos,
                      int64_t start_pos, v41_bf16* ring, int32_t ring_slots, int64_t ring_bs,
                      v41_stream stream) {
  const int64_t rows = (int64_t)batch * n_tokens;
  if (rows > 0 && out == nullptr && ring == nullptr)
    return fail(V41_EINVAL, "rope_fp8_rows: neither out nor ring given");
  int rc = check_rope_rows("rope_fp8_rows", in, in_ld, out, out_ld, batch, n_tokens, 1,
                           row_len, rope_dim, table, table_rows, pos, start_pos,
                           V41_FP8_BLOCK);
  if (rc) return rc;
  if (!aligned16(ring)) return fail(V41_EINVAL, "rope_fp8_rows: ring must be 16-byte aligned");
  if (ring != nullptr) {
    if (ring_slots <= 0) return fail(V41_EINVAL, "rope_fp8_rows: ring given with ring_slots <= 0");
    if (batch > 1 && ring_bs < (int64_t)ring_slots * row_len)
      return fail(V41_EINVAL, "rope_fp8_rows: ring_bs smaller than ring_slots * row_len");
    const char* r0 = reinterpret_cast<const char*>(ring);
    const char* i0 = reinterpret_cast<const char*>(in);
    const int64_t span_ring =
        ((batch > 1 ? (int64_t)(batch - 1) * ring_bs : 0) + (int64_t)ring_slots * row_len) * 2;
    const int64_t span_in = rows > 0 ? ((rows - 1) * in_ld + row_len) * 2 : 0;
    if (rows > 0 && i0 < r0 + span_ring && r0 < i0 + span_in)
      return fail(V41_EINVAL, "rope_fp8_rows: in overlaps the ring");
  }
  rc = check_device();
  if (rc) return rc;
  v41::RopeRowsArgs a{in, in_ld, out, out_ld, batch, n_tokens, 1, row_len, rope_dim,
                      table, table_rows, pos, start_pos, false, true, ring,
                      ring != nullptr ? ring_slots : 0, ring_bs};
  return launched(v41::launch_rope_rows(a, (hipStream_t)stream), "rope_fp8_rows");
}

int v41_candidate_blocks(const float* scores, int64_t n_sel_rows, int64_t n_cols,
                         int64_t scores_ld, int32_t cand_block, int32_t topk_blocks,
                         uint8_t* cand, int64_t cand_ld, v41_stream stream) {
  if (n_sel_rows < 0 || n_cols < 0) return fail(V41_EINVAL, "candidate_blocks: negative size");
  if (cand_block < 1) return fail(V41_EINVAL, "candidate_blocks: cand_block < 1");
  if (topk_blocks < 1) return fail(V41_EINVAL, "candidate_blocks: topk_blocks < 1");
  if (scores_ld < n_cols) return fail(V41_EINVAL, "candidate_blocks: scores_ld < n_cols");
  if (n_cols >= 0x7FFFFFFFLL) return fail(V41_EINVAL, "candidate_blocks: n_cols too large");
  const int64_t nb = (n_cols + cand_block - 1) / cand_block;
  if (nb > V41_MAX_CAND_BLOCKS)
    return fail(V41_EINVAL, "candidate_blocks: %lld blocks exceed %d", (long long)nb,
                V41_MAX_CAND_BLOCKS);
  if (cand_ld < nb) return fail(V41_EINVAL, "candidate_blocks: cand_ld < number of blocks");
  if (n_sel_rows > 0 && nb > 0 && (scores == nullptr || cand == nullptr))
    return fail(V41_EINVAL, "candidate_blocks: NULL scores/cand");
  int rc = check_device();
  if (rc) return rc;
  return launched(v41::launch_candidate_blocks(scores, n_sel_rows, n_cols, scores_ld,
                                               cand_block, topk_blocks, cand, cand_ld,
                                               (hipStream_t)stream),
                  "candidate_blocks");
}

namespace {

int check_linear(const char* who, const v41_bf16* a, int64_t lda, int64_t a_gs,
                 const v41_bf16* w, int64_t ldw, int64_t w_gs, const v41_bf16* y,
                 int64_t ldy, int64_t y_gs, int32_t M, int32_t N, int32_t K, int32_t groups,
                 const void* workspace, int64_t workspace_bytes) {
  if (M < 0 || N < 1 || groups < 1) return fail(V41_EINVAL, "%s: M < 0, N < 1 or groups < 1", who);
  if (K < 64 || K % 64 != 0) return fail(V41_EINVAL, "%s: K %d is not a positive multiple of 64",
                                         who, K);
  if (lda < K || ldw < K || ldy < N)
    return fail(V41_EINVAL, "%s: lda/ldw must be >= K and ldy >= N", who);
  if (lda % 8 != 0 || ldw % 8 != 0 || a_gs % 8 != 0 || w_gs % 8 != 0)
    return fail(V41_EINVAL, "%s: lda, ldw, a_gs and w_gs must be multiples of 8", who);
  if (groups > 1 && (a_gs < 0 || w_gs < (int64_t)N * ldw - (ldw - K) || y_gs < 0))
    return fail(V41_EINVAL, "%s: group strides out of range", who);
  if ((int64_t)groups * M * N >= ((int64_t)1 << 40))
    return fail(V41_EINVAL, "%s: output too large", who);
  if (M > 0 && (a == nullptr || w == nullptr || y == nullptr))
    return fail(V41_EINVAL, "%s: NULL a/w/y", who);
  if (!aligned16(a) || !aligned16(w) || !aligned16(workspace))
    return fail(V41_EINVAL, "%s: a, w and workspace must be 16-byte aligned", who);
  if (workspace_bytes < 0) return fail(V41_EINVAL, "%s: workspace_bytes < 0", who);
  return V41_OK;
}

}  // namespace

int64_t v41_linear_workspace_bytes(int32_t M, int32_t N, int32_t K, int32_t groups) {
  if (M <= 0 || N <= 0 || K <= 0 || groups <= 0) return 0;
  return v41::gemm_workspace_bytes(M, N, K, groups);
}

int v41_linear_bf16(const v41_bf16* a, int64_t lda, int64_t a_gs, const v41_bf16* w,
                    int64_t ldw, int64_t w_gs, v41_bf16* y, int64_t ldy, int64_t y_gs, int32_t M,
                    int32_t N, int32_t K, int32_t groups, void* workspace,
                    int64_t workspace_bytes, v41_stream stream) {
  int rc = check_linear("linear_bf16", a, lda, a_gs, w, ldw, w_gs, y, ldy, y_gs, M, N, K, groups,
                        workspace, workspace_bytes);
  if (rc) return rc;
  rc = check_device();
  if (rc) return rc;
  v41::LinearArgs la{a, lda, a_gs, w, ldw, w_gs, y, ldy, y_gs, M, N, K, groups, workspace,
                     workspace ? workspace_bytes : 0};
  return launched(v41::launch_linear_bf16(la, (hipStream_t)stream), "linear_bf16");
}

int64_t v41_grouped_output_workspace_bytes(int64_t n_tokens, int32_t n_heads, int32_t head_dim,
                                           int32_t groups, int32_t rank, int32_t dim) {
  if (n_tokens <= 0 || n_tokens > 0x7FFFFFFF || groups <= 0 || n_heads % groups != 0)
    return 0;
  const int32_t gw = n_heads / groups * head_dim;
  const int64_t w1 = v41::gemm_workspace_bytes((int32_t)n_tokens, rank, gw, groups);
  const int64_t w2 = v41::gemm_workspace_bytes((int32_t)n_tokens, dim, groups * rank, 1);
  return w1 > w2 ? w1 : w2;
}

int v41_grouped_output(v41_bf16* o, int64_t n_tokens, int32_t n_heads,
                       int32_t head_dim, int32_t groups, int32_t rank, int32_t dim,
                       const v41_bf16* wo_a, const v41_bf16* wo_b, v41_bf16* og, v41_bf16* x,
                       const float* rope_table, int64_t rope_rows, int32_t rope_dim,
                       const int32_t* pos, int64_t start_pos, void* workspace,
                       int64_t workspace_bytes, v41_stream stream) {
  const v41_bf16* o_bar = o;
  const char* who = "grouped_output";
  if (rope_table != nullptr && (int64_t)n_tokens * n_heads * (head_dim / 8) >= 0x7FFFFFFFLL)
    return fail(V41_EINVAL, "%s: too many rows to rotate", who);
  if (n_tokens < 0 || n_tokens > 0x7FFFFFFF) return fail(V41_EINVAL, "%s: n_tokens out of range", who);
  if (groups < 1 || n_heads < 1 || n_heads % groups != 0)
    return fail(V41_EINVAL, "%s: n_heads must be a positive multiple of groups", who);
  if (head_dim < 1 || rank < 1 || dim < 1)
    return fail(V41_EINVAL, "%s: head_dim, rank and dim must be positive", who);
  const int64_t gw = (int64_t)n_heads / groups * head_dim;
  const int64_t og_w = (int64_t)groups * rank;
  if (gw > 0x7FFFFFFF || og_w > 0x7FFFFFFF)
    return fail(V41_EINVAL, "%s: sizes out of range", who);
  const int32_t M = (int32_t)n_tokens;
  int rc = check_linear(who, o_bar, groups * gw, gw, wo_a, gw, (int64_t)rank * gw, og, og_w, rank,
                        M, rank, (int32_t)gw, groups, workspace, workspace_bytes);
  if (rc) return rc;
  rc = check_linear(who, og, og_w, 0, wo_b, og_w, 0, x, dim, 0, M, dim, (int32_t)og_w, 1,
                    workspace, workspace_bytes);
  if (rc) return rc;
  if (!aligned16(og)) return fail(V41_EINVAL, "%s: og must be 16-byte aligned", who);
  if (rope_table != nullptr) {
    if (rope_dim <= 0 || rope_dim % 8 != 0 || rope_dim > head_dim || head_dim % 8 != 0)
      return fail(V41_EINVAL, "%s: rope_dim must be a positive multiple of 8 within head_dim",
                  who);
    if (rope_rows < 1) return fail(V41_EINVAL, "%s: rope_rows < 1", who);
    if (!aligned16(rope_table) || !aligned16(pos))
      return fail(V41_EINVAL, "%s: rope_table and pos must be 16-byte aligned", who);
    if (pos == nullptr && (start_pos < 0 || start_pos + n_tokens > rope_rows))
      return fail(V41_EINVAL, "%s: positions outside the rope table", who);
  }
  rc = check_device();
  if (rc) return rc;
  hipStream_t s = (hipStream_t)stream;
  const int64_t wb = workspace ? workspace_bytes : 0;
  // o^g_{t, g} = O_bar_{t, heads of g} . W_OA,g^T (block diagonal over groups)
  if (rope_table != nullptr && M > 0) {
    // O_bar_{h,t,tail} = R_t^-1 O_{h,t,tail}, in place on o's rotated tails:
    // token t is sequence t at pos[t] (decode) or start_pos + t (a chunk)
    v41::RopeRowsArgs r{o, head_dim, o, head_dim, pos != nullptr ? M : 1,
                        pos != nullptr ? 1 : M, n_heads, head_dim, rope_dim, rope_table,
                        rope_rows, pos, start_pos, true, false, nullptr, 0, 0};
    rc = launched(v41::launch_rope_rows(r, s), "grouped_output inverse rotation");
    if (rc) return rc;
  }
  v41::LinearArgs l1{o_bar, groups * gw, gw, wo_a, gw, (int64_t)rank * gw, og, og_w, rank, M,
                     rank, (int32_t)gw, groups, workspace, wb};
  rc = launched(v41::launch_linear_bf16(l1, s), "grouped_output wo_a");
  if (rc) return rc;
  // Delta_t = o^g_t . W_OB^T
  v41::LinearArgs l2{og, og_w, 0, wo_b, og_w, 0, x, dim, 0, M, dim, (int32_t)og_w, 1, workspace,
                     wb};
  return launched(v41::launch_linear_bf16(l2, s), "grouped_output wo_b");
}

int v41_probe_hbm_read(const void* buf, int64_t bytes, int32_t nontemporal, uint32_t* sink,
                       v41_stream stream) {
  if (bytes < 0 || bytes % 16 != 0)
    return fail(V41_EINVAL, "probe_hbm_read: bytes must be a non-negative multiple of 16");
  if (bytes > 0 && (buf == nullptr || sink == nullptr))
    return fail(V41_EINVAL, "probe_hbm_read: NULL buf/sink");
  if (!aligned16(buf)) return fail(V41_EINVAL, "probe_hbm_read: buf must be 16-byte aligned");
  int rc = check_device();
  if (rc) return rc;
  if (bytes == 0) return V41_OK;
  return launched(v41::launch_probe_hbm_read(buf, bytes, nontemporal, sink, (hipStream_t)stream),
                  "probe_hbm_read");
}

int v41_probe_mfma(int32_t workgroups, int32_t iters, float* sink, v41_stream stream) {
  if (workgroups < 1 || iters < 1 || sink == nullptr)
    return fail(V41_EINVAL, "probe_mfma: workgroups and iters must be >= 1, sink non-NULL");
  int rc = check_device();
  if (rc) return rc;
  return launched(v41::launch_probe_mfma(workgroups, iters, sink, (hipStream_t)stream),
                  "probe_mfma");
}

int v41_decode_step(const v41_decode_step_args* a, v41_stream stream) {
  const char* who = "decode_step";
  if (a == nullptr) return fail(V41_EINVAL, "%s: NULL args", who);
  if (a->batch < 0) return fail(V41_EINVAL, "%s: batch < 0", who);
  if (a->n_heads < 1) return fail(V41_EINVAL, "%s: n_heads < 1", who);
  const int32_t D = a->head_dim;
  if (D != 64 && D != 128 && D != 256 && D != 512)
    return fail(V41_EINVAL, "%s: head_dim %d not in {64, 128, 256, 512}", who, D);
  if (a->window < 1) return fail(V41_EINVAL, "%s: window < 1", who);
  if (a->ratio < 0) return fail(V41_EINVAL, "%s: ratio < 0", who);
  const bool compressed = a->ratio >= 1;
  const int32_t topk = compressed ? a->topk : 0;
  if (compressed) {
    if (a->topk < 1) return fail(V41_EINVAL, "%s: topk < 1", who);
    if (a->index_heads < 1 || a->index_heads > V41_MAX_INDEX_HEADS)
      return fail(V41_EINVAL, "%s: index_heads %d outside 1..%d", who, a->index_heads,
                  V41_MAX_INDEX_HEADS);
    if (a->index_dim != 32 && a->index_dim != 64 && a->index_dim != 128)
      return fail(V41_EINVAL, "%s: index_dim %d not in {32, 64, 128}", who, a->index_dim);
    if (a->n_rows < 0 || a->n_rows >= 0x7FFFFFFFLL - a->window)
      return fail(V41_EINVAL, "%s: n_rows out of range", who);
  }
  const int64_t width = (int64_t)a->window + topk;
  if (width > V41_MAX_WIDTH)
    return fail(V41_EINVAL, "%s: window + topk = %lld exceeds the selection limit %d", who,
                (long long)width, V41_MAX_WIDTH);
  if (a->rope_dim < 0 || a->rope_dim % 8 != 0 || a->rope_dim > D)
    return fail(V41_EINVAL, "%s: rope_dim %d must be a multiple of 8 in 0..head_dim", who,
                a->rope_dim);
  if ((a->rope_dim > 0) != (a->rope_table != nullptr))
    return fail(V41_EINVAL, "%s: rope_table must be given exactly when rope_dim > 0", who);
  if (a->rope_dim > 0 && a->rope_rows < 1)
    return fail(V41_EINVAL, "%s: rope_rows < 1", who);
  if (a->batch > 1 && a->ring_bs < (int64_t)a->window * D)
    return fail(V41_EINVAL, "%s: ring_bs < window * head_dim", who);
  if (compressed && a->batch > 1 && a->n_rows > 0 &&
      (a->latent_bs < a->n_rows * D || a->kI_bs < a->n_rows * a->index_dim))
    return fail(V41_EINVAL, "%s: latent_bs/kI_bs smaller than one sequence's rows", who);
  if (a->ring_bs % 8 != 0 || a->latent_bs % 8 != 0 || a->kI_bs % 8 != 0)
    return fail(V41_EINVAL, "%s: ring_bs/latent_bs/kI_bs must be multiples of 8", who);
  if ((int64_t)a->batch * a->n_heads * (D / 8) >= 0x7FFFFFFFLL)
    return fail(V41_EINVAL, "%s: batch too large", who);
  if (a->batch > 0) {
    if (a->pos == nullptr || a->q == nullptr || a->kv_new == nullptr || a->ring == nullptr ||
        a->sink == nullptr || a->idx == nullptr || a->out == nullptr)
      return fail(V41_EINVAL, "%s: NULL pos/q/kv_new/ring/sink/idx/out", who);
    if (compressed && a->n_rows > 0 &&
        (a->latent == nullptr || a->kI == nullptr || a->qI == nullptr || a->w == nullptr ||
         a->scores == nullptr))
      return fail(V41_EINVAL, "%s: NULL latent/kI/qI/w/scores (no latent cache published)", who);
  }
  if (!aligned16(a->pos) || !aligned16(a->q) || !aligned16(a->kv_new) ||
      !aligned16(a->ring) || !aligned16(a->latent) || !aligned16(a->kI) ||
      !aligned16(a->qI) || !aligned16(a->rope_table) || !aligned16(a->out) ||
      !aligned16(a->workspace))
    return fail(V41_EINVAL, "%s: pointers must be 16-byte aligned", who);
  if (a->workspace_bytes < 0) return fail(V41_EINVAL, "%s: workspace_bytes < 0", who);
  int rc = check_device();
  if (rc) return rc;
  if (a->batch == 0) {
    g_err[0] = '\0';
    return V41_OK;
  }
  hipStream_t s = (hipStream_t)stream;
  v41::DecodeFrontArgs f;
  f.q = a->q;
  f.kv = a->kv_new;
  f.ring = a->ring;
  f.ring_bs = a->ring_bs;
  f.idx = a->idx;
  f.idx_ld = width;
  f.pos = a->pos;
  f.table = a->rope_table;
  f.table_rows = a->rope_rows;
  f.batch = a->batch;
  f.n_heads = a->n_heads;
  f.row_len = D;
  f.window = a->window;
  f.rope_dim = a->rope_dim;
  const int64_t n_rows = compressed ? a->n_rows : 0;
  if (compressed) {
    // the indexer scores with the front work as extra workgroups of the same
    // launch (the two touch disjoint buffers); start_pos 1 only marks the
    // decode form, the positions come from pos
    rc = launched(v41::launch_indexer_scores_front(a->qI, a->kI, a->kI_bs, a->w, nullptr, 0, 1,
                                                   a->batch, 1, 1, a->pos, a->ratio,
                                                   a->index_heads, a->index_dim, n_rows,
                                                   a->scores, n_rows, &f, s),
                  "decode_step front + indexer");
    if (rc) return rc;
    // with no compressed rows the top-k reads nothing and writes k absent entries
    rc = launched(v41::launch_topk_select(a->scores, a->batch, n_rows, n_rows, topk, a->window,
                                          a->idx + a->window, width, s),
                  "decode_step top-k");
    if (rc) return rc;
  } else {
    rc = launched(v41::launch_decode_front(f, s), "decode_step front");
    if (rc) return rc;
  }
  v41::AttnArgs t;
  t.q = a->q;
  t.rows_a = a->ring;
  t.rows_a_len = a->window;
  t.a_bs = a->ring_bs;
  t.rows_b = compressed && n_rows > 0 ? a->latent : nullptr;
  t.rows_b_len = compressed ? n_rows : 0;
  t.b_bs = a->latent_bs;
  t.idx = a->idx;
  t.width = (int32_t)width;
  t.idx_ld = width;
  t.sink = a->sink;
  t.scale = a->scale;
  t.batch = a->batch;
  t.n_tokens = 1;
  t.n_heads = a->n_heads;
  t.head_dim = D;
  t.out = a->out;
  t.workspace = a->workspace;
  t.workspace_bytes = a->workspace ? a->workspace_bytes : 0;
  return launched(v41::launch_sparse_attn_sink(t, s), "decode_step attention");
}

}  // extern "C"
