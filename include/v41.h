/*
 * v41.h -- C ABI of the MI355X (gfx950) hot path of DeepSeek-V4.1 compressed
 * sparse attention: fp8 round trip of kv rows, window selection, indexer
 * score, index top-k, and sparse attention with a per-head sink; the rotary
 * embedding (table, rotation of queries and output, and the window-key
 * epilogue rotation + fp8 + ring write) around it.
 *
 * Conventions shared by every call
 *  - bf16 values travel as raw uint16 bit patterns (v41_bf16).
 *  - Every data pointer is a device pointer owned by the caller; the library
 *    keeps no state between calls.  Only the calls with a `workspace`
 *    argument use scratch memory, and only the caller's; the one exception
 *    is v41_sparse_attn_sink_noalloc, which uses a static device array of
 *    the library.
 *  - Calls are asynchronous on `stream` (a hipStream_t; NULL is the null
 *    stream) and never synchronise the host.
 *  - Strides ("_ld" between rows, "_bs" between sequences) count elements,
 *    not bytes.
 *  - Return value: 0 on success; V41_EINVAL (-1) for an invalid argument,
 *    V41_EHIP (-2) for a HIP runtime or launch error, V41_EDEVICE (-3) when
 *    the current device is not a gfx950.  v41_last_error() then returns a
 *    message (thread-local, valid until the next call on the thread).
 *  - Index values that the host cannot see (idx contents) are not checked:
 *    an entry outside [0, rows_a_len + rows_b_len) is skipped like -1.
 *
 * Sources: the "deepseek_v41_ref::attn" rustdoc (function contracts
 * act_quant_inplace, pow2_ceil, window_topk_idxs, sparse_attn, the precision
 * paragraph and the ring-cache example); the "Compressed sparse attention"
 * layer page, section "All 25 steps" (FP8(W), S^I, I_t, J^w_t, the join
 * Y/J/G_t, the sink softmax A and O); the "attn_v41.rs" source page (module
 * invariants, SharedV41 and AttnV41Run).
 */
#ifndef V41_H
#define V41_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef uint16_t v41_bf16;
typedef void *v41_stream;

#define V41_OK 0
#define V41_EINVAL (-1)
#define V41_EHIP (-2)
#define V41_EDEVICE (-3)

/* Values per fp8 scale block (the rustdoc's FP8_BLOCK). */
#define V41_FP8_BLOCK 32
/* Widest selection sparse attention accepts (window + top-k), as in the
 * attn_v41.rs module invariant on the sparse_attn score buffer. */
#define V41_MAX_WIDTH 2048
/* Largest indexer head count one call takes. */
#define V41_MAX_INDEX_HEADS 64
/* Most candidate blocks per score row one v41_candidate_blocks call takes. */
#define V41_MAX_CAND_BLOCKS 32768

/* Message for the last non-zero status on this thread ("" if none). */
const char *v41_last_error(void);

/* ABI revision of this header. */
int v41_abi_version(void);

/*
 * fp8 round trip of kv rows ("deepseek_v41_ref::attn": act_quant_inplace and
 * pow2_ceil; "Compressed sparse attention", All 25 steps: W <- FP8(W)).
 *
 * For every row and every block of 32 consecutive values: amax = max |x|,
 * floored at 1e-4; s = 2^ceil(log2(amax / 448)) (binary32 division, exponent
 * from the IEEE fields); each x goes to x / s, clamped to +-448, rounded to
 * the nearest OCP E4M3FN value (ties to even, subnormals kept, sign of zero
 * kept), multiplied by s and stored as bf16.  The stored value is exact
 * (e4m3 times a power of two) except when it reaches 2^128, which rounds to
 * +-inf in bf16.
 *
 *   in       [rows][in_ld] bf16; the first row_len values of each row are read
 *   out      [rows][out_ld] bf16; may equal `in` (same ld) for in place.
 *            Pointing `out` at a ring slot with out_ld = one sequence's ring
 *            stride writes a batch of decode rows into their slots.
 *   row_len  multiple of 32, > 0; in_ld, out_ld >= row_len, multiples of 8
 *   ring     optional (NULL = none) window ring [ring_slots][row_len]: row r
 *            is token first_pos + r, and each of the last
 *            min(rows, ring_slots) rows is also written to ring slot
 *            (first_pos + r) mod ring_slots (the prefill's ring seeding).
 *   in, out, ring: 16-byte aligned.
 */
int v41_fp8_round_rows(const v41_bf16 *in, int64_t in_ld, v41_bf16 *out,
                       int64_t out_ld, int64_t rows, int32_t row_len,
                       v41_bf16 *ring, int32_t ring_slots, int64_t first_pos,
                       v41_stream stream);

/*
 * Window selection ("deepseek_v41_ref::attn": window_topk_idxs; "Compressed
 * sparse attention", All 25 steps: J^w_t = {max(0, t-127) .. t}).
 *
 *   start_pos == 0: cols = min(n_tokens, window); token t gets chunk rows
 *     max(0, t - window + 1) .. t ascending, then -1 up to cols.
 *   start_pos > 0: n_tokens must be 1; cols = window; the whole ring oldest
 *     first: slot (start_pos + 1 + c) mod window once start_pos >= window - 1,
 *     else slots 0 .. start_pos then -1.
 *   idx       int32 [batch][n_tokens][idx_ld] at idx + b*idx_bs + t*idx_ld
 *             (the first cols entries are written; the same for every b)
 *   cols_out  host pointer (nullable): receives cols.
 */
int v41_window_idx(int64_t start_pos, int32_t n_tokens, int32_t window,
                   int32_t batch, int32_t *idx, int64_t idx_ld, int64_t idx_bs,
                   int32_t *cols_out, v41_stream stream);

/*
 * Indexer score ("Compressed sparse attention", All 25 steps:
 * S^I_{t,j} = sum_h w^I_{t,h} ReLU(Q^I_{h,t} . K^I_j), visible for
 * j < floor((t+1)/ratio) and where the candidate mask M^c allows).
 *
 * Query q = b * n_tokens + t is the token at position start_pos + t of
 * sequence b; it sees n(q) = min(n_rows, floor((start_pos + t + 1) / ratio))
 * compressed positions, further limited by cand[q][j / cand_block] != 0 when
 * cand is given.  Every other column of its score row is -inf.
 *
 *   qI      bf16 [batch * n_tokens][n_heads][head_dim]
 *   kI      bf16 [batch] x [n_rows][head_dim] at kI + b*kI_bs (one key per
 *           compressed position, shared by all heads)
 *   w       f32 [batch * n_tokens][n_heads] (the 1/sqrt scaling already in)
 *   cand    u8 [batch * n_tokens][cand_width] or NULL; cand_block > 0
 *   scores  f32 [batch * n_tokens][scores_ld], scores_ld >= n_rows
 *   n_heads 1 .. 64; head_dim 32, 64 or 128; ratio >= 1; n_rows >= 0.
 * Products are bf16 x bf16 exact, accumulated in f32 on the matrix cores;
 * ReLU, the weights and the head sum in f32.
 */
int v41_indexer_scores(const v41_bf16 *qI, const v41_bf16 *kI, int64_t kI_bs,
                       const float *w, const uint8_t *cand, int32_t cand_width,
                       int32_t cand_block, int32_t batch, int32_t n_tokens,
                       int64_t start_pos, int32_t ratio, int32_t n_heads,
                       int32_t head_dim, int64_t n_rows, float *scores,
                       int64_t scores_ld, v41_stream stream);

/*
 * Index top-k ("Compressed sparse attention", All 25 steps: I_t = top_k of
 * S^I over the visible positions; "attn_v41.rs": the selection is offset past
 * the window rows and -1 marks an absent entry).
 *
 * Per score row: valid positions are those whose score is neither -inf nor
 * NaN.  The m = min(k, #valid) best (ranked by score descending; equal
 * scores, with +0 equal to -0, go to the lower position) form the selection,
 * a set, written as position + offset in ascending position order and
 * followed by -1 up to k entries.
 *
 *   scores  f32 [n_sel_rows][scores_ld], n_cols <= scores_ld
 *   idx     int32 [n_sel_rows][idx_ld]; entries 0 .. k-1 of each row are
 *           written (point it at the first compressed column of the joint
 *           index buffer)
 *   k       1 .. 2048
 */
int v41_topk_select(const float *scores, int64_t n_sel_rows, int64_t n_cols,
                    int64_t scores_ld, int32_t k, int32_t offset, int32_t *idx,
                    int64_t idx_ld, v41_stream stream);

/*
 * Candidate-block selection: the block-level candidate mask that the
 * candidate-source layer publishes and later index sources apply ("attn_v41"
 * module page: the candidate-block top-k selection; "attn_v41.rs":
 * SharedV41.candidates [queries][cand_width]; config candidate_block_size 8,
 * candidate_topk_blocks 2048).  The result is the `cand` input of
 * v41_indexer_scores.
 *
 * Per score row: block b covers positions [b * cand_block, (b + 1) *
 * cand_block); its score is the largest score of those positions that is
 * neither -inf nor NaN (the pages do not state the block score: this is the
 * reading taken).  The topk_blocks best blocks (score descending, equal
 * scores, +0 equal to -0, to the lower block; blocks with no valid score are
 * never chosen) get cand = 1, every other block 0.
 *
 *   scores  f32 [n_sel_rows][scores_ld], n_cols <= scores_ld
 *   cand    u8 [n_sel_rows][cand_ld]; the first ceil(n_cols / cand_block)
 *           bytes of each row are written, at most V41_MAX_CAND_BLOCKS
 *   cand_block, topk_blocks >= 1
 */
int v41_candidate_blocks(const float *scores, int64_t n_sel_rows, int64_t n_cols,
                         int64_t scores_ld, int32_t cand_block, int32_t topk_blocks,
                         uint8_t *cand, int64_t cand_ld, v41_stream stream);

/*
 * Sparse attention with the sink ("Compressed sparse attention", All 25
 * steps: G_t = Y[J_t], S = Q . G / sqrt(d), A = exp S / (exp s_h +
 * sum exp S), O = sum A G; "deepseek_v41_ref::attn": sparse_attn, f32 softmax,
 * -1 skipped, bf16 out; "attn_v41.rs": AttnV41Run).
 *
 * For query q = b * n_tokens + t and head h: the valid entries i of
 * idx[q][0 .. width) select row g_i = rows_a[b][ix] when ix < rows_a_len and
 * rows_b[b][ix - rows_a_len] otherwise; s_i = scale * (q_h . g_i);
 * o_h = sum_i exp(s_i) g_i / (exp(sink_h) + sum_i exp(s_i)).  One latent row
 * is both key and value.  A query with no valid entry gets o = 0.
 *
 *   q       bf16 [batch * n_tokens][n_heads][head_dim] (after RoPE)
 *   rows_a  bf16 [batch] x [rows_a_len][head_dim] at rows_a + b*a_bs (window
 *           rows: the chunk's own fp8-rounded rows at a prefill, the ring at
 *           a decode)
 *   rows_b  bf16 [batch] x [rows_b_len][head_dim] at rows_b + b*b_bs (the
 *           compressed latent rows); may be NULL only if rows_b_len == 0
 *   idx     int32 [batch * n_tokens][idx_ld], width <= min(idx_ld, 2048)
 *   sink    f32 [n_heads]; scale: f32 (1/sqrt(head_dim) in the method)
 *   out     bf16 [batch * n_tokens][n_heads][head_dim]
 *   head_dim 64, 128, 256 or 512; n_heads >= 1.
 *   workspace / workspace_bytes: optional device scratch (NULL / 0 allowed).
 *           With at least v41_sparse_attn_workspace_bytes(...) bytes the
 *           call may split one query's rows over several workgroups; with
 *           less it does not split.  The result is the same either way up to
 *           f32 rounding order.  Calls that share a workspace must not
 *           overlap in time.
 * QK^T and PV run as bf16 products with f32 accumulation; the softmax is in
 * f32; the probabilities enter PV as a pair of bf16 terms (high part plus
 * remainder), about 16 significant bits.
 */
int v41_sparse_attn_sink(const v41_bf16 *q, const v41_bf16 *rows_a,
                         int64_t rows_a_len, int64_t a_bs,
                         const v41_bf16 *rows_b, int64_t rows_b_len,
                         int64_t b_bs, const int32_t *idx, int32_t width,
                         int64_t idx_ld, const float *sink, float scale,
                         int32_t batch, int32_t n_tokens, int32_t n_heads,
                         int32_t head_dim, v41_bf16 *out, void *workspace,
                         int64_t workspace_bytes, v41_stream stream);

/* Workspace size that lets v41_sparse_attn_sink split rows as it prefers
 * for this shape (0 when it would not split). */
int64_t v41_sparse_attn_workspace_bytes(int32_t batch, int32_t n_tokens,
                                        int32_t n_heads, int32_t head_dim,
                                        int32_t width);

/* Bytes of the library's own device scratch array behind
 * v41_sparse_attn_sink_noalloc (per GPU, held until the process ends). */
#define V41_NOALLOC_SCRATCH_BYTES (32LL << 20)

/*
 * v41_sparse_attn_sink for callers that cannot allocate device memory: code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  Same arguments, meaning and result as v41_sparse_attn_sink
 * with a workspace of v41_sparse_attn_workspace_bytes(...) bytes, except that
 * the row-split partials go to a static device array of the library
 * (V41_NOALLOC_SCRATCH_BYTES per GPU) instead of a caller's workspace.
 *
 *  - Calls no hipMalloc/hipFree and no allocating library routine.  The
 *    first call on a device looks up that device's copy of the array
 *    (hipGetSymbolAddress), with that device current.
 *  - Returns V41_EINVAL, with a message, when the shape needs more than
 *    V41_NOALLOC_SCRATCH_BYTES of scratch (v41_sparse_attn_workspace_bytes
 *    tells how much it needs).
 *  - Every call on one GPU shares that GPU's array, which keeps the last
 *    call's partials: calls that overlap in time on one GPU (two streams,
 *    two host threads) race and give undefined results.  Serialise them.
 */
int v41_sparse_attn_sink_noalloc(const v41_bf16 *q, const v41_bf16 *rows_a,
                                 int64_t rows_a_len, int64_t a_bs,
                                 const v41_bf16 *rows_b, int64_t rows_b_len,
                                 int64_t b_bs, const int32_t *idx,
                                 int32_t width, int64_t idx_ld,
                                 const float *sink, float scale, int32_t batch,
                                 int32_t n_tokens, int32_t n_heads,
                                 int32_t head_dim, v41_bf16 *out,
                                 v41_stream stream);

/*
 * RoPE table at ratio 0 ("deepseek_v41_ref::attn": freqs_cis, the table
 * without YaRN, [seqlen][dim/2] pairs (cos, sin); rope_theta 10000 in the
 * config of the "Compressed sparse attention" layer page).
 *
 * table[p][i] = (cos a, sin a) with a = p * theta^(-2i / rope_dim) (the usual
 * rotary frequency ladder: the pages give the table's shape, not its
 * formula), computed in binary64 and rounded once to binary32.  Entries are
 * within one binary32 ulp plus 2^-32 of the real values.
 *
 *   table    f32 [n_pos][rope_dim / 2][2], 8-byte aligned
 *   rope_dim positive and even; theta > 0.
 */
int v41_rope_table(double theta, int32_t rope_dim, int64_t n_pos, float *table,
                   v41_stream stream);

/*
 * Rotation of the last rope_dim values of rows ("deepseek_v41_ref::attn":
 * apply_rotary; "Compressed sparse attention", All 25 steps:
 * Q_{...,448:} <- R_t Q on the queries and O_{h,t,448:} <- R_t^-1 O on the
 * attention output).
 *
 * Row r (of batch * n_tokens * rows_per_pos) belongs to sequence
 * b = r / (n_tokens * rows_per_pos) and token t = (r / rows_per_pos) mod
 * n_tokens, at position p = (pos ? pos[b] : start_pos) + t.  The rotated part
 * is read as rope_dim / 2 complex numbers, value 2i the real and 2i+1 the
 * imaginary part of number i, each multiplied by table[p][i] = c + i s
 * (by c - i s when inverse != 0): re = x0*c - x1*s and im = x0*s + x1*c with
 * every product and sum rounded to binary32 (no fused multiply-add), then
 * rounded to bf16.  Values before the rotated part are copied.
 *
 *   in, out  bf16 [rows][in_ld], [rows][out_ld]; out == in (same ld) rotates
 *            in place and then touches only the rotated part; otherwise the
 *            two must not overlap.  For queries [B*T][H][D]: rows_per_pos = H,
 *            row_len = in_ld = D.
 *   row_len  multiple of 8; rope_dim a multiple of 8, <= row_len
 *   table    f32 [table_rows][rope_dim / 2][2] (v41_rope_table's layout)
 *   pos      device int32 [batch] or NULL; with NULL, start_pos .. start_pos +
 *            n_tokens - 1 must lie in the table.  A row whose position falls
 *            outside [0, table_rows) (only possible through pos) is not
 *            written.
 *   in, out, table, pos: 16-byte aligned.
 */
int v41_rope_rows(const v41_bf16 *in, int64_t in_ld, v41_bf16 *out, int64_t out_ld,
                  int32_t batch, int32_t n_tokens, int32_t rows_per_pos, int32_t row_len,
                  int32_t rope_dim, const float *table, int64_t table_rows,
                  const int32_t *pos, int64_t start_pos, int32_t inverse,
                  v41_stream stream);

/*
 * The window-key epilogue in one pass: the rotation of v41_rope_rows on the
 * last rope_dim values (bf16 result), then the fp8 round trip of
 * v41_fp8_round_rows on the whole row, then the ring write ("Compressed
 * sparse attention", All 25 steps: W_{t,448:} <- R_t w^n_{t,448:}, then
 * W <- FP8(W); "deepseek_v41_ref::attn": the attention forward writes the new
 * kv rows into the cache's ring; "attn_v41.rs": the captured decode step's
 * ring_put takes the slot pos[0] mod window on the device).
 *
 * Row r = b * n_tokens + t is token t of sequence b at position
 * p = (pos ? pos[b] : start_pos) + t (one row per position: rows_per_pos 1).
 *
 *   out      bf16 [batch * n_tokens][out_ld] or NULL (ring only, as at a
 *            decode where the ring is the only home of the new row)
 *   ring     bf16 ring of sequence b at ring + b * ring_bs, [ring_slots]
 *            [row_len], or NULL; each of the last min(n_tokens, ring_slots)
 *            tokens of a sequence is also written to slot p mod ring_slots.
 *            The ring must not overlap in.
 *   row_len  multiple of 32 (the fp8 block); other arguments as for
 *            v41_rope_rows.  At least one of out and ring is given.
 */
int v41_rope_fp8_rows(const v41_bf16 *in, int64_t in_ld, v41_bf16 *out, int64_t out_ld,
                      int32_t batch, int32_t n_tokens, int32_t row_len, int32_t rope_dim,
                      const float *table, int64_t table_rows, const int32_t *pos,
                      int64_t start_pos, v41_bf16 *ring, int32_t ring_slots,
                      int64_t ring_bs, v41_stream stream);

/*
 * One bf16 projection on the matrix cores ("deepseek_v41_ref::attn"
 * precision paragraph: every projection is linear_bf16, f32 accumulation and
 * a bf16 result; weights are [out, in]):
 *   y_g[m][n] = sum_k a_g[m][k] * w_g[n][k]   for g < groups,
 * with a_g = a + g * a_gs, w_g = w + g * w_gs, y_g = y + g * y_gs (element
 * offsets).  groups > 1 is a block-diagonal projection such as wo_a (each
 * group of heads with its own block); groups == 1 a plain one such as wo_b.
 *
 *   a   bf16 rows of K values, row stride lda (>= K, multiple of 8)
 *   w   bf16 rows of K values, row stride ldw (>= K, multiple of 8)
 *   y   bf16 [M][ldy] per group (ldy >= N)
 *   K   a positive multiple of 64; M >= 0; N >= 1.
 *   workspace / workspace_bytes: optional device scratch; with at least
 *       v41_linear_workspace_bytes(...) bytes, a call with few rows (M <= 64)
 *       splits K over workgroups (f32 partial sums added in a fixed order).
 *       The result is the same up to f32 rounding order either way.  Calls
 *       sharing a workspace must not overlap in time.
 *   a, w, workspace: 16-byte aligned; a_gs and w_gs multiples of 8.
 */
int v41_linear_bf16(const v41_bf16 *a, int64_t lda, int64_t a_gs, const v41_bf16 *w,
                    int64_t ldw, int64_t w_gs, v41_bf16 *y, int64_t ldy, int64_t y_gs,
                    int32_t M, int32_t N, int32_t K, int32_t groups, void *workspace,
                    int64_t workspace_bytes, v41_stream stream);

/* Workspace size that lets v41_linear_bf16 split K as it prefers (0 when it
 * would not split). */
int64_t v41_linear_workspace_bytes(int32_t M, int32_t N, int32_t K, int32_t groups);

/*
 * The grouped output projection after the attention ("Compressed sparse
 * attention", All 25 steps, "Grouped output": o^g_{t,r} = [O_bar_{h,t}]_{h in r}
 * W_{OA,r}, then Delta = o^g W_{OB}; "attn_v41.rs": wo_a [groups * o_rank,
 * gw], wo_b [dim, groups * o_rank]).  Two v41_linear_bf16 launches: the
 * block-diagonal wo_a over the groups of contiguous heads, then wo_b over the
 * bf16 o^g.  O_bar is the attention output after the inverse rotation
 * (CSA: O_bar_{h,t,448:} = R_t^-1 O_{h,t,448:}): with rope_table given, o is
 * the attention output before it, and its rotated tails are first rotated
 * back in place (v41_rope_rows with inverse = 1), as the model code does to o;
 * with rope_table NULL, o is O_bar already and is only read.
 *
 *   o      bf16 [n_tokens][n_heads][head_dim]; gw = n_heads / groups * head_dim
 *   rope_table, rope_rows, rope_dim: the RoPE table (v41_rope_table's layout)
 *          and the rotated tail of each head (a multiple of 8), or NULL
 *   pos    device int32 [n_tokens] (token t is a sequence's token at pos[t],
 *          as at a decode), or NULL: token t at start_pos + t (a chunk; the
 *          positions must lie in the table); a token whose device position is
 *          outside the table keeps its tails unrotated
 *   wo_a   bf16 [groups * rank][gw]; wo_b bf16 [dim][groups * rank]
 *   og     bf16 [n_tokens][groups * rank] (written; the input of wo_b)
 *   x      bf16 [n_tokens][dim]
 *   n_heads a multiple of groups; gw and groups * rank multiples of 64.
 *   workspace: at least v41_grouped_output_workspace_bytes(...) bytes to
 *       split K at decode sizes (optional).
 */
int v41_grouped_output(v41_bf16 *o, int64_t n_tokens, int32_t n_heads,
                       int32_t head_dim, int32_t groups, int32_t rank, int32_t dim,
                       const v41_bf16 *wo_a, const v41_bf16 *wo_b, v41_bf16 *og, v41_bf16 *x,
                       const float *rope_table, int64_t rope_rows, int32_t rope_dim,
                       const int32_t *pos, int64_t start_pos, void *workspace,
                       int64_t workspace_bytes, v41_stream stream);

int64_t v41_grouped_output_workspace_bytes(int64_t n_tokens, int32_t n_heads,
                                           int32_t head_dim, int32_t groups, int32_t rank,
                                           int32_t dim);

/*
 * One whole decode step in one call, with every position read on the device,
 * so that a HIP graph captured once replays it at every later step (the
 * captured decode step of "attn_v41.rs": the graph's ring_put reads pos[0]
 * mod window on the device, and the per-step index buffers are rebuilt on the
 * device instead of being uploaded).  The step is the same computation as the
 * separate calls, in fewer launches:
 *   1. the front work: when rope_dim > 0, the q tails rotated in place
 *      (v41_rope_rows) and the new kv rows rotated; the kv rows through the
 *      fp8 round trip into ring slot pos[b] mod window (v41_fp8_round_rows /
 *      v41_rope_fp8_rows); the window indices of the whole ring, oldest first
 *      (v41_window_idx at a decode);
 *   2. when ratio >= 1: the indexer scores with n(b) =
 *      min(n_rows, floor((pos[b] + 1) / ratio)) (v41_indexer_scores), in the
 *      same launch as the front work; then the top-k written after the window
 *      columns, offset by window (v41_topk_select);
 *   3. the sparse attention with the sink over [ring ; latent rows]
 *      (v41_sparse_attn_sink).
 * Sequences may sit at different positions.  A sequence whose pos[b] is
 * negative, or (with rope) not below rope_rows, writes no ring row and has an
 * empty window; its q is not rotated.
 *
 * Buffers (device, 16-byte aligned; contiguous unless a stride is given):
 *   pos      int32 [batch]
 *   q        bf16 [batch][n_heads][head_dim] (before the rotation when
 *            rope_dim > 0; rotated in place)
 *   kv_new   bf16 [batch][head_dim]
 *   ring     bf16 [batch] x [window][head_dim] at ring + b * ring_bs
 *   latent   bf16 [batch] x [n_rows][head_dim] at latent + b * latent_bs
 *   kI       bf16 [batch] x [n_rows][index_dim] at kI + b * kI_bs
 *   qI, w    bf16 [batch][index_heads][index_dim], f32 [batch][index_heads]
 *   rope_table f32 [rope_rows][rope_dim / 2][2] (NULL iff rope_dim == 0)
 *   sink     f32 [n_heads]
 *   scores   f32 [batch][n_rows] (ratio >= 1)
 *   idx      int32 [batch][window + topk] (topk counted only at ratio >= 1)
 *   out      bf16 [batch][n_heads][head_dim]
 *   workspace as for v41_sparse_attn_sink with width = window + topk.
 * Geometry limits are those of the separate calls.  Calls sharing buffers
 * must not overlap in time.
 */
typedef struct v41_decode_step_args {
  int32_t batch;
  int32_t n_heads;
  int32_t head_dim;
  int32_t window;
  int32_t ratio;
  int32_t index_heads;
  int32_t index_dim;
  int32_t topk;
  int32_t rope_dim;
  float scale;
  int64_t n_rows;
  int64_t rope_rows;
  int64_t ring_bs;
  int64_t latent_bs;
  int64_t kI_bs;
  int64_t workspace_bytes;
  const int32_t *pos;
  v41_bf16 *q;
  const v41_bf16 *kv_new;
  v41_bf16 *ring;
  const v41_bf16 *latent;
  const v41_bf16 *kI;
  const v41_bf16 *qI;
  const float *w;
  const float *rope_table;
  const float *sink;
  float *scores;
  int32_t *idx;
  v41_bf16 *out;
  void *workspace;
} v41_decode_step_args;

int v41_decode_step(const v41_decode_step_args *args, v41_stream stream);

/*
 * Measurement helpers, not steps of the method: what this GPU reaches on
 * plain work, for stating throughput against measured ceilings beside the
 * published peaks.
 *
 * v41_probe_hbm_read reads `bytes` (a multiple of 16, buf 16-byte aligned)
 * once, 16 bytes per lane, grid-stride over 2048 workgroups of 256 threads,
 * with non-temporal loads when `nontemporal` is non-zero; nothing is
 * written (`sink`, one uint32, is written only under a condition the data
 * never meets, which keeps the loads).
 * v41_probe_mfma runs `workgroups` workgroups of four wavefronts, each
 * wavefront `iters` rounds of eight independent v_mfma_f32_16x16x32_bf16
 * (16384 flops each) on register operands: 524288 * workgroups * iters flops;
 * `sink` (one float) as above.
 */
int v41_probe_hbm_read(const void *buf, int64_t bytes, int32_t nontemporal,
                       uint32_t *sink, v41_stream stream);
int v41_probe_mfma(int32_t workgroups, int32_t iters, float *sink,
                   v41_stream stream);

#ifdef __cplusplus
}
#endif

#endif /* V41_H */
