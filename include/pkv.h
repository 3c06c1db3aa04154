/*
 * pkv.h -- C ABI of libpkv: attention over a paged K/V cache on AMD Instinct
 * MI355X (gfx950).
 *
 * Sources (page titles and sections):
 *   [P1] "Paged causal K/V cache and cached attention for VisualGen":
 *        Description / Cache, Description / Attention, Per-File QA
 *        Perspective, and the review threads on staged-token slot ids, on
 *        power-of-two pages and on the private-page regions
 *        (committed_private / current_private).
 *   [P5] "Support shared-prefix attention for n-sample requests in FMHA":
 *        commit messages on the n-sample path with CUDA graphs (up to 16
 *        query tokens per row), the FA4 prefix and tail passes, small-batch
 *        splits, MIN_SPLIT_TOKENS and the grouping check.
 *
 * Conventions shared by every call
 * --------------------------------
 * - All pointers are DEVICE pointers except `pool` (and the `pkv_pool`
 *   struct itself) and those a declaration marks HOST (block sizes and
 *   sizing results of the exact-window layout).  The caller owns every
 *   buffer; the library allocates no device memory and keeps no state
 *   between calls beyond a per-device cache of the compute-unit count.
 * - Every call is asynchronous on `stream` and never synchronises with the
 *   host, so a captured HIP graph replays it after the caller edits the
 *   device-side lengths, tables or slots in place ([P1] Description / Cache,
 *   graph-safety bullet).
 * - Argument checks run on the host before anything is launched.  A failed
 *   check returns a non-OK status, launches nothing and leaves every output
 *   untouched.  Zero tokens / zero rows return PKV_OK with no launch.
 * - Device-side contents are the caller's responsibility, as on the pages
 *   ([P1] Per-File QA Perspective on scatterKvSlots): slots and page ids in
 *   range, destination slots unique, kv_len <= the table row's capacity.
 *   Violations are undefined behaviour.
 * - Element strides and counts are in ELEMENTS of the stated dtype.
 */
#ifndef PKV_H_
#define PKV_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Same types as HIP's own hipStream_t and hipEvent_t (a repeated identical
 * typedef is legal). */
typedef struct ihipStream_t* hipStream_t;
typedef struct ihipEvent_t* hipEvent_t;

typedef enum {
  PKV_OK = 0,
  PKV_ERR_NULL = 1,        /* a required pointer is NULL                         */
  PKV_ERR_SHAPE = 2,       /* a size, stride or count is invalid                 */
  PKV_ERR_DTYPE = 3,       /* a dtype argument is not one of pkv_dtype           */
  PKV_ERR_UNSUPPORTED = 4, /* valid, but no kernel for this combination          */
  PKV_ERR_HIP = 5,         /* a kernel launch failed (hipGetLastError)           */
  PKV_ERR_ALIGN = 6,       /* a pointer or stride breaks the stated alignment    */
  PKV_ERR_SCRATCH = 7      /* the call needs more scratch than the no-allocation
                              entry point's device array holds                  */
} pkv_status;

typedef enum {
  PKV_F32 = 0,
  PKV_BF16 = 1,
  PKV_FP8_E4M3FN = 2 /* OCP e4m3fn codes; real value = code value * scale */
} pkv_dtype;

/*
 * A K/V page pool ([P1] Description / Cache: one pool and one page table,
 * a page holds the same tokens in every layer; one layer's pool per call).
 *
 * Layout: K and V are separate pools.  Page p starts at `k + p * page_stride`
 * (same stride for V) and holds [page_size, num_kv_heads, head_dim] elements,
 * contiguous.  So pool slot s = p * page_size + r ([P1] slot-id review thread:
 * int64 slot id = view_page * tokens_per_page + slot) is the row of
 * num_kv_heads * head_dim elements at page s / page_size, row s % page_size.
 * page_stride >= page_size * num_kv_heads * head_dim; a larger stride lets
 * K and V pages interleave in one allocation.
 *
 * page_size is a power of two ([P1] review thread: the commit-time layout
 * computes page and slot with shifts and masks).  The attention kernels need
 * page_size >= 16; the scatter takes any power of two.
 *
 * dtype PKV_FP8_E4M3FN: k_scale / v_scale are float [num_pages, num_kv_heads]
 * device arrays, the scale of each (page, kv head); NULL for other dtypes.
 */
typedef struct {
  void* k;
  void* v;
  int64_t page_stride;
  int64_t num_pages;
  int32_t page_size;
  int32_t num_kv_heads;
  int32_t head_dim;
  pkv_dtype dtype;
  const float* k_scale;
  const float* v_scale;
} pkv_pool;

/* Text of a status code (static storage). */
const char* pkv_status_string(pkv_status status);

/* ABI version: bumps when a signature or layout changes. */
int32_t pkv_abi_version(void);

/*
 * pkv_scatter_slots -- write new K/V token rows into pool slots.
 * [P1] Description / Cache (chunk K/V write bullet) and Per-File QA
 * Perspective on scatterKvSlots: the source is read once, with any token and
 * head stride (so K/V slices of a packed QKV projection need no copy), and
 * each token goes to one or two pool slots; optional source indices.
 *
 *   src_k, src_v       token i, kv head h starts at src + j * src_tok_stride
 *                      + h * src_head_stride with j = src_idx ? src_idx[i] : i;
 *                      head_dim elements contiguous; element type = pool dtype
 *                      (the bytes are copied as they are: fp8 stays fp8).
 *   src_idx            device int64 [n_tokens] or NULL.
 *   slots              device int64 [n_tokens]; slot < 0 means skip.
 *   slots2             device int64 [n_tokens] or NULL: second destination
 *                      (slot < 0 means skip).
 * Every (token, head) row is copied with the widest access (16, 8, 4, 2 or 1
 * bytes) that the pointers and strides allow.  Duplicate destinations race
 * (undefined which token wins).  fp8 scales are not touched.
 * Errors: NULL pool/k/v/src/slots -> PKV_ERR_NULL; n_tokens < 0, bad pool
 * geometry or strides -> PKV_ERR_SHAPE.
 */
pkv_status pkv_scatter_slots(const pkv_pool* pool, const void* src_k, const void* src_v,
                             int64_t src_tok_stride, int64_t src_head_stride,
                             const int64_t* src_idx, const int64_t* slots, const int64_t* slots2,
                             int64_t n_tokens, hipStream_t stream);

/*
 * pkv_attn_decode -- paged decode attention.
 * [P1] Description / Attention (paged attention over block-table rows) and
 * [P5] FA4 prefix / tail commit messages (n query rows share one table row:
 * the shared-prefix pass of an n-sample group; natural-log LSE returned for
 * the merge).
 *
 *   q            [num_tables, rows_per_table, num_q_heads, head_dim], q_dtype
 *                PKV_BF16 (or PKV_F32), contiguous.
 *   block_table  device int32 [num_tables, table_stride]: logical key p of
 *                row t is slot block_table[t][p / page_size] * page_size +
 *                p % page_size.  Entries at or past ceil(kv_lens[t] /
 *                page_size) are never read ([P5] grouping commit).
 *   kv_lens      device int32 [num_tables], 0 <= kv_lens[t] <= max_kv_len.
 *   max_kv_len   host upper bound of kv_lens (plans the work split).
 *   out          [num_tables, rows_per_table, num_q_heads, head_dim],
 *                out_dtype PKV_F32 or PKV_BF16.
 *   out_lse      NULL or float [num_tables, rows_per_table, num_q_heads]:
 *                ln sum_k exp(sm_scale * q.k).
 * Query head h reads kv head h / (num_q_heads / num_kv_heads).  A row with
 * kv_lens = 0 gets out = 0 and lse = -inf.
 *   workspace    NULL or device scratch of workspace_bytes (>= the value of
 *                pkv_attn_decode_workspace_bytes for the same shapes) used for
 *                cross-workgroup key splits and their merge.  With a NULL or
 *                smaller workspace the call runs unsplit (same result up to
 *                float rounding, possibly slower).  With a workspace, up to
 *                8192 table rows run as one balanced persistent grid
 *                (stream-K: the per-row tile prefix sums live in LDS); more
 *                rows run as fixed key splits of >= 512 tokens (the pages'
 *                rule), which balances less well on uneven lengths.
 * Kernels: q bf16 with K/V bf16 or fp8 run on bf16 MFMA; q fp32 (any K/V
 * dtype) runs on the vector ALUs.  head_dim 64 or 128.
 * sm_scale must be finite and > 0.
 * Errors: NULL pointers -> PKV_ERR_NULL; num_q_heads % num_kv_heads,
 * negative sizes, sm_scale <= 0 -> PKV_ERR_SHAPE; page_size < 16 ->
 * PKV_ERR_UNSUPPORTED; unknown dtype ->
 * PKV_ERR_DTYPE; other head_dim / dtype combinations or missing fp8 scales ->
 * PKV_ERR_UNSUPPORTED.
 */
size_t pkv_attn_decode_workspace_bytes(int32_t num_tables, int32_t rows_per_table, int32_t num_q_heads,
                                       int32_t num_kv_heads, int32_t head_dim, int32_t max_kv_len);

pkv_status pkv_attn_decode(const pkv_pool* pool, const void* q, pkv_dtype q_dtype,
                           int32_t num_tables, int32_t rows_per_table, int32_t num_q_heads,
                           const int32_t* block_table, int32_t table_stride, const int32_t* kv_lens,
                           int32_t max_kv_len, float sm_scale,
                           void* out, pkv_dtype out_dtype, float* out_lse,
                           void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * pkv_set_timing_events -- measurement hook.  While start or stop is not
 * NULL, the main kernel of every pkv_attn_decode / pkv_attn_decode_noalloc /
 * pkv_attn_decode_step / pkv_attn_decode_append / prefill call (the
 * stream-K, split or fp32 decode kernel; the prefill kernel; not a merge
 * kernel of split work, nor the scatter that pkv_attn_decode_append may run
 * first) is launched through hipExtLaunchKernel with these events, which
 * then carry that kernel's own start and end times: hipEventElapsedTime(start,
 * stop) is the kernel's duration, with no marker between it and its
 * neighbours.  Each such launch sets both events again, so after a call they
 * hold its main kernel's times.  NULL, NULL turns the hook off.  Process-wide
 * and not synchronised: set it while no other host thread calls the library.
 * The events are the caller's, created before the call.
 */
void pkv_set_timing_events(hipEvent_t start, hipEvent_t stop);

/*
 * pkv_attn_decode_noalloc -- pkv_attn_decode for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).
 *
 * Arguments, layouts, results and errors as pkv_attn_decode, without the
 * workspace: the cross-workgroup state lives in a file-scope device array of
 * 24 MiB that each GPU the library runs on holds until the process ends
 * (its device address is looked up once per device).  The call allocates
 * nothing.  The stream-K state of one workgroup per CU with head_dim 128 and
 * up to 8192 table rows takes about 16.2 MiB on a 256-CU device; a call whose
 * state does not fit (more than 8192 rows with key splits larger than the
 * array, or a device of more than 340 CUs) returns PKV_ERR_SCRATCH and
 * launches nothing.  Every call on one GPU uses that GPU's one array, which
 * keeps the last call's contents (nothing in it needs to start at zero):
 * calls that can overlap on one GPU (other streams, other host threads) race
 * and must be ordered by the caller.
 */
pkv_status pkv_attn_decode_noalloc(const pkv_pool* pool, const void* q, pkv_dtype q_dtype,
                                   int32_t num_tables, int32_t rows_per_table, int32_t num_q_heads,
                                   const int32_t* block_table, int32_t table_stride, const int32_t* kv_lens,
                                   int32_t max_kv_len, float sm_scale,
                                   void* out, pkv_dtype out_dtype, float* out_lse, hipStream_t stream);

/*
 * pkv_attn_decode_step -- paged decode of a multi-token step (speculative
 * verification: draft tokens + 1 per row).
 * [P5] commit on the n-sample path with CUDA graphs (one kernel serves up to
 * 16 query tokens per row, the verification steps of K draft tokens + 1) and
 * the FA4 tail commit (the step's K/V is written into the row's pages first,
 * then attended causally).
 *
 * As pkv_attn_decode with rows_per_table = q_len, except that the q_len rows
 * of table row t are the tokens of one step, already written as the last
 * q_len keys of the row: row j (0 <= j < q_len) attends logical keys
 * [0, kv_lens[t] - (q_len - 1 - j)).  A row left with no key (kv_lens[t] <
 * q_len - j) gets out = 0 and lse = -inf.  The workspace size is
 * pkv_attn_decode_workspace_bytes(num_tables, q_len, ...).  q_len >= 1 (the
 * pages' kernels serve up to 16; any count works here).
 * Errors: as pkv_attn_decode.
 */
pkv_status pkv_attn_decode_step(const pkv_pool* pool, const void* q, pkv_dtype q_dtype,
                                int32_t num_tables, int32_t q_len, int32_t num_q_heads,
                                const int32_t* block_table, int32_t table_stride, const int32_t* kv_lens,
                                int32_t max_kv_len, float sm_scale,
                                void* out, pkv_dtype out_dtype, float* out_lse,
                                void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * pkv_attn_decode_append -- write a step's K/V into the cache and attend, in
 * one call.
 * [P5] FA4 tail commit (the step's K/V goes into the row's pages first, then
 * is attended causally); "Paged causal K/V cache and cached attention for
 * VisualGen", Description / Cache (the chunk's K/V written into its slots
 * before attention).
 *
 * new_k, new_v: the step's tokens, element type of the pool, rows
 * [num_tables * q_len, num_kv_heads, head_dim] with token stride
 * new_tok_stride and kv-head stride new_head_stride (elements; the head_dim
 * elements of a row contiguous).  Token j of table row t (row t * q_len + j)
 * is logical key kv_lens[t] - q_len + j of that row: it is written, bytes
 * untouched, into that key's slot (page block_table[t][key / page_size], row
 * key % page_size), as pkv_scatter_slots would, and then every argument and
 * result is that of pkv_attn_decode_step over the updated pool.  Tokens whose
 * key would be negative (kv_lens[t] < q_len - j) are not written.  The slots
 * written must belong to the call alone (no other row's key maps to them).
 * With a stream-K workspace and kv heads in quads (one 16-row block per
 * row: q_len * num_q_heads / num_kv_heads <= 16), 16-byte aligned new_k /
 * new_v and strides, the decode kernel writes the tokens itself (no separate
 * launch); otherwise a scatter kernel runs first.  Either way the pool holds
 * the tokens when the call's work on the stream is done.
 * Errors: NULL new_k or new_v -> PKV_ERR_NULL; negative strides ->
 * PKV_ERR_SHAPE; the rest as pkv_attn_decode_step.
 */
pkv_status pkv_attn_decode_append(const pkv_pool* pool, const void* new_k, const void* new_v,
                                  int64_t new_tok_stride, int64_t new_head_stride,
                                  const void* q, pkv_dtype q_dtype,
                                  int32_t num_tables, int32_t q_len, int32_t num_q_heads,
                                  const int32_t* block_table, int32_t table_stride, const int32_t* kv_lens,
                                  int32_t max_kv_len, float sm_scale,
                                  void* out, pkv_dtype out_dtype, float* out_lse,
                                  void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * pkv_attn_decode_shared_prefix -- one n-sample decode step: shared prefix,
 * private tails and their merge.
 * [P5] commits on the n-sample path (rows whose tables start with the same
 * pages form a group whose shared pages are read once and merged with every
 * row's private tail; one fused kernel does prefix, tail and merge for up to
 * 16 query tokens per row) and the FA4 tail and split commits (the step's
 * tokens are attended causally in the tail; prefix and tail states are joined
 * in natural-log LSE; an empty run has LSE -inf).
 *
 *   q             [groups * samples, q_len, num_q_heads, head_dim] bf16,
 *                 contiguous; sample r belongs to group r / samples.
 *   prefix_table  device int32 [groups, prefix_stride], prefix_lens device
 *                 int32 [groups] (<= max_prefix_len): the group's shared keys.
 *   tail_table    device int32 [groups * samples, tail_stride], tail_lens
 *                 device int32 [groups * samples] (<= max_tail_len): the
 *                 sample's private keys, its step's q_len tokens last.
 *   out, out_lse  as pkv_attn_decode for q's shape.
 * Query token j of sample r attends prefix keys [0, prefix_lens[g]) and tail
 * keys [0, tail_lens[r] - (q_len - 1 - j)) (none when that is not positive).
 *   workspace     device scratch of at least
 *                 pkv_attn_decode_shared_prefix_workspace_bytes(...) bytes,
 *                 16-byte aligned, contents ignored: the fp32 states of the
 *                 prefix's key splits (>= 1024 keys each, <= 16) and of
 *                 the tails.  Two calls in flight need two workspaces.
 * Kernels: one launch of every prefix-split and tail workgroup (bf16 MFMA;
 * K/V bf16 or fp8 e4m3fn; head_dim 64 or 128; page_size >= 16), then one
 * merge launch.
 * Errors: as pkv_attn_decode; a missing or small workspace -> PKV_ERR_NULL /
 * PKV_ERR_SHAPE; q not bf16 or an fp32 pool -> PKV_ERR_UNSUPPORTED.
 */
size_t pkv_attn_decode_shared_prefix_workspace_bytes(int32_t groups, int32_t samples, int32_t q_len,
                                                     int32_t num_q_heads, int32_t head_dim, int32_t max_prefix_len);

pkv_status pkv_attn_decode_shared_prefix(const pkv_pool* pool, const void* q, pkv_dtype q_dtype, int32_t groups,
                                         int32_t samples, int32_t q_len, int32_t num_q_heads,
                                         const int32_t* prefix_table, int32_t prefix_stride,
                                         const int32_t* prefix_lens, int32_t max_prefix_len,
                                         const int32_t* tail_table, int32_t tail_stride, const int32_t* tail_lens,
                                         int32_t max_tail_len, float sm_scale, void* out, pkv_dtype out_dtype,
                                         float* out_lse, void* workspace, size_t workspace_bytes,
                                         hipStream_t stream);

/*
 * pkv_attn_decode_shared_prefix_append -- an n-sample step that writes its
 * tokens' K/V into the tails and attends, in one call.
 * [P5] commits on the n-sample path (the shared prefix read once per group,
 * every sample's private tail) and the FA4 tail commit (the step's K/V goes
 * into the row's pages first, then is attended causally).
 *
 * new_k, new_v: the step's tokens, element type of the pool, rows
 * [groups * samples * q_len, num_kv_heads, head_dim] with token stride
 * new_tok_stride and kv-head stride new_head_stride (elements; the head_dim
 * elements of a row contiguous).  Token j of sample r (row r * q_len + j) is
 * tail key tail_lens[r] - q_len + j: it is written, bytes untouched, into
 * that key's slot (page tail_table[r][key / page_size], row key % page_size),
 * and then every argument and result is that of
 * pkv_attn_decode_shared_prefix over the updated pool.  Tokens whose key
 * would be negative are not written.  The slots written must belong to the
 * call alone: no prefix key and no other tail key maps to them.
 * When a sample's rows fit 64 (q_len * num_q_heads / num_kv_heads <= 64) and
 * new_k / new_v and their strides are 16-byte aligned, the tail workgroups
 * write the tokens themselves (no separate launch); otherwise a scatter
 * kernel runs first.  Either way the pool holds the tokens when the call's
 * work on the stream is done.
 * Errors: NULL new_k or new_v -> PKV_ERR_NULL; negative strides ->
 * PKV_ERR_SHAPE; the rest as pkv_attn_decode_shared_prefix.
 */
pkv_status pkv_attn_decode_shared_prefix_append(const pkv_pool* pool, const void* new_k, const void* new_v,
                                                int64_t new_tok_stride, int64_t new_head_stride, const void* q,
                                                pkv_dtype q_dtype, int32_t groups, int32_t samples, int32_t q_len,
                                                int32_t num_q_heads, const int32_t* prefix_table,
                                                int32_t prefix_stride, const int32_t* prefix_lens,
                                                int32_t max_prefix_len, const int32_t* tail_table,
                                                int32_t tail_stride, const int32_t* tail_lens, int32_t max_tail_len,
                                                float sm_scale, void* out, pkv_dtype out_dtype, float* out_lse,
                                                void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * pkv_attn_prefill_block_causal -- paged prefill with causal blocks.
 * [P1] Description / Cache (frame-causal attention needs no mask: the new
 * tokens are cut into causal blocks, each with its own key count, full
 * attention inside a block and causal across blocks; a block's new tokens are
 * the last keys of its row) and Description / Attention (seq_len is the number
 * of real query tokens; padding rows are neither written nor attended and
 * their outputs are zero).
 *
 *   q                  query row i of batch b, head h starts at
 *                      q + (b * s_q + i) * q_tok_stride + h * q_head_stride;
 *                      head_dim contiguous (so q may be the Q slice of a packed
 *                      [B, s_q, Hq + 2 Hkv, D] projection).  q_dtype PKV_BF16.
 *   block_table        device int32 [batch, table_stride].
 *   n_ctx, seq_len     device int32 [batch]: cached keys before the new tokens
 *                      (pinned prefix + history) and real new tokens
 *                      (<= s_q).  The new tokens must already sit at logical
 *                      keys n_ctx .. n_ctx + seq_len - 1 of the table row.
 *   causal_block_size  > 0: query i < seq_len of block i / cbs sees logical
 *                      keys [0, n_ctx + min((i / cbs + 1) * cbs, seq_len));
 *                      0: one block (every real query sees n_ctx + seq_len).
 *   max_keys           host upper bound of n_ctx + seq_len.
 *   out                [batch, s_q, num_q_heads, head_dim] contiguous,
 *                      out_dtype PKV_BF16 or PKV_F32; rows i >= seq_len are 0.
 *   out_lse            NULL or float [batch, s_q, num_q_heads]; -inf for
 *                      padding rows.
 *   workspace          NULL, or device scratch of at least
 *                      pkv_attn_prefill_workspace_bytes(...) bytes,
 *                      256-byte aligned, contents ignored.  With it the query
 *                      tiles left over after the last full round of a
 *                      persistent grid are split along the keys and merged by
 *                      a second kernel on the same stream; with NULL (or too
 *                      small / misaligned) they run whole.  The size follows
 *                      the shape and the current device's CU count: two
 *                      partial states (66,560 bytes each) per workgroup of the
 *                      grid when some XCD's share of the query tiles leaves a
 *                      remainder to split, else 0 (no workspace needed).  On a
 *                      machine without a device it assumes the largest grid
 *                      (512 workgroups).  Two calls in flight at once need two
 *                      workspaces.
 * Kernel: K/V bf16 (head_dim 128 or 64, page_size >= 16) on bf16 MFMA, or
 * fp8 e4m3fn with k_scale / v_scale (head_dim 128, page_size >= 32): the fp8
 * rows are moved to LDS as they are; QK^T runs on fp8 MFMA from the raw K
 * codes, with q held per row as two e4m3 code sets (about 2^-8 relative,
 * near bf16's own rounding), and PV on bf16 MFMA over V widened exactly in
 * LDS.  The fp8 MFMA accumulates less exactly than fp32 when one product
 * dominates a 64-dim block: a q row with one dim 4096x the others comes back
 * with lse off by up to 0.33 (outputs within 0.05); rows whose largest
 * entry is up to a few hundred times the rest stay within 0.06.  The scale
 * of each (page, kv head) is applied in the softmax (K scale
 * on the scores, V scale on the probabilities and back out of their sum).  Scales
 * must be >= 0; a scale below 2^-100 acts as 2^-100 (so 0 gives keys of
 * score 0 and values of weight ~0, as code x 0 would, without 0 x inf).
 * Errors: as pkv_attn_decode; fp8 with another head_dim or page_size, or an
 * fp32 pool -> PKV_ERR_UNSUPPORTED.
 */
size_t pkv_attn_prefill_workspace_bytes(int32_t batch, int32_t s_q, int32_t num_q_heads, int32_t num_kv_heads,
                                        int32_t head_dim, int32_t max_keys);

pkv_status pkv_attn_prefill_block_causal(const pkv_pool* pool, const void* q, pkv_dtype q_dtype,
                                         int64_t q_tok_stride, int64_t q_head_stride,
                                         int32_t batch, int32_t s_q, int32_t num_q_heads,
                                         const int32_t* block_table, int32_t table_stride,
                                         const int32_t* n_ctx, const int32_t* seq_len,
                                         int32_t causal_block_size, int32_t max_keys, float sm_scale,
                                         void* out, pkv_dtype out_dtype, float* out_lse,
                                         void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * pkv_attn_prefill_block_causal_ragged -- the same prefill over a ragged
 * batch: [P1] Description / Cache runs a forward's causal blocks as one
 * ragged batch over the same table, each with its own key count, and block
 * sizes come with the geometry (they need not be equal).
 *
 * As pkv_attn_prefill_block_causal, except for where rows live:
 *   q_offsets          device int32 [batch + 1], non-decreasing: batch entry
 *                      b owns rows q_offsets[b] .. q_offsets[b + 1] - 1 of q,
 *                      out and out_lse (row i of entry b is row
 *                      q_offsets[b] + i), and seq_len[b] <= that row count.
 *                      Rows i in [seq_len[b], row count) are padding (0 and
 *                      -inf); nothing past an entry's rows is read or
 *                      written.
 *   q                  row r, head h at q + r * q_tok_stride + h * q_head_stride.
 *   out, out_lse       [q_offsets[batch], num_q_heads, head_dim] and
 *                      [q_offsets[batch], num_q_heads].
 *   max_rows           host upper bound of every entry's row count (it sizes
 *                      the query tiles; the workspace size is
 *                      pkv_attn_prefill_workspace_bytes with s_q = max_rows).
 * The exact-window layout's per-block tables, n_ctx and seq_len (blocks of
 * any sizes) drive it directly, with q_offsets the prefix sums of the block
 * sizes.
 * Errors: as pkv_attn_prefill_block_causal; NULL q_offsets -> PKV_ERR_NULL.
 */
pkv_status pkv_attn_prefill_block_causal_ragged(const pkv_pool* pool, const void* q, pkv_dtype q_dtype,
                                                int64_t q_tok_stride, int64_t q_head_stride,
                                                int32_t batch, int32_t max_rows, int32_t num_q_heads,
                                                const int32_t* q_offsets,
                                                const int32_t* block_table, int32_t table_stride,
                                                const int32_t* n_ctx, const int32_t* seq_len,
                                                int32_t causal_block_size, int32_t max_keys, float sm_scale,
                                                void* out, pkv_dtype out_dtype, float* out_lse,
                                                void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * pkv_merge_states -- join attention states over disjoint key sets.
 * [P5] FA4 tail commit (prefix and tail states joined by one merge kernel,
 * natural-log LSE) and small-batch split commit (an empty run has LSE -inf).
 *
 *   o_parts    float [num_states, rows, num_q_heads, head_dim], each state
 *              normalised over its own keys.
 *   lse_parts  float [num_states, rows, num_q_heads], natural log.
 *   out        [rows, num_q_heads, head_dim], out_dtype PKV_F32 or PKV_BF16.
 *   out_lse    NULL or float [rows, num_q_heads].
 * With m = max_i lse_i, w_i = exp(lse_i - m): out = sum_i w_i o_i / sum_i w_i,
 * lse = m + ln sum_i w_i.  If every lse_i is -inf: out = 0, lse = -inf, and
 * no o_i is read.  States with weight 0 never contribute (NaN-safe).
 * head_dim must be a multiple of 4.
 * Errors: NULL -> PKV_ERR_NULL; num_states < 1 or bad sizes -> PKV_ERR_SHAPE.
 */
pkv_status pkv_merge_states(const float* o_parts, const float* lse_parts, int32_t num_states, int64_t rows,
                            int32_t num_q_heads, int32_t head_dim, void* out, pkv_dtype out_dtype,
                            float* out_lse, hipStream_t stream);

/*
 * pkv_rotate_rows -- in-place rotation of the rows of a 2-D array (page-table
 * eviction).
 * [P1] Description / Cache (eviction from the rolling history window is an
 * in-place rotation of the page table on the device, not a reallocation).
 *
 *   data        device pointer to element (0, 0); element (r, c) is at byte
 *               (r * row_stride + c) * elem_size.  Rotated in place.
 *   rows, cols  >= 0.  row_stride >= cols (elements).
 *   elem_size   1, 2, 4, 8 or 16 bytes.
 *   shift       any integer: element c takes the old element
 *               (c + shift) mod cols (the first shift entries move to the
 *               end of the row).
 * rows == 0, cols <= 1 or shift == 0 mod cols: no launch (data may be NULL).
 * Errors: PKV_ERR_NULL (data NULL with work to do); PKV_ERR_SHAPE (negative
 * sizes, row_stride < cols); PKV_ERR_UNSUPPORTED (elem_size); PKV_ERR_ALIGN
 * (data not aligned to elem_size); PKV_ERR_HIP.
 */
pkv_status pkv_rotate_rows(void* data, int64_t rows, int64_t cols, int64_t row_stride, int32_t elem_size,
                           int64_t shift, hipStream_t stream);

/*
 * pkv_copy_slots -- pool-to-pool copy of key rows (private-page fill).
 * [P1] Description / Cache (commit fills the causal blocks' private pages
 * with one pool-to-pool copy; the copy's entry list carries sentinels).
 *
 *   pool          as for pkv_scatter_slots; layer l of a multi-layer pool
 *                 starts at k + l * layer_stride (and v + l * layer_stride).
 *   num_layers    >= 1; layer_stride (elements) >= num_pages * page_stride
 *                 when num_layers > 1.
 *   src_slots,    device int64 [n]: entry i copies slot src_slots[i] to slot
 *   dst_slots     dst_slots[i] (whole key row: every kv head and dim, K and
 *                 V) in every layer.  A negative source or destination is a
 *                 sentinel: the entry is skipped.  Destinations must be
 *                 distinct and no destination may be another entry's source
 *                 (otherwise the result is not defined).  Slots must lie in
 *                 the pool.  fp8 scales are not touched.
 * n == 0: no launch.
 * Errors: as pkv_scatter_slots; bad num_layers / layer_stride -> PKV_ERR_SHAPE.
 */
pkv_status pkv_copy_slots(const pkv_pool* pool, int32_t num_layers, int64_t layer_stride, const int64_t* src_slots,
                          const int64_t* dst_slots, int64_t n, hipStream_t stream);

/*
 * Exact-window layout.
 * [P1] Description / Cache (the sequence is [fixed region | rolling history
 * window | staged tokens]; a table row can start a key sequence only at a
 * page boundary, so each causal block gets private pages at the end of its
 * row holding the visible keys of the up to three partly visible pages --
 * fixed-region tail, window-start page, earlier keys on the block's start
 * page -- and then its own tokens, which stay the last keys of its row; at
 * commit one kernel reads the table and rewrites every per-block tensor in
 * place) and the review thread on the private regions (committed keys are
 * copied at commit, earlier blocks' staged keys every forward; at most
 * 3 (page_size - 1) copied keys per block).
 *
 * Geometry (logical key positions):
 *   - keys [0, committed) are history, staged token t is key committed + t;
 *   - the fixed region is [0, pin_tokens) and owns the first
 *     fixed_pages = ceil(pin_tokens / page_size) table entries;
 *   - the rolling region (keys >= pin_tokens) starts on a page of its own;
 *     the first `evicted` rolling tokens (whole pages) have been rotated out
 *     of the table, so rolling key x is on table entry
 *     fixed_pages + (x - pin_tokens - evicted) / page_size;
 *   - causal block b covers keys [s_b, s_b + block_sizes[b]), s_0 = committed,
 *     and sees [0, pin_tokens), [max(pin_tokens, s_b - window_tokens), s_b)
 *     and itself.
 * Commit sequence: after `committed` grows, evicted' =
 * pkv_window_evicted_tokens(...) and the rolling part of the table is rotated
 * left by (evicted' - evicted) / page_size entries (pkv_rotate_rows); then
 * pkv_causal_layout, then pkv_copy_slots over the commit list.  Each forward:
 * pkv_scatter_slots with (stage_slots, stage_slots2), pkv_copy_slots over the
 * current list, then attention over block_tables (one batch entry per causal
 * block: n_ctx keys before the block, seq_len new keys).
 */
typedef struct {
  int32_t fixed_pages;    /* table entries of the fixed region                       */
  int32_t rolling_pages;  /* rolling entries that always cover window and staged keys */
  int32_t private_pages;  /* private pages each causal block needs                   */
  int32_t table_width;    /* entries of a per-block row                              */
  int32_t list_stride;    /* commit / current list entries per block = 3 (ps - 1)    */
} pkv_causal_bounds;

#define PKV_MAX_CAUSAL_BLOCKS 64

/*
 * pkv_causal_layout_bounds -- sizes an exact-window geometry needs (host only:
 * block_sizes is a HOST int32 [num_blocks] array, bounds a HOST struct).
 *   rolling_pages = ceil((window + page_size - 1 + sum(block_sizes)) / page_size)
 *   private_pages = ceil((3 (page_size - 1) + max(block_sizes)) / page_size)
 *   table_width   = pin / page_size + window / page_size + private_pages
 * Errors: NULL -> PKV_ERR_NULL; page_size not a power of two, negative
 * sizes, a block size < 1, num_blocks outside 1..PKV_MAX_CAUSAL_BLOCKS or a
 * size beyond int32 -> PKV_ERR_SHAPE.
 */
pkv_status pkv_causal_layout_bounds(int32_t page_size, int64_t pin_tokens, int64_t window_tokens,
                                    const int32_t* block_sizes, int32_t num_blocks, pkv_causal_bounds* bounds);

/*
 * pkv_window_evicted_tokens -- rolling tokens no later block can see, in
 * whole pages (host only): floor(max(0, committed - window - pin) / ps) * ps.
 * Returns -1 for a page size that is not a power of two or a negative size.
 */
int64_t pkv_window_evicted_tokens(int32_t page_size, int64_t pin_tokens, int64_t window_tokens, int64_t committed);

/*
 * pkv_causal_layout -- rewrite every per-block tensor of an exact-window
 * geometry from the sequence's page table (one launch, no host data).
 *
 *   table          device int32 [table_len]: fixed pages, then rolling pages.
 *   private_pages  device int32 [num_blocks, private_stride]: pages owned by
 *                  each causal block, disjoint from the table's.
 *   block_sizes    HOST int32 [num_blocks] (values >= 1, num_blocks <= 64);
 *                  passed by value to the kernel.
 *   block_tables   device int32 [num_blocks, table_width]: block b's whole
 *                  visible pages (keys all visible and before the block), in
 *                  key order, then its private pages; a block with no other
 *                  visible key whose first key starts a rolling page reads
 *                  its own keys from their own pages instead.  Unused entries
 *                  are -1.
 *   n_ctx, seq_len device int32 [num_blocks]: keys before the block's own
 *                  tokens in its row, and block_sizes[b].
 *   stage_slots    device int64 [sum(block_sizes)]: staged token t's slot in
 *                  the sequence's own pages; stage_slots2: its copy in its
 *                  block's private pages (after the block's copied keys), or
 *                  -1 when the block reads its own pages.
 *   commit_src/dst device int64 [num_blocks * list_stride]: block b's entries
 *   current_src/dst start at b * list_stride, padded with -1 sentinels.  The
 *                  private pages hold the copied keys in key order; those
 *                  before `committed` are in the commit list, the others
 *                  (earlier blocks' staged keys) in the current list.
 *                  With list_stride 0 (page size 1) they may be NULL.
 * Every output is written whole (padding included); nothing else is touched.
 * Errors: NULL -> PKV_ERR_NULL; a bad geometry (as pkv_causal_layout_bounds),
 * evicted not a multiple of page_size or beyond pkv_window_evicted_tokens,
 * a table too short for the staged keys, private_stride / table_width /
 * list_stride below pkv_causal_layout_bounds, or keys beyond int32 ->
 * PKV_ERR_SHAPE.  Page ids are not checked.
 */
pkv_status pkv_causal_layout(const int32_t* table, int32_t table_len, const int32_t* private_pages,
                             int32_t private_stride, int32_t page_size, int64_t pin_tokens, int64_t window_tokens,
                             int64_t committed, int64_t evicted, const int32_t* block_sizes, int32_t num_blocks,
                             int32_t* block_tables, int32_t table_width, int32_t* n_ctx, int32_t* seq_len,
                             int64_t* stage_slots, int64_t* stage_slots2, int64_t* commit_src, int64_t* commit_dst,
                             int64_t* current_src, int64_t* current_dst, int32_t list_stride, hipStream_t stream);

/*
 * Device-side content checks (debugging aid).
 * [P1] Per-File QA Perspective (the scatter does not range-check device slot
 * ids; device slot bounds stay the caller's responsibility).  The attention
 * and copy calls trust their device inputs; these calls count the entries
 * that break that contract, reading only ids and lengths, never the pool.
 * One workgroup walks the input: meant for debugging, not for every step.
 *
 * pkv_check_slots: *bad (device int32) = number of slots[i] >= num_pages *
 *   page_size (negative entries are sentinels, valid).  n == 0 writes 0.
 * pkv_check_tables: *bad (device int32) = number of rows t whose kv_lens[t]
 *   is negative or above table_stride * page_size, or whose first
 *   ceil(kv_lens[t] / page_size) page ids are not all in [0, num_pages).
 * Both overwrite *bad (no zeroing needed) and run asynchronously on stream.
 * Errors: bad pool -> as pkv_scatter_slots; NULL -> PKV_ERR_NULL; negative
 * sizes -> PKV_ERR_SHAPE.
 */
pkv_status pkv_check_slots(const pkv_pool* pool, const int64_t* slots, int64_t n, int32_t* bad, hipStream_t stream);
pkv_status pkv_check_tables(const pkv_pool* pool, const int32_t* block_table, int32_t table_stride,
                            const int32_t* kv_lens, int32_t num_tables, int32_t* bad, hipStream_t stream);

/*
 * pkv_xcd_ids -- probe of workgroup placement (a diagnostic, not a hot path).
 * Launches num_workgroups workgroups of `threads` threads (64 .. 1024, a
 * multiple of 64) on stream; workgroup i writes the XCC_ID hardware register
 * of the XCD (accelerator complex die) it ran on to out[i] (device int32,
 * overwritten; the die index is in the low 4 bits).  The prefill's persistent
 * schedule (pkv_attn_prefill_block_causal) hands the kv heads of group x to
 * workgroups x, x + 8, x + 16, ... so that each K/V tile is fetched once into
 * one XCD's L2; it assumes that workgroups whose ids agree mod 8 run on one
 * XCD (the dispatcher deals them to the 8 XCDs round robin, starting where
 * earlier launches left off), which this probe checks for a given launch
 * shape.  Results are correct whatever the placement; only the L2 reuse
 * depends on it.
 * Errors: NULL out with num_workgroups > 0 -> PKV_ERR_NULL; a bad size or
 * thread count -> PKV_ERR_SHAPE; out not 4-byte aligned -> PKV_ERR_ALIGN;
 * num_workgroups == 0 -> PKV_OK, nothing launched.
 */
pkv_status pkv_xcd_ids(int32_t* out, int32_t num_workgroups, int32_t threads, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* PKV_H_ */
