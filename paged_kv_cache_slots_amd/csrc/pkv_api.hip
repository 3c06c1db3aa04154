// Host side of the libpkv C ABI: argument checks (before any HIP call), work
// planning and kernel dispatch.  No device memory is allocated here and no
// host synchronisation happens; see include/pkv.h for the contract.
#include <stdint.h>

#include <algorithm>

#include "pkv.h"
#include "pkv_internal.hpp"

namespace {

using namespace pkv;

constexpr int kAbiVersion = 2;
static_assert(kMaxCausalBlocks == PKV_MAX_CAUSAL_BLOCKS, "block limit of the ABI and the kernel differ");

// Key splits of the decode: chunks of at least 512 tokens and at most 16
// splits ("Support shared-prefix attention for n-sample requests in FMHA",
// split-KV and MIN_SPLIT_TOKENS commit messages).  The split count depends on
// host arguments only, so the workspace size is known before the call.
#ifndef PKV_MIN_SPLIT_TOKENS
#define PKV_MIN_SPLIT_TOKENS 512
#endif
#ifndef PKV_MAX_SPLITS
#define PKV_MAX_SPLITS 16
#endif
constexpr int kMinSplitTokens = PKV_MIN_SPLIT_TOKENS;
constexpr int kMaxSplits = PKV_MAX_SPLITS;
// Prefix splits of the fused n-sample step.  Its prefix workgroups share each
// tile through LDS across the four row blocks of the group, which makes a
// tile cheap next to a workgroup's start-up and the extra state every split
// adds to the merge; measured on the n-sample workload (2048-token prefixes),
// splits of at least 1024 keys beat the split decode's 512.
#ifndef PKV_SHARED_MIN_SPLIT_TOKENS
#define PKV_SHARED_MIN_SPLIT_TOKENS 1024
#endif
constexpr int kSharedMinSplitTokens = PKV_SHARED_MIN_SPLIT_TOKENS;

bool valid_dtype(int d) { return d == PKV_F32 || d == PKV_BF16 || d == PKV_FP8_E4M3FN; }
int elem_bytes(pkv_dtype d) { return d == PKV_F32 ? 4 : d == PKV_BF16 ? 2 : 1; }
ElemType elem_type(pkv_dtype d) { return d == PKV_F32 ? kF32 : d == PKV_BF16 ? kBF16 : kFP8; }
bool is_pow2(int64_t x) { return x > 0 && (x & (x - 1)) == 0; }
int log2i(int64_t x) {
  int s = 0;
  while ((int64_t(1) << s) < x) ++s;
  return s;
}
bool aligned(const void* p, int a) { return (reinterpret_cast<uintptr_t>(p) % (uintptr_t)a) == 0; }
int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

pkv_status check_pool(const pkv_pool* pool) {
  if (!pool || !pool->k || !pool->v) return PKV_ERR_NULL;
  if (!valid_dtype(pool->dtype)) return PKV_ERR_DTYPE;
  if (pool->num_pages < 1 || pool->num_kv_heads < 1 || pool->head_dim < 1) return PKV_ERR_SHAPE;
  if (!is_pow2(pool->page_size)) return PKV_ERR_SHAPE;
  if (pool->page_stride < (int64_t)pool->page_size * pool->num_kv_heads * pool->head_dim) return PKV_ERR_SHAPE;
  if (pool->dtype == PKV_FP8_E4M3FN && (!pool->k_scale || !pool->v_scale)) return PKV_ERR_NULL;
  return PKV_OK;
}

struct SplitPlan {
  int splits;
  int tiles_per_split;
};

SplitPlan plan_decode(int32_t max_kv_len, int min_split_tokens = kMinSplitTokens) {
  const int64_t tiles = std::max<int64_t>(1, ceil_div(std::max(max_kv_len, 0), 32));
  const int64_t by_len = ceil_div(std::max(max_kv_len, 1), min_split_tokens);
  const int splits = (int)std::min<int64_t>(kMaxSplits, std::max<int64_t>(1, by_len));
  return SplitPlan{splits, (int)ceil_div(tiles, splits)};
}

size_t decode_ws_bytes(int64_t rows, int32_t num_q_heads, int32_t head_dim, int splits) {
  if (splits <= 1) return 0;
  const int64_t plane = rows * num_q_heads;
  return (size_t)(splits * plane * (int64_t)(head_dim + 1) * (int64_t)sizeof(float));
}

// Stream-K workspace: prefix sums of tiles per table row, then the partial
// states (output rows, then their LSE) of every wave's two slots.
int64_t align256(int64_t x) { return (x + 255) & ~int64_t(255); }
int64_t sk_cum_bytes(int32_t num_tables) { return align256(4 * (int64_t)(num_tables + 1)); }
int64_t sk_rows() { return 2 * (int64_t)kMaxSkWaves * 16; }
size_t sk_ws_bytes(int32_t num_tables, int32_t head_dim, int64_t rows = sk_rows()) {
  return (size_t)(sk_cum_bytes(num_tables) + align256(rows * head_dim * 4) + align256(rows * 4));
}

// Compute units of the current device (queried once per device).
int device_cu_count() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  if (cached[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    cached[dev] = n;
  }
  return cached[dev];
}

// Sizes an exact-window geometry needs (see pkv_causal_layout_bounds).
bool window_sizes(int32_t page_size, int64_t pin, int64_t window, const int32_t* block_sizes, int32_t num_blocks,
                  pkv_causal_bounds* out, int64_t* total) {
  if (!is_pow2(page_size) || pin < 0 || window < 0 || !block_sizes) return false;
  if (num_blocks < 1 || num_blocks > kMaxCausalBlocks) return false;
  int64_t sum = 0, biggest = 0;
  for (int i = 0; i < num_blocks; ++i) {
    if (block_sizes[i] < 1) return false;
    sum += block_sizes[i];
    biggest = std::max<int64_t>(biggest, block_sizes[i]);
  }
  const int64_t ps = page_size, pieces = 3 * (ps - 1);
  const int64_t fixed = ceil_div(pin, ps), rolling = ceil_div(window + ps - 1 + sum, ps);
  const int64_t priv = ceil_div(pieces + biggest, ps), width = pin / ps + window / ps + priv;
  if (fixed + rolling > INT32_MAX || width > INT32_MAX || pieces > INT32_MAX) return false;
  out->fixed_pages = (int32_t)fixed;
  out->rolling_pages = (int32_t)rolling;
  out->private_pages = (int32_t)priv;
  out->table_width = (int32_t)width;
  out->list_stride = (int32_t)pieces;
  *total = sum;
  return true;
}

int64_t evicted_tokens(int64_t ps, int64_t pin, int64_t window, int64_t committed) {
  const int64_t first_needed = std::max<int64_t>(0, committed - window - pin);
  return first_needed / ps * ps;
}

}  // namespace

namespace pkv {
// The events of pkv_set_timing_events (process-wide; NULL: off).
static TimingEvents g_timing = {nullptr, nullptr};
TimingEvents timing_events() { return g_timing; }
}  // namespace pkv

extern "C" {

void pkv_set_timing_events(hipEvent_t start, hipEvent_t stop) { pkv::g_timing = {start, stop}; }

const char* pkv_status_string(pkv_status s) {
  switch (s) {
    case PKV_OK: return "ok";
    case PKV_ERR_NULL: return "a required pointer is NULL";
    case PKV_ERR_SHAPE: return "invalid size, stride or count";
    case PKV_ERR_DTYPE: return "unknown dtype";
    case PKV_ERR_UNSUPPORTED: return "no kernel for this head_dim / dtype / page_size combination";
    case PKV_ERR_HIP: return "kernel launch failed";
    case PKV_ERR_ALIGN: return "pointer or stride breaks the required alignment";
    case PKV_ERR_SCRATCH: return "the call needs more scratch than the no-allocation entry point's device array holds";
  }
  return "unknown status";
}

int32_t pkv_abi_version(void) { return kAbiVersion; }

// ---------------------------------------------------------------------------
// The scatter kernel over n_tokens rows, with explicit slots or (table !=
// NULL) in append mode; the widest vector every operand's alignment allows.
static hipError_t launch_scatter_rows(const pkv_pool* pool, const void* src_k, const void* src_v,
                                      int64_t src_tok_stride, int64_t src_head_stride, const int64_t* src_idx,
                                      const int64_t* slots, const int64_t* slots2, int64_t n_tokens,
                                      const int32_t* table, const int32_t* lens, int32_t table_stride,
                                      int32_t q_len, hipStream_t stream) {
  const int es = elem_bytes(pool->dtype);
  const int64_t row_b = (int64_t)pool->head_dim * es;
  int vec = 16;
  while (vec > 1) {
    const bool ok = row_b % vec == 0 && aligned(src_k, vec) && aligned(src_v, vec) && aligned(pool->k, vec) &&
                    aligned(pool->v, vec) && (src_tok_stride * es) % vec == 0 &&
                    (src_head_stride * es) % vec == 0 && (pool->page_stride * es) % vec == 0;
    if (ok) break;
    vec >>= 1;
  }
  ScatterParams p;
  p.src_k = static_cast<const uint8_t*>(src_k);
  p.src_v = static_cast<const uint8_t*>(src_v);
  p.pool_k = static_cast<uint8_t*>(pool->k);
  p.pool_v = static_cast<uint8_t*>(pool->v);
  p.src_idx = src_idx;
  p.slots = slots;
  p.slots2 = slots2;
  p.table = table;
  p.lens = lens;
  p.table_stride = table_stride;
  p.q_len = q_len;
  p.n_tokens = n_tokens;
  p.src_tok_stride_b = src_tok_stride * es;
  p.src_head_stride_b = src_head_stride * es;
  p.page_stride_b = pool->page_stride * es;
  p.row_stride_b = (int64_t)pool->num_kv_heads * row_b;
  p.page_shift = log2i(pool->page_size);
  p.num_kv_heads = pool->num_kv_heads;
  p.vecs_per_row = (int32_t)(row_b / vec);
  return launch_scatter(p, vec, stream);
}

pkv_status pkv_scatter_slots(const pkv_pool* pool, const void* src_k, const void* src_v, int64_t src_tok_stride,
                             int64_t src_head_stride, const int64_t* src_idx, const int64_t* slots,
                             const int64_t* slots2, int64_t n_tokens, hipStream_t stream) {
  pkv_status st = check_pool(pool);
  if (st != PKV_OK) return st;
  if (n_tokens < 0 || src_tok_stride < 0 || src_head_stride < 0) return PKV_ERR_SHAPE;
  if (n_tokens == 0) return PKV_OK;   // empty tensors may carry NULL pointers
  if (!src_k || !src_v || !slots) return PKV_ERR_NULL;
  return launch_scatter_rows(pool, src_k, src_v, src_tok_stride, src_head_stride, src_idx, slots, slots2, n_tokens,
                             nullptr, nullptr, 0, 0, stream) == hipSuccess
             ? PKV_OK
             : PKV_ERR_HIP;
}


// ---------------------------------------------------------------------------
size_t pkv_attn_decode_workspace_bytes(int32_t num_tables, int32_t rows_per_table, int32_t num_q_heads,
                                       int32_t num_kv_heads, int32_t head_dim, int32_t max_kv_len) {
  (void)num_kv_heads;
  if (num_tables <= 0 || rows_per_table <= 0 || num_q_heads <= 0 || head_dim <= 0) return 0;
  const SplitPlan plan = plan_decode(max_kv_len);
  const size_t split = decode_ws_bytes((int64_t)num_tables * rows_per_table, num_q_heads, head_dim, plan.splits);
  const size_t sk = num_tables <= kMaxSkTables ? sk_ws_bytes(num_tables, head_dim) : 0;
  return split > sk ? split : sk;
}

// Decode of num_tables x rows_per_table query rows; with `causal` the rows of
// a table row are the tokens of one step (row i sees len - (n - 1 - i) keys).
// With `scratch` the workspace is the no-allocation entry point's device
// array: the stream-K state is laid out for the launched grid only (2 slots x
// 64 rows per workgroup), and a call whose state would not fit is refused
// with PKV_ERR_SCRATCH instead of running with a smaller split.
static pkv_status decode_call(const pkv_pool* pool, const void* q, pkv_dtype q_dtype, int32_t num_tables,
                              int32_t rows_per_table, int32_t num_q_heads, const int32_t* block_table,
                              int32_t table_stride, const int32_t* kv_lens, int32_t max_kv_len, float sm_scale,
                              void* out, pkv_dtype out_dtype, float* out_lse, void* workspace,
                              size_t workspace_bytes, int32_t causal, hipStream_t stream, bool scratch = false,
                              const void* new_k = nullptr, const void* new_v = nullptr,
                              int64_t new_tok_stride = 0, int64_t new_head_stride = 0) {
  pkv_status st = check_pool(pool);
  if (st != PKV_OK) return st;
  const bool append = new_k != nullptr || new_v != nullptr;
  if (append && (new_tok_stride < 0 || new_head_stride < 0)) return PKV_ERR_SHAPE;
  if (!valid_dtype(q_dtype) || !valid_dtype(out_dtype)) return PKV_ERR_DTYPE;
  if (num_tables < 0 || rows_per_table < 1 || num_q_heads < 1 || table_stride < 1 || max_kv_len < 0 ||
      !(sm_scale > 0.f) || sm_scale > 3.0e38f)
    return PKV_ERR_SHAPE;
  if (num_q_heads % pool->num_kv_heads != 0) return PKV_ERR_SHAPE;
  if ((int64_t)max_kv_len > (int64_t)table_stride * pool->page_size) return PKV_ERR_SHAPE;
  if (num_tables == 0) return PKV_OK;   // empty tensors may carry NULL pointers
  if (!q || !block_table || !kv_lens || !out) return PKV_ERR_NULL;
  if (append && (!new_k || !new_v)) return PKV_ERR_NULL;
  const int D = pool->head_dim;
  if (D != 64 && D != 128) return PKV_ERR_UNSUPPORTED;
  if (pool->page_size < 16) return PKV_ERR_UNSUPPORTED;
  if (q_dtype == PKV_FP8_E4M3FN || out_dtype == PKV_FP8_E4M3FN) return PKV_ERR_UNSUPPORTED;
  const bool use_mfma = q_dtype == PKV_BF16 && pool->dtype != PKV_F32;
  const int es = elem_bytes(pool->dtype);
  if (use_mfma) {
    if (!aligned(pool->k, 16) || !aligned(pool->v, 16) || (pool->page_stride * es) % 16 != 0 || !aligned(q, 16) ||
        !aligned(out, 16))
      return PKV_ERR_ALIGN;
  } else if (!aligned(q, elem_bytes(q_dtype)) || !aligned(out, elem_bytes(out_dtype)) ||
             !aligned(pool->k, es) || !aligned(pool->v, es)) {
    return PKV_ERR_ALIGN;
  }

  if (scratch) {
    // the device array of the no-allocation entry point (looked up once per
    // device, after every argument check)
    hipError_t e = hipSuccess;
    workspace = noalloc_scratch(&e);
    if (!workspace) return PKV_ERR_HIP;
    workspace_bytes = kNoAllocScratchBytes;
  }
  const int64_t rows = (int64_t)num_tables * rows_per_table;
  // Stream-K (balanced persistent grid) when the workspace holds its state.
  const int R = rows_per_table * (num_q_heads / pool->num_kv_heads);
  const int sk_wr = sk_waves_per_worker(R);
  const int sk_rg = (int)ceil_div(ceil_div(R, 16), sk_wr);
  const int64_t sk_positions = (int64_t)num_tables * ceil_div(max_kv_len, 32) * pool->num_kv_heads * sk_rg;
  const int cus = use_mfma ? device_cu_count() : 0;
  // state rows of the stream-K slots: the public layout reserves them for the
  // largest grid; the scratch layout for the grid this device launches
  const int64_t sk_state_rows = scratch ? 128 * (int64_t)std::min(cus, kMaxSkWaves / 4) : sk_rows();
  const bool sk_shape = use_mfma && cus > 0 && num_tables <= kMaxSkTables && sk_positions < (int64_t(1) << 31);
  if (scratch && sk_shape && sk_ws_bytes(num_tables, D, sk_state_rows) > workspace_bytes) return PKV_ERR_SCRATCH;
  const bool use_sk = sk_shape && workspace && aligned(workspace, 256) &&
                      workspace_bytes >= sk_ws_bytes(num_tables, D, sk_state_rows);
  SplitPlan plan = plan_decode(max_kv_len);
  const size_t need = decode_ws_bytes(rows, num_q_heads, D, plan.splits);
  if (scratch && !use_sk && plan.splits > 1 && need > workspace_bytes) return PKV_ERR_SCRATCH;
  if (use_sk || (plan.splits > 1 && (!workspace || workspace_bytes < need || !aligned(workspace, 16)))) {
    plan.splits = 1;
    plan.tiles_per_split = (int)std::max<int64_t>(1, ceil_div(max_kv_len, 32));
  }

  DecodeParams p;
  p.k_pool = pool->k;
  p.v_pool = pool->v;
  p.k_scale = pool->k_scale;
  p.v_scale = pool->v_scale;
  p.q = q;
  p.table = block_table;
  p.kv_lens = kv_lens;
  p.out = out;
  p.out_lse = out_lse;
  p.ws_o = nullptr;
  p.ws_lse = nullptr;
  p.ws_cum = nullptr;
  p.new_k = nullptr;
  p.new_v = nullptr;
  p.new_tok_stride_b = 0;
  p.new_head_stride_b = 0;
  if (append) {
    // the head-parallel stream-K kernel writes the step's tokens itself (16-byte
    // rows and strides); every other path scatters them first, in append mode
    const bool fused = use_sk && sk_head_parallel(sk_wr, sk_rg, pool->num_kv_heads) && aligned(new_k, 16) &&
                       aligned(new_v, 16) && (new_tok_stride * es) % 16 == 0 && (new_head_stride * es) % 16 == 0;
    if (fused) {
      p.new_k = static_cast<const uint8_t*>(new_k);
      p.new_v = static_cast<const uint8_t*>(new_v);
      p.new_tok_stride_b = new_tok_stride * es;
      p.new_head_stride_b = new_head_stride * es;
    } else if (launch_scatter_rows(pool, new_k, new_v, new_tok_stride, new_head_stride, nullptr, nullptr, nullptr,
                                   (int64_t)num_tables * rows_per_table, block_table, kv_lens, table_stride,
                                   rows_per_table, stream) != hipSuccess) {
      return PKV_ERR_HIP;
    }
  }
  if (use_sk) {
    uint8_t* w = static_cast<uint8_t*>(workspace);
    p.ws_cum = reinterpret_cast<int32_t*>(w);
    p.ws_o = reinterpret_cast<float*>(w + sk_cum_bytes(num_tables));
    p.ws_lse = reinterpret_cast<float*>(w + sk_cum_bytes(num_tables) + align256(sk_state_rows * D * 4));
  } else if (plan.splits > 1) {
    p.ws_o = static_cast<float*>(workspace);
    p.ws_lse = p.ws_o + (int64_t)plan.splits * rows * num_q_heads * D;
  }
  p.page_stride = pool->page_stride;
  p.num_pages = pool->num_pages;
  p.page_shift = log2i(pool->page_size);
  p.num_kv_heads = pool->num_kv_heads;
  p.num_tables = num_tables;
  p.rows_per_table = rows_per_table;
  p.num_q_heads = num_q_heads;
  p.group = num_q_heads / pool->num_kv_heads;
  p.table_stride = table_stride;
  p.splits = plan.splits;
  p.tiles_per_split = plan.tiles_per_split;
  p.out_bf16 = out_dtype == PKV_BF16;
  p.n_workers = 0;
  p.row_groups = sk_rg;
  p.head_par = 0;
  p.causal = causal;
  p.write_state = 0;
  p.scale_log2 = sm_scale * 1.4426950408889634f;

  if (use_sk) return launch_decode_sk(p, elem_type(pool->dtype), D, cus, stream) == hipSuccess ? PKV_OK : PKV_ERR_HIP;
  hipError_t e = use_mfma ? launch_decode_mfma(p, elem_type(pool->dtype), D, stream)
                          : launch_decode_valu(p, elem_type(q_dtype), elem_type(pool->dtype), D, stream);
  if (e != hipSuccess) return PKV_ERR_HIP;
  if (plan.splits > 1) {
    MergeParams m;
    m.o_parts = p.ws_o;
    m.lse_parts = p.ws_lse;
    m.out = out;
    m.out_lse = out_lse;
    m.kv_lens = kv_lens;
    m.rows = rows;
    m.num_states = plan.splits;
    m.num_q_heads = num_q_heads;
    m.head_dim = D;
    m.rows_per_table = rows_per_table;
    m.keys_per_state = plan.tiles_per_split * 32;
    m.out_bf16 = out_dtype == PKV_BF16;
    if (launch_merge(m, stream) != hipSuccess) return PKV_ERR_HIP;
  }
  return PKV_OK;
}


pkv_status pkv_attn_decode(const pkv_pool* pool, const void* q, pkv_dtype q_dtype, int32_t num_tables,
                           int32_t rows_per_table, int32_t num_q_heads, const int32_t* block_table,
                           int32_t table_stride, const int32_t* kv_lens, int32_t max_kv_len, float sm_scale,
                           void* out, pkv_dtype out_dtype, float* out_lse, void* workspace, size_t workspace_bytes,
                           hipStream_t stream) {
  return decode_call(pool, q, q_dtype, num_tables, rows_per_table, num_q_heads, block_table, table_stride, kv_lens,
                     max_kv_len, sm_scale, out, out_dtype, out_lse, workspace, workspace_bytes, 0, stream);
}

pkv_status pkv_attn_decode_noalloc(const pkv_pool* pool, const void* q, pkv_dtype q_dtype, int32_t num_tables,
                                   int32_t rows_per_table, int32_t num_q_heads, const int32_t* block_table,
                                   int32_t table_stride, const int32_t* kv_lens, int32_t max_kv_len, float sm_scale,
                                   void* out, pkv_dtype out_dtype, float* out_lse, hipStream_t stream) {
  return decode_call(pool, q, q_dtype, num_tables, rows_per_table, num_q_heads, block_table, table_stride, kv_lens,
                     max_kv_len, sm_scale, out, out_dtype, out_lse, nullptr, 0, 0, stream, true);
}

size_t pkv_attn_decode_shared_prefix_workspace_bytes(int32_t groups, int32_t samples, int32_t q_len,
                                                     int32_t num_q_heads, int32_t head_dim, int32_t max_prefix_len) {
  if (groups < 0 || samples < 1 || q_len < 1 || num_q_heads < 1 || head_dim < 1 || max_prefix_len < 0) return 0;
  const int64_t states = plan_decode(max_prefix_len, kSharedMinSplitTokens).splits + 1;
  const int64_t rows = (int64_t)groups * samples * q_len;
  return (size_t)(states * rows * num_q_heads * (int64_t)(head_dim + 1) * (int64_t)sizeof(float));
}

// One n-sample step; with new_k / new_v the step's tokens are written into
// the tails' last q_len keys first (by the tail workgroups themselves when
// one workgroup covers each (tail, kv head), else by an append-mode scatter).
static pkv_status shared_call(const pkv_pool* pool, const void* q, pkv_dtype q_dtype, int32_t groups,
                              int32_t samples, int32_t q_len, int32_t num_q_heads, const int32_t* prefix_table,
                              int32_t prefix_stride, const int32_t* prefix_lens, int32_t max_prefix_len,
                              const int32_t* tail_table, int32_t tail_stride, const int32_t* tail_lens,
                              int32_t max_tail_len, float sm_scale, void* out, pkv_dtype out_dtype, float* out_lse,
                              void* workspace, size_t workspace_bytes, hipStream_t stream,
                              const void* new_k = nullptr, const void* new_v = nullptr, int64_t new_tok_stride = 0,
                              int64_t new_head_stride = 0) {
  pkv_status st = check_pool(pool);
  if (st != PKV_OK) return st;
  const bool append = new_k != nullptr || new_v != nullptr;
  if (append && (new_tok_stride < 0 || new_head_stride < 0)) return PKV_ERR_SHAPE;
  if (!valid_dtype(q_dtype) || !valid_dtype(out_dtype)) return PKV_ERR_DTYPE;
  if (groups < 0 || samples < 1 || q_len < 1 || num_q_heads < 1 || prefix_stride < 1 || tail_stride < 1 ||
      max_prefix_len < 0 || max_tail_len < 0 || !(sm_scale > 0.f) || sm_scale > 3.0e38f)
    return PKV_ERR_SHAPE;
  if (num_q_heads % pool->num_kv_heads != 0) return PKV_ERR_SHAPE;
  if ((int64_t)max_prefix_len > (int64_t)prefix_stride * pool->page_size ||
      (int64_t)max_tail_len > (int64_t)tail_stride * pool->page_size)
    return PKV_ERR_SHAPE;
  if ((int64_t)groups * samples * q_len > INT32_MAX / 2) return PKV_ERR_SHAPE;
  if (groups == 0) return PKV_OK;   // empty tensors may carry NULL pointers
  if (!q || !prefix_table || !prefix_lens || !tail_table || !tail_lens || !out || !workspace) return PKV_ERR_NULL;
  if (append && (!new_k || !new_v)) return PKV_ERR_NULL;
  const int D = pool->head_dim;
  if (D != 64 && D != 128) return PKV_ERR_UNSUPPORTED;
  if (pool->page_size < 16) return PKV_ERR_UNSUPPORTED;
  if (q_dtype != PKV_BF16 || pool->dtype == PKV_F32 || out_dtype == PKV_FP8_E4M3FN) return PKV_ERR_UNSUPPORTED;
  const int es = elem_bytes(pool->dtype);
  if (!aligned(pool->k, 16) || !aligned(pool->v, 16) || (pool->page_stride * es) % 16 != 0 || !aligned(q, 16) ||
      !aligned(out, 16) || !aligned(workspace, 16))
    return PKV_ERR_ALIGN;
  const size_t need = pkv_attn_decode_shared_prefix_workspace_bytes(groups, samples, q_len, num_q_heads, D,
                                                                    max_prefix_len);
  if (workspace_bytes < need) return PKV_ERR_SHAPE;

  const SplitPlan plan = plan_decode(max_prefix_len, kSharedMinSplitTokens);
  const int64_t rows = (int64_t)groups * samples * q_len;
  const int64_t plane = rows * num_q_heads;
  float* ws_o = static_cast<float*>(workspace);
  float* ws_lse = ws_o + (int64_t)(plan.splits + 1) * plane * D;

  DecodeParams pre;
  pre.k_pool = pool->k;
  pre.v_pool = pool->v;
  pre.k_scale = pool->k_scale;
  pre.v_scale = pool->v_scale;
  pre.q = q;
  pre.table = prefix_table;
  pre.kv_lens = prefix_lens;
  pre.out = nullptr;
  pre.out_lse = nullptr;
  pre.ws_o = ws_o;
  pre.ws_lse = ws_lse;
  pre.ws_cum = nullptr;
  pre.new_k = nullptr;
  pre.new_v = nullptr;
  pre.new_tok_stride_b = 0;
  pre.new_head_stride_b = 0;
  pre.page_stride = pool->page_stride;
  pre.num_pages = pool->num_pages;
  pre.page_shift = log2i(pool->page_size);
  pre.num_kv_heads = pool->num_kv_heads;
  pre.num_tables = groups;
  pre.rows_per_table = samples * q_len;
  pre.num_q_heads = num_q_heads;
  pre.group = num_q_heads / pool->num_kv_heads;
  pre.table_stride = prefix_stride;
  pre.splits = plan.splits;
  pre.tiles_per_split = plan.tiles_per_split;
  pre.out_bf16 = 0;
  pre.n_workers = 0;
  pre.row_groups = 0;
  pre.head_par = 0;
  pre.causal = 0;
  pre.write_state = 1;
  pre.scale_log2 = sm_scale * 1.4426950408889634f;

  DecodeParams tail = pre;
  tail.table = tail_table;
  tail.kv_lens = tail_lens;
  tail.ws_o = ws_o + (int64_t)plan.splits * plane * D;
  tail.ws_lse = ws_lse + (int64_t)plan.splits * plane;
  tail.num_tables = groups * samples;
  tail.rows_per_table = q_len;
  tail.table_stride = tail_stride;
  tail.splits = 1;
  tail.tiles_per_split = (int)std::max<int64_t>(1, ceil_div(max_tail_len, 32));
  tail.causal = 1;
  if (append) {
    // one tail workgroup per (sample, kv head) while its rows fit 64 (4 row
    // blocks): it writes its own tokens; otherwise scatter them first
    const bool fused = (int64_t)q_len * tail.group <= 64 && aligned(new_k, 16) && aligned(new_v, 16) &&
                       (new_tok_stride * es) % 16 == 0 && (new_head_stride * es) % 16 == 0;
    if (fused) {
      tail.new_k = static_cast<const uint8_t*>(new_k);
      tail.new_v = static_cast<const uint8_t*>(new_v);
      tail.new_tok_stride_b = new_tok_stride * es;
      tail.new_head_stride_b = new_head_stride * es;
    } else if (launch_scatter_rows(pool, new_k, new_v, new_tok_stride, new_head_stride, nullptr, nullptr, nullptr,
                                   (int64_t)groups * samples * q_len, tail_table, tail_lens, tail_stride, q_len,
                                   stream) != hipSuccess) {
      return PKV_ERR_HIP;
    }
  }

  if (launch_shared_prefix(pre, tail, elem_type(pool->dtype), D, stream) != hipSuccess) return PKV_ERR_HIP;
  MergeParams m;
  m.o_parts = ws_o;
  m.lse_parts = ws_lse;
  m.out = out;
  m.out_lse = out_lse;
  m.kv_lens = nullptr;
  m.rows = rows;
  m.num_states = plan.splits + 1;
  m.num_q_heads = num_q_heads;
  m.head_dim = D;
  m.rows_per_table = 1;
  m.keys_per_state = 1;
  m.out_bf16 = out_dtype == PKV_BF16;
  return launch_merge(m, stream) == hipSuccess ? PKV_OK : PKV_ERR_HIP;
}

pkv_status pkv_attn_decode_shared_prefix(const pkv_pool* pool, const void* q, pkv_dtype q_dtype, int32_t groups,
                                         int32_t samples, int32_t q_len, int32_t num_q_heads,
                                         const int32_t* prefix_table, int32_t prefix_stride,
                                         const int32_t* prefix_lens, int32_t max_prefix_len,
                                         const int32_t* tail_table, int32_t tail_stride, const int32_t* tail_lens,
                                         int32_t max_tail_len, float sm_scale, void* out, pkv_dtype out_dtype,
                                         float* out_lse, void* workspace, size_t workspace_bytes,
                                         hipStream_t stream) {
  return shared_call(pool, q, q_dtype, groups, samples, q_len, num_q_heads, prefix_table, prefix_stride, prefix_lens,
                     max_prefix_len, tail_table, tail_stride, tail_lens, max_tail_len, sm_scale, out, out_dtype,
                     out_lse, workspace, workspace_bytes, stream);
}

pkv_status pkv_attn_decode_shared_prefix_append(const pkv_pool* pool, const void* new_k, const void* new_v,
                                                int64_t new_tok_stride, int64_t new_head_stride, const void* q,
                                                pkv_dtype q_dtype, int32_t groups, int32_t samples, int32_t q_len,
                                                int32_t num_q_heads, const int32_t* prefix_table,
                                                int32_t prefix_stride, const int32_t* prefix_lens,
                                                int32_t max_prefix_len, const int32_t* tail_table,
                                                int32_t tail_stride, const int32_t* tail_lens, int32_t max_tail_len,
                                                float sm_scale, void* out, pkv_dtype out_dtype, float* out_lse,
                                                void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (groups > 0 && !new_k && !new_v) {   // (one of the two NULL is caught by shared_call)
    const pkv_status st = check_pool(pool);
    return st != PKV_OK ? st : PKV_ERR_NULL;
  }
  return shared_call(pool, q, q_dtype, groups, samples, q_len, num_q_heads, prefix_table, prefix_stride, prefix_lens,
                     max_prefix_len, tail_table, tail_stride, tail_lens, max_tail_len, sm_scale, out, out_dtype,
                     out_lse, workspace, workspace_bytes, stream, new_k, new_v, new_tok_stride, new_head_stride);
}

pkv_status pkv_attn_decode_step(const pkv_pool* pool, const void* q, pkv_dtype q_dtype, int32_t num_tables,
                                int32_t q_len, int32_t num_q_heads, const int32_t* block_table,
                                int32_t table_stride, const int32_t* kv_lens, int32_t max_kv_len, float sm_scale,
                                void* out, pkv_dtype out_dtype, float* out_lse, void* workspace,
                                size_t workspace_bytes, hipStream_t stream) {
  return decode_call(pool, q, q_dtype, num_tables, q_len, num_q_heads, block_table, table_stride, kv_lens,
                     max_kv_len, sm_scale, out, out_dtype, out_lse, workspace, workspace_bytes, 1, stream);
}

pkv_status pkv_attn_decode_append(const pkv_pool* pool, const void* new_k, const void* new_v,
                                  int64_t new_tok_stride, int64_t new_head_stride, const void* q, pkv_dtype q_dtype,
                                  int32_t num_tables, int32_t q_len, int32_t num_q_heads, const int32_t* block_table,
                                  int32_t table_stride, const int32_t* kv_lens, int32_t max_kv_len, float sm_scale,
                                  void* out, pkv_dtype out_dtype, float* out_lse, void* workspace,
                                  size_t workspace_bytes, hipStream_t stream) {
  if (num_tables > 0 && !new_k && !new_v) {   // (one of the two NULL is caught by decode_call)
    const pkv_status st = check_pool(pool);
    return st != PKV_OK ? st : PKV_ERR_NULL;
  }
  return decode_call(pool, q, q_dtype, num_tables, q_len, num_q_heads, block_table, table_stride, kv_lens,
                     max_kv_len, sm_scale, out, out_dtype, out_lse, workspace, workspace_bytes, 1, stream, false,
                     new_k, new_v, new_tok_stride, new_head_stride);
}
// ---------------------------------------------------------------------------
size_t pkv_attn_prefill_workspace_bytes(int32_t batch, int32_t s_q, int32_t num_q_heads, int32_t num_kv_heads,
                                        int32_t head_dim, int32_t max_keys) {
  (void)head_dim; (void)max_keys;
  if (batch <= 0 || s_q <= 0 || num_q_heads <= 0 || num_kv_heads <= 0 || num_q_heads % num_kv_heads != 0) return 0;
  // Two partial-state slots per workgroup of the persistent grid, needed only
  // when some XCD splits its leftover units along the keys.  Without a device
  // to ask for its CU count, the largest grid is assumed.
  const int cus = device_cu_count();
  if (cus <= 0) return (size_t)(2 * (int64_t)kMaxPrefillWorkgroups * (int64_t)prefill_slot_bytes());
  const int grid = prefill_grid(cus);
  if (prefill_tail_units(batch, s_q, num_q_heads, num_kv_heads, grid) == 0) return 0;
  return (size_t)(2 * (int64_t)grid * (int64_t)prefill_slot_bytes());
}

// Block-causal prefill; with q_offsets (device int32 [batch + 1]) batch entry
// b's rows are q_offsets[b] .. q_offsets[b + 1] - 1 of q / out / lse (ragged),
// else b * s_q .. b * s_q + s_q - 1 (padded).
static pkv_status prefill_call(const pkv_pool* pool, const void* q, pkv_dtype q_dtype, int64_t q_tok_stride,
                               int64_t q_head_stride, int32_t batch, int32_t s_q, int32_t num_q_heads,
                               const int32_t* q_offsets, const int32_t* block_table, int32_t table_stride,
                               const int32_t* n_ctx, const int32_t* seq_len, int32_t causal_block_size,
                               int32_t max_keys, float sm_scale, void* out, pkv_dtype out_dtype, float* out_lse,
                               void* workspace, size_t workspace_bytes, bool ragged, hipStream_t stream) {
  pkv_status st = check_pool(pool);
  if (st != PKV_OK) return st;
  if (!valid_dtype(q_dtype) || !valid_dtype(out_dtype)) return PKV_ERR_DTYPE;
  if (batch < 0 || s_q < 0 || num_q_heads < 1 || table_stride < 1 || max_keys < 0 || causal_block_size < 0 ||
      q_tok_stride < 0 || q_head_stride < 0 || !(sm_scale > 0.f) || sm_scale > 3.0e38f)
    return PKV_ERR_SHAPE;
  if (num_q_heads % pool->num_kv_heads != 0) return PKV_ERR_SHAPE;
  if ((int64_t)max_keys > (int64_t)table_stride * pool->page_size) return PKV_ERR_SHAPE;
  if (batch == 0 || s_q == 0) return PKV_OK;   // empty tensors may carry NULL pointers
  if (!q || !block_table || !n_ctx || !seq_len || !out || (ragged && !q_offsets)) return PKV_ERR_NULL;
  const int D = pool->head_dim;
  if (D != 64 && D != 128) return PKV_ERR_UNSUPPORTED;
  if (pool->page_size < 16) return PKV_ERR_UNSUPPORTED;
  if (q_dtype != PKV_BF16 || pool->dtype == PKV_F32 || out_dtype == PKV_FP8_E4M3FN) return PKV_ERR_UNSUPPORTED;
  const bool fp8 = pool->dtype == PKV_FP8_E4M3FN;
  if (fp8 && (D != 128 || pool->page_size < 32)) return PKV_ERR_UNSUPPORTED;
  if (!aligned(pool->k, 16) || !aligned(pool->v, 16) || (pool->page_stride * elem_bytes(pool->dtype)) % 16 != 0 ||
      !aligned(q, 16) ||
      (q_tok_stride * 2) % 16 != 0 || (q_head_stride * 2) % 16 != 0 || !aligned(out, 16) ||
      (ragged && !aligned(q_offsets, 4)))
    return PKV_ERR_ALIGN;

  PrefillParams p;
  p.k_pool = pool->k;
  p.v_pool = pool->v;
  p.k_scale = pool->k_scale;
  p.v_scale = pool->v_scale;
  p.kv_fp8 = fp8;
  p.q = static_cast<const uint16_t*>(q);
  p.table = block_table;
  p.n_ctx = n_ctx;
  p.seq_len = seq_len;
  p.q_offsets = ragged ? q_offsets : nullptr;
  p.out = out;
  p.out_lse = out_lse;
  p.page_stride = pool->page_stride;
  p.q_tok_stride = q_tok_stride;
  p.q_head_stride = q_head_stride;
  p.page_shift = log2i(pool->page_size);
  p.num_kv_heads = pool->num_kv_heads;
  p.batch = batch;
  p.s_q = s_q;
  p.num_q_heads = num_q_heads;
  p.group = num_q_heads / pool->num_kv_heads;
  p.table_stride = table_stride;
  p.causal_block_size = causal_block_size;
  p.q_tiles = 0;
  p.out_bf16 = out_dtype == PKV_BF16;
  p.scale_log2 = sm_scale * 1.4426950408889634f;
  p.ws_o = nullptr;
  const int cus = device_cu_count();
  const size_t need = pkv_attn_prefill_workspace_bytes(batch, s_q, num_q_heads, pool->num_kv_heads, D, max_keys);
  if (need > 0 && cus > 0 && workspace && aligned(workspace, 256) && workspace_bytes >= need)
    p.ws_o = static_cast<float*>(workspace);
  return launch_prefill_mfma(p, D, cus, stream) == hipSuccess ? PKV_OK : PKV_ERR_HIP;
}

pkv_status pkv_attn_prefill_block_causal(const pkv_pool* pool, const void* q, pkv_dtype q_dtype,
                                         int64_t q_tok_stride, int64_t q_head_stride, int32_t batch, int32_t s_q,
                                         int32_t num_q_heads, const int32_t* block_table, int32_t table_stride,
                                         const int32_t* n_ctx, const int32_t* seq_len, int32_t causal_block_size,
                                         int32_t max_keys, float sm_scale, void* out, pkv_dtype out_dtype,
                                         float* out_lse, void* workspace, size_t workspace_bytes,
                                         hipStream_t stream) {
  return prefill_call(pool, q, q_dtype, q_tok_stride, q_head_stride, batch, s_q, num_q_heads, nullptr, block_table,
                      table_stride, n_ctx, seq_len, causal_block_size, max_keys, sm_scale, out, out_dtype, out_lse,
                      workspace, workspace_bytes, false, stream);
}

pkv_status pkv_attn_prefill_block_causal_ragged(const pkv_pool* pool, const void* q, pkv_dtype q_dtype,
                                                int64_t q_tok_stride, int64_t q_head_stride, int32_t batch,
                                                int32_t max_rows, int32_t num_q_heads, const int32_t* q_offsets,
                                                const int32_t* block_table, int32_t table_stride,
                                                const int32_t* n_ctx, const int32_t* seq_len,
                                                int32_t causal_block_size, int32_t max_keys, float sm_scale,
                                                void* out, pkv_dtype out_dtype, float* out_lse, void* workspace,
                                                size_t workspace_bytes, hipStream_t stream) {
  return prefill_call(pool, q, q_dtype, q_tok_stride, q_head_stride, batch, max_rows, num_q_heads, q_offsets,
                      block_table, table_stride, n_ctx, seq_len, causal_block_size, max_keys, sm_scale, out,
                      out_dtype, out_lse, workspace, workspace_bytes, true, stream);
}

// ---------------------------------------------------------------------------
pkv_status pkv_merge_states(const float* o_parts, const float* lse_parts, int32_t num_states, int64_t rows,
                            int32_t num_q_heads, int32_t head_dim, void* out, pkv_dtype out_dtype, float* out_lse,
                            hipStream_t stream) {
  if (!valid_dtype(out_dtype)) return PKV_ERR_DTYPE;
  if (num_states < 1 || rows < 0 || num_q_heads < 1 || head_dim < 4 || head_dim % 4 != 0) return PKV_ERR_SHAPE;
  if (out_dtype == PKV_FP8_E4M3FN) return PKV_ERR_UNSUPPORTED;
  if (rows == 0) return PKV_OK;   // empty tensors may carry NULL pointers
  if (!o_parts || !lse_parts || !out) return PKV_ERR_NULL;
  if (!aligned(o_parts, 16) || !aligned(out, out_dtype == PKV_F32 ? 16 : 8)) return PKV_ERR_ALIGN;
  MergeParams m;
  m.o_parts = o_parts;
  m.lse_parts = lse_parts;
  m.out = out;
  m.out_lse = out_lse;
  m.kv_lens = nullptr;
  m.rows = rows;
  m.num_states = num_states;
  m.num_q_heads = num_q_heads;
  m.head_dim = head_dim;
  m.rows_per_table = 1;
  m.keys_per_state = 1;
  m.out_bf16 = out_dtype == PKV_BF16;
  return launch_merge(m, stream) == hipSuccess ? PKV_OK : PKV_ERR_HIP;
}


// ---------------------------------------------------------------------------
pkv_status pkv_rotate_rows(void* data, int64_t rows, int64_t cols, int64_t row_stride, int32_t elem_size,
                           int64_t shift, hipStream_t stream) {
  if (rows < 0 || cols < 0 || row_stride < cols) return PKV_ERR_SHAPE;
  if (elem_size != 1 && elem_size != 2 && elem_size != 4 && elem_size != 8 && elem_size != 16)
    return PKV_ERR_UNSUPPORTED;
  if (rows == 0 || cols <= 1) return PKV_OK;   // nothing moves; empty tensors may carry NULL pointers
  const int64_t s = ((shift % cols) + cols) % cols;
  if (s == 0) return PKV_OK;
  if (!data) return PKV_ERR_NULL;
  if (!aligned(data, elem_size)) return PKV_ERR_ALIGN;
  RotateParams p;
  p.data = static_cast<uint8_t*>(data);
  p.rows = rows;
  p.cols = cols;
  p.row_stride_b = row_stride * elem_size;
  p.shift = s;
  return launch_rotate(p, elem_size, stream) == hipSuccess ? PKV_OK : PKV_ERR_HIP;
}

// ---------------------------------------------------------------------------
pkv_status pkv_copy_slots(const pkv_pool* pool, int32_t num_layers, int64_t layer_stride, const int64_t* src_slots,
                          const int64_t* dst_slots, int64_t n, hipStream_t stream) {
  pkv_status st = check_pool(pool);
  if (st != PKV_OK) return st;
  if (n < 0 || num_layers < 1 || layer_stride < 0) return PKV_ERR_SHAPE;
  if (num_layers > 1 && layer_stride < pool->num_pages * pool->page_stride) return PKV_ERR_SHAPE;
  if (n == 0) return PKV_OK;   // empty tensors may carry NULL pointers
  if (!src_slots || !dst_slots) return PKV_ERR_NULL;
  const int es = elem_bytes(pool->dtype);
  const int64_t row_b = (int64_t)pool->num_kv_heads * pool->head_dim * es;
  int vec = 16;
  while (vec > 1) {
    const bool ok = row_b % vec == 0 && aligned(pool->k, vec) && aligned(pool->v, vec) &&
                    (pool->page_stride * es) % vec == 0 && (layer_stride * es) % vec == 0;
    if (ok) break;
    vec >>= 1;
  }
  CopySlotsParams p;
  p.pool_k = static_cast<uint8_t*>(pool->k);
  p.pool_v = static_cast<uint8_t*>(pool->v);
  p.src = src_slots;
  p.dst = dst_slots;
  p.n = n;
  p.layer_stride_b = layer_stride * es;
  p.page_stride_b = pool->page_stride * es;
  p.row_b = row_b;
  p.page_shift = log2i(pool->page_size);
  p.num_layers = num_layers;
  p.vecs_per_row = (int32_t)(row_b / vec);
  return launch_copy_slots(p, vec, stream) == hipSuccess ? PKV_OK : PKV_ERR_HIP;
}

// ---------------------------------------------------------------------------
pkv_status pkv_causal_layout_bounds(int32_t page_size, int64_t pin_tokens, int64_t window_tokens,
                                    const int32_t* block_sizes, int32_t num_blocks, pkv_causal_bounds* bounds) {
  if (!block_sizes || !bounds) return PKV_ERR_NULL;
  int64_t total = 0;
  return window_sizes(page_size, pin_tokens, window_tokens, block_sizes, num_blocks, bounds, &total) ? PKV_OK
                                                                                                    : PKV_ERR_SHAPE;
}

int64_t pkv_window_evicted_tokens(int32_t page_size, int64_t pin_tokens, int64_t window_tokens, int64_t committed) {
  if (!is_pow2(page_size) || pin_tokens < 0 || window_tokens < 0 || committed < 0) return -1;
  return evicted_tokens(page_size, pin_tokens, window_tokens, committed);
}

pkv_status pkv_causal_layout(const int32_t* table, int32_t table_len, const int32_t* private_pages,
                             int32_t private_stride, int32_t page_size, int64_t pin_tokens, int64_t window_tokens,
                             int64_t committed, int64_t evicted, const int32_t* block_sizes, int32_t num_blocks,
                             int32_t* block_tables, int32_t table_width, int32_t* n_ctx, int32_t* seq_len,
                             int64_t* stage_slots, int64_t* stage_slots2, int64_t* commit_src, int64_t* commit_dst,
                             int64_t* current_src, int64_t* current_dst, int32_t list_stride, hipStream_t stream) {
  if (!block_sizes) return PKV_ERR_NULL;
  pkv_causal_bounds need;
  int64_t total = 0;
  if (!window_sizes(page_size, pin_tokens, window_tokens, block_sizes, num_blocks, &need, &total))
    return PKV_ERR_SHAPE;
  if (!table || !private_pages || !block_tables || !n_ctx || !seq_len || !stage_slots || !stage_slots2)
    return PKV_ERR_NULL;
  if (list_stride > 0 && (!commit_src || !commit_dst || !current_src || !current_dst)) return PKV_ERR_NULL;
  const int64_t ps = page_size;
  if (committed < 0 || evicted < 0 || evicted % ps != 0) return PKV_ERR_SHAPE;
  if (evicted > evicted_tokens(ps, pin_tokens, window_tokens, committed)) return PKV_ERR_SHAPE;
  // every staged key must have a page in the table
  const int64_t n_fixed = need.fixed_pages, last = committed + total - 1;
  if (table_len < n_fixed) return PKV_ERR_SHAPE;
  if (last >= pin_tokens && (last - pin_tokens - evicted) / ps >= table_len - n_fixed) return PKV_ERR_SHAPE;
  if (private_stride < need.private_pages || table_width < need.table_width || list_stride < need.list_stride)
    return PKV_ERR_SHAPE;
  if (committed + total > INT32_MAX) return PKV_ERR_SHAPE;
  LayoutParams p;
  p.table = table;
  p.priv = private_pages;
  p.priv_stride = private_stride;
  p.n_fixed = (int32_t)n_fixed;
  p.ps_shift = log2i(ps);
  p.num_blocks = num_blocks;
  p.pin = pin_tokens;
  p.window = window_tokens;
  p.committed = committed;
  p.evicted = evicted;
  p.block_start[0] = committed;
  for (int i = 0; i < num_blocks; ++i) p.block_start[i + 1] = p.block_start[i] + block_sizes[i];
  for (int i = num_blocks + 1; i <= kMaxCausalBlocks; ++i) p.block_start[i] = p.block_start[num_blocks];
  p.block_tables = block_tables;
  p.table_width = table_width;
  p.list_stride = list_stride;
  p.n_ctx = n_ctx;
  p.seq_len = seq_len;
  p.stage_slots = stage_slots;
  p.stage_slots2 = stage_slots2;
  p.commit_src = commit_src;
  p.commit_dst = commit_dst;
  p.current_src = current_src;
  p.current_dst = current_dst;
  return launch_causal_layout(p, stream) == hipSuccess ? PKV_OK : PKV_ERR_HIP;
}

// ---------------------------------------------------------------------------
pkv_status pkv_xcd_ids(int32_t* out, int32_t num_workgroups, int32_t threads, hipStream_t stream) {
  if (num_workgroups < 0 || threads < 64 || threads > 1024 || threads % 64 != 0) return PKV_ERR_SHAPE;
  if (num_workgroups == 0) return PKV_OK;
  if (!out) return PKV_ERR_NULL;
  if (!aligned(out, 4)) return PKV_ERR_ALIGN;
  return launch_xcd_ids(out, num_workgroups, threads, stream) == hipSuccess ? PKV_OK : PKV_ERR_HIP;
}

pkv_status pkv_check_slots(const pkv_pool* pool, const int64_t* slots, int64_t n, int32_t* bad, hipStream_t stream) {
  pkv_status st = check_pool(pool);
  if (st != PKV_OK) return st;
  if (n < 0) return PKV_ERR_SHAPE;
  if (!bad || (n > 0 && !slots)) return PKV_ERR_NULL;
  const int64_t capacity = pool->num_pages * (int64_t)pool->page_size;
  return launch_check_slots(slots, n, capacity, bad, stream) == hipSuccess ? PKV_OK : PKV_ERR_HIP;
}

pkv_status pkv_check_tables(const pkv_pool* pool, const int32_t* block_table, int32_t table_stride,
                            const int32_t* kv_lens, int32_t num_tables, int32_t* bad, hipStream_t stream) {
  pkv_status st = check_pool(pool);
  if (st != PKV_OK) return st;
  if (num_tables < 0 || table_stride < 1) return PKV_ERR_SHAPE;
  if (!bad || (num_tables > 0 && (!block_table || !kv_lens))) return PKV_ERR_NULL;
  return launch_check_tables(block_table, table_stride, kv_lens, num_tables, log2i(pool->page_size),
                             pool->num_pages, bad, stream) == hipSuccess
             ? PKV_OK
             : PKV_ERR_HIP;
}

}  // extern "C"
