// Internal launch parameters and launchers of libpkv.  Host code validates the
// public arguments (pkv_api.hip) and then fills these plain structs, which the
// kernels take by value.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pkv.h"

namespace pkv {

enum ElemType : int { kF32 = 0, kBF16 = 1, kFP8 = 2 };

// Stream-K decode limits: table rows whose prefix sums fit LDS, and partial
// state rows in the workspace (2 slots x 16 rows per wave of every worker).
constexpr int kMaxSkTables = 8192;
constexpr int kMaxSkWaves = 4096;

// Device scratch of the no-allocation decode entry point (one array per GPU,
// file scope in noalloc.hip): the stream-K state of a grid of one workgroup
// per CU (2 slots x 64 rows per workgroup, 128 dims, LSE, and the prefix sums
// of up to kMaxSkTables rows) fits for up to 340 CUs.
constexpr size_t kNoAllocScratchBytes = size_t(24) << 20;
// Device address of that array on the current device (looked up once per
// device with hipGetSymbolAddress); NULL, with *err set, on failure.
void* noalloc_scratch(hipError_t* err);

// Prefill: workgroups of the persistent grid (2 partial-state slots each) and
// the most leftover units an XCD splits along the keys.
constexpr int kMaxPrefillWorkgroups = 512;
constexpr int kMaxTailUnits = 64;

struct ScatterParams {
  const uint8_t* src_k;
  const uint8_t* src_v;
  uint8_t* pool_k;
  uint8_t* pool_v;
  const int64_t* src_idx;   // nullable
  const int64_t* slots;     // NULL in append mode
  const int64_t* slots2;    // nullable
  // append mode (table != NULL): token x = t q_len + j goes to logical key
  // lens[t] - q_len + j of table row t (skipped when that key is negative)
  const int32_t* table;
  const int32_t* lens;
  int32_t table_stride;
  int32_t q_len;
  int64_t n_tokens;
  int64_t src_tok_stride_b;   // bytes
  int64_t src_head_stride_b;  // bytes
  int64_t page_stride_b;      // bytes
  int64_t row_stride_b;       // bytes between pool rows of one page (= Hkv * D * esize)
  int32_t page_shift;         // log2(page_size)
  int32_t num_kv_heads;
  int32_t vecs_per_row;       // head_dim * esize / vec_bytes
};

// One decode problem: rows (t, i, h) of q attend to the first kv_lens[t] logical keys of table row t.
struct DecodeParams {
  const void* k_pool;
  const void* v_pool;
  const float* k_scale;       // fp8 only
  const float* v_scale;
  const void* q;
  const int32_t* table;
  const int32_t* kv_lens;
  void* out;
  float* out_lse;             // nullable
  float* ws_o;                // [splits, T, n, Hq, D] when splits > 1
  float* ws_lse;              // [splits, T, n, Hq]
  int32_t* ws_cum;            // stream-K: [T + 1] prefix sums of tiles per table row
  // nullable: the step's tokens [T * rows_per_table, Hkv, D] (pool element
  // type, 16-byte aligned rows and strides), written into the row's last
  // rows_per_table keys, before they are read, by the workgroup that alone
  // reads them (head-parallel stream-K decode; n-sample tails)
  const uint8_t* new_k;
  const uint8_t* new_v;
  int64_t new_tok_stride_b;
  int64_t new_head_stride_b;
  int64_t page_stride;        // elements
  int32_t page_shift;
  int32_t num_kv_heads;
  int32_t num_tables;
  int32_t rows_per_table;     // n
  int32_t num_q_heads;
  int32_t group;              // Hq / Hkv
  int32_t table_stride;
  int32_t splits;             // cross-workgroup key splits
  int32_t tiles_per_split;    // 32-key tiles per split
  int32_t out_bf16;
  int32_t n_workers;          // stream-K workers (set by the launcher)
  int32_t row_groups;         // stream-K: row groups per (table row, kv head)
  int32_t head_par;           // stream-K, one 16-row block per unit: a workgroup's 4 waves take
                              // 4 kv heads of the same keys (set by the launcher)
  int32_t causal;             // rows of a table row are a step's tokens: row i sees len - (n - 1 - i) keys
  int32_t write_state;        // always leave the normalised state of split s in ws_o / ws_lse (empty too)
  float scale_log2;           // sm_scale * log2(e)
  int64_t num_pages;          // pages in the pool (page ids read ahead of the lengths are clamped below it)
};

struct MergeParams {
  const float* o_parts;       // [N, rows, Hq, D]
  const float* lse_parts;     // [N, rows, Hq]
  void* out;
  float* out_lse;             // nullable
  const int32_t* kv_lens;     // nullable: decode-split mode (valid states per table row)
  int64_t rows;
  int32_t num_states;
  int32_t num_q_heads;
  int32_t head_dim;
  int32_t rows_per_table;     // decode-split mode: rows per table row
  int32_t keys_per_state;     // decode-split mode: keys covered by one state
  int32_t out_bf16;
};

struct PrefillParams {
  const void* k_pool;
  const void* v_pool;
  const float* k_scale;       // fp8 pools: [num_pages, num_kv_heads]
  const float* v_scale;
  const uint16_t* q;          // bf16
  const int32_t* table;
  const int32_t* n_ctx;
  const int32_t* seq_len;
  const int32_t* q_offsets;   // NULL: entry b's rows are b * s_q ..; else [batch + 1] row offsets
  void* out;
  float* out_lse;
  float* ws_o;                // stream-K partial states (NULL: leftover units run whole)
  int64_t page_stride;
  int64_t q_tok_stride;
  int64_t q_head_stride;
  int32_t page_shift;
  int32_t num_kv_heads;
  int32_t batch;
  int32_t s_q;
  int32_t num_q_heads;
  int32_t group;
  int32_t table_stride;
  int32_t causal_block_size;
  int32_t q_tiles;            // ceil(s_q / q tile rows)
  int32_t out_bf16;
  int32_t kv_fp8;             // K/V e4m3fn (head_dim 128, page_size >= 32)
  float scale_log2;
};

// In-place rotation of rows: element c takes the old element (c + shift) mod cols.
struct RotateParams {
  uint8_t* data;
  int64_t rows;
  int64_t cols;
  int64_t row_stride_b;       // bytes between rows
  int64_t shift;              // normalised to 1 .. cols - 1
};

// Pool-to-pool copy of whole key rows (all heads, K and V) in every layer.
struct CopySlotsParams {
  uint8_t* pool_k;
  uint8_t* pool_v;
  const int64_t* src;
  const int64_t* dst;
  int64_t n;
  int64_t layer_stride_b;     // bytes between layers
  int64_t page_stride_b;      // bytes between pages
  int64_t row_b;              // bytes of one key row of a page (= Hkv * D * esize)
  int32_t page_shift;
  int32_t num_layers;
  int32_t vecs_per_row;       // row_b / vec_bytes
};

// Exact-window per-block layout (one workgroup per causal block).
constexpr int kMaxCausalBlocks = 64;
struct LayoutParams {
  const int32_t* table;       // [n_fixed + rolling pages]
  const int32_t* priv;        // [num_blocks, priv_stride]
  int32_t priv_stride;
  int32_t n_fixed;
  int32_t ps_shift;
  int32_t num_blocks;
  int64_t pin, window, committed, evicted;
  int64_t block_start[kMaxCausalBlocks + 1];   // committed + prefix sums of the block sizes
  int32_t* block_tables;
  int32_t table_width;
  int32_t list_stride;
  int32_t* n_ctx;
  int32_t* seq_len;
  int64_t* stage_slots;
  int64_t* stage_slots2;
  int64_t* commit_src;
  int64_t* commit_dst;
  int64_t* current_src;
  int64_t* current_dst;
};

// Measurement hook (pkv_set_timing_events): the events a call's main kernel
// is launched with; both NULL when the hook is off.
struct TimingEvents {
  hipEvent_t start;
  hipEvent_t stop;
};
TimingEvents timing_events();

}  // namespace pkv

// Launch of a call's main kernel.  With the hook on it goes through
// hipExtLaunchKernel, whose events take the kernel dispatch's own start and
// end times; otherwise it is a plain launch.
#define PKV_LAUNCH_MAIN(kernel, grid, block, smem, stream, ...)                                            \
  do {                                                                                                     \
    const ::pkv::TimingEvents ev_ = ::pkv::timing_events();                                                \
    if (ev_.start || ev_.stop)                                                                             \
      hipExtLaunchKernelGGL(kernel, grid, block, smem, stream, ev_.start, ev_.stop, 0u, __VA_ARGS__);      \
    else                                                                                                   \
      hipLaunchKernelGGL(kernel, grid, block, smem, stream, __VA_ARGS__);                                  \
  } while (0)

namespace pkv {

// Launchers: return hipGetLastError() of their launch.
hipError_t launch_scatter(const ScatterParams& p, int vec_bytes, hipStream_t stream);
// Whether the stream-K decode runs its head-parallel kernel (one 16-row
// block per unit, kv heads in quads), the one that can write a step's tokens.
inline bool sk_head_parallel(int waves_per_worker, int row_groups, int num_kv_heads) {
  return waves_per_worker == 1 && row_groups == 1 && num_kv_heads % 4 == 0;
}
hipError_t launch_decode_mfma(const DecodeParams& p, ElemType kv, int head_dim, hipStream_t stream);
int sk_waves_per_worker(int rows_per_unit);
hipError_t launch_decode_sk(const DecodeParams& p, ElemType kv, int head_dim, int sm_count, hipStream_t stream);
hipError_t launch_decode_valu(const DecodeParams& p, ElemType q, ElemType kv, int head_dim, hipStream_t stream);
// n-sample step: one launch of every (prefix split, kv head, group, row group)
// and (tail, kv head, row group) workgroup, each leaving its state.
hipError_t launch_shared_prefix(const DecodeParams& pre, const DecodeParams& tail, ElemType kv, int head_dim,
                                hipStream_t stream);
hipError_t launch_merge(const MergeParams& p, hipStream_t stream);
hipError_t launch_prefill_mfma(const PrefillParams& p, int head_dim, int sm_count, hipStream_t stream);
// The fp8 K/V prefill kernel alone on a grid of `grid` workgroups (prefill_fp8.hip).
hipError_t launch_prefill_kernel_fp8(const PrefillParams& p, int grid, hipStream_t stream);
int prefill_grid(int sm_count);
int prefill_tail_units(int32_t batch, int32_t s_q, int32_t num_q_heads, int32_t num_kv_heads, int grid);
hipError_t launch_rotate(const RotateParams& p, int elem_size, hipStream_t stream);
hipError_t launch_copy_slots(const CopySlotsParams& p, int vec_bytes, hipStream_t stream);
hipError_t launch_causal_layout(const LayoutParams& p, hipStream_t stream);
hipError_t launch_xcd_ids(int32_t* out, int32_t num_workgroups, int32_t threads, hipStream_t stream);
hipError_t launch_check_slots(const int64_t* slots, int64_t n, int64_t capacity, int32_t* bad, hipStream_t stream);
hipError_t launch_check_tables(const int32_t* table, int32_t stride, const int32_t* lens, int32_t rows,
                               int32_t page_shift, int64_t num_pages, int32_t* bad, hipStream_t stream);
int64_t prefill_units(int32_t batch, int32_t s_q, int32_t num_q_heads);
size_t prefill_slot_bytes();

}  // namespace pkv
