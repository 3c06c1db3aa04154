// Exact-window per-block layout.
//
// "Paged causal K/V cache and cached attention for VisualGen", Description /
// Cache: a table row can start a key sequence only at a page boundary, so at
// commit one kernel reads the sequence's page table and rewrites, in place,
// every per-block tensor the forwards read: each causal block's row (its
// fully visible pages, then private pages holding the visible keys of the
// partly visible pages and then the block's own tokens), its key counts, the
// slots the staged tokens are written to, and the two copy lists that fill
// the private pages (committed keys, copied at commit; earlier blocks' staged
// keys, copied after every forward's scatter).  The review thread on the
// private regions fixes their sizes: at most three partly visible pages per
// block, so at most 3 (page_size - 1) copied keys.
//
// Sequence geometry: logical key x < pin is in the fixed region, on table
// entry x / ps; the rolling region (x >= pin) starts on a page of its own and
// has had `evicted` tokens (whole pages) rotated out, so rolling key x is on
// table entry F + (x - pin - evicted) / ps, F = ceil(pin / ps).  A causal
// block [s, e) sees [0, pin), [max(pin, s - window), s) and itself.
//
// One workgroup per causal block.  The visible keys before the block are at
// most three ranges (fixed tail, window-start page, start page) around the
// whole pages, so a block's layout is a handful of integer ranges computed
// once per workgroup; the threads then write row entries, list entries and
// staged slots independently.  Page size is a power of two: page and offset
// are a shift and a mask.
#include "pkv_device.hpp"
#include "pkv_internal.hpp"

namespace pkv {

namespace {

constexpr int kLayoutThreads = 256;

struct BlockPlan {
  int64_t s, e;               // the block's own keys
  int64_t a0, a_len;          // fixed-region piece [a0, a0 + a_len)
  int64_t b0, b_len;          // window-start piece
  int64_t c0, c_len;          // start-page piece
  int64_t q0;                 // first whole rolling page (rolling page index)
  int32_t n_fixed_full, n_roll_full;
  int64_t pieces, committed_pieces;
  bool direct;                // own keys read from their own pages
  int64_t own_q0, own_pages;  // direct: rolling pages of the own keys
};

__device__ __forceinline__ int64_t clamp_len(int64_t lo, int64_t hi) { return hi > lo ? hi - lo : 0; }

// Keys of the range [lo, lo + len) that are below `limit`.
__device__ __forceinline__ int64_t below(int64_t lo, int64_t len, int64_t limit) {
  return limit <= lo ? 0 : (limit >= lo + len ? len : limit - lo);
}

__device__ BlockPlan plan_block(const LayoutParams& p, int b) {
  const int64_t ps = int64_t(1) << p.ps_shift;
  BlockPlan k;
  k.s = p.block_start[b];
  k.e = p.block_start[b + 1];
  const int64_t ws = k.s - p.window > p.pin ? k.s - p.window : p.pin;
  // fixed region: whole pages below min(pin, s), then the rest as one piece
  const int64_t fixed_end = k.s < p.pin ? k.s : p.pin;
  k.n_fixed_full = int32_t(fixed_end >> p.ps_shift);
  k.a0 = int64_t(k.n_fixed_full) << p.ps_shift;
  k.a_len = fixed_end - k.a0;
  // rolling region: [ws, s) split into a head piece, whole pages, a tail piece
  k.b0 = ws; k.b_len = 0; k.c0 = k.s; k.c_len = 0; k.q0 = 0; k.n_roll_full = 0;
  if (k.s > ws) {
    const int64_t r0 = ws - p.pin, r1 = k.s - p.pin;
    const int64_t q0 = (r0 + ps - 1) >> p.ps_shift, q1 = r1 >> p.ps_shift;
    if (q1 > q0) {
      k.q0 = q0;
      k.n_roll_full = int32_t(q1 - q0);
      k.b_len = clamp_len(ws, p.pin + (q0 << p.ps_shift));
      k.c0 = p.pin + (q1 << p.ps_shift);
      k.c_len = k.s - k.c0;
    } else {
      k.b_len = k.s - ws;
    }
  }
  k.pieces = k.a_len + k.b_len + k.c_len;
  k.committed_pieces = below(k.a0, k.a_len, p.committed) + below(k.b0, k.b_len, p.committed) +
                       below(k.c0, k.c_len, p.committed);
  k.direct = k.pieces == 0 && k.s >= p.pin && ((k.s - p.pin) & (ps - 1)) == 0;
  k.own_q0 = k.direct ? (k.s - p.pin) >> p.ps_shift : 0;
  k.own_pages = k.direct ? ((k.e - p.pin + ps - 1) >> p.ps_shift) - k.own_q0 : 0;
  return k;
}

// The k-th visible key before the block that is not on a whole page.
__device__ __forceinline__ int64_t piece_key(const BlockPlan& k, int64_t i) {
  if (i < k.a_len) return k.a0 + i;
  i -= k.a_len;
  if (i < k.b_len) return k.b0 + i;
  return k.c0 + (i - k.b_len);
}

// Slot of logical key x in the sequence's own pages.
__device__ __forceinline__ int64_t own_slot(const LayoutParams& p, int64_t x) {
  const int64_t mask = (int64_t(1) << p.ps_shift) - 1;
  if (x < p.pin) return (int64_t(p.table[x >> p.ps_shift]) << p.ps_shift) + (x & mask);
  const int64_t r = x - p.pin - p.evicted;
  return (int64_t(p.table[p.n_fixed + (r >> p.ps_shift)]) << p.ps_shift) + (r & mask);
}

__device__ __forceinline__ int64_t private_slot(const LayoutParams& p, int b, int64_t i) {
  const int64_t mask = (int64_t(1) << p.ps_shift) - 1;
  return (int64_t(p.priv[int64_t(b) * p.priv_stride + (i >> p.ps_shift)]) << p.ps_shift) + (i & mask);
}

__global__ void __launch_bounds__(kLayoutThreads) causal_layout_kernel(const LayoutParams p) {
  const int b = blockIdx.x;
  const BlockPlan k = plan_block(p, b);
  const int64_t ps = int64_t(1) << p.ps_shift;
  const int64_t size = k.e - k.s;
  const int32_t n_full = k.n_fixed_full + k.n_roll_full;
  const int64_t tail_pages = k.direct ? k.own_pages : (k.pieces + size + ps - 1) >> p.ps_shift;
  const int64_t ev_pages = p.evicted >> p.ps_shift;

  int32_t* row = p.block_tables + int64_t(b) * p.table_width;
  for (int j = threadIdx.x; j < p.table_width; j += kLayoutThreads) {
    int32_t v = -1;
    if (j < k.n_fixed_full) {
      v = p.table[j];
    } else if (j < n_full) {
      v = p.table[p.n_fixed + (k.q0 + (j - k.n_fixed_full)) - ev_pages];
    } else if (j - n_full < tail_pages) {
      const int64_t t = j - n_full;
      v = k.direct ? p.table[p.n_fixed + (k.own_q0 + t) - ev_pages] : p.priv[int64_t(b) * p.priv_stride + t];
    }
    row[j] = v;
  }

  const int64_t current_pieces = k.pieces - k.committed_pieces;
  const int64_t lb = int64_t(b) * p.list_stride;
  for (int i = threadIdx.x; i < p.list_stride; i += kLayoutThreads) {
    int64_t cs = -1, cd = -1, us = -1, ud = -1;
    if (i < k.committed_pieces) {
      cs = own_slot(p, piece_key(k, i));
      cd = private_slot(p, b, i);
    }
    if (i < current_pieces) {
      us = own_slot(p, piece_key(k, k.committed_pieces + i));
      ud = private_slot(p, b, k.committed_pieces + i);
    }
    p.commit_src[lb + i] = cs;
    p.commit_dst[lb + i] = cd;
    p.current_src[lb + i] = us;
    p.current_dst[lb + i] = ud;
  }

  for (int64_t i = threadIdx.x; i < size; i += kLayoutThreads) {
    const int64_t t = k.s - p.committed + i;
    p.stage_slots[t] = own_slot(p, k.s + i);
    p.stage_slots2[t] = k.direct ? -1 : private_slot(p, b, k.pieces + i);
  }

  if (threadIdx.x == 0) {
    p.n_ctx[b] = int32_t(int64_t(n_full) * ps + k.pieces);
    p.seq_len[b] = int32_t(size);
  }
}

}  // namespace

hipError_t launch_causal_layout(const LayoutParams& p, hipStream_t stream) {
  hipLaunchKernelGGL(causal_layout_kernel, dim3(p.num_blocks), dim3(kLayoutThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace pkv
