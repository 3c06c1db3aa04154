// Paged decode attention.
//
// "Paged causal K/V cache and cached attention for VisualGen", Description /
// Attention: attention over the keys a block-table row maps; "Support
// shared-prefix attention for n-sample requests in FMHA", FA4 prefix / tail
// commits: n query rows can share one table row (the shared-prefix pass of an
// n-sample group), the result carries a natural-log LSE for the merge, and
// the key range of a small grid is cut into splits joined by the LSE merge
// (split-KV commits: only when it pays, chunks of at least 512 tokens).
//
// Work unit: (table row t, kv head g, key split s, row group).  The query rows
// of a unit are R = rows_per_table * (Hq / Hkv) rows (sample i, head g*G + hh);
// they share every K/V byte the unit reads, so K/V are read from HBM once per
// unit.
//
// MFMA kernel (q bf16, K/V bf16 or fp8 e4m3fn):
//   * A wave owns a block of 16 query rows.  The key range is walked in tiles
//     of 32 logical keys = two 16-key halves, each inside one page (page_size
//     >= 16).  Page ids of the next 64 tiles are fetched with one vector load
//     and read back with readlane, so the table walk never stalls the loop.
//   * S^T[key][row] = K Q^T on v_mfma_f32_16x16x32_bf16: the A operand is a
//     key row (lane = key, 16-byte loads straight from the page), the B
//     operand is Q held in registers for the whole kernel.  The output gives
//     every lane one query row and 8 keys of the tile.
//   * Online softmax per row in the log2 domain; the running max is shared by
//     the four lanes of a row through two xor-shuffles.
//   * O^T[dim][row] += V^T P^T on the same MFMA: P^T is the score registers
//     converted to bf16 in place (no shuffle), V^T is built in registers from
//     an 8-key x (D/16)-dim block that each lane loads directly (a 16-lane
//     group reads whole 256-byte rows) and transposes with v_perm_b32.  The
//     output row of a lane is its softmax row, so rescaling needs no shuffle.
//   * fp8: codes are widened to bf16 exactly, two per instruction
//     (v_cvt_scalef32_pk_bf16_fp8 with scale 1; an e4m3 value fits bf16),
//     the per-(page, kv head) K scale multiplies the scores
//     and the V scale is folded into P before the PV product.
//   * Dead rows of a partial last page and poison pages are selected away
//     (scores to -inf, V rows to 0) before they can reach a product.
//   * Waves of a workgroup either own different row blocks or split the
//     tiles of one row block; split states are combined through LDS with the
//     merge formula.  Cross-workgroup splits write normalised partial states
//     and their LSE, joined by the merge kernel.
//
// VALU kernel (q fp32; any K/V dtype): one wave per (query row, split); the
// exact fp32 path for small or fp32 problems.
#include "pkv_device.hpp"
#include "pkv_internal.hpp"

namespace pkv {

namespace {

// Pages of the 16-key halves of up to 64 consecutive tiles of one wave:
// lane k holds the ids for tile `first + k * step`.
struct PageWindow {
  int32_t e0, e1;     // page of half 0 / half 1
  float ks0, ks1;     // fp8 K scale of (page, kv head) for both halves
  float vs0, vs1;
};

template <bool kFp8>
__device__ __forceinline__ PageWindow fetch_pages(const DecodeParams& p, const int32_t* trow, int g, int first,
                                                  int step, int te, int len) {
  const int lane = threadIdx.x & 63;
  const int tile = first + lane * step;
  PageWindow w{0, 0, 1.f, 1.f, 1.f, 1.f};
  if (tile < te) {
    const int key0 = tile * 32;
    w.e0 = trow[key0 >> p.page_shift];
    w.e1 = (p.page_shift >= 5 || key0 + 16 >= len) ? w.e0 : trow[(key0 + 16) >> p.page_shift];
    if constexpr (kFp8) {
      w.ks0 = p.k_scale[(int64_t)w.e0 * p.num_kv_heads + g];
      w.vs0 = p.v_scale[(int64_t)w.e0 * p.num_kv_heads + g];
      w.ks1 = p.k_scale[(int64_t)w.e1 * p.num_kv_heads + g];
      w.vs1 = p.v_scale[(int64_t)w.e1 * p.num_kv_heads + g];
    }
  }
  return w;
}

// The same window read without the row's length, so that it can be loaded
// together with it: entries for tiles below te, where te only bounds the
// table row (tile te - 1 starts inside its table_stride pages), and a second
// half's page outside the row is the first half's.  Entries past the row's
// last key are padding; a page id outside the pool is clamped into it, so
// that every id in the window names a real page (the tiles past the last key
// are never walked; rows of a walked tile past it are masked).
template <bool kFp8>
__device__ __forceinline__ PageWindow fetch_pages_ahead(const DecodeParams& p, const int32_t* trow, int g, int first,
                                                        int step, int te) {
  const int lane = threadIdx.x & 63;
  const int tile = first + lane * step;
  PageWindow w{0, 0, 1.f, 1.f, 1.f, 1.f};
  if (tile < te) {
    const int key0 = tile * 32;
    const uint32_t last = (uint32_t)(p.num_pages - 1);
    w.e0 = (int)min((uint32_t)trow[key0 >> p.page_shift], last);
    const int i1 = (key0 + 16) >> p.page_shift;
    w.e1 = (p.page_shift >= 5 || i1 >= p.table_stride) ? w.e0 : (int)min((uint32_t)trow[i1], last);
    if constexpr (kFp8) {
      w.ks0 = p.k_scale[(int64_t)w.e0 * p.num_kv_heads + g];
      w.vs0 = p.v_scale[(int64_t)w.e0 * p.num_kv_heads + g];
      w.ks1 = p.k_scale[(int64_t)w.e1 * p.num_kv_heads + g];
      w.vs1 = p.v_scale[(int64_t)w.e1 * p.num_kv_heads + g];
    }
  }
  return w;
}

__device__ __forceinline__ int rl(int v, int k) { return __builtin_amdgcn_readlane(v, k); }
__device__ __forceinline__ float rlf(float v, int k) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), k));
}

// Raw registers of one 32-key tile.
template <int D, bool kFp8>
struct TileRegs {
  static constexpr int NCH = D / 32;                  // 32-dim MFMA chunks of QK
  static constexpr int KLD = kFp8 ? NCH / 2 : NCH;    // 16-byte K loads per half
  static constexpr int VB = kFp8 ? D / 16 : D / 8;    // bytes per V block row (D/16 dims)
  u32x4 k[2][KLD];
  uint32_t v[8][VB / 4 > 0 ? VB / 4 : 1];             // 8 keys x (D/16) dims, as dwords
  float ks0, ks1, vs0, vs1;
};

// Byte offsets of this lane inside a page that stay fixed along the key walk.
struct LaneOffsets {
  int k;   // K: key row (lane & 15) of a 16-key half, dims chunk of lane group
  int v;   // V: key row 4 * (lane >> 4) of a half, dims (D/16) * (lane & 15)
};

// A raw buffer descriptor over one page's rows of one kv head.  With
// nbytes = 0 every load through it returns zeros without touching memory,
// which is how a prefetch past the end of the key range is made harmless.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t page_rsrc(const uint8_t* pool, int page, int64_t page_stride_b,
                                                            int64_t head_off_b, int nbytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(pool + (int64_t)page * page_stride_b + head_off_b),
                                           (short)0, nbytes, 0x00020000);
}

// Issue the loads of one tile (two 16-key halves at rows row0 / row1 of
// pages page0 / page1).  Addresses are SGPR descriptors + per-lane constant
// offsets, so the walk costs no vector address arithmetic.
template <int D, bool kFp8>
__device__ __forceinline__ void issue_tile(TileRegs<D, kFp8>& r, const uint8_t* kp, const uint8_t* vp, int page0,
                                           int page1, int row0, int row1, int64_t page_stride_b, int64_t head_off_b,
                                           int row_b, int nbytes, LaneOffsets lo) {
  using T = TileRegs<D, kFp8>;
  const __amdgpu_buffer_rsrc_t k0 = page_rsrc(kp, page0, page_stride_b, head_off_b, nbytes);
  const __amdgpu_buffer_rsrc_t k1 = page_rsrc(kp, page1, page_stride_b, head_off_b, nbytes);
  const __amdgpu_buffer_rsrc_t v0 = page_rsrc(vp, page0, page_stride_b, head_off_b, nbytes);
  const __amdgpu_buffer_rsrc_t v1 = page_rsrc(vp, page1, page_stride_b, head_off_b, nbytes);
#pragma unroll
  for (int c = 0; c < T::KLD; ++c) {
    r.k[0][c] = __builtin_amdgcn_raw_buffer_load_b128(k0, lo.k + 64 * c, row0 * row_b, 0);
    r.k[1][c] = __builtin_amdgcn_raw_buffer_load_b128(k1, lo.k + 64 * c, row1 * row_b, 0);
  }
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    const __amdgpu_buffer_rsrc_t rs = (t < 4) ? v0 : v1;
    const int soff = ((t < 4 ? row0 : row1) + (t & 3)) * row_b;
    if constexpr (T::VB == 16) {
      const u32x4 x = __builtin_amdgcn_raw_buffer_load_b128(rs, lo.v, soff, 0);
      r.v[t][0] = x[0]; r.v[t][1] = x[1]; r.v[t][2] = x[2]; r.v[t][3] = x[3];
    } else if constexpr (T::VB == 8) {
      const u32x2 x = __builtin_amdgcn_raw_buffer_load_b64(rs, lo.v, soff, 0);
      r.v[t][0] = x[0]; r.v[t][1] = x[1];
    } else {
      r.v[t][0] = __builtin_amdgcn_raw_buffer_load_b32(rs, lo.v, soff, 0);
    }
  }
}

// Running softmax state of one wave (16 rows, lane row = lane & 15).
template <int D>
struct RowState {
  static constexpr int DPL = D / 16;
  f32x4 o[DPL];   // O^T[dim DPL*(4j+i)+t'][row] in o[t'][i]
  float m;        // running max (log2 domain), shared by the row's 4 lanes
  float l;        // this lane's share of the running sum
};

template <int D, bool kFp8>
__device__ __forceinline__ void compute_tile(RowState<D>& st, TileRegs<D, kFp8>& r, const u32x4 (&q)[D / 32],
                                             float scale_log2, int key0, int len, int lim, int lim_lo) {
  using T = TileRegs<D, kFp8>;
  constexpr int NCH = T::NCH;
  constexpr int DPL = D / 16;
  const int lane = threadIdx.x & 63;
  const int j = lane >> 4;

  // ---- S^T = K Q^T for both 16-key halves
  f32x4 s[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      u32x4 a;
      if constexpr (kFp8) {
        const u32x4 raw = r.k[h][i >> 1];
        const int e = i & 1;
#pragma unroll
        for (int w = 0; w < 2; ++w) {
          const uint32_t dw = raw[2 * e + w];
          a[2 * w] = fp8x2_to_bf16x2<false>(dw);
          a[2 * w + 1] = fp8x2_to_bf16x2<true>(dw);
        }
      } else {
        a = r.k[h][i];
      }
      acc = mfma16x16x32_bf16(a, q[i], acc);
    }
    s[h] = acc;
  }
  // ---- scale (and fp8 K scale), mask keys at or past the lane's row limit
  // (lim; lim_lo <= every row's limit is wave-uniform)
  const float c0 = kFp8 ? scale_log2 * r.ks0 : scale_log2;
  const float c1 = kFp8 ? scale_log2 * r.ks1 : scale_log2;
  s[0] *= c0;
  s[1] *= c1;
  const bool partial = key0 + 32 > lim_lo;
  if (partial) {
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (key0 + 16 * h + 4 * j + i >= lim) s[h][i] = kNegInf;
  }
  // ---- online softmax (row max shared by the 4 lanes of a row)
  float mt = fmaxf(fmaxf(fmaxf(s[0][0], s[0][1]), fmaxf(s[0][2], s[0][3])),
                   fmaxf(fmaxf(s[1][0], s[1][1]), fmaxf(s[1][2], s[1][3])));
  mt = wave_max_xor(mt, 16);
  mt = wave_max_xor(mt, 32);
  const float m_new = fmaxf(st.m, mt);
  const float m_use = (m_new == kNegInf) ? 0.f : m_new;
  const float alpha = fast_exp2(st.m - m_use);
  float pv[8];
  float psum = 0.f;
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float e = fast_exp2(s[h][i] - m_use);
      pv[4 * h + i] = e;
      psum += e;
    }
  st.l = st.l * alpha + psum;
  st.m = m_new;
#pragma unroll
  for (int t = 0; t < DPL; ++t) st.o[t] *= alpha;
  if constexpr (kFp8) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      pv[i] *= r.vs0;
      pv[4 + i] *= r.vs1;
    }
  }
  u32x4 pb;
  pb[0] = pack_bf16x2(pv[0], pv[1]);
  pb[1] = pack_bf16x2(pv[2], pv[3]);
  pb[2] = pack_bf16x2(pv[4], pv[5]);
  pb[3] = pack_bf16x2(pv[6], pv[7]);

  // ---- V^T operands (8 keys of this lane group, one dim each); dead keys of
  // a tile past the row's last key are zeroed in place first (0 * NaN would
  // poison the sum).  Keys a causal row only masks are real and stay.
  constexpr int VW = T::VB / 4 > 0 ? T::VB / 4 : 1;   // raw dwords per key
  if (key0 + 32 > len) {
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const bool ok = key0 + 16 * (t >> 2) + 4 * j + (t & 3) < len;
#pragma unroll
      for (int w = 0; w < VW; ++w) r.v[t][w] = ok ? r.v[t][w] : 0u;
    }
  }
  if constexpr (!kFp8) {
    // dword w of key t holds dims 2w (low half) and 2w+1 (high half)
#pragma unroll
    for (int tp = 0; tp < DPL; ++tp) {
      const int w = tp >> 1;
      u32x4 a;
#pragma unroll
      for (int q2 = 0; q2 < 4; ++q2)
        a[q2] = (tp & 1) ? pack_hi16(r.v[2 * q2][w], r.v[2 * q2 + 1][w])
                         : pack_lo16(r.v[2 * q2][w], r.v[2 * q2 + 1][w]);
      st.o[tp] = mfma16x16x32_bf16(a, pb, st.o[tp]);
    }
  } else {
    // fp8: for dims (tp, tp+1) gather the codes of keys (2q, 2q+1) into one
    // dword [k0.tp, k1.tp, k0.tp+1, k1.tp+1], widen each half to two floats and
    // keep their high halves (exact bf16)
#pragma unroll
    for (int tp = 0; tp < DPL; tp += 2) {
      const int w = tp >> 2;
      const uint32_t sel = (tp & 2) ? 0x07030602u : 0x05010400u;
      u32x4 a0, a1;
#pragma unroll
      for (int q2 = 0; q2 < 4; ++q2) {
        const uint32_t mixed = perm_b32(r.v[2 * q2 + 1][w], r.v[2 * q2][w], sel);
        a0[q2] = fp8x2_to_bf16x2<false>(mixed);
        a1[q2] = fp8x2_to_bf16x2<true>(mixed);
      }
      st.o[tp] = mfma16x16x32_bf16(a0, pb, st.o[tp]);
      st.o[tp + 1] = mfma16x16x32_bf16(a1, pb, st.o[tp + 1]);
    }
  }
}

// Q operand chunks of this lane's query row (zeros for a padding row).  The
// dims of chunk i / lane group j match the K operand layout of the tile.
template <int D, bool kFp8>
__device__ __forceinline__ void load_q(u32x4 (&q)[D / 32], const DecodeParams& p, int64_t qrow, bool row_ok) {
  const int j = (threadIdx.x & 63) >> 4;
  const uint16_t* qp = reinterpret_cast<const uint16_t*>(p.q) + qrow * D;
#pragma unroll
  for (int i = 0; i < D / 32; ++i) {
    const int dim = kFp8 ? (64 * (i >> 1) + 16 * j + 8 * (i & 1)) : (32 * i + 8 * j);
    q[i] = row_ok ? ld16(qp + dim) : u32x4{0u, 0u, 0u, 0u};
  }
}

template <int D>
__device__ __forceinline__ void reset_state(RowState<D>& st) {
#pragma unroll
  for (int tp = 0; tp < D / 16; ++tp) st.o[tp] = f32x4{0.f, 0.f, 0.f, 0.f};
  st.m = kNegInf;
  st.l = 0.f;
}

// Walk the tiles first, first + step, ... (n of them) of one (table row, kv
// head): windows of 64 tiles get their page ids (and fp8 scales) with one
// vector load; inside a window every tile is prefetched one step ahead with
// unconditional loads (zero-range descriptor past the window's end).
// hook() runs once, just before the loads of tile hook_tile are issued.
// win0, when given, is the first window, already loaded.
struct NoHook {
  __device__ void operator()() const {}
};
template <int D, bool kFp8, typename Hook = NoHook>
__device__ __forceinline__ void walk_tiles(RowState<D>& st, const u32x4 (&q)[D / 32], const DecodeParams& p,
                                           const int32_t* trow, int g, int len, int lim, int lim_lo, int first,
                                           int step, int n, int hook_tile = -1, Hook hook = Hook{},
                                           const PageWindow* win0 = nullptr) {
  constexpr int esz = kFp8 ? 1 : 2;
  const int lane = threadIdx.x & 63;
  const int r_lane = lane & 15, j = lane >> 4;
  const uint8_t* kp = reinterpret_cast<const uint8_t*>(p.k_pool);
  const uint8_t* vp = reinterpret_cast<const uint8_t*>(p.v_pool);
  const int64_t page_stride_b = p.page_stride * esz;
  const int64_t head_off_b = (int64_t)g * D * esz;
  const int row_b = p.num_kv_heads * D * esz;
  const int page_bytes = (1 << p.page_shift) * row_b;
  const int pmask = (1 << p.page_shift) - 1;
  const LaneOffsets lo{r_lane * row_b + 16 * j, 4 * j * row_b + (D / 16) * r_lane * esz};
  const int te = first + (n - 1) * step + 1;   // one past the last tile walked
  TileRegs<D, kFp8> A, B;
  for (int w0 = 0; w0 < n; w0 += 64) {
    const PageWindow win = (win0 && w0 == 0) ? *win0 : fetch_pages<kFp8>(p, trow, g, first + w0 * step, step, te, len);
    const int n_win = n - w0 < 64 ? n - w0 : 64;
    auto issue = [&](TileRegs<D, kFp8>& X, int k) {
      const bool ok = k < n_win;
      const int kc = ok ? k : 0;
      if (ok && first + (w0 + k) * step == hook_tile) hook();
      const int key0 = (first + (w0 + kc) * step) * 32;
      issue_tile<D, kFp8>(X, kp, vp, rl(win.e0, kc), rl(win.e1, kc), key0 & pmask, (key0 + 16) & pmask,
                          page_stride_b, head_off_b, row_b, ok ? page_bytes : 0, lo);
      if constexpr (kFp8) {
        X.ks0 = rlf(win.ks0, kc);
        X.ks1 = rlf(win.ks1, kc);
        X.vs0 = rlf(win.vs0, kc);
        X.vs1 = rlf(win.vs1, kc);
      }
    };
    issue(A, 0);
    for (int k = 0; k < n_win; k += 2) {
      issue(B, k + 1);
      compute_tile<D, kFp8>(st, A, q, p.scale_log2, (first + (w0 + k) * step) * 32, len, lim, lim_lo);
      if (k + 1 >= n_win) break;
      issue(A, k + 2);
      compute_tile<D, kFp8>(st, B, q, p.scale_log2, (first + (w0 + k + 1) * step) * 32, len, lim, lim_lo);
    }
  }
}

// The same walk for the four waves of a workgroup that own different row
// blocks of one unit (bf16, D = 128): every wave needs the whole K/V tile, so
// each tile goes from HBM to registers to LDS once.  Wave w loads register
// slots 4 w .. 4 w + 3 of every lane (slots 0-7: the 16-byte K chunks of
// half 0 then half 1; 8-15: the V rows of half 0 then half 1), writes them to
// an LDS stage in that register image, and every wave reads the whole image
// back, so compute_tile sees exactly what its own loads would have returned.
// Two LDS stages, two tiles in flight per wave (a quarter tile each), one
// barrier per tile.  All four waves must call it with the same arguments.
template <int D>
__device__ __forceinline__ void walk_tiles_shared(RowState<D>& st, const u32x4 (&q)[D / 32], const DecodeParams& p,
                                                  const int32_t* trow, int g, int len, int lim, int lim_lo,
                                                  int first, int step, int n, const PageWindow* win0 = nullptr) {
  static_assert(D == 128, "the shared walk stages bf16 tiles of 128 dims");
  using T = TileRegs<D, false>;
  static_assert(T::KLD == 4 && T::VB == 16, "16 register slots of 16 bytes per lane");
  __shared__ u32x4 stage[2][16][64];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r_lane = lane & 15, j = lane >> 4;
  const uint8_t* kp = reinterpret_cast<const uint8_t*>(p.k_pool);
  const uint8_t* vp = reinterpret_cast<const uint8_t*>(p.v_pool);
  const int64_t page_stride_b = p.page_stride * 2;
  const int64_t head_off_b = (int64_t)g * D * 2;
  const int row_b = p.num_kv_heads * D * 2;
  const int page_bytes = (1 << p.page_shift) * row_b;
  const int pmask = (1 << p.page_shift) - 1;
  const LaneOffsets lo{r_lane * row_b + 16 * j, 4 * j * row_b + (D / 16) * r_lane * 2};
  const int te = first + (n - 1) * step + 1;
  // this wave's quarter of tile k of the window: wave 0 / 1 the K chunks of
  // half 0 / 1, wave 2 / 3 the V rows of half 0 / 1
  const bool is_k = wave < 2;
  const bool half1 = (wave & 1) != 0;
  auto issue = [&](u32x4 (&x)[4], const PageWindow& win, int w0, int k, int n_win) {
    const bool ok = k < n_win;
    const int kc = ok ? k : 0;
    const int key0 = (first + (w0 + kc) * step) * 32;
    const int page = half1 ? rl(win.e1, kc) : rl(win.e0, kc);
    const int row = ((half1 ? key0 + 16 : key0) & pmask);
    const __amdgpu_buffer_rsrc_t rs = page_rsrc(is_k ? kp : vp, page, page_stride_b, head_off_b, ok ? page_bytes : 0);
#pragma unroll
    for (int i = 0; i < 4; ++i)
      x[i] = is_k ? __builtin_amdgcn_raw_buffer_load_b128(rs, lo.k + 64 * i, row * row_b, 0)
                  : __builtin_amdgcn_raw_buffer_load_b128(rs, lo.v, (row + i) * row_b, 0);
  };
  auto put = [&](int b, const u32x4 (&x)[4]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) stage[b][4 * wave + i][lane] = x[i];
  };
  auto get = [&](int b, T& r) {
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int c = 0; c < 4; ++c) r.k[h][c] = stage[b][4 * h + c][lane];
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const u32x4 v = stage[b][8 + t][lane];
      r.v[t][0] = v[0]; r.v[t][1] = v[1]; r.v[t][2] = v[2]; r.v[t][3] = v[3];
    }
  };
  T r;
  for (int w0 = 0; w0 < n; w0 += 64) {
    const PageWindow win = (win0 && w0 == 0) ? *win0 : fetch_pages<false>(p, trow, g, first + w0 * step, step, te, len);
    const int n_win = n - w0 < 64 ? n - w0 : 64;
    u32x4 xa[4], xb[4];
    issue(xa, win, w0, 0, n_win);
    issue(xb, win, w0, 1, n_win);
    put(0, xa);
    __syncthreads();
    for (int k = 0; k < n_win; k += 2) {
      issue(xa, win, w0, k + 2, n_win);
      get(0, r);
      compute_tile<D, false>(st, r, q, p.scale_log2, (first + (w0 + k) * step) * 32, len, lim, lim_lo);
      put(1, xb);
      __syncthreads();
      if (k + 1 >= n_win) break;
      issue(xb, win, w0, k + 3, n_win);
      get(1, r);
      compute_tile<D, false>(st, r, q, p.scale_log2, (first + (w0 + k + 1) * step) * 32, len, lim, lim_lo);
      put(0, xa);
      __syncthreads();
    }
  }
}

// Store the normalised rows of a finished state: lane (r, j) holds dims
// DPL*(4j+i) + t' of row r.  `dst` points at the row's D outputs.
template <int D>
__device__ __forceinline__ void store_row(const RowState<D>& st, void* dst, bool bf16, float inv) {
  constexpr int DPL = D / 16;
  const int j = (threadIdx.x & 63) >> 4;
  if (bf16) {
    uint16_t* o = reinterpret_cast<uint16_t*>(dst);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      uint32_t w[DPL / 2];
#pragma unroll
      for (int tp = 0; tp < DPL; tp += 2) w[tp / 2] = pack_bf16x2(st.o[tp][i] * inv, st.o[tp + 1][i] * inv);
      uint16_t* d = o + DPL * (4 * j + i);
      if constexpr (DPL == 8) *reinterpret_cast<u32x4*>(d) = u32x4{w[0], w[1], w[2], w[3]};
      else *reinterpret_cast<u32x2*>(d) = u32x2{w[0], w[1]};
    }
  } else {
    float* o = reinterpret_cast<float*>(dst);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int tp = 0; tp < DPL; tp += 4)
        *reinterpret_cast<f32x4*>(o + DPL * (4 * j + i) + tp) =
            f32x4{st.o[tp][i] * inv, st.o[tp + 1][i] * inv, st.o[tp + 2][i] * inv, st.o[tp + 3][i] * inv};
  }
}

__device__ __forceinline__ void row_of(const DecodeParams& p, int t, int g, int r, int& qi, int64_t& qrow) {
  qi = r / p.group;
  const int qh = g * p.group + (r - qi * p.group);
  qrow = ((int64_t)t * p.rows_per_table + qi) * p.num_q_heads + qh;
}

// Keys row qi of a table row with len keys sees: all of them, or for a step
// of n causal tokens (the last n keys of the row) the keys up to its own.
__device__ __forceinline__ int row_limit(const DecodeParams& p, int len, int qi) {
  return p.causal ? len - (p.rows_per_table - 1 - qi) : len;
}

}  // namespace

// Write the step's tokens at keys [kb, ke) of table row t (key x is step
// token x - (len - n)) for kv head g into the pool: 16 bytes per thread and
// instruction, threads i0, i0 + ni, ... of the caller's range; then wait
// until this thread's stores have completed.
template <int D, bool kFp8>
__device__ __forceinline__ void append_rows(const DecodeParams& p, int t, int g, int len, int kb, int ke, int i0,
                                            int ni) {
  constexpr int esz = kFp8 ? 1 : 2;
  constexpr int CPR = D * esz / 16;   // 16-byte chunks per row
  const int n = p.rows_per_table;
  const int row_b = p.num_kv_heads * D * esz;
  const int64_t page_stride_b = p.page_stride * esz;
  const int pmask = (1 << p.page_shift) - 1;
  const int32_t* trow = p.table + (int64_t)t * p.table_stride;
  uint8_t* kp = const_cast<uint8_t*>(reinterpret_cast<const uint8_t*>(p.k_pool));
  uint8_t* vp = const_cast<uint8_t*>(reinterpret_cast<const uint8_t*>(p.v_pool));
  for (int i = i0; i < (ke - kb) * CPR; i += ni) {
    const int key = kb + i / CPR, c = i % CPR;
    const int64_t src = (int64_t)(t * n + key - (len - n)) * p.new_tok_stride_b + (int64_t)g * p.new_head_stride_b + 16 * c;
    const int64_t dst = (int64_t)trow[key >> p.page_shift] * page_stride_b + (int64_t)(key & pmask) * row_b +
                        (int64_t)g * D * esz + 16 * c;
    *reinterpret_cast<u32x4*>(kp + dst) = *reinterpret_cast<const u32x4*>(p.new_k + src);
    *reinterpret_cast<u32x4*>(vp + dst) = *reinterpret_cast<const u32x4*>(p.new_v + src);
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

// Up to 64 of the step's 16-byte chunks (keys [kb, ke) of table row t, kv
// head g; one per lane) held in registers until the walk issues the loads of
// the tile that holds them, and their pool offset (-1: none for this lane).
struct StepTokens {
  u32x4 k = {0u, 0u, 0u, 0u}, v = {0u, 0u, 0u, 0u};
  int64_t dst = -1;
};

template <int D, bool kFp8>
__device__ __forceinline__ StepTokens load_step_tokens(const DecodeParams& p, int t, int g, int len, int kb, int ke) {
  constexpr int esz = kFp8 ? 1 : 2;
  constexpr int CPR = D * esz / 16;
  const int lane = threadIdx.x & 63;
  StepTokens tk;
  if (lane < (ke - kb) * CPR) {
    const int n = p.rows_per_table;
    const int key = kb + lane / CPR, c = lane % CPR;
    const int64_t src = (int64_t)(t * n + key - (len - n)) * p.new_tok_stride_b + (int64_t)g * p.new_head_stride_b + 16 * c;
    tk.k = *reinterpret_cast<const u32x4*>(p.new_k + src);
    tk.v = *reinterpret_cast<const u32x4*>(p.new_v + src);
    const int32_t* trow = p.table + (int64_t)t * p.table_stride;
    tk.dst = (int64_t)trow[key >> p.page_shift] * p.page_stride * esz +
             (int64_t)(key & ((1 << p.page_shift) - 1)) * p.num_kv_heads * D * esz + (int64_t)g * D * esz + 16 * c;
  }
  return tk;
}

__device__ __forceinline__ void store_step_tokens(const DecodeParams& p, const StepTokens& tk) {
  if (tk.dst >= 0) {
    *reinterpret_cast<u32x4*>(const_cast<uint8_t*>(reinterpret_cast<const uint8_t*>(p.k_pool)) + tk.dst) = tk.k;
    *reinterpret_cast<u32x4*>(const_cast<uint8_t*>(reinterpret_cast<const uint8_t*>(p.v_pool)) + tk.dst) = tk.v;
  }
  asm volatile("" ::: "memory");
}

// ---------------------------------------------------------------------------
// Split kernel: one workgroup per (key split, kv head, table row, row group).
// Used without a stream-K workspace; with splits == 1 it needs no workspace.
// ---------------------------------------------------------------------------
// The work of one workgroup: key split s of (kv head g, table row t, row
// group rg), WP waves per 16-row block.
template <int D, bool kFp8, int WP>
__device__ __forceinline__ void decode_block(const DecodeParams& p, int s, int g, int t, int rg) {
  constexpr int WR = 4 / WP;
  constexpr int DPL = D / 16;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform
  const int wr = wave / WP, wp = wave - (wave / WP) * WP;
  const int lane = threadIdx.x & 63;
  const int r_lane = lane & 15, j = lane >> 4;
  const int R = p.rows_per_table * p.group;
  const int rb = rg * WR + wr;

  const int len = p.kv_lens[t];
  const int tb = s * p.tiles_per_split;
  const int first = tb + wp;
  const int32_t* trow = p.table + (int64_t)t * p.table_stride;
  // Q and this wave's first window of page ids do not depend on the length:
  // they are loaded together with it (the window bounded by the split and
  // the table row instead), which takes one memory round trip off the
  // workgroup's start.
  const int r = rb * 16 + r_lane;
  const bool row_ok = r < R;
  int qi;
  int64_t qrow;
  row_of(p, t, g, row_ok ? r : 0, qi, qrow);
  u32x4 q[D / 32];
  load_q<D, kFp8>(q, p, qrow, row_ok);
  const int cap = (int)min((int64_t)tb + p.tiles_per_split, (((int64_t)p.table_stride << p.page_shift) + 31) >> 5);
  const PageWindow win0 = fetch_pages_ahead<kFp8>(p, trow, g, first, WP, cap);
  const int tiles = (len + 31) >> 5;
  int te = tb + p.tiles_per_split;
  te = te < tiles ? te : tiles;
  if (p.splits > 1 && tb >= te && !p.write_state) return;   // empty split: the merge never reads it

  RowState<D> st;
  reset_state(st);
  const int n_mine = first < te ? (te - first + WP - 1) / WP : 0;
  // The step's tokens, when the call writes them (keys len - n .. len - 1 of
  // this split's keys; kv head g): the launch gives every (table row, kv
  // head) one workgroup, so only this workgroup reads them.  With one row
  // block (WP == 4) the wave that walks a token's tile is its only reader:
  // it loads up to 64 16-byte chunks (4 tokens of 128 bf16 dims) now and
  // stores them just before it issues that tile's loads, as the head-parallel
  // stream-K kernel does.  With several row blocks every wave reads each tile,
  // so the workgroup writes the tokens and meets at a barrier first.
  int hook_tile = -1;
  StepTokens tok;
  if (p.new_k) {
    constexpr int CPR = D * (kFp8 ? 1 : 2) / 16;   // 16-byte chunks per row
    const int kb = max(max(len - p.rows_per_table, 0), tb * 32), ke = min(len, te * 32);
    if constexpr (WP == 4) {
      // the token tiles are at most 2 consecutive ones (n <= 16 rows): the
      // one this wave walks, if any
      const int t0 = kb >> 5;
      const int kt = t0 + (((wp - (t0 - tb)) % WP) + WP) % WP;
      const int wb = max(kb, kt * 32), we = min(ke, kt * 32 + 32);
      if (wb < we && (we - wb) * CPR <= 64) {
        tok = load_step_tokens<D, kFp8>(p, t, g, len, wb, we);
        hook_tile = kt;
      } else if (wb < we) {
        append_rows<D, kFp8>(p, t, g, len, wb, we, lane, 64);
      }
    } else {
      if (kb < ke) append_rows<D, kFp8>(p, t, g, len, kb, ke, threadIdx.x, blockDim.x);
      __syncthreads();
    }
  }
  if constexpr (WP == 1 && D == 128 && !kFp8) {
    // four row blocks of one unit: every wave walks (the workgroup shares each tile through LDS)
    if (n_mine > 0)
      walk_tiles_shared<D>(st, q, p, trow, g, len, row_limit(p, len, qi), row_limit(p, len, 0), first, 1, n_mine,
                           &win0);
  } else {
    if (rb * 16 < R && n_mine > 0)
      walk_tiles<D, kFp8>(st, q, p, trow, g, len, row_limit(p, len, qi), row_limit(p, len, 0), first, WP, n_mine,
                          hook_tile, [&]() { store_step_tokens(p, tok); }, &win0);
  }

  st.l += __shfl_xor(st.l, 16, 64);
  st.l += __shfl_xor(st.l, 32, 64);

  // combine the WP tile-split waves of each row block through LDS
  if constexpr (WP > 1) {
    __shared__ float sm_ml[4][2][16];
    __shared__ f32x4 sm_o[4][64][DPL];
    if (j == 0) {
      sm_ml[wave][0][r_lane] = st.m;
      sm_ml[wave][1][r_lane] = st.l;
    }
#pragma unroll
    for (int tp = 0; tp < DPL; ++tp) sm_o[wave][lane][tp] = st.o[tp];
    __syncthreads();
    if (wp != 0) return;
    float m_all = kNegInf;
#pragma unroll
    for (int w = 0; w < WP; ++w) m_all = fmaxf(m_all, sm_ml[wave + w][0][r_lane]);
    const float m_use = m_all == kNegInf ? 0.f : m_all;
    float l_all = 0.f;
    f32x4 o_all[DPL];
#pragma unroll
    for (int tp = 0; tp < DPL; ++tp) o_all[tp] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int w = 0; w < WP; ++w) {
      const float f = fast_exp2(sm_ml[wave + w][0][r_lane] - m_use);
      l_all += f * sm_ml[wave + w][1][r_lane];
#pragma unroll
      for (int tp = 0; tp < DPL; ++tp) o_all[tp] += f * sm_o[wave + w][lane][tp];
    }
    st.m = m_all;
    st.l = l_all;
#pragma unroll
    for (int tp = 0; tp < DPL; ++tp) st.o[tp] = o_all[tp];
  }
  if (!row_ok) return;

  const bool empty = st.l == 0.f;
  const float inv = empty ? 0.f : 1.0f / st.l;
  const float lse = empty ? kNegInf : (st.m + fast_log2(st.l)) * kLn2;
  if (p.splits == 1 && !p.write_state) {
    store_row<D>(st, reinterpret_cast<uint8_t*>(p.out) + qrow * D * (p.out_bf16 ? 2 : 4), p.out_bf16, inv);
    if (p.out_lse && j == 0) p.out_lse[qrow] = lse;
  } else {
    const int64_t plane = (int64_t)p.num_tables * p.rows_per_table * p.num_q_heads;
    store_row<D>(st, p.ws_o + ((int64_t)s * plane + qrow) * D, false, inv);
    if (j == 0) p.ws_lse[(int64_t)s * plane + qrow] = lse;
  }
}

// Split kernel: grid (split, kv head, table row x row group).
template <int D, bool kFp8, int WP>
__global__ __launch_bounds__(256, 2) void decode_mfma_kernel(DecodeParams p) {
  // grid (tables x row groups, kv heads, splits): the table count takes the
  // x dimension, the only one not capped at 65535 blocks
  const int n_rg = gridDim.x / p.num_tables;
  const int t = blockIdx.x / n_rg;
  decode_block<D, kFp8, WP>(p, blockIdx.z, blockIdx.y, t, blockIdx.x - t * n_rg);
}

// Row blocks of 16 rows and waves per row block for R rows (as the split
// kernel's launcher chooses them).
__host__ __device__ constexpr int waves_per_block(int R) { return R <= 16 ? 4 : (R <= 32 ? 2 : 1); }
__host__ __device__ constexpr int row_groups_of(int R) { return R <= 32 ? 1 : ((R + 15) / 16 + 3) / 4; }

// n-sample step, prefix + tail in one launch ("Support shared-prefix attention
// for n-sample requests in FMHA": one kernel does the shared prefix, the
// private tails and, with the merge kernel after it, their merge).  Blocks
// [0, n_pre) are (prefix split, kv head, group, row group) work of `pre`: all
// samples' step tokens of a group share each prefix K/V tile.  The others are
// (tail, kv head, row group) work of `tail`, whose tokens are causal among
// themselves.  Each leaves a normalised state; the state of query row x is at
// row x of split s (prefix) or of split pre.splits (tail), so one N-state
// merge finishes the step.
template <int D, bool kFp8, int WPP, int WPT>
__global__ __launch_bounds__(256, 2) void shared_prefix_kernel(DecodeParams pre, DecodeParams tail, int n_pre) {
  const int b = blockIdx.x;
  if (b < n_pre) {
    const int s = b % pre.splits;
    const int rest = b / pre.splits;
    const int g = rest % pre.num_kv_heads;
    const int z = rest / pre.num_kv_heads;
    const int nrg = row_groups_of(pre.rows_per_table * pre.group);
    decode_block<D, kFp8, WPP>(pre, s, g, z / nrg, z % nrg);
  } else {
    const int bt = b - n_pre;
    const int g = bt % tail.num_kv_heads;
    const int z = bt / tail.num_kv_heads;
    const int nrg = row_groups_of(tail.rows_per_table * tail.group);
    decode_block<D, kFp8, WPT>(tail, 0, g, z / nrg, z % nrg);
  }
}

// Head-parallel stream-K worker (units of one 16-row block; kv heads a
// multiple of 4): a workgroup is one worker whose 4 waves take kv heads
// 4 hg .. 4 hg + 3 of the same keys.  The flattened positions are (table row
// t, head quad hg, tile k), cut into equal chunks, one per workgroup; every
// wave of a workgroup walks the same tiles, so the 4 heads' 256-byte segments
// of each key row (1 KiB, contiguous) are fetched together, and the other
// quads of the row are at the same offsets of their own chunks.  Slots: a
// cut unit's state goes to row 64 (2 w + s) + 16 wave + r of the workspace
// (s = 0 for the workgroup's first segment, 1 for its last).
template <int D, bool kFp8>
__device__ __forceinline__ void decode_sk_heads(const DecodeParams& p, const int32_t* cum, int R) {
  const int T = p.num_tables;
  const int HG = p.num_kv_heads >> 2;
  const int64_t N = (int64_t)cum[T] * HG;
  const int64_t C = (N + p.n_workers - 1) / p.n_workers;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int worker = blockIdx.x;
  const int lane = threadIdx.x & 63;
  const int r_lane = lane & 15, j = lane >> 4;
  const int64_t c_begin = (int64_t)worker * C;
  const int64_t c_end = c_begin + C < N ? c_begin + C : N;
  if (c_begin >= c_end) return;
  int t = 0;
  {
    int lo = 0, hi = T;   // invariant: cum[lo]*HG <= c_begin < cum[hi]*HG
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if ((int64_t)cum[mid] * HG <= c_begin) lo = mid; else hi = mid;
    }
    t = lo;
  }
  const bool row_ok = r_lane < R;
  int64_t c = c_begin;
  while (c < c_end) {
    const int tiles = cum[t + 1] - cum[t];
    if (tiles == 0) { ++t; continue; }
    const int64_t off = c - (int64_t)cum[t] * HG;
    const int hg = (int)(off / tiles);
    const int k0 = (int)(off - (int64_t)hg * tiles);
    const int k1 = (int64_t)tiles < k0 + (c_end - c) ? tiles : (int)(k0 + (c_end - c));
    const int g = 4 * hg + wave;
    int qi;
    int64_t qrow;
    row_of(p, t, g, row_ok ? r_lane : 0, qi, qrow);
    u32x4 q[D / 32];
    load_q<D, kFp8>(q, p, qrow, row_ok);
    RowState<D> st;
    reset_state(st);
    const int len = p.kv_lens[t];
    // The step's tokens (keys len - n .. len - 1) that fall in this
    // segment's tiles: this wave writes its kv head's rows, and only its own
    // walk reads them.  Up to 64 16-byte chunks (4 tokens of 128 bf16 dims)
    // are loaded now, one per lane, and stored just before the walk issues
    // the loads of the first tile that holds them, so the load latency hides
    // under the tiles before it; the wave's later loads of those rows follow
    // its stores in issue order.  More tokens are written before the walk.
    constexpr int CPR = D * (kFp8 ? 1 : 2) / 16;   // 16-byte chunks per row
    int hook_tile = -1;
    u32x4 tok_k = {0u, 0u, 0u, 0u}, tok_v = {0u, 0u, 0u, 0u};
    int64_t tok_dst = -1;
    if (p.new_k) {
      const int n = p.rows_per_table;
      const int kb = max(len - n, k0 * 32), ke = min(len, k1 * 32);
      if (kb < ke && (ke - kb) * CPR <= 64) {
        if (lane < (ke - kb) * CPR) {
          const int key = kb + lane / CPR, c = lane % CPR;
          const int64_t src = (int64_t)(t * n + key - (len - n)) * p.new_tok_stride_b +
                              (int64_t)g * p.new_head_stride_b + 16 * c;
          tok_k = *reinterpret_cast<const u32x4*>(p.new_k + src);
          tok_v = *reinterpret_cast<const u32x4*>(p.new_v + src);
          const int32_t* trow = p.table + (int64_t)t * p.table_stride;
          tok_dst = (int64_t)trow[key >> p.page_shift] * p.page_stride * (kFp8 ? 1 : 2) +
                    (int64_t)(key & ((1 << p.page_shift) - 1)) * p.num_kv_heads * D * (kFp8 ? 1 : 2) +
                    (int64_t)g * D * (kFp8 ? 1 : 2) + 16 * c;
        }
        hook_tile = kb / 32;
      } else if (kb < ke) {
        append_rows<D, kFp8>(p, t, g, len, kb, ke, lane, 64);
      }
    }
    auto store_tokens = [&]() {
      if (tok_dst >= 0) {
        *reinterpret_cast<u32x4*>(const_cast<uint8_t*>(reinterpret_cast<const uint8_t*>(p.k_pool)) + tok_dst) = tok_k;
        *reinterpret_cast<u32x4*>(const_cast<uint8_t*>(reinterpret_cast<const uint8_t*>(p.v_pool)) + tok_dst) = tok_v;
      }
      asm volatile("" ::: "memory");
    };
    walk_tiles<D, kFp8>(st, q, p, p.table + (int64_t)t * p.table_stride, g, len, row_limit(p, len, qi),
                        row_limit(p, len, 0), k0, 1, k1 - k0, hook_tile, store_tokens);
    st.l += __shfl_xor(st.l, 16, 64);
    st.l += __shfl_xor(st.l, 32, 64);
    const bool empty = st.l == 0.f;
    const float inv = empty ? 0.f : 1.0f / st.l;
    const float lse = empty ? kNegInf : (st.m + fast_log2(st.l)) * kLn2;
    if (row_ok) {
      if (k0 == 0 && k1 == tiles) {
        store_row<D>(st, reinterpret_cast<uint8_t*>(p.out) + qrow * D * (p.out_bf16 ? 2 : 4), p.out_bf16, inv);
        if (p.out_lse && j == 0) p.out_lse[qrow] = lse;
      } else {
        const int slot = 2 * worker + (c == c_begin ? 0 : 1);
        const int64_t prow = (int64_t)slot * 64 + wave * 16 + r_lane;
        store_row<D>(st, p.ws_o + prow * D, false, inv);
        if (j == 0) p.ws_lse[prow] = lse;
      }
    }
    c += k1 - k0;
    if (hg + 1 == HG) ++t;
  }
}

// ---------------------------------------------------------------------------
// Stream-K kernel: a persistent grid of workers (WR waves each: the row
// blocks of one (table row, kv head, row group) unit).  The flattened list of
// (unit, tile) positions is cut into equal contiguous chunks, one per worker,
// so every worker streams the same number of tiles whatever the length mix.
// A worker walks its chunk across unit boundaries: a unit it covers whole is
// stored as final output; a unit cut by a chunk boundary leaves a normalised
// partial state (output + LSE) in slot 2w (the worker's first segment) or
// 2w+1 (its last), joined afterwards by merge_sk_kernel.  The cut points
// depend only on the lengths, never on page ids, so results are independent
// of where pages sit in the pool.
// ---------------------------------------------------------------------------
// Prefix sums of the tiles per table row, cum[0..T], from kv_lens (every
// workgroup; ends with a barrier); workgroup 0 also leaves them in ws_cum for
// the merge.  Up to 64 rows: one wave's shuffle scan.
__device__ __forceinline__ void sk_prefix_sums(const DecodeParams& p, int32_t* cum, int32_t* part) {
  const int T = p.num_tables;
  if (T <= 64) {
    if (threadIdx.x < 64) {
      const int i = threadIdx.x;
      int v = i < T ? (p.kv_lens[i] + 31) >> 5 : 0;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const int u = __shfl_up(v, off, 64);
        if (i >= off) v += u;
      }
      if (i < T) cum[i + 1] = v;
      if (i == 0) cum[0] = 0;
    }
    __syncthreads();
  } else {
    const int per = (T + 255) / 256;
    const int lo = threadIdx.x * per;
    int run = 0;
    for (int i = 0; i < per && lo + i < T; ++i) run += (p.kv_lens[lo + i] + 31) >> 5;
    part[threadIdx.x] = run;
    __syncthreads();
    for (int off = 1; off < 256; off <<= 1) {
      const int v = threadIdx.x >= off ? part[threadIdx.x - off] : 0;
      __syncthreads();
      part[threadIdx.x] += v;
      __syncthreads();
    }
    int acc = part[threadIdx.x] - run;   // exclusive prefix of this thread's run
    for (int i = 0; i < per && lo + i < T; ++i) {
      cum[lo + i] = acc;
      acc += (p.kv_lens[lo + i] + 31) >> 5;
    }
    if (threadIdx.x == 255) cum[T] = part[255];
    __syncthreads();
  }
  if (blockIdx.x == 0)
    for (int i = threadIdx.x; i <= T; i += 256) p.ws_cum[i] = cum[i];
}

// Head-parallel stream-K kernel (see decode_sk_heads).
template <int D, bool kFp8>
__global__ __launch_bounds__(256, 2) void decode_skh_kernel(DecodeParams p) {
  __shared__ int32_t cum[kMaxSkTables + 1];
  __shared__ int32_t part[256];
  sk_prefix_sums(p, cum, part);
  decode_sk_heads<D, kFp8>(p, cum, p.rows_per_table * p.group);
}

template <int D, bool kFp8, int WR>
__global__ __launch_bounds__(256, 2) void decode_sk_kernel(DecodeParams p) {
  constexpr int WPW = 4 / WR;   // workers per workgroup
  __shared__ int32_t cum[kMaxSkTables + 1];
  __shared__ int32_t part[256];
  const int T = p.num_tables;
  sk_prefix_sums(p, cum, part);
  const int R = p.rows_per_table * p.group;
  const int HR = p.num_kv_heads * p.row_groups;   // units per table row
  const int64_t N = (int64_t)cum[T] * HR;
  const int64_t C = (N + p.n_workers - 1) / p.n_workers;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int worker = blockIdx.x * WPW + wave / WR;
  const int wr = wave - (wave / WR) * WR;
  const int lane = threadIdx.x & 63;
  const int r_lane = lane & 15, j = lane >> 4;
  const int64_t c_begin = (int64_t)worker * C;
  const int64_t c_end = c_begin + C < N ? c_begin + C : N;
  if (c_begin >= c_end) return;
  // the table row holding flattened position c_begin: largest t with cum[t]*HR <= c_begin
  int t = 0;
  {
    int lo = 0, hi = T;   // invariant: cum[lo]*HR <= c_begin < cum[hi]*HR
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if ((int64_t)cum[mid] * HR <= c_begin) lo = mid; else hi = mid;
    }
    t = lo;
  }
  int64_t c = c_begin;
  while (c < c_end) {
    const int tiles = cum[t + 1] - cum[t];
    if (tiles == 0) { ++t; continue; }
    const int64_t off = c - (int64_t)cum[t] * HR;
    const int ui = (int)(off / tiles);
    const int k0 = (int)(off - (int64_t)ui * tiles);
    const int k1 = (int64_t)tiles < k0 + (c_end - c) ? tiles : (int)(k0 + (c_end - c));
    const int g = ui / p.row_groups;
    const int rg = ui - g * p.row_groups;
    const int rb = rg * WR + wr;
    const int r = rb * 16 + r_lane;
    const bool row_ok = r < R;
    int qi;
    int64_t qrow;
    row_of(p, t, g, row_ok ? r : 0, qi, qrow);
    u32x4 q[D / 32];
    load_q<D, kFp8>(q, p, qrow, row_ok);
    RowState<D> st;
    reset_state(st);
    const int len = p.kv_lens[t];
    if constexpr (WR == 4 && D == 128 && !kFp8) {
      // one worker = the workgroup's four row blocks of one unit: every wave walks the segment
      walk_tiles_shared<D>(st, q, p, p.table + (int64_t)t * p.table_stride, g, len, row_limit(p, len, qi),
                           row_limit(p, len, 0), k0, 1, k1 - k0);
    } else {
      if (rb * 16 < R)
        walk_tiles<D, kFp8>(st, q, p, p.table + (int64_t)t * p.table_stride, g, len, row_limit(p, len, qi),
                            row_limit(p, len, 0), k0, 1, k1 - k0);
    }
    st.l += __shfl_xor(st.l, 16, 64);
    st.l += __shfl_xor(st.l, 32, 64);
    const bool empty = st.l == 0.f;
    const float inv = empty ? 0.f : 1.0f / st.l;
    const float lse = empty ? kNegInf : (st.m + fast_log2(st.l)) * kLn2;
    if (row_ok) {
      if (k0 == 0 && k1 == tiles) {
        store_row<D>(st, reinterpret_cast<uint8_t*>(p.out) + qrow * D * (p.out_bf16 ? 2 : 4), p.out_bf16, inv);
        if (p.out_lse && j == 0) p.out_lse[qrow] = lse;
      } else {
        const int slot = 2 * worker + (c == c_begin ? 0 : 1);
        const int64_t prow = (int64_t)slot * (16 * WR) + wr * 16 + r_lane;
        store_row<D>(st, p.ws_o + prow * D, false, inv);
        if (j == 0) p.ws_lse[prow] = lse;
      }
    }
    c += k1 - k0;
    if (ui + 1 == HR) ++t;
  }
}

// Joins the partial states of units cut by chunk boundaries, and writes the
// zero output / -inf LSE of table rows with no keys.  One thread per (row,
// 4 dims) of every unit; units a single worker finished are skipped.  The
// loads of each stage go out together (prefix sums, then LSEs and values of
// up to 8 pieces at a time), so a merge of up to 8 pieces costs two memory
// round trips rather than one per piece.
__global__ __launch_bounds__(256) void merge_sk_kernel(DecodeParams p, int wr_per_worker, int head_dim) {
  constexpr int PB = 8;
  const int D = head_dim;
  const int chunks = D >> 2;
  const int R = p.rows_per_table * p.group;
  const int64_t total = (int64_t)p.num_tables * p.num_kv_heads * R * chunks;
  const int64_t tid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (tid >= total) return;
  const int ch = (int)(tid % chunks);
  const int64_t rest = tid / chunks;
  const int r = (int)(rest % R);
  const int64_t tg = rest / R;
  const int g = (int)(tg % p.num_kv_heads);
  const int t = (int)(tg / p.num_kv_heads);
  const int rows_w = 16 * wr_per_worker;
  const int rg = r / rows_w;
  // head-parallel workers: position space (t, head quad, tile), 64 slot rows
  // per slot (4 waves x 16); otherwise (t, unit, tile), rows_w rows per slot
  const bool hp = p.head_par != 0;
  const int HR = hp ? (p.num_kv_heads >> 2) : p.num_kv_heads * p.row_groups;
  const int slot_rows = hp ? 64 : rows_w;
  const int slot_off = hp ? 16 * (g & 3) : 0;
  const int ux = hp ? (g >> 2) : g * p.row_groups + rg;
  const int T = p.num_tables;
  const int32_t cum_all = p.ws_cum[T], cum_t = p.ws_cum[t], cum_t1 = p.ws_cum[t + 1];
  const int64_t N = (int64_t)cum_all * HR;
  const int64_t C = (N + p.n_workers - 1) / p.n_workers;
  const int tiles = cum_t1 - cum_t;
  int qi;
  int64_t qrow;
  row_of(p, t, g, r, qi, qrow);
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  float lse_out = kNegInf;
  if (tiles > 0) {
    const int64_t F = (int64_t)cum_t * HR + (int64_t)ux * tiles;
    const int64_t w0 = F / C, w1 = (F + tiles - 1) / C;
    if (w0 == w1) return;   // finished by one worker
    const int row_in = slot_off + r - rg * rows_w;
    auto slot_row = [&](int64_t w) {
      const int64_t slot = (w == w0) ? (F == w0 * C ? 2 * w0 : 2 * w0 + 1) : 2 * w;
      return slot * slot_rows + row_in;
    };
    // one pass (LSE and outputs of PB pieces loaded together); the running
    // sums are rescaled when the running max grows
    float m = kNegInf, wsum = 0.f;
    for (int64_t w = w0; w <= w1; w += PB) {
      float l[PB];
      f32x4 v[PB];
#pragma unroll
      for (int j = 0; j < PB; ++j) {
        const bool ok = w + j <= w1;
        const int64_t sr = slot_row(ok ? w + j : w1);
        l[j] = ok ? p.ws_lse[sr] : kNegInf;
        v[j] = *reinterpret_cast<const f32x4*>(p.ws_o + sr * D + 4 * ch);
      }
      float mb = m;
#pragma unroll
      for (int j = 0; j < PB; ++j) mb = fmaxf(mb, l[j]);
      if (mb == kNegInf) continue;
      const float sc = m == kNegInf ? 0.f : fast_exp2((m - mb) * kLog2e);
      acc *= sc;
      wsum *= sc;
#pragma unroll
      for (int j = 0; j < PB; ++j) {
        // every piece holds keys, so its state is finite; padding entries weigh 0
        const float f = l[j] == kNegInf ? 0.f : fast_exp2((l[j] - mb) * kLog2e);
        acc += f * v[j];
        wsum += f;
      }
      m = mb;
    }
    if (m != kNegInf) {
      acc *= 1.0f / wsum;
      lse_out = m + fast_log2(wsum) * kLn2;
    }
  }
  const int64_t o_off = qrow * D + 4 * ch;
  if (p.out_bf16) {
    *reinterpret_cast<u32x2*>(reinterpret_cast<uint16_t*>(p.out) + o_off) =
        u32x2{pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3])};
  } else {
    *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(p.out) + o_off) = acc;
  }
  if (p.out_lse && ch == 0) p.out_lse[qrow] = lse_out;
}

// ---------------------------------------------------------------------------
// VALU kernel: one wave per (query row, split), fp32 arithmetic throughout.
// ---------------------------------------------------------------------------

template <int KV>
__device__ __forceinline__ float load_kv(const void* pool, int64_t idx) {
  if constexpr (KV == kF32) return reinterpret_cast<const float*>(pool)[idx];
  else if constexpr (KV == kBF16) return bf16_bits_to_f32(reinterpret_cast<const uint16_t*>(pool)[idx]);
  else return fp8x2_to_f32<false>(reinterpret_cast<const uint8_t*>(pool)[idx])[0];
}

template <int D, int QT, int KV>
__global__ __launch_bounds__(64) void decode_valu_kernel(DecodeParams p) {
  constexpr int DPT = D / 64;   // dims per lane in the PV product
  const int s = blockIdx.y;
  const int64_t qrow = blockIdx.x;   // (t * n + i) * Hq + h; x: not capped at 65535 blocks
  const int h = (int)(qrow % p.num_q_heads);
  const int t = (int)(qrow / ((int64_t)p.num_q_heads * p.rows_per_table));
  const int g = h / p.group;
  const int lane = threadIdx.x;
  const int len = p.kv_lens[t];
  const int tiles = (len + 31) >> 5;
  const int tb = s * p.tiles_per_split;
  int te = tb + p.tiles_per_split;
  te = te < tiles ? te : tiles;
  if (p.splits > 1 && tb >= te) return;
  const int kb = tb * 32;
  const int qi = (int)((qrow / p.num_q_heads) % p.rows_per_table);
  const int ke = min(te * 32, row_limit(p, len, qi));

  __shared__ float qs[D];
  for (int d = lane; d < D; d += 64) {
    if constexpr (QT == kF32) qs[d] = reinterpret_cast<const float*>(p.q)[qrow * D + d];
    else qs[d] = bf16_bits_to_f32(reinterpret_cast<const uint16_t*>(p.q)[qrow * D + d]);
  }
  __syncthreads();

  const int32_t* trow = p.table + (int64_t)t * p.table_stride;
  const int mask = (1 << p.page_shift) - 1;
  const int64_t row_elems = (int64_t)p.num_kv_heads * D;
  float m = kNegInf, l = 0.f;
  float o[DPT];
#pragma unroll
  for (int e = 0; e < DPT; ++e) o[e] = 0.f;

  for (int key0 = kb; key0 < ke; key0 += 64) {
    const int key = key0 + lane;
    float sc = kNegInf;
    int64_t kbase = 0;
    float kscale = 1.f;
    if (key < ke) {
      const int page = trow[key >> p.page_shift];
      kbase = (int64_t)page * p.page_stride + (int64_t)(key & mask) * row_elems + (int64_t)g * D;
      if constexpr (KV == kFP8) kscale = p.k_scale[(int64_t)page * p.num_kv_heads + g];
      float acc = 0.f;
      for (int d = 0; d < D; ++d) acc = fmaf(qs[d], load_kv<KV>(p.k_pool, kbase + d), acc);
      sc = acc * kscale * p.scale_log2;
    }
    float mt = sc;
#pragma unroll
    for (int x = 32; x >= 1; x >>= 1) mt = wave_max_xor(mt, x);
    const float m_new = fmaxf(m, mt);
    const float m_use = m_new == kNegInf ? 0.f : m_new;
    const float alpha = fast_exp2(m - m_use);
    const float pk = fast_exp2(sc - m_use);
    float ps = pk;
#pragma unroll
    for (int x = 32; x >= 1; x >>= 1) ps = wave_sum_xor(ps, x);
    l = l * alpha + ps;
    m = m_new;
#pragma unroll
    for (int e = 0; e < DPT; ++e) o[e] *= alpha;
    const int n_here = min(64, ke - key0);
    for (int kk = 0; kk < n_here; ++kk) {
      const float pj = __shfl(pk, kk, 64);
      const int kj = key0 + kk;
      const int page = trow[kj >> p.page_shift];
      float vscale = 1.f;
      if constexpr (KV == kFP8) vscale = p.v_scale[(int64_t)page * p.num_kv_heads + g];
      const int64_t vbase = (int64_t)page * p.page_stride + (int64_t)(kj & mask) * row_elems + (int64_t)g * D;
#pragma unroll
      for (int e = 0; e < DPT; ++e) o[e] = fmaf(pj * vscale, load_kv<KV>(p.v_pool, vbase + lane + 64 * e), o[e]);
    }
  }
  const bool empty = l == 0.f;
  const float inv = empty ? 0.f : 1.0f / l;
  const float lse = empty ? kNegInf : (m + fast_log2(l)) * kLn2;
  if (p.splits == 1) {
#pragma unroll
    for (int e = 0; e < DPT; ++e) {
      const int64_t idx = qrow * D + lane + 64 * e;
      if (p.out_bf16) reinterpret_cast<uint16_t*>(p.out)[idx] = f32_to_bf16_bits(o[e] * inv);
      else reinterpret_cast<float*>(p.out)[idx] = o[e] * inv;
    }
    if (p.out_lse && lane == 0) p.out_lse[qrow] = lse;
  } else {
    const int64_t plane = (int64_t)p.num_tables * p.rows_per_table * p.num_q_heads;
#pragma unroll
    for (int e = 0; e < DPT; ++e) p.ws_o[((int64_t)s * plane + qrow) * D + lane + 64 * e] = o[e] * inv;
    if (lane == 0) p.ws_lse[(int64_t)s * plane + qrow] = lse;
  }
}

// ---------------------------------------------------------------------------

template <int D, bool kFp8>
static hipError_t launch_mfma_d(const DecodeParams& p, hipStream_t stream) {
  const int R = p.rows_per_table * p.group;
  const int blocks16 = (R + 15) / 16;
  const dim3 block(256);
  if (blocks16 <= 1) {
    const dim3 grid(p.num_tables, p.num_kv_heads, p.splits);
    PKV_LAUNCH_MAIN((decode_mfma_kernel<D, kFp8, 4>), grid, block, 0, stream, p);
  } else if (blocks16 <= 2) {
    const dim3 grid(p.num_tables, p.num_kv_heads, p.splits);
    PKV_LAUNCH_MAIN((decode_mfma_kernel<D, kFp8, 2>), grid, block, 0, stream, p);
  } else {
    const int rg = (blocks16 + 3) / 4;
    const dim3 grid(p.num_tables * rg, p.num_kv_heads, p.splits);
    PKV_LAUNCH_MAIN((decode_mfma_kernel<D, kFp8, 1>), grid, block, 0, stream, p);
  }
  return hipGetLastError();
}

hipError_t launch_decode_mfma(const DecodeParams& p, ElemType kv, int head_dim, hipStream_t stream) {
  if (head_dim == 128) return kv == kFP8 ? launch_mfma_d<128, true>(p, stream) : launch_mfma_d<128, false>(p, stream);
  return kv == kFP8 ? launch_mfma_d<64, true>(p, stream) : launch_mfma_d<64, false>(p, stream);
}

int sk_waves_per_worker(int rows_per_unit) {
  const int blocks16 = (rows_per_unit + 15) / 16;
  return blocks16 <= 1 ? 1 : blocks16 <= 2 ? 2 : 4;
}

template <int D, bool kFp8, int WR>
static hipError_t launch_sk_dw(DecodeParams p, int sm_count, hipStream_t stream) {
  // one 16-row block per unit and kv heads in quads: head-parallel workgroups
  p.head_par = sk_head_parallel(WR, p.row_groups, p.num_kv_heads) ? 1 : 0;
  // One workgroup per CU.  With two per CU the first-resident one wins issue
  // and ends early while the other runs on alone, so one per CU loses no
  // bandwidth and walks chunks twice as long, with half the cut pieces and
  // start-ups.  Measured against two per CU: GQA call 0.1223 -> 0.1195 ms,
  // long fp8 decode 0.849 -> 0.844 ms, n-sample prefix (64-row units) and
  // tails 3 % each, 16 q / 2 kv heads 0.0390 -> 0.0359 ms; 192 workgroups ran
  // the same as 256, 128, 320 and 384 slower.
  const int grid = sm_count < kMaxSkWaves / 4 ? sm_count : kMaxSkWaves / 4;
  if (p.head_par) {
    p.n_workers = grid;
    PKV_LAUNCH_MAIN((decode_skh_kernel<D, kFp8>), dim3(grid), dim3(256), 0, stream, p);
  } else {
    p.n_workers = grid * (4 / WR);
    PKV_LAUNCH_MAIN((decode_sk_kernel<D, kFp8, WR>), dim3(grid), dim3(256), 0, stream, p);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int R = p.rows_per_table * p.group;
  const int64_t total = (int64_t)p.num_tables * p.num_kv_heads * R * (D / 4);
  hipLaunchKernelGGL(merge_sk_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, stream, p, WR, D);
  return hipGetLastError();
}

template <int D, bool kFp8>
static hipError_t launch_sk_d(const DecodeParams& p, int sm_count, hipStream_t stream) {
  switch (sk_waves_per_worker(p.rows_per_table * p.group)) {
    case 1: return launch_sk_dw<D, kFp8, 1>(p, sm_count, stream);
    case 2: return launch_sk_dw<D, kFp8, 2>(p, sm_count, stream);
    default: return launch_sk_dw<D, kFp8, 4>(p, sm_count, stream);
  }
}

template <int D, bool kFp8, int WPP>
static hipError_t launch_shared_d(const DecodeParams& pre, const DecodeParams& tail, int n_pre, int n_all,
                                  hipStream_t stream) {
  const int wpt = waves_per_block(tail.rows_per_table * tail.group);
  if (wpt == 4)
    hipLaunchKernelGGL((shared_prefix_kernel<D, kFp8, WPP, 4>), dim3(n_all), dim3(256), 0, stream, pre, tail, n_pre);
  else if (wpt == 2)
    hipLaunchKernelGGL((shared_prefix_kernel<D, kFp8, WPP, 2>), dim3(n_all), dim3(256), 0, stream, pre, tail, n_pre);
  else
    hipLaunchKernelGGL((shared_prefix_kernel<D, kFp8, WPP, 1>), dim3(n_all), dim3(256), 0, stream, pre, tail, n_pre);
  return hipGetLastError();
}

template <int D, bool kFp8>
static hipError_t launch_shared_dk(const DecodeParams& pre, const DecodeParams& tail, hipStream_t stream) {
  const int rp = pre.rows_per_table * pre.group, rt = tail.rows_per_table * tail.group;
  const int64_t n_pre = (int64_t)pre.splits * pre.num_kv_heads * pre.num_tables * row_groups_of(rp);
  const int64_t n_all = n_pre + (int64_t)tail.num_kv_heads * tail.num_tables * row_groups_of(rt);
  if (n_all == 0) return hipSuccess;
  const int wpp = waves_per_block(rp);
  if (wpp == 4) return launch_shared_d<D, kFp8, 4>(pre, tail, (int)n_pre, (int)n_all, stream);
  if (wpp == 2) return launch_shared_d<D, kFp8, 2>(pre, tail, (int)n_pre, (int)n_all, stream);
  return launch_shared_d<D, kFp8, 1>(pre, tail, (int)n_pre, (int)n_all, stream);
}

hipError_t launch_shared_prefix(const DecodeParams& pre, const DecodeParams& tail, ElemType kv, int head_dim,
                                hipStream_t stream) {
  const bool fp8 = kv == kFP8;
  if (head_dim == 128)
    return fp8 ? launch_shared_dk<128, true>(pre, tail, stream) : launch_shared_dk<128, false>(pre, tail, stream);
  return fp8 ? launch_shared_dk<64, true>(pre, tail, stream) : launch_shared_dk<64, false>(pre, tail, stream);
}

hipError_t launch_decode_sk(const DecodeParams& p, ElemType kv, int head_dim, int sm_count, hipStream_t stream) {
  if (head_dim == 128) return kv == kFP8 ? launch_sk_d<128, true>(p, sm_count, stream) : launch_sk_d<128, false>(p, sm_count, stream);
  return kv == kFP8 ? launch_sk_d<64, true>(p, sm_count, stream) : launch_sk_d<64, false>(p, sm_count, stream);
}

template <int D, int QT>
static hipError_t launch_valu_dq(const DecodeParams& p, ElemType kv, hipStream_t stream) {
  const dim3 grid((unsigned)((int64_t)p.num_tables * p.rows_per_table * p.num_q_heads), p.splits), block(64);
  if (kv == kF32) PKV_LAUNCH_MAIN((decode_valu_kernel<D, QT, kF32>), grid, block, 0, stream, p);
  else if (kv == kBF16) PKV_LAUNCH_MAIN((decode_valu_kernel<D, QT, kBF16>), grid, block, 0, stream, p);
  else PKV_LAUNCH_MAIN((decode_valu_kernel<D, QT, kFP8>), grid, block, 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_decode_valu(const DecodeParams& p, ElemType q, ElemType kv, int head_dim, hipStream_t stream) {
  if (head_dim == 128) return q == kF32 ? launch_valu_dq<128, kF32>(p, kv, stream) : launch_valu_dq<128, kBF16>(p, kv, stream);
  return q == kF32 ? launch_valu_dq<64, kF32>(p, kv, stream) : launch_valu_dq<64, kBF16>(p, kv, stream);
}

}  // namespace pkv
