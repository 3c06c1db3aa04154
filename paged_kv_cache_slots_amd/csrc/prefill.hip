// Block-causal paged prefill on bf16 MFMA.
//
// "Paged causal K/V cache and cached attention for VisualGen", Description /
// Cache: a forward's new tokens are cut into causal blocks that run as one
// ragged batch over the same block table, each block with its own key count;
// attention is full inside a block and causal across blocks, so no mask is
// needed beyond a per-query key limit.  Description / Attention: seq_len is
// the number of real query tokens; padding rows are neither attended nor
// attending and come back zero.
//
// Query row i < seq_len sees logical keys [0, n_ctx + min((i / cbs + 1) * cbs,
// seq_len)) of its table row; rows i >= seq_len get o = 0, lse = -inf.
//
// Work unit: 128 query rows of one query head (a q-tile).  Its keys are walked
// in tiles of 64.  A workgroup has 8 waves: 4 row blocks of 32 query rows x 2
// key halves (keys 0-31 / 32-63 of every tile).  Both waves of a row block
// share a SIMD and keep their own softmax state; they are joined at the end
// of a segment with the log-sum-exp merge.
//
//   * S^T[key][q] = K Q^T on v_mfma_f32_32x32x16_bf16 (A = K rows from LDS,
//     B = Q held in registers): each lane owns one query row and 16 keys.
//   * O^T[d][q] += V^T P^T on the same MFMA: P^T is the score registers in
//     bf16 (no shuffle); V^T operands come straight from the row-major V tile
//     through ds_read_b64_tr_b16 (each 16-lane group reads a 4-key x 16-dim
//     block and gets it transposed), so staging never transposes.
//   * Software pipeline: the QK^T MFMAs of tile t+1 are issued before the
//     softmax of tile t, so matrix cores and vector ALUs overlap within a wave.
//     K runs one tile ahead of V through two LDS buffers each; one barrier per
//     tile.  Global loads for the next stage are issued a full tile ahead.
//   * Loads never branch: keys at or past the unit's last visible key read a
//     valid row and are replaced by zeros, so dead page slots and table
//     entries past the last page never reach a product (and are never read).
//   * Schedule: a persistent grid, one 8-wave workgroup per CU.  Each XCD
//     (workgroup id mod 8) owns whole kv heads; its workgroups first run whole
//     units in rounds, all in lockstep along the keys, so every K/V tile of a
//     head is fetched once into the XCD's L2 and reused by all of its q-tiles.
//     The units left over after the last full round (fewer than the XCD's
//     workgroups) are split evenly along the keys over all of them (stream-K,
//     with a workspace): a unit cut into pieces leaves normalised partial
//     states, which a second, small kernel merges.  (Merging inside the main
//     kernel would need agent-scope fences; on this chip those write back and
//     invalidate the XCD's whole L2, evicting the K/V tiles every other
//     workgroup there is streaming.)  Without a workspace the leftover units
//     simply run whole.
#include "pkv_device.hpp"
#include "pkv_internal.hpp"

namespace pkv {

namespace {

constexpr int kKT = 64;            // keys per tile
constexpr int kQT = 128;           // query rows per unit
constexpr int kThreads = 512;      // 8 waves
constexpr int kTableCache = 1024;  // page ids cached in LDS
constexpr int kSlotFloats = 4 * 65 * 64;   // partial state: [row block][64 outputs + lse][lane]

template <int D>
struct PSmem {
  static constexpr int KROW = D * 2 + 16;   // odd multiple of 16 B: conflict-free 16-B row reads
  static constexpr int VROW = D * 2 + 64;   // 64 mod 256 B: the 4 rows x 2 dim halves of a transpose read hit distinct banks
  static constexpr int KB = kKT * KROW;
  static constexpr int VB = kKT * VROW;
  static constexpr int STAGES = 2 * KB + 2 * VB;
  static constexpr int COMBINE = 4 * 66 * 64 * 4;   // [row block][64 + 2 values][lane] floats
  static constexpr int BYTES = STAGES > COMBINE ? STAGES : COMBINE;
};

__device__ __forceinline__ int visible_keys(int i, int n_ctx, int seq, int cbs) {
  if (i >= seq) return 0;
  const int e = (i / cbs + 1) * cbs;
  return n_ctx + (e < seq ? e : seq);
}

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16* lds_v4i16_ptr;

// Transposed 8-byte LDS read (ds_read_b64_tr_b16): within each 16-lane group,
// lane o receives element (o % 4) of the 4-element rows addressed by lanes
// o / 4 + 4 i, i = 0..3.
__device__ __forceinline__ u32x2 lds_read_tr(const uint8_t* ptr) {
  const v4i16 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_v4i16_ptr)((__attribute__((address_space(3))) uint8_t*)(ptr)));
  return __builtin_bit_cast(u32x2, r);
}

// A unit: (batch, kv head, query head of the group, q-tile).
struct Unit {
  int b, g, h, row0, n_ctx, seq, cbs, kmax, tiles;
};

__device__ __forceinline__ Unit unit_of(const PrefillParams& p, int u) {
  Unit x;
  const int qt = u % p.q_tiles;
  const int r = u / p.q_tiles;
  const int hh = r % p.group;
  const int kvu = r / p.group;
  x.b = kvu / p.num_kv_heads;
  x.g = kvu - x.b * p.num_kv_heads;
  x.h = x.g * p.group + hh;
  x.row0 = qt * kQT;
  x.n_ctx = p.n_ctx[x.b];
  x.seq = p.seq_len[x.b];
  x.cbs = p.causal_block_size > 0 ? p.causal_block_size : (x.seq > 0 ? x.seq : 1);
  const int last = (x.row0 + kQT - 1 < x.seq - 1) ? x.row0 + kQT - 1 : x.seq - 1;
  x.kmax = x.row0 < x.seq ? visible_keys(last, x.n_ctx, x.seq, x.cbs) : 0;
  x.tiles = (x.kmax + kKT - 1) / kKT;
  return x;
}

// Schedule of one XCD: which units it owns, how many run whole in rounds, and
// the leftover ones split along the keys.  Shared by both kernels so that the
// merge finds the pieces where the main kernel left them.
struct XcdPlan {
  int per_kv;     // units per kv unit (query heads of the group x q-tiles)
  int ux;         // units owned by the XCD
  int dp_units;   // units run whole, in rounds
  int nt;         // leftover units (split when sk)
  int xcd;
  bool sk;
  __device__ int global_unit(int j) const { return (xcd + 8 * (j / per_kv)) * per_kv + j % per_kv; }
};

__device__ __forceinline__ XcdPlan xcd_plan(const PrefillParams& p, int xcd, int gx) {
  XcdPlan s;
  const int kv_units = p.batch * p.num_kv_heads;
  s.per_kv = p.group * p.q_tiles;
  const int nkv = kv_units > xcd ? (kv_units - xcd + 7) / 8 : 0;
  s.ux = nkv * s.per_kv;
  s.sk = p.ws_o != nullptr && s.ux % gx != 0 && s.ux % gx <= kMaxTailUnits;
  s.dp_units = s.sk ? (s.ux / gx) * gx : s.ux;
  s.nt = s.ux - s.dp_units;
  s.xcd = xcd;
  return s;
}

// Prefix sums of the tiles of the XCD's leftover units (cum[0..nt]); called
// by the whole workgroup, ends with a barrier.
__device__ __forceinline__ void tail_prefix(const PrefillParams& p, const XcdPlan& s, int32_t* cum) {
  for (int k = threadIdx.x; k < s.nt; k += blockDim.x) cum[k + 1] = unit_of(p, s.global_unit(s.dp_units + k)).tiles;
  __syncthreads();
  if (threadIdx.x == 0) {
    cum[0] = 0;
    for (int k = 1; k <= s.nt; ++k) cum[k] += cum[k - 1];
  }
  __syncthreads();
}

__device__ __forceinline__ int64_t tail_chunk(int64_t tiles, int gx) {
  const int64_t c = (tiles + gx - 1) / gx;
  return c > 0 ? c : 1;
}

// Store this lane's part of a finished output row: the lane holds dims
// 32 d + 8 (i / 4) + 4 hf + (i % 4) of row `row` of query head h.
template <int D>
__device__ __forceinline__ void store_rows(const PrefillParams& p, int b, int h, int row, int hf,
                                           const f32x16 (&v)[D / 32], float lse) {
  if (row >= p.s_q) return;
  const int64_t orow = ((int64_t)b * p.s_q + row) * p.num_q_heads + h;
  if (p.out_bf16) {
    uint16_t* op = reinterpret_cast<uint16_t*>(p.out) + orow * D;
#pragma unroll
    for (int d = 0; d < D / 32; ++d)
#pragma unroll
      for (int a = 0; a < 4; ++a)
        *reinterpret_cast<u32x2*>(op + 32 * d + 8 * a + 4 * hf) =
            u32x2{pack_bf16x2(v[d][4 * a], v[d][4 * a + 1]), pack_bf16x2(v[d][4 * a + 2], v[d][4 * a + 3])};
  } else {
    float* op = reinterpret_cast<float*>(p.out) + orow * D;
#pragma unroll
    for (int d = 0; d < D / 32; ++d)
#pragma unroll
      for (int a = 0; a < 4; ++a)
        *reinterpret_cast<f32x4*>(op + 32 * d + 8 * a + 4 * hf) =
            f32x4{v[d][4 * a], v[d][4 * a + 1], v[d][4 * a + 2], v[d][4 * a + 3]};
  }
  if (p.out_lse && hf == 0) p.out_lse[orow] = lse;
}

}  // namespace

template <int D>
__global__ __launch_bounds__(kThreads, 1) void prefill_kernel(PrefillParams p) {
  using S = PSmem<D>;
  constexpr int KSTEPS = D / 16;   // k-steps of QK^T
  constexpr int DB = D / 32;       // 32-dim output blocks
  constexpr int LPR = D / 32;      // 16-byte loads per staging thread (a quarter of a row)
  __shared__ __attribute__((aligned(16))) uint8_t smem[S::BYTES];
  __shared__ int32_t pages[kTableCache];
  __shared__ int32_t tcum[kMaxTailUnits + 1];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int ln = lane & 31, hf = lane >> 5;
  const int rb = wave & 3, kh = wave >> 2;
  const float c = p.scale_log2;

  // ---- schedule: XCD xcd owns kv units xcd, xcd + 8, ...; its Gx workgroups
  // run whole units in lockstep rounds, then split the leftover ones
  const int wi = blockIdx.x >> 3;
  const int Gx = gridDim.x >> 3;
  const XcdPlan plan = xcd_plan(p, blockIdx.x & 7, Gx);

  const int shift = p.page_shift;
  const int pmask = (1 << shift) - 1;
  const int64_t row_elems = (int64_t)p.num_kv_heads * D;
  const uint16_t* kpool = reinterpret_cast<const uint16_t*>(p.k_pool);
  const uint16_t* vpool = reinterpret_cast<const uint16_t*>(p.v_pool);
  uint8_t* kbuf0 = smem;
  uint8_t* vbuf0 = smem + 2 * S::KB;
  // staging role: waves 0-3 stage K rows, waves 4-7 V rows; 4 threads per row
  const bool stage_k = tid < 256;
  const int srow = (tid & 255) >> 2;   // key row within a tile
  const int squart = tid & 3;          // quarter of the row (D/4 dims)


  // one segment: tiles [t0, t1) of unit u (ut tiles in all).  F and C place
  // the segment in the XCD's stream-K order when it is a piece of a split unit.
  auto run = [&](int u, int t0, int t1, int ut, bool first_seg) {
    const Unit x = unit_of(p, u);
    const int32_t* trow = p.table + (int64_t)x.b * p.table_stride;
    const int my_row = x.row0 + 32 * rb + ln;
    const int my_lim = visible_keys(my_row, x.n_ctx, x.seq, x.cbs);
    const int wrow0 = x.row0 + 32 * rb;
    const int wmin = (wrow0 + 31 < x.seq) ? visible_keys(wrow0, x.n_ctx, x.seq, x.cbs) : 0;

    // Q operand of this row block: row ln, dims 16 s + 8 hf .. +8
    u32x4 q[KSTEPS];
    {
      const bool ok = my_row < x.seq;
      const uint16_t* qp =
          p.q + ((int64_t)x.b * p.s_q + (ok ? my_row : 0)) * p.q_tok_stride + (int64_t)x.h * p.q_head_stride;
#pragma unroll
      for (int s = 0; s < KSTEPS; ++s) q[s] = ok ? ld16(qp + 16 * s + 8 * hf) : u32x4{0u, 0u, 0u, 0u};
    }

    f32x16 o[DB];
#pragma unroll
    for (int d = 0; d < DB; ++d) o[d] = f32x16{};
    float mc = kNegInf, l = 0.f;   // exponent offset (log2 units) and running sum of this wave

    if (t1 > t0) {
      // page ids of the walked keys, refreshed if the segment spans more pages
      int page_base = (t0 * kKT) >> shift;
      const int last_page = (x.kmax - 1) >> shift;
      auto cache_pages = [&](int first) {
        __syncthreads();
        for (int i = tid; i < kTableCache && first + i <= last_page; i += kThreads) pages[i] = trow[first + i];
        page_base = first;
        __syncthreads();
      };
      cache_pages(page_base);

      // staging: this thread's 16-byte pieces of one key row (K or V) of tile t
      u32x4 st[LPR];
      auto fetch = [&](int t) {
        int key = t * kKT + srow;
        key = key < x.kmax ? key : x.kmax - 1;   // clamp: always a valid row; replaced by zeros below
        const int pg = pages[(key >> shift) - page_base];
        const uint16_t* src = (stage_k ? kpool : vpool) + (int64_t)pg * p.page_stride +
                              (int64_t)(key & pmask) * row_elems + (int64_t)x.g * D;
        // K: a contiguous quarter row per thread; V: 16-byte pieces squart, squart + 4, ...
        // (each layout keeps 16 consecutive lanes on distinct LDS banks when stored)
#pragma unroll
        for (int e = 0; e < LPR; ++e) st[e] = ld16(src + (stage_k ? (D / 4) * squart + 8 * e : 8 * (squart + 4 * e)));
      };
      auto commit = [&](int t, bool want_k, bool want_v) {
        const bool live = t * kKT + srow < x.kmax;
        if (stage_k ? want_k : want_v) {
          uint8_t* dst = stage_k ? kbuf0 + (t & 1) * S::KB + srow * S::KROW + (D / 2) * squart
                                 : vbuf0 + (t & 1) * S::VB + srow * S::VROW + 16 * squart;
#pragma unroll
          for (int e = 0; e < LPR; ++e)
            *reinterpret_cast<u32x4*>(dst + (stage_k ? 16 * e : 64 * e)) = live ? st[e] : u32x4{0u, 0u, 0u, 0u};
        }
      };
      // S^T for this wave's key half of tile t (K buffer t & 1)
      auto qk = [&](int t) {
        f32x16 acc = f32x16{};
        const uint8_t* krow = kbuf0 + (t & 1) * S::KB + (32 * kh + ln) * S::KROW + 16 * hf;
#pragma unroll
        for (int s = 0; s < KSTEPS; ++s)
          acc = mfma32x32x16_bf16(*reinterpret_cast<const u32x4*>(krow + 32 * s), q[s], acc);
        return acc;
      };

      // prologue: K(t0), V(t0) -> LDS; S(t0); K(t0+1) -> LDS
      const bool need_refresh = ((t1 * kKT - 1) >> shift) - page_base >= kTableCache;
      fetch(t0);
      commit(t0, true, true);
      __syncthreads();
      f32x16 sc = qk(t0);
      if (t0 + 1 < t1) {
        fetch(t0 + 1);
        commit(t0 + 1, true, false);
      }
      __syncthreads();

      for (int t = t0; t < t1; ++t) {
        // invariant: LDS holds K(t+1) (if any) and V(t); sc = S^T(t)
        const bool more_k = t + 2 < t1, more_v = t + 1 < t1;
        if (need_refresh && more_v) {
          const int want = (((more_k ? t + 2 : t + 1) * kKT + kKT - 1) >> shift) - page_base;
          if (want >= kTableCache) cache_pages(((t + 1) * kKT) >> shift);
        }
        // global loads of the next stage: K(t+2) or V(t+1), by role
        if (stage_k ? more_k : more_v) fetch(stage_k ? t + 2 : t + 1);
        // QK^T of tile t+1 (its MFMAs overlap the softmax below)
        f32x16 sn = f32x16{};
        if (more_v) sn = qk(t + 1);
        // ---- softmax of tile t (this wave's 32 keys, row = lane & 31)
        const int key0 = t * kKT + 32 * kh;
        if (key0 + 32 > wmin) {
#pragma unroll
          for (int i = 0; i < 16; ++i)
            if (key0 + 8 * (i >> 2) + 4 * hf + (i & 3) >= my_lim) sc[i] = kNegInf;
        }
        float mt = kNegInf;
#pragma unroll
        for (int i = 0; i < 16; ++i) mt = fmaxf(mt, sc[i]);
        mt = fmaxf(mt, __shfl_xor(mt, 32, 64));
        const float mtc = mt * c;
        const bool grow = mtc > mc + 8.0f;   // lazy rescale: the offset moves only by > 2^8
        if (__any(grow)) {
          const float mc_new = grow ? mtc : mc;
          const float alpha = (mc == kNegInf) ? 0.f : fast_exp2(mc - mc_new);
          l *= alpha;
#pragma unroll
          for (int d = 0; d < DB; ++d) o[d] *= alpha;
          mc = mc_new;
        }
        const float mcu = (mc == kNegInf) ? 0.f : mc;
        u32x4 pb[2];
        float psum = 0.f;
#pragma unroll
        for (int mu = 0; mu < 2; ++mu)
#pragma unroll
          for (int q2 = 0; q2 < 4; ++q2) {
            const float e0 = fast_exp2(fmaf(sc[8 * mu + 2 * q2], c, -mcu));
            const float e1 = fast_exp2(fmaf(sc[8 * mu + 2 * q2 + 1], c, -mcu));
            psum += e0 + e1;
            pb[mu][q2] = pack_bf16x2(e0, e1);
          }
        l += psum;
        // ---- O^T += V^T P^T: V^T operands by transposed LDS reads
        {
          const uint8_t* vb = vbuf0 + (t & 1) * S::VB;
          const int s16 = lane & 15;
          const int dh = (lane >> 4) & 1;
#pragma unroll
          for (int mu = 0; mu < 2; ++mu) {
            const int kb = 32 * kh + 16 * mu + 4 * hf + (s16 >> 2);
#pragma unroll
            for (int d = 0; d < DB; ++d) {
              const uint8_t* a0 = vb + kb * S::VROW + (32 * d + 16 * dh + 4 * (s16 & 3)) * 2;
              const u32x2 lo = lds_read_tr(a0);
              const u32x2 hi = lds_read_tr(a0 + 8 * S::VROW);
              o[d] = mfma32x32x16_bf16(u32x4{lo[0], lo[1], hi[0], hi[1]}, pb[mu], o[d]);
            }
          }
        }
        commit(stage_k ? t + 2 : t + 1, more_k, more_v);
        __syncthreads();
        sc = sn;
      }
    }

    // ---- join the two key halves of each row block through LDS
    l += __shfl_xor(l, 32, 64);
    __syncthreads();
    float* cmb = reinterpret_cast<float*>(smem) + rb * 66 * 64;   // [66][64] floats per row block
    if (kh == 1) {
#pragma unroll
      for (int d = 0; d < DB; ++d)
#pragma unroll
        for (int i = 0; i < 16; ++i) cmb[(16 * d + i) * 64 + lane] = o[d][i];
      cmb[64 * 64 + lane] = mc;
      cmb[65 * 64 + lane] = l;
    }
    __syncthreads();
    float lse = kNegInf;
    if (kh == 0) {
      const float mc1 = cmb[64 * 64 + lane], l1 = cmb[65 * 64 + lane];
      const float mx = fmaxf(mc, mc1);
      const float mxu = mx == kNegInf ? 0.f : mx;
      const float f0 = mc == kNegInf ? 0.f : fast_exp2(mc - mxu);
      const float f1 = mc1 == kNegInf ? 0.f : fast_exp2(mc1 - mxu);
      l = f0 * l + f1 * l1;
      const float inv = l == 0.f ? 0.f : 1.0f / l;
#pragma unroll
      for (int d = 0; d < DB; ++d)
#pragma unroll
        for (int i = 0; i < 16; ++i) o[d][i] = (f0 * o[d][i] + f1 * cmb[(16 * d + i) * 64 + lane]) * inv;
      lse = l == 0.f ? kNegInf : (mx + fast_log2(l)) * kLn2;
    }
    const bool whole = t0 == 0 && t1 == ut;
    if (whole) {
      if (kh == 0) store_rows<D>(p, x.b, x.h, my_row, hf, o, lse);
    } else if (kh == 0) {
      // partial state -> slot (2 per workgroup: its chunk's first / last
      // segment); prefill_merge_kernel combines the pieces after this kernel
      float* ps = p.ws_o + (2 * (int64_t)blockIdx.x + (first_seg ? 0 : 1)) * kSlotFloats;
#pragma unroll
      for (int d = 0; d < DB; ++d)
#pragma unroll
        for (int i = 0; i < 16; ++i) ps[(rb * 65 + 16 * d + i) * 64 + lane] = o[d][i];
      ps[(rb * 65 + 64) * 64 + lane] = lse;
    }
    __syncthreads();
  };

  for (int j = wi; j < plan.dp_units; j += Gx) {
    const int u = plan.global_unit(j);
    const int ut = unit_of(p, u).tiles;
    run(u, 0, ut, ut, true);
  }
  if (!plan.sk) return;

  // ---- leftover units of this XCD, split evenly along the keys
  tail_prefix(p, plan, tcum);
  const int nt = plan.nt;
  // leftover units without keys (q-tiles past seq_len) only need zero rows
  for (int k = wi; k < nt; k += Gx)
    if (tcum[k + 1] == tcum[k]) run(plan.global_unit(plan.dp_units + k), 0, 0, 0, true);
  const int64_t N = tcum[nt];
  const int64_t C = tail_chunk(N, Gx);
  const int64_t c_begin = (int64_t)wi * C;
  const int64_t c_end = c_begin + C < N ? c_begin + C : N;
  int k = 0;
  while (k < nt && tcum[k + 1] <= c_begin) ++k;
  for (int64_t cpos = c_begin; cpos < c_end; ++k) {
    const int ut = tcum[k + 1] - tcum[k];
    if (ut == 0) continue;
    const int t0 = (int)(cpos - tcum[k]);
    const int t1 = (int64_t)ut < t0 + (c_end - cpos) ? ut : (int)(t0 + (c_end - cpos));
    run(plan.global_unit(plan.dp_units + k), t0, t1, ut, cpos == c_begin);
    cpos += t1 - t0;
  }
}

// Merge of the split leftover units: workgroup (xcd, k) of a grid of
// 8 x kMaxTailUnits combines the pieces of leftover unit k of XCD xcd with
// the log-sum-exp merge, in key order.  The piece of chunk w sits in slot 2 w'
// of the main kernel's workgroup w' = xcd + 8 w, or in slot 2 w' + 1 when it
// is not the first segment of that chunk.  Thread (g, rb, lane) owns values
// 16 g .. 16 g + 15 of the slot rows of row block rb and lane, so each load
// instruction reads 256 contiguous bytes; piece loads go out 4 at a time.
template <int D>
__global__ __launch_bounds__(256 * (D / 32)) void prefill_merge_kernel(PrefillParams p, int main_grid) {
  constexpr int PB = 4;   // pieces per batch of loads
  __shared__ int32_t tcum[kMaxTailUnits + 1];
  const int xcd = blockIdx.x & 7;
  const int k = blockIdx.x >> 3;
  const int Gx = main_grid >> 3;
  const XcdPlan plan = xcd_plan(p, xcd, Gx);
  if (!plan.sk || k >= plan.nt) return;
  tail_prefix(p, plan, tcum);
  const int64_t F = tcum[k], ut = tcum[k + 1] - tcum[k];
  if (ut == 0) return;
  const int64_t C = tail_chunk(tcum[plan.nt], Gx);
  const int64_t w0 = F / C, w1 = (F + ut - 1) / C;
  if (w0 == w1) return;   // one chunk held the whole unit: stored by the main kernel

  const int lane = threadIdx.x & 63, rb = (threadIdx.x >> 6) & 3, g = threadIdx.x >> 8;
  const float* base = p.ws_o + (rb * 65) * 64 + lane;
  auto slot = [&](int64_t w) {
    return base + (2 * (xcd + 8 * w) + ((w == w0 && F != w0 * C) ? 1 : 0)) * (int64_t)kSlotFloats;
  };
  float m_all = kNegInf;
  for (int64_t w = w0; w <= w1; w += PB) {
    float l[PB];
#pragma unroll
    for (int j = 0; j < PB; ++j) l[j] = w + j <= w1 ? slot(w + j)[64 * 64] : kNegInf;
#pragma unroll
    for (int j = 0; j < PB; ++j) m_all = fmaxf(m_all, l[j]);
  }
  float acc[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) acc[i] = 0.f;
  float wsum = 0.f;
  if (m_all != kNegInf) {
    for (int64_t w = w0; w <= w1; w += PB) {
      float f[PB], v[PB][16];
#pragma unroll
      for (int j = 0; j < PB; ++j) {
        const bool ok = w + j <= w1;
        const float* pw = slot(ok ? w + j : w1);
        f[j] = ok ? pw[64 * 64] : kNegInf;
#pragma unroll
        for (int i = 0; i < 16; ++i) v[j][i] = pw[(16 * g + i) * 64];
      }
#pragma unroll
      for (int j = 0; j < PB; ++j) {
        // a piece with lse -inf has no keys (its values are zero): weight 0
        const float e = f[j] == kNegInf ? 0.f : fast_exp2((f[j] - m_all) * kLog2e);
        wsum += e;
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[i] += e * v[j][i];
      }
    }
    const float inv = 1.0f / wsum;
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[i] *= inv;
  }
  // lanes of one row block: row ln = lane % 32, values 16 g + i are dims
  // 32 g + 8 (i / 4) + 4 hf + (i % 4) (the MFMA accumulator layout)
  const Unit x = unit_of(p, plan.global_unit(plan.dp_units + k));
  const int row = x.row0 + 32 * rb + (lane & 31), hf = lane >> 5;
  if (row >= p.s_q) return;
  const int64_t orow = ((int64_t)x.b * p.s_q + row) * p.num_q_heads + x.h;
  if (p.out_bf16) {
    uint16_t* op = reinterpret_cast<uint16_t*>(p.out) + orow * D + 32 * g + 4 * hf;
#pragma unroll
    for (int a = 0; a < 4; ++a)
      *reinterpret_cast<u32x2*>(op + 8 * a) =
          u32x2{pack_bf16x2(acc[4 * a], acc[4 * a + 1]), pack_bf16x2(acc[4 * a + 2], acc[4 * a + 3])};
  } else {
    float* op = reinterpret_cast<float*>(p.out) + orow * D + 32 * g + 4 * hf;
#pragma unroll
    for (int a = 0; a < 4; ++a)
      *reinterpret_cast<f32x4*>(op + 8 * a) = f32x4{acc[4 * a], acc[4 * a + 1], acc[4 * a + 2], acc[4 * a + 3]};
  }
  if (p.out_lse && hf == 0 && g == 0)
    p.out_lse[orow] = m_all == kNegInf ? kNegInf : m_all + fast_log2(wsum) * kLn2;
}

hipError_t launch_prefill_mfma(const PrefillParams& p0, int head_dim, int sm_count, hipStream_t stream) {
  PrefillParams p = p0;
  p.q_tiles = (p.s_q + kQT - 1) / kQT;
  // persistent grid: one workgroup per CU (8 waves, 2 per SIMD), a multiple of 8 (one share per XCD)
  int g = sm_count > 0 ? sm_count : 8;
  if (g > kMaxPrefillWorkgroups) g = kMaxPrefillWorkgroups;
  g = g < 8 ? 8 : (g / 8) * 8;
  if (head_dim == 128)
    hipLaunchKernelGGL(prefill_kernel<128>, dim3((unsigned)g), dim3(kThreads), 0, stream, p);
  else
    hipLaunchKernelGGL(prefill_kernel<64>, dim3((unsigned)g), dim3(kThreads), 0, stream, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.ws_o == nullptr) return e;
  // merge only when some XCD splits its leftover units (the same test as the kernels')
  const int64_t kv_units = (int64_t)p.batch * p.num_kv_heads;
  const int64_t per_kv = (int64_t)p.group * p.q_tiles;
  const int gx = g / 8;
  bool any = false;
  for (int xcd = 0; xcd < 8; ++xcd) {
    const int64_t nkv = kv_units > xcd ? (kv_units - xcd + 7) / 8 : 0;
    const int64_t r = (nkv * per_kv) % gx;
    any = any || (r != 0 && r <= kMaxTailUnits);
  }
  if (!any) return e;
  if (head_dim == 128)
    hipLaunchKernelGGL(prefill_merge_kernel<128>, dim3(8 * kMaxTailUnits), dim3(1024), 0, stream, p, g);
  else
    hipLaunchKernelGGL(prefill_merge_kernel<64>, dim3(8 * kMaxTailUnits), dim3(512), 0, stream, p, g);
  return hipGetLastError();
}

int64_t prefill_units(int32_t batch, int32_t s_q, int32_t num_q_heads) {
  return (int64_t)batch * num_q_heads * ((s_q + kQT - 1) / kQT);
}

size_t prefill_slot_bytes() { return (size_t)kSlotFloats * sizeof(float); }

}  // namespace pkv
