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
// Workgroup: 4 waves x 32 query rows (a 128-row q-tile) of one query head.
// Keys are walked in tiles of 64 staged through double-buffered LDS:
//   * S^T[key][q] = K Q^T on v_mfma_f32_32x32x16_bf16 (A = K rows from LDS,
//     B = Q held in registers), so each lane owns one query row and 32 keys
//     of the tile: the row max needs one cross-half exchange.
//   * O^T[d][q] += V^T P^T on the same MFMA: P^T is the score registers in
//     bf16 (no shuffle), V^T comes from an LDS image of the tile transposed
//     in registers while staging.  The image stores keys in the order the
//     score registers hold them (bits 2 and 3 of the key index swapped), so
//     one 16-byte LDS read gives a lane its 8 keys of one dim.  The output
//     row of a lane is its softmax row, so rescaling needs no shuffle.
//   * Page ids of the walked range are cached in LDS once; keys at or past
//     the workgroup's last visible key are never fetched (zeros are staged),
//     so dead slots and table entries past the last page are never read.
//   * Workgroups are ordered so that all q-tiles (and all query heads of a
//     GQA group) reading one kv head land on the same XCD and share its L2.
#include "pkv_device.hpp"
#include "pkv_internal.hpp"

namespace pkv {

namespace {

constexpr int kKT = 64;          // keys per tile
constexpr int kQT = 128;         // query rows per workgroup
constexpr int kTableCache = 1024;

template <int D>
struct PrefillSmem {
  static constexpr int KROW = D * 2 + 16;       // padded K row (bytes)
  static constexpr int VROW = kKT * 2 + 16;     // padded V^T row (bytes)
  static constexpr int KBYTES = kKT * KROW;
  static constexpr int VBYTES = D * VROW;
  static constexpr int STAGE = KBYTES + VBYTES;
};

// Slot of key k (0..63) inside the V^T image: swap bits 2 and 3.
__device__ __forceinline__ int vt_slot(int k) { return (k & ~0xC) | ((k & 4) << 1) | ((k & 8) >> 1); }

__device__ __forceinline__ int visible_keys(int i, int n_ctx, int seq, int cbs) {
  if (i >= seq) return 0;
  const int e = (i / cbs + 1) * cbs;
  return n_ctx + (e < seq ? e : seq);
}

}  // namespace

template <int D>
__global__ __launch_bounds__(256, 2) void prefill_kernel(PrefillParams p) {
  using S = PrefillSmem<D>;
  constexpr int KSTEPS = D / 16;   // k-steps of the QK product
  constexpr int DB = D / 32;       // 32-dim blocks of the output
  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * S::STAGE];
  __shared__ int32_t pages[kTableCache];

  // ---- XCD-aware work mapping: kv unit (b, g) -> one XCD; its q heads x q-tiles follow
  const int L = blockIdx.x;
  const int xcd = L & 7;
  const int r = L >> 3;
  const int per_kv = p.group * p.q_tiles;
  const int kv_local = r / per_kv;
  const int rem = r - kv_local * per_kv;
  const int hh = rem / p.q_tiles;
  const int qt = rem - hh * p.q_tiles;
  const int kvu = kv_local * 8 + xcd;
  if (kvu >= p.batch * p.num_kv_heads) return;
  const int b = kvu / p.num_kv_heads;
  const int g = kvu - b * p.num_kv_heads;
  const int h = g * p.group + hh;

  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int ln = lane & 31, hf = lane >> 5;
  const int n_ctx = p.n_ctx[b];
  const int seq = p.seq_len[b];
  const int cbs = p.causal_block_size > 0 ? p.causal_block_size : (seq > 0 ? seq : 1);
  const int row0 = qt * kQT;
  const int last_real = (row0 + kQT - 1 < seq - 1) ? row0 + kQT - 1 : seq - 1;
  const int kmax = row0 < seq ? visible_keys(last_real, n_ctx, seq, cbs) : 0;
  const int n_tiles = (kmax + kKT - 1) / kKT;

  // this lane's query row and its key limit; the wave's smallest limit
  const int my_row = row0 + wave * 32 + ln;
  const int my_lim = visible_keys(my_row, n_ctx, seq, cbs);
  const int wrow0 = row0 + wave * 32;
  const int wmin = (wrow0 + 31 < seq) ? visible_keys(wrow0, n_ctx, seq, cbs) : 0;
  const bool wave_live = wrow0 < seq;

  // ---- Q operand (B of S^T = K Q^T): row ln, dims 16 s + 8 hf .. +8
  u32x4 q[KSTEPS];
  {
    const bool ok = my_row < seq;
    const uint16_t* qp = p.q + ((int64_t)b * p.s_q + (ok ? my_row : 0)) * p.q_tok_stride + (int64_t)h * p.q_head_stride;
#pragma unroll
    for (int s = 0; s < KSTEPS; ++s) q[s] = ok ? ld16(qp + 16 * s + 8 * hf) : u32x4{0u, 0u, 0u, 0u};
  }

  // ---- staging roles: threads 0..D-1 stage V^T blocks (8 keys x 8 dims each),
  // threads 128..255 stage K row halves
  constexpr int DB8 = D / 8;
  const int tid = threadIdx.x;
  const int shift = p.page_shift;
  const int pmask = (1 << shift) - 1;
  const int64_t row_elems = (int64_t)p.num_kv_heads * D;
  const uint16_t* kpool = reinterpret_cast<const uint16_t*>(p.k_pool);
  const uint16_t* vpool = reinterpret_cast<const uint16_t*>(p.v_pool);
  const int32_t* trow = p.table + (int64_t)b * p.table_stride;
  int page_base = 0;   // first logical page held in `pages`
  auto cache_pages = [&](int first_page) {
    const int n_pages = ((kmax + pmask) >> shift) - first_page;
    for (int i = tid; i < kTableCache && i < n_pages; i += 256) pages[i] = trow[first_page + i];
    page_base = first_page;
  };
  // registers of the tile in flight: V block (8 keys x 8 dims) or K row half (64 dims)
  u32x4 stage[8];
  auto fetch = [&](int kt) {
    const int key0 = kt * kKT;
    if (tid < 8 * DB8) {
      const int d8 = tid % DB8, grp = tid / DB8;   // grp bits: h(0) mu(1) beta(2)
      const int kb = 32 * (grp >> 2) + 16 * ((grp >> 1) & 1) + 4 * (grp & 1);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int key = key0 + kb + 8 * (e >> 2) + (e & 3);
        if (key < kmax) {
          const int pg = pages[(key >> shift) - page_base];
          stage[e] = ld16(vpool + (int64_t)pg * p.page_stride + (int64_t)(key & pmask) * row_elems +
                          (int64_t)g * D + 8 * d8);
        } else {
          stage[e] = u32x4{0u, 0u, 0u, 0u};
        }
      }
    } else if (tid >= 128) {
      const int t2 = tid - 128;
      const int key = key0 + (t2 >> 1);
      const int half = t2 & 1;
      if (key < kmax) {
        const int pg = pages[(key >> shift) - page_base];
        const uint16_t* src = kpool + (int64_t)pg * p.page_stride + (int64_t)(key & pmask) * row_elems +
                              (int64_t)g * D + (D / 2) * half;
#pragma unroll
        for (int e = 0; e < D / 16; ++e) stage[e] = ld16(src + 8 * e);
      } else {
#pragma unroll
        for (int e = 0; e < D / 16; ++e) stage[e] = u32x4{0u, 0u, 0u, 0u};
      }
    }
  };
  auto commit = [&](int buf) {
    uint8_t* base = smem + buf * S::STAGE;
    if (tid < 8 * DB8) {
      const int d8 = tid % DB8, grp = tid / DB8;
      const int slot0 = 32 * (grp >> 2) + 16 * ((grp >> 1) & 1) + 8 * (grp & 1);
      uint8_t* vt = base + S::KBYTES;
      // stage[e] = 8 dims of key e; write dim rows (8 keys each, in slot order)
#pragma unroll
      for (int dd = 0; dd < 8; ++dd) {
        const int w = dd >> 1;
        u32x4 o;
#pragma unroll
        for (int q2 = 0; q2 < 4; ++q2)
          o[q2] = (dd & 1) ? pack_hi16(stage[2 * q2][w], stage[2 * q2 + 1][w])
                           : pack_lo16(stage[2 * q2][w], stage[2 * q2 + 1][w]);
        *reinterpret_cast<u32x4*>(vt + (8 * d8 + dd) * S::VROW + slot0 * 2) = o;
      }
    } else if (tid >= 128) {
      const int t2 = tid - 128;
      uint8_t* krow = base + (t2 >> 1) * S::KROW + (t2 & 1) * D;
#pragma unroll
      for (int e = 0; e < D / 16; ++e) *reinterpret_cast<u32x4*>(krow + 16 * e) = stage[e];
    }
  };

  // ---- running state: O^T blocks, row max (raw score units) and sum
  f32x16 o[DB];
#pragma unroll
  for (int d = 0; d < DB; ++d) o[d] = f32x16{};
  float m = kNegInf, l = 0.f;
  const float c = p.scale_log2;

  if (n_tiles > 0) {
    cache_pages(0);
    __syncthreads();
    fetch(0);
    commit(0);
    __syncthreads();
  }
  for (int kt = 0; kt < n_tiles; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < n_tiles) {
      const int next_page = ((kt + 1) * kKT) >> shift;
      if (next_page + ((kKT - 1) >> shift) + 1 - page_base > kTableCache) {
        // page window exhausted: everyone is between tiles here, refresh it
        __syncthreads();
        cache_pages(next_page);
        __syncthreads();
      }
      fetch(kt + 1);
    }
    if (wave_live) {
      const uint8_t* base = smem + buf * S::STAGE;
      const int key0 = kt * kKT;
      // ---- S^T for the two 32-key blocks
      f32x16 sb[2];
#pragma unroll
      for (int blk = 0; blk < 2; ++blk) {
        f32x16 acc = f32x16{};
        const uint8_t* krow = base + (32 * blk + ln) * S::KROW + 16 * hf;
#pragma unroll
        for (int s = 0; s < KSTEPS; ++s) {
          const u32x4 a = *reinterpret_cast<const u32x4*>(krow + 32 * s);
          acc = mfma32x32x16_bf16(a, q[s], acc);
        }
        sb[blk] = acc;
      }
      // ---- mask keys past this row's limit (only where some row of the wave needs it)
      if (key0 + kKT > wmin) {
#pragma unroll
        for (int blk = 0; blk < 2; ++blk)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int key = key0 + 32 * blk + 8 * (i >> 2) + 4 * hf + (i & 3);
            if (key >= my_lim) sb[blk][i] = kNegInf;
          }
      }
      // ---- online softmax (row = lane & 31; the other half of the row is lane ^ 32)
      float mt = kNegInf;
#pragma unroll
      for (int blk = 0; blk < 2; ++blk)
#pragma unroll
        for (int i = 0; i < 16; ++i) mt = fmaxf(mt, sb[blk][i]);
      mt = fmaxf(mt, __shfl_xor(mt, 32, 64));
      const float m_new = fmaxf(m, mt);
      const float mc = (m_new == kNegInf) ? 0.f : m_new * c;
      const float alpha = (m == kNegInf) ? 0.f : fast_exp2(m * c - mc);
      m = m_new;
      float psum = 0.f;
      u32x4 pb[2][2];   // [blk][mu]: 8 bf16 probabilities, keys in score-register order
#pragma unroll
      for (int blk = 0; blk < 2; ++blk)
#pragma unroll
        for (int mu = 0; mu < 2; ++mu)
#pragma unroll
          for (int q2 = 0; q2 < 4; ++q2) {
            const float e0 = fast_exp2(fmaf(sb[blk][8 * mu + 2 * q2], c, -mc));
            const float e1 = fast_exp2(fmaf(sb[blk][8 * mu + 2 * q2 + 1], c, -mc));
            psum += e0 + e1;
            pb[blk][mu][q2] = pack_bf16x2(e0, e1);
          }
      l = l * alpha + psum;
#pragma unroll
      for (int d = 0; d < DB; ++d) o[d] *= alpha;
      // ---- O^T += V^T P^T
      const uint8_t* vt = base + S::KBYTES;
#pragma unroll
      for (int d = 0; d < DB; ++d) {
        const uint8_t* vrow = vt + (32 * d + ln) * S::VROW + 16 * hf;
#pragma unroll
        for (int blk = 0; blk < 2; ++blk)
#pragma unroll
          for (int mu = 0; mu < 2; ++mu) {
            const u32x4 a = *reinterpret_cast<const u32x4*>(vrow + (32 * blk + 16 * mu) * 2);
            o[d] = mfma32x32x16_bf16(a, pb[blk][mu], o[d]);
          }
      }
    }
    if (kt + 1 < n_tiles) commit(buf ^ 1);
    __syncthreads();
  }

  // ---- finish: full row sum, normalise, store (rows < s_q)
  l += __shfl_xor(l, 32, 64);
  if (my_row >= p.s_q) return;
  const bool empty = l == 0.f;
  const float inv = empty ? 0.f : 1.0f / l;
  const int64_t orow = ((int64_t)b * p.s_q + my_row) * p.num_q_heads + h;
  // lane holds dims 32 d + 8 (i / 4) + 4 hf + (i % 4) of its row
  if (p.out_bf16) {
    uint16_t* op = reinterpret_cast<uint16_t*>(p.out) + orow * D;
#pragma unroll
    for (int d = 0; d < DB; ++d)
#pragma unroll
      for (int a = 0; a < 4; ++a)
        *reinterpret_cast<u32x2*>(op + 32 * d + 8 * a + 4 * hf) =
            u32x2{pack_bf16x2(o[d][4 * a] * inv, o[d][4 * a + 1] * inv),
                  pack_bf16x2(o[d][4 * a + 2] * inv, o[d][4 * a + 3] * inv)};
  } else {
    float* op = reinterpret_cast<float*>(p.out) + orow * D;
#pragma unroll
    for (int d = 0; d < DB; ++d)
#pragma unroll
      for (int a = 0; a < 4; ++a)
        *reinterpret_cast<f32x4*>(op + 32 * d + 8 * a + 4 * hf) =
            f32x4{o[d][4 * a] * inv, o[d][4 * a + 1] * inv, o[d][4 * a + 2] * inv, o[d][4 * a + 3] * inv};
  }
  if (p.out_lse && hf == 0) p.out_lse[orow] = empty ? kNegInf : (m * c + fast_log2(l)) * kLn2;
}

hipError_t launch_prefill_mfma(const PrefillParams& p0, int head_dim, hipStream_t stream) {
  PrefillParams p = p0;
  p.q_tiles = (p.s_q + kQT - 1) / kQT;
  const int kv_units = p.batch * p.num_kv_heads;
  const int per_xcd = (kv_units + 7) / 8;
  const dim3 grid((unsigned)(8 * per_xcd * p.group * p.q_tiles)), block(256);
  if (head_dim == 128)
    hipLaunchKernelGGL(prefill_kernel<128>, grid, block, 0, stream, p);
  else
    hipLaunchKernelGGL(prefill_kernel<64>, grid, block, 0, stream, p);
  return hipGetLastError();
}

}  // namespace pkv
