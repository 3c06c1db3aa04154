#pragma once
// Block-causal paged prefill on bf16 MFMA: the kernel template, shared by the
// translation units that instantiate it (prefill.hip: bf16 K/V, the merge of
// leftover units and the launchers; prefill_fp8.hip: fp8 K/V, built with its
// own scheduler options).
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
// in tiles of 64.  A workgroup has 8 waves (two per SIMD): 4 row blocks of 32
// query rows x 2 key halves (keys 0-31 / 32-63 of every tile).  Both waves of
// a row block keep their own softmax state; they are joined at the end of a
// segment with the log-sum-exp merge.
//
//   * S^T[key][q] = K Q^T on v_mfma_f32_32x32x16_bf16 (A = K rows from LDS,
//     B = Q held in registers): each lane owns one query row and 16 keys.
//   * O^T[d][q] += V^T P^T on the same MFMA: P^T is the score registers in
//     bf16 (no shuffle); V^T operands come straight from the row-major V tile
//     through ds_read_b64_tr_b16 (each 16-lane group reads a 4-key x 16-dim
//     block and gets it transposed), so staging never transposes.
//   * K/V tiles go from HBM to LDS by LDS-DMA (buffer loads that write LDS
//     directly, no staging registers), four stages each, two tiles ahead
//     (a power of two, so a tile's stage is a mask rather than a modulo).
//     Rows are XOR-swizzled in 16-byte chunks instead of padded (the DMA
//     writes 1 KiB runs), keeping both operand read patterns conflict-free.
//   * Software pipeline of a wave, per tile t: exp of S(t) -> P(t); QK^T of
//     tile t+1; PV of tile t-1.  The two MFMA chains do not depend on the
//     vector work, so matrix cores and vector ALUs overlap within a wave as
//     well as across the two waves of a SIMD.  The lazy rescale (offset moves
//     only when a row max grows by 2^8) also rescales the pending P(t-1).
//     The loop is unrolled by two so score and P registers trade roles
//     instead of being copied; MFMAs are built in their VGPR form so the
//     scores feed the vector ALUs without accumulator-register moves.
//   * fp8 e4m3fn pools: the LDS-DMA copies raw codes (half the bytes).  QK^T
//     runs on 32x32x64 fp8 MFMAs straight from the raw K tile, with Q held
//     as two e4m3 code sets per row (hi, and 16x the residual through the
//     MFMA's 2^-4 block scale), so scores carry about 2^-8 relative error;
//     the page's K scale and Q's row scale multiply the scores.  PV stays on
//     bf16 MFMAs: each operand is read from the raw V tile with one 8-bit
//     transposed LDS read (8 codes of one dim per lane) and widened exactly
//     in registers, so V costs half the LDS operand reads of a bf16 tile.
//     P carries the page's V scale in its exponent.
//   * Loads never branch: rows of keys at or past the unit's last visible key
//     fall outside the LDS-DMA buffer's range and load zeros (finite; the
//     score is masked, P is exactly 0), so dead page slots and table entries
//     past the last page never reach a product.
//   * Schedule: a persistent grid, one 8-wave workgroup per CU.  The
//     dispatcher deals workgroups to the 8 XCDs round robin (from an XCD that
//     depends on earlier launches), so the workgroups whose ids agree mod 8
//     share one XCD.  Each such group owns whole kv heads; its workgroups
//     first run whole units in rounds, all in lockstep along the keys, so
//     every K/V tile of a head is fetched once into the XCD's L2 and reused by
//     all of its q-tiles.
//     The units left over after the last full round (fewer than the XCD's
//     workgroups) are split evenly along the keys over all of them (stream-K,
//     with a workspace): a unit cut into pieces leaves normalised partial
//     states, which a second, small kernel merges.  (Merging inside the main
//     kernel would need agent-scope fences; on this chip those write back and
//     invalidate the XCD's whole L2, evicting the K/V tiles every other
//     workgroup there is streaming.)  Without a workspace the leftover units
//     simply run whole.
#include <type_traits>

#include "pkv_device.hpp"
#include "pkv_internal.hpp"

namespace pkv {

namespace {

constexpr int kKT = 64;            // keys per tile
constexpr int kQT = 128;           // query rows per unit
constexpr int kThreads = 512;      // 8 waves, two per SIMD
constexpr int kTableCache = 1024;  // page ids cached in LDS
constexpr int kSlotFloats = 4 * 65 * 64;   // partial state: [row block][64 outputs + lse][lane]

// LDS of one workgroup: NST stages each of K and V, as the LDS-DMA writes
// them (bf16 rows, or raw fp8 rows that the MFMA operand reads take as they
// are).
template <int D, bool kFp8>
struct PSmem {
  static constexpr int ROWB = D * 2;              // bytes of one bf16 key row in LDS (no padding: XOR swizzle)
  static constexpr int TB = kKT * ROWB;           // bytes of one bf16 K or V tile
  static constexpr int DROWB = kFp8 ? D : 2 * D;  // bytes of one key row as the LDS-DMA writes it
  static constexpr int CH = DROWB / 16;           // 16-byte chunks per DMA row
  static constexpr int DTB = kKT * DROWB;         // bytes of one DMA tile
  static constexpr int NST = 4;                   // DMA pipeline stages of each of K and V
  static constexpr int STAGES = 2 * NST * DTB;   // K stages, V stages
  static constexpr int RPI = 1024 / DROWB;        // rows written by one LDS-DMA instruction (64 lanes x 16 B)
  static constexpr int IPW = kKT / RPI / 8;       // DMA instructions per wave per tile, for each of K and V
  static_assert(RPI * IPW == 8, "a wave writes 8 rows of each tile");
  static constexpr int COMBINE = 4 * 66 * 64 * 4;   // key-half join: [row block][64 + 2 values][lane] floats
  static constexpr int BYTES = STAGES > COMBINE ? STAGES : COMBINE;
};

// Chunk positions in LDS: chunk c of tile row r lives at position c ^ swz(r).
// K: the 16 rows of one 16-lane group of a 32x32x16 operand read land on 16
// distinct 16-byte bank slots.  V: the 4 rows x 32 bytes of one 16-lane group
// of a transposed read (and the two dim halves of a wave) land on distinct
// bank groups.
template <int D>
__device__ __forceinline__ int swz_k(int r) { return D == 128 ? (r & 15) : ((r >> 1) & 7); }
template <int D>
__device__ __forceinline__ int swz_v(int r) { return D == 128 ? 4 * (r & 3) : 2 * ((r >> 1) & 1); }
// Raw fp8 K rows (128 bytes, two to a 256-byte bank line): the 16 rows of a
// 16-lane operand read land on 16 distinct 16-byte bank slots.
__device__ __forceinline__ int swz_k8(int r) { return (r >> 1) & 7; }

typedef int i32x4_t __attribute__((ext_vector_type(4)));
typedef int i32x8_t __attribute__((ext_vector_type(8)));

// One LDS-DMA instruction (buffer_load_dwordx4 ... lds): every lane copies 16
// bytes at byte offset voff of the buffer [base, base + nbytes) to LDS byte
// address lds_dst + 16 * lane (base, nbytes and lds_dst uniform; lds_dst an
// offset from the workgroup's LDS base, so no generic-to-LDS pointer
// conversion and its null check per instruction); lanes outside the range
// write zeros.  Issued from asm so that the compiler's own wait counting does not
// see it: it would otherwise wait for every pending LDS-DMA before each LDS
// read it cannot prove disjoint (all of them here, the stages being a ring).
// Completion is waited for explicitly with wait_dma_and_barrier; extra
// operations in flight can only make the compiler's own vmcnt waits longer.
// No other code of this kernel uses M0.
__device__ __forceinline__ void dma16(const uint8_t* base, int nbytes, uint32_t lds_dst, int voff) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  i32x4_t d;
  d[0] = __builtin_amdgcn_readfirstlane((int)(uint32_t)a);
  d[1] = __builtin_amdgcn_readfirstlane((int)((uint32_t)(a >> 32) & 0xffffu));
  d[2] = __builtin_amdgcn_readfirstlane(nbytes);
  d[3] = 0x00020000;
  const int m0v = __builtin_amdgcn_readfirstlane((int)lds_dst);
  asm volatile("s_mov_b32 m0, %1\n\tbuffer_load_dwordx4 %0, %2, 0 offen lds" ::"v"(voff), "s"(m0v), "s"(d)
               : "memory");
}

// Wait until at most N of this wave's vector memory operations (here: LDS-DMA
// loads) are outstanding, then join the workgroup.  Written as one asm block
// with a memory clobber so that no LDS access moves across it.
template <int N>
__device__ __forceinline__ void wait_dma_and_barrier() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)\n\ts_waitcnt lgkmcnt(0)\n\ts_barrier" ::"n"(N) : "memory");
}

// Rows of batch entry b in q / out / lse: padded (b * s_q, s_q rows) or
// ragged (q_offsets[b], q_offsets[b + 1] - q_offsets[b] rows).  Rows at or
// past an entry's row count are neither read nor written.
__device__ __forceinline__ int64_t entry_row0(const PrefillParams& p, int b) {
  return p.q_offsets ? (int64_t)p.q_offsets[b] : (int64_t)b * p.s_q;
}
__device__ __forceinline__ int entry_rows(const PrefillParams& p, int b) {
  return p.q_offsets ? p.q_offsets[b + 1] - p.q_offsets[b] : p.s_q;
}

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

typedef int v2i32 __attribute__((ext_vector_type(2)));
// Transposed 8-byte LDS read of bytes (ds_read_b64_tr_b8): within each
// 16-lane group, lane o receives byte (o % 8) of the 8-byte rows addressed by
// lanes o / 8 + 2 i, i = 0..7, as its byte i.  (The fp8 prefill's PV rests on
// this layout; its parity tests against the oracle cover every operand.)
__device__ __forceinline__ u32x2 lds_read_tr8(const uint8_t* ptr) {
  const v2i32 r = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
      (__attribute__((address_space(3))) v2i32*)((__attribute__((address_space(3))) uint8_t*)(ptr)));
  return __builtin_bit_cast(u32x2, r);
}

// A unit: (batch, kv head, query head of the group, q-tile).
struct Unit {
  int b, g, h, row0, n_ctx, seq, cbs, kmax, tiles, rows;
  int64_t qrow0;   // the entry's first row in q / out
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
  x.rows = entry_rows(p, x.b);
  x.qrow0 = entry_row0(p, x.b);
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
__device__ __forceinline__ void store_rows(const PrefillParams& p, const Unit& x, int row, int hf,
                                           const f32x16 (&v)[D / 32], float lse) {
  if (row >= x.rows) return;
  const int h = x.h;
  const int64_t orow = (x.qrow0 + row) * p.num_q_heads + h;
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

// Scales of the cached pages of an fp8 pool (the scale of a (page, kv head)
// multiplies every code of its rows): the score multiplier c * k_scale, and
// log2 / reciprocal of v_scale, which is folded into the exponent of P and
// taken back out of the row sum.  Scales below 2^-100 (zero included) count
// as 2^-100: their rows then contribute nothing measurable instead of 0 * inf.
struct ScaleCache {
  float a, vlog, vinv;
};

template <int D, bool kFp8>
__global__ __launch_bounds__(kThreads, 1) void prefill_kernel(PrefillParams p) {
  using S = PSmem<D, kFp8>;
  constexpr int KSTEPS = D / 16;   // k-steps of QK^T
  constexpr int DB = D / 32;       // 32-dim output blocks
  __shared__ __attribute__((aligned(16))) uint8_t smem[S::BYTES];
  // LDS byte address of smem (the LDS-DMA destinations are offsets from it)
  const uint32_t smem_lds = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint8_t*)smem;
  __shared__ int32_t pages[kTableCache];
  __shared__ ScaleCache scales[kFp8 ? kTableCache : 1];
  __shared__ int32_t tcum[kMaxTailUnits + 1];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int ln = lane & 31, hf = lane >> 5;
  const int rb = wave & 3, kh = wave >> 2;   // row block, key half
  const float c = p.scale_log2;

  // ---- schedule: XCD xcd owns kv units xcd, xcd + 8, ...; its Gx workgroups
  // run whole units in lockstep rounds, then split the leftover ones
  const int wi = blockIdx.x >> 3;
  const int Gx = gridDim.x >> 3;
  const XcdPlan plan = xcd_plan(p, blockIdx.x & 7, Gx);

  const int shift = p.page_shift;
  const int pmask = (1 << shift) - 1;
  constexpr int esz = kFp8 ? 1 : 2;                    // bytes of a pool element
  const int row_b = p.num_kv_heads * D * esz;          // bytes between key rows of a page
  const int64_t page_stride_b = p.page_stride * esz;
  const uint8_t* kpool_b = reinterpret_cast<const uint8_t*>(p.k_pool);
  const uint8_t* vpool_b = reinterpret_cast<const uint8_t*>(p.v_pool);
  // A wave's LDS-DMA writes rows 8 wave .. 8 wave + 7 of each tile, 8
  // consecutive keys of one page (page_size >= 16).  Lane part of the byte
  // offset of DMA instruction j: its row i of the 8 times the row pitch plus
  // its 16-byte chunk, placed by the row's LDS swizzle.
  int koffs[S::IPW], voffs[S::IPW];
#pragma unroll
  for (int j = 0; j < S::IPW; ++j) {
    const int r = S::RPI * (wave * S::IPW + j) + lane / S::CH;   // row of the tile
    const int ck = kFp8 ? (lane % S::CH) ^ swz_k8(r) : (lane % S::CH) ^ swz_k<D>(r);
    const int cv = kFp8 ? (lane % S::CH) ^ swz_k8(r) : (lane % S::CH) ^ swz_v<D>(r);
    koffs[j] = (r - 8 * wave) * row_b + ck * 16;
    voffs[j] = (r - 8 * wave) * row_b + cv * 16;
  }

  // one segment: tiles [t0, t1) of unit u (ut tiles in all); first_seg tells
  // which of the workgroup's two slots a partial state goes to.
  auto run = [&](int u, int t0, int t1, int ut, bool first_seg) {
    const Unit x = unit_of(p, u);
    const int32_t* trow = p.table + (int64_t)x.b * p.table_stride;
    const int my_row = x.row0 + 32 * rb + ln;
    const int my_lim = visible_keys(my_row, x.n_ctx, x.seq, x.cbs);
    const int wrow0 = x.row0 + 32 * rb;
    const int wmin = (wrow0 + 31 < x.seq) ? visible_keys(wrow0, x.n_ctx, x.seq, x.cbs) : 0;

    // Q operand of this row block.  bf16 pools: row ln, dims 16 s + 8 hf .. +8
    // (bf16 MFMA).  fp8 pools: row ln, dims 64 j + 32 hf .. +32 (fp8 MFMA;
    // K's operand takes the same dims) as two e4m3 code sets with one scale
    // per row: with v = q / qsc (the row's largest |q| maps to 448),
    // hi = e4m3(v) and lo = e4m3(16 (v - hi)), so v = hi + lo / 16 to about
    // 2^-8 relative, near bf16's own rounding.
    u32x4 q[KSTEPS];
    i32x8_t q8[2], q8l[2];
    float qsc = 1.f;
    {
      const bool ok = my_row < x.seq && my_row < x.rows;
      const uint16_t* qp = p.q + (x.qrow0 + (ok ? my_row : 0)) * p.q_tok_stride + (int64_t)x.h * p.q_head_stride;
      if constexpr (!kFp8) {
#pragma unroll
        for (int s2 = 0; s2 < KSTEPS; ++s2) q[s2] = ok ? ld16(qp + 16 * s2 + 8 * hf) : u32x4{0u, 0u, 0u, 0u};
      } else {
        u32x4 raw[2][4];
        float amax = 0.f;
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
          for (int w = 0; w < 4; ++w) {
            raw[j][w] = ok ? ld16(qp + 64 * j + 32 * hf + 8 * w) : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
            for (int e = 0; e < 4; ++e)
              amax = fmaxf(amax, fmaxf(fabsf(__uint_as_float(raw[j][w][e] << 16)),
                                       fabsf(__uint_as_float(raw[j][w][e] & 0xffff0000u))));
          }
        {
          // lanes l and l ^ 32 hold the two halves of one row
          const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(amax), __float_as_uint(amax), false, false);
          amax = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
        }
        const float inv = amax > 0.f ? 448.0f / amax : 1.0f;
        qsc = amax > 0.f ? amax * (1.0f / 448.0f) : 1.0f;
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
          for (int k = 0; k < 8; ++k) {
            // code word k: dims 64 j + 32 hf + 4 k .. + 3, as bytes 0..3
            const uint32_t w0 = raw[j][k >> 1][2 * (k & 1)], w1 = raw[j][k >> 1][2 * (k & 1) + 1];
            const float v0 = __uint_as_float(w0 << 16) * inv, v1 = __uint_as_float(w0 & 0xffff0000u) * inv;
            const float v2 = __uint_as_float(w1 << 16) * inv, v3 = __uint_as_float(w1 & 0xffff0000u) * inv;
            int wd = __builtin_amdgcn_cvt_pk_fp8_f32(v0, v1, 0, false);
            wd = __builtin_amdgcn_cvt_pk_fp8_f32(v2, v3, wd, true);
            q8[j][k] = wd;
            const f32x2 h01 = __builtin_amdgcn_cvt_pk_f32_fp8(wd, false), h23 = __builtin_amdgcn_cvt_pk_f32_fp8(wd, true);
            int wl = __builtin_amdgcn_cvt_pk_fp8_f32(16.0f * (v0 - h01[0]), 16.0f * (v1 - h01[1]), 0, false);
            wl = __builtin_amdgcn_cvt_pk_fp8_f32(16.0f * (v2 - h23[0]), 16.0f * (v3 - h23[1]), wl, true);
            q8l[j][k] = wl;
          }
      }
    }

    f32x16 o[DB];
#pragma unroll
    for (int d = 0; d < DB; ++d) o[d] = f32x16{};
    float mc = kNegInf, l = 0.f;   // exponent offset (log2 units) and this lane's share of the row sum

    if (t1 > t0) {
      // page ids of the walked keys, refreshed if the segment spans more pages
      int page_base = (t0 * kKT) >> shift;
      const int last_page = (x.kmax - 1) >> shift;
      auto cache_pages = [&](int first) {
        __syncthreads();
        for (int i = tid; i < kTableCache && first + i <= last_page; i += kThreads) {
          const int pg = trow[first + i];
          pages[i] = pg;
          if constexpr (kFp8) {
            const int64_t si = (int64_t)pg * p.num_kv_heads + x.g;
            const float ks = fmaxf(p.k_scale[si], 0x1p-100f), vs = fmaxf(p.v_scale[si], 0x1p-100f);
            scales[i] = ScaleCache{c * ks, fast_log2(vs), 1.0f / vs};
          }
        }
        page_base = first;
        __syncthreads();
      };
      cache_pages(page_base);
      // Page ids of this wave's DMA rows for tiles tw0 .. tw0 + 63, one per
      // lane (read back with readlane: no LDS round trip per DMA).  Reloaded
      // when the DMA lookahead passes the window or the page cache moves;
      // entries past the cached pages are never used before a reload.
      int tw0 = t0, win = 0;
      auto load_window = [&](int tb) {
        const int key = min((tb + lane) * kKT + 8 * wave, x.kmax - 1);
        win = pages[min((key >> shift) - page_base, kTableCache - 1)];
        tw0 = tb;
      };
      load_window(t0);

      // LDS-DMA of tile t of K or V into its stage: this wave writes rows
      // 8 wave .. 8 wave + 7, keys kw .. kw + 7 of one page.  The buffer starts
      // at key kw's row and its range ends after the last key the segment
      // reads, so rows of keys past the unit's last visible key or past the
      // segment load zeros (a zero row is finite: its score is masked and its
      // P is 0), and tiles past the segment write only zeros into a free
      // stage: every iteration has the same loads in flight.
      const int64_t head_off_b = (int64_t)x.g * D * esz;
      const int klim = min(x.kmax, t1 * kKT);   // keys the segment reads: [.., klim)
      // DMA rings
      auto kstage = [&](int t) { return smem + ((t - t0 + S::NST) % S::NST) * S::DTB; };
      auto vstage = [&](int t) { return smem + (S::NST + (t - t0 + S::NST) % S::NST) * S::DTB; };
      // scales of this wave's key half of tile t (fp8; the half is one page).
      // A half wholly past the unit's last key (all its scores masked) takes
      // the last key's page, which is cached: its scale must be finite.
      auto tile_scales = [&](int t) {
        if constexpr (kFp8) return scales[(min(t * kKT + 32 * kh, x.kmax - 1) >> shift) - page_base];
        return ScaleCache{c, 0.f, 1.f};
      };
      auto dma_tile = [&](const uint8_t* pool_b, uint8_t* tile, int t, bool is_k) {
        const int kw = t * kKT + 8 * wave;
        // rows that hold keys the segment reads, clamped to 0..8 on the scalar
        // unit (left to itself the compiler takes a vector med3, a vector
        // multiply and a readfirstlane per tile)
        int rows;
        asm("s_max_i32 %0, %1, 0\n\ts_min_i32 %0, %0, 8" : "=s"(rows) : "s"(klim - kw) : "scc");
        // the window's lane t - tw0 holds kw's page while the tile is live (a
        // tile past the segment takes any cached page: it loads nothing)
        const int pg = __builtin_amdgcn_readlane(win, (t - tw0) & 63);
        // (page ids are never negative: an unsigned product needs no sign extension)
        const uint8_t* base = pool_b + (uint64_t)(uint32_t)pg * (uint64_t)page_stride_b + head_off_b +
                              (uint32_t)((kw & pmask) * row_b);
#pragma unroll
        for (int j = 0; j < S::IPW; ++j)
          dma16(base, rows * row_b, smem_lds + (uint32_t)(tile - smem) + S::RPI * (wave * S::IPW + j) * S::DROWB,
                is_k ? koffs[j] : voffs[j]);
      };
      // S^T of this wave's key half of K tile t: keys 32 kh + 8 (i / 4) + 4 hf + (i % 4)
      auto qk = [&](int t, f32x16& acc) {
        if constexpr (kFp8) {
          // fp8 pools: 32x32x64 fp8 MFMAs straight from the raw K tile, K
          // codes times Q's hi codes, then times its lo codes with the
          // MFMA's block scale 2^-4 on B (the K and Q scales multiply the
          // scores later)
          const int kr = 32 * kh + ln;
          const uint8_t* row = kstage(t) + kr * S::DROWB;
          const int sw = swz_k8(kr);
          acc = f32x16{};
#pragma unroll
          for (int j = 0; j < 2; ++j) {
            const int c0 = 4 * j + 2 * hf;
            const u32x4 lo = *reinterpret_cast<const u32x4*>(row + ((c0 ^ sw) << 4));
            const u32x4 hi = *reinterpret_cast<const u32x4*>(row + (((c0 + 1) ^ sw) << 4));
            const i32x8_t a = i32x8_t{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                                      (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
            acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, q8[j], acc, 0, 0, 0, 127, 0, 127);
            acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, q8l[j], acc, 0, 0, 0, 127, 0, 123);
          }
          return;
        }
        const uint8_t* kt = kstage(t);
        const int kr = 32 * kh + ln;
        u32x4 a[KSTEPS];
#pragma unroll
        for (int s2 = 0; s2 < KSTEPS; ++s2)
          a[s2] = *reinterpret_cast<const u32x4*>(kt + kr * S::ROWB + (((2 * s2 + hf) ^ swz_k<D>(kr)) << 4));
        acc = f32x16{};
#pragma unroll
        for (int s2 = 0; s2 < KSTEPS; ++s2) acc = mfma32x32x16_bf16(a[s2], q[s2], acc);
        // Keep 4 K operand reads in flight ahead of the MFMA chain.  Left to
        // itself the scheduler (at the register limit) issues each read right
        // before its MFMA and waits for it.
        if constexpr (!kFp8) {
          __builtin_amdgcn_sched_group_barrier(0x100, 4, 1);   // 4 LDS reads
#pragma unroll
          for (int i = 0; i < KSTEPS - 4; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 1);   // 1 MFMA
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 1);   // 1 LDS read
          }
          __builtin_amdgcn_sched_group_barrier(0x008, 4, 1);   // the last 4 MFMAs
        }
      };
      // O^T += V^T P^T over this wave's key half of V tile t; pk[mu] is the bf16
      // P of keys 32 kh + 16 mu + 8 (j / 4) + 4 hf + (j % 4), j = 0..7.  Lane
      // group (hf, dh) reads rows 32 kh + 16 mu + 4 hf + 0..3 (and + 8) of dims
      // 32 d + 16 dh .. + 15, transposed.
      auto pv = [&](int t, const u32x4 (&pk)[2]) {
        const uint8_t* vt = vstage(t);
        const int s16 = lane & 15;
        const int dh = (lane >> 4) & 1;
        if constexpr (kFp8) {
          // fp8 pools: one 8-bit transposed read per MFMA from the raw tile
          // (rows of D codes, 16-byte chunks swizzled by swz_k8).  Lane j of
          // 16-lane group g addresses key 32 kh + 16 mu + 8 (j / 8) + 4 (g / 2)
          // + (j / 2) % 4, dims 32 d + 16 (g % 2) + 8 (j % 2) .. + 7, so lane l
          // receives dim 32 d + l % 32 of the 8 keys of pk's order; the codes
          // widen exactly (scale 1) to the bf16 A operand.
          const int g = lane >> 4;
#pragma unroll
          for (int mu = 0; mu < 2; ++mu) {
            const int key = 32 * kh + 16 * mu + 8 * (s16 >> 3) + 4 * (g >> 1) + ((s16 >> 1) & 3);
            const uint8_t* rowp = vt + key * S::DROWB + 8 * (s16 & 1);
            const int sw = swz_k8(key);
            u32x2 raw[DB];
#pragma unroll
            for (int d = 0; d < DB; ++d) raw[d] = lds_read_tr8(rowp + (((2 * d + (g & 1)) ^ sw) << 4));
#pragma unroll
            for (int d = 0; d < DB; ++d) {
              const u32x4 a{
                  __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)raw[d][0], 1.0f, false)),
                  __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)raw[d][0], 1.0f, true)),
                  __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)raw[d][1], 1.0f, false)),
                  __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)raw[d][1], 1.0f, true))};
              o[d] = mfma32x32x16_bf16(a, pk[mu], o[d]);
            }
          }
          return;
        }
        u32x2 lo[2][DB], hi[2][DB];
#pragma unroll
        for (int mu = 0; mu < 2; ++mu) {
          const int r = 32 * kh + 16 * mu + 4 * hf + (s16 >> 2);
          const uint8_t* rowp = vt + r * S::ROWB + 8 * (s16 & 1);
          const int sw = swz_v<D>(r);
#pragma unroll
          for (int d = 0; d < DB; ++d) {
            const uint8_t* a0 = rowp + (((4 * d + 2 * dh + ((s16 & 3) >> 1)) ^ sw) << 4);
            lo[mu][d] = lds_read_tr(a0);
            hi[mu][d] = lds_read_tr(a0 + 8 * S::ROWB);
          }
        }
#pragma unroll
        for (int mu = 0; mu < 2; ++mu)
#pragma unroll
          for (int d = 0; d < DB; ++d)
            o[d] = mfma32x32x16_bf16(u32x4{lo[mu][d][0], lo[mu][d][1], hi[mu][d][0], hi[mu][d][1]}, pk[mu], o[d]);
      };
      // row max of this wave's 32 scores of tile t, masking keys at or past
      // the row's limit when the half reaches past the wave's smallest limit
      auto mask_max = [&](f32x16& sv, int t, auto masked) {
        if constexpr (decltype(masked)::value) {
          const int key0 = t * kKT + 32 * kh;
          if (key0 + 32 > wmin) {
#pragma unroll
            for (int i = 0; i < 16; ++i)
              if (key0 + 8 * (i >> 2) + 4 * hf + (i & 3) >= my_lim) sv[i] = kNegInf;
          }
        }
        float m0 = fmaxf(sv[0], sv[1]), m1 = fmaxf(sv[2], sv[3]);
#pragma unroll
        for (int i = 4; i < 16; i += 2) {
          m0 = fmaxf(m0, sv[i]);
          m1 = fmaxf(m1, sv[i + 1]);
        }
        const float m = fmaxf(m0, m1);
        // lanes l and l ^ 32 hold the same query row
        const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(m), __float_as_uint(m), false, false);
        return fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
      };

      // prologue: zeros into V(t0-1)'s stage (the first PV uses it with P = 0);
      // K(t0), K(t0+1), K(t0+2), V(t0) landed (a pair of steps starts with
      // nothing in flight); S(t0); a barrier (with four stages the first
      // pair's refills go to stages no wave has read or will read before it)
      const bool need_refresh = ((t1 * kKT - 1) >> shift) - page_base >= kTableCache;
      dma_tile(vpool_b, vstage(t0 - 1), t1, false);
      dma_tile(kpool_b, kstage(t0), t0, true);
      dma_tile(kpool_b, kstage(t0 + 1), t0 + 1, true);
      dma_tile(vpool_b, vstage(t0), t0, false);
      dma_tile(kpool_b, kstage(t0 + 2), t0 + 2, true);
      wait_dma_and_barrier<0>();
      f32x16 sA, sB;
      u32x4 pA[2], pB[2] = {u32x4{0u, 0u, 0u, 0u}, u32x4{0u, 0u, 0u, 0u}};
      qk(t0, sA);
      float mt = mask_max(sA, t0, std::true_type{});
      __syncthreads();

      // iteration t: exp of S(t) -> P(t); QK^T of tile t+1 (zeros past the
      // segment); PV of tile t-1 (P = 0 before the first); max of S(t+1).
      // s_cur / p_cur and s_next / p_prev trade roles between iterations.
      // Steps run in pairs (t, t + 1), t - t0 even, with one barrier at the
      // end of the pair.  The pair's first step refills K(t+3), K(t+4),
      // V(t+1), V(t+2) into the stages of K(t-1), K(t), V(t-3), V(t-2), all
      // last read before the previous pair's barrier; the pair reads K(t+1),
      // K(t+2), V(t-1), V(t), which landed before it.
      auto step = [&](int t, f32x16& s_cur, f32x16& s_next, u32x4 (&p_cur)[2], u32x4 (&p_prev)[2], auto masked,
                      auto second) {
        constexpr bool kSecond = decltype(second)::value;
        constexpr int ahead = 4;   // furthest tile the pair's refill loads
        if (!kSecond) {
          if (need_refresh) {
            const int last_t = t + ahead < t1 ? t + ahead : t1 - 1;
            if (((last_t * kKT + kKT - 1) >> shift) - page_base >= kTableCache) {
              cache_pages((t * kKT) >> shift);
              load_window(t);
            }
          }
          if (t + ahead >= tw0 + 64) load_window(t);
          dma_tile(kpool_b, kstage(t + 3), t + 3, true);
          dma_tile(kpool_b, kstage(t + 4), t + 4, true);
          dma_tile(vpool_b, vstage(t + 1), t + 1, false);
          dma_tile(vpool_b, vstage(t + 2), t + 2, false);
        }
        // lazy rescale: the offset of a row moves only when its max grows by
        // more than 8 (log2 units); P(t-1) is not yet in o, so it is rescaled too
        const ScaleCache sct = tile_scales(t);   // tile t's page stays cached across a refresh
        const float sa = sct.a * qsc;   // score multiplier of this tile and row
        const float mtc = mt * sa;
        const bool grow = mtc > mc + 8.0f;
        if (__any(grow)) {
          const float mc_new = grow ? mtc : mc;
          const float alpha = (mc == kNegInf) ? 0.f : fast_exp2(mc - mc_new);
          l *= alpha;
#pragma unroll
          for (int d = 0; d < DB; ++d) o[d] *= alpha;
#pragma unroll
          for (int k = 0; k < 2; ++k)
#pragma unroll
            for (int w = 0; w < 4; ++w) {
              const uint32_t v = p_prev[k][w];
              p_prev[k][w] = pack_bf16x2(__uint_as_float(v << 16) * alpha, __uint_as_float(v & 0xffff0000u) * alpha);
            }
          mc = mc_new;
        }
        // P of an fp8 tile carries the tile's V scale (exponent offset vlog);
        // the row sum takes it back out
        const float mcu = ((mc == kNegInf) ? 0.f : mc) - sct.vlog;
        float psum = 0.f;
#pragma unroll
        for (int mu = 0; mu < 2; ++mu)
#pragma unroll
          for (int q2 = 0; q2 < 4; ++q2) {
            const float e0 = fast_exp2(fmaf(s_cur[8 * mu + 2 * q2], sa, -mcu));
            const float e1 = fast_exp2(fmaf(s_cur[8 * mu + 2 * q2 + 1], sa, -mcu));
            psum += e0 + e1;
            p_cur[mu][q2] = pack_bf16x2(e0, e1);
          }
        if constexpr (kFp8) l = fmaf(psum, sct.vinv, l);
        else l += psum;
        // (No issue priority: with one barrier per pair of steps the two waves
        // of a SIMD drift into complementary phases by themselves; raising the
        // priority of the wave issuing MFMAs, a gain with a barrier per step,
        // measured 3.5 % slower here.)
        qk(t + 1, s_next);
        pv(t - 1, p_prev);
        mt = mask_max(s_next, t + 1, masked);
        // at the end of a pair every load has landed
        if constexpr (kSecond) wait_dma_and_barrier<0>();
      };
      // iteration t masks tile t+1: this wave's keys up to 64 t + 96 + 32 kh - 1.
      // It needs no mask when they lie wholly below every row's key limit.
      // (Waves may switch loops at different t: every pair of steps has the
      // same barriers.)
      const int off = 96 + 32 * kh;
      int t_mask = wmin < off ? t0 : (wmin - off) / kKT + 1;   // first t with 64 t + off > wmin
      t_mask = t_mask < t0 ? t0 : (t_mask > t1 ? t1 : t_mask);
      int t = t0;
      for (; t + 1 < t_mask; t += 2) {
        step(t, sA, sB, pA, pB, std::false_type{}, std::false_type{});
        step(t + 1, sB, sA, pB, pA, std::false_type{}, std::true_type{});
      }
      for (; t + 1 < t1; t += 2) {
        step(t, sA, sB, pA, pB, std::true_type{}, std::false_type{});
        step(t + 1, sB, sA, pB, pA, std::true_type{}, std::true_type{});
      }
      if (t < t1) {
        step(t, sA, sB, pA, pB, std::true_type{}, std::false_type{});
        pB[0] = pA[0];
        pB[1] = pA[1];
      }
      // PV of the last tile (its P is in pB), then drain the trailing
      // zero-range loads before the stages are reused
      pv(t1 - 1, pB);
      wait_dma_and_barrier<0>();
    }

    // ---- join the two key halves of each row block through LDS
    {
      const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(l), __float_as_uint(l), false, false);
      l = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
    }
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
      if (kh == 0) store_rows<D>(p, x, my_row, hf, o, lse);
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

}  // namespace pkv
