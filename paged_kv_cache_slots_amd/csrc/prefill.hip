// Block-causal paged prefill: the bf16 instantiations of prefill_kernel, the
// merge of leftover units split along the keys, and the launchers (the fp8
// K/V kernel is launched through prefill_fp8.hip).
#include "prefill_kernel.hpp"

namespace pkv {

// Merge of the split leftover units: workgroup (rb, k, xcd) of a grid of
// 4 x tail_units x 8 (tail_units: the largest leftover count of any XCD)
// combines, for row block rb, the pieces of leftover unit k of XCD xcd with
// the log-sum-exp merge, in key order.  The piece of
// chunk w sits in slot 2 w' of the main kernel's workgroup w' = xcd + 8 w, or
// in slot 2 w' + 1 when it is not the first segment of that chunk.  Thread
// (g, lane) owns values 16 g .. 16 g + 15 of the slot rows of row block rb
// and lane, so each load instruction reads 256 contiguous bytes; piece loads
// go out 8 at a time.  (One workgroup per row block rather than per unit:
// the merge is bound by load latency, so it wants many small workgroups.)
template <int D>
__global__ __launch_bounds__(64 * (D / 32)) void prefill_merge_kernel(PrefillParams p, int main_grid, int tail_units) {
  constexpr int PB = 8;   // pieces per batch of loads
  __shared__ int32_t tcum[kMaxTailUnits + 1];
  const int xcd = blockIdx.x & 7;
  const int k = (blockIdx.x >> 3) % tail_units;
  const int rb = (blockIdx.x >> 3) / tail_units;
  const int Gx = main_grid >> 3;
  const XcdPlan plan = xcd_plan(p, xcd, Gx);
  if (!plan.sk || k >= plan.nt) return;
  tail_prefix(p, plan, tcum);
  const int64_t F = tcum[k], ut = tcum[k + 1] - tcum[k];
  if (ut == 0) return;
  const int64_t C = tail_chunk(tcum[plan.nt], Gx);
  const int64_t w0 = F / C, w1 = (F + ut - 1) / C;
  if (w0 == w1) return;   // one chunk held the whole unit: stored by the main kernel

  const int lane = threadIdx.x & 63, g = threadIdx.x >> 6;
  const float* base = p.ws_o + (rb * 65) * 64 + lane;
  auto slot = [&](int64_t w) {
    return base + (2 * (xcd + 8 * w) + ((w == w0 && F != w0 * C) ? 1 : 0)) * (int64_t)kSlotFloats;
  };
  // one pass (LSE and values of PB pieces loaded together); the running sums
  // are rescaled when the running max grows
  float acc[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) acc[i] = 0.f;
  float m_all = kNegInf, wsum = 0.f;
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
    float mb = m_all;
#pragma unroll
    for (int j = 0; j < PB; ++j) mb = fmaxf(mb, f[j]);
    if (mb == kNegInf) continue;
    const float sc = m_all == kNegInf ? 0.f : fast_exp2((m_all - mb) * kLog2e);
    wsum *= sc;
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[i] *= sc;
#pragma unroll
    for (int j = 0; j < PB; ++j) {
      // a piece with lse -inf has no keys (its values are zero): weight 0
      const float e = f[j] == kNegInf ? 0.f : fast_exp2((f[j] - mb) * kLog2e);
      wsum += e;
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[i] += e * v[j][i];
    }
    m_all = mb;
  }
  if (m_all != kNegInf) {
    const float inv = 1.0f / wsum;
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[i] *= inv;
  }
  // lanes of one row block: row ln = lane % 32, values 16 g + i are dims
  // 32 g + 8 (i / 4) + 4 hf + (i % 4) (the MFMA accumulator layout)
  const Unit x = unit_of(p, plan.global_unit(plan.dp_units + k));
  const int row = x.row0 + 32 * rb + (lane & 31), hf = lane >> 5;
  if (row >= x.rows) return;
  const int64_t orow = (x.qrow0 + row) * p.num_q_heads + x.h;
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

// Persistent grid of the prefill: one workgroup per CU (8 waves, 2 per SIMD),
// a multiple of 8 (one share per XCD).
int prefill_grid(int sm_count) {
  int g = sm_count > 0 ? sm_count : 8;
  if (g > kMaxPrefillWorkgroups) g = kMaxPrefillWorkgroups;
  return g < 8 ? 8 : (g / 8) * 8;
}

// The largest count of leftover units any XCD splits along the keys (the
// kernels' xcd_plan with a workspace), 0 when every XCD's units divide
// evenly over its workgroups.
int prefill_tail_units(int32_t batch, int32_t s_q, int32_t num_q_heads, int32_t num_kv_heads, int grid) {
  const int64_t kv_units = (int64_t)batch * num_kv_heads;
  const int64_t per_kv = (int64_t)(num_q_heads / num_kv_heads) * ((s_q + kQT - 1) / kQT);
  const int gx = grid / 8;
  int tail_units = 0;
  for (int xcd = 0; xcd < 8; ++xcd) {
    const int64_t nkv = kv_units > xcd ? (kv_units - xcd + 7) / 8 : 0;
    const int64_t r = (nkv * per_kv) % gx;
    if (r != 0 && r <= kMaxTailUnits && r > tail_units) tail_units = (int)r;
  }
  return tail_units;
}

hipError_t launch_prefill_mfma(const PrefillParams& p0, int head_dim, int sm_count, hipStream_t stream) {
  PrefillParams p = p0;
  p.q_tiles = (p.s_q + kQT - 1) / kQT;
  const int g = prefill_grid(sm_count);
  hipError_t e;
  if (p.kv_fp8) {
    e = launch_prefill_kernel_fp8(p, g, stream);
  } else {
    if (head_dim == 128)
      PKV_LAUNCH_MAIN((prefill_kernel<128, false>), dim3((unsigned)g), dim3(kThreads), 0, stream, p);
    else
      PKV_LAUNCH_MAIN((prefill_kernel<64, false>), dim3((unsigned)g), dim3(kThreads), 0, stream, p);
    e = hipGetLastError();
  }
  if (e != hipSuccess) return e;
  if (p.ws_o == nullptr) return e;
  // merge only when some XCD splits its leftover units (the same test as the
  // kernels'); the grid covers the largest leftover count of any XCD
  const int tail_units = prefill_tail_units(p.batch, p.s_q, p.num_q_heads, p.num_kv_heads, g);
  if (tail_units == 0) return e;
  const dim3 mgrid((unsigned)(4 * 8 * tail_units));
  if (head_dim == 128)
    hipLaunchKernelGGL(prefill_merge_kernel<128>, mgrid, dim3(256), 0, stream, p, g, tail_units);
  else
    hipLaunchKernelGGL(prefill_merge_kernel<64>, mgrid, dim3(128), 0, stream, p, g, tail_units);
  return hipGetLastError();
}

int64_t prefill_units(int32_t batch, int32_t s_q, int32_t num_q_heads) {
  return (int64_t)batch * num_q_heads * ((s_q + kQT - 1) / kQT);
}

size_t prefill_slot_bytes() { return (size_t)kSlotFloats * sizeof(float); }

}  // namespace pkv
