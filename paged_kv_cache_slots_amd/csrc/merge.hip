// Attention-state merge by log-sum-exp.
//
// "Support shared-prefix attention for n-sample requests in FMHA": the FA4
// tail commit joins the shared-prefix state and each row's private-tail state
// with one merge kernel in natural-log LSE; the small-batch split commit makes
// an empty run carry LSE -inf, so merges skip it.
//
// For states i with output o_i (normalised over its keys) and lse_i:
//   m = max_i lse_i,  w_i = exp(lse_i - m),
//   o = sum_i w_i o_i / sum_i w_i,  lse = m + ln sum_i w_i;
// all states empty -> o = 0, lse = -inf.  A state whose weight is 0 is never
// read, so its output may hold anything (the decode splits rely on this).
//
// One thread owns 4 consecutive dims of one (row, head); it reads the N LSE
// values of its (row, head) (cached: the 32 threads of a row-head share them)
// and one float4 per state.  The same kernel merges the decode's split states:
// there the number of valid states of a row follows from its table row's
// kv_len, and the states past it are not read.
#include "pkv_device.hpp"
#include "pkv_internal.hpp"

namespace pkv {

template <bool kBf16Out>
__global__ __launch_bounds__(256) void merge_kernel(MergeParams p) {
  const int chunks = p.head_dim >> 2;
  const int64_t total = p.rows * (int64_t)p.num_q_heads * chunks;
  const int64_t tid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (tid >= total) return;
  const int c = (int)(tid % chunks);
  const int64_t rh = tid / chunks;            // row * Hq + h
  const int64_t row = rh / p.num_q_heads;
  const int64_t plane = p.rows * (int64_t)p.num_q_heads;

  int n_valid = p.num_states;
  if (p.kv_lens) {
    const int64_t len = p.kv_lens[row / p.rows_per_table];
    const int64_t need = (len + p.keys_per_state - 1) / p.keys_per_state;
    n_valid = need < n_valid ? (int)need : n_valid;
  }
  float m = kNegInf;
  for (int i = 0; i < n_valid; ++i) m = fmaxf(m, p.lse_parts[i * plane + rh]);

  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  float lse_out = kNegInf;
  if (m != kNegInf) {
    float wsum = 0.f;
    for (int i = 0; i < n_valid; ++i) {
      const float w = fast_exp2((p.lse_parts[i * plane + rh] - m) * kLog2e);
      if (w > 0.f) {
        const f32x4 o = *reinterpret_cast<const f32x4*>(p.o_parts + (i * plane + rh) * p.head_dim + 4 * c);
        acc += w * o;
        wsum += w;
      }
    }
    acc *= 1.0f / wsum;
    lse_out = m + fast_log2(wsum) * kLn2;
  }
  const int64_t o_off = rh * p.head_dim + 4 * c;
  if constexpr (kBf16Out) {
    u32x2 packed;
    packed[0] = pack_bf16x2(acc[0], acc[1]);
    packed[1] = pack_bf16x2(acc[2], acc[3]);
    *reinterpret_cast<u32x2*>(reinterpret_cast<uint16_t*>(p.out) + o_off) = packed;
  } else {
    *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(p.out) + o_off) = acc;
  }
  if (p.out_lse && c == 0) p.out_lse[rh] = lse_out;
}

hipError_t launch_merge(const MergeParams& p, hipStream_t stream) {
  const int64_t total = p.rows * (int64_t)p.num_q_heads * (p.head_dim >> 2);
  const dim3 grid((unsigned)((total + 255) / 256)), block(256);
  if (p.out_bf16)
    hipLaunchKernelGGL(merge_kernel<true>, grid, block, 0, stream, p);
  else
    hipLaunchKernelGGL(merge_kernel<false>, grid, block, 0, stream, p);
  return hipGetLastError();
}

}  // namespace pkv
