// Slot scatter: new K/V token rows -> pool slots.
//
// "Paged causal K/V cache and cached attention for VisualGen", Description /
// Cache (chunk K/V write): the source is read once with any token/head stride
// and every token lands in one or two pool slots; optional source indices.
// Slot s is row s & (page_size - 1) of page s >> log2(page_size) (review
// thread on slot ids: view_page * tokens_per_page + slot).
//
// One thread moves one vector (16, 8, 4, 2 or 1 bytes, the widest the host
// found legal) of one (token, kv head) row; consecutive threads walk a row,
// then the heads of a token, so a wave reads and writes whole rows.  Bytes
// are copied untouched, so fp8 codes stay codes.
#include "pkv_device.hpp"
#include "pkv_internal.hpp"

namespace pkv {

template <typename V>
__global__ __launch_bounds__(256) void scatter_kernel(ScatterParams p) {
  const uint32_t per_tok = (uint32_t)p.num_kv_heads * (uint32_t)p.vecs_per_row;
  const int64_t total = p.n_tokens * (int64_t)per_tok;
  const int64_t row_bytes = (int64_t)p.vecs_per_row * (int64_t)sizeof(V);
  const int64_t mask = (int64_t(1) << p.page_shift) - 1;
  for (int64_t w = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; w < total;
       w += (int64_t)gridDim.x * blockDim.x) {
    const int64_t tok = w / per_tok;
    const uint32_t rem = (uint32_t)(w - tok * per_tok);
    const uint32_t h = rem / (uint32_t)p.vecs_per_row;
    const uint32_t v = rem - h * (uint32_t)p.vecs_per_row;
    int64_t s1;
    if (p.table) {
      const int64_t t = tok / p.q_len;
      const int key = p.lens[t] - p.q_len + (int)(tok - t * p.q_len);
      s1 = key < 0 ? -1
                   : ((int64_t)p.table[t * p.table_stride + (key >> p.page_shift)] << p.page_shift) +
                         (key & (int)mask);
    } else {
      s1 = p.slots[tok];
    }
    const int64_t s2 = p.slots2 ? p.slots2[tok] : -1;
    if (s1 < 0 && s2 < 0) continue;
    const int64_t src_row = p.src_idx ? p.src_idx[tok] : tok;
    const int64_t src_off = src_row * p.src_tok_stride_b + (int64_t)h * p.src_head_stride_b + (int64_t)v * sizeof(V);
    const V kv = *reinterpret_cast<const V*>(p.src_k + src_off);
    const V vv = *reinterpret_cast<const V*>(p.src_v + src_off);
    const int64_t in_row = (int64_t)h * row_bytes + (int64_t)v * sizeof(V);
    if (s1 >= 0) {
      const int64_t dst = (s1 >> p.page_shift) * p.page_stride_b + (s1 & mask) * p.row_stride_b + in_row;
      *reinterpret_cast<V*>(p.pool_k + dst) = kv;
      *reinterpret_cast<V*>(p.pool_v + dst) = vv;
    }
    if (s2 >= 0) {
      const int64_t dst = (s2 >> p.page_shift) * p.page_stride_b + (s2 & mask) * p.row_stride_b + in_row;
      *reinterpret_cast<V*>(p.pool_k + dst) = kv;
      *reinterpret_cast<V*>(p.pool_v + dst) = vv;
    }
  }
}

hipError_t launch_scatter(const ScatterParams& p, int vec_bytes, hipStream_t stream) {
  const int64_t total = p.n_tokens * (int64_t)p.num_kv_heads * p.vecs_per_row;
  int64_t blocks = (total + 255) / 256;
  if (blocks > 8192) blocks = 8192;   // grid-stride beyond this
  const dim3 grid((unsigned)blocks), block(256);
  switch (vec_bytes) {
    case 16: hipLaunchKernelGGL(scatter_kernel<u32x4>, grid, block, 0, stream, p); break;
    case 8: hipLaunchKernelGGL(scatter_kernel<u32x2>, grid, block, 0, stream, p); break;
    case 4: hipLaunchKernelGGL(scatter_kernel<uint32_t>, grid, block, 0, stream, p); break;
    case 2: hipLaunchKernelGGL(scatter_kernel<uint16_t>, grid, block, 0, stream, p); break;
    default: hipLaunchKernelGGL(scatter_kernel<uint8_t>, grid, block, 0, stream, p); break;
  }
  return hipGetLastError();
}

}  // namespace pkv
