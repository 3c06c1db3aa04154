// Exact-window commit operations.
//
// "Paged causal K/V cache and cached attention for VisualGen", Description /
// Cache: eviction from the rolling history window rotates the page table in
// place on the device, and commit fills the blocks' private pages with one
// pool-to-pool copy whose entry list carries sentinels.
//
// Row rotation: element c of a row takes the old element (c + shift) mod
// cols.  One workgroup per row (grid-stride over rows, so any row count
// works).  A row that fits 32 KiB of LDS is staged there and written back
// rotated; a longer row is rotated in place by three reversals
// ([0, s), [s, n), [0, n)), each pass separated by a workgroup barrier.
//
// Slot copy: entry i copies slot src[i] to slot dst[i] (the whole key row:
// all kv heads, all dims, K and V) in every layer; a negative source or
// destination skips the entry.  One thread moves one vector of one (entry,
// layer) row; bytes are copied untouched.
#include "pkv_device.hpp"
#include "pkv_internal.hpp"

namespace pkv {

namespace {

constexpr int kRotThreads = 256;
constexpr int kRotLdsBytes = 32768;

template <typename T>
__device__ __forceinline__ void reverse_range(T* row, int64_t a, int64_t b) {
  const int64_t half = (b - a) >> 1;
  for (int64_t i = threadIdx.x; i < half; i += kRotThreads) {
    const T x = row[a + i];
    row[a + i] = row[b - 1 - i];
    row[b - 1 - i] = x;
  }
}

}  // namespace

template <typename T>
__global__ __launch_bounds__(kRotThreads) void rotate_lds_kernel(RotateParams p) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[kRotLdsBytes];
  T* buf = reinterpret_cast<T*>(smem);
  for (int64_t r = blockIdx.x; r < p.rows; r += gridDim.x) {
    T* row = reinterpret_cast<T*>(p.data + r * p.row_stride_b);
    for (int64_t c = threadIdx.x; c < p.cols; c += kRotThreads) buf[c] = row[c];
    __syncthreads();
    for (int64_t c = threadIdx.x; c < p.cols; c += kRotThreads) {
      int64_t s = c + p.shift;
      s = s >= p.cols ? s - p.cols : s;
      row[c] = buf[s];
    }
    __syncthreads();
  }
}

template <typename T>
__global__ __launch_bounds__(kRotThreads) void rotate_rev_kernel(RotateParams p) {
  for (int64_t r = blockIdx.x; r < p.rows; r += gridDim.x) {
    T* row = reinterpret_cast<T*>(p.data + r * p.row_stride_b);
    reverse_range(row, 0, p.shift);
    reverse_range(row, p.shift, p.cols);
    __syncthreads();
    reverse_range(row, 0, p.cols);
    __syncthreads();
  }
}

template <typename T>
static hipError_t launch_rotate_t(const RotateParams& p, hipStream_t stream) {
  const unsigned grid = (unsigned)(p.rows < 65535 ? p.rows : 65535);
  if (p.cols * (int64_t)sizeof(T) <= kRotLdsBytes)
    hipLaunchKernelGGL(rotate_lds_kernel<T>, dim3(grid), dim3(kRotThreads), 0, stream, p);
  else
    hipLaunchKernelGGL(rotate_rev_kernel<T>, dim3(grid), dim3(kRotThreads), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_rotate(const RotateParams& p, int elem_size, hipStream_t stream) {
  switch (elem_size) {
    case 1: return launch_rotate_t<uint8_t>(p, stream);
    case 2: return launch_rotate_t<uint16_t>(p, stream);
    case 4: return launch_rotate_t<uint32_t>(p, stream);
    case 8: return launch_rotate_t<uint64_t>(p, stream);
    default: return launch_rotate_t<u32x4>(p, stream);
  }
}

template <typename V>
__global__ __launch_bounds__(256) void copy_slots_kernel(CopySlotsParams p) {
  const int64_t per_entry = (int64_t)p.num_layers * p.vecs_per_row;
  const int64_t total = p.n * per_entry;
  const int64_t mask = (int64_t(1) << p.page_shift) - 1;
  for (int64_t w = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; w < total;
       w += (int64_t)gridDim.x * blockDim.x) {
    const int64_t e = w / per_entry;
    const int64_t rem = w - e * per_entry;
    const int64_t layer = rem / p.vecs_per_row;
    const int64_t v = rem - layer * p.vecs_per_row;
    const int64_t s = p.src[e], d = p.dst[e];
    if (s < 0 || d < 0) continue;
    const int64_t base = layer * p.layer_stride_b + v * (int64_t)sizeof(V);
    const int64_t so = base + (s >> p.page_shift) * p.page_stride_b + (s & mask) * p.row_b;
    const int64_t dof = base + (d >> p.page_shift) * p.page_stride_b + (d & mask) * p.row_b;
    const V kx = *reinterpret_cast<const V*>(p.pool_k + so);
    const V vx = *reinterpret_cast<const V*>(p.pool_v + so);
    *reinterpret_cast<V*>(p.pool_k + dof) = kx;
    *reinterpret_cast<V*>(p.pool_v + dof) = vx;
  }
}

hipError_t launch_copy_slots(const CopySlotsParams& p, int vec_bytes, hipStream_t stream) {
  const int64_t total = p.n * (int64_t)p.num_layers * p.vecs_per_row;
  int64_t blocks = (total + 255) / 256;
  if (blocks > 8192) blocks = 8192;   // grid-stride beyond this
  const dim3 grid((unsigned)blocks), block(256);
  switch (vec_bytes) {
    case 16: hipLaunchKernelGGL(copy_slots_kernel<u32x4>, grid, block, 0, stream, p); break;
    case 8: hipLaunchKernelGGL(copy_slots_kernel<u32x2>, grid, block, 0, stream, p); break;
    case 4: hipLaunchKernelGGL(copy_slots_kernel<uint32_t>, grid, block, 0, stream, p); break;
    case 2: hipLaunchKernelGGL(copy_slots_kernel<uint16_t>, grid, block, 0, stream, p); break;
    default: hipLaunchKernelGGL(copy_slots_kernel<uint8_t>, grid, block, 0, stream, p); break;
  }
  return hipGetLastError();
}

}  // namespace pkv
