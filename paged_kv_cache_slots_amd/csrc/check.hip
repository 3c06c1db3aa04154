// Device-side content checks (debugging aid).
//
// "Paged causal K/V cache and cached attention for VisualGen", Per-File QA
// Perspective: the scatter does not range-check device slot ids, and device
// slot bounds stay the caller's responsibility.  These kernels count the
// entries that would break that contract, reading only the ids and lengths
// (never the pool), so a bad entry is reported instead of touching memory.
//
// One workgroup walks the whole input (a debugging call, not a hot path):
// every thread counts its share, the workgroup sums through LDS and thread 0
// writes the total, so the result needs no zeroing and no atomics.
//
// Also here: the probe of where workgroups run.  The prefill's persistent
// schedule gives the kv heads of group x to workgroups x, x + 8, ... on the
// assumption that workgroups whose ids agree mod 8 run on one XCD (the
// dispatcher deals workgroups to the XCDs round robin); the probe lets a test
// (or a caller) check that on the device at hand.
#include "pkv_device.hpp"
#include "pkv_internal.hpp"

namespace pkv {

namespace {

constexpr int kCheckThreads = 1024;

__device__ __forceinline__ void write_total(int64_t mine, int32_t* bad) {
  __shared__ int64_t part[kCheckThreads / 64];
  for (int off = 32; off >= 1; off >>= 1) mine += __shfl_xor(mine, off, 64);
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = mine;
  __syncthreads();
  if (threadIdx.x == 0) {
    int64_t total = 0;
    for (int w = 0; w < kCheckThreads / 64; ++w) total += part[w];
    *bad = total > INT32_MAX ? INT32_MAX : (int32_t)total;
  }
}

__global__ void __launch_bounds__(kCheckThreads) check_slots_kernel(const int64_t* slots, int64_t n, int64_t capacity,
                                                                    int32_t* bad) {
  int64_t mine = 0;
  for (int64_t i = threadIdx.x; i < n; i += kCheckThreads) mine += slots[i] >= capacity ? 1 : 0;
  write_total(mine, bad);
}

__global__ void __launch_bounds__(kCheckThreads) check_tables_kernel(const int32_t* table, int32_t stride,
                                                                     const int32_t* lens, int32_t rows,
                                                                     int32_t page_shift, int64_t num_pages,
                                                                     int32_t* bad) {
  int64_t mine = 0;
  for (int r = threadIdx.x; r < rows; r += kCheckThreads) {
    const int64_t len = lens[r];
    bool wrong = len < 0 || len > ((int64_t)stride << page_shift);
    if (!wrong) {
      const int64_t used = (len + (int64_t(1) << page_shift) - 1) >> page_shift;
      for (int64_t j = 0; j < used && !wrong; ++j) {
        const int32_t pg = table[(int64_t)r * stride + j];
        wrong = pg < 0 || pg >= num_pages;
      }
    }
    mine += wrong ? 1 : 0;
  }
  write_total(mine, bad);
}

// Workgroup i writes the XCC_ID hardware register (the XCD it runs on) of
// its first wave to out[i].
__global__ void xcd_ids_kernel(int32_t* out) {
  const int v = __builtin_amdgcn_s_getreg(20 | (0 << 6) | (31 << 11));   // hwreg(HW_REG_XCC_ID), all 32 bits
  if (threadIdx.x == 0) out[blockIdx.x] = v;
}

}  // namespace

hipError_t launch_xcd_ids(int32_t* out, int32_t num_workgroups, int32_t threads, hipStream_t stream) {
  hipLaunchKernelGGL(xcd_ids_kernel, dim3((unsigned)num_workgroups), dim3((unsigned)threads), 0, stream, out);
  return hipGetLastError();
}

hipError_t launch_check_slots(const int64_t* slots, int64_t n, int64_t capacity, int32_t* bad, hipStream_t stream) {
  hipLaunchKernelGGL(check_slots_kernel, dim3(1), dim3(kCheckThreads), 0, stream, slots, n, capacity, bad);
  return hipGetLastError();
}

hipError_t launch_check_tables(const int32_t* table, int32_t stride, const int32_t* lens, int32_t rows,
                               int32_t page_shift, int64_t num_pages, int32_t* bad, hipStream_t stream) {
  hipLaunchKernelGGL(check_tables_kernel, dim3(1), dim3(kCheckThreads), 0, stream, table, stride, lens, rows,
                     page_shift, num_pages, bad);
  return hipGetLastError();
}

}  // namespace pkv
