// The fp8 K/V instantiation of the block-causal prefill kernel, in a
// translation unit of its own so that it is built with its own scheduler
// options (the bf16 kernel keeps the defaults).
#include "prefill_kernel.hpp"

namespace pkv {

hipError_t launch_prefill_kernel_fp8(const PrefillParams& p, int grid, hipStream_t stream) {
  PKV_LAUNCH_MAIN((prefill_kernel<128, true>), dim3((unsigned)grid), dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace pkv
