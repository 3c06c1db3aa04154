// Block-causal paged prefill (placeholder until the MFMA kernel lands).
#include "pkv_device.hpp"
#include "pkv_internal.hpp"

namespace pkv {

hipError_t launch_prefill_mfma(const PrefillParams& p, int head_dim, hipStream_t stream) {
  (void)p; (void)head_dim; (void)stream;
  return hipErrorNotSupported;
}

}  // namespace pkv
