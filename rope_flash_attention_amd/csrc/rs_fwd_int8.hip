// Blockwise int8 Q'/K' forward variant (see rope_sdpa_fwd in include/rope_sdpa.h).
#include "rs_device.hpp"

namespace rs {

int launch_fwd_int8(int dtype, int D, const FwdParams& p, void* stream) {
  (void)dtype; (void)D; (void)p; (void)stream;
  return (int)hipErrorNotSupported;
}

}  // namespace rs
