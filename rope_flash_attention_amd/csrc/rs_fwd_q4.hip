// The blockwise int4 forward (codes in [-7, 7], one per byte, on int8 MFMA) for every mask
// kind and causal: codes quantized in the attention kernel (mode 5) or read from the
// quantizer pass (mode 6).  The kernel template is rs_fwd_kernel.hpp's.
#include "rs_fwd_kernel.hpp"

namespace rs {

template <typename T>
static int launch_q4_t(int D, int mask_kind, bool causal, int mode, const FwdParams& p, void* stream) {
  return mode == 6 ? launch_fwd_q_d<T, 6>(D, mask_kind, causal, p, stream)
                   : launch_fwd_q_d<T, 5>(D, mask_kind, causal, p, stream);
}

int launch_fwd_q4(int dtype, int D, int mask_kind, bool causal, int mode, const FwdParams& p, void* stream) {
  if (mode != 5 && mode != 6) return -1;
  return dtype == F16 ? launch_q4_t<_Float16>(D, mask_kind, causal, mode, p, stream)
                      : launch_q4_t<__bf16>(D, mask_kind, causal, mode, p, stream);
}

}  // namespace rs
