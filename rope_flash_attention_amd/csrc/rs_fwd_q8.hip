// The blockwise int8 forward (Q'K'^T on int8 MFMA) for every mask kind and causal: codes
// quantized in the attention kernel (mode 1) or read from the quantizer pass (mode 2).  The
// kernel template is rs_fwd_kernel.hpp's.
#include "rs_fwd_kernel.hpp"

namespace rs {

template <typename T>
static int launch_q8_t(int D, int mask_kind, bool causal, int mode, const FwdParams& p, void* stream) {
  return mode == 2 ? launch_fwd_q_d<T, 2>(D, mask_kind, causal, p, stream)
                   : launch_fwd_q_d<T, 1>(D, mask_kind, causal, p, stream);
}

int launch_fwd_q8(int dtype, int D, int mask_kind, bool causal, int mode, const FwdParams& p, void* stream) {
  if (mode != 1 && mode != 2) return -1;
  return dtype == F16 ? launch_q8_t<_Float16>(D, mask_kind, causal, mode, p, stream)
                      : launch_q8_t<__bf16>(D, mask_kind, causal, mode, p, stream);
}

}  // namespace rs
