// Plain attention forward, no rotation (the caller passes no tables): the same kernels as
// the fused forward with the rotation left out, in their own translation unit.  It is the
// attention half of the eager path (a rotation pass, then attention) that the fused forward
// replaces (page "Metal Flash Attention", section "Fused RoPE + SDPA").
#include "rs_fwd_kernel.hpp"

namespace rs {

int launch_fwd_plain(int dtype, int D, int mask_kind, bool causal, const FwdParams& p, void* stream) {
  switch (dtype) {
    case F32: return launch_fwd_dt<float, false>(D, mask_kind, causal, p, stream);
    case F16: return launch_fwd_dt<_Float16, false>(D, mask_kind, causal, p, stream);
    default: return launch_fwd_dt<__bf16, false>(D, mask_kind, causal, p, stream);
  }
}

}  // namespace rs
