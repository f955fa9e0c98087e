// Forward with the Q/K prologue of flux-style attention: Q and K RMS-normalized over the head
// dimension (x / sqrt(mean x^2 + eps) * w, in fp32) and/or read in fp32 while V, O and the
// matrix products are in bf16/fp16 (the autocast layout of the diffusers issue "Flux-family
// attention: flash-attn and other backends fail in an autocast context", sections "Describe
// the bug" and "Root cause, in order").
//
// K is prepared once, by kprep_kernel: normalized, rotated and rounded to the compute dtype
// into the workspace.  The attention kernel then reads K' like plain attention reads K (no
// tables in the key loop), while Q is normalized and rotated in the attention kernel's own
// prologue.  Folding K's prologue into the key loop instead would repeat it for every query
// tile and, with fp32 K, double the bytes of every K tile read; its registers also push the
// key loop past its budget.  The preparation is one read of K and one write of K' (HBM-bound).
#include "rs_fwd_kernel.hpp"

namespace rs {

// One row of K per D/8 consecutive threads, 8 elements (4 rotation pairs) per thread.
template <typename TI, typename TO, bool NORM>
__global__ __launch_bounds__(256) void kprep_kernel(KPrepParams p) {
  const int tpr = p.D / 8;  // threads per row (8 or 16: a row never straddles a wave)
  const int64_t rows = (int64_t)p.B * p.H * p.S;
  const int64_t n = rows * tpr;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) {
    // n and the stride are multiples of tpr: the threads of a row stay in the loop together
    const int ch = (int)(i % tpr);
    const int64_t row = i / tpr;
    const int s = (int)(row % p.S);
    const int64_t bh = row / p.S;
    const int h = (int)(bh % p.H), b = (int)(bh / p.H);
    const TI* src = (const TI*)p.x.ptr + b * p.x.sb + h * p.x.sh + (int64_t)s * p.x.ss + ch * 8;
    float x[8];
    if constexpr (sizeof(TI) == 4) {
      const float4 a = *(const float4*)src, c = *(const float4*)(src + 4);
      x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
      x[4] = c.x; x[5] = c.y; x[6] = c.z; x[7] = c.w;
    } else {
      typedef TI v8 __attribute__((ext_vector_type(8)));
      const v8 v = *(const v8*)src;
#pragma unroll
      for (int e = 0; e < 8; ++e) x[e] = to_f(v[e]);
    }
    if constexpr (NORM) {
      float ssq = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) ssq = fmaf(x[e], x[e], ssq);
      for (int off = tpr / 2; off >= 1; off >>= 1) ssq += __shfl_xor(ssq, off, tpr);
      const float inv = 1.f / __builtin_sqrtf(ssq * (1.f / (float)p.D) + p.eps);
      const float4 wa = *(const float4*)(p.w + ch * 8), wb = *(const float4*)(p.w + ch * 8 + 4);
      const float wv[8] = {wa.x, wa.y, wa.z, wa.w, wb.x, wb.y, wb.z, wb.w};
#pragma unroll
      for (int e = 0; e < 8; ++e) x[e] = x[e] * inv * wv[e];
    }
    // packed table row: (cos, sin) of pair i at floats 2i, 2i + 1
    const float* tr = p.tab.ptr + b * p.tab.sb + (int64_t)s * p.D + ch * 8;
    const float4 t0 = *(const float4*)tr, t1 = *(const float4*)(tr + 4);
    const float cc[4] = {t0.x, t0.z, t1.x, t1.z}, ss[4] = {t0.y, t0.w, t1.y, t1.w};
    typedef TO vo __attribute__((ext_vector_type(8)));
    vo y;
#pragma unroll
    for (int pp = 0; pp < 4; ++pp) {
      const float2 rr = rot_pair_fma(x[2 * pp], x[2 * pp + 1], cc[pp], ss[pp]);
      y[2 * pp] = from_f<TO>(rr.x);
      y[2 * pp + 1] = from_f<TO>(rr.y);
    }
    *(vo*)((TO*)p.out + row * p.D + ch * 8) = y;
  }
}

template <typename TI, typename TO>
static int launch_kprep_t(bool norm, const KPrepParams& p, void* stream) {
  const int64_t n = (int64_t)p.B * p.H * p.S * (p.D / 8);
  int64_t blocks = (n + 255) / 256;
  if (blocks > 16384) blocks = 16384;
  if (blocks < 1) blocks = 1;
  if (norm)
    hipLaunchKernelGGL((kprep_kernel<TI, TO, true>), dim3((unsigned)blocks), dim3(256), 0, (hipStream_t)stream, p);
  else
    hipLaunchKernelGGL((kprep_kernel<TI, TO, false>), dim3((unsigned)blocks), dim3(256), 0, (hipStream_t)stream, p);
  return (int)hipGetLastError();
}

int launch_kprep(int dtype, int qkm, const KPrepParams& p, void* stream) {
  const bool norm = (qkm & 1) != 0, f32in = (qkm & 2) != 0;
  switch (dtype) {
    case F32: return launch_kprep_t<float, float>(norm, p, stream);
    case F16: return f32in ? launch_kprep_t<float, _Float16>(norm, p, stream)
                           : launch_kprep_t<_Float16, _Float16>(norm, p, stream);
    default: return f32in ? launch_kprep_t<float, __bf16>(norm, p, stream)
                          : launch_kprep_t<__bf16, __bf16>(norm, p, stream);
  }
}

template <typename T, int D, int QKM>
static int launch_qk_t(int mask_kind, bool causal, const FwdParams& p, void* stream) {
  if (causal) return launch_fwd_t<T, D, MASK_NONE, true, 0, true, false, QKM>(p, stream);
  if (mask_kind == MASK_BOOL) return launch_fwd_t<T, D, MASK_BOOL, false, 0, true, false, QKM>(p, stream);
  return launch_fwd_t<T, D, MASK_NONE, false, 0, true, false, QKM>(p, stream);
}

template <typename T, int QKM>
static int launch_qk_d(int D, int mask_kind, bool causal, const FwdParams& p, void* stream) {
  return D == 64 ? launch_qk_t<T, 64, QKM>(mask_kind, causal, p, stream)
                 : launch_qk_t<T, 128, QKM>(mask_kind, causal, p, stream);
}

template <typename T>
static int launch_qk_m(int D, int mask_kind, bool causal, int qkm, const FwdParams& p, void* stream) {
  switch (qkm) {
    case 4: return launch_qk_d<T, 4>(D, mask_kind, causal, p, stream);
    case 5: return launch_qk_d<T, 5>(D, mask_kind, causal, p, stream);
    case 6: return launch_qk_d<T, 6>(D, mask_kind, causal, p, stream);
    case 7: return launch_qk_d<T, 7>(D, mask_kind, causal, p, stream);
    default: return -1;
  }
}

int launch_fwd_qk(int dtype, int D, int mask_kind, bool causal, int qkm, const FwdParams& p, void* stream) {
  switch (dtype) {
    case F32:  // fp32 throughout: normalization only
      return qkm == 5 ? launch_qk_d<float, 5>(D, mask_kind, causal, p, stream) : -1;
    case F16: return launch_qk_m<_Float16>(D, mask_kind, causal, qkm, p, stream);
    default: return launch_qk_m<__bf16>(D, mask_kind, causal, qkm, p, stream);
  }
}

}  // namespace rs
