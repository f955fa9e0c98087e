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

// One position s per D/8 consecutive threads (8 elements, 4 rotation pairs, per thread), for a
// group of up to kKprepHeads heads of one sample: the table row is read once for all of them
// (one group's rows of K span all heads; re-reading the caller's pair-duplicated tables per
// head would move more bytes than K itself), and every head's row is loaded before the first
// is rotated.  With PACK the first head group also writes the packed (cos, sin) rows that the
// attention kernel's Q prologue reads, and workgroup 0 clears the control words (the work of
// pack_tables_kernel, in the same launch).  Grid: (row blocks) x (head groups) x (samples),
// flattened; no thread divides by S or H.
constexpr int kKprepHeads = 8;

template <typename TI, typename TO, bool NORM, bool PACK, bool VEC>
__global__ __launch_bounds__(256) void kprep_kernel(KPrepParams p) {
  constexpr int HG = kKprepHeads;
  const int tpr = p.D / 8, rpw = 256 / tpr;  // threads per row (8 or 16: within a wave), rows per workgroup
  const int tid = threadIdx.x, ch = tid % tpr, r0 = tid / tpr;
  const int nbs = (p.S + rpw - 1) / rpw, ngr = (p.H + HG - 1) / HG;
  const int blk = blockIdx.x % nbs, t = blockIdx.x / nbs;
  const int g = t % ngr, b = t / ngr;
  if (PACK && blockIdx.x == 0 && tid < 2) p.pk.ctrl[tid] = 0u;
  const int srow = blk * rpw + r0;
  const int sc = min(srow, p.S - 1);  // rows past S: loads of a valid row, no store
  const int h0 = g * HG, nh = min(HG, p.H - h0);

  // the rows of every head of the group
  float x[HG][8];
  const TI* xs = (const TI*)p.x.ptr + b * p.x.sb + (int64_t)sc * p.x.ss + ch * 8;
#pragma unroll
  for (int j = 0; j < HG; ++j) {
    if (j >= nh) break;
    const TI* src = xs + (h0 + j) * p.x.sh;
    if constexpr (sizeof(TI) == 4) {
      const float4 a = *(const float4*)src, c = *(const float4*)(src + 4);
      x[j][0] = a.x; x[j][1] = a.y; x[j][2] = a.z; x[j][3] = a.w;
      x[j][4] = c.x; x[j][5] = c.y; x[j][6] = c.z; x[j][7] = c.w;
    } else {
      typedef TI v8 __attribute__((ext_vector_type(8)));
      const v8 v = *(const v8*)src;
#pragma unroll
      for (int e = 0; e < 8; ++e) x[j][e] = to_f(v[e]);
    }
  }
  // the table row, once: the caller's pair-duplicated rows, even entries
  const int tb = p.pk.Bt > 1 ? b : 0;
  const float* cr = p.pk.cos + tb * p.pk.c_sb + (int64_t)sc * p.pk.c_ss + ch * 8;
  const float* sr = p.pk.sin + tb * p.pk.s_sb + (int64_t)sc * p.pk.s_ss + ch * 8;
  float cc[4], ss[4];
  if constexpr (VEC) {  // 16-byte aligned table rows
    const float4 c0 = *(const float4*)cr, c1 = *(const float4*)(cr + 4);
    const float4 s0 = *(const float4*)sr, s1 = *(const float4*)(sr + 4);
    cc[0] = c0.x; cc[1] = c0.z; cc[2] = c1.x; cc[3] = c1.z;
    ss[0] = s0.x; ss[1] = s0.z; ss[2] = s1.x; ss[3] = s1.z;
  } else {
#pragma unroll
    for (int pp = 0; pp < 4; ++pp) {
      cc[pp] = cr[2 * pp];
      ss[pp] = sr[2 * pp];
    }
  }
  if (PACK && g == 0 && b < p.pk.Bt && srow < p.S) {
    float* pr = p.pk.out + ((int64_t)b * p.S + srow) * p.D + ch * 8;
    *(float4*)pr = make_float4(cc[0], ss[0], cc[1], ss[1]);
    *(float4*)(pr + 4) = make_float4(cc[2], ss[2], cc[3], ss[3]);
  }

  TO* out = (TO*)p.out + (((int64_t)b * p.H + h0) * p.S + srow) * p.D + ch * 8;
#pragma unroll
  for (int j = 0; j < HG; ++j) {
    if (j >= nh) break;
    if constexpr (NORM) {  // the tpr threads of a row share its sum of squares
      float ssq = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) ssq = fmaf(x[j][e], x[j][e], ssq);
      for (int off = tpr / 2; off >= 1; off >>= 1) ssq += __shfl_xor(ssq, off, tpr);
      const float inv = 1.f / __builtin_sqrtf(ssq * (1.f / (float)p.D) + p.eps);
      const float4 wa = *(const float4*)(p.w + ch * 8), wb = *(const float4*)(p.w + ch * 8 + 4);
      const float wv[8] = {wa.x, wa.y, wa.z, wa.w, wb.x, wb.y, wb.z, wb.w};
#pragma unroll
      for (int e = 0; e < 8; ++e) x[j][e] = x[j][e] * inv * wv[e];
    }
    typedef TO vo __attribute__((ext_vector_type(8)));
    vo y;
#pragma unroll
    for (int pp = 0; pp < 4; ++pp) {
      const float2 rr = rot_pair_fma(x[j][2 * pp], x[j][2 * pp + 1], cc[pp], ss[pp]);
      y[2 * pp] = from_f<TO>(rr.x);
      y[2 * pp + 1] = from_f<TO>(rr.y);
    }
    if (srow < p.S) *(vo*)(out + (int64_t)j * p.S * p.D) = y;
  }
}

template <typename TI, typename TO, bool PACK, bool VEC>
static int launch_kprep_t(bool norm, const KPrepParams& p, void* stream) {
  const int rpw = 256 / (p.D / 8);
  const int64_t blocks = (int64_t)((p.S + rpw - 1) / rpw) * ((p.H + kKprepHeads - 1) / kKprepHeads) * p.B;
  if (blocks < 1 || blocks > 0x7fffffff) return -1;
  if (norm)
    hipLaunchKernelGGL((kprep_kernel<TI, TO, true, PACK, VEC>), dim3((unsigned)blocks), dim3(256), 0,
                       (hipStream_t)stream, p);
  else
    hipLaunchKernelGGL((kprep_kernel<TI, TO, false, PACK, VEC>), dim3((unsigned)blocks), dim3(256), 0,
                       (hipStream_t)stream, p);
  return (int)hipGetLastError();
}

template <typename TI, typename TO>
static int launch_kprep_p(bool norm, const KPrepParams& p, void* stream) {
  const PackParams& t = p.pk;
  const bool vec = ((uintptr_t)t.cos % 16 == 0) && ((uintptr_t)t.sin % 16 == 0) && t.c_ss % 4 == 0 &&
                   t.s_ss % 4 == 0 && t.c_sb % 4 == 0 && t.s_sb % 4 == 0;
  if (p.pk.out)
    return vec ? launch_kprep_t<TI, TO, true, true>(norm, p, stream) : launch_kprep_t<TI, TO, true, false>(norm, p, stream);
  return vec ? launch_kprep_t<TI, TO, false, true>(norm, p, stream) : launch_kprep_t<TI, TO, false, false>(norm, p, stream);
}

int launch_kprep(int dtype, int qkm, const KPrepParams& p, void* stream) {
  const bool norm = (qkm & 1) != 0, f32in = (qkm & 2) != 0;
  switch (dtype) {
    case F32: return launch_kprep_p<float, float>(norm, p, stream);
    case F16: return f32in ? launch_kprep_p<float, _Float16>(norm, p, stream)
                           : launch_kprep_p<_Float16, _Float16>(norm, p, stream);
    default: return f32in ? launch_kprep_p<float, __bf16>(norm, p, stream)
                          : launch_kprep_p<__bf16, __bf16>(norm, p, stream);
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
