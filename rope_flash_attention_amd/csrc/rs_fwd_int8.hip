// Blockwise int8 / int4 quantization of the rotated Q and K (forward with
// RS_FLAG_QUANT_INT8_QK or RS_FLAG_QUANT_INT4_QK, and the quantizer pass).
//
// The pages (page "Metal Flash Attention", SimpleTuner docs, sections "Requirements" and
// "Enable In SimpleTuner") name int8 and int4 modes with blockwise quantization but not what
// is quantized.  Reading implemented here and in the quantized attention kernel: Q' = R(Q)
// and K' = R(K) are evaluated in fp32 (each product and each sum rounded, no fused
// multiply-add), then each (b, h, block of 64 tokens) spanning all of D gets, with
// qmax = 127 (int8) or 7 (int4),
//     amax  = max |x'|                   over the block's valid rows
//     inv   = fp32(qmax / amax)          (correctly rounded division)
//     code  = round-half-even(fp32(x' * inv)), clamped to [-qmax, qmax]
//     scale = fp32(amax / qmax)
// and an all-zero block gets codes 0 and scale 0.  Scores are then
//     s = softmax_scale * scale_q * scale_k * (codes_q . codes_k),
// the integer product being exact on int8 MFMA (|sum| <= 128 * 127^2 < 2^31); int4 codes
// are stored one per byte and take the same instruction.
//
// One workgroup of 256 threads per (block, head, sample, tensor): it holds the block's
// rotated values in registers (64 rows x D / 256 threads), reduces the block maximum through
// LDS, and writes the codes (rows past S as zeros, up to the slice's allocated rows) and
// the scale.
#include "rs_device.hpp"

namespace rs {

constexpr int kQuantBlock = 64;

template <typename T, int D, bool DEQ>
__global__ __launch_bounds__(256) void quant_kernel(QuantParams p) {
  constexpr int UPR = D / 8;                 // 8-element units per row
  constexpr int UPT = kQuantBlock * UPR / 256;  // units per thread
  static_assert(UPT * 256 == kQuantBlock * UPR, "block split");
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int blk = blockIdx.x, h = blockIdx.y, b = blockIdx.z >> 1, which = blockIdx.z & 1;
  if (h >= p.Hx[which]) return;  // K with fewer heads than Q (grouped-query attention)
  const Opnd x = p.x[which];
  const T* xb = (const T*)x.ptr + b * x.sb + h * x.sh;
  const float* tab = p.tab.ptr + b * p.tab.sb;  // (cos, sin) pairs, D floats per row

  float v[UPT][8];
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < UPT; ++i) {
    const int u = tid + 256 * i, row = u / UPR, ch = u % UPR;
    const int s = blk * kQuantBlock + row;
    if (s < p.S) {
      typedef T v8 __attribute__((ext_vector_type(8)));
      const v8 e = *(const v8*)(xb + (int64_t)s * x.ss + ch * 8);
      const float4 t0 = *(const float4*)(tab + (int64_t)s * D + ch * 8);
      const float4 t1 = *(const float4*)(tab + (int64_t)s * D + ch * 8 + 4);
      const float cs[8] = {t0.x, t0.y, t0.z, t0.w, t1.x, t1.y, t1.z, t1.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float2 r = rot_pair(to_f(e[2 * j]), to_f(e[2 * j + 1]), cs[2 * j], cs[2 * j + 1]);
        v[i][2 * j] = r.x;
        v[i][2 * j + 1] = r.y;
        amax = fmaxf(amax, fmaxf(fabsf(r.x), fabsf(r.y)));
      }
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) v[i][j] = 0.f;
    }
  }
  // block maximum: within the wave, then across the four waves
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off, 64));
  __shared__ float red[4];
  if (lane == 0) red[wave] = amax;
  __syncthreads();
  amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  const float inv = amax > 0.f ? p.qmax / amax : 0.f;
  const float scale = amax > 0.f ? amax / p.qmax : 0.f;

  if constexpr (DEQ) {  // the dequantized values, code * scale, in the input dtype
    T* db = (T*)p.deq[which] + ((int64_t)b * p.Hx[which] + h) * p.S * D;
#pragma unroll
    for (int i = 0; i < UPT; ++i) {
      const int u = tid + 256 * i, row = u / UPR, ch = u % UPR;
      const int s = blk * kQuantBlock + row;
      if (s >= p.S) continue;
      typedef T v8 __attribute__((ext_vector_type(8)));
      v8 y;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        float c = __builtin_rintf(v[i][j] * inv);  // round half to even
        c = fminf(fmaxf(c, -p.qmax), p.qmax);
        y[j] = from_f<T>(c * scale);
      }
      *(v8*)(db + (int64_t)s * D + ch * 8) = y;
    }
    return;
  }

  int8_t* cb = p.codes[which] + b * p.c_sb[which] + h * p.c_sh[which];
#pragma unroll
  for (int i = 0; i < UPT; ++i) {
    const int u = tid + 256 * i, row = u / UPR, ch = u % UPR;
    const int s = blk * kQuantBlock + row;
    if (s >= p.rows) continue;
    uint32_t w[2] = {0u, 0u};
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      float c = __builtin_rintf(v[i][j] * inv);  // round half to even
      c = fminf(fmaxf(c, -p.qmax), p.qmax);
      w[j >> 2] |= ((uint32_t)(int)c & 0xffu) << (8 * (j & 3));
    }
    *(uint2*)(cb + (int64_t)s * D + ch * 8) = make_uint2(w[0], w[1]);
  }
  if (tid == 0) p.scales[which][((int64_t)b * p.Hx[which] + h) * p.nblk + blk] = scale;
}

template <typename T, bool DEQ>
static int launch_quant_td(const QuantParams& p, void* stream) {
  const dim3 grid(p.nblk, p.H, 2 * p.B);
  if (p.D == 64)
    hipLaunchKernelGGL((quant_kernel<T, 64, DEQ>), grid, dim3(256), 0, (hipStream_t)stream, p);
  else
    hipLaunchKernelGGL((quant_kernel<T, 128, DEQ>), grid, dim3(256), 0, (hipStream_t)stream, p);
  return (int)hipGetLastError();
}

template <typename T>
static int launch_quant_t(const QuantParams& p, void* stream) {
  return p.deq[0] ? launch_quant_td<T, true>(p, stream) : launch_quant_td<T, false>(p, stream);
}

int launch_quant_int8(int dtype, const QuantParams& p, void* stream) {
  return dtype == F16 ? launch_quant_t<_Float16>(p, stream) : launch_quant_t<__bf16>(p, stream);
}

}  // namespace rs
