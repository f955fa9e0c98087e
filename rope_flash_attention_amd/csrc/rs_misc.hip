// Small kernels around attention on the caller's stream:
//  * table packing: the caller's pair-duplicated fp32 cos/sin tables (page "Metal Flash
//    Attention", section "Fused RoPE + SDPA": cos[2i] == cos[2i+1]) are repacked into one
//    array of (cos, sin) pairs per position, halving the table bytes the attention kernels
//    stream and making each pair one 8-byte read.  Q and K are not touched.
//  * bool-mask tile classification: each 64 x 64 block of the mask (at the mask's own
//    broadcast extents) is reduced to all-true / all-false / mixed, so attention can skip
//    all-false blocks and run all-true blocks with no mask reads (same page, section
//    "Enable In SimpleTuner": all-true bool masks are detected and skipped).  A device
//    counter records masks that were all-true everywhere.
#include "rs_device.hpp"

namespace rs {

__device__ unsigned long long g_all_true_masks = 0;

__global__ __launch_bounds__(256) void pack_tables_kernel(PackParams p) {
  if (blockIdx.x == 0 && threadIdx.x < 2) p.ctrl[threadIdx.x] = 0u;
  const int half = p.D / 2;
  const int64_t n = (int64_t)p.Bt * p.S * half;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) {
    const int pp = (int)(i % half);
    const int64_t bs = i / half;
    const int s = (int)(bs % p.S);
    const int b = (int)(bs / p.S);
    float2 v;
    v.x = p.cos[b * p.c_sb + (int64_t)s * p.c_ss + 2 * pp];
    v.y = p.sin[b * p.s_sb + (int64_t)s * p.s_ss + 2 * pp];
    ((float2*)p.out)[i] = v;
  }
}

int launch_pack_tables(const PackParams& p, void* stream) {
  const int64_t n = (int64_t)p.Bt * p.S * (p.D / 2);
  int64_t blocks = (n + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL(pack_tables_kernel, dim3((unsigned)blocks), dim3(256), 0, (hipStream_t)stream, p);
  return (int)hipGetLastError();
}

// The eager rotation pass: out = R(x) over a [B, H, S, D] operand, one 16-byte chunk of a row
// per thread (8 elements of bf16/fp16, 4 of fp32), reading the even entries of the caller's
// pair-duplicated fp32 tables.  Each product and sum is rounded to fp32 (no fused
// multiply-add), then the result to the operand's dtype.  Bound by HBM: one read and one
// write of x (the tables stay in cache across heads).
template <typename T>
__global__ __launch_bounds__(256) void rotate_kernel(RotateParams p) {
  constexpr int EPC = 16 / (int)sizeof(T);
  const int cpr = p.D / EPC;  // chunks per row
  const int64_t n = (int64_t)p.B * p.H * p.S * cpr;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) {
    const int ch = (int)(i % cpr);
    int64_t r = i / cpr;
    const int s = (int)(r % p.S);
    r /= p.S;
    const int h = (int)(r % p.H);
    const int b = (int)(r / p.H);
    typedef T vE __attribute__((ext_vector_type(EPC)));
    const vE x = *(const vE*)((const T*)p.x.ptr + b * p.x.sb + h * p.x.sh + (int64_t)s * p.x.ss + ch * EPC);
    const float* cr = p.cos + b * p.c_sb + (int64_t)s * p.c_ss + ch * EPC;
    const float* sr = p.sin + b * p.s_sb + (int64_t)s * p.s_ss + ch * EPC;
    vE y;
#pragma unroll
    for (int pp = 0; pp < EPC / 2; ++pp) {
      const float2 rr = rot_pair(to_f(x[2 * pp]), to_f(x[2 * pp + 1]), cr[2 * pp], sr[2 * pp]);
      y[2 * pp] = from_f<T>(rr.x);
      y[2 * pp + 1] = from_f<T>(rr.y);
    }
    *(vE*)((T*)p.out + b * p.o_sb + h * p.o_sh + (int64_t)s * p.o_ss + ch * EPC) = y;
  }
}

int launch_rotate(int dtype, const RotateParams& p, void* stream) {
  const int epc = dtype == F32 ? 4 : 8;
  const int64_t n = (int64_t)p.B * p.H * p.S * (p.D / epc);
  int64_t blocks = (n + 255) / 256;
  if (blocks > 8192) blocks = 8192;
  if (blocks < 1) blocks = 1;
  const dim3 g((unsigned)blocks), t(256);
  switch (dtype) {
    case F32: hipLaunchKernelGGL(rotate_kernel<float>, g, t, 0, (hipStream_t)stream, p); break;
    case F16: hipLaunchKernelGGL(rotate_kernel<_Float16>, g, t, 0, (hipStream_t)stream, p); break;
    default: hipLaunchKernelGGL(rotate_kernel<__bf16>, g, t, 0, (hipStream_t)stream, p); break;
  }
  return (int)hipGetLastError();
}

// grid: (key tiles, query tiles, nb * nh) over the mask's own extents
__global__ __launch_bounds__(256) void classify_kernel(ClassifyParams p) {
  __shared__ unsigned s_bits;
  const int kt = blockIdx.x, qt = blockIdx.y, bh = blockIdx.z;
  const int bm = bh / p.nh, hm = bh % p.nh;
  if (threadIdx.x == 0) s_bits = 0u;
  __syncthreads();
  const int rows = min(kMaskTile, p.Sq - qt * kMaskTile);
  const int keys = min(kMaskTile, p.Sk - kt * kMaskTile);
  unsigned bits = 0u;
  // 64 rows x 64 keys: four threads per row, 16 keys each
  const int row = threadIdx.x >> 2, k0 = (threadIdx.x & 3) * 16;
  if (row < rows && k0 < keys) {
    const uint8_t* src = (const uint8_t*)p.mask.ptr + bm * p.mask.sb + hm * p.mask.sh +
                         (int64_t)(qt * kMaskTile + row) * p.mask.sq + (int64_t)(kt * kMaskTile + k0) * p.mask.sk;
    const int n = min(16, keys - k0);
    for (int e = 0; e < n; ++e) bits |= src[(int64_t)e * p.mask.sk] ? 1u : 2u;
  }
  if (bits) atomicOr(&s_bits, bits);
  __syncthreads();
  if (threadIdx.x == 0) {
    const unsigned st = s_bits;
    p.tiles[((int64_t)bh * gridDim.y + qt) * gridDim.x + kt] = (uint8_t)st;
    if (st & 2u) atomicOr(&p.ctrl[0], 1u);
    __threadfence();
    const unsigned ticket = atomicAdd(&p.ctrl[1], 1u);
    if (ticket == (unsigned)p.total_blocks - 1u) {
      __threadfence();
      const unsigned any_false = atomicOr(&p.ctrl[0], 0u);
      if (!any_false) atomicAdd(&g_all_true_masks, 1ull);
    }
  }
}

int launch_classify(const ClassifyParams& p, void* stream) {
  const int nqt = (p.Sq + kMaskTile - 1) / kMaskTile;
  const int nkt = (p.Sk + kMaskTile - 1) / kMaskTile;
  hipLaunchKernelGGL(classify_kernel, dim3(nkt, nqt, p.nb * p.nh), dim3(256), 0, (hipStream_t)stream, p);
  return (int)hipGetLastError();
}

int read_all_true_counter(uint64_t* value, bool reset) {
  unsigned long long v = 0;
  hipError_t e = hipMemcpyFromSymbol(&v, HIP_SYMBOL(g_all_true_masks), sizeof(v), 0, hipMemcpyDeviceToHost);
  if (e != hipSuccess) return (int)e;
  *value = v;
  if (reset) {
    v = 0;
    e = hipMemcpyToSymbol(HIP_SYMBOL(g_all_true_masks), &v, sizeof(v), 0, hipMemcpyHostToDevice);
  }
  return (int)e;
}

}  // namespace rs
