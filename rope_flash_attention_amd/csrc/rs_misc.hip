// Small preparation kernels that run before attention on the caller's stream:
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
