// Device-side building blocks shared by the forward and backward kernels (gfx950 only).
//
// MFMA fragment conventions (v_mfma_f32_32x32x{16,16,2}): a wave computes a 32 x 32 fp32 block
// C += A B.  Lane l = 32*hh + r feeds row r of A and column r of B with KPL consecutive
// contraction elements starting at hh*KPL (KPL = 8 for bf16/f16, 1 for fp32); a k-step
// therefore covers KSTEP = 2*KPL contraction indices.  Only two facts of the hardware
// layout are relied on: A and B lanes pair their elements on the same contraction index,
// and lane (r, hh) receives C[8*(i/4) + 4*hh + (i%4)][r] in accumulator register i.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "rs_internal.h"

namespace rs {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int i32x16 __attribute__((ext_vector_type(16)));
typedef int i32x4 __attribute__((ext_vector_type(4)));

template <typename T>
struct Mf;

template <>
struct Mf<__bf16> {
  using frag = bf16x8;
  static constexpr int KPL = 8;
  __device__ static inline f32x16 mma(frag a, frag b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
};

template <>
struct Mf<_Float16> {
  using frag = f16x8;
  static constexpr int KPL = 8;
  __device__ static inline f32x16 mma(frag a, frag b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
  }
};

template <>
struct Mf<float> {
  using frag = float;
  static constexpr int KPL = 1;
  __device__ static inline f32x16 mma(frag a, frag b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
  }
};

__device__ inline f32x16 zero16() {
  f32x16 z;
#pragma unroll
  for (int i = 0; i < 16; ++i) z[i] = 0.f;
  return z;
}

__device__ inline i32x16 izero16() {
  i32x16 z;
#pragma unroll
  for (int i = 0; i < 16; ++i) z[i] = 0;
  return z;
}

// Accumulator register i of lane half hh holds row 8*(i/4) + 4*hh + (i%4) of the C block.
__device__ inline int c_row(int i, int hh) { return 8 * (i >> 2) + 4 * hh + (i & 3); }

// Row permutation of 32-row operand blocks held in LDS: swapping bits 2 and 3 makes the
// accumulator rows that one lane holds (after the swap) eight consecutive indices per
// k-step of the following product: register i = 8c + e of lane half hh then refers to
// index 16c + 8hh + e.  The permutation is an involution.
__device__ inline int sig32(int r) { return (r & ~12) | ((r & 4) << 1) | ((r & 8) >> 1); }
__device__ inline int perm_row(int j) { return (j & ~31) | sig32(j & 31); }
// Index (within a 32 block) carried by accumulator register i of lane half hh once the
// A rows were permuted with sig32.
__device__ inline int c_idx_sig(int i, int hh) { return 16 * (i >> 3) + 8 * hh + (i & 7); }

// XOR swizzle of 16-byte units for transposed tiles whose rows are 128 bytes long.
__device__ inline int swz(int row) { return (row ^ (row >> 3)) & 7; }

// XOR swizzle of the 16-byte chunks of row-major V tiles: four consecutive rows put the
// same logical 64-byte column block on four different 64-byte bank ranges.
template <int NCHUNK>
__device__ inline int vsw(int row) { return ((row & 3) << 2) & (NCHUNK - 1); }

// 16 bytes per lane from a buffer straight into LDS: lane i writes [lds + 16i, lds + 16i + 16).
// Bytes outside the buffer's range read as zero.  (Kept out of line of the kernels' lambdas:
// the host compilation pass drops template kernels that use this builtin inside a lambda.)
__device__ inline void buffer_load_lds16(__amdgpu_buffer_rsrc_t rs, char* lds, uint32_t voff, uint32_t soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void*)lds, 16, voff, soff, 0, 0);
}

// Buffer descriptor for one tile of a buffer-loaded operand: base = the tile's first byte,
// range = the bytes of the operand that remain from there.  The per-lane offset then
// covers the whole distance from the base, so every read of the tile is range-checked and
// bytes at or past the operand's end read as zero (the scalar offset stays 0).
// Callers pass workgroup-uniform values only; they are read from the first lane so that the
// descriptor stays in scalar registers even where the compiler cannot prove uniformity
// (it would otherwise loop over the distinct descriptors of the lanes on every load).
__device__ inline __amdgpu_buffer_rsrc_t tile_rsrc(const void* base, int64_t tile_off, int64_t total) {
  const int64_t rem = total - tile_off;
  const int n = __builtin_amdgcn_readfirstlane(rem <= 0 ? 0 : (rem >= 0x7fffffff ? 0x7fffffff : (int)rem));
  const uint64_t a = (uint64_t)((const char*)base + tile_off);
  const uint64_t au = ((uint64_t)__builtin_amdgcn_readfirstlane((uint32_t)(a >> 32)) << 32) |
                      (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)a);
  return __builtin_amdgcn_make_buffer_rsrc((void*)au, (short)0, n, 0x00020000);
}

// Descriptor for the tile of rows row0.. of a row-major operand of nrows rows (stride_bytes
// apart, the last row_bytes long): bytes at or past the operand's end read as zero.  Takes
// 32-bit sizes only, so nothing 64-bit is held in scalar registers between tiles.
__device__ inline __amdgpu_buffer_rsrc_t rows_rsrc(const void* base, int row0, int nrows, int stride_bytes,
                                                   int row_bytes) {
  const int64_t off = (int64_t)row0 * stride_bytes;
  const int64_t total = (int64_t)(nrows - 1) * stride_bytes + row_bytes;
  return tile_rsrc(base, off, total);
}

// Waits for this wave's outstanding memory loads (including loads that write LDS directly)
// and then for every wave of the workgroup.
__device__ inline void wait_vmem_and_sync() {
  __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0), expcnt(7), lgkmcnt(15)
  __syncthreads();
}
// Instruction schedule for a chain of N matrix products fed from LDS, each product
// consuming RPM LDS reads: AHEAD products' worth of reads are issued first, then each
// product is followed by the reads of the product AHEAD places later.  Without it the
// scheduler tends to pair every read with its product and wait out each LDS round trip.
// Must follow the reads and products it orders, in the same basic block; SYNC separates
// independent chains of one block.
template <int N, int RPM, int AHEAD, int SYNC>
__device__ inline void sched_reads_ahead() {
  static_assert(AHEAD >= 1 && AHEAD <= N, "read-ahead depth");
  __builtin_amdgcn_sched_group_barrier(0x100, AHEAD * RPM, SYNC);  // LDS reads
#pragma unroll
  for (int i = 0; i < N - AHEAD; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, SYNC);  // one matrix product
    __builtin_amdgcn_sched_group_barrier(0x100, RPM, SYNC);
  }
  __builtin_amdgcn_sched_group_barrier(0x008, AHEAD, SYNC);
}

// Instruction schedule interleaving a chain of N matrix products fed from LDS (RPM reads
// each; AHEAD products' reads are issued first) with up to VPM vector-ALU instructions after
// each product, so that the wave's own vector work runs in the shadow of its matrix work.
// Same placement rules as sched_reads_ahead.
template <int N, int RPM, int AHEAD, int VPM, int SYNC>
__device__ inline void sched_mfma_interleave() {
  static_assert(AHEAD >= 1 && AHEAD <= N, "read-ahead depth");
  __builtin_amdgcn_sched_group_barrier(0x100, AHEAD * RPM, SYNC);  // LDS reads
#pragma unroll
  for (int i = 0; i < N; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, SYNC);  // one matrix product
    if (i < N - AHEAD) __builtin_amdgcn_sched_group_barrier(0x100, RPM, SYNC);
    __builtin_amdgcn_sched_group_barrier(0x002, VPM, SYNC);  // vector ALU
  }
}

// As sched_mfma_interleave, with the wave's vector-memory loads spread through the chain:
// LEAD of them before the first product, then one after every second product.  (All waves
// issuing a tile's loads at once stall at issue until the load pipeline drains.)
template <int N, int RPM, int AHEAD, int VPM, int LEAD, int SYNC>
__device__ inline void sched_mfma_interleave_loads() {
  static_assert(AHEAD >= 1 && AHEAD <= N, "read-ahead depth");
  __builtin_amdgcn_sched_group_barrier(0x020, LEAD, SYNC);         // vector-memory loads
  __builtin_amdgcn_sched_group_barrier(0x100, AHEAD * RPM, SYNC);  // LDS reads
#pragma unroll
  for (int i = 0; i < N; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, SYNC);  // one matrix product
    if (i < N - AHEAD) __builtin_amdgcn_sched_group_barrier(0x100, RPM, SYNC);
    __builtin_amdgcn_sched_group_barrier(0x002, VPM, SYNC);  // vector ALU
    if (i % 2 == 1) __builtin_amdgcn_sched_group_barrier(0x020, 1, SYNC);
  }
}

// Interleaved-pair rotation with each product and sum rounded to fp32 (no fused
// multiply-add), so that quantized codes computed from it are reproducible exactly.
__device__ inline float2 rot_pair(float x0, float x1, float c, float s) {
#pragma clang fp contract(off)
  float2 r;
  r.x = x0 * c - x1 * s;
  r.y = x0 * s + x1 * c;
  return r;
}

constexpr float kLog2eF = 1.4426950408889634f;
constexpr float kLn2F = 0.6931471805599453f;

// Rotation of one pair with fused multiply-adds: the form the forward uses for Q and K (the
// quantized variants use rot_pair), and the backward with it, so that both round the same
// rotated values.
__device__ inline float2 rot_pair_fma(float x0, float x1, float c, float s) {
  float2 r;
  r.x = fmaf(x0, c, -x1 * s);
  r.y = fmaf(x0, s, x1 * c);
  return r;
}

// Inverse (transposed) rotation of a gradient pair: (g0 c + g1 s, -g0 s + g1 c).
__device__ inline float2 rot_pair_t(float g0, float g1, float c, float s) {
#pragma clang fp contract(off)
  float2 r;
  r.x = g0 * c + g1 * s;
  r.y = g1 * c - g0 * s;
  return r;
}

template <typename T>
__device__ inline float to_f(T x) { return (float)x; }

template <typename T>
__device__ inline T from_f(float x) { return (T)x; }

// Exchange with the lane 32 positions away (the other half of the wave): returns
// (own, partner) combined by the caller.
__device__ inline float xhalf_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ inline float xhalf_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ inline float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Maximum over the 64 lanes of a wave of non-negative, non-NaN floats (whose bit patterns
// order like unsigned integers): four DPP steps within each row of 16 lanes (neighbour pairs,
// pairs of pairs, half-row mirror, row mirror), then the four rows' first lanes through
// scalar registers.  Exact, so the same as any other reduction order.  All lanes active.
__device__ inline float wave_max_nonneg(float v) {
  uint32_t x = __float_as_uint(v);
  x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0xB1, 0xF, 0xF, false));   // quad_perm 1,0,3,2
  x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x4E, 0xF, 0xF, false));   // quad_perm 2,3,0,1
  x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x141, 0xF, 0xF, false));  // row_half_mirror
  x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x140, 0xF, 0xF, false));  // row_mirror
  const uint32_t r0 = (uint32_t)__builtin_amdgcn_readlane((int)x, 0), r1 = (uint32_t)__builtin_amdgcn_readlane((int)x, 16);
  const uint32_t r2 = (uint32_t)__builtin_amdgcn_readlane((int)x, 32), r3 = (uint32_t)__builtin_amdgcn_readlane((int)x, 48);
  return __uint_as_float(max(max(r0, r1), max(r2, r3)));
}

// Blockwise quantizer code of x: round half to even of the fp32 product x * inv, returned in
// the low byte (two's complement) of the result.  Adding 1.5 * 2^23 to the product, with the
// sum rounded to fp32, rounds it to an integer (ties to even) kept in the low mantissa bits;
// valid for |x * inv| < 2^22.  The two operations stay separate (no fused multiply-add):
// the product is rounded first, as the definition says.  Callers have |x| <= amax and
// inv = fp32(QMAX / amax), so the product never leaves [-QMAX, QMAX] after rounding and
// no clamp is needed.
__device__ inline uint32_t quant_bits(float x, float inv) {
#pragma clang fp contract(off)
  const float y = x * inv + 12582912.0f;
  return __float_as_uint(y);
}

// Work-item order for a 1-D grid: consecutive workgroups land on different XCDs (round
// robin over 8), so renumber such that each XCD receives a contiguous range of items and
// neighbouring query tiles of one head share that XCD's L2.
__device__ inline int xcd_remap(int L, int N) {
  const int xcd = L & 7, local = L >> 3;
  const int per = N >> 3, rem = N & 7;
  return xcd * per + (xcd < rem ? xcd : rem) + local;
}

// ---- bool / additive mask access -------------------------------------------------------

// 64 x 64 tile state of a bool mask for query tile qt64 and key tile kt64 of (b, h).
__device__ inline uint8_t mask_tile_state(const MaskView& mv, int b, int h, int qt64, int kt64) {
  const int qi = mv.t_nqt > 1 ? qt64 : 0;
  const int ki = mv.t_nkt > 1 ? kt64 : 0;
  return mv.tiles[b * mv.t_sb + h * mv.t_sh + (int64_t)qi * mv.t_nkt + ki];
}

// Eight consecutive keys j0..j0+7 of query row i: 8 bits, bit e set = attend.  Keys >= S
// read as excluded.  j0 is a multiple of 8.
__device__ inline uint32_t mask_bits8(const MaskView& mv, const uint8_t* row, int j0, int S) {
  if (mv.key_bcast) {
    return row[0] ? 0xffu : 0u;
  }
  uint32_t bits = 0;
  if (j0 + 8 <= S) {
    uint2 w = *(const uint2*)(row + j0);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      bits |= (((w.x >> (8 * e)) & 0xffu) ? 1u : 0u) << e;
      bits |= (((w.y >> (8 * e)) & 0xffu) ? 1u : 0u) << (e + 4);
    }
  } else {
    for (int e = 0; e < 8; ++e)
      if (j0 + e < S && row[j0 + e]) bits |= 1u << e;
  }
  return bits;
}

// Eight consecutive additive mask values (in the mask's dtype) as floats.
template <typename T>
__device__ inline void mask_add8(const MaskView& mv, const char* row, int j0, int S, float* out) {
  if (mv.key_bcast) {
    float v = mv.dtype == F32 ? *(const float*)row : to_f(*(const T*)row);
#pragma unroll
    for (int e = 0; e < 8; ++e) out[e] = v;
    return;
  }
  if (mv.dtype == F32) {
    const float* r = (const float*)row;
    if (j0 + 8 <= S) {
      float4 a = *(const float4*)(r + j0), c = *(const float4*)(r + j0 + 4);
      out[0] = a.x; out[1] = a.y; out[2] = a.z; out[3] = a.w;
      out[4] = c.x; out[5] = c.y; out[6] = c.z; out[7] = c.w;
    } else {
      for (int e = 0; e < 8; ++e) out[e] = (j0 + e < S) ? r[j0 + e] : 0.f;
    }
  } else {
    const T* r = (const T*)row;
    if (j0 + 8 <= S) {
      typedef T v8 __attribute__((ext_vector_type(8)));
      v8 a = *(const v8*)(r + j0);
#pragma unroll
      for (int e = 0; e < 8; ++e) out[e] = to_f(a[e]);
    } else {
      for (int e = 0; e < 8; ++e) out[e] = (j0 + e < S) ? to_f(r[j0 + e]) : 0.f;
    }
  }
}

__device__ inline const char* mask_row_ptr(const MaskView& mv, int b, int h, int i, int elem) {
  return (const char*)mv.ptr + (b * mv.sb + h * mv.sh + (int64_t)i * mv.sq) * elem;
}

}  // namespace rs
