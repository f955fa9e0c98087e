// Backward kernels for 16-bit inputs at D = 128 on 16x16x32 MFMA.
//
// Same mathematics as rs_bwd.hip (page "Metal Flash Attention", section "Fused RoPE +
// SDPA": gradients with respect to the pre-rotation Q and K through the inverse rotation):
//    P = exp2(S' - LSE log2 e) with S' = scale log2(e) Q'K'^T,  dP = dO V^T,
//    dS = P o (dP - delta),  dV = P^T dO,  dK = R^T (scale dS^T Q'),  dQ = R^T (scale dS K').
//
// The 16x16 products keep a wave's accumulators small (a 16 x 128 block is 32 registers
// instead of 64 for 32 rows), so eight waves of one workgroup fit two per SIMD:
//  * dq16:   workgroup = 128 queries (16 per wave, one per lane column); Q' (times
//            scale log2 e) and dO stay in registers as B operands; K' (rotated once by
//            kprep_kernel) and V tiles go straight from memory into LDS, two 64-key tiles per
//            barrier; per 64-key tile S'^T = K' Q'^T, dP^T = V dO^T (row reads),
//            dQ'^T += K'^T dS^T (transposed reads).  Launched first: it also writes its rows
//            of Q' (times scale log2 e, rounded to the input dtype as the forward rounds them)
//            and their delta = sum_d dO O to the workspace for dkdv16.
// Both recompute the scores from the forward's rounded operands (Q' scale log2 e, K'), so
// that P matches the forward's row log-sum-exp.
//  * dkdv16: workgroup = 128 keys (16 per wave); K' and V stay in registers; Q' (times
//            scale log2 e, from dq16) and dO tiles of 64 queries go straight from memory
//            into LDS; per tile S' = Q' K'^T, dP = dO V^T, dV^T += dO^T P, dK'^T += Q'^T dS;
//            waves 0-3 and 4-7 work half a tile apart (three LDS buffers per operand, one
//            barrier per tile, see the kernel).
// The score rows are read in a permuted order so that the four accumulator rows a lane holds
// in two consecutive 16-row blocks are eight consecutive contraction indices of the next
// product: P and dS go from accumulators to B operands without leaving registers.
// LDS tiles are 64 rows of 256 bytes with 16-byte chunks XOR-swizzled per row so that both
// the row reads (16 lanes x 16 bytes) and the transposed reads (32 lanes x 8 bytes) touch
// distinct banks.  Deterministic: no atomics.
#include "rs_device.hpp"

namespace rs {

namespace {

constexpr float kL2e = 1.4426950408889634f;
constexpr int kMaxStateTiles16 = kMaxBoolMaskSeq / 64;  // 64-row tiles of a bool-masked call

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));

template <typename T>
struct M16;
template <>
struct M16<__bf16> {
  __device__ static inline f32x4 mma(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
};
template <>
struct M16<_Float16> {
  __device__ static inline f32x4 mma(f16x8 a, f16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
  }
};

// Swizzle of 256-byte LDS rows: logical 16-byte chunk ch of row r sits at ch ^ msk16(r).
// Row bits 0-1 go to mask bits 1-2, bit 3 to mask bit 0, bit 3 xor bit 4 to mask bit 3:
// the row reads (rows r0 + {0..3, 8..11, 16..19, 24..27}) and the transposed reads (four
// consecutive rows, two 16-lane groups eight rows apart) then hit distinct banks whether a
// pass serves 128 or 256 bytes.
__device__ inline int msk16(int row) {
  return ((row & 3) << 1) | ((row >> 3) & 1) | ((((row >> 3) ^ (row >> 4)) & 1) << 3);
}
__device__ inline int lds_off(int row, int byte) { return row * 256 + (((byte >> 4) ^ msk16(row)) << 4) + (byte & 15); }

// Row of a 64-row tile that lane row rho of 16-row block kb reads.  With this order the
// accumulator rows 4g..4g+3 of blocks 2s and 2s+1 are tile rows 32s + 8g + 0..7.
__device__ inline int blk_row(int kb, int rho) { return 32 * (kb >> 1) + 8 * (rho >> 2) + 4 * (kb & 1) + (rho & 3); }

// Per-lane LDS byte offsets of the two access patterns.  The swizzle only depends on row
// bits 0, 1, 3 and 4, which the lane fixes; block and k-step terms are plain additions,
// so one register per pattern serves every block and buffer.
//  * row reads: lane (c, g) reads 16 bytes of row blk_row(kb, c) at column 64t + 16g:
//      offset = row_rd[t] + 256 (32 (kb >> 1) + 4 (kb & 1));
//  * transposed reads: rows r0 + 4h + (c >> 2) (r0 = 32s + 8g), 8 bytes at column
//    16db + 4(c & 3) (16-bit elements): offset = tr_rd[db] + 256 (32 s + 4 h).
struct LaneOffsets {
  int row_rd[4];
  int tr_rd[8];
  __device__ void init(int c, int g) {
    const int rl = 8 * (c >> 2) + (c & 3);
#pragma unroll
    for (int t = 0; t < 4; ++t) row_rd[t] = lds_off(rl, 64 * t + 16 * g);
    const int rt = 8 * g + (c >> 2);
#pragma unroll
    for (int db = 0; db < 8; ++db) tr_rd[db] = lds_off(rt, 2 * (16 * db + 4 * (c & 3)));
  }
};
__device__ inline int blk_off(int kb) { return 256 * (32 * (kb >> 1) + 4 * (kb & 1)); }

// A fragment of a transposed operand: element e = tile[32s + 8g + e][16db + c] (16-bit
// elements), from two transposed 8-byte reads per lane.
template <typename F>
__device__ inline F tr_frag(const char* tile, const LaneOffsets& lo_, int s, int db) {
  const char* a = tile + lo_.tr_rd[db] + 256 * 32 * s;
  const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)a);
  const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(a + 256 * 4));
  F f;
  *(s16x4*)&f = lo;
  *((s16x4*)&f + 1) = hi;
  return f;
}

// B fragments of one row (D = 128): element e of fragment t = row[32t + 8g + e]; kRowMul:
// multiplied by `mul` (a row rotated already); kRowRaw: as stored.
constexpr int kRowRaw = 0, kRowMul = 2;
template <typename T, int MODE>
__device__ inline void row_frags(typename Mf<T>::frag* f, const T* row, int g, float mul) {
  typedef T v8 __attribute__((ext_vector_type(8)));
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const int d0 = 32 * t + 8 * g;
    v8 x = *(const v8*)(row + d0);
    if constexpr (MODE == kRowMul) {
#pragma unroll
      for (int e = 0; e < 8; ++e) x[e] = from_f<T>(to_f(x[e]) * mul);
    }
    f[t] = x;
  }
}

// B fragments of a Q row rotated with its packed table row and multiplied by `mul` (the
// forward's Q' scale log2 e, rounded once to the input dtype as the forward rounds it), also
// written to `dst` unless it is null: the dQ kernel writes these rows for the dK/dV kernel,
// whose scores then use the forward's rounded operands too.
// Every load is issued before the first store (a store in between would make the compiler
// issue the later loads again, one round trip each).
template <typename T>
__device__ inline void row_frags_qrot(typename Mf<T>::frag* f, T* dst, const T* row, const float* trow, int g,
                                      float mul) {
  typedef T v8 __attribute__((ext_vector_type(8)));
  v8 x[4];
  float4 ta[4], tb[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const int d0 = 32 * t + 8 * g;
    x[t] = *(const v8*)(row + d0);
    ta[t] = *(const float4*)(trow + d0);
    tb[t] = *(const float4*)(trow + d0 + 4);
  }
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const float cc[4] = {ta[t].x, ta[t].z, tb[t].x, tb[t].z}, ss[4] = {ta[t].y, ta[t].w, tb[t].y, tb[t].w};
    v8 y;
#pragma unroll
    for (int pp = 0; pp < 4; ++pp) {
      const float2 r = rot_pair_fma(to_f(x[t][2 * pp]), to_f(x[t][2 * pp + 1]), cc[pp], ss[pp]);
      y[2 * pp] = from_f<T>(r.x * mul);
      y[2 * pp + 1] = from_f<T>(r.y * mul);
    }
    f[t] = y;
    if (dst) *(v8*)(dst + 32 * t + 8 * g) = y;
  }
}

// Direct-to-LDS loads of a 64-row tile of a [*, 128] 16-bit operand (rows past the end of
// the slice read as zero): each wave issues two 1 KB loads.
struct DmaTile {
  const void* base;
  int64_t total;  // bytes of the (b, h) slice
  uint32_t voff[2];
  uint32_t row_bytes;
  __device__ void init(const void* base_, int64_t ss, int S, int wave, int lane) {
    base = base_;
    total = ((int64_t)(S - 1) * ss + 128) * 2;
    row_bytes = (uint32_t)(ss * 2);
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int byte = (wave * 2 + i) * 1024 + lane * 16;
      const int row = byte >> 8, pch = (byte & 255) >> 4;
      voff[i] = (uint32_t)(row * (int)row_bytes + ((pch ^ msk16(row)) << 4));
    }
  }
  __device__ void issue(char* tile, int row0, int wave) {
    const __amdgpu_buffer_rsrc_t rs = tile_rsrc(base, (int64_t)row0 * row_bytes, total);
#pragma unroll
    for (int i = 0; i < 2; ++i) buffer_load_lds16(rs, tile + (wave * 2 + i) * 1024, voff[i], 0);
  }
};

}  // namespace

// ---------------------------------------------------------------------------------------
// K arrives rotated (K' in the workspace, contiguous): its tiles go straight from memory
// into LDS like V's, with no table in the key loop.  QROT: Q arrives rotated too (Q' in the
// workspace, the dequantized values of the quantized forward): it is only scaled, and not
// written back.
// Without causal masking a step runs two 64-key tiles (NT) between barriers: the LDS buffers
// hold both, and the next step's pair streams into the other buffers meanwhile (FLUX B=2
// backward 1.3% faster; the causal kernel's short key ranges run one tile per step, which
// measured faster there).
template <typename T, int MASK, bool CAUSAL, bool QROT>
__global__ __launch_bounds__(512, 1) void dq16_kernel(BwdParams p) {
  using frag = typename Mf<T>::frag;
  using M = M16<T>;
  constexpr int D = 128, BM = 128, BN = 64, TILE = BN * 256, NT = CAUSAL ? 1 : 2;
  __shared__ __attribute__((aligned(16))) char sk0[NT * TILE];
  __shared__ __attribute__((aligned(16))) char sk1[NT * TILE];
  __shared__ __attribute__((aligned(16))) char sv0[NT * TILE];
  __shared__ __attribute__((aligned(16))) char sv1[NT * TILE];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int c = lane & 15, g = lane >> 4;
  const int S = p.shp.S;
  const int nqt = (S + BM - 1) / BM;
  // causal: workgroup w runs two query tiles of one head, the longest (nqt - 1 - i) and the
  // shortest (i), so that every workgroup has the same number of key tiles whatever order
  // the workgroups are placed on the CUs in
  const int npairs = (nqt + 1) / 2;
  const int itemw = xcd_remap(blockIdx.x, gridDim.x);
#pragma unroll 1
  for (int pu = 0; pu < (CAUSAL ? 2 : 1); ++pu) {
  const int ip = CAUSAL ? itemw % npairs : 0;
  if (CAUSAL && pu == 1 && ip == nqt - 1 - ip) break;
  const int qt = CAUSAL ? (pu == 0 ? nqt - 1 - ip : ip) : itemw % nqt;
  const int bh = CAUSAL ? itemw / npairs : itemw / nqt;
  const int hd = bh % p.shp.H, b = bh / p.shp.H;
  if (pu > 0) __syncthreads();  // LDS of the previous tile
  const int q0 = qt * BM;
  const int m = q0 + 16 * wave + c;
  const int mc = m < S ? m : S - 1;

  const int hk = hd / p.shp.group;  // K/V head (grouped-query attention)
  const T* kbase = (const T*)p.k.ptr + b * p.k.sb + hk * p.k.sh;
  const T* vbase = (const T*)p.v.ptr + b * p.v.sb + hk * p.v.sh;
  const float* tab = p.tab.ptr + b * p.tab.sb;

  frag qf[4], gf[4];
  if constexpr (QROT) {
    row_frags<T, kRowMul>(qf, (const T*)p.qrot + ((int64_t)bh * S + mc) * D, g, p.shp.scale_log2);
  } else {
    row_frags_qrot<T>(qf, m < S ? (T*)p.qrot + ((int64_t)bh * S + m) * D : nullptr,
                      (const T*)p.q.ptr + b * p.q.sb + hd * p.q.sh + (int64_t)mc * p.q.ss, tab + (int64_t)mc * D, g,
                      p.shp.scale_log2);
  }
  row_frags<T, kRowRaw>(gf, (const T*)p.dout.ptr + b * p.dout.sb + hd * p.dout.sh + (int64_t)mc * p.dout.ss, g,
                        1.f);
  const int64_t rowid = ((int64_t)b * p.shp.H + hd) * S + mc;
  const float lse_v = p.lse[rowid];
  const float l2 = (m >= S || lse_v == -INFINITY) ? INFINITY : lse_v * kL2e;
  // delta = sum_d dO O of the row in fp32: this lane's 32 elements, then the four lanes of the
  // row (c, c + 16, c + 32, c + 48); written to the workspace for the dK/dV kernel
  float dlt = 0.f;
  {
    typedef T v8 __attribute__((ext_vector_type(8)));
    const T* orow = (const T*)p.o.ptr + b * p.o.sb + hd * p.o.sh + (int64_t)mc * p.o.ss;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const v8 ov = *(const v8*)(orow + 32 * t + 8 * g);
#pragma unroll
      for (int e = 0; e < 8; ++e) dlt = fmaf(to_f(ov[e]), to_f(gf[t][e]), dlt);
    }
    dlt += __shfl_xor(dlt, 16, 64);
    dlt += __shfl_xor(dlt, 32, 64);
    if (g == 0 && m < S) p.delta[rowid] = dlt;
  }
  const f32x4 cinit = {-l2, -l2, -l2, -l2};  // S'^T - LSE log2 e through the accumulator
  const f32x4 z4 = {0.f, 0.f, 0.f, 0.f};

  f32x4 dq[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) dq[i] = z4;

  const int nkt = (S + BN - 1) / BN;
  int kt_end = nkt;
  if (CAUSAL) kt_end = min(nkt, (min(q0 + BM, S) - 1) / BN + 1);
  auto tile_state_mem = [&](int kt) -> uint32_t {
    const int bm = p.mask.t_sb ? b : 0, hm = p.mask.t_sh ? hd : 0;
    uint32_t st = mask_tile_state(p.mask, bm, hm, 2 * qt, kt);
    if (2 * qt + 1 < (S + kMaskTile - 1) / kMaskTile) st |= mask_tile_state(p.mask, bm, hm, 2 * qt + 1, kt);
    return st;
  };
  // tile states gathered once into LDS (see the forward kernel)
  __shared__ uint8_t s_tstate[MASK == MASK_BOOL ? kMaxStateTiles16 : 1];
  if constexpr (MASK == MASK_BOOL) {
    for (int i = tid; i < kt_end; i += 512) s_tstate[i] = (uint8_t)tile_state_mem(i);
    __syncthreads();
  }
  auto tile_state = [&](int kt) -> uint32_t {
    if constexpr (MASK == MASK_BOOL) {
      return (uint32_t)s_tstate[kt];
    } else {
      return TILE_MIXED;
    }
  };
  auto next_tile = [&](int kt) -> int {
    if constexpr (MASK == MASK_BOOL) {
      while (kt < kt_end && tile_state(kt) == TILE_ALL_FALSE) ++kt;
    }
    return kt;
  };

  LaneOffsets lo;
  lo.init(c, g);
  DmaTile dkt, dv;  // K' and V tiles
  dkt.init(kbase, p.k.ss, S, wave, lane);
  dv.init(vbase, p.v.ss, S, wave, lane);
  const int bm = p.mask.sb ? b : 0, hm = p.mask.sh ? hd : 0;
  // the tiles of one step (kt_end where the step has fewer) into buffers sK, sV
  auto issue = [&](int ka, int kb2, char* sKd, char* sVd) {
    if (ka < kt_end) {
      dkt.issue(sKd, ka * BN, wave);
      dv.issue(sVd, ka * BN, wave);
    }
    if (NT == 2 && kb2 < kt_end) {
      dkt.issue(sKd + TILE, kb2 * BN, wave);
      dv.issue(sVd + TILE, kb2 * BN, wave);
    }
  };

  // one 64-key tile kt from LDS tiles sK, sV
  auto tile = [&](int kt, const char* sK, const char* sV) __attribute__((always_inline)) {
    const int kv0 = kt * BN;

    // S'^T - l2 and dP^T: rows = keys (permuted order), column = this lane's query
    f32x4 sacc[4], dpacc[4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      frag ka[4], va[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) ka[t] = *(const frag*)(sK + lo.row_rd[t] + blk_off(kb));
#pragma unroll
      for (int t = 0; t < 4; ++t) va[t] = *(const frag*)(sV + lo.row_rd[t] + blk_off(kb));
#pragma unroll
      for (int t = 0; t < 4; ++t) sacc[kb] = M::mma(ka[t], qf[t], t == 0 ? cinit : sacc[kb]);
#pragma unroll
      for (int t = 0; t < 4; ++t) dpacc[kb] = M::mma(va[t], gf[t], t == 0 ? z4 : dpacc[kb]);
    }
    sched_reads_ahead<32, 1, 12, 0>();

    // exclusions (keys past the end, causal, masks), P and dS
    if constexpr (MASK == MASK_ADD) {
      const int esz = p.mask.dtype == F32 ? 4 : 2;
      const char* mrow = mask_row_ptr(p.mask, bm, hm, p.mask.sq ? mc : 0, esz);
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        float mv[8];
        mask_add8<T>(p.mask, mrow, kv0 + 32 * half + 8 * g, S, mv);
#pragma unroll
        for (int e = 0; e < 8; ++e) sacc[2 * half + (e >> 2)][e & 3] = fmaf(mv[e], kL2e, sacc[2 * half + (e >> 2)][e & 3]);
      }
    }
    uint32_t st = TILE_ALL_TRUE;
    if constexpr (MASK == MASK_BOOL) st = tile_state(kt);
    const bool check = kv0 + BN > S || (CAUSAL && kv0 + BN - 1 > q0) || (MASK == MASK_BOOL && st != TILE_ALL_TRUE);
    uint32_t bits[2] = {0xffu, 0xffu};
    if (check) {
      if constexpr (MASK == MASK_BOOL) {
        if (st != TILE_ALL_TRUE) {
          const uint8_t* brow = (const uint8_t*)mask_row_ptr(p.mask, bm, hm, p.mask.sq ? mc : 0, 1);
          bits[0] = mask_bits8(p.mask, brow, kv0 + 8 * g, S);
          bits[1] = mask_bits8(p.mask, brow, kv0 + 32 + 8 * g, S);
        }
      }
    }
    frag dsf[2];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float pv = fast_exp2(sacc[kb][i]);
        if (check) {
          const int e = 4 * (kb & 1) + i;  // key = kv0 + 32 (kb >> 1) + 8 g + e
          const int j = kv0 + 32 * (kb >> 1) + 8 * g + e;
          bool ok = j < S && ((bits[kb >> 1] >> e) & 1u);
          if (CAUSAL) ok = ok && j <= m;
          if (!ok) pv = 0.f;
        }
        dsf[kb >> 1][4 * (kb & 1) + i] = from_f<T>(pv * (dpacc[kb][i] - dlt));
      }

    // dQ'^T += K'^T dS^T: rows = head dim, column = this lane's query
#pragma unroll
    for (int db = 0; db < 8; ++db)
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) dq[db] = M::mma(tr_frag<frag>(sK, lo, ks, db), dsf[ks], dq[db]);
    sched_reads_ahead<16, 2, 3, 1>();
  };

  // step: tiles kt and kt2 (kt2 = kt_end when the step has one)
  int kt = next_tile(0);
  int kt2 = NT == 2 && kt < kt_end ? next_tile(kt + 1) : kt_end;
  issue(kt, kt2, sk0, sv0);
  wait_vmem_and_sync();

  auto body = [&](auto stage_c) {
    constexpr int stage = decltype(stage_c)::value;
    const char* sK = stage ? sk1 : sk0;
    const char* sV = stage ? sv1 : sv0;
    const int ktn = next_tile((kt2 < kt_end ? kt2 : kt) + 1);
    const int ktn2 = NT == 2 && ktn < kt_end ? next_tile(ktn + 1) : kt_end;
    issue(ktn, ktn2, stage ? sk0 : sk1, stage ? sv0 : sv1);
    tile(kt, sK, sV);
    if (NT == 2 && kt2 < kt_end) tile(kt2, sK + TILE, sV + TILE);
    wait_vmem_and_sync();
    kt = ktn;
    kt2 = ktn2;
  };
  while (kt < kt_end) {
    body(std::integral_constant<int, 0>{});
    if (kt >= kt_end) break;
    body(std::integral_constant<int, 1>{});
  }

  // dQ = R^T (scale dQ'): lane holds d = 16 db + 4 g + i of its query row
  if (m < S) {
    char* orow = (char*)p.dq + ((int64_t)b * p.dq_sb + (int64_t)hd * p.dq_sh + (int64_t)m * p.dq_ss) * 2;
    const float* trow = tab + (int64_t)m * D;
#pragma unroll
    for (int db = 0; db < 8; ++db) {
      const int d0 = 16 * db + 4 * g;
      const float4 cs = *(const float4*)(trow + d0);  // pairs d0/2, d0/2 + 1
      const float sc = p.shp.scale;
      const float2 a = rot_pair_t(dq[db][0] * sc, dq[db][1] * sc, cs.x, cs.y);
      const float2 e = rot_pair_t(dq[db][2] * sc, dq[db][3] * sc, cs.z, cs.w);
      typedef T v4 __attribute__((ext_vector_type(4)));
      v4 w;
      w[0] = from_f<T>(a.x);
      w[1] = from_f<T>(a.y);
      w[2] = from_f<T>(e.x);
      w[3] = from_f<T>(e.y);
      *(v4*)(orow + d0 * 2) = w;
    }
  }
  }
}

// ---------------------------------------------------------------------------------------
// K arrives rotated (K' in the workspace).  QS: the Q' tiles (from the dQ kernel) carry the
// forward's factor scale log2 e, so the scores are the forward's products of its rounded
// operands and K' is used as it is; dK' then carries log2 e, taken out with ln 2 at the end.
// Otherwise (the quantized backward's dequantized Q') K' is scaled here.
template <typename T, int MASK, bool CAUSAL, bool QS>
__global__ __launch_bounds__(512, 1) void dkdv16_kernel(BwdParams p) {
  using frag = typename Mf<T>::frag;
  using M = M16<T>;
  constexpr int D = 128, BNK = 128, BMQ = 64, TILE = BMQ * 256;
  // three buffers of each: tile i uses buffer i % 3 (see the step loop)
  __shared__ __attribute__((aligned(16))) char sq0[TILE];
  __shared__ __attribute__((aligned(16))) char sq1[TILE];
  __shared__ __attribute__((aligned(16))) char sq2[TILE];
  __shared__ __attribute__((aligned(16))) char sd0[TILE];
  __shared__ __attribute__((aligned(16))) char sd1[TILE];
  __shared__ __attribute__((aligned(16))) char sd2[TILE];
  __shared__ __attribute__((aligned(16))) float sl0[2 * BMQ];  // l2 then delta per query
  __shared__ __attribute__((aligned(16))) float sl1[2 * BMQ];
  __shared__ __attribute__((aligned(16))) float sl2[2 * BMQ];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int c = lane & 15, g = lane >> 4;
  const int S = p.shp.S;
  const int nkt = (S + BNK - 1) / BNK;
  // workgroup = one key tile of one (b, K/V head); with grouped-query attention it runs the
  // query tiles of every query head of the group, dK and dV accumulating across them
  const int item = xcd_remap(blockIdx.x, gridDim.x);
  // causal: workgroup runs key tiles ip and nkt - 1 - ip of one slice (nqt - 2 ip and
  // 2 ip + 2 query tiles: the same total in every workgroup)
  const int npairs = (nkt + 1) / 2;
  const int bh = CAUSAL ? item / npairs : item / nkt;
  const int ip = CAUSAL ? item % npairs : item % nkt;
  const int hk = bh % p.shp.Hkv, b = bh / p.shp.Hkv;
#pragma unroll 1
  for (int pu = 0; pu < (CAUSAL ? 2 : 1); ++pu) {
  if (CAUSAL && pu == 1 && ip == nkt - 1 - ip) break;
  if (pu > 0) __syncthreads();  // LDS of the first key tile
  const int kt = CAUSAL && pu == 1 ? nkt - 1 - ip : ip;
  const int k0 = kt * BNK;
  const int j = k0 + 16 * wave + c;  // this lane's key
  const int jc = j < S ? j : S - 1;

  const float* tab = p.tab.ptr + b * p.tab.sb;
  int hd = 0;  // the query head whose tiles are being run
  const T* dobase = nullptr;
  const float* lse = nullptr;
  const float* dlt = nullptr;

  // K' (times scale log2 e unless the Q' tiles carry it) and V of this lane's key as B fragments
  frag kf[4], vf[4];
  row_frags<T, QS ? kRowRaw : kRowMul>(kf, (const T*)p.k.ptr + b * p.k.sb + hk * p.k.sh + (int64_t)jc * p.k.ss, g,
                                       p.shp.scale_log2);
  row_frags<T, kRowRaw>(vf, (const T*)p.v.ptr + b * p.v.sb + hk * p.v.sh + (int64_t)jc * p.v.ss, g, 1.f);
  const f32x4 z4 = {0.f, 0.f, 0.f, 0.f};
  f32x4 dv[8], dk[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    dv[i] = z4;
    dk[i] = z4;
  }

  const int nqt = (S + BMQ - 1) / BMQ;
  const int qt_begin = CAUSAL ? k0 / BMQ : 0;
  auto tile_state_mem = [&](int qt) -> uint32_t {
    const int bm = p.mask.t_sb ? b : 0, hm = p.mask.t_sh ? hd : 0;
    const int nk64 = (S + kMaskTile - 1) / kMaskTile;
    uint32_t st = mask_tile_state(p.mask, bm, hm, qt, 2 * kt);
    if (2 * kt + 1 < nk64) st |= mask_tile_state(p.mask, bm, hm, qt, 2 * kt + 1);
    return st;
  };
  __shared__ uint8_t s_tstate[MASK == MASK_BOOL ? kMaxStateTiles16 : 1];
  auto tile_state = [&](int qt) -> uint32_t {
    if constexpr (MASK == MASK_BOOL) {
      return (uint32_t)s_tstate[qt];
    } else {
      return TILE_MIXED;
    }
  };
  auto next_tile = [&](int qt) -> int {
    if constexpr (MASK == MASK_BOOL) {
      while (qt < nqt && tile_state(qt) == TILE_ALL_FALSE) ++qt;
    }
    return qt;
  };

  LaneOffsets lo;
  lo.init(c, g);
  DmaTile dqr;  // Q' tiles, rotated by the dQ kernel (launched first)
  DmaTile dd;
  float lreg = 0.f;  // thread t < 64: l2 of query q0 + t; 64 <= t < 128: delta of q0 + t - 64
  auto load_tile = [&](int qt, char* sQ, char* sD) {
    const int q0 = qt * BMQ;
    dqr.issue(sQ, q0, wave);
    dd.issue(sD, q0, wave);
    if (tid < 2 * BMQ) {
      const int i = q0 + (tid & (BMQ - 1));
      if (tid < BMQ) {
        const float lv = i < S ? lse[i] : -INFINITY;
        lreg = lv == -INFINITY ? INFINITY : lv * kL2e;  // +inf makes P = 0 for empty rows
      } else {
        lreg = i < S ? dlt[i] : 0.f;
      }
    }
  };
  auto store_tile = [&](float* sL) {
    if (tid < 2 * BMQ) sL[tid] = lreg;
  };
  const int bm = p.mask.sb ? b : 0;
  int hm = 0;

  // S' and dP of one query tile: rows = queries (permuted order), column = this lane's key
  auto rows = [&](const char* sQ, const char* sD, f32x4* sacc, f32x4* dpacc) __attribute__((always_inline)) {
#pragma unroll
    for (int qb = 0; qb < 4; ++qb) {
      frag qa[4], ga[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) qa[t] = *(const frag*)(sQ + lo.row_rd[t] + blk_off(qb));
#pragma unroll
      for (int t = 0; t < 4; ++t) ga[t] = *(const frag*)(sD + lo.row_rd[t] + blk_off(qb));
#pragma unroll
      for (int t = 0; t < 4; ++t) sacc[qb] = M::mma(qa[t], kf[t], t == 0 ? z4 : sacc[qb]);
#pragma unroll
      for (int t = 0; t < 4; ++t) dpacc[qb] = M::mma(ga[t], vf[t], t == 0 ? z4 : dpacc[qb]);
    }
    sched_reads_ahead<32, 1, 16, 0>();
  };
  // P and dS of query tile qt (l2 and delta in sL) as B fragments
  auto softmax = [&](int qt, const float* sL, f32x4* sacc, f32x4* dpacc, frag* pf_out, frag* sf_out)
                     __attribute__((always_inline)) {
    const int q0 = qt * BMQ;
    frag pf[2], sf[2];  // built from scratch: every element is written
    // accumulator row 4g + i of block qb is query q0 + 32 (qb >> 1) + 8 g + 4 (qb & 1) + i
    if constexpr (MASK == MASK_ADD) {
      const int jj = p.mask.key_bcast ? 0 : jc;
#pragma unroll
      for (int qb = 0; qb < 4; ++qb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int qi = min(q0 + 32 * (qb >> 1) + 8 * g + 4 * (qb & 1) + i, S - 1);
          float mvv;
          if (p.mask.dtype == F32)
            mvv = ((const float*)mask_row_ptr(p.mask, bm, hm, p.mask.sq ? qi : 0, 4))[jj];
          else
            mvv = to_f(((const T*)mask_row_ptr(p.mask, bm, hm, p.mask.sq ? qi : 0, 2))[jj]);
          sacc[qb][i] = fmaf(mvv, kL2e, sacc[qb][i]);
        }
    }
    uint32_t st = TILE_ALL_TRUE;
    if constexpr (MASK == MASK_BOOL) st = tile_state(qt);
    const bool check = (CAUSAL && q0 < k0 + BNK - 1) || (MASK == MASK_BOOL && st != TILE_ALL_TRUE);
#pragma unroll
    for (int qb = 0; qb < 4; ++qb) {
      const int r0 = 32 * (qb >> 1) + 8 * g + 4 * (qb & 1);  // tile-local query of register 0
      const float4 lv = *(const float4*)(sL + r0);
      const float4 dl = *(const float4*)(sL + BMQ + r0);
      const float l4[4] = {lv.x, lv.y, lv.z, lv.w}, d4[4] = {dl.x, dl.y, dl.z, dl.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float pv = fast_exp2(sacc[qb][i] - l4[i]);
        if (check) {
          const int qi = q0 + r0 + i;
          bool ok = true;
          if (CAUSAL) ok = j <= qi;
          if constexpr (MASK == MASK_BOOL) {
            if (st != TILE_ALL_TRUE && ok && qi < S) {
              const uint8_t* brow = (const uint8_t*)mask_row_ptr(p.mask, bm, hm, p.mask.sq ? qi : 0, 1);
              ok = brow[p.mask.key_bcast ? 0 : jc] != 0;
            }
          }
          if (!ok) pv = 0.f;
        }
        pf[qb >> 1][4 * (qb & 1) + i] = from_f<T>(pv);
        sf[qb >> 1][4 * (qb & 1) + i] = from_f<T>(pv * (dpacc[qb][i] - d4[i]));
      }
    }
    // computed here: left alone, the compiler sinks this arithmetic to the products that
    // use it (after the barrier), which keeps the fp32 scores alive instead
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      i32x4 w = __builtin_bit_cast(i32x4, pf[h]);
      asm volatile("" : "+v"(w));
      pf_out[h] = __builtin_bit_cast(frag, w);
      w = __builtin_bit_cast(i32x4, sf[h]);
      asm volatile("" : "+v"(w));
      sf_out[h] = __builtin_bit_cast(frag, w);
    }
  };
  // dV^T += dO^T P, dK'^T += Q'^T dS: rows = head dim, column = this lane's key
  auto cols = [&](const char* sQ, const char* sD, const frag* pf, const frag* sf) __attribute__((always_inline)) {
#pragma unroll
    for (int db = 0; db < 8; ++db)
#pragma unroll
      for (int qs = 0; qs < 2; ++qs) {
        dv[db] = M::mma(tr_frag<frag>(sD, lo, qs, db), pf[qs], dv[db]);
        dk[db] = M::mma(tr_frag<frag>(sQ, lo, qs, db), sf[qs], dk[db]);
      }
    sched_reads_ahead<32, 2, 3, 1>();
  };

  // The two waves of a SIMD work half a tile apart: in the step of tile i, waves 0-3 take the
  // tile's scores (row reads) and then its gradient products (transposed reads); waves 4-7
  // first finish the previous tile's gradient products (its P and dS kept in registers),
  // then take this tile's scores.  Each half of a step then has one wave per SIMD on each
  // kind of product, and the LDS serves both kinds of reads at once.  Tile i sits in buffer
  // i % 3: the step of tile i reads buffers i % 3 and (waves 4-7) (i - 1) % 3, and loads tile
  // i + 1 into buffer (i + 1) % 3 from its start, the buffer of tile i - 2, which the previous
  // step finished with: one barrier per step.  The two wave groups run separate loops (one
  // branch outside), so that neither carries the other's registers.
#pragma unroll 1
  for (int gq = 0; gq < p.shp.group; ++gq) {
  hd = hk * p.shp.group + gq;
  dobase = (const T*)p.dout.ptr + b * p.dout.sb + hd * p.dout.sh;
  lse = p.lse + ((int64_t)b * p.shp.H + hd) * S;
  dlt = p.delta + ((int64_t)b * p.shp.H + hd) * S;
  hm = p.mask.sh ? hd : 0;
  dqr.init((const T*)p.qrot + ((int64_t)b * p.shp.H + hd) * S * D, D, S, wave, lane);
  dd.init(dobase, p.dout.ss, S, wave, lane);
  if (gq > 0) __syncthreads();  // LDS of the previous head's last tile and tile states
  if constexpr (MASK == MASK_BOOL) {
    for (int i = tid; i < nqt; i += 512) s_tstate[i] = (uint8_t)tile_state_mem(i);
    __syncthreads();
  }
  int qt = next_tile(qt_begin);
  if (qt < nqt) {
    load_tile(qt, sq0, sd0);
    store_tile(sl0);
  }
  wait_vmem_and_sync();
  frag pf[2], sf[2];
  auto bufq = [&](int k) -> char* { return k == 0 ? sq0 : (k == 1 ? sq1 : sq2); };
  auto bufd = [&](int k) -> char* { return k == 0 ? sd0 : (k == 1 ? sd1 : sd2); };
  auto bufl = [&](int k) -> float* { return k == 0 ? sl0 : (k == 1 ? sl1 : sl2); };
  if (__builtin_amdgcn_readfirstlane(wave) < 4) {
    auto body = [&](auto stage_c) __attribute__((always_inline)) {
      constexpr int st = decltype(stage_c)::value;
      char* sQ = bufq(st);
      char* sD = bufd(st);
      float* sL = bufl(st);
      const int qtn = next_tile(qt + 1);
      f32x4 sacc[4], dpacc[4];
      rows(sQ, sD, sacc, dpacc);
      softmax(qt, sL, sacc, dpacc, pf, sf);
      if (qtn < nqt) load_tile(qtn, bufq((st + 1) % 3), bufd((st + 1) % 3));
      cols(sQ, sD, pf, sf);
      if (qtn < nqt) store_tile(bufl((st + 1) % 3));
      wait_vmem_and_sync();
      qt = qtn;
    };
    while (qt < nqt) {
      body(std::integral_constant<int, 0>{});
      if (qt >= nqt) break;
      body(std::integral_constant<int, 1>{});
      if (qt >= nqt) break;
      body(std::integral_constant<int, 2>{});
    }
  } else {
    bool has_prev = false;
    auto body = [&](auto stage_c) __attribute__((always_inline)) {
      constexpr int st = decltype(stage_c)::value;
      char* sQ = bufq(st);
      char* sD = bufd(st);
      float* sL = bufl(st);
      const int qtn = next_tile(qt + 1);
      if (has_prev) cols(bufq((st + 2) % 3), bufd((st + 2) % 3), pf, sf);  // the previous tile
      if (qtn < nqt) load_tile(qtn, bufq((st + 1) % 3), bufd((st + 1) % 3));
      f32x4 sacc[4], dpacc[4];
      rows(sQ, sD, sacc, dpacc);
      softmax(qt, sL, sacc, dpacc, pf, sf);
      if (qtn < nqt) store_tile(bufl((st + 1) % 3));
      wait_vmem_and_sync();
      has_prev = true;
      qt = qtn;
    };
    int last = 0;  // buffer of the last tile
    while (qt < nqt) {
      body(std::integral_constant<int, 0>{});
      last = 0;
      if (qt >= nqt) break;
      body(std::integral_constant<int, 1>{});
      last = 1;
      if (qt >= nqt) break;
      body(std::integral_constant<int, 2>{});
      last = 2;
    }
    if (has_prev) cols(bufq(last), bufd(last), pf, sf);
  }
  }  // query heads of the group

  if (j < S) {
    char* vrow = (char*)p.dv + ((int64_t)b * p.dv_sb + (int64_t)hk * p.dv_sh + (int64_t)j * p.dv_ss) * 2;
    char* krow = (char*)p.dk + ((int64_t)b * p.dk_sb + (int64_t)hk * p.dk_sh + (int64_t)j * p.dk_ss) * 2;
    const float* trow = tab + (int64_t)j * D;
    typedef T v4 __attribute__((ext_vector_type(4)));
#pragma unroll
    for (int db = 0; db < 8; ++db) {
      const int d0 = 16 * db + 4 * g;
      v4 w;
#pragma unroll
      for (int i = 0; i < 4; ++i) w[i] = from_f<T>(dv[db][i]);
      *(v4*)(vrow + d0 * 2) = w;
      const float4 cs = *(const float4*)(trow + d0);
      const float sc = QS ? kLn2F : p.shp.scale;
      const float2 a = rot_pair_t(dk[db][0] * sc, dk[db][1] * sc, cs.x, cs.y);
      const float2 e = rot_pair_t(dk[db][2] * sc, dk[db][3] * sc, cs.z, cs.w);
      w[0] = from_f<T>(a.x);
      w[1] = from_f<T>(a.y);
      w[2] = from_f<T>(e.x);
      w[3] = from_f<T>(e.y);
      *(v4*)(krow + d0 * 2) = w;
    }
  }
  }  // key tiles of the workgroup
}

// ---------------------------------------------------------------------------------------
template <typename T, int MASK, bool CAUSAL, bool QROT>
static int launch_bwd16_t(const BwdParams& p, void* stream) {
  const int S = p.shp.S, BH = p.shp.B * p.shp.H;
  // dQ first: it also writes Q' and delta for the dK/dV kernel.  Causal: two query tiles of
  // one head per workgroup (see the kernel)
  const int grid_q = CAUSAL ? ((S + 127) / 128 + 1) / 2 * BH : ((S + 127) / 128) * BH;
  hipLaunchKernelGGL((dq16_kernel<T, MASK, CAUSAL, QROT>), dim3(grid_q), dim3(512), 0, (hipStream_t)stream, p);
  int e = (int)hipGetLastError();
  if (e) return e;
  const int nkt = (S + 127) / 128;
  const int grid_k = (CAUSAL ? (nkt + 1) / 2 : nkt) * p.shp.B * p.shp.Hkv;
  hipLaunchKernelGGL((dkdv16_kernel<T, MASK, CAUSAL, !QROT>), dim3(grid_k), dim3(512), 0, (hipStream_t)stream, p);
  return (int)hipGetLastError();
}

template <typename T, bool QROT>
static int launch_bwd16_dt(int mask_kind, bool causal, const BwdParams& p, void* stream) {
  if (causal) return launch_bwd16_t<T, MASK_NONE, true, QROT>(p, stream);
  switch (mask_kind) {
    case MASK_BOOL: return launch_bwd16_t<T, MASK_BOOL, false, QROT>(p, stream);
    case MASK_ADD: return launch_bwd16_t<T, MASK_ADD, false, QROT>(p, stream);
    default: return launch_bwd16_t<T, MASK_NONE, false, QROT>(p, stream);
  }
}

template <typename T>
static int launch_bwd16_pre(int mask_kind, bool causal, int pre, const BwdParams& p, void* stream) {
  switch (pre) {
    case 1: return launch_bwd16_dt<T, false>(mask_kind, causal, p, stream);
    case 3: return launch_bwd16_dt<T, true>(mask_kind, causal, p, stream);
    default: return -1;
  }
}

// dK/dV and dQ for 16-bit inputs at D = 128 (the dQ kernel computes delta).  pre: 1 K'
// prepared in p.k (kprep_kernel); 3 Q' (p.qrot) and K' (p.k) both prepared (the dequantized
// values of the quantized forward).
int launch_bwd16(int dtype, int mask_kind, bool causal, int pre, const BwdParams& p, void* stream) {
  return dtype == F16 ? launch_bwd16_pre<_Float16>(mask_kind, causal, pre, p, stream)
                      : launch_bwd16_pre<__bf16>(mask_kind, causal, pre, p, stream);
}

}  // namespace rs
