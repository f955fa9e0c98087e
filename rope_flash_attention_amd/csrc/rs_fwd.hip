// Forward kernel: rotary embedding of Q and K in registers + flash attention on MFMA.
//
// Computes, per (b, h) and query tile (page "Metal Flash Attention", section "Fused RoPE +
// SDPA"):  O = softmax(scale * R(Q) R(K)^T + M) V, with the softmax accumulated online in
// fp32 (section "Enable In SimpleTuner": fp16/bf16 keep fp32 softmax accumulation and the
// output is in the input dtype).
//
// Work decomposition (one workgroup = BM/32 waves, 32 query rows per wave, one (b, h);
// BM = 256 for bf16/fp16, 128 for fp32):
//  * each lane owns one query row m (lane r of wave w: m = q0 + 32w + r) and half of the
//    contraction elements of each k-step; Q is loaded once, rotated in fp32 with the packed
//    (cos, sin) table, rounded to the input dtype and kept in registers as MFMA B fragments;
//  * K/V tiles of BN keys stream through LDS, double buffered: K is rotated in registers on
//    its way in (never written back to memory), V is transposed into 128-byte rows with an
//    XOR swizzle so the P.V operand is one 16-byte LDS read per lane;
//  * S^T = K' Q'^T lands with one query per lane, so row max / row sum need one exchange
//    between wave halves and the P^T fragments feed O^T += V^T P^T directly from registers;
//  * the all-true / all-false state of each 64x64 bool-mask tile (computed beforehand on the
//    device) lets all-false tiles be skipped and all-true tiles run without mask reads;
//    causal tiles above the diagonal are never visited.
#include "rs_device.hpp"

namespace rs {

template <typename T>
struct FwdCfg {
  static constexpr int BM = sizeof(T) == 4 ? 128 : 256;  // query rows per workgroup
  static constexpr int BN = sizeof(T) == 4 ? 32 : 64;    // keys per LDS tile
  static constexpr int NT = 2 * BM;                      // threads: one wave per 32 rows
};

template <typename T, int D, int MASK, bool CAUSAL>
__global__ __launch_bounds__(FwdCfg<T>::NT, 1) void fwd_kernel(FwdParams p) {
  using M = Mf<T>;
  using frag = typename M::frag;
  constexpr int KPL = M::KPL, KSTEP = 2 * KPL;
  constexpr int BM = FwdCfg<T>::BM, BN = FwdCfg<T>::BN, NT = FwdCfg<T>::NT;
  constexpr int NQK = D / KSTEP;   // k-steps of Q'K'^T
  constexpr int NKB = BN / 32;     // 32-key blocks per tile
  constexpr int NDB = D / 32;      // 32-wide blocks of the head dim
  constexpr int ES = (int)sizeof(T);
  constexpr int EPC = 16 / ES;     // elements per 16-byte chunk
  constexpr int KP = D * ES + 16;  // K' LDS row pitch in bytes (padded)
  constexpr int KBYTES = BN * KP;
  constexpr int VROW = BN * ES;    // V^T row: 128 bytes
  static_assert(VROW == 128, "V^T rows are 8 swizzle units of 16 bytes");
  constexpr int VBYTES = D * VROW;
  constexpr int STAGE = KBYTES + VBYTES;
  constexpr int CPR = D / EPC;     // 16-byte chunks per K row
  constexpr int KCPT = BN * CPR / NT;
  static_assert(KCPT * NT == BN * CPR, "K tile split");
  constexpr int NC = D / EPC;      // V items: d-chunks x 4-key groups
  constexpr int NG = BN / 4;
  constexpr int VIT = NC * NG;
  static_assert(VIT <= NT && NC % 8 == 0 && NG % 2 == 0, "V tile split");

  __shared__ __attribute__((aligned(16))) char smem[2 * STAGE];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r = lane & 31, hh = lane >> 5;
  const int S = p.shp.S;

  // ---- work item -------------------------------------------------------------------------
  const int item = xcd_remap(blockIdx.x, gridDim.x);
  int qt = item % p.num_qt;
  const int bh = item / p.num_qt;
  const int hd = bh % p.shp.H, b = bh / p.shp.H;
  if (CAUSAL) qt = p.num_qt - 1 - qt;  // longest rows first
  const int q0 = qt * BM;
  const int m = q0 + wave * 32 + r;
  const int mc = m < S ? m : S - 1;

  const T* qbase = (const T*)p.q.ptr + b * p.q.sb + hd * p.q.sh;
  const T* kbase = (const T*)p.k.ptr + b * p.k.sb + hd * p.k.sh;
  const T* vbase = (const T*)p.v.ptr + b * p.v.sb + hd * p.v.sh;
  const float* tab = p.tab.ptr + b * p.tab.sb;  // float2 pairs, row stride D/2 pairs = D floats

  // ---- Q: load, rotate in fp32, round, keep as B fragments ---------------------------------
  frag qf[NQK];
  {
    const T* qrow = qbase + (int64_t)mc * p.q.ss;
    const float* trow = tab + (int64_t)mc * D;
    if constexpr (KPL == 8) {
#pragma unroll
      for (int t = 0; t < NQK; ++t) {
        const int d0 = t * 16 + hh * 8;
        typedef T v8 __attribute__((ext_vector_type(8)));
        v8 x = *(const v8*)(qrow + d0);
        const float4 cs0 = *(const float4*)(trow + d0);      // pairs d0/2, d0/2+1
        const float4 cs1 = *(const float4*)(trow + d0 + 4);  // pairs d0/2+2, d0/2+3
        const float cc[4] = {cs0.x, cs0.z, cs1.x, cs1.z};
        const float ss[4] = {cs0.y, cs0.w, cs1.y, cs1.w};
#pragma unroll
        for (int pp = 0; pp < 4; ++pp) {
          float2 rr = rot_pair(to_f(x[2 * pp]), to_f(x[2 * pp + 1]), cc[pp], ss[pp]);
          qf[t][2 * pp] = from_f<T>(rr.x);
          qf[t][2 * pp + 1] = from_f<T>(rr.y);
        }
      }
    } else {
#pragma unroll
      for (int t = 0; t < NQK; ++t) {  // element d = 2t + hh of pair t
        const float2 x = *(const float2*)(qrow + 2 * t);
        const float2 cs = *(const float2*)(trow + 2 * t);
        const float2 rr = rot_pair(x.x, x.y, cs.x, cs.y);
        qf[t] = hh ? rr.y : rr.x;
      }
    }
  }

  // ---- KV tile range -----------------------------------------------------------------------
  const int nkt = (S + BN - 1) / BN;
  int kt_end = nkt;
  if (CAUSAL) {
    const int last_row = min(q0 + BM, S) - 1;
    kt_end = min(nkt, last_row / BN + 1);
  }
  // bool masks: per-tile states over 64x64 blocks; this workgroup covers BM/64 of them
  // along the queries.
  auto tile_state = [&](int kt) -> uint32_t {
    if constexpr (MASK == MASK_BOOL) {
      const int kt64 = (kt * BN) / kMaskTile;
      const int bm = p.mask.t_sb ? b : 0, hm = p.mask.t_sh ? hd : 0;
      const int nq64 = (S + kMaskTile - 1) / kMaskTile;
      uint32_t st = 0;
      for (int u = 0; u < BM / kMaskTile; ++u) {
        const int q64 = (q0 / kMaskTile) + u;
        if (q64 < nq64) st |= mask_tile_state(p.mask, bm, hm, q64, kt64);
      }
      return st;
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

  // ---- global -> register staging of one KV tile ------------------------------------------
  uint4 kx[KCPT];
  float4 kt4[KCPT][EPC / 4];
  uint4 vx[4];
  // V item of this thread: bits [2:0] -> d-chunk low bits, bit 3 -> key-group bit 0,
  // remaining bits split between high d-chunk bits and high key-group bits.  Sixteen
  // consecutive lanes then write sixteen distinct 8-byte slots of the swizzled V^T rows.
  const int v_c = (tid & 7) + 8 * ((tid >> 4) % (NC / 8));
  const int v_g = ((tid >> 3) & 1) + 2 * ((tid >> 4) / (NC / 8));
  const bool v_act = tid < VIT;

  auto load_tile = [&](int kt) {
    const int kv0 = kt * BN;
#pragma unroll
    for (int it = 0; it < KCPT; ++it) {
      const int ci = tid + NT * it;
      const int key = ci / CPR, cc = ci % CPR;
      const int j = kv0 + key;
      if (j < S) {
        kx[it] = *(const uint4*)(kbase + (int64_t)j * p.k.ss + cc * EPC);
        const float* tr = tab + (int64_t)j * D + cc * EPC;  // EPC/2 pairs = EPC floats
#pragma unroll
        for (int u = 0; u < EPC / 4; ++u) kt4[it][u] = *(const float4*)(tr + 4 * u);
      } else {
        kx[it] = make_uint4(0, 0, 0, 0);
#pragma unroll
        for (int u = 0; u < EPC / 4; ++u) kt4[it][u] = make_float4(0.f, 0.f, 0.f, 0.f);
      }
    }
    if (v_act) {
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const int j = kv0 + 4 * v_g + rr;
        vx[rr] = j < S ? *(const uint4*)(vbase + (int64_t)j * p.v.ss + v_c * EPC) : make_uint4(0, 0, 0, 0);
      }
    }
  };

  auto store_tile = [&](int stage) {
    char* sK = smem + stage * STAGE;
    char* sV = sK + KBYTES;
#pragma unroll
    for (int it = 0; it < KCPT; ++it) {
      const int ci = tid + NT * it;
      const int key = ci / CPR, cc = ci % CPR;
      const float* tf = (const float*)&kt4[it][0];  // (c, s) per pair
      uint4 outw;
      if constexpr (ES == 2) {
        typedef T v8 __attribute__((ext_vector_type(8)));
        v8 x = *(const v8*)&kx[it];
        v8 y;
#pragma unroll
        for (int pp = 0; pp < 4; ++pp) {
          float2 rr = rot_pair(to_f(x[2 * pp]), to_f(x[2 * pp + 1]), tf[2 * pp], tf[2 * pp + 1]);
          y[2 * pp] = from_f<T>(rr.x);
          y[2 * pp + 1] = from_f<T>(rr.y);
        }
        outw = *(const uint4*)&y;
      } else {
        const float* x = (const float*)&kx[it];
        float y[4];
#pragma unroll
        for (int pp = 0; pp < 2; ++pp) {
          float2 rr = rot_pair(x[2 * pp], x[2 * pp + 1], tf[2 * pp], tf[2 * pp + 1]);
          y[2 * pp] = rr.x;
          y[2 * pp + 1] = rr.y;
        }
        outw = *(const uint4*)y;
      }
      *(uint4*)(sK + perm_row(key) * KP + cc * 16) = outw;
    }
    if (v_act) {
      const int kb0 = 4 * v_g * ES;  // byte column of the 4-key group
      const int unit = kb0 >> 4, off = kb0 & 15;
#pragma unroll
      for (int dd = 0; dd < EPC; ++dd) {
        const int d = v_c * EPC + dd;
        char* dst = sV + d * VROW + ((unit ^ swz(d)) << 4) + off;
        if constexpr (ES == 2) {
          const uint16_t* e0 = (const uint16_t*)&vx[0];
          const uint16_t* e1 = (const uint16_t*)&vx[1];
          const uint16_t* e2 = (const uint16_t*)&vx[2];
          const uint16_t* e3 = (const uint16_t*)&vx[3];
          uint2 w;
          w.x = (uint32_t)e0[dd] | ((uint32_t)e1[dd] << 16);
          w.y = (uint32_t)e2[dd] | ((uint32_t)e3[dd] << 16);
          *(uint2*)dst = w;
        } else {
          uint4 w;
          w.x = ((const uint32_t*)&vx[0])[dd];
          w.y = ((const uint32_t*)&vx[1])[dd];
          w.z = ((const uint32_t*)&vx[2])[dd];
          w.w = ((const uint32_t*)&vx[3])[dd];
          *(uint4*)dst = w;
        }
      }
    }
  };

  // ---- online softmax state ----------------------------------------------------------------
  f32x16 oacc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) oacc[db] = zero16();
  float m_run = -INFINITY, l_run = 0.f;
  const float c2 = p.shp.scale_log2;

  int kt = next_tile(0);
  if (kt < kt_end) {
    load_tile(kt);
    store_tile(0);
  }
  __syncthreads();
  int stage = 0;

  while (kt < kt_end) {
    const int ktn = next_tile(kt + 1);
    if (ktn < kt_end) load_tile(ktn);

    const char* sK = smem + stage * STAGE;
    const char* sV = sK + KBYTES;
    const int kv0 = kt * BN;

    // S^T = K' Q'^T : rows = keys, columns = this wave's 32 queries
    f32x16 sacc[NKB];
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      sacc[kb] = zero16();
#pragma unroll
      for (int t = 0; t < NQK; ++t) {
        const frag a = *(const frag*)(sK + (32 * kb + r) * KP + (t * KSTEP + hh * KPL) * ES);
        sacc[kb] = M::mma(a, qf[t], sacc[kb]);
      }
    }

    // exclusions: sequence tail, causal diagonal, masks
    const bool tail = kv0 + BN > S;
    const bool diag = CAUSAL && (kv0 + BN - 1 > q0);
    uint32_t st = TILE_ALL_TRUE;
    if constexpr (MASK == MASK_BOOL) st = tile_state(kt);
    if constexpr (MASK == MASK_ADD) {
      const int bm = p.mask.sb ? b : 0, hm = p.mask.sh ? hd : 0;
      const int esz = p.mask.dtype == F32 ? 4 : ES;
      const char* mrow = mask_row_ptr(p.mask, bm, hm, p.mask.sq ? mc : 0, esz);
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          float mv[8];
          mask_add8<T>(p.mask, mrow, kv0 + 32 * kb + 16 * c + 8 * hh, S, mv);
#pragma unroll
          for (int e = 0; e < 8; ++e) sacc[kb][8 * c + e] = fmaf(mv[e], p.shp.inv_scale, sacc[kb][8 * c + e]);
        }
    }
    if (tail || diag || (MASK == MASK_BOOL && st != TILE_ALL_TRUE)) {
      const uint8_t* brow = nullptr;
      if constexpr (MASK == MASK_BOOL) {
        const int bm = p.mask.sb ? b : 0, hm = p.mask.sh ? hd : 0;
        brow = (const uint8_t*)mask_row_ptr(p.mask, bm, hm, p.mask.sq ? mc : 0, 1);
      }
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          const int j0 = kv0 + 32 * kb + 16 * c + 8 * hh;
          uint32_t bits = 0xffu;
          if constexpr (MASK == MASK_BOOL) {
            if (st != TILE_ALL_TRUE) bits = mask_bits8(p.mask, brow, j0, S);
          }
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const int j = j0 + e;
            bool ok = j < S && ((bits >> e) & 1u);
            if (CAUSAL) ok = ok && j <= m;
            if (!ok) sacc[kb][8 * c + e] = -INFINITY;
          }
        }
    }

    // online softmax (scores in raw dot units; exp2 with scale*log2(e) folded in)
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) mx = fmaxf(mx, sacc[kb][i]);
    mx = xhalf_max(mx);
    const float m_new = fmaxf(m_run, mx);
    const float m_use = m_new == -INFINITY ? 0.f : m_new;
    const float alpha = fast_exp2((m_run - m_use) * c2);
    const float msc = m_use * c2;
    float rs = 0.f;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float pv = fast_exp2(fmaf(sacc[kb][i], c2, -msc));
        sacc[kb][i] = pv;
        rs += pv;
      }
    l_run = l_run * alpha + rs;
    m_run = m_new;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int i = 0; i < 16; ++i) oacc[db][i] *= alpha;

    // O^T += V^T P^T
    if constexpr (KPL == 8) {
      frag pf[NKB][2];
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int c = 0; c < 2; ++c)
#pragma unroll
          for (int e = 0; e < 8; ++e) pf[kb][c][e] = from_f<T>(sacc[kb][8 * c + e]);
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        const int d = 32 * db + r;
        const char* vrow = sV + d * VROW;
        const int sw = swz(d);
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
          for (int c = 0; c < 2; ++c) {
            const int unit = 4 * kb + 2 * c + hh;  // keys 32kb + 16c + 8hh .. +7
            const frag a = *(const frag*)(vrow + ((unit ^ sw) << 4));
            oacc[db] = M::mma(a, pf[kb][c], oacc[db]);
          }
      }
    } else {
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        const int d = 32 * db + r;
        const char* vrow = sV + d * VROW;
        const int sw = swz(d);
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int key = 32 * kb + c_idx_sig(i, hh);
            const float a = *(const float*)(vrow + (((key >> 2) ^ sw) << 4) + (key & 3) * 4);
            oacc[db] = M::mma(a, sacc[kb][i], oacc[db]);
          }
      }
    }

    if (ktn < kt_end) store_tile(stage ^ 1);
    __syncthreads();
    stage ^= 1;
    kt = ktn;
  }

  // ---- epilogue ------------------------------------------------------------------------------
  const float l = xhalf_sum(l_run);
  const float inv_l = l > 0.f ? 1.f / l : 0.f;
  if (m < S) {
    char* orow = (char*)p.o + ((int64_t)b * p.o_sb + (int64_t)hd * p.o_sh + (int64_t)m * p.o_ss) * ES;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d0 = 32 * db + 8 * g + 4 * hh;
        if constexpr (ES == 2) {
          typedef T v4 __attribute__((ext_vector_type(4)));
          v4 w;
#pragma unroll
          for (int e = 0; e < 4; ++e) w[e] = from_f<T>(oacc[db][4 * g + e] * inv_l);
          *(v4*)(orow + d0 * ES) = w;
        } else {
          float4 w = make_float4(oacc[db][4 * g] * inv_l, oacc[db][4 * g + 1] * inv_l,
                                 oacc[db][4 * g + 2] * inv_l, oacc[db][4 * g + 3] * inv_l);
          *(float4*)(orow + d0 * ES) = w;
        }
      }
    if (p.lse && hh == 0) {
      p.lse[((int64_t)b * p.shp.H + hd) * S + m] = l > 0.f ? m_run * p.shp.scale + logf(l) : -INFINITY;
    }
  }
}

template <typename T, int D, int MASK, bool CAUSAL>
static int launch_fwd_t(const FwdParams& p, void* stream) {
  const int grid = p.num_qt * p.shp.H * p.shp.B;
  hipLaunchKernelGGL((fwd_kernel<T, D, MASK, CAUSAL>), dim3(grid), dim3(FwdCfg<T>::NT), 0,
                     (hipStream_t)stream, p);
  return (int)hipGetLastError();
}

template <typename T, int D>
static int launch_fwd_d(int mask_kind, bool causal, const FwdParams& p, void* stream) {
  if (causal) return launch_fwd_t<T, D, MASK_NONE, true>(p, stream);
  switch (mask_kind) {
    case MASK_BOOL: return launch_fwd_t<T, D, MASK_BOOL, false>(p, stream);
    case MASK_ADD: return launch_fwd_t<T, D, MASK_ADD, false>(p, stream);
    default: return launch_fwd_t<T, D, MASK_NONE, false>(p, stream);
  }
}

template <typename T>
static int launch_fwd_dt(int D, int mask_kind, bool causal, const FwdParams& p, void* stream) {
  return D == 64 ? launch_fwd_d<T, 64>(mask_kind, causal, p, stream)
                 : launch_fwd_d<T, 128>(mask_kind, causal, p, stream);
}

int launch_fwd_int8(int dtype, int D, const FwdParams& p, void* stream);

int launch_fwd(int dtype, int D, int mask_kind, bool causal, bool int8, const FwdParams& p, void* stream) {
  if (int8) return launch_fwd_int8(dtype, D, p, stream);
  switch (dtype) {
    case F32: return launch_fwd_dt<float>(D, mask_kind, causal, p, stream);
    case F16: return launch_fwd_dt<_Float16>(D, mask_kind, causal, p, stream);
    default: return launch_fwd_dt<__bf16>(D, mask_kind, causal, p, stream);
  }
}

int fwd_block_m(int dtype) { return dtype == F32 ? FwdCfg<float>::BM : FwdCfg<__bf16>::BM; }

}  // namespace rs
