// Backward kernels: recompute-based attention backward through the rotation.
//
// Page "Metal Flash Attention" (SimpleTuner docs), section "Fused RoPE + SDPA": gradients
// are returned with respect to the pre-rotation Q and K by applying the inverse rotation
// (the same pairwise rotation with sin negated) to dQ' and dK'.  With P recomputed from the
// saved row normaliser LSE:
//    P = exp(scale S - LSE),  dV = P^T dO,  dP = dO V^T,  delta_i = sum_d dO_id O_id,
// (the scores recomputed from the forward's rounded operands: Q' scale log2 e and K')
//    dS = P o (dP - delta),   dQ' = scale dS K',  dK' = scale dS^T Q',
//    dQ = R^T dQ',  dK = R^T dK'.
// These 32x32 kernels serve fp32 inputs and D = 64 (16-bit inputs at D = 128 take the
// kernels of rs_bwd16.hip).  Three launches, no atomics (results are deterministic):
//   bwd_pre : delta per row;
//   dkdv    : one workgroup per 128 keys (32 per wave), looping over query tiles; K' and V
//             stay in registers, Q' and dO stream through LDS in row and transposed forms;
//   dq      : one workgroup per 128 queries, looping over key tiles; Q' and dO stay in
//             registers, K' (row and transposed) and V stream through LDS.
// Q and K are rotated in registers wherever they are loaded; no rotated copy is stored.
// PRE (the quantized backward at D = 64): Q' and K' arrive already rotated (the dequantized
// values the quantized forward attended with, in the workspace) and are only scaled.
#include "rs_device.hpp"

namespace rs {

// ---------------------------------------------------------------------------------------
// delta_i = sum_d dO_id O_id  (fp32)
template <typename T, int D>
__global__ __launch_bounds__(256) void bwd_pre_kernel(BwdParams p) {
  constexpr int ES = (int)sizeof(T), EPC = 16 / ES;
  constexpr int LPR = D / EPC;  // lanes per row
  constexpr int RPB = 256 / LPR;
  const int S = p.shp.S;
  const int64_t nrows = (int64_t)p.shp.B * p.shp.H * S;
  const int64_t gi = (int64_t)blockIdx.x * RPB + threadIdx.x / LPR;
  const int li = threadIdx.x % LPR;
  float acc = 0.f;
  if (gi < nrows) {
    const int i = (int)(gi % S);
    const int64_t bhx = gi / S;
    const int hd = (int)(bhx % p.shp.H), b = (int)(bhx / p.shp.H);
    const T* orow = (const T*)p.o.ptr + b * p.o.sb + hd * p.o.sh + (int64_t)i * p.o.ss + li * EPC;
    const T* grow = (const T*)p.dout.ptr + b * p.dout.sb + hd * p.dout.sh + (int64_t)i * p.dout.ss + li * EPC;
    typedef T vE __attribute__((ext_vector_type(EPC)));
    const vE ov = *(const vE*)orow;
    const vE gv = *(const vE*)grow;
#pragma unroll
    for (int e = 0; e < EPC; ++e) acc = fmaf(to_f(ov[e]), to_f(gv[e]), acc);
  }
#pragma unroll
  for (int w = LPR / 2; w >= 1; w >>= 1) acc += __shfl_xor(acc, w, LPR);
  if (gi < nrows && li == 0) p.delta[gi] = acc;
}

// ---------------------------------------------------------------------------------------
// Staging of a [ROWS x D] tile (rows = queries or keys) from HBM into LDS.  One item =
// 4 consecutive rows x one 16-byte column chunk; the thread->item mapping is the one the
// forward uses for V so that transposed writes are bank-conflict free.  Optionally rotates
// (Q, K) with the packed (cos, sin) table, and writes a row-major copy (rows permuted by
// perm_row, padded pitch) and/or a transposed copy (D rows of ROWS elements, 128 bytes,
// 16-byte units XOR-swizzled).
template <typename T, int D, int ROWS, bool ROT>
struct Stager {
  static constexpr int ES = (int)sizeof(T), EPC = 16 / ES;
  static constexpr int NC = D / EPC, NG = ROWS / 4, ITEMS = NC * NG;
  static constexpr int RP = D * ES + 16;  // row-major pitch (bytes)
  static constexpr int TROW = ROWS * ES;  // transposed row (bytes)
  static_assert(TROW == 128, "transposed rows are 128 bytes");
  static_assert(ITEMS <= 256 && NC % 8 == 0 && NG % 2 == 0, "item split");
  uint4 x[4];
  float4 t[4][ROT ? EPC / 4 : 1];
  int c, g;
  bool act;

  __device__ void init(int tid) {
    c = (tid & 7) + 8 * ((tid >> 4) % (NC / 8));
    g = ((tid >> 3) & 1) + 2 * ((tid >> 4) / (NC / 8));
    act = tid < ITEMS;
  }
  __device__ void load(const T* base, int64_t ss, int row0, int S, const float* tab) {
    if (!act) return;
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      const int j = row0 + 4 * g + rr;
      if (j < S) {
        x[rr] = *(const uint4*)(base + (int64_t)j * ss + c * EPC);
        if constexpr (ROT) {
          const float* tr = tab + (int64_t)j * D + c * EPC;
#pragma unroll
          for (int u = 0; u < EPC / 4; ++u) t[rr][u] = *(const float4*)(tr + 4 * u);
        }
      } else {
        x[rr] = make_uint4(0, 0, 0, 0);
        if constexpr (ROT) {
#pragma unroll
          for (int u = 0; u < EPC / 4; ++u) t[rr][u] = make_float4(0.f, 0.f, 0.f, 0.f);
        }
      }
    }
  }
  // rotated (ROT) as the forward rotates, multiplied by `mul` and rounded once
  __device__ void rotate(float mul) {
    if constexpr (!ROT) {
      if (mul == 1.f) return;
    }
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      const float* tf = (const float*)&t[rr][0];
      if constexpr (ES == 2) {
        typedef T v8 __attribute__((ext_vector_type(8)));
        v8 v = *(const v8*)&x[rr];
#pragma unroll
        for (int pp = 0; pp < 4; ++pp) {
          float2 q = make_float2(to_f(v[2 * pp]), to_f(v[2 * pp + 1]));
          if constexpr (ROT) q = rot_pair_fma(q.x, q.y, tf[2 * pp], tf[2 * pp + 1]);
          v[2 * pp] = from_f<T>(q.x * mul);
          v[2 * pp + 1] = from_f<T>(q.y * mul);
        }
        x[rr] = *(const uint4*)&v;
      } else {
        float* v = (float*)&x[rr];
#pragma unroll
        for (int pp = 0; pp < 2; ++pp) {
          float2 q = make_float2(v[2 * pp], v[2 * pp + 1]);
          if constexpr (ROT) q = rot_pair_fma(q.x, q.y, tf[2 * pp], tf[2 * pp + 1]);
          v[2 * pp] = q.x * mul;
          v[2 * pp + 1] = q.y * mul;
        }
      }
    }
  }
  __device__ void store_rows(char* sR) const {
    if (!act) return;
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) *(uint4*)(sR + perm_row(4 * g + rr) * RP + c * 16) = x[rr];
  }
  __device__ void store_t(char* sT) const {
    if (!act) return;
    const int kb0 = 4 * g * ES;
    const int unit = kb0 >> 4, off = kb0 & 15;
#pragma unroll
    for (int dd = 0; dd < EPC; ++dd) {
      const int d = c * EPC + dd;
      char* dst = sT + d * TROW + ((unit ^ swz(d)) << 4) + off;
      if constexpr (ES == 2) {
        const uint16_t* e0 = (const uint16_t*)&x[0];
        const uint16_t* e1 = (const uint16_t*)&x[1];
        const uint16_t* e2 = (const uint16_t*)&x[2];
        const uint16_t* e3 = (const uint16_t*)&x[3];
        uint2 w;
        w.x = (uint32_t)e0[dd] | ((uint32_t)e1[dd] << 16);
        w.y = (uint32_t)e2[dd] | ((uint32_t)e3[dd] << 16);
        *(uint2*)dst = w;
      } else {
        uint4 w;
        w.x = ((const uint32_t*)&x[0])[dd];
        w.y = ((const uint32_t*)&x[1])[dd];
        w.z = ((const uint32_t*)&x[2])[dd];
        w.w = ((const uint32_t*)&x[3])[dd];
        *(uint4*)dst = w;
      }
    }
  }
};

// B fragments of one lane: row `row` of a [*, D] operand, contraction element
// t*KSTEP + hh*KPL + e, optionally rotated (fp32 math, as the forward rotates), multiplied
// by `mul` and rounded once to T.
template <typename T, int D, bool ROT>
__device__ inline void load_row_frags(typename Mf<T>::frag* f, const T* rowp, const float* trow, int hh,
                                      float mul = 1.f) {
  constexpr int KPL = Mf<T>::KPL, KSTEP = 2 * KPL, NQK = D / KSTEP;
  if constexpr (KPL == 8) {
#pragma unroll
    for (int t = 0; t < NQK; ++t) {
      const int d0 = t * 16 + hh * 8;
      typedef T v8 __attribute__((ext_vector_type(8)));
      v8 x = *(const v8*)(rowp + d0);
      if constexpr (ROT) {
        const float4 cs0 = *(const float4*)(trow + d0);
        const float4 cs1 = *(const float4*)(trow + d0 + 4);
        const float cc[4] = {cs0.x, cs0.z, cs1.x, cs1.z};
        const float ss[4] = {cs0.y, cs0.w, cs1.y, cs1.w};
#pragma unroll
        for (int pp = 0; pp < 4; ++pp) {
          float2 rr = rot_pair_fma(to_f(x[2 * pp]), to_f(x[2 * pp + 1]), cc[pp], ss[pp]);
          x[2 * pp] = from_f<T>(rr.x * mul);
          x[2 * pp + 1] = from_f<T>(rr.y * mul);
        }
      } else if (mul != 1.f) {
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] = from_f<T>(to_f(x[e]) * mul);
      }
      f[t] = x;
    }
  } else {
#pragma unroll
    for (int t = 0; t < NQK; ++t) {
      const float2 x = *(const float2*)(rowp + 2 * t);
      if constexpr (ROT) {
        const float2 cs = *(const float2*)(trow + 2 * t);
        const float2 rr = rot_pair_fma(x.x, x.y, cs.x, cs.y);
        f[t] = (hh ? rr.y : rr.x) * mul;
      } else {
        f[t] = (hh ? x.y : x.x) * mul;
      }
    }
  }
}

template <typename T, int D>
__device__ inline void zero_frags(typename Mf<T>::frag* f) {
  constexpr int NQK = D / (2 * Mf<T>::KPL);
#pragma unroll
  for (int t = 0; t < NQK; ++t) {
    if constexpr (Mf<T>::KPL == 8) {
#pragma unroll
      for (int e = 0; e < 8; ++e) f[t][e] = from_f<T>(0.f);
    } else {
      f[t] = 0.f;
    }
  }
}

// Writes a 32 x D block held transposed in accumulators (acc[db] register i = element
// (d = 32db + c_row(i, hh), row)) to row `row` of a [*, D] output, times `mul`, optionally
// with the inverse rotation of each (2p, 2p+1) pair.
template <typename T, int D, bool ROT_T>
__device__ inline void store_acc_row(char* orow, const f32x16* acc, float mul, const float* trow, int hh) {
  constexpr int ES = (int)sizeof(T), NDB = D / 32;
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int d0 = 32 * db + 8 * g + 4 * hh;
      float v[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = acc[db][4 * g + e] * mul;
      if constexpr (ROT_T) {
        const float4 cs = *(const float4*)(trow + d0);  // pairs d0/2, d0/2 + 1
        const float2 a = rot_pair_t(v[0], v[1], cs.x, cs.y);
        const float2 c = rot_pair_t(v[2], v[3], cs.z, cs.w);
        v[0] = a.x; v[1] = a.y; v[2] = c.x; v[3] = c.y;
      }
      if constexpr (ES == 2) {
        typedef T v4 __attribute__((ext_vector_type(4)));
        v4 w;
#pragma unroll
        for (int e = 0; e < 4; ++e) w[e] = from_f<T>(v[e]);
        *(v4*)(orow + d0 * ES) = w;
      } else {
        *(float4*)(orow + d0 * ES) = make_float4(v[0], v[1], v[2], v[3]);
      }
    }
}

constexpr float kLog2e = 1.4426950408889634f;

// ---------------------------------------------------------------------------------------
// dK / dV: workgroup = 128 keys of one (b, h); wave w owns keys k0 + 32w .. +31.
template <typename T>
struct DkdvCfg {
  static constexpr int BNK = 128;                      // keys per workgroup
  static constexpr int BMQ = sizeof(T) == 4 ? 32 : 64;  // queries per LDS tile
};

// PRE: Q and K arrive rotated (p.q, p.k point at Q' and K' in the workspace, e.g. the
// dequantized values of the quantized forward): no rotation on load; the epilogues still
// apply the inverse rotation.
template <typename T, int D, int MASK, bool CAUSAL, bool PRE>
__global__ __launch_bounds__(256, 1) void dkdv_kernel(BwdParams p) {
  using M = Mf<T>;
  using frag = typename M::frag;
  constexpr int KPL = M::KPL, KSTEP = 2 * KPL, NQK = D / KSTEP, NDB = D / 32;
  constexpr int ES = (int)sizeof(T);
  constexpr int BNK = DkdvCfg<T>::BNK, BMQ = DkdvCfg<T>::BMQ, NMB = BMQ / 32;
  using St = Stager<T, D, BMQ, !PRE>;
  using Sd = Stager<T, D, BMQ, false>;
  constexpr int RB = BMQ * St::RP, TB = D * St::TROW;
  constexpr int OFF_Q = 0, OFF_QT = RB, OFF_DO = RB + TB, OFF_DOT = 2 * RB + TB, OFF_L = 2 * RB + 2 * TB;
  constexpr int STAGE = OFF_L + 2 * BMQ * 4;
  __shared__ __attribute__((aligned(16))) char smem[2 * STAGE];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r = lane & 31, hh = lane >> 5;
  const int S = p.shp.S;
  const int nkt = (S + BNK - 1) / BNK;
  // workgroup = one key tile of one (b, K/V head); with grouped-query attention it runs the
  // query tiles of every query head of the group, dK and dV accumulating across them
  const int item = xcd_remap(blockIdx.x, gridDim.x);
  const int kt = item % nkt;
  const int bh = item / nkt;
  const int hk = bh % p.shp.Hkv, b = bh / p.shp.Hkv;
  const int k0 = kt * BNK;
  const int j = k0 + 32 * wave + r;  // this lane's key
  const int jc = j < S ? j : S - 1;

  const float* tab = p.tab.ptr + b * p.tab.sb;
  int hd = 0;  // the query head whose tiles are being run
  const T* qbase = nullptr;
  const T* dobase = nullptr;
  const float* lse = nullptr;
  const float* dlt = nullptr;
  auto set_head = [&](int h) {
    hd = h;
    qbase = (const T*)p.q.ptr + b * p.q.sb + hd * p.q.sh;
    dobase = (const T*)p.dout.ptr + b * p.dout.sb + hd * p.dout.sh;
    lse = p.lse + ((int64_t)b * p.shp.H + hd) * S;
    dlt = p.delta + ((int64_t)b * p.shp.H + hd) * S;
  };

  // K' and V of this lane's key as B fragments (column = key)
  frag kf[NQK], vf[NQK];
  if (j < S) {
    load_row_frags<T, D, !PRE>(kf, (const T*)p.k.ptr + b * p.k.sb + hk * p.k.sh + (int64_t)j * p.k.ss,
                               tab + (int64_t)j * D, hh);
    load_row_frags<T, D, false>(vf, (const T*)p.v.ptr + b * p.v.sb + hk * p.v.sh + (int64_t)j * p.v.ss,
                                nullptr, hh);
  } else {
    zero_frags<T, D>(kf);
    zero_frags<T, D>(vf);
  }

  f32x16 dv_acc[NDB], dk_acc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) {
    dv_acc[db] = zero16();
    dk_acc[db] = zero16();
  }

  // query tile range
  const int nqt = (S + BMQ - 1) / BMQ;
  const int qt_begin = CAUSAL ? k0 / BMQ : 0;
  auto tile_state = [&](int qt) -> uint32_t {
    if constexpr (MASK == MASK_BOOL) {
      const int bm = p.mask.t_sb ? b : 0, hm = p.mask.t_sh ? hd : 0;
      const int q64 = (qt * BMQ) / kMaskTile;
      const int nk64 = (S + kMaskTile - 1) / kMaskTile;
      uint32_t st = 0;
      for (int u = 0; u < BNK / kMaskTile; ++u) {
        const int k64 = k0 / kMaskTile + u;
        if (k64 < nk64) st |= mask_tile_state(p.mask, bm, hm, q64, k64);
      }
      return st;
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

  St sq;
  Sd sdo;
  sq.init(tid);
  sdo.init(tid);
  float l_reg = 0.f, d_reg = 0.f;
  auto load_tile = [&](int qt) {
    const int q0 = qt * BMQ;
    sq.load(qbase, p.q.ss, q0, S, tab);
    sdo.load(dobase, p.dout.ss, q0, S, nullptr);
    if (tid < BMQ) {
      const int i = q0 + tid;
      const float lv = i < S ? lse[i] : -INFINITY;
      l_reg = lv == -INFINITY ? INFINITY : lv * kLog2e;  // +inf makes P = 0 for empty rows
      d_reg = i < S ? dlt[i] : 0.f;
    }
  };
  auto store_tile = [&](int stage) {
    char* base = smem + stage * STAGE;
    sq.rotate(p.shp.scale_log2);  // Q' scale log2 e: the forward's score operand
    sq.store_rows(base + OFF_Q);
    sq.store_t(base + OFF_QT);
    sdo.store_rows(base + OFF_DO);
    sdo.store_t(base + OFF_DOT);
    if (tid < BMQ) {
      ((float*)(base + OFF_L))[tid] = l_reg;
      ((float*)(base + OFF_L))[BMQ + tid] = d_reg;
    }
  };

#pragma unroll 1
  for (int g = 0; g < p.shp.group; ++g) {
  set_head(hk * p.shp.group + g);
  if (g > 0) __syncthreads();  // LDS of the previous head's last tile
  int qt = next_tile(qt_begin);
  if (qt < nqt) {
    load_tile(qt);
    store_tile(0);
  }
  __syncthreads();
  int stage = 0;
  while (qt < nqt) {
    const int qtn = next_tile(qt + 1);
    if (qtn < nqt) load_tile(qtn);
    const char* base = smem + stage * STAGE;
    const int q0 = qt * BMQ;

    // S = Q' K'^T  (rows = queries of this tile, column = this lane's key)
    f32x16 sacc[NMB], dpacc[NMB];
#pragma unroll
    for (int mb = 0; mb < NMB; ++mb) {
      sacc[mb] = zero16();
      dpacc[mb] = zero16();
#pragma unroll
      for (int t = 0; t < NQK; ++t) {
        const int co = (t * KSTEP + hh * KPL) * ES;
        const frag a = *(const frag*)(base + OFF_Q + (32 * mb + r) * St::RP + co);
        sacc[mb] = M::mma(a, kf[t], sacc[mb]);
        const frag g = *(const frag*)(base + OFF_DO + (32 * mb + r) * St::RP + co);
        dpacc[mb] = M::mma(g, vf[t], dpacc[mb]);
      }
    }

    // P = exp2(S - LSE log2 e) on attended entries (S from the forward's operands Q' scale
    // log2 e and K', in log2 units), 0 elsewhere; dS = P (dP - delta)
    const float* sl = (const float*)(base + OFF_L);
    const bool tail = q0 + BMQ > S || k0 + BNK > S;
    const bool diag = CAUSAL && (q0 < k0 + BNK - 1);
    uint32_t st = TILE_ALL_TRUE;
    if constexpr (MASK == MASK_BOOL) st = tile_state(qt);
    const bool check = tail || diag || (MASK == MASK_BOOL && st != TILE_ALL_TRUE);
    const int bm = p.mask.sb ? b : 0, hm = p.mask.sh ? hd : 0;
    if constexpr (MASK == MASK_ADD) {
      // additive mask values of this lane's key for its 16 query rows per 32-row block
      const int jj = p.mask.key_bcast ? 0 : jc;
      if (p.mask.dtype == F32) {
#pragma unroll
        for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int qi = min(q0 + 32 * mb + c_idx_sig(i, hh), S - 1);
            const float* mrow = (const float*)mask_row_ptr(p.mask, bm, hm, p.mask.sq ? qi : 0, 4);
            sacc[mb][i] = fmaf(mrow[jj], kLog2eF, sacc[mb][i]);
          }
      } else {
#pragma unroll
        for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int qi = min(q0 + 32 * mb + c_idx_sig(i, hh), S - 1);
            const T* mrow = (const T*)mask_row_ptr(p.mask, bm, hm, p.mask.sq ? qi : 0, ES);
            sacc[mb][i] = fmaf(to_f(mrow[jj]), kLog2eF, sacc[mb][i]);
          }
      }
    }
#pragma unroll
    for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const int mr0 = 32 * mb + 16 * c + 8 * hh;  // 8 consecutive query rows (tile-local)
        const float4 la = *(const float4*)(sl + mr0), lb = *(const float4*)(sl + mr0 + 4);
        const float4 da = *(const float4*)(sl + BMQ + mr0), dbv = *(const float4*)(sl + BMQ + mr0 + 4);
        const float lv[8] = {la.x, la.y, la.z, la.w, lb.x, lb.y, lb.z, lb.w};
        const float dv[8] = {da.x, da.y, da.z, da.w, dbv.x, dbv.y, dbv.z, dbv.w};
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int i = q0 + mr0 + e;
          const float s = sacc[mb][8 * c + e];
          bool ok = true;
          if (check) {
            ok = i < S && j < S;
            if (CAUSAL) ok = ok && j <= i;
            if constexpr (MASK == MASK_BOOL) {
              if (st != TILE_ALL_TRUE && ok) {
                const uint8_t* brow = (const uint8_t*)mask_row_ptr(p.mask, bm, hm, p.mask.sq ? i : 0, 1);
                ok = brow[p.mask.key_bcast ? 0 : j] != 0;
              }
            }
          }
          const float pv = ok ? fast_exp2(s - lv[e]) : 0.f;
          sacc[mb][8 * c + e] = pv;
          dpacc[mb][8 * c + e] = pv * (dpacc[mb][8 * c + e] - dv[e]);
        }
      }

    // dV^T += dO^T P ;  dK'^T += Q'^T dS
    if constexpr (KPL == 8) {
      frag pf[NMB][2], sf[NMB][2];
#pragma unroll
      for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
        for (int c = 0; c < 2; ++c)
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            pf[mb][c][e] = from_f<T>(sacc[mb][8 * c + e]);
            sf[mb][c][e] = from_f<T>(dpacc[mb][8 * c + e]);
          }
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        const int d = 32 * db + r;
        const int sw = swz(d);
        const char* dot_row = base + OFF_DOT + d * St::TROW;
        const char* qt_row = base + OFF_QT + d * St::TROW;
#pragma unroll
        for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
          for (int c = 0; c < 2; ++c) {
            const int unit = 4 * mb + 2 * c + hh;
            const frag a = *(const frag*)(dot_row + ((unit ^ sw) << 4));
            dv_acc[db] = M::mma(a, pf[mb][c], dv_acc[db]);
            const frag bq = *(const frag*)(qt_row + ((unit ^ sw) << 4));
            dk_acc[db] = M::mma(bq, sf[mb][c], dk_acc[db]);
          }
      }
    } else {
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        const int d = 32 * db + r;
        const int sw = swz(d);
        const char* dot_row = base + OFF_DOT + d * St::TROW;
        const char* qt_row = base + OFF_QT + d * St::TROW;
#pragma unroll
        for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int mq = 32 * mb + c_idx_sig(i, hh);
            const int off = (((mq >> 2) ^ sw) << 4) + (mq & 3) * 4;
            dv_acc[db] = M::mma(*(const float*)(dot_row + off), sacc[mb][i], dv_acc[db]);
            dk_acc[db] = M::mma(*(const float*)(qt_row + off), dpacc[mb][i], dk_acc[db]);
          }
      }
    }

    if (qtn < nqt) store_tile(stage ^ 1);
    __syncthreads();
    stage ^= 1;
    qt = qtn;
  }
  }  // query heads of the group

  if (j < S) {
    char* dvrow = (char*)p.dv + ((int64_t)b * p.dv_sb + (int64_t)hk * p.dv_sh + (int64_t)j * p.dv_ss) * ES;
    store_acc_row<T, D, false>(dvrow, dv_acc, 1.f, nullptr, hh);
    char* dkrow = (char*)p.dk + ((int64_t)b * p.dk_sb + (int64_t)hk * p.dk_sh + (int64_t)j * p.dk_ss) * ES;
    store_acc_row<T, D, true>(dkrow, dk_acc, kLn2F, tab + (int64_t)j * D, hh);  // (Q' carried log2 e)
  }
}

// ---------------------------------------------------------------------------------------
// dQ: workgroup = 128 queries of one (b, h); lane owns query m = q0 + 32w + r.
template <typename T>
struct DqCfg {
  static constexpr int BM = 128;
  static constexpr int BN = sizeof(T) == 4 ? 32 : 64;
};

template <typename T, int D, int MASK, bool CAUSAL, bool PRE>
__global__ __launch_bounds__(256, 1) void dq_kernel(BwdParams p) {
  using M = Mf<T>;
  using frag = typename M::frag;
  constexpr int KPL = M::KPL, KSTEP = 2 * KPL, NQK = D / KSTEP, NDB = D / 32;
  constexpr int ES = (int)sizeof(T);
  constexpr int BM = DqCfg<T>::BM, BN = DqCfg<T>::BN, NKB = BN / 32;
  using Sk = Stager<T, D, BN, !PRE>;
  using Sv = Stager<T, D, BN, false>;
  constexpr int RB = BN * Sk::RP, TB = D * Sk::TROW;
  constexpr int OFF_K = 0, OFF_KT = RB, OFF_V = RB + TB;
  constexpr int STAGE = 2 * RB + TB;
  __shared__ __attribute__((aligned(16))) char smem[2 * STAGE];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r = lane & 31, hh = lane >> 5;
  const int S = p.shp.S;
  const int nqt = (S + BM - 1) / BM;
  const int item = xcd_remap(blockIdx.x, gridDim.x);
  int qt = item % nqt;
  const int bh = item / nqt;
  const int hd = bh % p.shp.H, b = bh / p.shp.H;
  if (CAUSAL) qt = nqt - 1 - qt;
  const int q0 = qt * BM;
  const int m = q0 + 32 * wave + r;
  const int mc = m < S ? m : S - 1;

  const int hk = hd / p.shp.group;  // K/V head (grouped-query attention)
  const T* kbase = (const T*)p.k.ptr + b * p.k.sb + hk * p.k.sh;
  const T* vbase = (const T*)p.v.ptr + b * p.v.sb + hk * p.v.sh;
  const float* tab = p.tab.ptr + b * p.tab.sb;

  frag qf[NQK], gf[NQK];
  load_row_frags<T, D, !PRE>(qf, (const T*)p.q.ptr + b * p.q.sb + hd * p.q.sh + (int64_t)mc * p.q.ss,
                             tab + (int64_t)mc * D, hh, p.shp.scale_log2);  // the forward's Q' scale log2 e
  load_row_frags<T, D, false>(gf, (const T*)p.dout.ptr + b * p.dout.sb + hd * p.dout.sh + (int64_t)mc * p.dout.ss,
                              nullptr, hh);
  const int64_t rowid = ((int64_t)b * p.shp.H + hd) * S + mc;
  const float lse_v = p.lse[rowid];
  const float l2 = lse_v == -INFINITY ? INFINITY : lse_v * kLog2e;
  const float dlt = p.delta[rowid];

  f32x16 dq_acc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) dq_acc[db] = zero16();

  const int nkt = (S + BN - 1) / BN;
  int kt_end = nkt;
  if (CAUSAL) kt_end = min(nkt, (min(q0 + BM, S) - 1) / BN + 1);
  auto tile_state = [&](int kt) -> uint32_t {
    if constexpr (MASK == MASK_BOOL) {
      const int bm = p.mask.t_sb ? b : 0, hm = p.mask.t_sh ? hd : 0;
      const int kt64 = (kt * BN) / kMaskTile;
      uint32_t st = mask_tile_state(p.mask, bm, hm, 2 * qt, kt64);
      if (2 * qt + 1 < (S + kMaskTile - 1) / kMaskTile) st |= mask_tile_state(p.mask, bm, hm, 2 * qt + 1, kt64);
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

  Sk sk;
  Sv sv;
  sk.init(tid);
  sv.init(tid);
  auto load_tile = [&](int kt) {
    sk.load(kbase, p.k.ss, kt * BN, S, tab);
    sv.load(vbase, p.v.ss, kt * BN, S, nullptr);
  };
  auto store_tile = [&](int stage) {
    char* base = smem + stage * STAGE;
    sk.rotate(1.f);
    sk.store_rows(base + OFF_K);
    sk.store_t(base + OFF_KT);
    sv.store_rows(base + OFF_V);
  };

  int kt = next_tile(0);
  if (kt < kt_end) {
    load_tile(kt);
    store_tile(0);
  }
  __syncthreads();
  int stage = 0;
  const int bm = p.mask.sb ? b : 0, hm = p.mask.sh ? hd : 0;
  while (kt < kt_end) {
    const int ktn = next_tile(kt + 1);
    if (ktn < kt_end) load_tile(ktn);
    const char* base = smem + stage * STAGE;
    const int kv0 = kt * BN;

    f32x16 sacc[NKB], dpacc[NKB];
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      sacc[kb] = zero16();
      dpacc[kb] = zero16();
#pragma unroll
      for (int t = 0; t < NQK; ++t) {
        const int co = (t * KSTEP + hh * KPL) * ES;
        const frag a = *(const frag*)(base + OFF_K + (32 * kb + r) * Sk::RP + co);
        sacc[kb] = M::mma(a, qf[t], sacc[kb]);
        const frag vv = *(const frag*)(base + OFF_V + (32 * kb + r) * Sk::RP + co);
        dpacc[kb] = M::mma(vv, gf[t], dpacc[kb]);
      }
    }

    const bool tail = kv0 + BN > S;
    const bool diag = CAUSAL && (kv0 + BN - 1 > q0);
    uint32_t st = TILE_ALL_TRUE;
    if constexpr (MASK == MASK_BOOL) st = tile_state(kt);
    if constexpr (MASK == MASK_ADD) {
      const int esz = p.mask.dtype == F32 ? 4 : ES;
      const char* mrow = mask_row_ptr(p.mask, bm, hm, p.mask.sq ? mc : 0, esz);
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          float mv[8];
          mask_add8<T>(p.mask, mrow, kv0 + 32 * kb + 16 * c + 8 * hh, S, mv);
#pragma unroll
          for (int e = 0; e < 8; ++e) sacc[kb][8 * c + e] = fmaf(mv[e], kLog2eF, sacc[kb][8 * c + e]);
        }
    }
    const bool check = tail || diag || (MASK == MASK_BOOL && st != TILE_ALL_TRUE);
    const uint8_t* brow = nullptr;
    if constexpr (MASK == MASK_BOOL) brow = (const uint8_t*)mask_row_ptr(p.mask, bm, hm, p.mask.sq ? mc : 0, 1);
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const int j0 = kv0 + 32 * kb + 16 * c + 8 * hh;
        uint32_t bits = 0xffu;
        if (check) {
          if constexpr (MASK == MASK_BOOL) {
            if (st != TILE_ALL_TRUE) bits = mask_bits8(p.mask, brow, j0, S);
          }
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          bool ok = true;
          if (check) {
            const int jj = j0 + e;
            ok = jj < S && m < S && ((bits >> e) & 1u);
            if (CAUSAL) ok = ok && jj <= m;
          }
          const float pv = ok ? fast_exp2(sacc[kb][8 * c + e] - l2) : 0.f;
          sacc[kb][8 * c + e] = pv * (dpacc[kb][8 * c + e] - dlt);  // dS^T
        }
      }

    // dQ'^T += K'^T dS^T
    if constexpr (KPL == 8) {
      frag sf[NKB][2];
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int c = 0; c < 2; ++c)
#pragma unroll
          for (int e = 0; e < 8; ++e) sf[kb][c][e] = from_f<T>(sacc[kb][8 * c + e]);
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        const int d = 32 * db + r;
        const int sw = swz(d);
        const char* krow = base + OFF_KT + d * Sk::TROW;
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
          for (int c = 0; c < 2; ++c) {
            const int unit = 4 * kb + 2 * c + hh;
            const frag a = *(const frag*)(krow + ((unit ^ sw) << 4));
            dq_acc[db] = M::mma(a, sf[kb][c], dq_acc[db]);
          }
      }
    } else {
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        const int d = 32 * db + r;
        const int sw = swz(d);
        const char* krow = base + OFF_KT + d * Sk::TROW;
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int key = 32 * kb + c_idx_sig(i, hh);
            const float a = *(const float*)(krow + (((key >> 2) ^ sw) << 4) + (key & 3) * 4);
            dq_acc[db] = M::mma(a, sacc[kb][i], dq_acc[db]);
          }
      }
    }

    if (ktn < kt_end) store_tile(stage ^ 1);
    __syncthreads();
    stage ^= 1;
    kt = ktn;
  }

  if (m < S) {
    char* dqrow = (char*)p.dq + ((int64_t)b * p.dq_sb + (int64_t)hd * p.dq_sh + (int64_t)m * p.dq_ss) * ES;
    store_acc_row<T, D, true>(dqrow, dq_acc, p.shp.scale, tab + (int64_t)m * D, hh);
  }
}

// ---------------------------------------------------------------------------------------
template <typename T, int D, int MASK, bool CAUSAL, bool PRE = false>
static int launch_bwd_t(const BwdParams& p, hipStream_t s) {
  constexpr int LPR = D * (int)sizeof(T) / 16, RPB = 256 / LPR;
  const int64_t nrows = (int64_t)p.shp.B * p.shp.H * p.shp.S;
  hipLaunchKernelGGL((bwd_pre_kernel<T, D>), dim3((unsigned)((nrows + RPB - 1) / RPB)), dim3(256), 0, s, p);
  int e = (int)hipGetLastError();
  if (e) return e;
  const int nk = (p.shp.S + DkdvCfg<T>::BNK - 1) / DkdvCfg<T>::BNK;
  hipLaunchKernelGGL((dkdv_kernel<T, D, MASK, CAUSAL, PRE>), dim3(nk * p.shp.Hkv * p.shp.B), dim3(256), 0, s, p);
  e = (int)hipGetLastError();
  if (e) return e;
  const int nq = (p.shp.S + DqCfg<T>::BM - 1) / DqCfg<T>::BM;
  hipLaunchKernelGGL((dq_kernel<T, D, MASK, CAUSAL, PRE>), dim3(nq * p.shp.H * p.shp.B), dim3(256), 0, s, p);
  return (int)hipGetLastError();
}

template <typename T, int D, bool PRE = false>
static int launch_bwd_d(int mask_kind, bool causal, const BwdParams& p, hipStream_t s) {
  if (causal) return launch_bwd_t<T, D, MASK_NONE, true, PRE>(p, s);
  switch (mask_kind) {
    case MASK_BOOL: return launch_bwd_t<T, D, MASK_BOOL, false, PRE>(p, s);
    case MASK_ADD: return launch_bwd_t<T, D, MASK_ADD, false, PRE>(p, s);
    default: return launch_bwd_t<T, D, MASK_NONE, false, PRE>(p, s);
  }
}

template <typename T>
static int launch_bwd_dt(int D, int mask_kind, bool causal, const BwdParams& p, hipStream_t s) {
  return D == 64 ? launch_bwd_d<T, 64>(mask_kind, causal, p, s) : launch_bwd_d<T, 128>(mask_kind, causal, p, s);
}

int launch_bwd16(int dtype, int mask_kind, bool causal, int pre, const BwdParams& p, void* stream);

// 16-bit inputs at D = 128 use the 16x16 kernels of rs_bwd16.hip (whose dQ kernel computes
// delta on the way; no pre-pass).
template <typename T>
static int launch_bwd_16bit(int dtype, int D, int mask_kind, bool causal, int pre, const BwdParams& p,
                            hipStream_t s) {
  if (D == 64) {  // (pre: 0, or 3 for the quantized backward's Q' and K')
    if (pre == 3) return launch_bwd_d<T, 64, true>(mask_kind, causal, p, s);
    return pre == 0 ? launch_bwd_d<T, 64>(mask_kind, causal, p, s) : -1;
  }
  return launch_bwd16(dtype, mask_kind, causal, pre, p, s);
}

int launch_bwd(int dtype, int D, int mask_kind, bool causal, int pre, const BwdParams& p, void* stream) {
  hipStream_t s = (hipStream_t)stream;
  switch (dtype) {
    case F32: return pre == 0 ? launch_bwd_dt<float>(D, mask_kind, causal, p, s) : -1;
    case F16: return launch_bwd_16bit<_Float16>(dtype, D, mask_kind, causal, pre, p, s);
    default: return launch_bwd_16bit<__bf16>(dtype, D, mask_kind, causal, pre, p, s);
  }
}

}  // namespace rs
