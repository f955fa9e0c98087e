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
//    (cos, sin) table, multiplied by scale*log2(e) (scores come out in log2 units), rounded
//    to the input dtype and kept in registers as MFMA B fragments;
//  * K/V tiles of BN keys stream through LDS, double buffered: K is rotated in registers on
//    its way in (never written back to memory); V goes from memory straight into a
//    row-major LDS tile (buffer loads with an LDS destination, chunks XOR-swizzled per row)
//    and the P.V operand is read transposed from it;
//  * S^T = K' Q'^T lands with one query per lane, so the row max needs one exchange between
//    wave halves and the P^T fragments feed O^T += V^T P^T directly from registers;
//  * the running row max m enters the S product through the MFMA accumulator (C = -m), so
//    P = exp2(S) needs no per-score arithmetic; m (and with it O and the row sum) is only
//    rescaled when a tile raises some row's max by more than 2^8 (exact: the max is only a
//    range guard), which after the first tiles almost never happens;
//  * row sums accumulate the rounded P pairs with dot2 instructions (the same values that
//    multiply V);
//  * the all-true / all-false state of each 64x64 bool-mask tile (computed beforehand on the
//    device) lets all-false tiles be skipped and all-true tiles run without mask reads;
//    causal tiles above the diagonal are never visited.
#pragma once
#include <algorithm>
#include <type_traits>

#include "rs_device.hpp"

namespace rs {

template <typename T>
struct FwdCfg {
  static constexpr int BM = sizeof(T) == 4 ? 128 : 256;  // query rows per workgroup
  static constexpr int BN = sizeof(T) == 4 ? 32 : 64;    // keys per LDS tile
  static constexpr int NT = 2 * BM;                      // threads: one wave per 32 rows
};

constexpr float kRescaleLog2 = 8.f;  // rescale when a row max grows by more than 2^8

// Row-sum of eight rounded probabilities (one fragment) into acc.
__device__ inline float frag_sum(bf16x8 f, float acc) {
  typedef __bf16 v2 __attribute__((ext_vector_type(2)));
  const v2 one = {(__bf16)1.0f, (__bf16)1.0f};
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    v2 x = {f[2 * e], f[2 * e + 1]};
    acc = __builtin_amdgcn_fdot2_f32_bf16(x, one, acc, false);
  }
  return acc;
}
__device__ inline float frag_sum(f16x8 f, float acc) {
  typedef _Float16 v2 __attribute__((ext_vector_type(2)));
  const v2 one = {(_Float16)1.0f, (_Float16)1.0f};
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    v2 x = {f[2 * e], f[2 * e + 1]};
    acc = __builtin_amdgcn_fdot2(x, one, acc, false);
  }
  return acc;
}

constexpr int kMaxStateTiles = kMaxBoolMaskSeq / 32;  // key tiles (32 keys or more) of a bool-masked call
constexpr int QK_AHEAD = 4;  // K' fragment reads kept in flight ahead of the QK^T products
constexpr int PV_AHEAD = 3;  // V^T fragments (two reads each) in flight ahead of the P.V products

// QI8: blockwise quantized variant; Q'K'^T runs on int8 MFMA with exact int32 sums, scaled
// into the fp32 scores once per tile.  QI8 & 3 = 1: the rotated Q' and K' are quantized
// here, per (b, h, 64-token block), to codes with one fp32 scale: Q once per workgroup from
// its own four 64-row blocks, K per 64-key tile (one tile is one block) with the tile's amax
// reduced over the workgroup through LDS; no code reaches memory.  QI8 & 3 = 2: the codes
// and scales come from the quantizer pass (quant_kernel) and K code tiles go straight into
// LDS.  QI8 & 4: int4 codes (range [-7, 7], one per byte; CDNA4 has no int4 matrix
// instruction, and such codes are exact int8 operands), else int8 codes ([-127, 127]).
// QEXP (with QI8 & 3 = 1): code export mode for tests, which writes the codes and scales
// instead of the output.
// ROPE = false: plain attention, Q and K used as given (no tables read, no rotation).
// QKM: the Q/K prologue.  Bit 0: Q is RMS-normalized over the head dimension (weights
// p.qnw) before its rotation; bit 1: Q is stored in fp32 while V, O and the matrix products
// are in T (the autocast layout of flux-style attention); bit 2: K arrives already
// normalized and rotated, in T (kprep_kernel's output), so the key loop reads no tables.
template <typename T, int D, int MASK, bool CAUSAL, int QI8 = 0, bool ROPE = true, bool QEXP = false, int QKM = 0>
__global__ __launch_bounds__(FwdCfg<T>::NT, 1) void fwd_kernel(FwdParams p) {
  static_assert(!QI8 || sizeof(T) == 2, "quantized variant: 16-bit inputs");
  static_assert(ROPE || !QI8, "the int8 variant rotates");
  constexpr int QM = QI8 & 3;                     // 1: quantized here, 2: codes from the quantizer pass
  constexpr float QMAX = (QI8 & 4) ? 7.f : 127.f;  // code range: int4 or int8
  static_assert(!QEXP || QM == 1, "code export is the in-kernel quantization mode");
  static_assert(QKM == 0 || (ROPE && !QI8 && (QKM & 4)), "Q/K prologue: rotating path, K prepared");
  constexpr bool NORM = (QKM & 1) != 0;
  using TQ = typename std::conditional<(QKM & 2) != 0, float, T>::type;  // Q storage type
  static_assert((QKM & 2) == 0 || sizeof(T) == 2, "fp32 Q/K with 16-bit V");
  constexpr bool KROT = ROPE && (QKM & 4) == 0;  // K rotated in the key loop
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
  constexpr int VRB = D * ES;      // V row bytes in LDS (row-major, unpadded)
  constexpr int VBYTES = BN * VRB;
  constexpr int CPR = D / EPC;     // 16-byte chunks per V row
  constexpr int KCPT = BN * CPR / NT;  // 16-byte K chunks per thread and tile
  static_assert(KCPT * NT == BN * CPR, "K tile split");
  constexpr int NW = NT / 64;
  constexpr int VLD = VBYTES / 1024 / NW;  // direct-to-LDS V loads per wave (1 KB each)
  // int8 K' tiles: BN rows of D code bytes, 16-byte chunks XOR-swizzled per row
  constexpr int NQ8 = D / 32;              // k-steps of the int8 product (32 codes each)
  constexpr int K8CH = D / 16;             // 16-byte chunks per code row
  constexpr int K8RPB = 256 / D;           // code rows per 256-byte bank sweep
  constexpr int K8LD = BN * D / 1024;      // 1 KB direct-to-LDS loads per code tile
  static_assert(!QI8 || BN == 64, "int8 tiles coincide with the 64-token quantization blocks");
  static_assert(VLD * NW * 1024 == VBYTES, "V tile split");

  // Separate LDS objects per buffer: the compiler can then tell that reads of one V buffer
  // do not depend on the direct-to-LDS loads in flight into the other.
  __shared__ __attribute__((aligned(16))) char sk0[KBYTES];
  __shared__ __attribute__((aligned(16))) char sk1[KBYTES];
  __shared__ __attribute__((aligned(16))) char sv0[VBYTES];
  __shared__ __attribute__((aligned(16))) char sv1[VBYTES];
  // additive masks in the input's 16-bit dtype: the [BM x BN] mask tile goes straight into
  // LDS with the K/V tile (rows of BN * 2 bytes, 16-byte chunks swizzled per row)
  // MASK_ADD_TILE: an additive mask whose [BM x BN] tiles go straight into LDS with the K/V
  // tiles (the launcher picks it when the mask is in the input's 16-bit dtype, broadcast over
  // neither queries nor keys, S % 8 == 0 and a slice fits a buffer descriptor); MASK_ADD reads
  // the mask from memory where it is applied.  Separate instantiations keep the registers of
  // one path out of the other.
  constexpr bool kMaskTileLds = MASK == MASK_ADD_TILE;
  // additive masks: the running max is subtracted where the mask is added (one more vector
  // operation per score) instead of entering through the accumulator, which frees the 16
  // registers of that accumulator image
  constexpr bool kAddMask = MASK == MASK_ADD || MASK == MASK_ADD_TILE;
  static_assert(!kMaskTileLds || ES == 2, "mask tiles in LDS: 16-bit inputs");
  constexpr int MROW = BN * 2, MBYTES = kMaskTileLds ? BM * MROW : 16;
  __shared__ __attribute__((aligned(16))) char sm0[MBYTES];
  __shared__ __attribute__((aligned(16))) char sm1[MBYTES];

  if (p.gate_mode != 0) {  // bool mask: run only if this is the right kernel for the mask
    const unsigned some_excluded = __builtin_amdgcn_readfirstlane(p.gate[0]);
    if ((some_excluded == 0u) != (p.gate_mode == 1)) return;
  }
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r = lane & 31, hh = lane >> 5;
  const int S = p.shp.S;
  const float c2 = p.shp.scale_log2;

  // ---- work decomposition ----------------------------------------------------------------
  // A unit is one (b, h, query tile) over all its key tiles.  Without split, workgroup w
  // runs unit w.  With split (no causal; bool masks may skip all-false key tiles, so their
  // pieces can be shorter than planned, or empty: an empty piece writes O = 0 and LSE = -inf,
  // which the merge weighs as zero), the first
  // split_full workgroups run one whole unit each and the remaining units' (unit, key tile)
  // iterations are cut into split_grid equal contiguous ranges, one per further workgroup
  // (these start as the whole units finish, so the cut units' work is spread over the whole
  // GPU instead of leaving it part-idle in a last round); a unit cut between workgroups is
  // processed as pieces, each writing its normalized output and row log-sum-exp to a slot,
  // which fwd_merge_kernel then combines.
  const int nkt_all = (S + BN - 1) / BN;
  constexpr bool kCanSplit = !CAUSAL;

  // one piece: key tiles [t0, t1) of unit `item` (t1 < 0: the unit's whole range); a cut
  // piece writes to slot `slot` (workgroup w of the ranges owns slots 2w and 2w + 1)
  auto piece = [&](const int item, const int t0, const int t1, const int slot) __attribute__((always_inline)) {
  int qt = item % p.num_qt;
  const int bh = item / p.num_qt;
  const int hd = bh % p.shp.H, b = bh / p.shp.H;
  if (CAUSAL) qt = p.num_qt - 1 - qt;  // longest rows first
  const int q0 = qt * BM;
  const int m = q0 + wave * 32 + r;
  const int mc = m < S ? m : S - 1;

  const int hk = hd / p.shp.group;  // K/V head (grouped-query attention)
  const TQ* qbase = (const TQ*)p.q.ptr + b * p.q.sb + hd * p.q.sh;
  const T* kbase = (const T*)p.k.ptr + b * p.k.sb + hk * p.k.sh;
  const T* vbase = (const T*)p.v.ptr + b * p.v.sb + hk * p.v.sh;
  const float* tab = p.tab.ptr + b * p.tab.sb;  // float2 pairs, row stride D/2 pairs = D floats

  // ---- Q: load, rotate in fp32, scale by scale*log2(e), round, keep as B fragments --------
  // (int8 variant: rotated, quantized with the amax of its 64-row block, kept as codes; the
  // scales enter once per tile)
  using QF = typename std::conditional<QI8 != 0, i32x4[NQ8], frag[NQK]>::type;
  QF qf;
  float q8scale = 0.f;
  const int nblk = (S + 63) / 64;  // int8 quantization blocks of a (b, h) slice
  if constexpr (QM == 2) {
    const int slice = b * p.shp.H + hd;  // (b, h) index into the codes and scales
    const int8_t* qrow = p.qc + ((int64_t)slice * p.sp + mc) * D;
#pragma unroll
    for (int t = 0; t < NQ8; ++t) qf[t] = *(const i32x4*)(qrow + 32 * t + 16 * hh);
    q8scale = p.qsc[(int64_t)slice * (p.sp / 64) + mc / 64] * c2;  // mc < S: always a valid block
  } else if constexpr (QM == 1) {
    // this lane holds elements 32t + 16hh + e (e < 16) of row mc, rotated with every product
    // and sum rounded to fp32 (the quantizer's integer decisions are then reproducible)
    const T* qrow = qbase + (int64_t)mc * p.q.ss;
    const float* trow = tab + (int64_t)mc * D;
    float qv[NQ8][16];
    float amx = 0.f;
#pragma unroll
    for (int t = 0; t < NQ8; ++t) {
      const int d0 = 32 * t + 16 * hh;
      typedef T v8 __attribute__((ext_vector_type(8)));
      const v8 xa = *(const v8*)(qrow + d0), xb = *(const v8*)(qrow + d0 + 8);
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const float4 cs = *(const float4*)(trow + d0 + 4 * u);  // pairs (d0 + 4u) / 2 + {0, 1}
#pragma unroll
        for (int w2 = 0; w2 < 2; ++w2) {
          const int e = 4 * u + 2 * w2;
          const float x0 = to_f(e < 8 ? xa[e] : xb[e - 8]), x1 = to_f(e < 8 ? xa[e + 1] : xb[e - 7]);
          const float2 rr = rot_pair(x0, x1, w2 ? cs.z : cs.x, w2 ? cs.w : cs.y);
          qv[t][e] = rr.x;
          qv[t][e + 1] = rr.y;
          amx = fmaxf(amx, fmaxf(fabsf(rr.x), fabsf(rr.y)));
        }
      }
    }
    if (m >= S) amx = 0.f;  // a block's amax is over its valid rows
    amx = wave_max_nonneg(amx);
    // a 64-row block is the 32 rows of waves 2j and 2j + 1
    __shared__ float s_qamax[NW];
    if (lane == 0) s_qamax[wave] = amx;
    __syncthreads();
    const float am = fmaxf(s_qamax[wave & ~1], s_qamax[wave | 1]);
    const float inv = am > 0.f ? QMAX / am : 0.f;
    const float qsc = am > 0.f ? am / QMAX : 0.f;
#pragma unroll
    for (int t = 0; t < NQ8; ++t) {
      uint32_t wv[4] = {0u, 0u, 0u, 0u};
#pragma unroll
      for (int e = 0; e < 16; ++e) wv[e >> 2] |= (quant_bits(qv[t][e], inv) & 0xffu) << (8 * (e & 3));
      qf[t] = i32x4{(int)wv[0], (int)wv[1], (int)wv[2], (int)wv[3]};
    }
    q8scale = qsc * c2;
    if constexpr (QEXP) {
      if (m < S) {
        int8_t* crow = p.xq_codes + (((int64_t)b * p.shp.H + hd) * S + m) * D;
#pragma unroll
        for (int t = 0; t < NQ8; ++t) *(i32x4*)(crow + 32 * t + 16 * hh) = qf[t];
      }
      const int row0 = q0 + 32 * wave;
      if (lane == 0 && (wave & 1) == 0 && row0 < S)
        p.xq_scales[((int64_t)b * p.shp.H + hd) * nblk + row0 / 64] = qsc;
    }
  } else {
    const TQ* qrow = qbase + (int64_t)mc * p.q.ss;
    const float* trow = tab + (int64_t)mc * D;
    if constexpr (KPL == 8) {
      // this lane holds elements t * 16 + hh * 8 + e of its row, the partner lane (the other
      // half of the wave) the rest
      float xq[NQK][8];
#pragma unroll
      for (int t = 0; t < NQK; ++t) {
        const int d0 = t * 16 + hh * 8;
        if constexpr (sizeof(TQ) == 4) {
          const float4 a = *(const float4*)(qrow + d0), c = *(const float4*)(qrow + d0 + 4);
          xq[t][0] = a.x; xq[t][1] = a.y; xq[t][2] = a.z; xq[t][3] = a.w;
          xq[t][4] = c.x; xq[t][5] = c.y; xq[t][6] = c.z; xq[t][7] = c.w;
        } else {
          typedef T v8 __attribute__((ext_vector_type(8)));
          const v8 x = *(const v8*)(qrow + d0);
#pragma unroll
          for (int e = 0; e < 8; ++e) xq[t][e] = to_f(x[e]);
        }
      }
      if constexpr (NORM) {  // x / sqrt(mean x^2 + eps) * w over the whole row
        float ssq = 0.f;
#pragma unroll
        for (int t = 0; t < NQK; ++t)
#pragma unroll
          for (int e = 0; e < 8; ++e) ssq = fmaf(xq[t][e], xq[t][e], ssq);
        ssq = xhalf_sum(ssq);
        const float inv = 1.f / __builtin_sqrtf(ssq * (1.f / D) + p.norm_eps);
#pragma unroll
        for (int t = 0; t < NQK; ++t) {
          const int d0 = t * 16 + hh * 8;
          const float4 wa = *(const float4*)(p.qnw + d0), wb = *(const float4*)(p.qnw + d0 + 4);
          const float wv[8] = {wa.x, wa.y, wa.z, wa.w, wb.x, wb.y, wb.z, wb.w};
#pragma unroll
          for (int e = 0; e < 8; ++e) xq[t][e] = xq[t][e] * inv * wv[e];
        }
      }
#pragma unroll
      for (int t = 0; t < NQK; ++t) {
        const int d0 = t * 16 + hh * 8;
        if constexpr (!ROPE) {
#pragma unroll
          for (int e = 0; e < 8; ++e) qf[t][e] = from_f<T>(xq[t][e] * c2);
          continue;
        }
        const float4 cs0 = *(const float4*)(trow + d0);      // pairs d0/2, d0/2+1
        const float4 cs1 = *(const float4*)(trow + d0 + 4);  // pairs d0/2+2, d0/2+3
        const float cc[4] = {cs0.x, cs0.z, cs1.x, cs1.z};
        const float ss[4] = {cs0.y, cs0.w, cs1.y, cs1.w};
#pragma unroll
        for (int pp = 0; pp < 4; ++pp) {
          float2 rr = rot_pair_fma(xq[t][2 * pp], xq[t][2 * pp + 1], cc[pp], ss[pp]);
          qf[t][2 * pp] = from_f<T>(rr.x * c2);
          qf[t][2 * pp + 1] = from_f<T>(rr.y * c2);
        }
      }
    } else {
      // fp32: every lane reads its whole row (element d = 2t + hh of pair t is its own)
      float inv = 1.f;
      if constexpr (NORM) {
        float ssq = 0.f;
#pragma unroll
        for (int t = 0; t < NQK; ++t) {
          const float2 x = *(const float2*)(qrow + 2 * t);
          ssq = fmaf(x.x, x.x, fmaf(x.y, x.y, ssq));
        }
        inv = 1.f / __builtin_sqrtf(ssq * (1.f / D) + p.norm_eps);
      }
#pragma unroll
      for (int t = 0; t < NQK; ++t) {  // element d = 2t + hh of pair t
        float2 x = *(const float2*)(qrow + 2 * t);
        if constexpr (NORM) {
          const float2 wq = *(const float2*)(p.qnw + 2 * t);
          x.x = x.x * inv * wq.x;
          x.y = x.y * inv * wq.y;
        }
        if constexpr (!ROPE) {
          qf[t] = (hh ? x.y : x.x) * c2;
          continue;
        }
        const float2 cs = *(const float2*)(trow + 2 * t);
        const float2 rr = rot_pair_fma(x.x, x.y, cs.x, cs.y);
        qf[t] = (hh ? rr.y : rr.x) * c2;
      }
    }
  }

  // ---- KV tile range -----------------------------------------------------------------------
  const int nkt = nkt_all;
  int kt_end = t1 >= 0 ? t1 : nkt;
  if (CAUSAL) {
    const int last_row = min(q0 + BM, S) - 1;
    kt_end = min(nkt, last_row / BN + 1);
  }
  // bool masks: per-tile states over 64x64 blocks; this workgroup covers BM/64 of them
  // along the queries.
  auto tile_state_mem = [&](int kt) __attribute__((always_inline)) -> uint32_t {
    const int kt64 = (kt * BN) / kMaskTile;
    const int bm = p.mask.t_sb ? b : 0, hm = p.mask.t_sh ? hd : 0;
    const int nq64 = (S + kMaskTile - 1) / kMaskTile;
    uint32_t st = 0;
    for (int u = 0; u < BM / kMaskTile; ++u) {
      const int q64 = (q0 / kMaskTile) + u;
      if (q64 < nq64) st |= mask_tile_state(p.mask, bm, hm, q64, kt64);
    }
    return st;
  };
  // the workgroup's combined tile states, gathered once into LDS (scalar loads in the loop
  // would make every wait for them also wait for all outstanding LDS reads)
  // (the host limits bool-masked sequences to kMaxStateTiles key tiles)
  __shared__ uint8_t s_tstate[MASK == MASK_BOOL ? kMaxStateTiles : 1];
  // and s_next[kt] = the first tile at or after kt that is not all-false (kt_end if none) in
  // bits 0-13, with that tile's state in bits 14-15: the key loop then finds its next tile and
  // its state with one LDS read instead of a scan.  Wave 0 fills it in chunks of 64 tiles from
  // the end: a ballot of the chunk's non-skipped tiles gives each lane the next one at or
  // after it, and the chunk's first one carries to the chunk before.
  __shared__ uint16_t s_next[MASK == MASK_BOOL ? kMaxStateTiles : 1];
  if constexpr (MASK == MASK_BOOL) {
    for (int i = tid; i < kt_end; i += NT) s_tstate[i] = (uint8_t)tile_state_mem(i);
    __syncthreads();
    if (wave == 0) {
      int carry = kt_end;
      for (int c0 = kt_end > 0 ? ((kt_end - 1) / 64) * 64 : -64; c0 >= 0; c0 -= 64) {
        const int i = c0 + lane;
        const bool keep = i < kt_end && s_tstate[i] != TILE_ALL_FALSE;
        const uint64_t vm = __builtin_amdgcn_ballot_w64(keep);
        const uint64_t rest = vm >> lane;
        const int nx = rest ? i + (int)__builtin_ctzll(rest) : carry;
        if (i < kt_end) s_next[i] = (uint16_t)(nx | (nx < kt_end ? (int)s_tstate[nx] << 14 : 0));
        carry = vm ? c0 + (int)__builtin_ctzll(vm) : carry;
      }
    }
    __syncthreads();
  }
  // (the states are read from LDS, which the compiler takes for per-lane values: the
  // result, the same in every lane, is read from the first lane to keep it scalar)
  // (bool masks: the tile index and its state in bits 14-15; a tile at or past kt_end is
  // returned as it is, with state 0)
  auto next_tile = [&](int kt) __attribute__((always_inline)) -> int {
    if constexpr (MASK == MASK_BOOL) {
      if (kt < kt_end) kt = __builtin_amdgcn_readfirstlane((int)s_next[kt]);
    }
    return kt;
  };
  // index and state parts of next_tile's result (other masks: the index alone, any size)
  auto tile_idx = [](int v) __attribute__((always_inline)) -> int { return MASK == MASK_BOOL ? v & 0x3fff : v; };
  auto tile_st = [](int v) __attribute__((always_inline)) -> uint32_t { return MASK == MASK_BOOL ? (uint32_t)v >> 14 : 0u; };

  // ---- global -> register staging of one KV tile ------------------------------------------
  uint4 kx[KCPT];
  float4 kt4[KCPT][EPC / 4];
  // tile-relative element offsets of this thread's K chunks (the tile base is uniform and
  // stays in scalar registers)
  constexpr int KROWS_PER_IT = NT / CPR;  // K rows covered by one pass of all threads
  const int k_key0 = tid / CPR, k_cc = tid % CPR;
  const int k_off = k_key0 * (int)p.k.ss + k_cc * EPC;
  const int t_off = k_key0 * D + k_cc * EPC;
  // V goes straight from memory into a row-major LDS tile (buffer loads with an LDS
  // destination: lane i of a load writes bytes [16i, 16i+16) of a 1 KB block).  The byte
  // range check of the buffer turns rows at or past S into zeros.  16-byte chunks of row j
  // sit at chunk ^ vsw(j) so that the transposed reads below touch distinct banks.
  uint32_t v_voff[VLD];
#pragma unroll
  for (int i = 0; i < VLD; ++i) {
    const int byte = (wave * VLD + i) * 1024 + lane * 16;  // LDS byte within the V tile
    const int row = byte / VRB, pch = (byte % VRB) / 16;
    v_voff[i] = (uint32_t)(row * (int)p.v.ss * ES + ((pch ^ vsw<CPR>(row)) * 16));
  }

  // additive mask tiles (see sm0/sm1)
  const void* mbase = nullptr;
  auto msw = [](int row) __attribute__((always_inline)) { return (row & 7) ^ ((row >> 3) & 1); };
  if constexpr (kMaskTileLds) {
    // (S % 8 == 0: every 16-byte chunk of a valid key run lies inside the mask's last row)
    const int bm = p.mask.sb ? b : 0, hm = p.mask.sh ? hd : 0;
    mbase = mask_row_ptr(p.mask, bm, hm, 0, 2);
  }
  // The 1 KB load i of wave w covers tile rows 32w + 8i + lane/8, 16-byte chunk lane % 8 of
  // each: the swizzled chunk is (lane % 8) ^ (lane / 8) ^ (i & 1), so a lane's offset is one
  // of two values (even or odd i) plus 8i rows (added to the per-lane offset, which the
  // descriptor's range check covers: rows at or past S read as zero).
  constexpr int ML = BM * MROW / 1024 / NW;
  static_assert(!kMaskTileLds || (MROW == 128 && ML * 1024 == 32 * MROW), "mask tile: 32 rows of 128 bytes per wave");
  uint32_t m_voff[2] = {0u, 0u};
  uint32_t m_lds = 0u;  // byte of this lane's 16-byte chunk 0 of its row, XOR-able with 16 (4kb + 2c)
  if constexpr (kMaskTileLds) {
    const int row = 32 * wave + (lane >> 3);
    const int rstride = (int)p.mask.sq * 2;
#pragma unroll
    for (int par = 0; par < 2; ++par)
      m_voff[par] = (uint32_t)(row * rstride + ((((lane & 7) ^ (lane >> 3)) ^ par) << 4));
    const int rl = 32 * wave + r;
    m_lds = (uint32_t)(rl * MROW + ((hh ^ msw(rl)) << 4));
  }
  auto dma_mask = [&](int kt, char* sM) __attribute__((always_inline)) {
    if constexpr (kMaskTileLds) {
      const int rstride = (int)p.mask.sq * 2;
      const __amdgpu_buffer_rsrc_t rs =
          rows_rsrc((const char*)mbase + kt * BN * 2, q0, S, rstride, (S - kt * BN) * 2);
#pragma unroll
      for (int i = 0; i < ML; ++i)
        buffer_load_lds16(rs, sM + (wave * ML + i) * 1024, m_voff[i & 1] + (uint32_t)(8 * i * rstride), 0);
    }
  };

  // K of tile kt and its table rows into registers, through buffer descriptors: rows at or
  // past S read as zeros, and every call issues the same loads (so the wait for them can
  // let later loads stay in flight)
  auto load_k_rows = [&](int kt) __attribute__((always_inline)) {
    if constexpr (QM == 2) return;
    const __amdgpu_buffer_rsrc_t krs = rows_rsrc(kbase, kt * BN, S, (int)p.k.ss * ES, D * ES);
#pragma unroll
    for (int it = 0; it < KCPT; ++it)
      kx[it] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                                             krs, (uint32_t)((k_off + it * KROWS_PER_IT * (int)p.k.ss) * ES), 0, 0));
  };
  auto load_k_tab = [&](int kt) __attribute__((always_inline)) {
    if constexpr (!KROT || QM == 2) return;
    const __amdgpu_buffer_rsrc_t trs = rows_rsrc(tab, kt * BN, S, D * 4, D * 4);
#pragma unroll
    for (int it = 0; it < KCPT; ++it)
#pragma unroll
      for (int u = 0; u < EPC / 4; ++u)
        kt4[it][u] = __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(
                                                    trs, (uint32_t)((t_off + it * KROWS_PER_IT * D + 4 * u) * 4), 0, 0));
  };
  auto load_k = [&](int kt) __attribute__((always_inline)) {
    load_k_rows(kt);
    load_k_tab(kt);
  };

  // this wave's share of V of tile kt straight into the LDS buffer sV
  auto dma_v = [&](int kt, char* sV) __attribute__((always_inline)) {
    const __amdgpu_buffer_rsrc_t rs = rows_rsrc(vbase, kt * BN, S, (int)p.v.ss * ES, D * ES);
#pragma unroll
    for (int i = 0; i < VLD; ++i) buffer_load_lds16(rs, sV + (wave * VLD + i) * 1024, v_voff[i], 0);
  };

  // int8 variant: the K' code tile in LDS.  LDS row j holds key perm_row(j) (the row order
  // the score fragments need, as for the rotated K' tiles), its 16-byte chunk c (codes
  // 16c .. 16c + 15) at c ^ k8sw(j).
  auto k8sw = [](int row) __attribute__((always_inline)) { return (row / K8RPB) & (K8CH - 1); };
  // the amax of the K tile being quantized, one value per wave; two slots, alternating with
  // the destination buffer, so that a wave writing the next tile's slot never overtakes one
  // still reading the previous tile's
  __shared__ float s_kamax[QI8 ? 2 : 1][NW];
  const int hk_export = QEXP && qt == 0 && hd % p.shp.group == 0;  // one writer per (b, K/V head)
  // codes from the quantizer pass: this wave's 1 KB share of a code tile straight into LDS
  // (code rows past the padded sequence read as zero)
  const int slice_k = b * p.shp.Hkv + hk;  // (b, K/V head) index into the K codes and scales
  const int8_t* kcodes = QM == 2 ? p.kc + (int64_t)slice_k * p.sp * D : nullptr;
  uint32_t k8_voff = 0;
  if constexpr (QM == 2) {
    const int byte = wave * 1024 + lane * 16;
    const int row = byte / D, pch = (byte % D) / 16;
    k8_voff = (uint32_t)(perm_row(row) * D + ((pch ^ k8sw(row)) << 4));
  }
  auto dma_k = [&](int kt, char* sK) __attribute__((always_inline)) {
    if constexpr (QM == 2) {
      if (wave < K8LD)
        buffer_load_lds16(tile_rsrc(kcodes, (int64_t)kt * BN * D, (int64_t)p.sp * D), sK + wave * 1024, k8_voff, 0);
    }
  };

  // K' of the tile held in kx/kt4 into LDS buffer sK (tile kt: int8 export only).  int8
  // variant: rotate (fp32, rounded products), reduce the tile's amax over the workgroup,
  // quantize, store codes; returns the tile's scale (other variants: 0).
  auto store_tile = [&](char* sK, int kt) __attribute__((always_inline)) -> float {
    if constexpr (QM == 2) return kt < nkt_all ? p.ksc[(int64_t)slice_k * (p.sp / 64) + kt] : 0.f;
    if constexpr (QM == 1) {
      float kv[KCPT][8];
      float amx = 0.f;
#pragma unroll
      for (int it = 0; it < KCPT; ++it) {
        const float* tf = (const float*)&kt4[it][0];
        typedef T v8 __attribute__((ext_vector_type(8)));
        const v8 x = *(const v8*)&kx[it];
#pragma unroll
        for (int pp = 0; pp < 4; ++pp) {
          const float2 rr = rot_pair(to_f(x[2 * pp]), to_f(x[2 * pp + 1]), tf[2 * pp], tf[2 * pp + 1]);
          kv[it][2 * pp] = rr.x;
          kv[it][2 * pp + 1] = rr.y;
          amx = fmaxf(amx, fmaxf(fabsf(rr.x), fabsf(rr.y)));  // rows past S were read as zeros
        }
      }
      amx = wave_max_nonneg(amx);
      const int slot = sK == sk0 ? 0 : 1;
      if (lane == 0) s_kamax[slot][wave] = amx;
      __syncthreads();
      float am = s_kamax[slot][0];
#pragma unroll
      for (int w2 = 1; w2 < NW; ++w2) am = fmaxf(am, s_kamax[slot][w2]);
      const float inv = am > 0.f ? QMAX / am : 0.f;
#pragma unroll
      for (int it = 0; it < KCPT; ++it) {
        uint32_t wv[2] = {0u, 0u};
#pragma unroll
        for (int e = 0; e < 8; ++e) wv[e >> 2] |= (quant_bits(kv[it][e], inv) & 0xffu) << (8 * (e & 3));
        const int key = k_key0 + it * KROWS_PER_IT, lrow = perm_row(key);
        *(uint2*)(sK + lrow * D + (((k_cc >> 1) ^ k8sw(lrow)) << 4) + (k_cc & 1) * 8) = make_uint2(wv[0], wv[1]);
        if constexpr (QEXP) {
          const int j = kt * BN + key;
          if (hk_export && kt < nkt_all && j < S)
            *(uint2*)(p.xk_codes + (((int64_t)b * p.shp.Hkv + hk) * S + j) * D + k_cc * 8) = make_uint2(wv[0], wv[1]);
        }
      }
      const float ksc = am > 0.f ? am / QMAX : 0.f;
      if constexpr (QEXP) {
        if (hk_export && kt < nkt_all && tid == 0) p.xk_scales[((int64_t)b * p.shp.Hkv + hk) * nblk + kt] = ksc;
      }
      return ksc;
    }
#pragma unroll
    for (int it = 0; it < KCPT; ++it) {
      const float* tf = (const float*)&kt4[it][0];  // (c, s) per pair
      uint4 outw;
      if constexpr (!KROT) {
        outw = kx[it];
      } else if constexpr (ES == 2) {
        typedef T v8 __attribute__((ext_vector_type(8)));
        v8 x = *(const v8*)&kx[it];
        v8 y;
#pragma unroll
        for (int pp = 0; pp < 4; ++pp) {
          float2 rr = rot_pair_fma(to_f(x[2 * pp]), to_f(x[2 * pp + 1]), tf[2 * pp], tf[2 * pp + 1]);
          y[2 * pp] = from_f<T>(rr.x);
          y[2 * pp + 1] = from_f<T>(rr.y);
        }
        outw = *(const uint4*)&y;
      } else {
        const float* x = (const float*)&kx[it];
        float y[4];
#pragma unroll
        for (int pp = 0; pp < 2; ++pp) {
          float2 rr = rot_pair_fma(x[2 * pp], x[2 * pp + 1], tf[2 * pp], tf[2 * pp + 1]);
          y[2 * pp] = rr.x;
          y[2 * pp + 1] = rr.y;
        }
        outw = *(const uint4*)y;
      }
      *(uint4*)(sK + perm_row(k_key0 + it * KROWS_PER_IT) * KP + k_cc * 16) = outw;
    }
    return 0.f;
  };

  // ---- online softmax state ----------------------------------------------------------------
  f32x16 oacc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) oacc[db] = zero16();
  float m_run = -INFINITY;  // running row max, log2 units
  float m_base = 0.f;       // value subtracted inside the S product (negm = -m_base)
  float l_run = 0.f;        // this lane's partial row sum
  f32x16 negm = zero16();

  // per-lane constant parts of the LDS addresses
  const int k_rd = r * KP + hh * KPL * ES;  // K' A-fragment: row r of each 32-key block
  // V^T A-fragments from the row-major V tile.  bf16/fp16: a transposed 8-byte read by each
  // 16-lane group G hands lane l the 4 keys key0..key0+3 at column 32db + (l % 32), when
  // source lane s of the group points at row key0 + s/4, columns +4(s%4)..+3 of that
  // column block; two reads (keys +0..3, +4..7) make one 8-key fragment.
  const int ls = lane & 15, G = lane >> 4;
  const int v_row_l = 8 * (G >> 1) + (ls >> 2);       // + 32kb + 16c + 4q
  const int v_colb = 2 * (16 * (G & 1) + 4 * (ls & 3));  // byte column within a 64-byte d-block
  int v_rd[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) {
    const int chunk = (db * 64 + v_colb) / 16;
    v_rd[db] = v_row_l * VRB + ((chunk ^ vsw<CPR>(v_row_l)) * 16) + (v_colb & 15);
  }

  // S^T - m_base = K' Q'^T + C for one tile: rows = keys, columns = this wave's 32 queries.
  // (int8 variant: exact integer sums per 32-key block, turned into scores right away with
  // the tile's K scale ksc: s = sum * scale_q * scale_k * scale * log2(e) - m_base.)
  auto qk = [&](const char* sK, f32x16* sacc, float ksc) __attribute__((always_inline)) {
    if constexpr (QI8) {
      const float f = q8scale * ksc;
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        i32x4 ka[NQ8];
        const int row = 32 * kb + r;
#pragma unroll
        for (int t = 0; t < NQ8; ++t)
          ka[t] = *(const i32x4*)(sK + row * D + (((2 * t + hh) ^ k8sw(row)) << 4));
        i32x16 ia = izero16();
#pragma unroll
        for (int t = 0; t < NQ8; ++t) ia = __builtin_amdgcn_mfma_i32_32x32x32_i8(ka[t], qf[t], ia, 0, 0, 0);
#pragma unroll
        for (int i = 0; i < 16; ++i) sacc[kb][i] = kAddMask ? (float)ia[i] * f : fmaf((float)ia[i], f, -m_base);
      }
    } else {
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        frag ka[NQK];
#pragma unroll
        for (int t = 0; t < NQK; ++t) ka[t] = *(const frag*)(sK + k_rd + (32 * kb) * KP + t * KSTEP * ES);
#pragma unroll
        for (int t = 0; t < NQK; ++t) sacc[kb] = M::mma(ka[t], qf[t], t == 0 ? (kAddMask ? zero16() : negm) : sacc[kb]);
      }
    }
  };

  // exclusions of one tile: sequence tail, causal diagonal, masks
  // (bool masks: st = the tile's state, carried with its index from the lookup)
  auto fixup = [&](int kt, uint32_t st_in, f32x16* sacc, const char* sM) __attribute__((always_inline)) {
    const int kv0 = kt * BN;
    const bool tail = kv0 + BN > S;
    const bool diag = CAUSAL && (kv0 + BN - 1 > q0);
    uint32_t st = TILE_ALL_TRUE;
    if constexpr (MASK == MASK_BOOL) st = st_in;
    if constexpr (MASK == MASK_ADD || MASK == MASK_ADD_TILE) {
      if constexpr (kMaskTileLds) {
        // row 32 wave + r of the tile, keys 32kb + 16c + 8hh .. +7 = logical chunk 4kb + 2c + hh,
        // stored at chunk (4kb + 2c + hh) ^ msw(row): m_lds ^ 16 (4kb + 2c)
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
          for (int c = 0; c < 2; ++c) {
            typedef T v8 __attribute__((ext_vector_type(8)));
            const v8 mv = *(const v8*)(sM + (m_lds ^ (uint32_t)(16 * (4 * kb + 2 * c))));
#pragma unroll
            for (int e = 0; e < 8; ++e) sacc[kb][8 * c + e] = fmaf(to_f(mv[e]), kLog2eF, sacc[kb][8 * c + e]) - m_base;
          }
        }
      } else {
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
            for (int e = 0; e < 8; ++e) sacc[kb][8 * c + e] = fmaf(mv[e], kLog2eF, sacc[kb][8 * c + e]) - m_base;
          }
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
  };

  // lazy online softmax, part 1: the tile's row max (mx, log2 units relative to m_base) and
  // whether some row max grows by more than 2^8 (wave-uniform); only then is m rescaled
  auto check = [&](const f32x16* sacc, float& mx) __attribute__((always_inline)) -> bool {
    float x = sacc[0][0];
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int i = (kb == 0 ? 1 : 0); i < 16; ++i) x = fmaxf(x, sacc[kb][i]);
    x = xhalf_max(x);
    mx = x;
    return __builtin_amdgcn_ballot_w64(x > (m_run - m_base) + kRescaleLog2) != 0;
  };
  auto rescale = [&](f32x16* sacc, float mx) __attribute__((always_inline)) {
    const float m_new = fmaxf(m_run, mx + m_base);
    const bool dead = m_new == -INFINITY;  // no attended key so far
    const float alpha = dead ? 1.f : fast_exp2(m_run - m_new);
    const float shift = dead ? 0.f : m_new - m_base;
    l_run *= alpha;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int i = 0; i < 16; ++i) oacc[db][i] *= alpha;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) sacc[kb][i] -= shift;
    m_run = m_new;
    m_base = dead ? 0.f : m_new;
#pragma unroll
    for (int i = 0; i < 16; ++i) negm[i] = -m_base;
  };

  // part 2: P = exp2(S), rounded to T into MFMA fragments for 16-bit types, and row sums
  using PT = typename std::conditional<KPL == 8, frag[NKB][2], f32x16[NKB]>::type;
  auto probs = [&](f32x16* sacc, PT& pt) __attribute__((always_inline)) {
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) sacc[kb][i] = fast_exp2(sacc[kb][i]);
    if constexpr (KPL == 8) {
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int c = 0; c < 2; ++c) {
#pragma unroll
          for (int e = 0; e < 8; ++e) pt[kb][c][e] = from_f<T>(sacc[kb][8 * c + e]);
          l_run = frag_sum(pt[kb][c], l_run);
        }
    } else {
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
        for (int i = 0; i < 16; ++i) l_run += sacc[kb][i];
        pt[kb] = sacc[kb];
      }
    }
  };

  // O^T += V^T P^T
  auto pv = [&](const char* sV, PT& pt) __attribute__((always_inline)) {
    if constexpr (KPL == 8) {
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
          for (int c = 0; c < 2; ++c) {
            // rows 32kb + 16c (+4 for the second half) keep (row & 3), so the swizzle term of
            // v_rd stays valid: only whole-row offsets are added
            typedef short s4 __attribute__((ext_vector_type(4)));
            const char* base = sV + v_rd[db] + (32 * kb + 16 * c) * VRB;
            const s4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s4*)base);
            const s4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s4*)(base + 4 * VRB));
            frag a;
            *(s4*)&a = lo;
            *((s4*)&a + 1) = hi;
            oacc[db] = M::mma(a, pt[kb][c], oacc[db]);
          }
      }
    } else {
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int key = 32 * kb + c_idx_sig(i, hh);
            const int col = 4 * (32 * db + r);  // byte column of element d = 32db + r
            const float a = *(const float*)(sV + key * VRB + (((col >> 4) ^ vsw<CPR>(key)) << 4) + (col & 15));
            oacc[db] = M::mma(a, pt[kb][i], oacc[db]);
          }
      }
    }
  };

  // ---- key-tile loop: software pipelined over the visiting order t_0 < t_1 < ... ----------
  // Iteration i:
  //   (rare) rescale for S(t_i), as its check decided;
  //   phase A: S(t_{i+1}) = K'(t_{i+1}) Q'^T on MFMA, interleaved with P(t_i) = exp2(S(t_i))
  //            and its row sums, and with the loads of K(t_{i+2}) into registers and of
  //            V(t_{i+1}) and the mask tile of t_{i+2} into LDS;
  //   phase B: O^T += V(t_i)^T P(t_i)^T on MFMA, interleaved with the rotation of K(t_{i+2})
  //            into LDS and the max check of S(t_{i+1}) (after its exclusions);
  //   wait for the loads issued, barrier.
  // Tile t_j uses buffer j & 1 of each pair (sk, sv, sm): phase A reads K' of t_{i+1} while
  // phase B writes K' of t_{i+2}; V of t_i is read while V of t_{i+1} arrives; the mask tile
  // of t_{i+1} is read while that of t_{i+2} arrives.  A wave's matrix and vector work thus
  // overlap whatever phase the other wave of its SIMD is in.
  f32x16 sacc[2][NKB];
  float mx = 0.f;     // row max of the current tile's scores (valid where need was computed)
  bool need = false;  // the current tile raises some row max by more than 2^8
  const int ktp = next_tile(t0);
  int kt = tile_idx(ktp);
  const int kt1p = kt < kt_end ? next_tile(kt + 1) : kt_end;
  int kt1 = tile_idx(kt1p);
  uint32_t st_t1 = tile_st(kt1p);  // bool masks: state of t_{i+1}
  // bool masks: the lookup of the tile after t_{i+1}, one step ahead
  int kt2p = kt1 < kt_end ? next_tile(kt1 + 1) : kt_end;
  float ks0 = 0.f, ks_t1 = 0.f;  // int8: K scales of tiles t_0 and t_{i+1}
  if (kt < kt_end) {
    load_k(kt);
    dma_k(kt, sk0);
    dma_v(kt, sv0);
    dma_mask(kt, sm0);
    ks0 = store_tile(sk0, kt);
    if (kt1 < kt_end) {
      load_k(kt1);
      dma_k(kt1, sk1);
      dma_mask(kt1, sm1);
      ks_t1 = store_tile(sk1, kt1);
    }
  }
  wait_vmem_and_sync();
  if (kt < kt_end) {
    qk(sk0, sacc[0], ks0);
    fixup(kt, tile_st(ktp), sacc[0], sm0);
    need = check(sacc[0], mx);
  }
  __syncthreads();  // sk0 and sm0 are refilled in the first iteration
  auto body = [&](auto stage_c) __attribute__((always_inline)) {
    constexpr int st = decltype(stage_c)::value;  // i & 1
    f32x16* s_cur = sacc[st];
    f32x16* s_nxt = sacc[st ^ 1];
    const char* sKr = st ? sk0 : sk1;  // K' of t_{i+1}
    char* sKw = st ? sk1 : sk0;        // K' of t_{i+2}
    const char* sVr = st ? sv1 : sv0;  // V of t_i
    char* sVw = st ? sv0 : sv1;        // V of t_{i+1}
    const char* sMr = st ? sm0 : sm1;  // mask tile of t_{i+1}
    char* sMw = st ? sm1 : sm0;        // mask tile of t_{i+2}
    if (need) rescale(s_cur, mx);
    const bool has1 = kt1 < kt_end;
    int kt2 = has1 ? next_tile(kt1 + 1) : kt_end;
    uint32_t st_t2 = 0u;
    int kt3_raw = 0;  // bool masks: lookup of the tile after t_{i+2}, made scalar after the barrier
    if constexpr (MASK == MASK_BOOL) {
      const int pk = has1 ? kt2p : kt_end;
      kt2 = tile_idx(pk);
      st_t2 = tile_st(pk);
      kt3_raw = kt2 + 1 < kt_end ? (int)s_next[min(kt2 + 1, kMaxStateTiles - 1)] : kt_end;
    }
    // issued whether or not t_{i+1} and t_{i+2} exist (tile kt_end then: in range or read
    // as zeros, into buffers that are not read again), so the counts of loads in flight are
    // the same on every path and the wait for K(t_{i+2}) leaves the V loads in flight; the
    // mask tile (additive masks in LDS) goes first, as it comes from memory rather than L2
    dma_mask(kt2, sMw);
    load_k(kt2);
    dma_v(kt1, sVw);
    dma_k(kt2, sKw);

    // phase A (one straight block: without t_{i+1} the products run on a stale K' buffer
    // and their result is ignored)
    PT pt;
    qk(sKr, s_nxt, ks_t1);
    probs(s_cur, pt);
    if constexpr (KPL == 8) {
      if constexpr (QM == 2) {
        sched_mfma_interleave<NKB * NQ8, 1, NKB * NQ8, 8, 0>();
      } else if constexpr (QM == 1) {
        sched_mfma_interleave_loads<NKB * NQ8, 1, NKB * NQ8, 8, 4, 0>();
      } else {
        sched_mfma_interleave_loads<NKB * NQK, 1, QK_AHEAD, 4, kMaskTileLds ? 6 : 2, 0>();
      }
      // keep P(t_i) and its row sums here: left alone, the compiler moves them next to
      // their use in phase B, out of the shadow of these products
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          i32x4 w = __builtin_bit_cast(i32x4, pt[kb][c]);
          asm volatile("" : "+v"(w));
          pt[kb][c] = __builtin_bit_cast(frag, w);
        }
      asm volatile("" : "+v"(l_run));
    }
    // (additive mask tiles: the compiler barrier keeps the mask reads of phase B from being
    // hoisted into phase A, where their registers would add to its peak)
    if constexpr (kMaskTileLds) asm volatile("" ::: "memory");
    // phase B
    if (has1) fixup(kt1, st_t1, s_nxt, sMr);
    pv(sVr, pt);
    // (stale registers when there is no t_{i+2}: the buffer is not read)
    const float ks_t2 = store_tile(sKw, kt2);
    need = check(s_nxt, mx) && has1;
    if constexpr (KPL == 8) sched_mfma_interleave<NDB * NKB * 2, 2, PV_AHEAD, 6, 1>();
    wait_vmem_and_sync();
    kt = kt1;
    kt1 = kt2;
    ks_t1 = ks_t2;
    if constexpr (MASK == MASK_BOOL) {
      st_t1 = st_t2;
      kt2p = __builtin_amdgcn_readfirstlane(kt3_raw);
    }
  };
  while (kt < kt_end) {
    body(std::integral_constant<int, 0>{});
    if (kt >= kt_end) break;
    body(std::integral_constant<int, 1>{});
  }

  // ---- epilogue ------------------------------------------------------------------------------
  // (a piece of a cut unit writes its normalized output and row log-sum-exp to its slot, in
  // the same form as a whole unit does; fwd_merge_kernel combines the pieces)
  const float l = xhalf_sum(l_run);
  const float inv_l = l > 0.f ? 1.f / l : 0.f;
  if (!QEXP && m < S) {  // (code export mode: no output)
    char* orow = slot >= 0 ? (char*)p.part_o + ((int64_t)slot * BM + (m - q0)) * D * ES
                           : (char*)p.o + ((int64_t)b * p.o_sb + (int64_t)hd * p.o_sh +
                                                 (int64_t)m * p.o_ss) * ES;
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
    float* lse = slot >= 0 ? p.part_lse + (int64_t)slot * BM + (m - q0)
                           : p.lse ? p.lse + ((int64_t)b * p.shp.H + hd) * S + m : nullptr;
    if (lse && hh == 0) {
      *lse = l > 0.f ? (m_run + __log2f(l)) * kLn2F : -INFINITY;
    }
  }
  };

  // pieces of this workgroup, one call site (the body is inlined once)
  int whole_unit = -1;  // >= 0: this workgroup runs that one unit whole
  int w = 0;
  int64_t it = 0, it_end = 0;
  const int64_t G = p.split_grid, W = p.split_iters;
  // causal: workgroup w runs two units of one head, query tiles num_qt - 1 - i and i (the
  // longest with the shortest), so that every workgroup has the same number of key tiles
  // whatever order the workgroups are placed on the CUs in
  int pair_b = -1;
  if constexpr (CAUSAL) {
    const int npairs = (p.num_qt + 1) / 2;
    const int itemp = xcd_remap(blockIdx.x, gridDim.x);
    const int bh = itemp / npairs, i = itemp % npairs;
    whole_unit = bh * p.num_qt + i;  // (the unit's query tile is num_qt - 1 - i, see piece)
    if (i != p.num_qt - 1 - i) pair_b = bh * p.num_qt + (p.num_qt - 1 - i);
  } else if (!kCanSplit || p.split_iters == 0) {
    whole_unit = xcd_remap(blockIdx.x, gridDim.x);
  } else if ((int)blockIdx.x < p.split_full) {
    whole_unit = xcd_remap(blockIdx.x, p.split_full);
  } else {
    // (split_full is a multiple of 8, so tail workgroup tw sits on XCD tw % 8 like the others)
    w = __builtin_amdgcn_readfirstlane(xcd_remap((int)blockIdx.x - p.split_full, p.split_grid));
    it = (int64_t)w * W / G;
    it_end = (int64_t)(w + 1) * W / G;
  }
  // (the piece coordinates are the same in every lane: read from the first lane they stay in
  // scalar registers, not in vector registers held through the whole piece)
  auto uni = [](int x) __attribute__((always_inline)) { return __builtin_amdgcn_readfirstlane(x); };
  for (int n = 0;; ++n) {
    int item, t0 = 0, t1 = -1, slot = -1;
    if (whole_unit >= 0) {
      if (n > 1 || (n == 1 && pair_b < 0)) break;
      item = n == 0 ? whole_unit : pair_b;
    } else {
      if (it >= it_end) break;
      const int u = uni((int)(it / nkt_all));
      t0 = uni((int)(it - (int64_t)u * nkt_all));
      const int te = uni((int)min((int64_t)nkt_all, t0 + (it_end - it)));
      item = p.split_full + u;
      if (t0 > 0 || te < nkt_all) {  // a cut piece: first one in slot 2w, a later one in 2w + 1
        t1 = te;
        slot = 2 * w + (n > 0 ? 1 : 0);
      }
      it += te - t0;
    }
    if (n > 0) __syncthreads();  // LDS of the previous piece
    piece(uni(item), uni(t0), uni(t1), uni(slot));
  }
}

// Combines the pieces of the cut units: per row, LSE = log sum_s exp(LSE_s) and
// O = sum_s exp(LSE_s - LSE) O_s over the pieces in range order (a fixed order: the result
// does not depend on timing).  One workgroup per (cut unit, 32 rows); 8 threads per row, 16
// elements of the head dimension each.  A unit has at most kMaxPieces pieces (the planner
// keeps at least 8 key tiles per range), so all loads of a row can be issued together.
constexpr int kMaxPieces = 4;
template <typename T, int D>
__global__ __launch_bounds__(256) void fwd_merge_kernel(FwdParams p) {
  constexpr int BM = FwdCfg<T>::BM;
  constexpr int PER = D / 8;  // elements per thread
  const int u = blockIdx.x / (BM / 32);
  const int r = (blockIdx.x % (BM / 32)) * 32 + (threadIdx.x >> 3), c = (threadIdx.x & 7) * PER;
  const int S = p.shp.S, nkt = (S + FwdCfg<T>::BN - 1) / FwdCfg<T>::BN;
  const int item = p.split_full + u;
  const int qt = item % p.num_qt, bh = item / p.num_qt;
  const int hd = bh % p.shp.H, b = bh / p.shp.H;
  const int m = qt * BM + r;
  if (m >= S) return;
  const int64_t G = p.split_grid, W = p.split_iters, u0 = (int64_t)u * nkt;
  const int w_lo = (int)(((u0 + 1) * G + W - 1) / W) - 1;
  const int w_hi = (int)(((u0 + nkt) * G + W - 1) / W) - 1;
  const int n = min(w_hi - w_lo + 1, kMaxPieces);
  int sl[kMaxPieces];
  float ls[kMaxPieces];
  typedef T vp __attribute__((ext_vector_type(PER)));
  vp o[kMaxPieces];
#pragma unroll
  for (int j = 0; j < kMaxPieces; ++j) {
    const int w = w_lo + j;
    sl[j] = 2 * w + ((int)(((int64_t)w * W / G) / nkt) == u ? 0 : 1);
    if (j < n) {
      ls[j] = p.part_lse[(int64_t)sl[j] * BM + r];
      o[j] = *(const vp*)((const T*)p.part_o + ((int64_t)sl[j] * BM + r) * D + c);
    } else {
      ls[j] = -INFINITY;
    }
  }
  float mx = -INFINITY;
#pragma unroll
  for (int j = 0; j < kMaxPieces; ++j) mx = fmaxf(mx, ls[j]);
  float acc[PER];
#pragma unroll
  for (int e = 0; e < PER; ++e) acc[e] = 0.f;
  float sum = 0.f;
  if (mx != -INFINITY) {
#pragma unroll
    for (int j = 0; j < kMaxPieces; ++j) {
      if (j >= n) break;
      const float f = __expf(ls[j] - mx);  // 0 for a piece with no attended key
      sum += f;
#pragma unroll
      for (int e = 0; e < PER; ++e) acc[e] = fmaf(f, to_f(o[j][e]), acc[e]);
    }
  }
  const float inv = sum > 0.f ? 1.f / sum : 0.f;
  vp outv;
#pragma unroll
  for (int e = 0; e < PER; ++e) outv[e] = from_f<T>(acc[e] * inv);
  *(vp*)((T*)p.o + (int64_t)b * p.o_sb + (int64_t)hd * p.o_sh + (int64_t)m * p.o_ss + c) = outv;
  if (p.lse && c == 0) p.lse[((int64_t)b * p.shp.H + hd) * S + m] = sum > 0.f ? mx + __logf(sum) : -INFINITY;
}

template <typename T, int D, int MASK, bool CAUSAL, int QI8 = 0, bool ROPE = true, bool QEXP = false, int QKM = 0>
static int launch_fwd_t(const FwdParams& p, void* stream) {
  const int grid = p.split_iters > 0 ? p.split_full + p.split_grid
                   : CAUSAL        ? (p.num_qt + 1) / 2 * p.shp.H * p.shp.B
                                   : p.num_qt * p.shp.H * p.shp.B;
  if (p.ev_start) (void)hipEventRecord((hipEvent_t)p.ev_start, (hipStream_t)stream);
  if constexpr (MASK == MASK_BOOL) {
    // an all-true bool mask runs the unmasked kernel (same schedule, same slots): decided on
    // the device by the gate word, with no host synchronisation
    FwdParams pn = p;
    pn.gate_mode = 1;
    hipLaunchKernelGGL((fwd_kernel<T, D, MASK_NONE, CAUSAL, QI8, ROPE, QEXP, QKM>), dim3(grid), dim3(FwdCfg<T>::NT), 0,
                       (hipStream_t)stream, pn);
    FwdParams pb = p;
    pb.gate_mode = 2;
    hipLaunchKernelGGL((fwd_kernel<T, D, MASK, CAUSAL, QI8, ROPE, QEXP, QKM>), dim3(grid), dim3(FwdCfg<T>::NT), 0,
                       (hipStream_t)stream, pb);
  } else {
    hipLaunchKernelGGL((fwd_kernel<T, D, MASK, CAUSAL, QI8, ROPE, QEXP, QKM>), dim3(grid), dim3(FwdCfg<T>::NT), 0,
                       (hipStream_t)stream, p);
  }
  if (p.ev_stop) (void)hipEventRecord((hipEvent_t)p.ev_stop, (hipStream_t)stream);
  if (p.split_iters > 0) {
    const int cut = p.num_qt * p.shp.H * p.shp.B - p.split_full;
    hipLaunchKernelGGL((fwd_merge_kernel<T, D>), dim3(cut * (FwdCfg<T>::BM / 32)), dim3(256), 0,
                       (hipStream_t)stream, p);
  }
  return (int)hipGetLastError();
}

template <typename T, int D, bool ROPE, int QI8 = 0>
static int launch_fwd_d(int mask_kind, bool causal, const FwdParams& p, void* stream) {
  if (causal) return launch_fwd_t<T, D, MASK_NONE, true, QI8, ROPE>(p, stream);
  switch (mask_kind) {
    case MASK_BOOL: return launch_fwd_t<T, D, MASK_BOOL, false, QI8, ROPE>(p, stream);
    case MASK_ADD:
      if constexpr (sizeof(T) == 2) {
        if (p.mask.dtype != F32 && !p.mask.key_bcast && p.mask.sq != 0 && p.shp.S % 8 == 0 &&
            p.mask.sq * 2 * FwdCfg<T>::BM < ((int64_t)1 << 31))
          return launch_fwd_t<T, D, MASK_ADD_TILE, false, QI8, ROPE>(p, stream);
      }
      return launch_fwd_t<T, D, MASK_ADD, false, QI8, ROPE>(p, stream);
    default: return launch_fwd_t<T, D, MASK_NONE, false, QI8, ROPE>(p, stream);
  }
}

template <typename T, bool ROPE>
static int launch_fwd_dt(int D, int mask_kind, bool causal, const FwdParams& p, void* stream) {
  return D == 64 ? launch_fwd_d<T, 64, ROPE>(mask_kind, causal, p, stream)
                 : launch_fwd_d<T, 128, ROPE>(mask_kind, causal, p, stream);
}

template <typename T, int QI8>
static int launch_fwd_q_d(int D, int mask_kind, bool causal, const FwdParams& p, void* stream) {
  return D == 64 ? launch_fwd_d<T, 64, true, QI8>(mask_kind, causal, p, stream)
                 : launch_fwd_d<T, 128, true, QI8>(mask_kind, causal, p, stream);
}


}  // namespace rs
