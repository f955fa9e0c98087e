// Internal parameter blocks shared by the host library and the gfx950 kernels.
// Nothing here is part of the public ABI (include/rope_sdpa.h is).
#pragma once
#include <stddef.h>
#include <stdint.h>

namespace rs {

enum DType : int { F32 = 0, F16 = 1, BF16 = 2, BOOL8 = 3 };
enum MaskKind : int { MASK_NONE = 0, MASK_BOOL = 1, MASK_ADD = 2 };
// Forward kernel only: an additive mask staged through LDS in tiles (chosen by the launcher).
constexpr int MASK_ADD_TILE = 3;

// Tile states of a bool mask over 64 x 64 (query x key) blocks: bit0 = some key attended,
// bit1 = some key excluded.  OR-ing states combines blocks.
enum : uint8_t { TILE_ALL_TRUE = 1, TILE_ALL_FALSE = 2, TILE_MIXED = 3 };
constexpr int kMaskTile = 64;
// Longest sequence accepted with a bool mask: the kernels keep the mask's tile states of a
// whole key (or query) range in LDS.
constexpr int kMaxBoolMaskSeq = 262144;

// A [B, H, S, D] operand: base pointer and element strides of dims 0..2 (dim 3 is contiguous).
struct Opnd {
  const void* ptr;
  int64_t sb, sh, ss;
};

// A mask as the kernels read it.  Strides are "effective": 0 on broadcast dimensions.
struct MaskView {
  const void* ptr;
  int64_t sb, sh, sq, sk;
  int dtype;  // BOOL8, F32, F16 or BF16
  int key_bcast;  // size[3] == 1
  // tile states (bool masks only): [nb][nh][nqt][nkt] uint8, dims follow the mask's own extents
  const uint8_t* tiles;
  int64_t t_sb, t_sh;  // 0 when broadcast over b / h
  int t_nqt, t_nkt;    // 1 when the mask is broadcast over queries / keys
};

struct AttnShape {
  int B, H, S;
  int Hkv, group;    // K/V heads and query heads per K/V head (grouped-query attention:
                     // query head h reads K/V head h / group); Hkv == H, group == 1 otherwise
  float scale;       // softmax scale
  float scale_log2;  // scale * log2(e)
};

// Packed rotation table: per (sample, position) D/2 pairs of (cos, sin) as float2.
struct Table {
  const float* ptr;  // float2 pairs, contiguous [Bt][S][D/2]
  int64_t sb;        // 0 when shared by every sample
};

struct FwdParams {
  Opnd q, k, v;
  void* o;
  int64_t o_sb, o_sh, o_ss;
  float* lse;  // nullable, contiguous [B, H, S]
  Table tab;
  MaskView mask;
  AttnShape shp;
  int num_qt;  // query tiles per (b, h)
  // blockwise int8 variant with codes from the quantizer pass: codes of the rotated Q and K,
  // [B][H|Hkv][sp][D] int8 with sp = S rounded up to 64 (padding rows zero), and their fp32
  // scales [B][H|Hkv][sp / 64]
  const int8_t* qc;
  const int8_t* kc;
  const float* qsc;
  const float* ksc;
  int sp;
  // blockwise int8 variant, code export mode only (the test-only export of the codes the
  // kernel computes): contiguous Q codes [B][H][S][D], K codes [B][Hkv][S][D] and their fp32
  // scales [B][H][nblk], [B][Hkv][nblk] (nblk = ceil(S / 64))
  int8_t* xq_codes;
  int8_t* xk_codes;
  float* xq_scales;
  float* xk_scales;
  // measurement only: HIP events recorded on the launch stream right before the attention
  // kernel and right after it (before the merge launch); null: none
  void* ev_start;
  void* ev_stop;
  // Q/K RMSNorm weights (fp32 [D], device; used when the launch asks for the normalization)
  const float* qnw;
  const float* knw;
  float norm_eps;
  // bool masks: the unmasked and the masked kernel are both enqueued; each reads the mask
  // classifier's word gate[0] (nonzero: some key is excluded) at entry and returns at once
  // unless gate_mode says it is the one to run (1: gate[0] == 0, 2: gate[0] != 0; 0: always)
  const unsigned* gate;
  int gate_mode;
  // split of the work (see the forward kernel): split_iters = 0 for one workgroup per unit
  int split_full;       // units run whole by the first workgroups (a multiple of 8)
  int split_grid;       // further workgroups sharing the remaining units' key tiles
  int64_t split_iters;  // (unit, key tile) iterations of the remaining units
  void* part_o;         // pieces' normalized outputs: two slots of [BM][D] per further workgroup
  float* part_lse;      // pieces' row log-sum-exp: two slots of [BM] per further workgroup
};

struct BwdParams {
  Opnd q, k, v, o, dout;
  void* dq;
  int64_t dq_sb, dq_sh, dq_ss;
  void* dk;
  int64_t dk_sb, dk_sh, dk_ss;
  void* dv;
  int64_t dv_sb, dv_sh, dv_ss;
  const float* lse;  // contiguous [B, H, S]
  float* delta;      // workspace, contiguous [B, H, S]
  void* qrot;        // workspace (16-bit inputs, D = 128): Q' = R(Q) [B, H, S, D] in the input
                     // dtype, written by the dQ kernel and read by the dK/dV kernel
  Table tab;
  MaskView mask;
  AttnShape shp;
};

struct PackParams {
  const float* cos;
  const float* sin;
  int64_t c_sb, c_ss, s_sb, s_ss;  // element strides of the [Bt, 1, S, D] tables (dims 0 and 2)
  float* out;                      // float2 pairs [Bt][S][D/2]
  int Bt, S, D;
  unsigned* ctrl;                  // control words cleared for the mask classifier
};

// Rotation + blockwise int8 quantization of Q (x[0]) and K (x[1]): the quantizer pass of
// the pre-quantized int8 mode.
struct QuantParams {
  Opnd x[2];
  Table tab;
  int8_t* codes[2];          // [B][Hx][rows][D] with the strides below
  int64_t c_sb[2], c_sh[2];  // element strides of the codes over b and h
  int rows;                  // allocated rows per (b, h) slice (>= S); rows past S are written as 0
  float* scales[2];          // [B][Hx][nblk]
  int Hx[2];                 // heads of Q (H) and of K (Hkv)
  int B, H, S, D, nblk;
  float qmax;                // code range [-qmax, qmax]: 127 (int8) or 7 (int4)
  // dequantizing mode (the quantized backward): when deq[0] is set, the pass writes
  // code * scale rounded to the input dtype, contiguous [B][Hx][S][D], instead of codes and
  // scales
  void* deq[2];
};

// The eager rotation pass (rope_sdpa_rotate): out = R(x) for a [B, H, S, D] operand.
struct RotateParams {
  Opnd x;
  void* out;
  int64_t o_sb, o_sh, o_ss;
  const float* cos;
  const float* sin;
  int64_t c_sb, c_ss, s_sb, s_ss;  // element strides of the [Bt, 1, S, D] tables (dims 0 and 2)
  int B, H, S, D;
};

struct ClassifyParams {
  MaskView mask;  // bool
  int nb, nh, Sq, Sk;  // mask extents (1 on broadcast dimensions)
  uint8_t* tiles;      // [nb][nh][nqt][nkt]
  unsigned* ctrl;      // ctrl[0] = some block excluded a key, ctrl[1] = finished blocks
  int total_blocks;
};

// Host-side launchers (defined in the .hip files).  Each returns 0 on success or a HIP error.
int launch_pack_tables(const PackParams& p, void* stream);
int launch_classify(const ClassifyParams& p, void* stream);
int fwd_block_m(int dtype);  // query rows per forward workgroup
int fwd_block_n(int dtype);  // keys per forward tile
// Split plan of a forward call on the current device (all zero: one workgroup per unit).
struct SplitPlan {
  int full, grid;
  int64_t iters;
  size_t slot_bytes;  // bytes of one partial-state slot
  int64_t cut_units;  // units whose key tiles are shared out
};
SplitPlan fwd_split_plan(int dtype, int D, bool int8, bool causal, int mask_kind, int64_t units, int nkt);
// int8: 0 = none, 1 = quantized in the attention kernel, 2 = codes from the quantizer pass
int launch_fwd(int dtype, int D, int mask_kind, bool causal, int int8, const FwdParams& p, void* stream);
int launch_quant_int8(int dtype, const QuantParams& p, void* stream);
// K of the Q/K prologue, prepared once: RMS-normalized (optional), rotated with the packed
// tables and rounded to the compute dtype, into a contiguous [B][H][S][D] buffer (H = the
// K/V head count).  Input in the compute dtype, or fp32 beside 16-bit V.
struct KPrepParams {
  Opnd x;
  void* out;
  // the caller's tables (cos, sin, strides, Bt: always read); out and ctrl set: the launch
  // also writes the packed tables and clears the control words (pack_tables_kernel's work)
  PackParams pk;
  const float* w;  // RMSNorm weights [D] (normalizing launches only)
  float eps;
  int B, H, S, D;
};
// qkm: bit 0 normalize, bit 1 fp32 input
int launch_kprep(int dtype, int qkm, const KPrepParams& p, void* stream);
// The forward with the Q/K prologue (qkm: bit 0 Q normalized, bit 1 Q in fp32 beside 16-bit V,
// bit 2 set: K prepared by launch_kprep); no mask, bool mask or causal.
int launch_fwd_qk(int dtype, int D, int mask_kind, bool causal, int qkm, const FwdParams& p, void* stream);
// The forward without rotation (no tables: plain attention).
int launch_fwd_plain(int dtype, int D, int mask_kind, bool causal, const FwdParams& p, void* stream);
int launch_rotate(int dtype, const RotateParams& p, void* stream);
// The int8 forward in code export mode (no output written; see FwdParams).
int launch_fwd_int8_export(int dtype, int D, bool int4, const FwdParams& p, void* stream);
// pre (16-bit inputs at D = 128 only, else 0): 0 Q and K rotated in the backward kernels; 1 K'
// prepared in p.k (contiguous); 3 Q' in p.qrot and K' in p.k both prepared (the quantized
// backward's dequantized values)
int launch_bwd(int dtype, int D, int mask_kind, bool causal, int pre, const BwdParams& p, void* stream);
// Reads (and optionally clears) the device-side count of all-true bool masks.
int read_all_true_counter(uint64_t* value, bool reset);

// Library-owned device scratch of rope_sdpa_fwd_noalloc (rs_scratch.hip): its size, and its
// device address on the current device (looked up once per device); 0 or a HIP error.
constexpr size_t kScratchBytes = (size_t)64 << 20;
int scratch_address(void** ptr);

}  // namespace rs
