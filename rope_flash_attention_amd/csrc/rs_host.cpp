// Host side of the C ABI declared in include/rope_sdpa.h: argument validation (pure host
// code that never dereferences a device pointer), workspace layout, device checks,
// dispatch counters and kernel launch on the caller's stream.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <cstring>
#include <mutex>
#include <utility>
#include <vector>

#include "../../include/rope_sdpa.h"
#include "rs_internal.h"

namespace {
constexpr uint32_t kQuantFlags = RS_FLAG_QUANT_INT8_QK | RS_FLAG_QUANT_INT4_QK;
}  // namespace

namespace {

using namespace rs;

struct Counters {
  std::atomic<uint64_t> fwd_instream{0}, fwd_autograd{0}, bwd_calls{0}, masked_bool{0},
      masked_additive{0}, causal{0}, quant_int8{0}, quant_bwd{0}, errors{0};
};
Counters g_ctr;

// Kernel timing for measurement (rope_sdpa_debug_kernel_timing): one pair of HIP events per
// timed forward call, recorded around its attention kernel.
struct KernelTiming {
  std::mutex mu;
  bool on = false;
  std::vector<std::pair<hipEvent_t, hipEvent_t>> ev;
  size_t used = 0;
} g_timing;

// The next event pair for a forward call (null when timing is off or events cannot be made).
bool timing_events(void** start, void** stop) {
  std::lock_guard<std::mutex> lk(g_timing.mu);
  if (!g_timing.on) return false;
  if (g_timing.used == g_timing.ev.size()) {
    hipEvent_t a = nullptr, b = nullptr;
    if (hipEventCreate(&a) != hipSuccess) return false;
    if (hipEventCreate(&b) != hipSuccess) {
      (void)hipEventDestroy(a);
      return false;
    }
    g_timing.ev.emplace_back(a, b);
  }
  *start = g_timing.ev[g_timing.used].first;
  *stop = g_timing.ev[g_timing.used].second;
  ++g_timing.used;
  return true;
}

rs_status fail(rs_status s) {
  g_ctr.errors.fetch_add(1, std::memory_order_relaxed);
  return s;
}

size_t elem_size(int dt) {
  switch (dt) {
    case RS_F32: return 4;
    case RS_F16: return 2;
    case RS_BF16: return 2;
    case RS_BOOL: return 1;
    default: return 0;
  }
}

size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Checks a [B,H,S,D]-like operand: pointer, dtype, exact sizes, contiguous last dim,
// 16-byte base alignment and 16-byte multiples for the strides of non-trivial dims.
rs_status check_bhsd(const rs_tensor* t, int dtype, const int64_t* size, bool empty = false) {
  if (!t || (!t->data && !empty)) return RS_ERR_NULL;
  if (t->dtype != dtype) return RS_ERR_DTYPE;
  if (t->reserved != 0) return RS_ERR_INVALID;
  for (int i = 0; i < 4; ++i)
    if (t->size[i] != size[i]) return RS_ERR_SHAPE;
  if (empty) return RS_OK;  // no element is addressed: strides and base are not looked at
  if (t->stride[3] != 1) return RS_ERR_STRIDE;
  const int64_t es = (int64_t)elem_size(dtype);
  for (int i = 0; i < 3; ++i) {
    if (t->size[i] <= 1) continue;
    if (t->stride[i] < 0 || (t->stride[i] * es) % 16 != 0) return RS_ERR_STRIDE;
  }
  // row offsets inside a tile of up to 256 rows are 32-bit in the kernels, and one (b, h)
  // slice is addressed through a buffer descriptor with a 32-bit byte range
  if (t->size[2] > 1 && t->stride[2] >= ((int64_t)1 << 23)) return RS_ERR_STRIDE;
  if ((t->size[2] * t->stride[2] + t->size[3]) * es >= ((int64_t)1 << 31)) return RS_ERR_STRIDE;
  if (((uintptr_t)t->data) % 16 != 0) return RS_ERR_ALIGN;
  return RS_OK;
}


struct Shape {
  int64_t B, H, S, D;
  int qdtype;   // dtype of Q and K (that of V, or f32 with 16-bit V)
  int qkm;      // Q/K prologue: bit 0 RMSNorm, bit 1 fp32 Q/K with 16-bit V
  bool kprep;   // forward: K rotated (and normalized) once into the workspace by kprep_kernel
  bool rope;    // rotation tables given (both NULL: plain attention, forward only)
  int64_t Hkv;  // heads of K and V (grouped-query attention: H % Hkv == 0)
  bool empty;  // B, H or S is 0: a valid call with nothing to compute
  int dtype;
  float scale;
  int64_t Bt;
  int64_t mB, mH, mQ, mK;  // mask extents (0 when there is no mask)
};

rs_status check_table(const rs_tensor* t, const Shape& s, int64_t* bt) {
  if (!t || (!t->data && !s.empty)) return RS_ERR_NULL;
  if (t->dtype != RS_F32) return RS_ERR_DTYPE;
  if (t->reserved != 0) return RS_ERR_INVALID;
  if (!(t->size[0] == 1 || t->size[0] == s.B) || t->size[1] != 1 || t->size[2] != s.S || t->size[3] != s.D)
    return RS_ERR_SHAPE;
  *bt = t->size[0];
  if (s.empty) return RS_OK;  // not read
  if (t->stride[3] != 1) return RS_ERR_STRIDE;
  if (t->stride[0] < 0 || t->stride[2] < 0) return RS_ERR_STRIDE;
  if (((uintptr_t)t->data) % 4 != 0) return RS_ERR_ALIGN;
  *bt = t->size[0];
  return RS_OK;
}

// Validates everything both directions share: Q/K/V, tables, mask, flags and scale.
rs_status validate_args(const rs_args* a, Shape* out) {
  if (!a || !a->q || !a->k || !a->v) return RS_ERR_NULL;
  if ((a->cos == nullptr) != (a->sin == nullptr)) return RS_ERR_NULL;  // both or neither
  const rs_tensor* q = a->q;
  const int dt = a->v->dtype;  // the compute dtype: V, O and the matrix products
  if (dt != RS_F32 && dt != RS_F16 && dt != RS_BF16) return RS_ERR_DTYPE;
  const int qdt = q->dtype;
  if (qdt != dt && !(qdt == RS_F32 && dt != RS_F32)) return RS_ERR_DTYPE;
  Shape s{};
  s.qdtype = qdt;
  s.qkm = qdt != dt ? 2 : 0;
  s.B = q->size[0];
  s.H = q->size[1];
  s.S = q->size[2];
  s.D = q->size[3];
  s.dtype = dt;
  if (s.B < 0 || s.H < 0 || s.S < 0) return RS_ERR_SHAPE;
  s.empty = s.B == 0 || s.H == 0 || s.S == 0;
  if (!q->data && !s.empty) return RS_ERR_NULL;
  if (s.D != 64 && s.D != 128) return RS_ERR_SHAPE;
  if (s.S > (int64_t)1 << 24) return RS_ERR_SHAPE;
  const int64_t nqt = (s.S + 127) / 128;
  if (s.B * s.H * nqt >= ((int64_t)1 << 31) || s.B * s.H * s.S >= ((int64_t)1 << 31)) return RS_ERR_SHAPE;
  const int64_t sz[4] = {s.B, s.H, s.S, s.D};
  rs_status st;
  if ((st = check_bhsd(q, qdt, sz, s.empty)) != RS_OK) return st;
  // K in Q's dtype, V in the compute dtype, Hkv heads with H % Hkv == 0 (grouped-query
  // attention when Hkv < H)
  if (a->k->dtype != qdt) return RS_ERR_DTYPE;
  s.Hkv = a->k->size[1];
  if (s.H == 0 ? s.Hkv != 0 : (s.Hkv <= 0 || s.H % s.Hkv != 0)) return RS_ERR_SHAPE;
  const int64_t szkv[4] = {s.B, s.Hkv, s.S, s.D};
  if ((st = check_bhsd(a->k, qdt, szkv, s.empty)) != RS_OK) return st;
  if ((st = check_bhsd(a->v, dt, szkv, s.empty)) != RS_OK) return st;
  // optional Q/K RMSNorm: both weights or neither
  if ((a->q_norm_weight == nullptr) != (a->k_norm_weight == nullptr)) return RS_ERR_INVALID;
  if (a->q_norm_weight) {
    if (!std::isfinite(a->norm_eps) || a->norm_eps < 0.f) return RS_ERR_INVALID;
    if (((uintptr_t)a->q_norm_weight) % 16 != 0 || ((uintptr_t)a->k_norm_weight) % 16 != 0) return RS_ERR_ALIGN;
    s.qkm |= 1;
  }
  s.rope = a->cos != nullptr;
  if (s.rope) {
    int64_t bt_c = 0, bt_s = 0;
    if ((st = check_table(a->cos, s, &bt_c)) != RS_OK) return st;
    if ((st = check_table(a->sin, s, &bt_s)) != RS_OK) return st;
    if (bt_c != bt_s) return RS_ERR_SHAPE;
    s.Bt = bt_c;
  } else {
    s.Bt = 0;  // no packed tables
  }

  if (a->flags & ~(uint32_t)(RS_FLAG_CAUSAL | kQuantFlags | RS_FLAG_QUANT_INT8_PREPASS | RS_FLAG_K_PREPASS))
    return RS_ERR_INVALID;
  if ((a->flags & kQuantFlags) == kQuantFlags) return RS_ERR_INVALID;  // int8 or int4, not both
  if ((a->flags & RS_FLAG_QUANT_INT8_PREPASS) && !(a->flags & kQuantFlags)) return RS_ERR_INVALID;
  const bool causal = (a->flags & RS_FLAG_CAUSAL) != 0;
  if (!(std::isfinite(a->scale)) || a->scale < 0.f) return RS_ERR_INVALID;
  s.scale = a->scale == 0.f ? (float)(1.0 / std::sqrt((double)s.D)) : a->scale;

  if (a->mask_kind == RS_MASK_NONE) {
    if (a->mask) return RS_ERR_INVALID;
  } else if (a->mask_kind == RS_MASK_BOOL || a->mask_kind == RS_MASK_ADDITIVE) {
    const rs_tensor* m = a->mask;
    if (!m || (!m->data && !s.empty)) return RS_ERR_NULL;
    if (causal) return RS_ERR_INVALID;
    if (m->reserved != 0) return RS_ERR_INVALID;
    if (a->mask_kind == RS_MASK_BOOL) {
      if (m->dtype != RS_BOOL) return RS_ERR_DTYPE;
    } else if (m->dtype != RS_F32 && m->dtype != dt) {
      return RS_ERR_DTYPE;
    }
    const int64_t full[4] = {s.B, s.H, s.S, s.S};
    for (int i = 0; i < 4; ++i)
      if (m->size[i] != 1 && m->size[i] != full[i]) return RS_ERR_SHAPE;
    const int64_t es = (int64_t)elem_size(m->dtype);
    if (!s.empty) {  // an empty call reads no mask element
      if (m->size[3] > 1 && m->stride[3] != 1) return RS_ERR_STRIDE;
      for (int i = 0; i < 3; ++i) {
        if (m->size[i] <= 1) continue;
        if (m->stride[i] < 0) return RS_ERR_STRIDE;
        if (m->size[3] > 1 && (m->stride[i] * es) % 16 != 0) return RS_ERR_STRIDE;
      }
      if (m->size[3] > 1 && ((uintptr_t)m->data) % 16 != 0) return RS_ERR_ALIGN;
      if (((uintptr_t)m->data) % es != 0) return RS_ERR_ALIGN;
    }
    s.mB = m->size[0];
    s.mH = m->size[1];
    s.mQ = m->size[2];
    s.mK = m->size[3];
  } else {
    return RS_ERR_INVALID;
  }
  if (s.qkm != 0 && (!s.rope || a->mask_kind == RS_MASK_ADDITIVE)) return RS_ERR_UNSUPPORTED;
  if (a->flags & kQuantFlags) {
    if (dt == RS_F32 || !s.rope || s.qkm != 0) return RS_ERR_UNSUPPORTED;
  }
  if (a->mask_kind == RS_MASK_BOOL) {
    if (s.S > kMaxBoolMaskSeq) return RS_ERR_SHAPE;
    // grid limits of the tile classifier (y: query tiles, z: mask batch x heads)
    if ((s.mQ + kMaskTile - 1) / kMaskTile > 65535 || s.mB * s.mH > 65535) return RS_ERR_SHAPE;
  }
  // K rotated once into the workspace by a pass of its own (kprep_kernel) instead of in the
  // attention kernel's key loop: on request (RS_FLAG_K_PREPASS: the 16-bit rotating forward
  // without quantization or additive mask), and always for the Q/K prologue
  if (a->flags & RS_FLAG_K_PREPASS) {
    if (!s.rope || dt == RS_F32 || (a->flags & kQuantFlags) || a->mask_kind == RS_MASK_ADDITIVE)
      return RS_ERR_UNSUPPORTED;
  }
  s.kprep = s.qkm != 0 || (a->flags & RS_FLAG_K_PREPASS) != 0;
  *out = s;
  return RS_OK;
}

struct Layout {
  size_t ctrl, table, tiles, delta, qrot, qc, kc, qs, ks, kprep, part, cnt, total;
  int64_t nqt, nkt;
  int64_t sp, nblk;  // pre-quantized int8: padded rows per (b, h) slice and 64-token blocks
  SplitPlan split;   // forward only: work split over the current device's workgroups
};

// int8: quantization mode (quant_mode): 0 none, 1 quantized in the attention kernel, 2 codes
// from the quantizer pass, + 4 for int4 codes
Layout layout(const Shape& s, int mask_kind, bool backward, int int8, bool causal) {
  Layout L{};
  size_t off = 0;
  L.ctrl = off;
  off += 256;
  L.table = off;
  off += round_up((size_t)s.Bt * s.S * s.D * sizeof(float), 256);  // D/2 float2 per row
  L.tiles = off;
  if (mask_kind == RS_MASK_BOOL) {
    L.nqt = (s.mQ + kMaskTile - 1) / kMaskTile;
    L.nkt = (s.mK + kMaskTile - 1) / kMaskTile;
    off += round_up((size_t)(s.mB * s.mH * L.nqt * L.nkt), 256);
  }
  L.delta = off;
  if (backward) off += round_up((size_t)(s.B * s.H * s.S) * sizeof(float), 256);
  // (backward, 16-bit: Q' at D = 128, and at D = 64 for the quantized backward's Q^')
  const bool bwd_prep = backward && s.dtype != F32 && (s.D == 128 || int8 != 0);
  L.qrot = off;
  if (bwd_prep) off += round_up((size_t)(s.B * s.H * s.S * s.D) * 2, 256);
  if (!backward && (int8 & 3) == 2) {
    L.nblk = (s.S + 63) / 64;
    L.sp = L.nblk * 64;
    L.qc = off;
    off += round_up((size_t)(s.B * s.H * L.sp * s.D), 256);
    L.kc = off;
    off += round_up((size_t)(s.B * s.Hkv * L.sp * s.D), 256);
    L.qs = off;
    off += round_up((size_t)(s.B * s.H * L.nblk) * sizeof(float), 256);
    L.ks = off;
    off += round_up((size_t)(s.B * s.Hkv * L.nblk) * sizeof(float), 256);
  }
  L.kprep = off;  // K' = R(K) rotated once: [B][Hkv][S][D] in the compute dtype
  if ((!backward && s.kprep) || bwd_prep)
    off += round_up((size_t)(s.B * s.Hkv * s.S * s.D) * elem_size(s.dtype), 256);
  if (!backward) {
    const int64_t bm = fwd_block_m(s.dtype), bn = fwd_block_n(s.dtype);
    const int64_t units = s.B * s.H * ((s.S + bm - 1) / bm);
    L.split = fwd_split_plan(s.dtype, (int)s.D, int8 != 0, causal, mask_kind, units, (int)((s.S + bn - 1) / bn));
    if (L.split.iters > 0) {
      L.part = off;
      off += round_up(2 * (size_t)L.split.grid * L.split.slot_bytes, 256);
      L.cnt = off;  // the pieces' row log-sum-exp
      off += round_up(2 * (size_t)L.split.grid * bm * sizeof(float), 256);
    }
  }
  L.total = off;
  return L;
}

// One check per device: the library is built for gfx950 only.
std::mutex g_dev_mu;
int g_dev_ok[64] = {0};  // 0 unknown, 1 ok, -1 not usable

rs_status current_device_ok() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return RS_ERR_NO_DEVICE;
  std::lock_guard<std::mutex> lk(g_dev_mu);
  if (g_dev_ok[dev] == 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) {
      g_dev_ok[dev] = -1;
    } else {
      g_dev_ok[dev] = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : -1;
    }
  }
  return g_dev_ok[dev] == 1 ? RS_OK : RS_ERR_NO_DEVICE;
}

MaskView mask_view(const rs_args* a, const Shape& s, const Layout& L, char* ws) {
  MaskView mv{};
  if (a->mask_kind == RS_MASK_NONE) return mv;
  const rs_tensor* m = a->mask;
  mv.ptr = m->data;
  mv.sb = m->size[0] > 1 ? m->stride[0] : 0;
  mv.sh = m->size[1] > 1 ? m->stride[1] : 0;
  mv.sq = m->size[2] > 1 ? m->stride[2] : 0;
  mv.sk = m->size[3] > 1 ? m->stride[3] : 0;
  mv.dtype = m->dtype;
  mv.key_bcast = m->size[3] == 1;
  if (a->mask_kind == RS_MASK_BOOL) {
    mv.tiles = (const uint8_t*)(ws + L.tiles);
    mv.t_nqt = (int)L.nqt;
    mv.t_nkt = (int)L.nkt;
    mv.t_sh = s.mH > 1 ? L.nqt * L.nkt : 0;
    mv.t_sb = s.mB > 1 ? s.mH * L.nqt * L.nkt : 0;
  }
  return mv;
}

AttnShape attn_shape(const Shape& s) {
  AttnShape a{};
  a.B = (int)s.B;
  a.H = (int)s.H;
  a.S = (int)s.S;
  a.Hkv = (int)s.Hkv;
  a.group = s.Hkv > 0 ? (int)(s.H / s.Hkv) : 1;
  a.scale = s.scale;
  a.scale_log2 = (float)((double)s.scale * 1.4426950408889634);
  return a;
}

// Enqueues the preparation kernels shared by both directions.
Opnd opnd(const rs_tensor* t) {
  Opnd o;
  o.ptr = t->data;
  o.sb = t->stride[0];
  o.sh = t->stride[1];
  o.ss = t->stride[2];
  return o;
}

PackParams pack_params(const rs_args* a, const Shape& s, const Layout& L, char* ws) {
  PackParams pp{};  // (no tables, Bt = 0: the launch only clears the control words)
  if (s.rope) {
    pp.cos = (const float*)a->cos->data;
    pp.sin = (const float*)a->sin->data;
    pp.c_sb = a->cos->size[0] > 1 ? a->cos->stride[0] : 0;
    pp.c_ss = a->cos->stride[2];
    pp.s_sb = a->sin->size[0] > 1 ? a->sin->stride[0] : 0;
    pp.s_ss = a->sin->stride[2];
  }
  pp.out = (float*)(ws + L.table);
  pp.Bt = (int)s.Bt;
  pp.S = (int)s.S;
  pp.D = (int)s.D;
  pp.ctrl = (unsigned*)(ws + L.ctrl);
  return pp;
}

// K' = R(K) (RMS-normalized first when the Q/K prologue asks for it) into the workspace, in
// the same launch as the table packing and the clearing of the control words.
rs_status launch_kprep_packed(const rs_args* a, const Shape& s, const Layout& L, char* ws, hipStream_t stream) {
  KPrepParams kp{};
  kp.x = opnd(a->k);
  kp.out = ws + L.kprep;
  kp.pk = pack_params(a, s, L, ws);
  kp.w = a->k_norm_weight;
  kp.eps = a->norm_eps;
  kp.B = (int)s.B;
  kp.H = (int)s.Hkv;
  kp.S = (int)s.S;
  kp.D = (int)s.D;
  return launch_kprep(s.dtype, s.qkm, kp, stream) != 0 ? RS_ERR_LAUNCH : RS_OK;
}

// Table packing (unless a K preparation launch already did it) and bool-mask classification.
rs_status prepare(const rs_args* a, const Shape& s, const Layout& L, char* ws, hipStream_t stream,
                  bool pack = true) {
  if (pack && launch_pack_tables(pack_params(a, s, L, ws), stream) != 0) return RS_ERR_LAUNCH;
  if (a->mask_kind == RS_MASK_BOOL) {
    ClassifyParams cp{};
    cp.mask = mask_view(a, s, L, ws);
    cp.nb = (int)s.mB;
    cp.nh = (int)s.mH;
    cp.Sq = (int)s.mQ;
    cp.Sk = (int)s.mK;
    cp.tiles = (uint8_t*)(ws + L.tiles);
    cp.ctrl = (unsigned*)(ws + L.ctrl);
    cp.total_blocks = (int)(s.mB * s.mH * L.nqt * L.nkt);
    if (launch_classify(cp, stream) != 0) return RS_ERR_LAUNCH;
  }
  return RS_OK;
}


// 0 none; 1 quantized in the attention kernel, 2 codes from the quantizer pass; + 4 for int4
int int8_mode(uint32_t flags) {
  if (!(flags & kQuantFlags)) return 0;
  return ((flags & RS_FLAG_QUANT_INT8_PREPASS) ? 2 : 1) | ((flags & RS_FLAG_QUANT_INT4_QK) ? 4 : 0);
}

QuantParams quant_params(const rs_args* a, const Shape& s, const Layout& L, char* ws) {
  QuantParams qp{};
  qp.x[0] = opnd(a->q);
  qp.x[1] = opnd(a->k);
  qp.tab.ptr = (const float*)(ws + L.table);
  qp.tab.sb = s.Bt > 1 ? s.S * s.D : 0;
  qp.codes[0] = (int8_t*)(ws + L.qc);
  qp.codes[1] = (int8_t*)(ws + L.kc);
  qp.c_sh[0] = qp.c_sh[1] = L.sp * s.D;
  qp.c_sb[0] = s.H * L.sp * s.D;
  qp.c_sb[1] = s.Hkv * L.sp * s.D;
  qp.rows = (int)L.sp;
  qp.scales[0] = (float*)(ws + L.qs);
  qp.scales[1] = (float*)(ws + L.ks);
  qp.qmax = (a->flags & RS_FLAG_QUANT_INT4_QK) ? 7.f : 127.f;
  qp.Hx[0] = (int)s.H;
  qp.Hx[1] = (int)s.Hkv;
  qp.B = (int)s.B;
  qp.H = (int)s.H;
  qp.S = (int)s.S;
  qp.D = (int)s.D;
  qp.nblk = (int)L.nblk;
  return qp;
}

rs_status check_ws(void* ws, size_t ws_bytes, const Layout& L) {
  if (!ws || ws_bytes < L.total) return RS_ERR_WORKSPACE;
  if (((uintptr_t)ws) % 256 != 0) return RS_ERR_ALIGN;
  return RS_OK;
}

}  // namespace

extern "C" {

int rope_sdpa_abi_version(void) { return ROPE_SDPA_ABI_VERSION; }

rs_status rope_sdpa_debug_kernel_timing(int enable) {
  std::lock_guard<std::mutex> lk(g_timing.mu);
  g_timing.on = enable != 0;
  g_timing.used = 0;
  return RS_OK;
}

rs_status rope_sdpa_debug_kernel_time(double* total_ms, uint64_t* launches) {
  if (!total_ms || !launches) return fail(RS_ERR_NULL);
  std::lock_guard<std::mutex> lk(g_timing.mu);
  double t = 0.0;
  for (size_t i = 0; i < g_timing.used; ++i) {
    float ms = 0.f;
    if (hipEventSynchronize(g_timing.ev[i].second) != hipSuccess ||
        hipEventElapsedTime(&ms, g_timing.ev[i].first, g_timing.ev[i].second) != hipSuccess)
      return fail(RS_ERR_LAUNCH);
    t += ms;
  }
  *total_ms = t;
  *launches = g_timing.used;
  return RS_OK;
}

const char* rope_sdpa_status_string(rs_status st) {
  switch (st) {
    case RS_OK: return "RS_OK: success";
    case RS_ERR_NULL: return "RS_ERR_NULL: a required pointer is NULL";
    case RS_ERR_DTYPE: return "RS_ERR_DTYPE: unsupported dtype or Q/K/V/O dtypes differ";
    case RS_ERR_SHAPE: return "RS_ERR_SHAPE: inconsistent or unsupported sizes (D must be 64 or 128)";
    case RS_ERR_STRIDE: return "RS_ERR_STRIDE: last-dim stride must be 1 and other strides multiples of 16 bytes";
    case RS_ERR_ALIGN: return "RS_ERR_ALIGN: base pointer misaligned (16 bytes; workspace 256 bytes)";
    case RS_ERR_UNSUPPORTED: return "RS_ERR_UNSUPPORTED: combination not implemented";
    case RS_ERR_WORKSPACE: return "RS_ERR_WORKSPACE: workspace missing or too small";
    case RS_ERR_INVALID: return "RS_ERR_INVALID: bad flags, mask kind, scale, or causal with a mask";
    case RS_ERR_NO_DEVICE: return "RS_ERR_NO_DEVICE: no current gfx950 device";
    case RS_ERR_LAUNCH: return "RS_ERR_LAUNCH: kernel launch failed";
    case RS_ERR_SCRATCH:
      return "RS_ERR_SCRATCH: the call needs more device scratch than rope_sdpa_fwd_noalloc has "
             "(rope_sdpa_noalloc_scratch_bytes()); use rope_sdpa_fwd with a workspace";
  }
  return "unknown rs_status";
}

rs_status rope_sdpa_workspace_size(const rs_args* args, int backward, size_t* bytes) {
  if (!bytes) return fail(RS_ERR_NULL);
  Shape s;
  rs_status st = validate_args(args, &s);
  if (st != RS_OK) return fail(st);
  *bytes = s.empty ? 0
                   : layout(s, args->mask_kind, backward != 0, int8_mode(args->flags),
                            (args->flags & RS_FLAG_CAUSAL) != 0)
                         .total;
  return RS_OK;
}

}  // extern "C"

namespace {

// The forward of both entry points: `ws` is the caller's workspace (rope_sdpa_fwd) or, when
// `scratch` is set, the library's device scratch (rope_sdpa_fwd_noalloc), looked up after
// validation and the device check.
rs_status fwd_impl(const rs_args* a, const rs_tensor* o, float* lse, void* ws, size_t ws_bytes, void* stream,
                   bool scratch) {
  Shape s;
  rs_status st = validate_args(a, &s);
  if (st != RS_OK) return fail(st);
  const int64_t sz[4] = {s.B, s.H, s.S, s.D};
  if (!o) return fail(RS_ERR_NULL);
  if (o->data && o->dtype != s.dtype) return fail(RS_ERR_DTYPE);
  if ((st = check_bhsd(o, s.dtype, sz, s.empty)) != RS_OK) return fail(st);
  if (lse && ((uintptr_t)lse) % 4 != 0) return fail(RS_ERR_ALIGN);
  if (s.empty) return RS_OK;  // nothing to compute: no workspace or device needed
  const int int8 = int8_mode(a->flags);
  const bool causal_flag = (a->flags & RS_FLAG_CAUSAL) != 0;
  Layout L = layout(s, a->mask_kind, false, int8, causal_flag);
  if (scratch && L.total > kScratchBytes && s.kprep && s.qkm == 0) {
    s.kprep = false;  // the fixed scratch cannot hold K': rotate K in the key loop instead
    L = layout(s, a->mask_kind, false, int8, causal_flag);
  }
  if (scratch) {
    if (L.total > kScratchBytes) return fail(RS_ERR_SCRATCH);
    if ((st = current_device_ok()) != RS_OK) return fail(st);
    if (scratch_address(&ws) != 0) return fail(RS_ERR_NO_DEVICE);
    ws_bytes = kScratchBytes;
  }
  if ((st = check_ws(ws, ws_bytes, L)) != RS_OK) return fail(st);
  if ((st = current_device_ok()) != RS_OK) return fail(st);

  char* w = (char*)ws;
  hipStream_t strm = (hipStream_t)stream;
  // K prepared once into the workspace (with the tables packed in the same launch), then read
  // as K' by the attention kernel
  if (s.kprep && (st = launch_kprep_packed(a, s, L, w, strm)) != RS_OK) return fail(st);
  if ((st = prepare(a, s, L, w, strm, !s.kprep)) != RS_OK) return fail(st);
  if ((int8 & 3) == 2 && launch_quant_int8(s.dtype, quant_params(a, s, L, w), strm) != 0) return fail(RS_ERR_LAUNCH);
  FwdParams p{};
  p.q = opnd(a->q);
  p.k = opnd(a->k);
  p.v = opnd(a->v);
  p.o = o->data;
  p.o_sb = o->stride[0];
  p.o_sh = o->stride[1];
  p.o_ss = o->stride[2];
  p.lse = lse;
  p.tab.ptr = s.rope ? (const float*)(w + L.table) : nullptr;
  p.tab.sb = s.Bt > 1 ? s.S * s.D : 0;
  p.mask = mask_view(a, s, L, w);
  p.gate = (const unsigned*)(w + L.ctrl);  // (used by the bool-mask launch only)
  p.shp = attn_shape(s);
  const int bm = fwd_block_m(s.dtype);
  p.num_qt = (int)((s.S + bm - 1) / bm);
  const bool causal = (a->flags & RS_FLAG_CAUSAL) != 0;
  if ((int8 & 3) == 2) {
    p.qc = (const int8_t*)(w + L.qc);
    p.kc = (const int8_t*)(w + L.kc);
    p.qsc = (const float*)(w + L.qs);
    p.ksc = (const float*)(w + L.ks);
    p.sp = (int)L.sp;
  }
  if (L.split.iters > 0) {
    p.split_full = L.split.full;
    p.split_grid = L.split.grid;
    p.split_iters = L.split.iters;
    p.part_o = w + L.part;
    p.part_lse = (float*)(w + L.cnt);
  }
  p.qnw = a->q_norm_weight;
  p.knw = a->k_norm_weight;
  p.norm_eps = a->norm_eps;
  if (!scratch) timing_events(&p.ev_start, &p.ev_stop);
  if (s.kprep) {
    p.k.ptr = w + L.kprep;
    p.k.sb = s.Hkv * s.S * s.D;
    p.k.sh = s.S * s.D;
    p.k.ss = s.D;
  }
  const int lerr = !s.rope        ? launch_fwd_plain(s.dtype, (int)s.D, a->mask_kind, causal, p, strm)
                   : s.kprep    ? launch_fwd_qk(s.dtype, (int)s.D, a->mask_kind, causal, s.qkm | 4, p, strm)
                                : launch_fwd(s.dtype, (int)s.D, a->mask_kind, causal, int8, p, strm);
  if (lerr != 0) return fail(RS_ERR_LAUNCH);

  (lse ? g_ctr.fwd_autograd : g_ctr.fwd_instream).fetch_add(1, std::memory_order_relaxed);
  if (a->mask_kind == RS_MASK_BOOL) g_ctr.masked_bool.fetch_add(1, std::memory_order_relaxed);
  if (a->mask_kind == RS_MASK_ADDITIVE) g_ctr.masked_additive.fetch_add(1, std::memory_order_relaxed);
  if (causal) g_ctr.causal.fetch_add(1, std::memory_order_relaxed);
  if (int8) g_ctr.quant_int8.fetch_add(1, std::memory_order_relaxed);
  return RS_OK;
}

}  // namespace

extern "C" {

rs_status rope_sdpa_fwd(const rs_args* a, const rs_tensor* o, float* lse, void* ws, size_t ws_bytes,
                        void* stream) {
  return fwd_impl(a, o, lse, ws, ws_bytes, stream, false);
}

rs_status rope_sdpa_fwd_noalloc(const rs_args* a, const rs_tensor* o, float* lse, void* stream) {
  return fwd_impl(a, o, lse, nullptr, 0, stream, true);
}

size_t rope_sdpa_noalloc_scratch_bytes(void) { return kScratchBytes; }

rs_status rope_sdpa_debug_quantize_qk(const rs_args* a, int8_t* q_codes, int8_t* k_codes, float* q_scales,
                                      float* k_scales, void* ws, size_t ws_bytes, void* stream) {
  Shape s;
  rs_status st = validate_args(a, &s);
  if (st != RS_OK) return fail(st);
  if (!(a->flags & kQuantFlags)) return fail(RS_ERR_INVALID);
  if (s.empty) return RS_OK;
  if (!q_codes || !k_codes || !q_scales || !k_scales) return fail(RS_ERR_NULL);
  if (((uintptr_t)q_codes) % 8 != 0 || ((uintptr_t)k_codes) % 8 != 0) return fail(RS_ERR_ALIGN);
  if (((uintptr_t)q_scales) % 4 != 0 || ((uintptr_t)k_scales) % 4 != 0) return fail(RS_ERR_ALIGN);
  const Layout L = layout(s, a->mask_kind, false, 1, false);
  if ((st = check_ws(ws, ws_bytes, L)) != RS_OK) return fail(st);
  if ((st = current_device_ok()) != RS_OK) return fail(st);
  char* w = (char*)ws;
  hipStream_t strm = (hipStream_t)stream;
  if ((st = prepare(a, s, L, w, strm)) != RS_OK) return fail(st);
  // the int8 forward itself, in its code export mode: the codes it computes, not a copy
  FwdParams p{};
  p.q = opnd(a->q);
  p.k = opnd(a->k);
  p.v = opnd(a->v);
  p.tab.ptr = (const float*)(w + L.table);
  p.tab.sb = s.Bt > 1 ? s.S * s.D : 0;
  p.shp = attn_shape(s);
  p.num_qt = (int)((s.S + fwd_block_m(s.dtype) - 1) / fwd_block_m(s.dtype));
  p.xq_codes = q_codes;
  p.xk_codes = k_codes;
  p.xq_scales = q_scales;
  p.xk_scales = k_scales;
  if (launch_fwd_int8_export(s.dtype, (int)s.D, (a->flags & RS_FLAG_QUANT_INT4_QK) != 0, p, strm) != 0)
    return fail(RS_ERR_LAUNCH);
  return RS_OK;
}

rs_status rope_sdpa_bwd(const rs_args* a, const rs_tensor* o, const float* lse, const rs_tensor* dout,
                        const rs_tensor* dq, const rs_tensor* dk, const rs_tensor* dv, void* ws,
                        size_t ws_bytes, void* stream) {
  Shape s;
  rs_status st = validate_args(a, &s);
  if (st != RS_OK) return fail(st);
  const bool quant = (a->flags & kQuantFlags) != 0;
  if (!s.rope) return fail(RS_ERR_UNSUPPORTED);  // the backward is the fused one: tables required
  if (s.qkm != 0) return fail(RS_ERR_UNSUPPORTED);  // no backward through the Q/K prologue
  const int64_t sz[4] = {s.B, s.H, s.S, s.D};
  const int64_t szkv[4] = {s.B, s.Hkv, s.S, s.D};
  if (!o || !dout || !dq || !dk || !dv || (!lse && !s.empty)) return fail(RS_ERR_NULL);
  const rs_tensor* ts[5] = {o, dout, dq, dk, dv};
  for (const rs_tensor* t : ts) {
    if (t->data && t->dtype != s.dtype) return fail(RS_ERR_DTYPE);
    if ((st = check_bhsd(t, s.dtype, (t == dk || t == dv) ? szkv : sz, s.empty)) != RS_OK) return fail(st);
  }
  if (((uintptr_t)lse) % 4 != 0) return fail(RS_ERR_ALIGN);
  if (s.empty) return RS_OK;
  const Layout L = layout(s, a->mask_kind, true, int8_mode(a->flags), (a->flags & RS_FLAG_CAUSAL) != 0);
  if ((st = check_ws(ws, ws_bytes, L)) != RS_OK) return fail(st);
  if ((st = current_device_ok()) != RS_OK) return fail(st);

  char* w = (char*)ws;
  hipStream_t strm = (hipStream_t)stream;
  // 16-bit at D = 128: K' = R(K) once into the workspace (the dQ kernel then streams K' tiles
  // with no table), in the launch that packs the tables; quantized: the dequantized Q' and K'
  // the forward attended with, by the quantizer pass (after the table packing)
  const bool kprep = s.dtype != F32 && s.D == 128 && !quant;
  if (kprep && (st = launch_kprep_packed(a, s, L, w, strm)) != RS_OK) return fail(st);
  if ((st = prepare(a, s, L, w, strm, !kprep)) != RS_OK) return fail(st);
  BwdParams p{};
  p.q = opnd(a->q);
  p.k = opnd(a->k);
  p.v = opnd(a->v);
  p.o = opnd(o);
  p.dout = opnd(dout);
  p.dq = dq->data;
  p.dq_sb = dq->stride[0];
  p.dq_sh = dq->stride[1];
  p.dq_ss = dq->stride[2];
  p.dk = dk->data;
  p.dk_sb = dk->stride[0];
  p.dk_sh = dk->stride[1];
  p.dk_ss = dk->stride[2];
  p.dv = dv->data;
  p.dv_sb = dv->stride[0];
  p.dv_sh = dv->stride[1];
  p.dv_ss = dv->stride[2];
  p.lse = lse;
  p.delta = (float*)(w + L.delta);
  p.qrot = w + L.qrot;
  p.tab.ptr = (const float*)(w + L.table);
  p.tab.sb = s.Bt > 1 ? s.S * s.D : 0;
  p.mask = mask_view(a, s, L, w);
  p.shp = attn_shape(s);
  const bool causal = (a->flags & RS_FLAG_CAUSAL) != 0;
  int pre = 0;
  if (s.dtype != F32 && (s.D == 128 || quant)) {
    if (quant) {
      QuantParams qp = quant_params(a, s, L, w);
      qp.nblk = (int)((s.S + 63) / 64);
      qp.deq[0] = w + L.qrot;
      qp.deq[1] = w + L.kprep;
      if (launch_quant_int8(s.dtype, qp, strm) != 0) return fail(RS_ERR_LAUNCH);
      pre = 3;
      if (s.D != 128) {  // the 32x32 kernels read Q^' as Q
        p.q.ptr = w + L.qrot;
        p.q.sb = s.H * s.S * s.D;
        p.q.sh = s.S * s.D;
        p.q.ss = s.D;
      }
    } else {
      pre = 1;
    }
    p.k.ptr = w + L.kprep;
    p.k.sb = s.Hkv * s.S * s.D;
    p.k.sh = s.S * s.D;
    p.k.ss = s.D;
  }
  if (launch_bwd(s.dtype, (int)s.D, a->mask_kind, causal, pre, p, strm) != 0) return fail(RS_ERR_LAUNCH);

  g_ctr.bwd_calls.fetch_add(1, std::memory_order_relaxed);
  if (quant) g_ctr.quant_bwd.fetch_add(1, std::memory_order_relaxed);
  if (a->mask_kind == RS_MASK_BOOL) g_ctr.masked_bool.fetch_add(1, std::memory_order_relaxed);
  if (a->mask_kind == RS_MASK_ADDITIVE) g_ctr.masked_additive.fetch_add(1, std::memory_order_relaxed);
  if (causal) g_ctr.causal.fetch_add(1, std::memory_order_relaxed);
  return RS_OK;
}

rs_status rope_sdpa_rotate(const rs_tensor* x, const rs_tensor* cos, const rs_tensor* sin, const rs_tensor* out,
                           void* stream) {
  if (!x || !cos || !sin || !out) return fail(RS_ERR_NULL);
  const int dt = x->dtype;
  if (dt != RS_F32 && dt != RS_F16 && dt != RS_BF16) return fail(RS_ERR_DTYPE);
  Shape s{};
  s.B = x->size[0];
  s.H = x->size[1];
  s.S = x->size[2];
  s.D = x->size[3];
  s.dtype = dt;
  if (s.B < 0 || s.H < 0 || s.S < 0) return fail(RS_ERR_SHAPE);
  s.empty = s.B == 0 || s.H == 0 || s.S == 0;
  if (s.D != 64 && s.D != 128) return fail(RS_ERR_SHAPE);
  if (s.B * s.H * s.S >= ((int64_t)1 << 31)) return fail(RS_ERR_SHAPE);
  const int64_t sz[4] = {s.B, s.H, s.S, s.D};
  rs_status st;
  if ((st = check_bhsd(x, dt, sz, s.empty)) != RS_OK) return fail(st);
  if (out->data && out->dtype != dt) return fail(RS_ERR_DTYPE);
  if ((st = check_bhsd(out, dt, sz, s.empty)) != RS_OK) return fail(st);
  int64_t bt_c = 0, bt_s = 0;
  if ((st = check_table(cos, s, &bt_c)) != RS_OK) return fail(st);
  if ((st = check_table(sin, s, &bt_s)) != RS_OK) return fail(st);
  if (bt_c != bt_s) return fail(RS_ERR_SHAPE);
  if (s.empty) return RS_OK;
  if ((st = current_device_ok()) != RS_OK) return fail(st);
  RotateParams rp{};
  rp.x = opnd(x);
  rp.out = out->data;
  rp.o_sb = out->stride[0];
  rp.o_sh = out->stride[1];
  rp.o_ss = out->stride[2];
  rp.cos = (const float*)cos->data;
  rp.sin = (const float*)sin->data;
  rp.c_sb = cos->size[0] > 1 ? cos->stride[0] : 0;
  rp.c_ss = cos->stride[2];
  rp.s_sb = sin->size[0] > 1 ? sin->stride[0] : 0;
  rp.s_ss = sin->stride[2];
  rp.B = (int)s.B;
  rp.H = (int)s.H;
  rp.S = (int)s.S;
  rp.D = (int)s.D;
  if (launch_rotate(dt, rp, stream) != 0) return fail(RS_ERR_LAUNCH);
  return RS_OK;
}

void rope_sdpa_get_stats(rs_stats* out) {
  if (!out) return;
  std::memset(out, 0, sizeof(*out));
  out->fwd_instream = g_ctr.fwd_instream.load();
  out->fwd_autograd = g_ctr.fwd_autograd.load();
  out->bwd_calls = g_ctr.bwd_calls.load();
  out->masked_bool = g_ctr.masked_bool.load();
  out->masked_additive = g_ctr.masked_additive.load();
  out->causal = g_ctr.causal.load();
  out->quant_int8 = g_ctr.quant_int8.load();
  out->errors = g_ctr.errors.load();
  out->quant_bwd = g_ctr.quant_bwd.load();
  if (current_device_ok() == RS_OK) {
    uint64_t v = 0;
    if (hipDeviceSynchronize() == hipSuccess && read_all_true_counter(&v, false) == 0) out->mask_all_true_skipped = v;
  }
}

void rope_sdpa_reset_stats(void) {
  g_ctr.fwd_instream = 0;
  g_ctr.fwd_autograd = 0;
  g_ctr.bwd_calls = 0;
  g_ctr.masked_bool = 0;
  g_ctr.masked_additive = 0;
  g_ctr.causal = 0;
  g_ctr.quant_int8 = 0;
  g_ctr.quant_bwd = 0;
  g_ctr.errors = 0;
  if (current_device_ok() == RS_OK) {
    uint64_t v = 0;
    if (hipDeviceSynchronize() == hipSuccess) read_all_true_counter(&v, true);
  }
}

}  // extern "C"
