// Drives the C ABI of include/rope_sdpa.h on the host only (HIP runtime calls and kernel
// launchers replaced by tests/host/hip_stubs.cpp), built with g++ under AddressSanitizer and
// UndefinedBehaviorSanitizer: valid calls of every kind must return RS_OK with every
// workspace-derived pointer inside the workspace; invalid calls must return the documented
// status and launch nothing.  Device pointers are fake, aligned addresses that the host code
// must never dereference.  Exit status 0 = all checks passed.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <vector>

#include "rope_sdpa.h"

namespace stub {
extern const char* ws_lo;
extern size_t ws_bytes;
extern int launches;
extern bool no_device;
}  // namespace stub

static int g_fail = 0, g_checks = 0;
#define CHECK(cond, ...)                          \
  do {                                            \
    ++g_checks;                                   \
    if (!(cond)) {                                \
      ++g_fail;                                   \
      std::fprintf(stderr, "FAIL line %d: ", __LINE__); \
      std::fprintf(stderr, __VA_ARGS__);          \
      std::fprintf(stderr, "\n");                 \
    }                                             \
  } while (0)

static uintptr_t g_next = (uintptr_t)1 << 40;  // fake device addresses, 4 KiB apart
static void* fake_ptr() {
  g_next += 4096;
  return (void*)g_next;
}

static size_t esize(int dt) { return dt == RS_F32 ? 4 : dt == RS_BOOL ? 1 : 2; }

// A contiguous tensor of the given sizes (strides in elements).
static rs_tensor tensor(int dt, int64_t s0, int64_t s1, int64_t s2, int64_t s3) {
  rs_tensor t{};
  t.data = fake_ptr();
  t.dtype = dt;
  t.size[0] = s0;
  t.size[1] = s1;
  t.size[2] = s2;
  t.size[3] = s3;
  t.stride[3] = 1;
  t.stride[2] = s3;
  t.stride[1] = s2 * s3;
  t.stride[0] = s1 * s2 * s3;
  return t;
}

struct Case {
  rs_tensor q, k, v, cos, sin, mask, o, dout, dq, dk, dv;
  rs_args a{};
  bool has_mask = false;
  Case(int dt, int64_t B, int64_t H, int64_t S, int64_t D, int64_t Bt = 1, int64_t Hkv = -1) {
    if (Hkv < 0) Hkv = H;
    q = tensor(dt, B, H, S, D);
    k = tensor(dt, B, Hkv, S, D);
    v = tensor(dt, B, Hkv, S, D);
    o = tensor(dt, B, H, S, D);
    dout = tensor(dt, B, H, S, D);
    dq = tensor(dt, B, H, S, D);
    dk = tensor(dt, B, Hkv, S, D);
    dv = tensor(dt, B, Hkv, S, D);
    cos = tensor(RS_F32, Bt, 1, S, D);
    sin = tensor(RS_F32, Bt, 1, S, D);
    link();
  }
  void link() {
    a.q = &q;
    a.k = &k;
    a.v = &v;
    a.cos = &cos;
    a.sin = &sin;
    a.mask = has_mask ? &mask : nullptr;
  }
  void set_mask(int kind, int dt, int64_t m0, int64_t m1, int64_t m2, int64_t m3) {
    mask = tensor(dt, m0, m1, m2, m3);
    if (m3 > 1) {  // rows padded to 16 bytes
      const int64_t per = 16 / (int64_t)esize(dt);
      const int64_t row = (m3 + per - 1) / per * per;
      mask.stride[2] = row;
      mask.stride[1] = m2 * row;
      mask.stride[0] = m1 * m2 * row;
    }
    has_mask = true;
    a.mask_kind = kind;
    link();
  }
};

// Runs forward (and backward when asked) with an exactly sized, 256-byte aligned workspace.
static rs_status run(Case& c, bool backward, size_t ws_slack = 0, size_t ws_shift = 0) {
  size_t n = 0;
  rs_status st = rope_sdpa_workspace_size(&c.a, backward ? 1 : 0, &n);
  if (st != RS_OK) return st;
  std::vector<char> buf(n + 512 + ws_slack);
  char* ws = (char*)(((uintptr_t)buf.data() + 255) / 256 * 256) + ws_shift;
  stub::ws_lo = ws;
  stub::ws_bytes = n + ws_slack;
  float* lse = (float*)fake_ptr();
  if (!backward) return rope_sdpa_fwd(&c.a, &c.o, lse, n ? ws : nullptr, n + ws_slack, nullptr);
  return rope_sdpa_bwd(&c.a, &c.o, lse, &c.dout, &c.dq, &c.dk, &c.dv, n ? ws : nullptr, n + ws_slack, nullptr);
}

static void expect_error(Case& c, bool backward, rs_status want, const char* what) {
  const int before = stub::launches;
  const rs_status st = run(c, backward);
  CHECK(st == want, "%s: got %d, want %d", what, (int)st, (int)want);
  CHECK(stub::launches == before, "%s: launched after an error", what);
}

int main() {
  const int dts[3] = {RS_F32, RS_F16, RS_BF16};
  // ---- valid calls: every dtype, head dim, mask kind, causal, int8, per-sample tables --------
  for (int dt : dts)
    for (int D : {64, 128})
      for (int S : {1, 77, 300, 1104})
        for (int variant = 0; variant < 7; ++variant)
          for (int bwd = 0; bwd < 2; ++bwd) {
            Case c(dt, 2, 3, S, D, variant == 6 ? 2 : 1);
            if (variant == 1) c.a.flags = RS_FLAG_CAUSAL;
            if (variant == 2) c.set_mask(RS_MASK_BOOL, RS_BOOL, 2, 1, 1, S);
            if (variant == 3) c.set_mask(RS_MASK_BOOL, RS_BOOL, 2, 3, S, S);
            if (variant == 4) c.set_mask(RS_MASK_ADDITIVE, RS_F32, 1, 3, S, S);
            if (variant == 5) c.set_mask(RS_MASK_ADDITIVE, dt, 2, 3, 1, S);
            const int before = stub::launches;
            const rs_status st = run(c, bwd != 0);
            CHECK(st == RS_OK, "valid call dt=%d D=%d S=%d variant=%d bwd=%d: status %d", dt, D, S, variant, bwd,
                  (int)st);
            CHECK(stub::launches > before, "valid call launched nothing");
          }
  // grouped-query attention: 6 query heads over 3, 2 or 1 K/V heads
  for (int dt : dts)
    for (int Hkv : {3, 2, 1})
      for (int bwd = 0; bwd < 2; ++bwd) {
        Case c(dt, 2, 6, 300, 128, 1, Hkv);
        CHECK(run(c, bwd != 0) == RS_OK, "GQA dt=%d Hkv=%d bwd=%d", dt, Hkv, bwd);
        Case ci(dt == RS_F32 ? RS_BF16 : dt, 2, 6, 300, 128, 1, Hkv);
        ci.a.flags = RS_FLAG_QUANT_INT8_QK | (bwd ? RS_FLAG_QUANT_INT8_PREPASS : 0u);
        CHECK(run(ci, false) == RS_OK, "GQA int8 Hkv=%d", Hkv);
      }
  for (int dt : {RS_F16, RS_BF16})
    for (int S : {64, 77, 4608})
      for (uint32_t bits : {(uint32_t)RS_FLAG_QUANT_INT8_QK, (uint32_t)RS_FLAG_QUANT_INT4_QK})
        for (uint32_t extra : {0u, (uint32_t)RS_FLAG_QUANT_INT8_PREPASS}) {
          Case c(dt, 1, 4, S, 128);
          c.a.flags = bits | extra;
          CHECK(run(c, false) == RS_OK, "quantized forward S=%d flags=%u", S, bits | extra);
        }
  { Case c(RS_BF16, 1, 2, 128, 64); c.a.flags = RS_FLAG_QUANT_INT8_QK | RS_FLAG_QUANT_INT4_QK;
    expect_error(c, false, RS_ERR_INVALID, "int8 and int4"); }
  // the quantized forward and backward take every mask kind and causal
  for (uint32_t bits : {(uint32_t)RS_FLAG_QUANT_INT8_QK, (uint32_t)RS_FLAG_QUANT_INT4_QK})
    for (int variant = 0; variant < 4; ++variant)
      for (int bwd = 0; bwd < 2; ++bwd) {
        Case c(RS_BF16, 2, 3, 300, 128);
        c.a.flags = bits;
        if (variant == 1) c.a.flags |= RS_FLAG_CAUSAL;
        if (variant == 2) c.set_mask(RS_MASK_BOOL, RS_BOOL, 2, 1, 1, 300);
        if (variant == 3) c.set_mask(RS_MASK_ADDITIVE, RS_BF16, 1, 3, 300, 300);
        CHECK(run(c, bwd != 0) == RS_OK, "quantized flags=%u variant=%d bwd=%d", bits, variant, bwd);
      }
  { Case c(RS_BF16, 1, 2, 128, 64); c.a.flags = RS_FLAG_QUANT_INT8_PREPASS;
    expect_error(c, false, RS_ERR_INVALID, "prepass without int8"); }
  // plain attention (no tables): forward only
  for (int dt : dts)
    for (int variant = 0; variant < 3; ++variant) {
      Case c(dt, 2, 3, 300, 128);
      c.a.cos = c.a.sin = nullptr;
      if (variant == 1) c.a.flags = RS_FLAG_CAUSAL;
      if (variant == 2) c.set_mask(RS_MASK_BOOL, RS_BOOL, 2, 1, 1, 300);
      c.a.cos = c.a.sin = nullptr;  // (set_mask relinks them)
      CHECK(run(c, false) == RS_OK, "plain forward dt=%d variant=%d", dt, variant);
      c.a.cos = c.a.sin = nullptr;
      expect_error(c, true, RS_ERR_UNSUPPORTED, "plain backward");
    }
  // fp32 Q/K beside 16-bit V, and the Q/K RMSNorm prologue: forward only
  for (int dt : dts)
    for (int mixed = 0; mixed < 2; ++mixed)
      for (int norm = 0; norm < 2; ++norm)
        for (int variant = 0; variant < 4; ++variant) {
          if (!mixed && !norm) continue;
          if (mixed && dt == RS_F32) continue;
          Case c(dt, 2, 6, 300, variant == 3 ? 64 : 128, variant == 3 ? 2 : 1, variant == 3 ? 2 : 6);
          if (mixed) c.q.dtype = c.k.dtype = RS_F32;
          if (norm) {
            c.a.q_norm_weight = (const float*)fake_ptr();
            c.a.k_norm_weight = (const float*)fake_ptr();
            c.a.norm_eps = 1e-6f;
          }
          if (variant == 1) c.a.flags = RS_FLAG_CAUSAL;
          if (variant == 2) c.set_mask(RS_MASK_BOOL, RS_BOOL, 2, 1, 1, 300);
          CHECK(run(c, false) == RS_OK, "Q/K prologue dt=%d mixed=%d norm=%d variant=%d", dt, mixed, norm, variant);
          expect_error(c, true, RS_ERR_UNSUPPORTED, "Q/K prologue backward");
          c.set_mask(RS_MASK_ADDITIVE, RS_F32, 1, 1, 1, 300);
          c.a.flags = 0;
          expect_error(c, false, RS_ERR_UNSUPPORTED, "Q/K prologue with an additive mask");
        }
  { Case c(RS_BF16, 1, 2, 128, 64); c.q.dtype = c.k.dtype = RS_F32; c.a.cos = c.a.sin = nullptr;
    expect_error(c, false, RS_ERR_UNSUPPORTED, "fp32 Q/K without tables"); }
  { Case c(RS_BF16, 1, 2, 128, 64); c.q.dtype = c.k.dtype = RS_F32; c.a.flags = RS_FLAG_QUANT_INT8_QK;
    expect_error(c, false, RS_ERR_UNSUPPORTED, "fp32 Q/K with int8"); }
  { Case c(RS_BF16, 1, 2, 128, 64); c.a.q_norm_weight = (const float*)fake_ptr();
    expect_error(c, false, RS_ERR_INVALID, "one norm weight"); }
  { Case c(RS_BF16, 1, 2, 128, 64); c.a.q_norm_weight = (const float*)fake_ptr();
    c.a.k_norm_weight = (const float*)fake_ptr(); c.a.norm_eps = -1.f;
    expect_error(c, false, RS_ERR_INVALID, "negative norm eps"); }
  { Case c(RS_BF16, 1, 2, 128, 64); c.a.q_norm_weight = (const float*)fake_ptr();
    c.a.k_norm_weight = (const float*)((uintptr_t)fake_ptr() + 4);
    expect_error(c, false, RS_ERR_ALIGN, "misaligned norm weight"); }
  { Case c(RS_BF16, 1, 2, 128, 64); c.a.sin = nullptr; expect_error(c, false, RS_ERR_NULL, "one table missing"); }
  { Case c(RS_BF16, 1, 2, 128, 64); c.a.cos = c.a.sin = nullptr; c.a.flags = RS_FLAG_QUANT_INT8_QK;
    expect_error(c, false, RS_ERR_UNSUPPORTED, "int8 without tables"); }
  // the eager rotation pass
  for (int dt : dts) {
    Case c(dt, 2, 3, 77, 128, 2);
    const int before = stub::launches;
    CHECK(rope_sdpa_rotate(&c.q, &c.cos, &c.sin, &c.o, nullptr) == RS_OK, "rotate dt=%d", dt);
    CHECK(rope_sdpa_rotate(&c.q, &c.cos, &c.sin, &c.q, nullptr) == RS_OK, "rotate in place dt=%d", dt);
    CHECK(stub::launches == before + 2, "rotate launches");
    c.o.dtype = dt == RS_F32 ? RS_BF16 : RS_F32;
    CHECK(rope_sdpa_rotate(&c.q, &c.cos, &c.sin, &c.o, nullptr) == RS_ERR_DTYPE, "rotate out dtype");
    CHECK(rope_sdpa_rotate(&c.q, &c.cos, nullptr, &c.o, nullptr) == RS_ERR_NULL, "rotate without sin");
    Case e(dt, 2, 3, 77, 96);
    CHECK(rope_sdpa_rotate(&e.q, &e.cos, &e.sin, &e.o, nullptr) == RS_ERR_SHAPE, "rotate D = 96");
    CHECK(stub::launches == before + 2, "rotate launched on error");
  }
  // K rotated by a pass of its own (RS_FLAG_K_PREPASS): 16-bit, rotating, no quantization, no
  // additive mask
  for (int dt : {RS_F16, RS_BF16})
    for (int variant = 0; variant < 4; ++variant) {
      Case c(dt, 2, 6, 300, variant == 3 ? 64 : 128, variant == 3 ? 2 : 1, variant == 3 ? 3 : 6);
      c.a.flags = RS_FLAG_K_PREPASS;
      if (variant == 1) c.a.flags |= RS_FLAG_CAUSAL;
      if (variant == 2) c.set_mask(RS_MASK_BOOL, RS_BOOL, 2, 1, 1, 300);
      CHECK(run(c, false) == RS_OK, "K pre-pass dt=%d variant=%d", dt, variant);
    }
  { Case c(RS_F32, 1, 2, 128, 64); c.a.flags = RS_FLAG_K_PREPASS; expect_error(c, false, RS_ERR_UNSUPPORTED, "K pre-pass fp32"); }
  { Case c(RS_BF16, 1, 2, 128, 64); c.a.flags = RS_FLAG_K_PREPASS | RS_FLAG_QUANT_INT8_QK;
    expect_error(c, false, RS_ERR_UNSUPPORTED, "K pre-pass int8"); }
  { Case c(RS_BF16, 1, 2, 128, 64); c.a.flags = RS_FLAG_K_PREPASS; c.set_mask(RS_MASK_ADDITIVE, RS_F32, 1, 1, 1, 128);
    expect_error(c, false, RS_ERR_UNSUPPORTED, "K pre-pass additive"); }
  { Case c(RS_BF16, 1, 2, 128, 64); c.a.flags = RS_FLAG_K_PREPASS; c.a.cos = c.a.sin = nullptr;
    expect_error(c, false, RS_ERR_UNSUPPORTED, "K pre-pass without tables"); }
  // kernel timing for measurement: one event pair per timed forward call
  {
    CHECK(rope_sdpa_debug_kernel_timing(1) == RS_OK, "timing on");
    for (int i = 0; i < 3; ++i) {
      Case c(RS_BF16, 1, 2, 300, 128);
      CHECK(run(c, false) == RS_OK, "timed forward");
    }
    double ms = -1.0;
    uint64_t n = 0;
    CHECK(rope_sdpa_debug_kernel_time(&ms, &n) == RS_OK && n == 3 && ms == 0.75, "timing read: %llu calls, %g ms",
          (unsigned long long)n, ms);
    CHECK(rope_sdpa_debug_kernel_time(nullptr, &n) == RS_ERR_NULL, "timing read NULL");
    CHECK(rope_sdpa_debug_kernel_timing(0) == RS_OK, "timing off");
    Case c(RS_BF16, 1, 2, 300, 128);
    CHECK(run(c, false) == RS_OK, "untimed forward");
    CHECK(rope_sdpa_debug_kernel_time(&ms, &n) == RS_OK && n == 0, "timing off: no pairs");
  }
  // empty calls: no workspace, nothing launched, data pointers may be NULL
  for (int e = 0; e < 3; ++e) {
    Case c(RS_BF16, e == 0 ? 0 : 2, e == 1 ? 0 : 3, e == 2 ? 0 : 64, 64);
    c.q.data = c.k.data = c.v.data = c.o.data = nullptr;
    size_t n = 1;
    CHECK(rope_sdpa_workspace_size(&c.a, 0, &n) == RS_OK && n == 0, "empty workspace size");
    const int before = stub::launches;
    CHECK(rope_sdpa_fwd(&c.a, &c.o, nullptr, nullptr, 0, nullptr) == RS_OK, "empty forward");
    CHECK(stub::launches == before, "empty forward launched");
  }

  // ---- invalid calls ---------------------------------------------------------------------
  {
    size_t n;
    CHECK(rope_sdpa_workspace_size(nullptr, 0, &n) == RS_ERR_NULL, "null args");
    Case c(RS_BF16, 1, 2, 128, 64);
    CHECK(rope_sdpa_workspace_size(&c.a, 0, nullptr) == RS_ERR_NULL, "null size pointer");
  }
  { Case c(RS_BF16, 1, 2, 128, 64); c.a.q = nullptr; expect_error(c, false, RS_ERR_NULL, "null q"); }
  { Case c(RS_BF16, 1, 2, 128, 64); c.q.data = nullptr; expect_error(c, false, RS_ERR_NULL, "null q data"); }
  { Case c(RS_BF16, 1, 2, 128, 64); c.q.dtype = RS_F16; c.k.dtype = RS_F16; expect_error(c, false, RS_ERR_DTYPE, "f16 Q/K with bf16 V"); }
  { Case c(RS_F32, 1, 2, 128, 64); c.q.dtype = c.k.dtype = RS_BF16; expect_error(c, false, RS_ERR_DTYPE, "bf16 Q/K with f32 V"); }
  { Case c(RS_BF16, 1, 2, 128, 64); c.q.dtype = RS_F32; expect_error(c, false, RS_ERR_DTYPE, "fp32 Q with bf16 K"); }
  { Case c(RS_BF16, 1, 2, 128, 64); c.o.dtype = RS_F16; expect_error(c, false, RS_ERR_DTYPE, "output dtype"); }
  { Case c(RS_BOOL, 1, 2, 128, 64); expect_error(c, false, RS_ERR_DTYPE, "bool q"); }
  { Case c(RS_BF16, 1, 2, 128, 96); expect_error(c, false, RS_ERR_SHAPE, "D = 96"); }
  { Case c(RS_BF16, 1, 6, 128, 64, 1, 4); expect_error(c, false, RS_ERR_SHAPE, "H % Hkv != 0"); }
  { Case c(RS_BF16, 1, 6, 128, 64, 1, 2); c.v.size[1] = 3; expect_error(c, false, RS_ERR_SHAPE, "V heads differ from K"); }
  { Case c(RS_BF16, 1, 6, 128, 64, 1, 2); c.dk.size[1] = 6; expect_error(c, true, RS_ERR_SHAPE, "dK at the query head count"); }
  { Case c(RS_BF16, 1, 2, 128, 64); c.k.size[2] = 127; expect_error(c, false, RS_ERR_SHAPE, "K rows"); }
  { Case c(RS_BF16, 1, 2, 128, 64); c.q.stride[3] = 2; expect_error(c, false, RS_ERR_STRIDE, "stride[3]"); }
  { Case c(RS_BF16, 1, 2, 128, 64); c.v.stride[2] = 65; expect_error(c, false, RS_ERR_STRIDE, "row stride"); }
  { Case c(RS_BF16, 1, 2, 128, 64); c.q.stride[2] = (int64_t)1 << 23; expect_error(c, false, RS_ERR_STRIDE, "huge row stride"); }
  { Case c(RS_BF16, 1, 2, 128, 64); c.q.data = (char*)c.q.data + 8; expect_error(c, false, RS_ERR_ALIGN, "q base"); }
  { Case c(RS_BF16, 1, 2, 128, 64); c.q.reserved = 1; expect_error(c, false, RS_ERR_INVALID, "reserved"); }
  { Case c(RS_BF16, 1, 2, 128, 64); c.a.flags = 1u << 7; expect_error(c, false, RS_ERR_INVALID, "unknown flag"); }
  { Case c(RS_BF16, 1, 2, 128, 64); c.a.scale = -1.f; expect_error(c, false, RS_ERR_INVALID, "negative scale"); }
  { Case c(RS_BF16, 1, 2, 128, 64); c.a.scale = std::nanf(""); expect_error(c, false, RS_ERR_INVALID, "NaN scale"); }
  { Case c(RS_BF16, 1, 2, 128, 64); c.a.mask_kind = 7; expect_error(c, false, RS_ERR_INVALID, "mask kind"); }
  { Case c(RS_BF16, 1, 2, 128, 64); c.set_mask(RS_MASK_BOOL, RS_BOOL, 1, 1, 1, 128); c.a.flags = RS_FLAG_CAUSAL;
    expect_error(c, false, RS_ERR_INVALID, "causal with a mask"); }
  { Case c(RS_BF16, 1, 2, 128, 64); c.set_mask(RS_MASK_BOOL, RS_F32, 1, 1, 1, 128); expect_error(c, false, RS_ERR_DTYPE, "bool mask dtype"); }
  { Case c(RS_BF16, 1, 2, 128, 64); c.set_mask(RS_MASK_ADDITIVE, RS_F16, 1, 1, 1, 128); expect_error(c, false, RS_ERR_DTYPE, "additive mask dtype"); }
  { Case c(RS_BF16, 2, 2, 128, 64); c.set_mask(RS_MASK_BOOL, RS_BOOL, 3, 1, 1, 128); expect_error(c, false, RS_ERR_SHAPE, "mask batch"); }
  { Case c(RS_BF16, 1, 2, 128, 64); c.set_mask(RS_MASK_ADDITIVE, RS_F32, 1, 1, 128, 128); c.mask.stride[2] = 130;
    expect_error(c, false, RS_ERR_STRIDE, "mask row stride"); }
  { Case c(RS_BF16, 1, 2, 128, 64); c.a.mask_kind = RS_MASK_BOOL; expect_error(c, false, RS_ERR_NULL, "bool kind without mask"); }
  { Case c(RS_BF16, 1, 2, 128, 64); c.set_mask(RS_MASK_BOOL, RS_BOOL, 1, 1, 1, 128); c.a.mask_kind = RS_MASK_NONE;
    expect_error(c, false, RS_ERR_INVALID, "mask with kind none"); }
  { Case c(RS_BF16, 1, 2, 128, 64); c.cos.size[2] = 64; expect_error(c, false, RS_ERR_SHAPE, "table rows"); }
  { Case c(RS_BF16, 1, 2, 128, 64); c.cos.dtype = RS_F16; expect_error(c, false, RS_ERR_DTYPE, "table dtype"); }
  { Case c(RS_BF16, 2, 2, 128, 64, 2); c.sin.size[0] = 1; c.sin.stride[0] = 0; expect_error(c, false, RS_ERR_SHAPE, "table batch mismatch"); }
  { Case c(RS_F32, 1, 2, 128, 64); c.a.flags = RS_FLAG_QUANT_INT8_QK; expect_error(c, false, RS_ERR_UNSUPPORTED, "int8 fp32"); }
  // the quantized backward: int8 and int4, D = 64 and 128, grouped-query included
  for (uint32_t bits : {(uint32_t)RS_FLAG_QUANT_INT8_QK, (uint32_t)RS_FLAG_QUANT_INT4_QK})
    for (int D : {64, 128})
      for (int Hkv : {4, 2}) {
        Case c(RS_BF16, 2, 4, 300, D, 1, Hkv);
        c.a.flags = bits;
        CHECK(run(c, true) == RS_OK, "quantized backward flags=%u D=%d Hkv=%d", bits, D, Hkv);
      }
  { Case c(RS_BF16, 1, 2, 128, 64);
    const int before = stub::launches;
    std::vector<char> buf(1 << 20);
    char* ws = (char*)(((uintptr_t)buf.data() + 255) / 256 * 256);
    size_t n = 0;
    rope_sdpa_workspace_size(&c.a, 0, &n);
    CHECK(rope_sdpa_fwd(&c.a, &c.o, nullptr, ws, n - 1, nullptr) == RS_ERR_WORKSPACE, "workspace one byte short");
    CHECK(rope_sdpa_fwd(&c.a, &c.o, nullptr, nullptr, n, nullptr) == RS_ERR_WORKSPACE, "null workspace");
    CHECK(rope_sdpa_fwd(&c.a, &c.o, nullptr, ws + 16, n, nullptr) == RS_ERR_ALIGN, "workspace alignment");
    CHECK(rope_sdpa_fwd(&c.a, &c.o, (float*)((char*)fake_ptr() + 2), ws, n, nullptr) == RS_ERR_ALIGN, "lse alignment");
    CHECK(rope_sdpa_bwd(&c.a, &c.o, nullptr, &c.dout, &c.dq, &c.dk, &c.dv, ws, n, nullptr) == RS_ERR_NULL, "bwd without lse");
    CHECK(stub::launches == before, "an invalid call launched"); }
  { Case c(RS_BF16, 1, 2, 128, 64);
    stub::no_device = true;
    expect_error(c, false, RS_ERR_NO_DEVICE, "no device");
    stub::no_device = false; }

  // status strings and stats
  for (int s = 0; s >= -12; --s) CHECK(rope_sdpa_status_string((rs_status)s) != nullptr, "status string %d", s);
  rs_stats stats{};
  rope_sdpa_get_stats(&stats);
  CHECK(stats.errors > 0 && stats.fwd_autograd > 0 && stats.bwd_calls > 0, "stats");
  rope_sdpa_reset_stats();
  rope_sdpa_get_stats(&stats);
  CHECK(stats.errors == 0 && stats.fwd_autograd == 0, "reset stats");
  CHECK(rope_sdpa_abi_version() == ROPE_SDPA_ABI_VERSION, "abi version");

  std::printf("%d checks, %d failed, %d launches\n", g_checks, g_fail, stub::launches);
  return g_fail == 0 ? 0 : 1;
}
