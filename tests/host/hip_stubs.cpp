// Host-only stand-ins for the HIP runtime calls and kernel launchers of the library, so that
// its host code (argument validation, workspace layout, parameter blocks) can be built with
// g++ under AddressSanitizer / UndefinedBehaviorSanitizer and run without a GPU.
//
// The launchers launch nothing.  They count calls and check that every pointer the host code
// derived from the caller's workspace lies inside it, with room for what the kernel writes
// or reads there; a violation aborts the run.
#include <hip/hip_runtime.h>

#include <cstdio>
#include <cstdlib>
#include <cstring>

#include "rs_internal.h"

namespace stub {
const char* ws_lo = nullptr;  // the workspace of the call in progress (set by the driver)
size_t ws_bytes = 0;
int launches = 0;
bool no_device = false;

void need(const void* p, size_t bytes, const char* what) {
  const char* c = (const char*)p;
  if (!ws_lo || c < ws_lo || c + bytes > ws_lo + ws_bytes) {
    std::fprintf(stderr, "workspace range violated: %s [%p, +%zu) outside [%p, +%zu)\n", what, p, bytes,
                 (const void*)ws_lo, ws_bytes);
    std::abort();
  }
}
}  // namespace stub

extern "C" {
hipError_t hipGetDevice(int* dev) {
  if (stub::no_device) return hipErrorNoDevice;
  *dev = 0;
  return hipSuccess;
}
hipError_t hipGetDevicePropertiesR0600(hipDeviceProp_tR0600* prop, int) {
  std::memset(prop, 0, sizeof(*prop));
  std::strcpy(prop->gcnArchName, "gfx950:sramecc+:xnack-");
  return hipSuccess;
}
hipError_t hipDeviceSynchronize(void) { return hipSuccess; }
// events: fake handles, never dereferenced by the host code
hipError_t hipEventCreate(hipEvent_t* e) {
  static uintptr_t next = 0x1000;
  next += 16;
  *e = (hipEvent_t)next;
  return hipSuccess;
}
hipError_t hipEventDestroy(hipEvent_t) { return hipSuccess; }
hipError_t hipEventSynchronize(hipEvent_t e) { return e ? hipSuccess : hipErrorInvalidValue; }
hipError_t hipEventElapsedTime(float* ms, hipEvent_t a, hipEvent_t b) {
  if (!a || !b || a == b) return hipErrorInvalidValue;
  *ms = 0.25f;
  return hipSuccess;
}
}

namespace rs {

int fwd_block_m(int dtype) { return dtype == F32 ? 128 : 256; }
int fwd_block_n(int dtype) { return dtype == F32 ? 32 : 64; }

// A split plan of the same form as the device planner's (whole units, then ranges of the
// remaining units' key tiles over further workgroups) on a pretend 8-workgroup device, so
// that the layout of the pieces' slots is exercised.
SplitPlan fwd_split_plan(int dtype, int D, bool, bool causal, int, int64_t units, int nkt) {
  SplitPlan sp{};
  if (causal || units <= 8 || units % 8 == 0 || nkt < 4) return sp;
  sp.full = (int)(units / 8 * 8);
  sp.cut_units = units - sp.full;
  sp.grid = 8;
  sp.iters = sp.cut_units * nkt;
  sp.slot_bytes = (size_t)fwd_block_m(dtype) * D * (dtype == F32 ? 4 : 2);
  return sp;
}

int launch_pack_tables(const PackParams& p, void*) {
  ++stub::launches;
  stub::need(p.out, (size_t)p.Bt * p.S * p.D * sizeof(float), "packed tables");
  stub::need(p.ctrl, 2 * sizeof(unsigned), "control words");
  return 0;
}

int launch_classify(const ClassifyParams& p, void*) {
  ++stub::launches;
  const int64_t nq = (p.Sq + kMaskTile - 1) / kMaskTile, nk = (p.Sk + kMaskTile - 1) / kMaskTile;
  stub::need(p.tiles, (size_t)(p.nb * p.nh * nq * nk), "mask tile states");
  stub::need(p.ctrl, 2 * sizeof(unsigned), "control words");
  if (p.total_blocks != p.nb * p.nh * nq * nk) std::abort();
  return 0;
}

int launch_fwd(int dtype, int D, int, bool, int int8, const FwdParams& p, void*) {
  ++stub::launches;
  const int B = p.shp.B, H = p.shp.H, S = p.shp.S;
  stub::need(p.tab.ptr, (size_t)(p.tab.sb ? B : 1) * S * D * sizeof(float), "packed tables");
  if (p.mask.tiles) stub::need(p.mask.tiles, 1, "mask tile states");
  if (p.shp.Hkv <= 0 || H % p.shp.Hkv != 0 || p.shp.group != H / p.shp.Hkv) std::abort();
  if (int8 && (p.xq_codes || p.xk_codes)) std::abort();  // the forward never exports codes
  if (int8 != 0 && int8 != 1 && int8 != 2 && int8 != 5 && int8 != 6) std::abort();
  if ((int8 & 3) == 2) {  // codes and scales of the quantizer pass in the workspace
    stub::need(p.qc, (size_t)B * H * p.sp * D, "q codes");
    stub::need(p.kc, (size_t)B * p.shp.Hkv * p.sp * D, "k codes");
    stub::need(p.qsc, (size_t)B * H * (p.sp / 64) * sizeof(float), "q scales");
    stub::need(p.ksc, (size_t)B * p.shp.Hkv * (p.sp / 64) * sizeof(float), "k scales");
  } else if (p.qc || p.kc) {
    std::abort();
  }
  if (p.split_iters > 0) {
    const size_t bm = (size_t)fwd_block_m(dtype), es = dtype == F32 ? 4 : 2;
    stub::need(p.part_o, 2 * (size_t)p.split_grid * bm * D * es, "pieces' outputs");
    stub::need(p.part_lse, 2 * (size_t)p.split_grid * bm * sizeof(float), "pieces' LSE");
  }
  return 0;
}

int launch_fwd_plain(int, int, int, bool, const FwdParams& p, void*) {
  ++stub::launches;
  if (p.tab.ptr != nullptr) std::abort();  // plain attention reads no tables
  return 0;
}

int launch_kprep(int dtype, int qkm, const KPrepParams& p, void*) {
  ++stub::launches;
  const size_t es = dtype == F32 ? 4 : 2;
  stub::need(p.out, (size_t)p.B * p.H * p.S * p.D * es, "prepared K");
  if (!p.pk.cos || !p.pk.sin || p.pk.Bt < 1 || p.pk.S != p.S || p.pk.D != p.D) std::abort();
  if (p.pk.out) {  // with the table packing
    stub::need(p.pk.out, (size_t)p.pk.Bt * p.S * p.D * sizeof(float), "packed tables");
    stub::need(p.pk.ctrl, 2 * sizeof(unsigned), "control words");
  }
  if ((qkm & 1) != (p.w != nullptr)) std::abort();
  if ((qkm & 2) && dtype == F32) std::abort();
  if (p.D != 64 && p.D != 128) std::abort();
  return 0;
}

int launch_fwd_qk(int dtype, int D, int, bool, int qkm, const FwdParams& p, void*) {
  ++stub::launches;
  const int B = p.shp.B, S = p.shp.S;
  stub::need(p.tab.ptr, (size_t)(p.tab.sb ? B : 1) * S * D * sizeof(float), "packed tables");
  if (qkm < 4 || qkm > 7) std::abort();
  // K is the prepared, contiguous K' in the workspace
  const size_t es = dtype == F32 ? 4 : 2;
  stub::need(p.k.ptr, (size_t)B * p.shp.Hkv * S * D * es, "prepared K");
  if (p.k.ss != D || p.k.sh != (int64_t)S * D || p.k.sb != (int64_t)p.shp.Hkv * S * D) std::abort();
  if ((qkm & 1) != (p.qnw != nullptr) || (p.qnw == nullptr) != (p.knw == nullptr)) std::abort();
  if ((qkm & 2) && dtype == F32) std::abort();  // fp32 Q/K only beside 16-bit V
  if (p.qc || p.kc || p.xq_codes || p.xk_codes) std::abort();
  if (p.split_iters > 0) {
    const size_t bm = (size_t)fwd_block_m(dtype), es = dtype == F32 ? 4 : 2;
    stub::need(p.part_o, 2 * (size_t)p.split_grid * bm * D * es, "pieces' outputs");
    stub::need(p.part_lse, 2 * (size_t)p.split_grid * bm * sizeof(float), "pieces' LSE");
  }
  return 0;
}

int launch_rotate(int, const RotateParams& p, void*) {
  ++stub::launches;
  if (!p.cos || !p.sin || !p.out || p.B <= 0 || p.H <= 0 || p.S <= 0 || (p.D != 64 && p.D != 128)) std::abort();
  return 0;
}

int launch_quant_int8(int, const QuantParams& p, void*) {
  ++stub::launches;
  if (p.qmax != 127.f && p.qmax != 7.f) std::abort();
  if (p.nblk != (p.S + 63) / 64) std::abort();
  if (p.deq[0]) {  // dequantizing mode (the quantized backward): T values, no codes
    for (int w = 0; w < 2; ++w) stub::need(p.deq[w], (size_t)p.B * p.Hx[w] * p.S * p.D * 2, "dequantized values");
    return 0;
  }
  stub::need(p.tab.ptr, (size_t)(p.tab.sb ? p.B : 1) * p.S * p.D * sizeof(float), "packed tables");
  for (int w = 0; w < 2; ++w) {
    stub::need(p.codes[w], (size_t)p.B * p.Hx[w] * p.rows * p.D, "codes");
    stub::need(p.scales[w], (size_t)p.B * p.Hx[w] * p.nblk * sizeof(float), "scales");
  }
  return 0;
}

int launch_fwd_int8_export(int, int, bool, const FwdParams& p, void*) {
  ++stub::launches;
  if (!p.xq_codes || !p.xk_codes || !p.xq_scales || !p.xk_scales || p.split_iters != 0) std::abort();
  stub::need(p.tab.ptr, (size_t)(p.tab.sb ? p.shp.B : 1) * p.shp.S * 4 * 64, "packed tables");
  return 0;
}

int launch_bwd(int dtype, int D, int, bool, int pre, const BwdParams& p, void*) {
  ++stub::launches;
  const int B = p.shp.B, H = p.shp.H, S = p.shp.S;
  if (p.shp.Hkv <= 0 || H % p.shp.Hkv != 0 || p.shp.group != H / p.shp.Hkv) std::abort();
  stub::need(p.tab.ptr, (size_t)(p.tab.sb ? B : 1) * S * D * sizeof(float), "packed tables");
  stub::need(p.delta, (size_t)B * H * S * sizeof(float), "delta");
  if (dtype != F32 && (D == 128 || pre == 3)) {
    stub::need(p.qrot, (size_t)B * H * S * D * 2, "rotated Q");
    if (pre != 1 && pre != 3) std::abort();  // K' prepared in the workspace
    stub::need(p.k.ptr, (size_t)B * p.shp.Hkv * S * D * 2, "prepared K");
    if (p.k.ss != D || p.k.sh != (int64_t)S * D || p.k.sb != (int64_t)p.shp.Hkv * S * D) std::abort();
    if (D != 128 && p.q.ptr != p.qrot) std::abort();  // the 32x32 kernels read Q^' as Q
  } else if (pre != 0) {
    std::abort();
  }
  return 0;
}

int read_all_true_counter(uint64_t* value, bool) {
  *value = 0;
  return 0;
}

// The library's device scratch: host memory standing in for it, registered with the range
// checks of the launchers when looked up.
int scratch_address(void** ptr) {
  static char* mem = nullptr;
  if (!mem) mem = (char*)std::aligned_alloc(256, kScratchBytes);
  stub::ws_lo = mem;
  stub::ws_bytes = kScratchBytes;
  *ptr = mem;
  return 0;
}

}  // namespace rs
