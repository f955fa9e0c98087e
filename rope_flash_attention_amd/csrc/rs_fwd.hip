// Forward launchers (rotation in the kernel), the work split planner and block sizes.  The
// kernel templates are in rs_fwd_kernel.hpp; rs_fwd_plain.hip instantiates the variant
// without rotation.
#include <mutex>

#include "rs_fwd_kernel.hpp"

namespace rs {

// the quantized forward's instantiations, one translation unit per code width
int launch_fwd_q8(int dtype, int D, int mask_kind, bool causal, int mode, const FwdParams& p, void* stream);
int launch_fwd_q4(int dtype, int D, int mask_kind, bool causal, int mode, const FwdParams& p, void* stream);

int launch_fwd(int dtype, int D, int mask_kind, bool causal, int int8, const FwdParams& p, void* stream) {
  if (int8 & 4) return launch_fwd_q4(dtype, D, mask_kind, causal, int8, p, stream);
  if (int8) return launch_fwd_q8(dtype, D, mask_kind, causal, int8, p, stream);
  switch (dtype) {
    case F32: return launch_fwd_dt<float, true>(D, mask_kind, causal, p, stream);
    case F16: return launch_fwd_dt<_Float16, true>(D, mask_kind, causal, p, stream);
    default: return launch_fwd_dt<__bf16, true>(D, mask_kind, causal, p, stream);
  }
}

// The quantized forward in code export mode (tests): one workgroup per unit, no split, no
// output.  QI8 = 1 (int8) or 5 (int4).
template <typename T, int QI8>
static int launch_fwd_int8_export_t(int D, const FwdParams& p, void* stream) {
  return D == 64 ? launch_fwd_t<T, 64, MASK_NONE, false, QI8, true, true>(p, stream)
                 : launch_fwd_t<T, 128, MASK_NONE, false, QI8, true, true>(p, stream);
}

int launch_fwd_int8_export(int dtype, int D, bool int4, const FwdParams& p, void* stream) {
  if (int4)
    return dtype == F16 ? launch_fwd_int8_export_t<_Float16, 5>(D, p, stream)
                        : launch_fwd_int8_export_t<__bf16, 5>(D, p, stream);
  return dtype == F16 ? launch_fwd_int8_export_t<_Float16, 1>(D, p, stream)
                      : launch_fwd_int8_export_t<__bf16, 1>(D, p, stream);
}

int fwd_block_m(int dtype) { return dtype == F32 ? FwdCfg<float>::BM : FwdCfg<__bf16>::BM; }
int fwd_block_n(int dtype) { return dtype == F32 ? FwdCfg<float>::BN : FwdCfg<__bf16>::BN; }
int fwd_waves(int dtype) { return (dtype == F32 ? FwdCfg<float>::NT : FwdCfg<__bf16>::NT) / 64; }

template <typename T, int D, bool QI8>
static int resident_per_cu() {
  int n = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, fwd_kernel<T, D, MASK_NONE, false, QI8 ? 1 : 0>, FwdCfg<T>::NT, 0) !=
      hipSuccess)
    return 0;
  return n;
}

// Resident forward workgroups per CU and CU count, queried once per (device, variant) and
// kept: the split planner runs on every forward call (and on every workspace query).
static int resident_per_cu_query(int dtype, int D, bool int8) {
  const bool d64 = D == 64;
  if (dtype == F32) return d64 ? resident_per_cu<float, 64, false>() : resident_per_cu<float, 128, false>();
  if (dtype == F16)
    return int8 ? (d64 ? resident_per_cu<_Float16, 64, true>() : resident_per_cu<_Float16, 128, true>())
                : (d64 ? resident_per_cu<_Float16, 64, false>() : resident_per_cu<_Float16, 128, false>());
  return int8 ? (d64 ? resident_per_cu<__bf16, 64, true>() : resident_per_cu<__bf16, 128, true>())
              : (d64 ? resident_per_cu<__bf16, 64, false>() : resident_per_cu<__bf16, 128, false>());
}

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_occ_mu;
int g_occ_cus[kMaxDevices] = {0};
int g_occ_per[kMaxDevices][12] = {{0}};  // [dtype (3) x D (2) x int8 (2)], 0 = not queried yet
}  // namespace

static bool occupancy(int dtype, int D, bool int8, int* cus, int* per) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return false;
  const int key = (dtype % 3) * 4 + (D == 64 ? 2 : 0) + (int8 ? 1 : 0);
  std::lock_guard<std::mutex> lk(g_occ_mu);
  if (g_occ_cus[dev] == 0) {
    int c = 0;
    if (hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || c <= 0) return false;
    g_occ_cus[dev] = c;
  }
  if (g_occ_per[dev][key] == 0) {
    const int n = resident_per_cu_query(dtype, D, int8);
    if (n <= 0) return false;
    g_occ_per[dev][key] = n;
  }
  *cus = g_occ_cus[dev];
  *per = g_occ_per[dev][key];
  return true;
}

SplitPlan fwd_split_plan(int dtype, int D, bool int8, bool causal, int mask_kind, int64_t units, int nkt) {
  SplitPlan sp{};
  if (causal || units <= 0 || nkt < 16) return sp;
  int cus = 0, per = 0;
  if (!occupancy(dtype, D, int8, &cus, &per)) return sp;
  const int64_t g = (int64_t)cus * per & ~(int64_t)7;  // resident workgroups, a multiple of 8
  if (g < 8) return sp;
  const int64_t full = units / g * g, cut = units - full;
  if (cut == 0) return sp;
  const int64_t iters = cut * nkt;
  // at least nkt / (kMaxPieces - 1) key tiles per range: a unit then meets at most
  // kMaxPieces ranges (fwd_merge_kernel relies on it)
  const int64_t grid = std::min<int64_t>(g, iters / std::max<int64_t>(8, (nkt + kMaxPieces - 2) / (kMaxPieces - 1)));
  if (grid <= cut) return sp;  // no more workgroups than units: nothing gained
  // time in key-tile steps: one unit per workgroup, against whole units plus an equal share
  // of the rest (plus about two steps for publishing and merging the pieces)
  const int64_t plain = (units + g - 1) / g * nkt;
  const int64_t split = full / g * nkt + (iters + grid - 1) / grid + 2;
  if (split * 100 > plain * 97) return sp;  // keep the plain schedule unless ~3% is gained
  sp.full = (int)full;
  sp.grid = (int)grid;
  sp.iters = iters;
  sp.cut_units = cut;
  sp.slot_bytes = (size_t)fwd_block_m(dtype) * D * (dtype == F32 ? 4 : 2);  // normalized O rows
  return sp;
}

}  // namespace rs
