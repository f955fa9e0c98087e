"""ctypes mirror of include/rope_sdpa.h (argument marshalling only; no compute here)."""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "librope_sdpa.so")

RS_OK = 0
STATUS_NAMES = {
    0: "RS_OK", -1: "RS_ERR_NULL", -2: "RS_ERR_DTYPE", -3: "RS_ERR_SHAPE", -4: "RS_ERR_STRIDE",
    -5: "RS_ERR_ALIGN", -6: "RS_ERR_UNSUPPORTED", -7: "RS_ERR_WORKSPACE", -8: "RS_ERR_INVALID",
    -9: "RS_ERR_NO_DEVICE", -10: "RS_ERR_LAUNCH", -11: "RS_ERR_SCRATCH",
}
RS_F32, RS_F16, RS_BF16, RS_BOOL = 0, 1, 2, 3
RS_MASK_NONE, RS_MASK_BOOL, RS_MASK_ADDITIVE = 0, 1, 2
RS_FLAG_CAUSAL, RS_FLAG_QUANT_INT8_QK, RS_FLAG_QUANT_INT8_PREPASS, RS_FLAG_QUANT_INT4_QK = 1, 2, 4, 8
RS_FLAG_K_PREPASS = 16

# Every symbol include/rope_sdpa.h declares.
EXPORTED = (
    "rope_sdpa_workspace_size", "rope_sdpa_fwd", "rope_sdpa_bwd", "rope_sdpa_status_string",
    "rope_sdpa_get_stats", "rope_sdpa_reset_stats", "rope_sdpa_abi_version", "rope_sdpa_debug_quantize_qk",
    "rope_sdpa_debug_kernel_timing", "rope_sdpa_debug_kernel_time",
    "rope_sdpa_fwd_noalloc", "rope_sdpa_noalloc_scratch_bytes", "rope_sdpa_rotate",
)


class RsTensor(ctypes.Structure):
    _fields_ = [
        ("data", ctypes.c_void_p),
        ("dtype", ctypes.c_int32),
        ("reserved", ctypes.c_int32),
        ("size", ctypes.c_int64 * 4),
        ("stride", ctypes.c_int64 * 4),
    ]


class RsArgs(ctypes.Structure):
    _fields_ = [
        ("q", ctypes.POINTER(RsTensor)),
        ("k", ctypes.POINTER(RsTensor)),
        ("v", ctypes.POINTER(RsTensor)),
        ("cos", ctypes.POINTER(RsTensor)),
        ("sin", ctypes.POINTER(RsTensor)),
        ("mask", ctypes.POINTER(RsTensor)),
        ("mask_kind", ctypes.c_int32),
        ("flags", ctypes.c_uint32),
        ("scale", ctypes.c_float),
        ("q_norm_weight", ctypes.c_void_p),
        ("k_norm_weight", ctypes.c_void_p),
        ("norm_eps", ctypes.c_float),
    ]


class RsStats(ctypes.Structure):
    _fields_ = [(n, ctypes.c_uint64) for n in (
        "fwd_instream", "fwd_autograd", "bwd_calls", "masked_bool", "masked_additive", "causal",
        "quant_int8", "mask_all_true_skipped", "errors", "quant_bwd")]


_lib = None
ABI_VERSION = 3  # ROPE_SDPA_ABI_VERSION of include/rope_sdpa.h that these structures mirror


def load(path: str = LIB_PATH):
    """Load the HIP library; raises if it has not been built (there is no fallback path)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(
            f"{path} is missing: build the HIP library first (python -c 'import __graft_entry__ as g; g.build()')")
    lib = ctypes.CDLL(path)
    lib.rope_sdpa_abi_version.restype = ctypes.c_int
    if lib.rope_sdpa_abi_version() != ABI_VERSION:
        raise RuntimeError(f"{path} has ABI version {lib.rope_sdpa_abi_version()}, this binding needs "
                           f"{ABI_VERSION}: rebuild the HIP library")
    P = ctypes.POINTER
    lib.rope_sdpa_workspace_size.argtypes = [P(RsArgs), ctypes.c_int, P(ctypes.c_size_t)]
    lib.rope_sdpa_workspace_size.restype = ctypes.c_int
    lib.rope_sdpa_fwd.argtypes = [P(RsArgs), P(RsTensor), ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t,
                                  ctypes.c_void_p]
    lib.rope_sdpa_fwd.restype = ctypes.c_int
    lib.rope_sdpa_fwd_noalloc.argtypes = [P(RsArgs), P(RsTensor), ctypes.c_void_p, ctypes.c_void_p]
    lib.rope_sdpa_fwd_noalloc.restype = ctypes.c_int
    lib.rope_sdpa_noalloc_scratch_bytes.argtypes = []
    lib.rope_sdpa_noalloc_scratch_bytes.restype = ctypes.c_size_t
    lib.rope_sdpa_rotate.argtypes = [P(RsTensor), P(RsTensor), P(RsTensor), P(RsTensor), ctypes.c_void_p]
    lib.rope_sdpa_rotate.restype = ctypes.c_int
    lib.rope_sdpa_bwd.argtypes = [P(RsArgs), P(RsTensor), ctypes.c_void_p, P(RsTensor), P(RsTensor), P(RsTensor),
                                  P(RsTensor), ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
    lib.rope_sdpa_bwd.restype = ctypes.c_int
    lib.rope_sdpa_status_string.argtypes = [ctypes.c_int]
    lib.rope_sdpa_status_string.restype = ctypes.c_char_p
    lib.rope_sdpa_get_stats.argtypes = [P(RsStats)]
    lib.rope_sdpa_get_stats.restype = None
    lib.rope_sdpa_reset_stats.argtypes = []
    lib.rope_sdpa_reset_stats.restype = None
    lib.rope_sdpa_debug_quantize_qk.argtypes = [P(RsArgs), ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                                ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
    lib.rope_sdpa_debug_quantize_qk.restype = ctypes.c_int
    lib.rope_sdpa_debug_kernel_timing.argtypes = [ctypes.c_int]
    lib.rope_sdpa_debug_kernel_timing.restype = ctypes.c_int
    lib.rope_sdpa_debug_kernel_time.argtypes = [P(ctypes.c_double), P(ctypes.c_uint64)]
    lib.rope_sdpa_debug_kernel_time.restype = ctypes.c_int
    lib.rope_sdpa_abi_version.argtypes = []
    lib.rope_sdpa_abi_version.restype = ctypes.c_int
    _lib = lib
    return lib


def make_tensor(data_ptr: int, dtype_code: int, size, stride) -> RsTensor:
    t = RsTensor()
    t.data = data_ptr
    t.dtype = dtype_code
    t.reserved = 0
    for i in range(4):
        t.size[i] = int(size[i])
        t.stride[i] = int(stride[i])
    return t


def status_string(code: int) -> str:
    return load().rope_sdpa_status_string(code).decode()
