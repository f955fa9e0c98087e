"""Boundary tests that run without a GPU.

The library must load, export every function include/rope_sdpa.h declares, and reject
every malformed call on the host before touching the device.  Device pointers here are
fake addresses: validation never dereferences them, and a well-formed call on a machine
with no gfx950 device returns RS_ERR_NO_DEVICE.
"""
import ctypes
import os
import re

import pytest

from rope_flash_attention_amd import _abi
from rope_flash_attention_amd._abi import (RS_BF16, RS_BOOL, RS_F16, RS_F32, RS_FLAG_CAUSAL,
                                           RS_FLAG_QUANT_INT8_QK, RS_FLAG_QUANT_INT4_QK, RS_FLAG_K_PREPASS, RS_MASK_ADDITIVE, RS_MASK_BOOL,
                                           RS_MASK_NONE, RsArgs, RsStats, make_tensor)

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "rope_sdpa.h")

ERR = {v: k for k, v in _abi.STATUS_NAMES.items()}
BASE = 0x7F0000000000  # fake, 256-byte aligned device addresses


def lib():
    if not os.path.exists(_abi.LIB_PATH):
        pytest.skip("library not built (run __graft_entry__.build())")
    return _abi.load()


def test_exports_every_declared_symbol():
    L = lib()
    text = open(HEADER).read()
    declared = set(re.findall(r"\b(rope_sdpa_\w+)\s*\(", text))
    assert declared == set(_abi.EXPORTED)
    for name in declared:
        assert hasattr(L, name), name


def test_version_and_status_strings():
    L = lib()
    assert L.rope_sdpa_abi_version() == 3
    for code, name in _abi.STATUS_NAMES.items():
        assert _abi.status_string(code).startswith(name)
    assert "unknown" in _abi.status_string(-99)


class Call:
    """A well-formed forward call on fake pointers; tests break one thing at a time."""

    def __init__(self, B=2, H=3, S=100, D=128, dt=RS_BF16, es=2):
        self.B, self.H, self.S, self.D, self.dt, self.es = B, H, S, D, dt, es
        n = B * H * S * D * es
        c = lambda i, d=dt, size=(B, H, S, D), stride=(H * S * D, S * D, D, 1): make_tensor(
            BASE + i * (1 << 32), d, size, stride)
        self.q, self.k, self.v, self.o = c(0), c(1), c(2), c(3)
        self.cos = make_tensor(BASE + 4 * (1 << 32), RS_F32, (1, 1, S, D), (S * D, S * D, D, 1))
        self.sin = make_tensor(BASE + 5 * (1 << 32), RS_F32, (1, 1, S, D), (S * D, S * D, D, 1))
        self.mask = None
        self.kind = RS_MASK_NONE
        self.flags = 0
        self.scale = 0.0
        self.lse = BASE + 6 * (1 << 32)
        self.ws = BASE + 7 * (1 << 32)
        self.ws_bytes = 1 << 30

    def args(self):
        a = RsArgs()
        a.q, a.k, a.v = ctypes.pointer(self.q), ctypes.pointer(self.k), ctypes.pointer(self.v)
        a.cos, a.sin = ctypes.pointer(self.cos), ctypes.pointer(self.sin)
        a.mask = ctypes.pointer(self.mask) if self.mask is not None else None
        a.mask_kind, a.flags, a.scale = self.kind, self.flags, self.scale
        return a

    def fwd(self):
        a = self.args()
        return lib().rope_sdpa_fwd(ctypes.byref(a), ctypes.byref(self.o), self.lse, self.ws, self.ws_bytes, None)

    def ws_size(self, backward=0):
        a = self.args()
        n = ctypes.c_size_t(0)
        st = lib().rope_sdpa_workspace_size(ctypes.byref(a), backward, ctypes.byref(n))
        return st, n.value


def test_well_formed_call_reaches_the_device_check():
    c = Call()
    assert c.fwd() == ERR["RS_ERR_NO_DEVICE"]


@pytest.mark.parametrize("mutate,expect", [
    (lambda c: setattr(c.q, "data", None), "RS_ERR_NULL"),
    (lambda c: setattr(c, "cos", None) if False else setattr(c.cos, "data", None), "RS_ERR_NULL"),
    (lambda c: setattr(c.k, "dtype", RS_F32), "RS_ERR_DTYPE"),     # fp32 K with bf16 Q/V (autocast case)
    (lambda c: setattr(c.v, "dtype", RS_F16), "RS_ERR_DTYPE"),
    (lambda c: setattr(c.o, "dtype", RS_F32), "RS_ERR_DTYPE"),
    (lambda c: setattr(c.cos, "dtype", RS_BF16), "RS_ERR_DTYPE"),
    (lambda c: c.k.size.__setitem__(2, 99), "RS_ERR_SHAPE"),
    (lambda c: c.cos.size.__setitem__(2, 99), "RS_ERR_SHAPE"),
    (lambda c: c.cos.size.__setitem__(0, 3), "RS_ERR_SHAPE"),
    (lambda c: c.q.stride.__setitem__(3, 2), "RS_ERR_STRIDE"),
    (lambda c: c.v.stride.__setitem__(2, 132), "RS_ERR_STRIDE"),  # 264 bytes: not a multiple of 16
    (lambda c: setattr(c.q, "data", BASE + 8), "RS_ERR_ALIGN"),
    (lambda c: setattr(c, "ws", BASE + 7 * (1 << 32) + 64), "RS_ERR_ALIGN"),
    (lambda c: setattr(c, "ws_bytes", 16), "RS_ERR_WORKSPACE"),
    (lambda c: setattr(c, "ws", None), "RS_ERR_WORKSPACE"),
    (lambda c: setattr(c, "flags", 1 << 5), "RS_ERR_INVALID"),
    (lambda c: setattr(c, "scale", -1.0), "RS_ERR_INVALID"),
    (lambda c: setattr(c, "scale", float("nan")), "RS_ERR_INVALID"),
    (lambda c: setattr(c, "kind", 7), "RS_ERR_INVALID"),
    (lambda c: setattr(c, "lse", BASE + 2), "RS_ERR_ALIGN"),
])
def test_forward_validation(mutate, expect):
    c = Call()
    mutate(c)
    assert c.fwd() == ERR[expect]


def test_head_dim_must_be_64_or_128():
    for D, want in [(64, "RS_ERR_NO_DEVICE"), (128, "RS_ERR_NO_DEVICE"), (96, "RS_ERR_SHAPE"), (256, "RS_ERR_SHAPE")]:
        assert Call(D=D).fwd() == ERR[want]


def _bool_mask(c, size, stride, dtype=RS_BOOL):
    c.mask = make_tensor(BASE + 9 * (1 << 32), dtype, size, stride)
    c.kind = RS_MASK_BOOL if dtype == RS_BOOL else RS_MASK_ADDITIVE


def test_mask_validation():
    c = Call()
    _bool_mask(c, (2, 1, 1, 100), (112, 0, 0, 1))
    assert c.fwd() == ERR["RS_ERR_NO_DEVICE"]
    _bool_mask(c, (2, 1, 1, 100), (100, 0, 0, 1))  # per-batch rows must start 16-byte aligned
    assert c.fwd() == ERR["RS_ERR_STRIDE"]
    _bool_mask(c, (2, 3, 100, 100), (30000, 10000, 100, 1))  # 100-byte rows: not 16-byte multiples
    assert c.fwd() == ERR["RS_ERR_STRIDE"]
    _bool_mask(c, (2, 3, 100, 100), (3 * 100 * 112, 100 * 112, 112, 1))  # padded rows are fine
    assert c.fwd() == ERR["RS_ERR_NO_DEVICE"]
    _bool_mask(c, (2, 1, 5, 100), (100, 0, 0, 1))  # Sq extent must be 1 or S
    assert c.fwd() == ERR["RS_ERR_SHAPE"]
    _bool_mask(c, (1, 1, 1, 100), (0, 0, 0, 1), dtype=RS_F16)  # additive mask: f32 or q dtype only
    assert c.fwd() == ERR["RS_ERR_DTYPE"]
    _bool_mask(c, (1, 1, 1, 100), (0, 0, 0, 1), dtype=RS_BF16)
    assert c.fwd() == ERR["RS_ERR_NO_DEVICE"]
    _bool_mask(c, (1, 1, 1, 100), (0, 0, 0, 1))
    c.flags = RS_FLAG_CAUSAL  # causal together with a mask
    assert c.fwd() == ERR["RS_ERR_INVALID"]
    c2 = Call()
    c2.kind = RS_MASK_BOOL  # kind without a mask
    assert c2.fwd() == ERR["RS_ERR_NULL"]
    c3 = Call()
    _bool_mask(c3, (1, 1, 1, 100), (0, 0, 0, 1))
    c3.kind = RS_MASK_NONE  # a mask given with kind "none"
    assert c3.fwd() == ERR["RS_ERR_INVALID"]


def test_bool_mask_length_limit():
    """Bool masks gather their key-tile states into LDS: S <= 262144, longer is RS_ERR_SHAPE
    (before any device work); other mask kinds have no such limit."""
    for S, want in [(262144, "RS_ERR_NO_DEVICE"), (262145, "RS_ERR_SHAPE")]:
        c = Call(B=1, H=1, S=S, D=64)
        _bool_mask(c, (1, 1, 1, S), (0, 0, 0, 1))
        assert c.fwd() == ERR[want], S
        c.mask, c.kind = None, RS_MASK_NONE
        assert c.fwd() == ERR["RS_ERR_NO_DEVICE"], S


def test_int8_flag_limits():
    c = Call(dt=RS_F32, es=4)
    c.flags = RS_FLAG_QUANT_INT8_QK
    assert c.fwd() == ERR["RS_ERR_UNSUPPORTED"]
    c = Call()  # causal and masks are valid with quantization: only the missing device stops them
    c.flags = RS_FLAG_QUANT_INT8_QK | RS_FLAG_CAUSAL
    assert c.fwd() == ERR["RS_ERR_NO_DEVICE"]
    c = Call()
    _bool_mask(c, (2, 1, 1, 100), (112, 0, 0, 1))
    c.flags = RS_FLAG_QUANT_INT8_QK
    assert c.fwd() == ERR["RS_ERR_NO_DEVICE"]
    c = Call()
    c.flags = RS_FLAG_QUANT_INT8_QK  # a valid int8 request: only the missing device stops it
    assert c.fwd() == ERR["RS_ERR_NO_DEVICE"]


def test_int8_workspace_holds_no_codes():
    """The int8 forward quantizes Q' and K' inside the attention kernel: its workspace is the
    16-bit forward's (no codes or scales in memory)."""
    c = Call(B=2, H=3, S=100, D=128)
    st, n = c.ws_size(0)
    c.flags = RS_FLAG_QUANT_INT8_QK
    st8, n8 = c.ws_size(0)
    assert st == 0 and st8 == 0
    assert n8 == n
    c.flags = RS_FLAG_K_PREPASS  # K rotated by a pass of its own: + K' in the workspace
    st, nk = c.ws_size(0)
    assert st == 0 and nk == n + -(-(2 * 3 * 100 * 128 * 2) // 256) * 256


def test_debug_quantize_validation():
    L = lib()
    c = Call(B=2, H=3, S=100, D=128)
    c.flags = RS_FLAG_QUANT_INT8_QK
    a = c.args()
    ptr = lambda i: BASE + (20 + i) * (1 << 32)
    st = L.rope_sdpa_debug_quantize_qk(ctypes.byref(a), ptr(0), ptr(1), ptr(2), ptr(3), c.ws, c.ws_bytes, None)
    assert st == ERR["RS_ERR_NO_DEVICE"]
    st = L.rope_sdpa_debug_quantize_qk(ctypes.byref(a), None, ptr(1), ptr(2), ptr(3), c.ws, c.ws_bytes, None)
    assert st == ERR["RS_ERR_NULL"]
    st = L.rope_sdpa_debug_quantize_qk(ctypes.byref(a), ptr(0) + 4, ptr(1), ptr(2), ptr(3), c.ws, c.ws_bytes, None)
    assert st == ERR["RS_ERR_ALIGN"]
    st = L.rope_sdpa_debug_quantize_qk(ctypes.byref(a), ptr(0), ptr(1), ptr(2) + 2, ptr(3), c.ws, c.ws_bytes, None)
    assert st == ERR["RS_ERR_ALIGN"]
    st = L.rope_sdpa_debug_quantize_qk(ctypes.byref(a), ptr(0), ptr(1), ptr(2), ptr(3), c.ws, 64, None)
    assert st == ERR["RS_ERR_WORKSPACE"]
    c.flags = 0
    a = c.args()
    st = L.rope_sdpa_debug_quantize_qk(ctypes.byref(a), ptr(0), ptr(1), ptr(2), ptr(3), c.ws, c.ws_bytes, None)
    assert st == ERR["RS_ERR_INVALID"]


def test_strided_views_are_accepted():
    # BSHD projection viewed as BHSD: strides (S*H*D, D, H*D, 1)
    c = Call()
    B, H, S, D = c.B, c.H, c.S, c.D
    for t in (c.q, c.k, c.v):
        for i, s in enumerate((S * H * D, D, H * D, 1)):
            t.stride[i] = s
    assert c.fwd() == ERR["RS_ERR_NO_DEVICE"]


def test_workspace_size_layout():
    c = Call(B=2, H=3, S=100, D=128)
    st, n = c.ws_size(0)
    assert st == 0
    table = 100 * 128 * 4  # (cos, sin) pairs: D/2 float2 per position
    kprime = -(-(2 * 3 * 100 * 128 * 2) // 256) * 256  # K' = R(K) or Q' = R(Q), 16-bit
    assert n == 256 + -(-table // 256) * 256
    st, nb = c.ws_size(1)
    # backward (16-bit, D = 128): + delta (fp32 per row) + Q' + K', both in the input dtype
    assert st == 0 and nb == n + -(-(2 * 3 * 100 * 4) // 256) * 256 + 2 * kprime
    f = Call(B=2, H=3, S=100, D=128, dt=RS_F32, es=4)
    st, nf = f.ws_size(0)
    st2, nfb = f.ws_size(1)
    assert st == 0 and st2 == 0 and nfb == nf + -(-(2 * 3 * 100 * 4) // 256) * 256  # fp32: no Q'
    _bool_mask(c, (2, 1, 1, 100), (112, 0, 0, 1))
    st, nm = c.ws_size(0)
    assert st == 0 and nm == n + 256  # 2 x 1 x 1 x 2 tile states, padded
    c.cos.size[0] = 2
    c.sin.size[0] = 2
    c.mask, c.kind = None, RS_MASK_NONE
    st, n2 = c.ws_size(0)
    assert st == 0 and n2 == 256 + -(-(2 * table) // 256) * 256


def test_backward_validation_and_error_counter():
    L = lib()
    L.rope_sdpa_reset_stats()
    c = Call()
    a = c.args()
    t = lambda i: make_tensor(BASE + (10 + i) * (1 << 32), RS_BF16, (2, 3, 100, 128), (3 * 100 * 128, 100 * 128, 128, 1))
    do, dq, dk, dv = t(0), t(1), t(2), t(3)
    st = L.rope_sdpa_bwd(ctypes.byref(a), ctypes.byref(c.o), c.lse, ctypes.byref(do), ctypes.byref(dq),
                         ctypes.byref(dk), ctypes.byref(dv), c.ws, c.ws_bytes, None)
    assert st == ERR["RS_ERR_NO_DEVICE"]
    st = L.rope_sdpa_bwd(ctypes.byref(a), ctypes.byref(c.o), None, ctypes.byref(do), ctypes.byref(dq),
                         ctypes.byref(dk), ctypes.byref(dv), c.ws, c.ws_bytes, None)
    assert st == ERR["RS_ERR_NULL"]
    dv.dtype = RS_F32
    st = L.rope_sdpa_bwd(ctypes.byref(a), ctypes.byref(c.o), c.lse, ctypes.byref(do), ctypes.byref(dq),
                         ctypes.byref(dk), ctypes.byref(dv), c.ws, c.ws_bytes, None)
    assert st == ERR["RS_ERR_DTYPE"]
    c.flags = RS_FLAG_QUANT_INT8_QK  # the quantized backward (D = 128) is accepted: no device here
    a = c.args()
    dv.dtype = RS_BF16
    st = L.rope_sdpa_bwd(ctypes.byref(a), ctypes.byref(c.o), c.lse, ctypes.byref(do), ctypes.byref(dq),
                         ctypes.byref(dk), ctypes.byref(dv), c.ws, c.ws_bytes, None)
    assert st == ERR["RS_ERR_NO_DEVICE"]
    c.flags = RS_FLAG_QUANT_INT8_QK | RS_FLAG_QUANT_INT4_QK
    a = c.args()
    st = L.rope_sdpa_bwd(ctypes.byref(a), ctypes.byref(c.o), c.lse, ctypes.byref(do), ctypes.byref(dq),
                         ctypes.byref(dk), ctypes.byref(dv), c.ws, c.ws_bytes, None)
    assert st == ERR["RS_ERR_INVALID"]
    s = RsStats()
    L.rope_sdpa_get_stats(ctypes.byref(s))
    assert s.errors == 5 and s.bwd_calls == 0 and s.fwd_instream == 0 and s.quant_bwd == 0


@pytest.mark.parametrize("dims", [dict(B=0), dict(H=0), dict(S=0)])
def test_empty_calls_are_valid_no_ops(dims):
    """B, H or S = 0: validated like any call, NULL data accepted, RS_OK with no device."""
    L = lib()
    c = Call(**dims)
    for t in (c.q, c.k, c.v, c.o, c.cos, c.sin):
        t.data = None
    c.lse, c.ws, c.ws_bytes = None, None, 0
    c.q.stride[3] = 0  # an empty tensor's strides are not looked at (torch may hand any)
    _bool_mask(c, (1, 1, 1, c.S), (0, 0, 0, 3))
    c.mask.data = None
    assert c.ws_size(0) == (0, 0) and c.ws_size(1) == (0, 0)
    assert c.fwd() == 0
    a = c.args()
    shape = (c.B, c.H, c.S, c.D)
    t = lambda: make_tensor(None, RS_BF16, shape, (c.H * c.S * c.D, c.S * c.D, c.D, 1))
    do, dq, dk, dv = t(), t(), t(), t()
    st = L.rope_sdpa_bwd(ctypes.byref(a), ctypes.byref(c.o), None, ctypes.byref(do), ctypes.byref(dq),
                         ctypes.byref(dk), ctypes.byref(dv), None, 0, None)
    assert st == 0
    c.mask, c.kind = None, RS_MASK_NONE
    c.flags = RS_FLAG_QUANT_INT8_QK
    assert c.fwd() == 0
    a = c.args()
    assert L.rope_sdpa_debug_quantize_qk(ctypes.byref(a), None, None, None, None, None, 0, None) == 0
    # still validated: a wrong dtype or size is an error even with nothing to compute
    c.flags = 0
    c.v.dtype = RS_F16
    assert c.fwd() == ERR["RS_ERR_DTYPE"]
    c.v.dtype = RS_BF16
    c.k.size[3] = 64
    assert c.fwd() == ERR["RS_ERR_SHAPE"]


def test_negative_sizes_are_rejected():
    c = Call()
    for t in (c.q, c.k, c.v, c.o):
        t.size[2] = -1
    assert c.fwd() == ERR["RS_ERR_SHAPE"]


def test_noalloc_forward_validates_and_bounds_its_scratch():
    """The allocation-free forward runs the forward's checks; a call whose workspace would
    exceed the library's static scratch returns RS_ERR_SCRATCH before any device access."""
    L = lib()
    assert L.rope_sdpa_noalloc_scratch_bytes() == 64 << 20
    c = Call()
    a = c.args()
    assert L.rope_sdpa_fwd_noalloc(ctypes.byref(a), ctypes.byref(c.o), c.lse, None) == ERR["RS_ERR_NO_DEVICE"]
    c.k.dtype = RS_F32
    a = c.args()
    assert L.rope_sdpa_fwd_noalloc(ctypes.byref(a), ctypes.byref(c.o), c.lse, None) == ERR["RS_ERR_DTYPE"]
    # per-sample tables of 64 samples at S = 4608: 151 MB of packed tables > 64 MiB
    big = Call(B=64, H=1, S=4608, D=128)
    big.cos = make_tensor(BASE + 4 * (1 << 32), RS_F32, (64, 1, 4608, 128), (4608 * 128, 4608 * 128, 128, 1))
    big.sin = make_tensor(BASE + 5 * (1 << 32), RS_F32, (64, 1, 4608, 128), (4608 * 128, 4608 * 128, 128, 1))
    a = big.args()
    assert L.rope_sdpa_fwd_noalloc(ctypes.byref(a), ctypes.byref(big.o), big.lse, None) == ERR["RS_ERR_SCRATCH"]
