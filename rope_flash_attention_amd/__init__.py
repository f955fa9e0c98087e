"""Fused rotary position embedding + scaled dot-product attention on AMD MI355X (gfx950).

Python binding over the C ABI in include/rope_sdpa.h.  This module only marshals
arguments: every step of the computation runs in the library's HIP kernels, on the
caller's current HIP stream; PyTorch provides device memory and streams.  There is no
fallback implementation: if the library is missing or rejects a call, an error is raised.

Entry point (page "Metal Flash Attention", SimpleTuner docs, section "Fused RoPE + SDPA"):

    rope_scaled_dot_product_attention(query, key, value, rope_cos, rope_sin,
                                      attn_mask=None, is_causal=False, scale=None)

query/key/value are BHSD (strided views accepted); key and value may have fewer heads than
query (grouped-query / multi-query attention: query head h reads K/V head h * Hkv / H, and K is
rotated at its own head count); rope_cos/rope_sin are pair-duplicated
tables of shape [S, D], [1, S, D] or [B, S, D] in any float dtype (normalised to fp32),
masks are bool (True = attend) or additive float, broadcastable, up to 4-D.  Gradients
flow to query, key (pre-rotation) and value.

Forward only: query and key may be fp32 beside an fp16/bf16 value (the autocast layout of
flux-style attention; the output takes value's dtype), and q_norm_weight/k_norm_weight apply
RMSNorm over the head dimension to query and key before the rotation, inside the kernel.
"""
from __future__ import annotations

import ctypes

import torch

from . import _abi
from ._abi import (RS_BF16, RS_BOOL, RS_F16, RS_F32, RS_FLAG_CAUSAL, RS_FLAG_K_PREPASS, RS_FLAG_QUANT_INT4_QK,
                   RS_FLAG_QUANT_INT8_PREPASS, RS_FLAG_QUANT_INT8_QK, RS_MASK_ADDITIVE, RS_MASK_BOOL, RS_MASK_NONE,
                   RsArgs, RsStats, make_tensor)

# quantization= values -> flags: "int8" / "int4" quantize in the attention kernel (no codes
# in memory), "..._prepass" has a quantizer pass write the codes first (same results, faster)
_QUANT_FLAGS = {None: 0, "int8": RS_FLAG_QUANT_INT8_QK, "int8_prepass": RS_FLAG_QUANT_INT8_QK | RS_FLAG_QUANT_INT8_PREPASS,
                "int4": RS_FLAG_QUANT_INT4_QK, "int4_prepass": RS_FLAG_QUANT_INT4_QK | RS_FLAG_QUANT_INT8_PREPASS}

__all__ = [
    "rope_scaled_dot_product_attention", "rope_sdpa_fwd", "rope_sdpa_bwd", "rope_sdpa_workspace_size",
    "rope_sdpa_get_stats", "rope_sdpa_reset_stats", "rope_sdpa_abi_version", "rope_sdpa_status_string",
    "get_dispatch_stats", "RopeSdpaError", "library_path", "rope_sdpa_debug_quantize_qk", "debug_quantize_qk",
    "rope_sdpa_fwd_noalloc", "rope_sdpa_noalloc_scratch_bytes", "rope_sdpa_rotate", "rope_rotate",
    "scaled_dot_product_attention", "rope_sdpa_debug_kernel_timing", "rope_sdpa_debug_kernel_time",
]

_DT = {torch.float32: RS_F32, torch.float16: RS_F16, torch.bfloat16: RS_BF16, torch.bool: RS_BOOL}


class RopeSdpaError(RuntimeError):
    def __init__(self, code: int):
        self.code = code
        super().__init__(_abi.status_string(code))


def library_path() -> str:
    return _abi.LIB_PATH


def _check(code: int):
    if code != 0:
        raise RopeSdpaError(code)


def _desc(t: torch.Tensor) -> _abi.RsTensor:
    if t.dim() != 4:
        raise ValueError("expected a 4-D tensor")
    return make_tensor(t.data_ptr(), _DT[t.dtype], t.shape, t.stride())


def _tables4(t: torch.Tensor, device) -> torch.Tensor:
    """[S,D] | [1,S,D] | [B,S,D] in any float dtype -> fp32 [Bt, 1, S, D] view on `device`."""
    if t.dim() == 2:
        t = t.unsqueeze(0)
    if t.dim() != 3:
        raise ValueError("rope tables must be [S, D], [1, S, D] or [B, S, D]")
    t = t.to(device=device, dtype=torch.float32)
    if t.stride(-1) != 1:
        t = t.contiguous()
    return t.unsqueeze(1)


def _mask4(mask: torch.Tensor | None, qdtype):
    if mask is None:
        return None, RS_MASK_NONE
    while mask.dim() < 4:
        mask = mask.unsqueeze(0)
    if mask.dim() != 4:
        raise ValueError("attn_mask must have at most 4 dimensions")
    if mask.dtype == torch.bool:
        kind = RS_MASK_BOOL
    else:
        kind = RS_MASK_ADDITIVE
        if mask.dtype not in (torch.float32, qdtype):
            mask = mask.to(torch.float32)
    if mask.shape[-1] > 1:
        es = mask.element_size()
        ok = mask.stride(-1) == 1 and mask.data_ptr() % 16 == 0 and all(
            (st * es) % 16 == 0 for st, n in zip(mask.stride()[:3], mask.shape[:3]) if n > 1)
        if not ok:
            # rows of the mask must start on 16-byte boundaries: copy into a padded buffer
            n = mask.shape[-1]
            pad = -(-n * es // 16) * 16 // es
            buf = torch.empty((*mask.shape[:3], pad), dtype=mask.dtype, device=mask.device)
            buf[..., :n].copy_(mask)
            mask = buf[..., :n]
    return mask, kind


class _Call:
    """Holds the ctypes descriptors of one call (kept alive for the duration of the call)."""

    def __init__(self, q, k, v, cos4, sin4, mask, mask_kind, causal, scale, quant=None, norm=None, k_prepass=False):
        self.tq, self.tk, self.tv = _desc(q), _desc(k), _desc(v)
        self.tc = _desc(cos4) if cos4 is not None else None  # no tables: plain attention
        self.ts = _desc(sin4) if sin4 is not None else None
        self.tm = _desc(mask) if mask is not None else None
        a = RsArgs()
        a.q, a.k, a.v = ctypes.pointer(self.tq), ctypes.pointer(self.tk), ctypes.pointer(self.tv)
        a.cos = ctypes.pointer(self.tc) if self.tc is not None else None
        a.sin = ctypes.pointer(self.ts) if self.ts is not None else None
        a.mask = ctypes.pointer(self.tm) if self.tm is not None else None
        a.mask_kind = mask_kind
        a.flags = (RS_FLAG_CAUSAL if causal else 0) | _QUANT_FLAGS[quant] | (RS_FLAG_K_PREPASS if k_prepass else 0)
        a.scale = 0.0 if scale is None else float(scale)
        if norm is not None:  # (q weights, k weights, eps): fp32 [D] device tensors
            self.norm = norm
            a.q_norm_weight, a.k_norm_weight = norm[0].data_ptr(), norm[1].data_ptr()
            a.norm_eps = float(norm[2])
        self.args = a

    def workspace(self, backward: bool, device) -> torch.Tensor:
        n = ctypes.c_size_t(0)
        _check(_abi.load().rope_sdpa_workspace_size(ctypes.byref(self.args), int(backward), ctypes.byref(n)))
        return torch.empty(int(n.value), dtype=torch.uint8, device=device)


def _stream(device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def _forward(q, k, v, cos4, sin4, mask, mask_kind, causal, scale, need_lse, quant=None, norm=None, k_prepass=False):
    lib = _abi.load()
    call = _Call(q, k, v, cos4, sin4, mask, mask_kind, causal, scale, quant, norm, k_prepass)
    B, H, S, D = q.shape
    o = torch.empty((B, H, S, D), dtype=v.dtype, device=q.device)  # the compute dtype
    lse = torch.empty((B, H, S), dtype=torch.float32, device=q.device) if need_lse else None
    ws = call.workspace(False, q.device)
    to = _desc(o)
    _check(lib.rope_sdpa_fwd(ctypes.byref(call.args), ctypes.byref(to),
                             lse.data_ptr() if lse is not None else None,
                             ws.data_ptr(), ws.numel(), _stream(q.device)))
    return o, lse


def _backward(q, k, v, cos4, sin4, mask, mask_kind, causal, scale, o, lse, do, quant=None):
    lib = _abi.load()
    call = _Call(q, k, v, cos4, sin4, mask, mask_kind, causal, scale, quant)
    dq = torch.empty(q.shape, dtype=q.dtype, device=q.device)
    dk = torch.empty(k.shape, dtype=q.dtype, device=q.device)  # K/V heads (grouped-query attention)
    dv = torch.empty(v.shape, dtype=q.dtype, device=q.device)
    ws = call.workspace(True, q.device)
    tdo, tdq, tdk, tdv, to = _desc(do), _desc(dq), _desc(dk), _desc(dv), _desc(o)
    _check(lib.rope_sdpa_bwd(ctypes.byref(call.args), ctypes.byref(to), lse.data_ptr(), ctypes.byref(tdo),
                             ctypes.byref(tdq), ctypes.byref(tdk), ctypes.byref(tdv),
                             ws.data_ptr(), ws.numel(), _stream(q.device)))
    return dq, dk, dv


class _RopeSdpaFn(torch.autograd.Function):
    @staticmethod
    def forward(ctx, q, k, v, cos4, sin4, mask, mask_kind, causal, scale, quant=None):
        o, lse = _forward(q, k, v, cos4, sin4, mask, mask_kind, causal, scale, need_lse=True, quant=quant)
        ctx.save_for_backward(q, k, v, cos4, sin4, o, lse, mask if mask is not None else torch.empty(0))
        ctx.has_mask = mask is not None
        ctx.mask_kind, ctx.causal, ctx.scale, ctx.quant = mask_kind, causal, scale, quant
        return o

    @staticmethod
    def backward(ctx, do):
        q, k, v, cos4, sin4, o, lse, mask = ctx.saved_tensors
        if do.stride(-1) != 1 or do.data_ptr() % 16 != 0 or any(
                (s * do.element_size()) % 16 for s, n in zip(do.stride()[:3], do.shape[:3]) if n > 1):
            do = do.contiguous()
        dq, dk, dv = _backward(q, k, v, cos4, sin4, mask if ctx.has_mask else None, ctx.mask_kind, ctx.causal,
                               ctx.scale, o, lse, do, ctx.quant)
        return dq, dk, dv, None, None, None, None, None, None, None


def _norm_args(query, q_norm_weight, k_norm_weight, norm_eps):
    """(q weights, k weights, eps) as fp32 [D] device tensors, or None without normalization."""
    if q_norm_weight is None and k_norm_weight is None:
        return None
    if q_norm_weight is None or k_norm_weight is None:
        raise ValueError("q_norm_weight and k_norm_weight go together")
    D = query.shape[-1]
    w = [t.to(device=query.device, dtype=torch.float32).contiguous() for t in (q_norm_weight, k_norm_weight)]
    if any(t.shape != (D,) for t in w):
        raise ValueError(f"norm weights must have shape [{D}]")
    return w[0], w[1], float(norm_eps)


def _check_dtypes(query, key, value):
    """Q and K share a dtype; V the same, or 16-bit beside fp32 Q/K (forward only)."""
    if query.dtype != key.dtype:
        raise RopeSdpaError(-2)
    if query.dtype != value.dtype and not (query.dtype == torch.float32 and value.dtype in (torch.float16,
                                                                                           torch.bfloat16)):
        raise RopeSdpaError(-2)


def rope_scaled_dot_product_attention(query, key, value, rope_cos, rope_sin, attn_mask=None, is_causal=False,
                                      scale=None, quantization=None, q_norm_weight=None, k_norm_weight=None,
                                      norm_eps=1e-6, k_prepass=False):
    """softmax(scale * R(Q) R(K)^T + mask) V with R the interleaved-pair rotation of the tables.

    quantization: None, "int8" for the blockwise int8 Q'/K' forward quantized in the attention
    kernel, or "int8_prepass" for the same forward with the codes written by a quantizer pass
    first (bit-identical results, faster); "int4" / "int4_prepass" the same with codes in
    [-7, 7].  Gradients pass the quantizer straight through: the backward runs at the
    dequantized rotated Q and K the forward attended with.

    q_norm_weight, k_norm_weight ([D] each, together or not at all): RMSNorm of query and key
    over the head dimension, x / sqrt(mean(x^2) + norm_eps) * w in fp32, before the rotation.
    fp32 query/key with fp16/bf16 value are read in fp32 and rounded to value's dtype after the
    rotation; the output has value's dtype.  Both are forward only (no gradient).

    k_prepass: rotate K once per (batch, K/V head) by a pass of its own instead of in the
    attention kernel's key loop (RS_FLAG_K_PREPASS: bit-identical results, K' goes through HBM).
    """
    if not (query.is_cuda and key.is_cuda and value.is_cuda):
        raise ValueError("query, key and value must be device tensors")
    _check_dtypes(query, key, value)
    cos4 = _tables4(rope_cos, query.device)
    sin4 = _tables4(rope_sin, query.device)
    mask, kind = _mask4(attn_mask, value.dtype)
    if quantization not in _QUANT_FLAGS:
        raise ValueError("quantization must be None, 'int8', 'int8_prepass', 'int4' or 'int4_prepass'")
    norm = _norm_args(query, q_norm_weight, k_norm_weight, norm_eps)
    needs_grad = torch.is_grad_enabled() and (query.requires_grad or key.requires_grad or value.requires_grad)
    if quantization is not None and needs_grad and norm is None and query.dtype == value.dtype:
        return _RopeSdpaFn.apply(query, key, value, cos4, sin4, mask, kind, bool(is_causal), scale, quantization)
    if quantization is not None or norm is not None or query.dtype != value.dtype:
        if needs_grad:
            raise RopeSdpaError(-6)
        return _forward(query, key, value, cos4, sin4, mask, kind, bool(is_causal), scale, False,
                        quant=quantization, norm=norm)[0]
    if needs_grad:
        return _RopeSdpaFn.apply(query, key, value, cos4, sin4, mask, kind, bool(is_causal), scale)
    return _forward(query, key, value, cos4, sin4, mask, kind, bool(is_causal), scale, need_lse=False,
                    k_prepass=k_prepass)[0]


def rope_sdpa_fwd_with_lse(query, key, value, rope_cos, rope_sin, attn_mask=None, is_causal=False, scale=None,
                           quantization=None, q_norm_weight=None, k_norm_weight=None, norm_eps=1e-6,
                           k_prepass=False):
    """Forward returning (O, LSE) without autograd (LSE is fp32 [B, H, S], natural log)."""
    _check_dtypes(query, key, value)
    mask, kind = _mask4(attn_mask, value.dtype)
    return _forward(query, key, value, _tables4(rope_cos, query.device), _tables4(rope_sin, query.device),
                    mask, kind, bool(is_causal), scale, need_lse=True, quant=quantization,
                    norm=_norm_args(query, q_norm_weight, k_norm_weight, norm_eps), k_prepass=k_prepass)


def rope_rotate(x, rope_cos, rope_sin, out=None):
    """The eager rotation pass: R(x) for a BHSD tensor (its own HIP kernel, rope_sdpa_rotate).
    Each product and sum in fp32 without fused multiply-add, rounded to x's dtype."""
    lib = _abi.load()
    cos4, sin4 = _tables4(rope_cos, x.device), _tables4(rope_sin, x.device)
    if out is None:
        out = torch.empty(x.shape, dtype=x.dtype, device=x.device)
    tx, tc, ts, to = _desc(x), _desc(cos4), _desc(sin4), _desc(out)
    _check(lib.rope_sdpa_rotate(ctypes.byref(tx), ctypes.byref(tc), ctypes.byref(ts), ctypes.byref(to),
                                _stream(x.device)))
    return out


def scaled_dot_product_attention(query, key, value, attn_mask=None, is_causal=False, scale=None):
    """Plain attention, no rotation (the same HIP forward kernels without the tables): the
    attention half of the eager path.  Forward only: gradients are not available here."""
    if torch.is_grad_enabled() and (query.requires_grad or key.requires_grad or value.requires_grad):
        raise RopeSdpaError(-6)
    mask, kind = _mask4(attn_mask, query.dtype)
    return _forward(query, key, value, None, None, mask, kind, bool(is_causal), scale, need_lse=False)[0]


def debug_quantize_qk(query, key, rope_cos, rope_sin, bits=8):
    """The int8 (bits=8) or int4 (bits=4) codes and scales the quantized forward computes, for tests.

    Returns (q_codes, q_scales, k_codes, k_scales): int8 [B, H|Hkv, S, D] and fp32 [B, H|Hkv, ceil(S/64)].
    """
    lib = _abi.load()
    cos4, sin4 = _tables4(rope_cos, query.device), _tables4(rope_sin, query.device)
    call = _Call(query, key, key, cos4, sin4, None, 0, False, None, quant={8: "int8", 4: "int4"}[bits])
    B, H, S, D = query.shape
    nb = -(-S // 64)
    Hkv = key.shape[1]
    qc = torch.empty((B, H, S, D), dtype=torch.int8, device=query.device)
    kc = torch.empty((B, Hkv, S, D), dtype=torch.int8, device=query.device)
    qs = torch.empty((B, H, nb), dtype=torch.float32, device=query.device)
    ks = torch.empty((B, Hkv, nb), dtype=torch.float32, device=query.device)
    ws = call.workspace(False, query.device)
    _check(lib.rope_sdpa_debug_quantize_qk(ctypes.byref(call.args), qc.data_ptr(), kc.data_ptr(), qs.data_ptr(),
                                           ks.data_ptr(), ws.data_ptr(), ws.numel(), _stream(query.device)))
    return qc, qs, kc, ks


def rope_sdpa_bwd_explicit(query, key, value, rope_cos, rope_sin, out, lse, dout, attn_mask=None,
                           is_causal=False, scale=None):
    """Backward as a plain call: returns (dQ, dK, dV) w.r.t. the unrotated inputs."""
    mask, kind = _mask4(attn_mask, query.dtype)
    return _backward(query, key, value, _tables4(rope_cos, query.device), _tables4(rope_sin, query.device),
                     mask, kind, bool(is_causal), scale, out, lse, dout)


# ---- C-ABI names, re-exported -------------------------------------------------------------
def rope_sdpa_fwd(args, o, lse_ptr, ws_ptr, ws_bytes, stream) -> int:
    return _abi.load().rope_sdpa_fwd(args, o, lse_ptr, ws_ptr, ws_bytes, stream)


def rope_sdpa_fwd_noalloc(args, o, lse_ptr, stream) -> int:
    return _abi.load().rope_sdpa_fwd_noalloc(args, o, lse_ptr, stream)


def rope_sdpa_noalloc_scratch_bytes() -> int:
    return int(_abi.load().rope_sdpa_noalloc_scratch_bytes())


def rope_sdpa_bwd(args, o, lse_ptr, dout, dq, dk, dv, ws_ptr, ws_bytes, stream) -> int:
    return _abi.load().rope_sdpa_bwd(args, o, lse_ptr, dout, dq, dk, dv, ws_ptr, ws_bytes, stream)


def rope_sdpa_debug_quantize_qk(args, q_codes_ptr, k_codes_ptr, q_scales_ptr, k_scales_ptr, ws_ptr, ws_bytes,
                                stream) -> int:
    return _abi.load().rope_sdpa_debug_quantize_qk(args, q_codes_ptr, k_codes_ptr, q_scales_ptr, k_scales_ptr,
                                                   ws_ptr, ws_bytes, stream)


def rope_sdpa_rotate(x, cos, sin, out, stream) -> int:
    return _abi.load().rope_sdpa_rotate(x, cos, sin, out, stream)


def rope_sdpa_workspace_size(args, backward: int) -> int:
    n = ctypes.c_size_t(0)
    _check(_abi.load().rope_sdpa_workspace_size(args, int(backward), ctypes.byref(n)))
    return int(n.value)


def rope_sdpa_status_string(code: int) -> str:
    return _abi.status_string(code)


def rope_sdpa_get_stats() -> dict:
    s = RsStats()
    _abi.load().rope_sdpa_get_stats(ctypes.byref(s))
    return {name: int(getattr(s, name)) for name, _ in RsStats._fields_}


def rope_sdpa_reset_stats() -> None:
    _abi.load().rope_sdpa_reset_stats()


def rope_sdpa_debug_kernel_timing(enable: bool) -> None:
    """Measurement: record HIP events around each forward's attention kernel (see the header)."""
    _check(_abi.load().rope_sdpa_debug_kernel_timing(int(bool(enable))))


def rope_sdpa_debug_kernel_time():
    """(total milliseconds, launches) of the attention kernels timed since timing was enabled."""
    ms, n = ctypes.c_double(0.0), ctypes.c_uint64(0)
    _check(_abi.load().rope_sdpa_debug_kernel_time(ctypes.byref(ms), ctypes.byref(n)))
    return ms.value, n.value


def rope_sdpa_abi_version() -> int:
    return int(_abi.load().rope_sdpa_abi_version())


def get_dispatch_stats() -> dict:
    """Dispatch counters under the names the page uses: rope_instream counts no-grad calls,
    rope_autograd counts gradient calls, mask_all_true_skipped counts all-true bool masks."""
    s = rope_sdpa_get_stats()
    return {
        "rope_instream": s["fwd_instream"],
        "rope_autograd": s["fwd_autograd"],
        "backward": s["bwd_calls"],
        "masked_bool": s["masked_bool"],
        "masked_additive": s["masked_additive"],
        "causal": s["causal"],
        "quantized_int8": s["quant_int8"],
        "quantized_autograd": s["quant_bwd"],
        "mask_all_true_skipped": s["mask_all_true_skipped"],
        "errors": s["errors"],
        "pytorch_fallback": 0,
    }
