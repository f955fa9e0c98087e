"""Plain float64 NumPy oracle for fused RoPE + SDPA.  TEST INFRASTRUCTURE ONLY.

Only tests/, the smoke check and the bench's CPU-baseline leg may call this module.
It shares nothing with the HIP path.  Every step is the definition written out; the
only structure added is that query rows are processed in chunks (each chunk takes
an exact softmax over all keys of its rows, so chunking changes nothing but memory)
and that (batch, head) pairs may be mapped over a thread pool.

Citations name the page and section the step follows:
  [FR]  "Metal Flash Attention" (SimpleTuner docs), section "Fused RoPE + SDPA"
  [DF]  diffusers issue "Flux-family attention: flash-attn and other backends fail in an
        autocast context", sections "Describe the bug" and "Root cause, in order"
  [EN]  same page, section "Enable In SimpleTuner"
  [RQ]  same page, section "Requirements"
  [PR]  SimpleTuner pull request "metal-flash-attention: causal training ungated;
        fused RoPE + Attention for Flux1/Flux2, Z-Image and Krea"
Where the pages are silent the reading taken is stated at the function.
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np


def _np64(x) -> np.ndarray:
    """Exact float64 upcast of a torch tensor or array (bf16/fp16/fp32 values are exact in float64)."""
    if x is None:
        return None
    if hasattr(x, "detach"):
        import torch

        x = x.detach().to("cpu")
        if x.dtype == torch.bool:
            return x.numpy()
        return x.to(torch.float64).numpy()
    x = np.asarray(x)
    return x if x.dtype == np.bool_ else x.astype(np.float64)


def _tables4(t: np.ndarray) -> np.ndarray:
    """Cos/sin table as [Bt, 1, S, D] (Bt = 1 or B): shapes [S,D], [1,S,D], [B,S,D] are accepted [FR]."""
    t = np.asarray(t, dtype=np.float64)
    if t.ndim == 2:
        t = t[None]
    assert t.ndim == 3, "rope tables are [S,D], [1,S,D] or [B,S,D]"
    return t[:, None, :, :]


# --------------------------------------------------------------------------------------
# Rotation  [FR]: interleaved-pair rotary embedding applied to Q and K (not V); the
# complex-multiply formulation (x_2i + i x_2i+1) * (cos + i sin) is the same rotation.
# --------------------------------------------------------------------------------------
def _pair_swap(x: np.ndarray) -> np.ndarray:
    """J(x): J(x)[2i] = -x[2i+1], J(x)[2i+1] = x[2i]  (multiplication by i on each pair)."""
    out = np.empty_like(x)
    out[..., 0::2] = -x[..., 1::2]
    out[..., 1::2] = x[..., 0::2]
    return out


def rope_rotate(x, cos, sin) -> np.ndarray:
    """R(x) = x * cos + J(x) * sin on [B, H, S, D] with per-position tables [FR].

    With pair-duplicated tables this is x'_2i = x_2i c - x_2i+1 s, x'_2i+1 = x_2i s + x_2i+1 c.
    """
    x = _np64(x)
    c, s = _tables4(_np64(cos)), _tables4(_np64(sin))
    return x * c + _pair_swap(x) * s


def rope_rotate_vjp(g, cos, sin) -> np.ndarray:
    """Exact vector-Jacobian product of rope_rotate w.r.t. x (the gradient of the unrotated input).

    gx_2i   =  g_2i c_2i   + g_2i+1 s_2i+1
    gx_2i+1 = -g_2i s_2i   + g_2i+1 c_2i+1
    For pair-duplicated tables this is the same pairwise rotation with sin negated,
    which is how [FR] states the backward of the fused path.
    """
    g = _np64(g)
    c, s = _tables4(_np64(cos)), _tables4(_np64(sin))
    gc = g * c
    gs = g * s
    out = np.empty_like(g)
    out[..., 0::2] = gc[..., 0::2] + gs[..., 1::2]
    out[..., 1::2] = -gs[..., 0::2] + gc[..., 1::2]
    return out


# --------------------------------------------------------------------------------------
# Masks  [EN]: bool masks mean True = attend; additive float masks are added to the
# scores; batched [B,H,Sq,Skv] and broadcast shapes such as [B,1,1,Skv] (up to 4-D).
# Reading: the additive mask is added after scaling and is not itself scaled (the page
# mirrors the PyTorch SDPA signature, whose convention this is).
# --------------------------------------------------------------------------------------
def _additive(m, kind):
    """bool -> 0 where True, -inf where False; additive -> the values, as float64."""
    m = _np64(m)
    if kind == "bool":
        return np.where(m.astype(bool), 0.0, -np.inf)
    return m.astype(np.float64)


class _LazyMask:
    """A 4-D mask kept in its own dtype; (b, h, rows) slices are converted on demand so that
    full-size [B, H, S, S] masks never need a float64 copy."""

    def __init__(self, mask, kind):
        while mask.dim() < 4 if hasattr(mask, "dim") else np.ndim(mask) < 4:
            mask = mask[None]
        self.m, self.kind = mask, kind
        self.shape = tuple(mask.shape)

    def __getitem__(self, bh):
        b, h = bh
        return _LazyHead(self.m[b, h], self.kind)


class _LazyHead:
    def __init__(self, m2, kind):
        self.m2, self.kind = m2, kind
        self.shape = tuple(m2.shape)

    def __getitem__(self, rows):
        return _additive(self.m2[rows], self.kind)


def mask_to_additive(mask, kind: str):
    """The mask as additive float64 values broadcastable to [B,H,Sq,Skv], or None.  Large
    masks stay lazy: indexing [b, h] and then rows converts only that slice."""
    if kind in (None, "none") or mask is None:
        return None
    if kind not in ("bool", "additive"):
        raise ValueError(f"unknown mask kind {kind!r}")
    if (mask.numel() if hasattr(mask, "numel") else np.size(mask)) <= (1 << 22):
        m = _additive(mask, kind)
        while m.ndim < 4:
            m = m[None]
        return m
    return _LazyMask(mask, kind)


def _mask_slice(madd, b: int, h: int):
    if madd is None:
        return None
    return madd[b if madd.shape[0] > 1 else 0, h if madd.shape[1] > 1 else 0]


def _scores(qr_rows, kr, scale, mrows, causal, rows):
    """s_ij = scale <q'_i, k'_j> + m_ij, with -inf above the diagonal when causal (top-left aligned)."""
    s = scale * (qr_rows @ kr.T)
    if mrows is not None:
        s = s + mrows
    if causal:
        s = np.where(np.arange(kr.shape[0])[None, :] > rows[:, None], -np.inf, s)
    return s


def _softmax_rows(s):
    """Exact row softmax.  A row whose every score is -inf has no key to attend: P = 0, LSE = -inf."""
    m = s.max(axis=1)
    ok = np.isfinite(m)
    m0 = np.where(ok, m, 0.0)
    e = np.exp(s - m0[:, None])
    l = e.sum(axis=1)
    p = np.where(ok[:, None], e / np.where(ok, l, 1.0)[:, None], 0.0)
    lse = np.where(ok, m0 + np.log(np.where(ok, l, 1.0)), -np.inf)
    return p, lse


def _mask_rows(mhead, rows):
    if mhead is None:
        return None
    return mhead[rows] if mhead.shape[0] > 1 else mhead[0:1]


def _map_heads(fn, pairs, workers):
    if workers <= 1 or len(pairs) <= 1:
        return [fn(p) for p in pairs]
    with ThreadPoolExecutor(max_workers=workers) as ex:
        return list(ex.map(fn, pairs))


def _blas_single_thread():
    try:
        from threadpoolctl import threadpool_limits

        return threadpool_limits(limits=1)
    except Exception:  # pragma: no cover - threadpoolctl is present in this image
        import contextlib

        return contextlib.nullcontext()


def attention_forward(qr, kr, v, scale, madd=None, causal=False, rows=None, pairs=None,
                      chunk=512, workers=1):
    """O = softmax(scale * Q' K'^T + M) V and LSE per row, on already-rotated Q', K'.

    qr, kr, v: float64 [B, H, S, D].  rows: optional query indices to evaluate (all by
    default).  pairs: optional list of (b, h) to evaluate (all by default).
    Returns (O [len(pairs), len(rows), D], LSE [len(pairs), len(rows)]) when pairs is
    given, else ([B, H, rows, D], [B, H, rows]).
    """
    B, H, Sq, D = qr.shape
    idx = np.arange(Sq) if rows is None else np.asarray(rows, dtype=np.int64)
    plist = [(b, h) for b in range(B) for h in range(H)] if pairs is None else list(pairs)

    def one(bh):
        b, h = bh
        mh = _mask_slice(madd, b, h)
        O = np.empty((len(idx), v.shape[-1]))
        L = np.empty(len(idx))
        for c0 in range(0, len(idx), chunk):
            r = idx[c0:c0 + chunk]
            s = _scores(qr[b, h, r], kr[b, h], scale, _mask_rows(mh, r), causal, r)
            p, lse = _softmax_rows(s)
            O[c0:c0 + len(r)] = p @ v[b, h]
            L[c0:c0 + len(r)] = lse
        return O, L

    with _blas_single_thread() if workers > 1 else _null():
        res = _map_heads(one, plist, workers)
    O = np.stack([r[0] for r in res])
    L = np.stack([r[1] for r in res])
    if pairs is None:
        O = O.reshape(B, H, len(idx), -1)
        L = L.reshape(B, H, len(idx))
    return O, L


def attention_backward(qr, kr, v, do, scale, madd=None, causal=False, pairs=None, chunk=512, workers=1):
    """Gradients of sum(O * dO) w.r.t. Q', K', V (rotated frame), textbook softmax backward.

    dV = P^T dO;  dP = dO V^T;  delta_i = sum_j P_ij dP_ij;  dS = P o (dP - delta);
    dQ' = scale dS K';  dK' = scale dS^T Q'.
    Returns (dqr, dkr, dv), each [B,H,S,D] (or [len(pairs),S,D] when pairs is given).
    """
    B, H, Sq, D = qr.shape
    Skv = kr.shape[2]
    plist = [(b, h) for b in range(B) for h in range(H)] if pairs is None else list(pairs)

    def one(bh):
        b, h = bh
        mh = _mask_slice(madd, b, h)
        dq = np.zeros((Sq, D))
        dk = np.zeros((Skv, D))
        dv = np.zeros((Skv, v.shape[-1]))
        for c0 in range(0, Sq, chunk):
            r = np.arange(c0, min(Sq, c0 + chunk))
            s = _scores(qr[b, h, r], kr[b, h], scale, _mask_rows(mh, r), causal, r)
            p, _ = _softmax_rows(s)
            dov = do[b, h, r]
            dv += p.T @ dov
            dp = dov @ v[b, h].T
            delta = (p * dp).sum(axis=1)
            ds = p * (dp - delta[:, None])
            dq[r] = scale * (ds @ kr[b, h])
            dk += scale * (ds.T @ qr[b, h, r])
        return dq, dk, dv

    with _blas_single_thread() if workers > 1 else _null():
        res = _map_heads(one, plist, workers)
    out = [np.stack([r[i] for r in res]) for i in range(3)]
    if pairs is None:
        out = [o.reshape(B, H, *o.shape[1:]) for o in out]
    return tuple(out)


def _null():
    import contextlib

    return contextlib.nullcontext()


def _resolve_scale(scale, D):
    """[FR]: scale=None means 1/sqrt(D), taken here as the float64 nearest to the exact value
    (1/math.sqrt(D) can be one ulp off, e.g. at D = 128)."""
    if scale is not None:
        return float(scale)
    from decimal import Decimal, localcontext

    with localcontext() as ctx:
        ctx.prec = 60
        return float(Decimal(1) / Decimal(int(D)).sqrt())


def _kv_group(H, Hkv):
    """Query heads per K/V head (grouped-query attention, [FR]): query head h reads K/V head
    h // (H / Hkv) = h Hkv / H.  Hkv == H is ordinary multi-head attention."""
    if Hkv <= 0 or H % Hkv != 0:
        raise ValueError(f"{H} query heads cannot share {Hkv} K/V heads evenly")
    return H // Hkv


def expand_kv(x, H):
    """[B, Hkv, S, D] -> [B, H, S, D]: each K/V head repeated for the query heads that read it
    ([FR]: GQA inputs are rotated at the K/V head count and expanded afterwards)."""
    G = _kv_group(H, x.shape[1])
    return np.repeat(x, G, axis=1) if G > 1 else x


def reduce_kv(g, Hkv):
    """Gradient of expand_kv: [B, H, S, D] -> [B, Hkv, S, D], summing each group's heads."""
    B, H = g.shape[:2]
    G = _kv_group(H, Hkv)
    return g.reshape(B, Hkv, G, *g.shape[2:]).sum(axis=2) if G > 1 else g


def rms_norm(x, w, eps):
    """RMSNorm over the head dimension, as flux-style attention applies it to Q and K just
    before the rotation ([DF] root cause): x / sqrt(mean_d x_d^2 + eps) * w_d, in float64."""
    x = _np64(x)
    w = _np64(w)
    return x / np.sqrt((x * x).mean(axis=-1, keepdims=True) + float(eps)) * w


def rope_sdpa_forward(q, k, v, cos, sin, mask=None, mask_kind="none", causal=False, scale=None,
                      rows=None, pairs=None, workers=1, q_norm_weight=None, k_norm_weight=None, norm_eps=1e-6):
    """Fused RoPE + SDPA forward [FR]: rotate Q and K, then exact attention.  K and V may have
    fewer heads than Q (grouped-query attention): they are rotated at their own head count and
    expanded afterwards.  With q_norm_weight / k_norm_weight, Q / K are RMS-normalized over
    the head dimension first (rms_norm).  Returns (O, LSE)."""
    q64, k64, v64 = _np64(q), _np64(k), _np64(v)
    if q_norm_weight is not None:
        q64 = rms_norm(q64, q_norm_weight, norm_eps)
    if k_norm_weight is not None:
        k64 = rms_norm(k64, k_norm_weight, norm_eps)
    qr = rope_rotate(q64, cos, sin)
    kr = expand_kv(rope_rotate(k64, cos, sin), q64.shape[1])
    v64 = expand_kv(v64, q64.shape[1])
    madd = mask_to_additive(mask, mask_kind)
    return attention_forward(qr, kr, v64, _resolve_scale(scale, q64.shape[-1]), madd, causal,
                             rows=rows, pairs=pairs, workers=workers)


def rope_sdpa_backward(q, k, v, cos, sin, do, mask=None, mask_kind="none", causal=False, scale=None,
                       pairs=None, workers=1):
    """Gradients w.r.t. the unrotated Q, K and V [FR]: attention backward in the rotated frame,
    then the exact VJP of the rotation on dQ' and dK'.  The mask and tables get no gradient.
    Returns (dQ, dK, dV).  With grouped-query attention (K, V with Hkv < H heads) dK and dV
    have Hkv heads: the gradients of the expanded heads are summed over each group (the VJP of
    the expansion) before the inverse rotation; `pairs` is then not accepted.
    """
    q64, k64, v64, do64 = _np64(q), _np64(k), _np64(v), _np64(do)
    H, Hkv = q64.shape[1], k64.shape[1]
    qr = rope_rotate(q64, cos, sin)
    kr = expand_kv(rope_rotate(k64, cos, sin), H)
    v64 = expand_kv(v64, H)
    madd = mask_to_additive(mask, mask_kind)
    if Hkv != H and pairs is not None:
        raise ValueError("pairs are not supported with grouped-query attention")
    dqr, dkr, dv = attention_backward(qr, kr, v64, do64, _resolve_scale(scale, q64.shape[-1]), madd,
                                      causal, pairs=pairs, workers=workers)
    if pairs is None:
        dkr, dv = reduce_kv(dkr, Hkv), reduce_kv(dv, Hkv)
        return rope_rotate_vjp(dqr, cos, sin), rope_rotate_vjp(dkr, cos, sin), dv
    # per-pair tables: index the batch of each (b, h)
    c, s = _np64(cos), _np64(sin)
    if c.ndim == 2:
        c, s = c[None], s[None]
    dq = np.stack([rope_rotate_vjp(dqr[i][None, None], c[b if c.shape[0] > 1 else 0][None],
                                   s[b if s.shape[0] > 1 else 0][None])[0, 0]
                   for i, (b, _) in enumerate(pairs)])
    dk = np.stack([rope_rotate_vjp(dkr[i][None, None], c[b if c.shape[0] > 1 else 0][None],
                                   s[b if s.shape[0] > 1 else 0][None])[0, 0]
                   for i, (b, _) in enumerate(pairs)])
    return dq, dk, dv


# --------------------------------------------------------------------------------------
# Blockwise int8 variant.  The pages name an int8 mode with blockwise quantization
# ([EN] quantized aliases; [RQ] QUANT_INT8 / QUANT_BLOCK_WISE) but do not say what is
# quantized.  Reading taken: the rotated Q and K are quantized symmetrically to
# [-127, 127] with one fp32 scale per (batch, head, 64-token block) spanning all of D;
# V stays in the input precision.  Because the quantizer turns floating point into
# integers, it takes its decisions in fp32, the precision of the kernel that must
# reproduce them: the rotation is two fp32 products each rounded, then an fp32
# sum/difference rounded (no fused multiply-add); inv = fp32(127 / amax); code =
# round-half-even(fp32(x * inv)) clipped to [-127, 127]; the dequantization scale is
# fp32(amax / 127); an all-zero block gets code 0 and scale 0.
# The int4 alias ([EN]: "-int4" sets QUANT_INT4 with QUANT_BLOCK_WISE) takes the same
# reading with qmax = 7: codes in [-7, 7], inv = fp32(7 / amax), scale = fp32(amax / 7).
# --------------------------------------------------------------------------------------
def rope_rotate_f32(x, cos, sin) -> np.ndarray:
    """Rotation evaluated in fp32 with every product and sum rounded to fp32 (no FMA)."""
    import torch

    if hasattr(x, "detach"):
        x = x.detach().to("cpu").to(torch.float32).numpy()
    x = np.asarray(x, dtype=np.float32)
    c = _tables4(_np64(cos)).astype(np.float32)
    s = _tables4(_np64(sin)).astype(np.float32)
    x0, x1 = x[..., 0::2], x[..., 1::2]
    out = np.empty_like(x)
    out[..., 0::2] = (x0 * c[..., 0::2]) - (x1 * s[..., 0::2])
    out[..., 1::2] = (x0 * s[..., 1::2]) + (x1 * c[..., 1::2])
    return out


def quantize_blockwise(xr32: np.ndarray, block: int = 64, qmax: int = 127):
    """Symmetric codes in [-qmax, qmax] and fp32 scales per (b, h, block of `block` tokens).

    Returns (codes int8 [B,H,S,D], scales float32 [B,H,ceil(S/block)]).  A final
    partial block uses only its valid rows.
    """
    xr32 = np.asarray(xr32, dtype=np.float32)
    B, H, S, D = xr32.shape
    nb = (S + block - 1) // block
    qm = np.float32(qmax)
    codes = np.zeros((B, H, S, D), dtype=np.int8)
    scales = np.zeros((B, H, nb), dtype=np.float32)
    for t in range(nb):
        blk = xr32[:, :, t * block:(t + 1) * block, :]
        amax = np.abs(blk).max(axis=(2, 3)).astype(np.float32)  # [B,H]
        sc = (amax / qm).astype(np.float32)
        inv = (qm / np.where(amax > 0, amax, np.float32(1.0))).astype(np.float32)
        qv = np.rint(blk * inv[:, :, None, None])  # fp32 product, round half to even
        qv = np.clip(qv, -qmax, qmax)
        qv = np.where((amax > 0)[:, :, None, None], qv, 0)
        codes[:, :, t * block:(t + 1) * block, :] = qv.astype(np.int8)
        scales[:, :, t] = np.where(amax > 0, sc, np.float32(0.0))
    return codes, scales


def quantize_blockwise_int8(xr32: np.ndarray, block: int = 64):
    """int8 codes ([-127, 127]) and scales: quantize_blockwise with qmax = 127."""
    return quantize_blockwise(xr32, block, 127)


def quantize_blockwise_int4(xr32: np.ndarray, block: int = 64):
    """int4 codes ([-7, 7], held in int8) and scales: quantize_blockwise with qmax = 7."""
    return quantize_blockwise(xr32, block, 7)


def dequantize_blockwise(codes: np.ndarray, scales: np.ndarray, block: int = 64) -> np.ndarray:
    """x_hat = scale_t * code, in float64."""
    S = codes.shape[2]
    sc = np.repeat(scales.astype(np.float64), block, axis=2)[:, :, :S]
    return codes.astype(np.float64) * sc[..., None]


def _qmax(bits: int) -> int:
    return {8: 127, 4: 7}[bits]


def quantized_qk(q, k, cos, sin, bits=8, block=64):
    """The dequantized rotated Q and K the quantized variant attends with (float64), at
    their own head counts."""
    qc, qs = quantize_blockwise(rope_rotate_f32(q, cos, sin), block, _qmax(bits))
    kc, ks = quantize_blockwise(rope_rotate_f32(k, cos, sin), block, _qmax(bits))
    return dequantize_blockwise(qc, qs, block), dequantize_blockwise(kc, ks, block)


def rope_sdpa_forward_quant(q, k, v, cos, sin, bits=8, scale=None, rows=None, pairs=None, block=64, workers=1,
                            codes=None, mask=None, mask_kind="none", causal=False):
    """Quantized variant (bits = 8 or 4): rotate in fp32, quantize Q' and K' blockwise,
    attend on the dequantized values (with masks and causal as the unquantized forward:
    [EN] the quantized dispatchers take the same masks).

    `codes` may carry externally supplied ((q_codes, q_scales), (k_codes, k_scales)) so the
    attention part can be checked on exactly those quantized values.
    Returns (O, LSE).
    """
    if codes is None:
        qh, kh = quantized_qk(q, k, cos, sin, bits, block)
    else:
        (qc, qs), (kc, ks) = codes
        qh, kh = dequantize_blockwise(qc, qs, block), dequantize_blockwise(kc, ks, block)
    kh = expand_kv(kh, qh.shape[1])  # K quantized at its own head count
    v64 = expand_kv(_np64(v), qh.shape[1])
    return attention_forward(qh, kh, v64, _resolve_scale(scale, qh.shape[-1]), mask_to_additive(mask, mask_kind),
                             causal, rows=rows, pairs=pairs, workers=workers)


def rope_sdpa_forward_int8(q, k, v, cos, sin, scale=None, rows=None, pairs=None, block=64, workers=1,
                           codes=None):
    """int8 variant: rope_sdpa_forward_quant with bits = 8."""
    return rope_sdpa_forward_quant(q, k, v, cos, sin, 8, scale, rows, pairs, block, workers, codes)


def rope_sdpa_backward_quant(q, k, v, cos, sin, do, bits=8, scale=None, block=64, workers=1, mask=None,
                             mask_kind="none", causal=False):
    """Gradients of the quantized variant w.r.t. the unrotated Q, K and V ([EN]: quantized
    training goes through a quantized autograd entry point; [RQ] names it).  The pages do
    not say how a gradient passes the quantizer.  Reading taken (straight-through): the
    quantize-dequantize step counts as the identity in the backward, so the attention
    backward runs at the values the forward attended with (the dequantized Q', K' and V),
    and its dQ', dK' go unchanged into the inverse rotation.  Returns (dQ, dK, dV); dK and
    dV at the K/V head count (summed over each group)."""
    do64 = _np64(do)
    qh, kh = quantized_qk(q, k, cos, sin, bits, block)
    H, Hkv = qh.shape[1], kh.shape[1]
    dqh, dkh, dv = attention_backward(qh, expand_kv(kh, H), expand_kv(_np64(v), H), do64,
                                      _resolve_scale(scale, qh.shape[-1]), mask_to_additive(mask, mask_kind),
                                      causal, workers=workers)
    dkh, dv = reduce_kv(dkh, Hkv), reduce_kv(dv, Hkv)
    return rope_rotate_vjp(dqh, cos, sin), rope_rotate_vjp(dkh, cos, sin), dv


def default_workers() -> int:
    return len(os.sched_getaffinity(0))
