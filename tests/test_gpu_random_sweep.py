"""Seeded random sweep of small configurations: forward (O, LSE) and, for most cases, the
backward (dQ, dK, dV) against the oracle.

Each case draws its own batch, head counts (grouped-query K/V included), ragged sequence
length, head dim, dtype, mask kind and broadcast shape (or causal), per-sample or shared
tables, explicit or default scale, and contiguous or [B, S, H, D]-strided inputs, so that
combinations the fixed grids do not list are covered too.  The case list is fixed by the
seed below; a failure names its case.
"""
import os

import numpy as np
import pytest
import torch

import synthetic as syn
import rope_flash_attention_amd as rfa
from oracle import rope_sdpa_backward, rope_sdpa_forward
from parity_util import check_grad, check_lse, check_out, dev, to64

pytestmark = pytest.mark.gpu

# RS_SWEEP_SCALE multiplies the case counts (a longer sweep on request; the seeds stay fixed,
# so the default cases are always the first ones)
_SCALE = max(1, int(os.environ.get("RS_SWEEP_SCALE", "1")))
N_CASES = 100 * _SCALE


def _cases():
    r = np.random.default_rng(20261203)
    out = []
    for i in range(N_CASES):
        B = int(r.choice([1, 2, 3]))
        H = int(r.choice([1, 2, 3, 4, 6]))
        Hkv = int(r.choice([d for d in range(1, H + 1) if H % d == 0]))
        S = int(r.integers(1, 601))
        D = int(r.choice([64, 128]))
        dtype = str(r.choice(["bf16", "f16", "f32"]))
        variant = str(r.choice(["none", "causal", "bool", "additive"]))
        shape = None
        if variant in ("bool", "additive"):
            shape = tuple(int(full) if r.random() < 0.5 else 1 for full in (B, H, S))
            shape = shape + (S if r.random() < 0.8 else 1,)
        per_sample = bool(r.random() < 0.3)
        scale = None if r.random() < 0.6 else float(r.uniform(0.05, 0.3))
        strided = bool(r.random() < 0.3)
        grad = bool(r.random() < 0.7)
        out.append(dict(i=i, B=B, H=H, Hkv=Hkv, S=S, D=D, dtype=dtype, variant=variant, shape=shape,
                        per_sample=per_sample, scale=scale, strided=strided, grad=grad))
    return out


CASES = _cases()


def _bshd(t, d):
    """The same values as a [B, H, S, D] view of a contiguous [B, S, H, D] device tensor."""
    return t.transpose(1, 2).contiguous().to(d).transpose(1, 2)


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"c{c['i']}_b{c['B']}h{c['H']}kv{c['Hkv']}s{c['S']}"
                         f"d{c['D']}_{c['dtype']}_{c['variant']}{'_g' if c['grad'] else ''}")
def test_random_case(case):
    c = case
    kw = {}
    if c["variant"] == "causal":
        kw = dict(causal=True)
    elif c["variant"] != "none":
        kw = dict(mask_kind=c["variant"], mask_shape=c["shape"])
    w = syn.random_small(c["B"], c["H"], c["S"], c["D"], c["dtype"], seed=900 + c["i"],
                         per_sample_tables=c["per_sample"], with_grad=c["grad"],
                         kv_heads=c["Hkv"] if c["Hkv"] < c["H"] else None, **kw)
    d = dev()
    if c["strided"]:
        q, k, v = (_bshd(t, d) for t in (w.q, w.k, w.v))
    else:
        q, k, v = (t.to(d) for t in (w.q, w.k, w.v))
    m = w.mask.to(d) if w.mask is not None else None
    okw = dict(mask=w.mask, mask_kind=w.mask_kind, causal=w.causal, scale=c["scale"], workers=8)
    O_ref, L_ref = rope_sdpa_forward(w.q, w.k, w.v, w.cos, w.sin, **okw)
    if c["grad"]:
        q, k, v = (t.detach().requires_grad_() for t in (q, k, v))
        o = rfa.rope_scaled_dot_product_attention(q, k, v, w.cos.to(d), w.sin.to(d), attn_mask=m,
                                                  is_causal=w.causal, scale=c["scale"])
        o.backward(w.do.to(d))
        torch.cuda.synchronize()
        check_out("O", to64(o), O_ref, c["dtype"])
        grads = rope_sdpa_backward(w.q, w.k, w.v, w.cos, w.sin, w.do, **okw)
        for name, g, ref in zip(("dQ", "dK", "dV"), (q.grad, k.grad, v.grad), grads):
            check_grad(name, to64(g), ref, c["dtype"])
    else:
        o, lse = rfa.rope_sdpa_fwd_with_lse(q, k, v, w.cos.to(d), w.sin.to(d), attn_mask=m,
                                            is_causal=w.causal, scale=c["scale"])
        torch.cuda.synchronize()
        check_out("O", to64(o), O_ref, c["dtype"])
        check_lse(to64(lse), L_ref, c["dtype"])


# ---- forward-only variants ----------------------------------------------------------------
# K rotated by its own pass, the Q/K RMSNorm prologue, fp32 Q/K beside 16-bit V, and the
# blockwise int8 / int4 forwards in both quantization modes, each under the mask kinds it
# takes, on random shapes.

N_VARIANT_CASES = 64 * _SCALE
MODES = ["k_prepass", "rmsnorm", "f32qk", "f32qk_rmsnorm", "int8", "int4", "int8_prepass", "int4_prepass"]


def _variant_cases():
    r = np.random.default_rng(20261204)
    out = []
    for i in range(N_VARIANT_CASES):
        mode = MODES[i % len(MODES)]
        B = int(r.choice([1, 2]))
        H = int(r.choice([1, 2, 4, 6]))
        Hkv = int(r.choice([d for d in range(1, H + 1) if H % d == 0]))
        S = int(r.integers(1, 520))
        D = int(r.choice([64, 128]))
        vdtype = str(r.choice(["bf16", "f16"]))
        kinds = ["none", "causal", "bool"] + (["additive"] if mode.startswith("int") else [])
        variant = str(r.choice(kinds))
        shape = None
        if variant in ("bool", "additive"):
            shape = tuple(int(full) if r.random() < 0.5 else 1 for full in (B, H, S))
            shape = shape + (S if r.random() < 0.8 else 1,)
        scale = None if r.random() < 0.6 else float(r.uniform(0.05, 0.3))
        out.append(dict(i=i, mode=mode, B=B, H=H, Hkv=Hkv, S=S, D=D, vdtype=vdtype, variant=variant,
                        shape=shape, scale=scale, per_sample=bool(r.random() < 0.3)))
    return out


VARIANT_CASES = _variant_cases()


@pytest.mark.parametrize("case", VARIANT_CASES, ids=lambda c: f"v{c['i']}_{c['mode']}_b{c['B']}h{c['H']}kv{c['Hkv']}"
                         f"s{c['S']}d{c['D']}_{c['vdtype']}_{c['variant']}")
def test_random_forward_variant(case):
    from oracle import rope_sdpa_forward_quant

    c = case
    kw = {}
    if c["variant"] == "causal":
        kw = dict(causal=True)
    elif c["variant"] != "none":
        kw = dict(mask_kind=c["variant"], mask_shape=c["shape"])
    seed = 1900 + c["i"]
    w = syn.random_small(c["B"], c["H"], c["S"], c["D"], c["vdtype"], seed=seed, per_sample_tables=c["per_sample"],
                         kv_heads=c["Hkv"] if c["Hkv"] < c["H"] else None, **kw)
    q, k = w.q, w.k
    mode = c["mode"]
    if mode.startswith("f32qk"):  # fp32 Q and K with values off the 16-bit grid
        q = syn.normal(seed, syn.STREAM_Q, tuple(w.q.shape), "f32")
        k = syn.normal(seed, syn.STREAM_K, tuple(w.k.shape), "f32")
    norm = None
    if mode.endswith("rmsnorm"):
        g = np.random.default_rng(seed)
        norm = (torch.from_numpy(g.uniform(0.5, 1.5, c["D"]).astype(np.float32)),
                torch.from_numpy(g.uniform(0.5, 1.5, c["D"]).astype(np.float32)), 1e-6)
    d = dev()
    m = w.mask.to(d) if w.mask is not None else None
    gkw = dict(attn_mask=m, is_causal=w.causal, scale=c["scale"])
    okw = dict(mask=w.mask, mask_kind=w.mask_kind, causal=w.causal, scale=c["scale"], workers=8)
    if mode.startswith("int"):
        gkw["quantization"] = mode
        O_ref, L_ref = rope_sdpa_forward_quant(q, k, w.v, w.cos, w.sin, bits=4 if mode.startswith("int4") else 8,
                                               **okw)
    else:
        if mode == "k_prepass":
            gkw["k_prepass"] = True
        if norm is not None:
            gkw.update(q_norm_weight=norm[0].to(d), k_norm_weight=norm[1].to(d), norm_eps=norm[2])
            okw.update(q_norm_weight=norm[0], k_norm_weight=norm[1], norm_eps=norm[2])
        O_ref, L_ref = rope_sdpa_forward(q, k, w.v, w.cos, w.sin, **okw)
    with torch.no_grad():
        o, lse = rfa.rope_sdpa_fwd_with_lse(q.to(d), k.to(d), w.v.to(d), w.cos.to(d), w.sin.to(d), **gkw)
    torch.cuda.synchronize()
    assert o.dtype == w.v.dtype
    check_out("O", to64(o), O_ref, c["vdtype"])
    check_lse(to64(lse), L_ref, c["vdtype"])


# ---- forwards whose units are cut into key ranges -----------------------------------------
# With at least 16 key tiles and fewer units than resident workgroups, the forward cuts the
# units' key ranges into pieces on separate workgroups and merges them (no causal masking);
# these cases reach that path with random lengths, heads, masks and dtypes.

N_SPLIT_CASES = 24 * _SCALE


def _split_cases():
    r = np.random.default_rng(20261205)
    out = []
    for i in range(N_SPLIT_CASES):
        B = int(r.choice([1, 2]))
        H = int(r.choice([1, 2, 3]))
        Hkv = int(r.choice([d for d in range(1, H + 1) if H % d == 0]))
        S = int(r.integers(1024, 2600))
        D = int(r.choice([64, 128]))
        dtype = str(r.choice(["bf16", "f16", "f32"]))
        variant = str(r.choice(["none", "bool", "additive"]))
        shape = None
        if variant != "none":
            shape = (int(r.choice([1, B])), int(r.choice([1, H])), int(r.choice([1, S])), S)
        out.append(dict(i=i, B=B, H=H, Hkv=Hkv, S=S, D=D, dtype=dtype, variant=variant, shape=shape,
                        scale=None if r.random() < 0.6 else float(r.uniform(0.05, 0.3)),
                        lse=bool(r.random() < 0.7)))
    return out


SPLIT_CASES = _split_cases()


@pytest.mark.parametrize("case", SPLIT_CASES, ids=lambda c: f"s{c['i']}_b{c['B']}h{c['H']}kv{c['Hkv']}s{c['S']}"
                         f"d{c['D']}_{c['dtype']}_{c['variant']}{'_lse' if c['lse'] else ''}")
def test_random_split_forward(case):
    c = case
    kw = {} if c["variant"] == "none" else dict(mask_kind=c["variant"], mask_shape=c["shape"])
    w = syn.random_small(c["B"], c["H"], c["S"], c["D"], c["dtype"], seed=2900 + c["i"],
                         kv_heads=c["Hkv"] if c["Hkv"] < c["H"] else None, **kw)
    d = dev()
    m = w.mask.to(d) if w.mask is not None else None
    gkw = dict(attn_mask=m, scale=c["scale"])
    with torch.no_grad():
        if c["lse"]:
            o, lse = rfa.rope_sdpa_fwd_with_lse(w.q.to(d), w.k.to(d), w.v.to(d), w.cos.to(d), w.sin.to(d), **gkw)
        else:
            o = rfa.rope_scaled_dot_product_attention(w.q.to(d), w.k.to(d), w.v.to(d), w.cos.to(d), w.sin.to(d),
                                                      **gkw)
    torch.cuda.synchronize()
    O_ref, L_ref = rope_sdpa_forward(w.q, w.k, w.v, w.cos, w.sin, mask=w.mask, mask_kind=w.mask_kind,
                                     scale=c["scale"], workers=8)
    check_out("O", to64(o), O_ref, c["dtype"])
    if c["lse"]:
        check_lse(to64(lse), L_ref, c["dtype"])


# ---- bool masks with whole excluded tiles ---------------------------------------------------
# Element-wise random masks almost never leave a 64 x 64 tile all-false, so the skipping of
# all-false key tiles (and the next-tile table built for it) is reached here: runs of
# excluded keys (key padding, [B, 1, 1, S] or [B, H, 1, S]) or excluded key and query ranges
# ([B, 1, S, S]: whole rows excluded give O = 0 and LSE = -inf), of random positions and
# lengths, at lengths up to 2600 (the longer ones take the split schedule).

N_RUN_CASES = 32 * _SCALE


def _runs(r, S, n_max, len_max, min_keep=0):
    """Bool [S]: True except for 1..n_max runs of random start and length 1..len_max, drawn
    again until at least min_keep positions stay True."""
    while True:
        keep = np.ones(S, dtype=bool)
        for _ in range(int(r.integers(1, n_max + 1))):
            a = int(r.integers(0, S))
            keep[a:a + int(r.integers(1, len_max + 1))] = False
        if keep.sum() >= min_keep:
            return keep


def _run_cases():
    r = np.random.default_rng(20261206)
    out = []
    for i in range(N_RUN_CASES):
        B = int(r.choice([1, 2]))
        H = int(r.choice([1, 2, 3, 4]))
        Hkv = int(r.choice([d for d in range(1, H + 1) if H % d == 0]))
        S = int(r.integers(64, 2601))
        out.append(dict(i=i, B=B, H=H, Hkv=Hkv, S=S, D=int(r.choice([64, 128])),
                        dtype=str(r.choice(["bf16", "f16", "f32"])),
                        form=str(r.choice(["keys", "keys_per_head", "keys_and_queries"])),
                        scale=None if r.random() < 0.6 else float(r.uniform(0.05, 0.3)),
                        grad=bool(r.random() < 0.7) and S <= 1200))
    return out


RUN_CASES = _run_cases()


def _run_mask(c):
    """The case's bool mask (True = attend), drawn from its own seed.  Key masks keep at least
    S/8 keys (and 2): with a single key left in every row the exact gradients of Q and K
    vanish, and a relative error bound then measures only rounding noise against zero."""
    r = np.random.default_rng(30000 + c["i"])
    B, H, S = c["B"], c["H"], c["S"]
    nk = max(2, S // 8)
    if c["form"] == "keys":
        m = np.stack([_runs(r, S, 4, 400, nk) for _ in range(B)])[:, None, None, :]
    elif c["form"] == "keys_per_head":
        m = np.stack([np.stack([_runs(r, S, 4, 400, nk) for _ in range(H)]) for _ in range(B)])[:, :, None, :]
    else:
        m = np.stack([_runs(r, S, 3, 300)[:, None] & _runs(r, S, 4, 400, nk)[None, :] for _ in range(B)])[:, None]
    return torch.from_numpy(np.ascontiguousarray(m))


@pytest.mark.parametrize("case", RUN_CASES, ids=lambda c: f"r{c['i']}_b{c['B']}h{c['H']}kv{c['Hkv']}s{c['S']}"
                         f"d{c['D']}_{c['dtype']}_{c['form']}{'_g' if c['grad'] else ''}")
def test_random_bool_runs(case):
    c = case
    mask = _run_mask(c)
    w = syn.random_small(c["B"], c["H"], c["S"], c["D"], c["dtype"], seed=3900 + c["i"], with_grad=c["grad"],
                         kv_heads=c["Hkv"] if c["Hkv"] < c["H"] else None)
    d = dev()
    q, k, v = (t.to(d) for t in (w.q, w.k, w.v))
    okw = dict(mask=mask, mask_kind="bool", scale=c["scale"], workers=8)
    O_ref, L_ref = rope_sdpa_forward(w.q, w.k, w.v, w.cos, w.sin, **okw)
    if c["grad"]:
        q, k, v = (t.detach().requires_grad_() for t in (q, k, v))
        o = rfa.rope_scaled_dot_product_attention(q, k, v, w.cos.to(d), w.sin.to(d), attn_mask=mask.to(d),
                                                  scale=c["scale"])
        o.backward(w.do.to(d))
        torch.cuda.synchronize()
        check_out("O", to64(o), O_ref, c["dtype"])
        grads = rope_sdpa_backward(w.q, w.k, w.v, w.cos, w.sin, w.do, **okw)
        for name, g, ref in zip(("dQ", "dK", "dV"), (q.grad, k.grad, v.grad), grads):
            check_grad(name, to64(g), ref, c["dtype"])
    else:
        with torch.no_grad():
            o, lse = rfa.rope_sdpa_fwd_with_lse(q, k, v, w.cos.to(d), w.sin.to(d), attn_mask=mask.to(d),
                                                scale=c["scale"])
        torch.cuda.synchronize()
        check_out("O", to64(o), O_ref, c["dtype"])
        check_lse(to64(lse), L_ref, c["dtype"])
