"""The allocation-free forward (rope_sdpa_fwd_noalloc) through the C ABI against the forward
with a caller workspace (rope_sdpa_fwd): the same kernels, so O and LSE must agree bit for
bit.  Two calls in a row, the second with a smaller input, so that the second call runs on
scratch that still holds the first call's contents; each case mixes the parts of the
workspace layout that the scratch replaces (packed tables, bool-mask tile states, the
pieces of cut units)."""
import ctypes

import pytest
import torch

import synthetic as syn
import rope_flash_attention_amd as rfa
from rope_flash_attention_amd import _abi
from rope_flash_attention_amd._abi import RS_FLAG_QUANT_INT8_QK, RsArgs, make_tensor

pytestmark = pytest.mark.gpu

_DT = {torch.float32: _abi.RS_F32, torch.float16: _abi.RS_F16, torch.bfloat16: _abi.RS_BF16,
       torch.bool: _abi.RS_BOOL}


def _desc(t):
    return make_tensor(t.data_ptr(), _DT[t.dtype], t.shape, t.stride())


def _run(w, noalloc, int8=False, qk=None, norm=None, k_prepass=False):
    """One forward through the C ABI on device copies of workload w (Q and K replaced by `qk`
    when given; `norm` = (q weights, k weights, eps) for the RMSNorm prologue): returns
    (O, LSE)."""
    d = torch.device("cuda:0")
    q, k, v = (t.to(d) for t in ((w.q, w.k) if qk is None else qk) + (w.v,))
    cos = w.cos.to(d).unsqueeze(1)
    sin = w.sin.to(d).unsqueeze(1)
    mask = None
    if w.mask is not None:  # rows padded to 16 bytes where needed, as the binding does
        mask, _ = rfa._mask4(w.mask.to(d), q.dtype)
    keep = [_desc(x) for x in (q, k, v, cos, sin)]
    tm = _desc(mask) if mask is not None else None
    a = RsArgs()
    a.q, a.k, a.v, a.cos, a.sin = (ctypes.pointer(t) for t in keep)
    a.mask = ctypes.pointer(tm) if tm is not None else None
    a.mask_kind = {"none": _abi.RS_MASK_NONE, "bool": _abi.RS_MASK_BOOL, "additive": _abi.RS_MASK_ADDITIVE}[w.mask_kind]
    a.flags = (RS_FLAG_QUANT_INT8_QK if int8 else 0) | (_abi.RS_FLAG_K_PREPASS if k_prepass else 0)
    a.scale = 0.0
    if norm is not None:
        wq, wk = norm[0].to(d), norm[1].to(d)
        a.q_norm_weight, a.k_norm_weight, a.norm_eps = wq.data_ptr(), wk.data_ptr(), norm[2]
    o = torch.empty(q.shape, dtype=v.dtype, device=d)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=d)
    to = _desc(o)
    lib = _abi.load()
    stream = torch.cuda.current_stream(d).cuda_stream
    if noalloc:
        st = lib.rope_sdpa_fwd_noalloc(ctypes.byref(a), ctypes.byref(to), lse.data_ptr(), stream)
    else:
        n = ctypes.c_size_t(0)
        assert lib.rope_sdpa_workspace_size(ctypes.byref(a), 0, ctypes.byref(n)) == 0
        ws = torch.empty(int(n.value), dtype=torch.uint8, device=d)
        st = lib.rope_sdpa_fwd(ctypes.byref(a), ctypes.byref(to), lse.data_ptr(), ws.data_ptr(), ws.numel(), stream)
    assert st == 0, _abi.status_string(st)
    torch.cuda.synchronize()
    return o, lse


def _case(name):
    if name == "flux":  # 432 units: the last round's units are cut into pieces
        return syn.flux(batch=1, heads=24, grid=64, dtype="bf16", seed=2000)
    if name == "flux_b3":  # K' (81 MiB) would not fit the scratch
        return syn.flux(batch=3, heads=24, grid=64, dtype="bf16", seed=2001)
    if name == "flux_bool":
        w = syn.flux(batch=2, heads=8, grid=64, dtype="bf16", seed=3000)
        w.mask = syn.key_padding_mask(syn.key_padding_lengths(3000, 2), 512, w.q.shape[2])
        w.mask_kind = "bool"
        return w
    if name == "small_split":  # S = 1104: few units, cut
        return syn.random_small(1, 3, 1104, 128, "bf16", seed=130)
    if name == "small_fp32_mask":
        return syn.random_small(2, 2, 300, 64, "f32", seed=131, mask_kind="bool", mask_shape=(2, 2, 300, 300))
    if name == "tiny":
        return syn.random_small(1, 1, 77, 128, "f16", seed=132)
    raise ValueError(name)


@pytest.mark.parametrize("first,second", [("flux", "small_split"), ("flux_bool", "small_fp32_mask"),
                                          ("small_split", "tiny"), ("flux_b3", "flux"),
                                          ("flux_b3_k_prepass", "flux_k_prepass")])
def test_noalloc_matches_workspace_forward_on_two_calls(first, second):
    """(with RS_FLAG_K_PREPASS: the B=3 call cannot hold K' in the scratch and rotates K in the
    key loop instead, the B=1 call prepares K' in the scratch; both equal the workspace call)"""
    for name in (first, second):
        kp = name.endswith("_k_prepass")
        w = _case(name.removesuffix("_k_prepass"))
        o_ref, l_ref = _run(w, noalloc=False, k_prepass=kp)
        o, l = _run(w, noalloc=True, k_prepass=kp)
        assert torch.equal(o, o_ref), name
        assert torch.equal(l, l_ref), name


def test_noalloc_qk_prologue_two_calls():
    """fp32 Q/K with RMSNorm beside bf16 V (K' prepared in the scratch), then a smaller call."""
    for B, H, grid, seed in ((1, 8, 64, 140), (1, 2, 16, 141)):
        w = syn.flux(batch=B, heads=H, grid=grid, dtype="bf16", seed=seed)
        qk = (syn.normal(seed, syn.STREAM_Q, tuple(w.q.shape), "f32", 4.0),
              syn.normal(seed, syn.STREAM_K, tuple(w.k.shape), "f32", 4.0))
        norm = (*syn.norm_weights(seed, 128), 1e-6)
        o_ref, l_ref = _run(w, noalloc=False, qk=qk, norm=norm)
        o, l = _run(w, noalloc=True, qk=qk, norm=norm)
        assert torch.equal(o, o_ref) and torch.equal(l, l_ref)


def test_noalloc_int8_and_rejection():
    w = syn.flux(batch=1, heads=4, grid=64, dtype="bf16", seed=2000)
    o_ref, l_ref = _run(w, noalloc=False, int8=True)
    o, l = _run(w, noalloc=True, int8=True)
    assert torch.equal(o, o_ref) and torch.equal(l, l_ref)
    # per-sample tables of 32 samples at S = 4608 need 75 MB of packed tables: rejected
    d = torch.device("cuda:0")
    B, H, S, D = 32, 1, 4608, 128
    q = torch.zeros(B, H, S, D, dtype=torch.bfloat16, device=d)
    tab = torch.zeros(B, 1, S, D, dtype=torch.float32, device=d)
    keep = [_desc(x) for x in (q, q, q, tab, tab)]
    a = RsArgs()
    a.q, a.k, a.v, a.cos, a.sin = (ctypes.pointer(t) for t in keep)
    a.mask, a.mask_kind, a.flags, a.scale = None, 0, 0, 0.0
    o = torch.full_like(q, 7.0)
    to = _desc(o)
    st = _abi.load().rope_sdpa_fwd_noalloc(ctypes.byref(a), ctypes.byref(to), None,
                                           torch.cuda.current_stream(d).cuda_stream)
    torch.cuda.synchronize()
    assert _abi.STATUS_NAMES[st] == "RS_ERR_SCRATCH"
    assert torch.all(o == 7.0)  # nothing launched
