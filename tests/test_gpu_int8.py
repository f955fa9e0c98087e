"""GPU parity of the blockwise int8 forward (RS_FLAG_QUANT_INT8_QK) against the CPU oracle.

Two separate checks, as the oracle's int8 reading prescribes:
  * the integer decisions: the GPU's int8 codes and fp32 scales (test-only export
    rope_sdpa_debug_quantize_qk) must equal, bit for bit, the oracle's quantizer applied to
    the oracle's fp32 rotation of the same inputs (both decide in fp32 with the same
    roundings, so no code may differ);
  * the attention on those values: the GPU output must match the float64 oracle run from the
    GPU's own codes and scales, within the bf16/fp16 output tolerance.
"""
import numpy as np
import pytest
import torch

import synthetic as syn
import rope_flash_attention_amd as rfa
from oracle import quantize_blockwise_int8, rope_rotate_f32, rope_sdpa_forward_int8
from parity_util import check_lse, check_out, dev, to64

pytestmark = pytest.mark.gpu


def _gpu_codes(q, k, cos, sin):
    d = dev()
    qc, qs, kc, ks = rfa.debug_quantize_qk(q.to(d) if not q.is_cuda else q, k.to(d) if not k.is_cuda else k,
                                           cos.to(d), sin.to(d))
    torch.cuda.synchronize()
    return qc.cpu().numpy(), qs.cpu().numpy(), kc.cpu().numpy(), ks.cpu().numpy()


def _check_codes(w, got):
    qc, qs, kc, ks = got
    eqc, eqs = quantize_blockwise_int8(rope_rotate_f32(w.q, w.cos, w.sin))
    ekc, eks = quantize_blockwise_int8(rope_rotate_f32(w.k, w.cos, w.sin))
    for name, g, e in (("q codes", qc, eqc), ("k codes", kc, ekc)):
        nd = int((g != e).sum())
        assert nd == 0, f"{name}: {nd} of {e.size} codes differ"
    for name, g, e in (("q scales", qs, eqs), ("k scales", ks, eks)):
        assert np.array_equal(g.view(np.uint32), e.view(np.uint32)), f"{name} differ"
    # properties of the reading: |code| <= 127, and 127 is reached in every nonzero block
    for c, sc in ((qc, qs), (kc, ks)):
        assert np.abs(c.astype(np.int32)).max() <= 127
        B, H, S, D = c.shape
        for t in range(sc.shape[2]):
            blk = np.abs(c[:, :, t * 64:(t + 1) * 64].astype(np.int32)).reshape(B, H, -1).max(axis=2)
            assert np.all((blk == 127) | (sc[:, :, t] == 0))


def _run_int8(w, need_lse=True, q=None, k=None, v=None, mode="int8"):
    d = dev()
    q = w.q.to(d) if q is None else q
    k = w.k.to(d) if k is None else k
    v = w.v.to(d) if v is None else v
    with torch.no_grad():
        if need_lse:
            o, lse = rfa.rope_sdpa_fwd_with_lse(q, k, v, w.cos.to(d), w.sin.to(d), scale=w.scale,
                                                quantization=mode)
        else:
            o = rfa.rope_scaled_dot_product_attention(q, k, v, w.cos.to(d), w.sin.to(d), scale=w.scale,
                                                      quantization=mode)
            lse = None
    torch.cuda.synchronize()
    return o, lse


@pytest.mark.parametrize("case", ["small_d64", "small_d128", "split", "gqa", "f16_per_sample"])
def test_prepass_mode_is_bitwise_the_in_kernel_mode(case):
    """The pre-quantized mode (a quantizer pass writes the codes, the attention kernel streams
    them) and the default mode (the attention kernel quantizes in registers) take the same
    integer decisions and run the same attention arithmetic: O and LSE are equal bit for bit."""
    if case == "small_d64":
        w = syn.random_small(2, 3, 77, 64, "bf16", seed=140)
    elif case == "small_d128":
        w = syn.random_small(2, 3, 300, 128, "bf16", seed=141)
    elif case == "split":  # S = 1104: units cut over the last round
        w = syn.random_small(1, 3, 1104, 128, "bf16", seed=142)
    elif case == "gqa":
        w = syn.random_small(2, 6, 200, 128, "bf16", seed=143, kv_heads=2)
    else:
        w = syn.random_small(2, 2, 130, 128, "f16", seed=144, per_sample_tables=True)
    o1, l1 = _run_int8(w, mode="int8")
    o2, l2 = _run_int8(w, mode="int8_prepass")
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("S", [1, 77, 300])
def test_int8_small(dtype, D, S):
    w = syn.random_small(2, 3, S, D, dtype=dtype, seed=40 + S + D, per_sample_tables=(S == 77))
    codes = _gpu_codes(w.q, w.k, w.cos, w.sin)
    _check_codes(w, codes)
    o, lse = _run_int8(w)
    qc, qs, kc, ks = codes
    O_ref, L_ref = rope_sdpa_forward_int8(w.q, w.k, w.v, w.cos, w.sin, scale=w.scale,
                                          codes=((qc, qs), (kc, ks)), workers=8)
    check_out("O", to64(o), O_ref, dtype)
    check_lse(to64(lse), L_ref, dtype)
    # the oracle quantizing on its own reaches the same values (the codes are equal)
    O_ind, _ = rope_sdpa_forward_int8(w.q, w.k, w.v, w.cos, w.sin, scale=w.scale, workers=8)
    assert np.array_equal(O_ind, O_ref)


def test_int8_strided_views_and_no_lse():
    """BSHD projections viewed as BHSD; the no-LSE entry gives the same output."""
    w = syn.random_small(2, 4, 200, 128, dtype="bf16", seed=91)
    d = dev()
    views = [t.transpose(1, 2).contiguous().to(d).transpose(1, 2) for t in (w.q, w.k, w.v)]
    o1, lse = _run_int8(w, q=views[0], k=views[1], v=views[2])
    o2, _ = _run_int8(w, need_lse=False, q=views[0], k=views[1], v=views[2])
    assert torch.equal(o1, o2)
    codes = _gpu_codes(views[0], views[1], w.cos, w.sin)
    _check_codes(w, codes)
    qc, qs, kc, ks = codes
    O_ref, L_ref = rope_sdpa_forward_int8(w.q, w.k, w.v, w.cos, w.sin, codes=((qc, qs), (kc, ks)), workers=8)
    check_out("O", to64(o1), O_ref, "bf16")
    check_lse(to64(lse), L_ref, "bf16")


def test_int8_zero_block_and_explicit_scale():
    """An all-zero 64-token block of K gets scale 0 and codes 0; its keys score 0."""
    w = syn.random_small(1, 2, 192, 128, dtype="bf16", seed=92)
    w.k[:, :, 64:128] = 0
    w.scale = 0.05
    codes = _gpu_codes(w.q, w.k, w.cos, w.sin)
    _check_codes(w, codes)
    assert np.all(codes[3][:, :, 1] == 0) and np.all(codes[2][:, :, 64:128] == 0)
    o, lse = _run_int8(w)
    qc, qs, kc, ks = codes
    O_ref, L_ref = rope_sdpa_forward_int8(w.q, w.k, w.v, w.cos, w.sin, scale=0.05,
                                          codes=((qc, qs), (kc, ks)), workers=8)
    check_out("O", to64(o), O_ref, "bf16")
    check_lse(to64(lse), L_ref, "bf16")


def test_int8_determinism_and_counter():
    w = syn.random_small(1, 2, 130, 64, dtype="f16", seed=93)
    rfa.rope_sdpa_reset_stats()
    o1, _ = _run_int8(w, need_lse=False)
    o2, _ = _run_int8(w, need_lse=False)
    o3, _ = _run_int8(w, need_lse=False, mode="int8_prepass")
    assert torch.equal(o1, o2) and torch.equal(o1, o3)
    assert rfa.rope_sdpa_get_stats()["quant_int8"] == 3


def test_int8_rejections():
    """fp32 inputs have no quantized path, and the quantized path takes no Q/K RMSNorm
    prologue (forward or with gradients)."""
    w = syn.random_small(1, 2, 64, 64, dtype="bf16", seed=94)
    d = dev()
    q, k, v = (t.to(d) for t in (w.q, w.k, w.v))
    nw = torch.ones(64, device=d, dtype=torch.float32)
    with torch.no_grad(), pytest.raises(rfa.RopeSdpaError):
        rfa.rope_scaled_dot_product_attention(q, k, v, w.cos.to(d), w.sin.to(d), quantization="int8",
                                              q_norm_weight=nw, k_norm_weight=nw)
    qg = q.clone().requires_grad_(True)
    with pytest.raises(rfa.RopeSdpaError):
        rfa.rope_scaled_dot_product_attention(qg, k, v, w.cos.to(d), w.sin.to(d), quantization="int8",
                                              q_norm_weight=nw, k_norm_weight=nw)
    w32 = syn.random_small(1, 2, 64, 64, dtype="f32", seed=94)
    with pytest.raises(rfa.RopeSdpaError):
        rfa.rope_scaled_dot_product_attention(*(t.to(d) for t in (w32.q, w32.k, w32.v)), w32.cos.to(d),
                                              w32.sin.to(d), quantization="int8")


def _full_heads(w, heads):
    """Codes and scales of the named heads bit-exact against the oracle's quantizer; every row
    of O and LSE of those heads against the oracle run from the GPU's own codes."""
    d = dev()
    q, k, v = (t.to(d) for t in (w.q, w.k, w.v))
    o, lse = _run_int8(w, q=q, k=k, v=v)
    qc, qs, kc, ks = _gpu_codes(q, k, w.cos, w.sin)
    del q, k, v
    hs = list(heads)
    sub = syn.Workload("sub", w.q[:, hs], w.k[:, hs], w.v[:, hs], w.cos, w.sin)
    codes = (qc[:, hs], qs[:, hs], kc[:, hs], ks[:, hs])
    _check_codes(sub, codes)
    O_ref, L_ref = rope_sdpa_forward_int8(sub.q, sub.k, sub.v, sub.cos, sub.sin,
                                          codes=((codes[0], codes[1]), (codes[2], codes[3])), workers=8)
    got = np.stack([to64(o[0, h]) for h in hs])
    gl = np.stack([to64(lse[0, h]) for h in hs])
    check_out("O", got, O_ref.reshape(got.shape), "bf16")
    check_lse(gl, L_ref.reshape(gl.shape), "bf16")


def test_int8_flux_two_full_heads():
    """FLUX joint attention B=1, H=24, S=4608, D=128, 3-axis RoPE: heads 0 and 23 whole."""
    w = syn.flux(batch=1, heads=24, grid=64, dtype="bf16", seed=2000)
    _full_heads(w, (0, 23))


def test_int8_long_two_full_heads():
    """Long FLUX sequence B=1, H=48, S=16896 (512 text + 128x128 image), D=128: heads 0 and 47
    whole."""
    w = syn.flux(batch=1, heads=48, grid=128, dtype="bf16", seed=5000)
    _full_heads(w, (0, 47))


def test_int8_prepass_long_is_bitwise_the_in_kernel_mode():
    """The long shape in both int8 modes: every output and LSE element equal."""
    w = syn.flux(batch=1, heads=48, grid=128, dtype="bf16", seed=5000)
    o1, l1 = _run_int8(w, mode="int8")
    o2, l2 = _run_int8(w, mode="int8_prepass")
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_int8_split_key_ranges():
    """int8 forward on a shape whose units' key ranges are split and merged (S = 1104)."""
    w = syn.random_small(1, 3, 1104, 128, dtype="bf16", seed=131)
    codes = _gpu_codes(w.q, w.k, w.cos, w.sin)
    o, lse = _run_int8(w)
    qc, qs, kc, ks = codes
    O_ref, L_ref = rope_sdpa_forward_int8(w.q, w.k, w.v, w.cos, w.sin, scale=w.scale,
                                          codes=((qc, qs), (kc, ks)), workers=8)
    check_out("O", to64(o), O_ref, "bf16")
    check_lse(to64(lse), L_ref, "bf16")
