"""GPU parity of the blockwise int4 forward (RS_FLAG_QUANT_INT4_QK) against the CPU oracle.

Same two checks as the int8 forward: the GPU's int4 codes (in [-7, 7], one per byte) and
fp32 scales equal the oracle's quantizer bit for bit, and the GPU output matches the float64
oracle run from the GPU's own codes (page "Metal Flash Attention", section "Enable In
SimpleTuner": the "-int4" alias sets QUANT_INT4 with blockwise quantization)."""
import numpy as np
import pytest
import torch

import synthetic as syn
import rope_flash_attention_amd as rfa
from oracle import quantize_blockwise_int4, rope_rotate_f32, rope_sdpa_forward_quant
from parity_util import check_lse, check_out, dev, to64

pytestmark = pytest.mark.gpu


def _gpu_codes(q, k, cos, sin):
    d = dev()
    qc, qs, kc, ks = rfa.debug_quantize_qk(q.to(d), k.to(d), cos.to(d), sin.to(d), bits=4)
    torch.cuda.synchronize()
    return qc.cpu().numpy(), qs.cpu().numpy(), kc.cpu().numpy(), ks.cpu().numpy()


def _check_codes(w, got):
    qc, qs, kc, ks = got
    eqc, eqs = quantize_blockwise_int4(rope_rotate_f32(w.q, w.cos, w.sin))
    ekc, eks = quantize_blockwise_int4(rope_rotate_f32(w.k, w.cos, w.sin))
    for name, g, e in (("q codes", qc, eqc), ("k codes", kc, ekc)):
        nd = int((g != e).sum())
        assert nd == 0, f"{name}: {nd} of {e.size} codes differ"
    for name, g, e in (("q scales", qs, eqs), ("k scales", ks, eks)):
        assert np.array_equal(g.view(np.uint32), e.view(np.uint32)), f"{name} differ"
    for c, sc in ((qc, qs), (kc, ks)):
        assert np.abs(c.astype(np.int32)).max() <= 7
        B, H, S, D = c.shape
        for t in range(sc.shape[2]):
            blk = np.abs(c[:, :, t * 64:(t + 1) * 64].astype(np.int32)).reshape(B, H, -1).max(axis=2)
            assert np.all((blk == 7) | (sc[:, :, t] == 0))


def _run(w, mode="int4", need_lse=True):
    d = dev()
    with torch.no_grad():
        o, lse = rfa.rope_sdpa_fwd_with_lse(w.q.to(d), w.k.to(d), w.v.to(d), w.cos.to(d), w.sin.to(d),
                                            scale=w.scale, quantization=mode)
    torch.cuda.synchronize()
    return o, lse


def _compare(w, dtype):
    codes = _gpu_codes(w.q, w.k, w.cos, w.sin)
    _check_codes(w, codes)
    o, lse = _run(w)
    qc, qs, kc, ks = codes
    O_ref, L_ref = rope_sdpa_forward_quant(w.q, w.k, w.v, w.cos, w.sin, bits=4, scale=w.scale,
                                           codes=((qc, qs), (kc, ks)), workers=8)
    check_out("O", to64(o), O_ref, dtype)
    check_lse(to64(lse), L_ref, dtype)


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("S", [1, 77, 300])
def test_int4_small(dtype, D, S):
    w = syn.random_small(2, 3, S, D, dtype=dtype, seed=240 + S + D, per_sample_tables=(S == 77))
    _compare(w, dtype)


@pytest.mark.parametrize("case", ["small_d64", "split", "gqa"])
def test_int4_prepass_mode_is_bitwise_the_in_kernel_mode(case):
    if case == "small_d64":
        w = syn.random_small(2, 3, 77, 64, "bf16", seed=250)
    elif case == "split":
        w = syn.random_small(1, 3, 1104, 128, "bf16", seed=251)
    else:
        w = syn.random_small(2, 6, 200, 128, "bf16", seed=252, kv_heads=2)
    o1, l1 = _run(w, "int4")
    o2, l2 = _run(w, "int4_prepass")
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_int4_gqa_and_split():
    _compare(syn.random_small(2, 6, 200, 128, "bf16", seed=253, kv_heads=2), "bf16")
    _compare(syn.random_small(1, 3, 1104, 128, "bf16", seed=254), "bf16")


def test_int4_flux_two_full_heads():
    """FLUX B=1, H=24, S=4608, D=128: heads 0 and 23, every row of O and LSE, codes bit-exact."""
    w = syn.flux(batch=1, heads=24, grid=64, dtype="bf16", seed=2000)
    o, lse = _run(w)
    qc, qs, kc, ks = _gpu_codes(w.q, w.k, w.cos, w.sin)
    hs = [0, 23]
    sub = syn.Workload("sub", w.q[:, hs], w.k[:, hs], w.v[:, hs], w.cos, w.sin)
    codes = (qc[:, hs], qs[:, hs], kc[:, hs], ks[:, hs])
    _check_codes(sub, codes)
    O_ref, L_ref = rope_sdpa_forward_quant(sub.q, sub.k, sub.v, sub.cos, sub.sin, bits=4,
                                           codes=((codes[0], codes[1]), (codes[2], codes[3])), workers=8)
    got = np.stack([to64(o[0, h]) for h in hs])
    gl = np.stack([to64(lse[0, h]) for h in hs])
    check_out("O", got, O_ref.reshape(got.shape), "bf16")
    check_lse(gl, L_ref.reshape(gl.shape), "bf16")


def test_int4_rejections():
    w = syn.random_small(1, 2, 64, 64, dtype="f32", seed=255)
    d = dev()
    q, k, v = (t.to(d) for t in (w.q, w.k, w.v))
    with pytest.raises(rfa.RopeSdpaError):
        rfa.rope_scaled_dot_product_attention(q, k, v, w.cos.to(d), w.sin.to(d), quantization="int4")
