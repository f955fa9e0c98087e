"""Pins for the oracle's int4 quantizer and for the straight-through backward of the
quantized variants (CPU only).

Page "Metal Flash Attention" (SimpleTuner docs), section "Enable In SimpleTuner": the "-int4"
alias sets QUANT_INT4 with blockwise quantization, and quantized training goes through a
quantized autograd entry point (section "Requirements" names it).  The readings taken (codes
in [-7, 7] per 64-token block; the gradient passes the quantizer unchanged) are checked
through properties any such quantizer must satisfy, a brute-force nearest-code search,
finite differences where the quantized function is smooth (V), and agreement with the
independently pinned unquantized backward on inputs whose rotation lands on the code grid.
"""
import numpy as np
import pytest
import torch

import synthetic as syn
from oracle import (attention_forward, quantize_blockwise_int4, quantize_blockwise_int8,
                    rope_rotate_f32, rope_rotate_vjp, rope_sdpa_backward, rope_sdpa_backward_quant,
                    rope_sdpa_forward, rope_sdpa_forward_quant)
from oracle.rope_sdpa_ref import dequantize_blockwise


def test_int4_codes_range_max_and_roundtrip():
    rs = np.random.default_rng(190)
    x = (rs.standard_normal((2, 3, 150, 32)) * rs.uniform(0.1, 10, (2, 3, 1, 1))).astype(np.float32)
    x[0, 1, 0:64] = 0.0  # an all-zero block
    codes, scales = quantize_blockwise_int4(x)
    assert codes.dtype == np.int8 and scales.shape == (2, 3, 3)
    assert codes.min() >= -7 and codes.max() <= 7
    for b in range(2):
        for h in range(3):
            for t in range(3):
                blk = codes[b, h, 64 * t:64 * (t + 1)]
                if b == 0 and h == 1 and t == 0:
                    assert scales[b, h, t] == 0 and np.all(blk == 0)
                else:
                    assert np.abs(blk).max() == 7
                    amax = np.float32(np.abs(x[b, h, 64 * t:64 * (t + 1)]).max())
                    assert scales[b, h, t] == amax / np.float32(7)
    xh = dequantize_blockwise(codes, scales)
    err = np.abs(xh - x.astype(np.float64))
    bound = np.repeat(scales.astype(np.float64), 64, axis=2)[:, :, :150, None] * (0.5 + 1e-5)
    assert np.all(err <= bound)


def test_int4_brute_force_nearest_code_with_ties_to_even():
    rs = np.random.default_rng(191)
    x = rs.standard_normal((1, 1, 64, 8)).astype(np.float32)
    x[0, 0, 0, 0] = 3.5  # amax -> inv = 2, scale = 0.5 exactly
    x[0, 0, 1, 1] = 1.25   # x * inv = 2.5: a tie, to 2
    x[0, 0, 2, 2] = -1.75  # -3.5: a tie, to -4
    x[0, 0, 3, 3] = 0.25   # 0.5: a tie, to 0
    codes, scales = quantize_blockwise_int4(x)
    assert scales[0, 0, 0] == np.float32(0.5)
    assert codes[0, 0, 1, 1] == 2 and codes[0, 0, 2, 2] == -4 and codes[0, 0, 3, 3] == 0
    inv = np.float32(7.0) / np.float32(3.5)
    cands = np.arange(-7, 8)
    for idx in np.ndindex(x.shape):
        t = np.float32(x[idx]) * inv
        d = np.abs(cands - np.float64(t))
        best = cands[d == d.min()]
        want = best[0] if len(best) == 1 else best[best % 2 == 0][0]
        assert codes[idx] == want, (idx, t)


@pytest.mark.parametrize("bits", [8, 4])
def test_quant_forward_is_definition_on_dequantized_values(bits):
    w = syn.random_small(1, 2, 192, 64, "bf16", seed=193)
    quant = quantize_blockwise_int8 if bits == 8 else quantize_blockwise_int4
    O, L = rope_sdpa_forward_quant(w.q, w.k, w.v, w.cos, w.sin, bits=bits)
    qc, qs = quant(rope_rotate_f32(w.q, w.cos, w.sin))
    kc, ks = quant(rope_rotate_f32(w.k, w.cos, w.sin))
    O2, L2 = attention_forward(dequantize_blockwise(qc, qs), dequantize_blockwise(kc, ks), w.v.double().numpy(),
                               1 / 8.0)
    np.testing.assert_array_equal(O, O2)
    np.testing.assert_array_equal(L, L2)


def test_int4_is_coarser_than_int8():
    w = syn.random_small(1, 2, 256, 64, "bf16", seed=194)
    Oref, _ = rope_sdpa_forward(w.q, w.k, w.v, w.cos, w.sin)
    e8 = np.abs(rope_sdpa_forward_quant(w.q, w.k, w.v, w.cos, w.sin, bits=8)[0] - Oref).max()
    e4 = np.abs(rope_sdpa_forward_quant(w.q, w.k, w.v, w.cos, w.sin, bits=4)[0] - Oref).max()
    assert e8 < e4 < 0.5 * np.abs(Oref).max()


@pytest.mark.parametrize("bits", [8, 4])
def test_quant_backward_dv_matches_finite_differences(bits):
    """V is not quantized: the quantized forward is linear in V, so central differences of
    L = sum(O * dO) give dV exactly (up to rounding)."""
    w = syn.random_small(1, 2, 70, 64, "f32", seed=195, with_grad=True)
    dq, dk, dv = rope_sdpa_backward_quant(w.q, w.k, w.v, w.cos, w.sin, w.do, bits=bits)
    do = w.do.double().numpy()
    v = w.v.double().numpy()
    rs = np.random.default_rng(195)
    for _ in range(6):
        idx = tuple(int(rs.integers(0, n)) for n in v.shape)
        h = 1e-3
        vp, vm = v.copy(), v.copy()
        vp[idx] += h
        vm[idx] -= h
        Lp = (rope_sdpa_forward_quant(w.q, w.k, vp, w.cos, w.sin, bits=bits)[0] * do).sum()
        Lm = (rope_sdpa_forward_quant(w.q, w.k, vm, w.cos, w.sin, bits=bits)[0] * do).sum()
        assert abs((Lp - Lm) / (2 * h) - dv[idx]) <= 1e-8 * max(1.0, abs(dv[idx]))


def _on_grid(shape, bits, seed, cos, sin):
    """fp32 inputs x whose fp32 rotation lands within rounding of codes * 2^-3 (every block
    reaching the full code range), and those codes."""
    qmax = {8: 127, 4: 7}[bits]
    rs = np.random.default_rng(seed)
    codes = rs.integers(-qmax, qmax + 1, size=shape)
    codes[..., ::64, 0] = qmax  # each 64-row block holds +qmax
    target = codes.astype(np.float64) * 2.0 ** -3
    # inverse rotation R^T (the tables are pair-duplicated): R^T = VJP of R
    x = rope_rotate_vjp(target, cos, sin).astype(np.float32)
    return torch.from_numpy(x), codes


@pytest.mark.parametrize("bits", [8, 4])
def test_quant_backward_is_unquantized_backward_on_the_code_grid(bits):
    """Straight-through: where R(Q) and R(K) sit on the code grid, quantization changes
    nothing, and the quantized backward must equal the unquantized one (pinned on its own
    by finite differences), grouped-query reduction included."""
    B, H, Hkv, S, D = 1, 4, 2, 128, 64
    w = syn.random_small(B, H, S, D, "f32", seed=196, with_grad=True, kv_heads=Hkv)
    q, qcodes = _on_grid((B, H, S, D), bits, 197, w.cos, w.sin)
    k, kcodes = _on_grid((B, Hkv, S, D), bits, 198, w.cos, w.sin)
    quant = quantize_blockwise_int8 if bits == 8 else quantize_blockwise_int4
    assert np.array_equal(quant(rope_rotate_f32(q, w.cos, w.sin))[0], qcodes)
    assert np.array_equal(quant(rope_rotate_f32(k, w.cos, w.sin))[0], kcodes)
    got = rope_sdpa_backward_quant(q, k, w.v, w.cos, w.sin, w.do, bits=bits)
    ref = rope_sdpa_backward(q, k, w.v, w.cos, w.sin, w.do)
    for g, r in zip(got, ref):
        np.testing.assert_allclose(g, r, rtol=1e-4, atol=1e-5 * np.abs(r).max())
