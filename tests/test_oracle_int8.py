"""Pins for the oracle's blockwise int8 variant (CPU only).

The page "Metal Flash Attention" (SimpleTuner docs), sections "Requirements" and
"Enable In SimpleTuner", names an int8 mode with blockwise quantization; the reading
taken (rotated Q and K quantized symmetrically per 64-token block, V unquantized) is
checked here through properties any such quantizer must satisfy, a brute-force
nearest-code search, and the exactness of integer dot products.
"""
import numpy as np
import torch

import synthetic as syn
from oracle import (attention_forward, quantize_blockwise_int8, rope_rotate_f32,
                    rope_sdpa_forward, rope_sdpa_forward_int8)
from oracle.rope_sdpa_ref import dequantize_blockwise


def test_codes_range_max_and_roundtrip():
    rs = np.random.default_rng(90)
    x = (rs.standard_normal((2, 3, 150, 32)) * rs.uniform(0.1, 10, (2, 3, 1, 1))).astype(np.float32)
    x[1, 2, 64:128] = 0.0  # an all-zero block
    codes, scales = quantize_blockwise_int8(x)
    assert codes.dtype == np.int8 and scales.shape == (2, 3, 3)
    assert codes.min() >= -127 and codes.max() <= 127
    for b in range(2):
        for h in range(3):
            for t in range(3):
                blk = codes[b, h, 64 * t:64 * (t + 1)]
                if b == 1 and h == 2 and t == 1:
                    assert scales[b, h, t] == 0 and np.all(blk == 0)
                else:
                    assert np.abs(blk).max() == 127
    xh = dequantize_blockwise(codes, scales)
    err = np.abs(xh - x.astype(np.float64))
    bound = np.repeat(scales.astype(np.float64), 64, axis=2)[:, :, :150, None] * (0.5 + 1e-5)
    assert np.all(err <= bound)


def test_brute_force_nearest_code_with_ties_to_even():
    rs = np.random.default_rng(91)
    x = rs.standard_normal((1, 1, 64, 8)).astype(np.float32)
    x[0, 0, 0, 0] = 4.0  # amax -> scale = 4/127
    sc = np.float32(4.0) / np.float32(127.0)
    inv = np.float32(127.0) / np.float32(4.0)
    x[0, 0, 1, 1] = np.float32(2.5) / inv  # lands (near) a tie
    x[0, 0, 2, 2] = np.float32(0.5) * np.float32(4.0) / np.float32(127.0)
    codes, scales = quantize_blockwise_int8(x)
    assert scales[0, 0, 0] == sc
    cands = np.arange(-127, 128)
    for idx in np.ndindex(x.shape):
        t = np.float32(x[idx]) * inv  # the fp32 product the quantizer decides on
        d = np.abs(cands - np.float64(t))
        best = cands[d == d.min()]
        want = best[0] if len(best) == 1 else best[best % 2 == 0][0]
        assert codes[idx] == want, (idx, t)


def test_integer_scores_are_exact():
    rs = np.random.default_rng(92)
    x = rs.standard_normal((1, 1, 128, 128)).astype(np.float32)
    y = rs.standard_normal((1, 1, 128, 128)).astype(np.float32)
    qc, qs = quantize_blockwise_int8(x)
    kc, ks = quantize_blockwise_int8(y)
    acc = qc[0, 0].astype(np.int64) @ kc[0, 0].astype(np.int64).T
    assert np.abs(acc).max() <= 128 * 127 * 127 < 2 ** 31
    qh = dequantize_blockwise(qc, qs)[0, 0]
    kh = dequantize_blockwise(kc, ks)[0, 0]
    sq = np.repeat(qs[0, 0].astype(np.float64), 64)[:, None]
    sk = np.repeat(ks[0, 0].astype(np.float64), 64)[None, :]
    np.testing.assert_allclose(qh @ kh.T, sq * sk * acc, rtol=1e-13, atol=1e-13)


def test_int8_forward_is_definition_on_dequantized_values_and_close_to_exact():
    w = syn.random_small(1, 2, 192, 64, "bf16", seed=93)
    O8, L8 = rope_sdpa_forward_int8(w.q, w.k, w.v, w.cos, w.sin)
    qc, qs = quantize_blockwise_int8(rope_rotate_f32(w.q, w.cos, w.sin))
    kc, ks = quantize_blockwise_int8(rope_rotate_f32(w.k, w.cos, w.sin))
    O, L = attention_forward(dequantize_blockwise(qc, qs), dequantize_blockwise(kc, ks),
                             w.v.double().numpy(), 1 / 8.0)
    np.testing.assert_array_equal(O8, O)
    # and the quantized attention stays near the unquantized one
    Oref, _ = rope_sdpa_forward(w.q, w.k, w.v, w.cos, w.sin)
    assert np.abs(O8 - Oref).max() < 0.05 * np.abs(Oref).max()
    # supplying the codes explicitly gives the same result
    O8b, _ = rope_sdpa_forward_int8(w.q, w.k, w.v, w.cos, w.sin, codes=((qc, qs), (kc, ks)))
    np.testing.assert_array_equal(O8b, O8)


def test_partial_final_block_uses_valid_rows_only():
    rs = np.random.default_rng(94)
    x = rs.standard_normal((1, 1, 70, 16)).astype(np.float32)
    codes, scales = quantize_blockwise_int8(x)
    assert scales.shape == (1, 1, 2)
    assert scales[0, 0, 1] == np.float32(np.abs(x[0, 0, 64:]).max()) / np.float32(127)
    assert torch.from_numpy(codes).abs().max() == 127
