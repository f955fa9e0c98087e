"""Pins for the oracle's Q/K RMSNorm prologue (CPU only).

The diffusers issue "Flux-family attention: flash-attn and other backends fail in an autocast
context" (sections "Describe the bug", "Root cause, in order") describes flux-style attention
normalizing Q and K with RMSNorm (per head, over the head dimension) just before the rotary
embedding, which under autocast leaves Q and K in fp32 while V stays bf16.  The oracle's
rms_norm is checked against torch's own rms_norm in float64, and the normalized forward
against the plain forward run on inputs normalized by torch.
"""
import numpy as np
import torch
import torch.nn.functional as F

import synthetic as syn
from oracle import rms_norm, rope_sdpa_forward


def test_rms_norm_matches_torch():
    rs = np.random.default_rng(60)
    x = rs.standard_normal((2, 3, 17, 128)) * rs.uniform(0.01, 30, (2, 3, 17, 1))
    w = rs.uniform(0.5, 2.0, 128)
    for eps in (1e-6, 1e-2):
        ref = F.rms_norm(torch.from_numpy(x), (128,), torch.from_numpy(w), eps).numpy()
        np.testing.assert_allclose(rms_norm(x, w, eps), ref, rtol=1e-14, atol=1e-14)


def test_rms_norm_invariants():
    """Unit weights give rows of RMS ~1 (exactly sqrt(mean x^2 / (mean x^2 + eps))), and the
    norm is invariant to scaling a row when eps is negligible."""
    rs = np.random.default_rng(61)
    x = rs.standard_normal((4, 64))
    y = rms_norm(x, np.ones(64), 0.0)
    np.testing.assert_allclose(np.sqrt((y ** 2).mean(axis=-1)), 1.0, rtol=1e-14)
    np.testing.assert_allclose(rms_norm(7.5 * x, np.ones(64), 0.0), y, rtol=1e-13)


def test_normalized_forward_equals_forward_on_normalized_inputs():
    w = syn.random_small(1, 2, 50, 64, "f32", seed=62)
    rs = np.random.default_rng(63)
    wq, wk = rs.uniform(0.5, 2, 64), rs.uniform(0.5, 2, 64)
    O1, L1 = rope_sdpa_forward(w.q, w.k, w.v, w.cos, w.sin, q_norm_weight=wq, k_norm_weight=wk, norm_eps=1e-6)
    qn = F.rms_norm(w.q.double(), (64,), torch.from_numpy(wq), 1e-6)
    kn = F.rms_norm(w.k.double(), (64,), torch.from_numpy(wk), 1e-6)
    O2, L2 = rope_sdpa_forward(qn, kn, w.v, w.cos, w.sin)
    np.testing.assert_allclose(O1, O2, rtol=0, atol=1e-13)
    np.testing.assert_allclose(L1, L2, rtol=0, atol=1e-12)
