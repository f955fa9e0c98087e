"""Why the bf16 gradient tolerance is read as an RMS ratio (CPU only).

The parity bound for bf16 gradients is 5e-2 relative to the gradient RMS.  Read as
max|error| / RMS(gradient), it cannot be met by ANY implementation that returns bf16
gradients on the causal training shape: rounding the exact float64 gradient itself to
bf16 already exceeds it, because a few gradient entries (e.g. dV of the first keys, which
every causal query attends) are tens of RMS in size.  The tests therefore check
RMS(error) / RMS(gradient) <= 5e-2, plus a max|error| <= 0.5 RMS guard against localized
faults; this file pins the fact behind that choice.
"""
import numpy as np
import torch

import synthetic as syn
from oracle import rope_sdpa_backward


def test_exact_gradient_rounded_to_bf16_fails_max_reading_but_not_rms_reading():
    w = syn.causal_1axis(batch=1, heads=1, seq=2048, dim=128, dtype="bf16", seed=4200)
    grads = rope_sdpa_backward(w.q, w.k, w.v, w.cos, w.sin, w.do, causal=True)
    max_ratio, rms_ratio = [], []
    for g in grads:
        gb = torch.from_numpy(g).to(torch.bfloat16).double().numpy()
        rms = np.sqrt((g ** 2).mean())
        max_ratio.append(np.abs(gb - g).max() / rms)
        rms_ratio.append(np.sqrt(((gb - g) ** 2).mean()) / rms)
    assert max(max_ratio) > 5e-2          # the max reading is infeasible for bf16 outputs
    assert max(rms_ratio) < 5e-3          # output rounding alone uses < 1/10 of the RMS budget
