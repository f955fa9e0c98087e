"""Pins behind the tolerance readings of the GPU parity tests (CPU only).

Gradients.  The parity bound for bf16 gradients is 5e-2 relative to the gradient RMS.
Read as max|error| / RMS(gradient), it cannot be met by ANY implementation that returns
bf16 gradients on the causal training shape: rounding the exact float64 gradient itself
to bf16 already exceeds it, because a few gradient entries (e.g. dV of the first keys,
which every causal query attends) are tens of RMS in size.  On the FLUX training shape
the rounded exact gradient fits, but a backward on bf16 matrix products (which must round
Q', K', P and dS to bf16) does not.  The tests therefore check RMS(error) / RMS(gradient)
<= 5e-2, plus max|error| <= 4 max(5e-2, floor) RMS(gradient) against localized faults
(floor = the bf16 rounding error of the exact gradient; an otherwise exact bf16-product
backward reaches ~2.5x the larger of the two, the kernel's own arithmetic 3.1x on one row
of the FLUX GQA workload, and a localized fault, e.g. a wrong tile, gives errors of the
order of the gradient itself, tens of times more).

Outputs.  With Q, K ~ N(0, 4^2) the bf16 rounding of the rotated Q' and K' alone moves O
past the stated 2e-2 of max|O|; see test_large_logit_output_bound.
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


def _bf16(x):
    return torch.from_numpy(np.ascontiguousarray(x)).to(torch.float32).to(torch.bfloat16).double().numpy()


def test_large_logit_output_bound():
    """Q, K ~ N(0, 4^2) (the large-logit GPU case): a bf16 matrix-core kernel must round the
    rotated Q' (times scale log2 e) and K' to bf16 before QK^T.  That rounding alone, with
    everything else exact, moves O by more than the stated 2e-2 of max|O| (so the stated
    bound cannot hold there for any such kernel), but by less than 4e-2: the GPU test bounds
    O by twice that, 8e-2.  LSE moves by far less, and keeps the stated 2e-2."""
    import math

    from oracle import attention_forward, rope_rotate, rope_sdpa_forward

    w = syn.random_small(1, 2, 200, 128, "bf16", seed=26, std=4.0)
    O_ref, L_ref = rope_sdpa_forward(w.q, w.k, w.v, w.cos, w.sin)
    scale = 1.0 / math.sqrt(128)
    c2 = scale * math.log2(math.e)
    qr = rope_rotate(w.q, w.cos, w.sin)
    kr = rope_rotate(w.k, w.cos, w.sin)
    O_p, L_p = attention_forward(_bf16(qr * c2) / c2, _bf16(kr), w.v.double().numpy(), scale)
    e_o = np.abs(O_p - O_ref).max() / np.abs(O_ref).max()
    e_l = np.abs(L_p - L_ref).max() / np.abs(L_ref).max()
    assert 2e-2 < e_o < 4e-2, e_o
    assert e_l < 2e-2 / 4, e_l


def _ideal_bf16_backward_ratios(w, b, h, causal):
    """Gradient errors of a backward on bf16 matrix products that is otherwise exact: float64
    arithmetic with only the roundings such products force (Q' and K' rounded to bf16 as the
    forward rounds them, P rounded for dV = P^T dO, dS rounded for dQ' = dS K' and
    dK' = dS^T Q', outputs rounded to bf16).  Per tensor: (max|err| / RMS, RMS(err) / RMS,
    floor = max|bf16(grad) - grad| / RMS)."""
    import math

    from oracle import attention_forward, rope_rotate, rope_rotate_vjp, rope_sdpa_backward

    q, k, v, do = (t[b:b + 1, h:h + 1].double().numpy() for t in (w.q, w.k, w.v, w.do))
    cos = w.cos[b:b + 1] if w.cos.shape[0] > 1 else w.cos
    sin = w.sin[b:b + 1] if w.sin.shape[0] > 1 else w.sin
    dq_ref, dk_ref, dv_ref = rope_sdpa_backward(q, k, v, cos, sin, do, causal=causal)
    S, D = q.shape[2], q.shape[3]
    scale = 1.0 / math.sqrt(D)
    qr, kr = rope_rotate(q, cos, sin)[0, 0], rope_rotate(k, cos, sin)[0, 0]
    _, lse = attention_forward(qr[None, None], kr[None, None], v, scale, causal=causal)
    qb, kb = _bf16(qr), _bf16(kr)
    s = scale * (qb @ kb.T)
    if causal:
        s = np.where(np.arange(S)[None, :] > np.arange(S)[:, None], -np.inf, s)
    P = np.exp(s - lse[0, 0][:, None])
    V, dO = v[0, 0], do[0, 0]
    dP = dO @ V.T
    delta = (P * dP).sum(axis=1)
    dS = _bf16(P * (dP - delta[:, None]))
    dq = _bf16(rope_rotate_vjp((scale * (dS @ kb))[None, None], cos, sin)[0, 0])
    dk = _bf16(rope_rotate_vjp((scale * (dS.T @ qb))[None, None], cos, sin)[0, 0])
    dv = _bf16(_bf16(P).T @ dO)
    out = {}
    for name, g, r in (("dQ", dq, dq_ref[0, 0]), ("dK", dk, dk_ref[0, 0]), ("dV", dv, dv_ref[0, 0])):
        rms = np.sqrt((r ** 2).mean())
        out[name] = (np.abs(g - r).max() / rms, np.sqrt(((g - r) ** 2).mean()) / rms,
                     np.abs(_bf16(r) - r).max() / rms)
    return out


def test_bf16_matrix_operands_exceed_max_reading_on_flux_training_shape():
    """On the non-causal FLUX training shape (B=2, H=24, S=4608, D=128) the exact gradient
    rounded to bf16 stays within max|error| <= 5e-2 RMS(gradient), but a backward built on
    bf16 matrix products cannot: with only the roundings such products force, head
    (b, h) = (1, 5) exceeds the max reading on dK, while its RMS error stays near 4e-3."""
    w = syn.flux(batch=2, heads=24, grid=64, dtype="bf16", seed=4100, with_grad=True)
    ratios = _ideal_bf16_backward_ratios(w, 1, 5, causal=False)
    assert all(floor < 5e-2 for _, _, floor in ratios.values()), ratios
    assert max(m for m, _, _ in ratios.values()) > 5e-2, ratios
    assert all(e < 1e-2 for _, e, _ in ratios.values()), ratios
    assert all(m <= 3 * max(5e-2, floor) for m, _, floor in ratios.values()), ratios


def test_max_error_guard_admits_an_ideal_bf16_backward():
    """On a small causal case (B=2, H=2, S=300, D=128, the GPU test's seed) an otherwise exact
    backward on bf16 matrix products already reaches more than twice the floor and 1.8x the
    stated bound, so a guard of twice the larger would reject the ideal kernel."""
    w = syn.random_small(2, 2, 300, 128, "bf16", seed=5 + 300 + 128, causal=True, with_grad=True)
    worst = 0.0
    for b in range(2):
        for h in range(2):
            for m, e, floor in _ideal_bf16_backward_ratios(w, b, h, causal=True).values():
                worst = max(worst, m / max(5e-2, floor))
                assert m <= 3 * max(5e-2, floor) and e < 1e-2
    assert worst > 1.5, worst


def test_kernel_arithmetic_reaches_three_times_the_bound_on_gqa_flux_row():
    """The GPU backward folds scale log2(e) into Q' before rounding it to bf16 (one multiply per
    element instead of one per score) and normalizes P with the forward's LSE, itself summed
    from bf16-rounded P.  That arithmetic, emulated in float64 for one row of the FLUX GQA
    workload (B=2, H=24 over Hkv=6, S=4608, per-sample tables; query head 21 of item 0, query
    3357), puts dQ off by 0.156 RMS(dQ): 3.1x max(5e-2, floor), where rounding Q' before the
    scaling gives a quarter of that on this row.  So a max-error guard of 3x would reject the
    kernel's own arithmetic; the GPU tests use 4x.  (The GPU's worst dQ element on that
    workload is this one, with this error.)"""
    import math

    from oracle import expand_kv, rope_rotate, rope_rotate_vjp, rope_sdpa_backward

    w = syn.flux(batch=2, heads=24, grid=64, dtype="bf16", seed=740, with_grad=True, kv_heads=6,
                 per_sample_tables=True)
    dq_all = rope_sdpa_backward(w.q, w.k, w.v, w.cos, w.sin, w.do, workers=8)[0]
    rms = np.sqrt((dq_all ** 2).mean())
    floor = np.abs(_bf16(dq_all) - dq_all).max() / rms
    b, h, i = 0, 21, 3357
    hk = h // 4
    scale = 1.0 / math.sqrt(128)
    l2e = math.log2(math.e)
    c, s = w.cos[b:b + 1], w.sin[b:b + 1]
    qr = rope_rotate(w.q[b:b + 1, h:h + 1], c, s)[0, 0, i]
    kr = rope_rotate(w.k[b:b + 1, hk:hk + 1], c, s)[0, 0]
    V, dO = w.v[b, hk].double().numpy(), w.do[b, h, i].double().numpy()

    def row_err(prescale):
        qb = _bf16(qr * scale * l2e) if prescale else _bf16(qr) * scale * l2e
        kb = _bf16(kr)
        s2 = kb @ qb  # log2 units
        mx = s2.max()
        pf = _bf16(np.exp2(s2 - mx))  # the forward's rounded P, its row sum and output
        lse2 = mx + np.log2(pf.sum())
        O = _bf16((pf @ V) / pf.sum())
        P = np.exp2(s2 - lse2)
        dP = V @ dO
        dS = _bf16(P * (dP - dO @ O))
        dq = _bf16(rope_rotate_vjp((scale * (dS @ kb))[None, None, None], c[:, i:i + 1], s[:, i:i + 1])[0, 0, 0])
        return np.abs(dq - dq_all[b, h, i]).max() / rms

    bound = max(5e-2, floor)
    e_kernel, e_unscaled = row_err(True), row_err(False)
    assert 3 * bound < e_kernel < 4 * bound, (e_kernel, bound)
    assert e_unscaled < e_kernel / 2, (e_unscaled, e_kernel)
