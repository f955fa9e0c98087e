"""Pins for the oracle's forward attention (CPU only).

Definition: page "Metal Flash Attention" (SimpleTuner docs), section "Fused RoPE + SDPA"
(softmax(scale Q'K'^T + mask) V, scale = 1/sqrt(D) when not given) and section
"Enable In SimpleTuner" (bool True = attend, additive masks, broadcast shapes,
all-true masks equivalent to no mask).  The oracle is checked against a pure-Python
textbook softmax without max subtraction, against torch's float64 SDPA as a library
routine, against hand-derived closed forms, and against mask equivalences.
"""
import json
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import synthetic as syn
from oracle import attention_forward, mask_to_additive, rope_rotate, rope_sdpa_forward

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _naive_attention(q, k, v, scale, allowed=None):
    """Pure-Python loops, no max subtraction: O_i = sum_j e^{s_ij} v_j / sum_j e^{s_ij}."""
    Sq, D = q.shape
    Skv = k.shape[0]
    O = [[0.0] * v.shape[1] for _ in range(Sq)]
    for i in range(Sq):
        w = []
        for j in range(Skv):
            if allowed is not None and not allowed[i][j]:
                w.append(0.0)
                continue
            dot = 0.0
            for d in range(D):
                dot += float(q[i][d]) * float(k[j][d])
            w.append(math.exp(scale * dot))
        z = sum(w)
        for e in range(v.shape[1]):
            O[i][e] = sum(w[j] * float(v[j][e]) for j in range(Skv)) / z
    return np.array(O)


def test_naive_softmax_tiny():
    rs = np.random.default_rng(10)
    B, H, S, D = 1, 2, 6, 4
    q = rs.standard_normal((B, H, S, D)) * 0.5
    k = rs.standard_normal((B, H, S, D)) * 0.5
    v = rs.standard_normal((B, H, S, D))
    c = rs.uniform(-1, 1, (S, D // 2)).repeat(2, axis=1)
    s = np.sqrt(1 - c ** 2)
    O, _ = rope_sdpa_forward(q, k, v, c, s)
    qr, kr = rope_rotate(q, c, s), rope_rotate(k, c, s)
    for h in range(H):
        ref = _naive_attention(qr[0, h], kr[0, h], v[0, h], 1.0 / math.sqrt(D))
        np.testing.assert_allclose(O[0, h], ref, rtol=1e-12, atol=1e-13)


def test_naive_softmax_with_bool_mask_and_causal():
    rs = np.random.default_rng(11)
    S, D = 5, 4
    q = rs.standard_normal((1, 1, S, D)) * 0.5
    k = rs.standard_normal((1, 1, S, D)) * 0.5
    v = rs.standard_normal((1, 1, S, D))
    c, s = np.ones((S, D)), np.zeros((S, D))
    allowed = rs.random((S, S)) < 0.6
    allowed[:, 0] = True
    O, _ = rope_sdpa_forward(q, k, v, c, s, mask=torch.from_numpy(allowed), mask_kind="bool")
    np.testing.assert_allclose(O[0, 0], _naive_attention(q[0, 0], k[0, 0], v[0, 0], 0.5, allowed), rtol=1e-12)
    Oc, _ = rope_sdpa_forward(q, k, v, c, s, causal=True)
    tril = [[j <= i for j in range(S)] for i in range(S)]
    np.testing.assert_allclose(Oc[0, 0], _naive_attention(q[0, 0], k[0, 0], v[0, 0], 0.5, tril), rtol=1e-12)


@pytest.mark.parametrize("case", ["none", "bool4d", "bool_bcast", "additive", "causal", "scale"])
def test_matches_torch_sdpa_float64(case):
    """With the oracle's rotation (pinned separately), attention equals torch's float64 SDPA."""
    rs = np.random.default_rng(12)
    B, H, S, D = 2, 3, 37, 16
    q = rs.standard_normal((B, H, S, D))
    k = rs.standard_normal((B, H, S, D))
    v = rs.standard_normal((B, H, S, D))
    cos, sin = syn.rope_tables(np.arange(S), (D,), 10000.0)
    kw = {}
    tmask = None
    if case == "bool4d":
        m = torch.from_numpy(rs.random((B, H, S, S)) < 0.7)
        m[..., 0] = True
        kw = dict(mask=m, mask_kind="bool")
        tmask = m
    elif case == "bool_bcast":
        m = torch.from_numpy(rs.random((B, 1, 1, S)) < 0.7)
        m[..., 3] = True
        kw = dict(mask=m, mask_kind="bool")
        tmask = m
    elif case == "additive":
        m = torch.from_numpy(rs.standard_normal((1, H, S, S)))
        kw = dict(mask=m, mask_kind="additive")
        tmask = m
    elif case == "causal":
        kw = dict(causal=True)
    elif case == "scale":
        kw = dict(scale=0.3)
    O, _ = rope_sdpa_forward(q, k, v, cos, sin, **kw)
    qr = torch.from_numpy(rope_rotate(q, cos, sin))
    kr = torch.from_numpy(rope_rotate(k, cos, sin))
    ref = F.scaled_dot_product_attention(qr, kr, torch.from_numpy(v), attn_mask=tmask,
                                         is_causal=(case == "causal"),
                                         scale=0.3 if case == "scale" else None)
    np.testing.assert_allclose(O, ref.numpy(), rtol=1e-10, atol=1e-12)


def test_closed_form_zero_query_is_mean_of_valid_values():
    rs = np.random.default_rng(13)
    B, H, S, D = 1, 2, 9, 8
    q = np.zeros((B, H, S, D))
    k = rs.standard_normal((B, H, S, D))
    v = rs.standard_normal((B, H, S, D))
    cos, sin = syn.rope_tables(np.arange(S), (D,), 10000.0)
    valid = np.array([1, 0, 1, 1, 0, 0, 1, 1, 0], dtype=bool)
    m = torch.from_numpy(valid.reshape(1, 1, 1, S))
    O, L = rope_sdpa_forward(q, k, v, cos, sin, mask=m, mask_kind="bool")
    np.testing.assert_allclose(O, np.broadcast_to(v[:, :, valid].mean(axis=2, keepdims=True), O.shape), rtol=1e-13)
    np.testing.assert_allclose(L, np.log(valid.sum()), rtol=1e-14)


def test_closed_form_single_valid_key_and_causal_first_row():
    rs = np.random.default_rng(14)
    S, D = 7, 8
    q, k, v = (rs.standard_normal((1, 1, S, D)) for _ in range(3))
    cos, sin = syn.rope_tables(np.arange(S), (D,), 10000.0)
    m = torch.zeros(1, 1, 1, S, dtype=torch.bool)
    m[..., 4] = True
    O, _ = rope_sdpa_forward(q, k, v, cos, sin, mask=m, mask_kind="bool")
    np.testing.assert_allclose(O[0, 0], np.broadcast_to(v[0, 0, 4], (S, D)), rtol=1e-14)
    Oc, Lc = rope_sdpa_forward(q, k, v, cos, sin, causal=True)
    np.testing.assert_allclose(Oc[0, 0, 0], v[0, 0, 0], rtol=1e-14)
    qr, kr = rope_rotate(q, cos, sin), rope_rotate(k, cos, sin)
    np.testing.assert_allclose(Lc[0, 0, 0], (qr[0, 0, 0] @ kr[0, 0, 0]) / math.sqrt(D), rtol=1e-13)


def test_all_true_mask_equals_no_mask_exactly():
    w = syn.random_small(2, 2, 40, 16, "f32", seed=15)
    O0, L0 = rope_sdpa_forward(w.q, w.k, w.v, w.cos, w.sin)
    for shape in [(2, 2, 40, 40), (2, 1, 1, 40), (40,)]:
        m = torch.ones(shape, dtype=torch.bool)
        O1, L1 = rope_sdpa_forward(w.q, w.k, w.v, w.cos, w.sin, mask=m, mask_kind="bool")
        np.testing.assert_array_equal(O1, O0)
        np.testing.assert_array_equal(L1, L0)


def test_causal_equals_tril_bool_and_bool_equals_additive():
    w = syn.random_small(1, 2, 33, 16, "f32", seed=16)
    Oc, Lc = rope_sdpa_forward(w.q, w.k, w.v, w.cos, w.sin, causal=True)
    tril = torch.tril(torch.ones(33, 33, dtype=torch.bool))
    Ot, Lt = rope_sdpa_forward(w.q, w.k, w.v, w.cos, w.sin, mask=tril, mask_kind="bool")
    np.testing.assert_array_equal(Oc, Ot)
    np.testing.assert_array_equal(Lc, Lt)
    add = torch.where(tril, 0.0, float("-inf"))
    Oa, La = rope_sdpa_forward(w.q, w.k, w.v, w.cos, w.sin, mask=add, mask_kind="additive")
    np.testing.assert_array_equal(Oa, Ot)
    np.testing.assert_array_equal(La, Lt)


def test_fully_masked_rows_give_zero_and_neg_inf_lse():
    w = syn.random_small(1, 1, 8, 8, "f32", seed=17)
    m = torch.ones(1, 1, 8, 8, dtype=torch.bool)
    m[0, 0, 3] = False
    O, L = rope_sdpa_forward(w.q, w.k, w.v, w.cos, w.sin, mask=m, mask_kind="bool")
    assert np.all(O[0, 0, 3] == 0) and L[0, 0, 3] == -np.inf
    assert np.all(np.isfinite(O)) and np.isfinite(np.delete(L[0, 0], 3)).all()


def test_row_and_head_subsets_match_full():
    w = syn.random_small(2, 3, 70, 16, "f32", seed=18, mask_kind="bool", mask_shape=(2, 1, 70, 70))
    O, L = rope_sdpa_forward(w.q, w.k, w.v, w.cos, w.sin, mask=w.mask, mask_kind="bool", causal=False)
    rows = [0, 5, 69, 33]
    pairs = [(1, 2), (0, 0)]
    Os, Ls = rope_sdpa_forward(w.q, w.k, w.v, w.cos, w.sin, mask=w.mask, mask_kind="bool", rows=rows, pairs=pairs)
    for i, (b, h) in enumerate(pairs):
        np.testing.assert_array_equal(Os[i], O[b, h, rows])
        np.testing.assert_array_equal(Ls[i], L[b, h, rows])


def test_thread_pool_matches_serial():
    w = syn.random_small(2, 2, 50, 16, "f32", seed=19)
    a = rope_sdpa_forward(w.q, w.k, w.v, w.cos, w.sin, workers=1)
    b = rope_sdpa_forward(w.q, w.k, w.v, w.cos, w.sin, workers=4)
    np.testing.assert_array_equal(a[0], b[0])


def test_golden_default_scale():
    g = json.load(open(os.path.join(GOLD, "default_scale_d128.json")))
    D = g["D"]
    rs = np.random.default_rng(20)
    q, k, v = (rs.standard_normal((1, 1, 5, D)) for _ in range(3))
    c, s = np.ones((5, D)), np.zeros((5, D))
    O_default, _ = rope_sdpa_forward(q, k, v, c, s)
    O_explicit, _ = rope_sdpa_forward(q, k, v, c, s, scale=g["scale"])
    np.testing.assert_array_equal(O_default, O_explicit)


def _ev(expr):
    return eval(expr, {"__builtins__": {}}, {"e": math.e, "log": math.log})


def test_golden_worked_example_quarter_turn():
    g = json.load(open(os.path.join(GOLD, "worked_example_quarter_turn.json")))
    arr = lambda key: np.array(g[key], dtype=np.float64)[None, None]
    for causal, ko, kl in [(False, "expected_O", "expected_LSE"), (True, "expected_causal_O", "expected_causal_LSE")]:
        O, L = rope_sdpa_forward(arr("q"), arr("k"), arr("v"), np.array(g["cos"]), np.array(g["sin"]),
                                 scale=g["scale"], causal=causal)
        expO = np.array([[_ev(x) for x in row] for row in g[ko]])
        expL = np.array([_ev(x) for x in g[kl]])
        np.testing.assert_allclose(O[0, 0], expO, rtol=1e-14)
        np.testing.assert_allclose(L[0, 0], expL, rtol=1e-14)


def test_mask_to_additive_broadcast_ranks():
    m = mask_to_additive(torch.tensor([True, False, True]), "bool")
    assert m.shape == (1, 1, 1, 3)
    np.testing.assert_array_equal(m[0, 0, 0], [0.0, -np.inf, 0.0])
    out, _ = attention_forward(np.zeros((1, 1, 2, 2)), np.zeros((1, 1, 3, 2)),
                               np.arange(6, dtype=np.float64).reshape(1, 1, 3, 2), 1.0, m)
    np.testing.assert_allclose(out[0, 0], [[2.0, 3.0], [2.0, 3.0]])
