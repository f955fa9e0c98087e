"""Pins for the oracle's rotation (CPU only).

The rotation follows the page "Metal Flash Attention" (SimpleTuner docs), section
"Fused RoPE + SDPA": interleaved adjacent pairs, pair-duplicated cos/sin tables, the
complex-multiply formulation being the same rotation, and the backward applying the
same pairwise rotation with sin negated.  Each test checks the oracle against an
independent fact: complex arithmetic, exact quarter turns, norm preservation, the
relative-position property, and a numerical Jacobian.
"""
import numpy as np
import pytest
import torch

import synthetic as syn
from oracle import rope_rotate, rope_rotate_vjp, rope_rotate_f32


def _f64_tables(positions, D, theta=10000.0):
    ang = np.repeat(syn.rope_angles(positions, D, theta), 2, axis=1)
    return np.cos(ang), np.sin(ang)


def test_matches_complex_multiply():
    rs = np.random.default_rng(0)
    x = rs.standard_normal((2, 3, 17, 16))
    cos, sin = syn.rope_tables(np.arange(17), (16,), 10000.0)
    out = rope_rotate(x, cos, sin)
    z = x[..., 0::2] + 1j * x[..., 1::2]
    w = cos.double().numpy()[None, None, :, 0::2] + 1j * sin.double().numpy()[None, None, :, 0::2]
    zr = z * w
    np.testing.assert_allclose(out[..., 0::2], zr.real, rtol=0, atol=1e-13)
    np.testing.assert_allclose(out[..., 1::2], zr.imag, rtol=0, atol=1e-13)


def test_quarter_and_half_turns_exact():
    x = np.array([[[[3.0, 5.0, -2.0, 7.0]]]])
    c = np.array([[0.0, 0.0, -1.0, -1.0]])
    s = np.array([[1.0, 1.0, 0.0, 0.0]])
    out = rope_rotate(x, c, s)
    # quarter turn (x0, x1) -> (-x1, x0); half turn -> (-x0, -x1)
    np.testing.assert_array_equal(out[0, 0, 0], [-5.0, 3.0, 2.0, -7.0])


def test_identity_tables_are_identity():
    x = np.random.default_rng(1).standard_normal((1, 2, 5, 8))
    out = rope_rotate(x, np.ones((5, 8)), np.zeros((5, 8)))
    np.testing.assert_array_equal(out, x)


def test_preserves_pair_norms():
    rs = np.random.default_rng(2)
    x = rs.standard_normal((1, 2, 64, 32))
    c, s = _f64_tables(np.arange(64), 32)
    out = rope_rotate(x, c, s)
    n_in = x[..., 0::2] ** 2 + x[..., 1::2] ** 2
    n_out = out[..., 0::2] ** 2 + out[..., 1::2] ** 2
    np.testing.assert_allclose(n_out, n_in, rtol=1e-13)


@pytest.mark.parametrize("shift", [1, 7, 300])
def test_scores_depend_only_on_position_difference(shift):
    rs = np.random.default_rng(3)
    D, S = 16, 20
    q = rs.standard_normal((1, 1, S, D))
    k = rs.standard_normal((1, 1, S, D))
    c0, s0 = _f64_tables(np.arange(S), D)
    c1, s1 = _f64_tables(np.arange(S) + shift, D)
    sc0 = rope_rotate(q, c0, s0)[0, 0] @ rope_rotate(k, c0, s0)[0, 0].T
    sc1 = rope_rotate(q, c1, s1)[0, 0] @ rope_rotate(k, c1, s1)[0, 0].T
    np.testing.assert_allclose(sc1, sc0, rtol=0, atol=1e-11)


def test_three_axis_shift_invariance_per_axis():
    """With 3-axis tables, shifting one axis of every token's id leaves all scores unchanged."""
    rs = np.random.default_rng(4)
    ids = syn.flux_ids(4, 3)
    D = 128
    q = rs.standard_normal((1, 1, len(ids), D))
    k = rs.standard_normal((1, 1, len(ids), D))

    def tables(idv):
        ang = np.concatenate([syn.rope_angles(idv[:, a], d, 10000.0) for a, d in enumerate((16, 56, 56))], 1)
        ang = np.repeat(ang, 2, 1)
        return np.cos(ang), np.sin(ang)

    c0, s0 = tables(ids)
    sc0 = rope_rotate(q, c0, s0)[0, 0] @ rope_rotate(k, c0, s0)[0, 0].T
    for a in range(3):
        shifted = ids.copy()
        shifted[:, a] += 11
        c1, s1 = tables(shifted)
        sc1 = rope_rotate(q, c1, s1)[0, 0] @ rope_rotate(k, c1, s1)[0, 0].T
        np.testing.assert_allclose(sc1, sc0, rtol=0, atol=1e-10)


def test_vjp_matches_numerical_jacobian_general_tables():
    """The VJP is exact for any tables, duplicated or not (the rotation is linear in x)."""
    rs = np.random.default_rng(5)
    D, S = 6, 3
    c = rs.standard_normal((S, D))
    s = rs.standard_normal((S, D))
    x = rs.standard_normal((1, 1, S, D))
    g = rs.standard_normal((1, 1, S, D))
    J = np.zeros((S * D, S * D))
    for idx in range(S * D):
        e = np.zeros(S * D)
        e[idx] = 1.0
        J[:, idx] = rope_rotate(e.reshape(1, 1, S, D), c, s).ravel()
    np.testing.assert_allclose(rope_rotate_vjp(g, c, s).ravel(), J.T @ g.ravel(), rtol=0, atol=1e-13)
    np.testing.assert_allclose(rope_rotate(x, c, s).ravel(), J @ x.ravel(), rtol=0, atol=1e-13)


def test_vjp_is_inverse_rotation_for_duplicated_tables():
    rs = np.random.default_rng(6)
    c, s = _f64_tables(np.arange(33), 64)
    x = rs.standard_normal((2, 2, 33, 64))
    np.testing.assert_allclose(rope_rotate_vjp(rope_rotate(x, c, s), c, s), x, rtol=0, atol=1e-13)
    # "same pairwise rotation with sin negated"
    np.testing.assert_allclose(rope_rotate_vjp(x, c, s), rope_rotate(x, c, -s), rtol=0, atol=0)


def test_per_sample_tables_index_batch():
    rs = np.random.default_rng(7)
    x = rs.standard_normal((2, 1, 4, 8))
    c = rs.standard_normal((2, 4, 8))
    s = rs.standard_normal((2, 4, 8))
    out = rope_rotate(x, c, s)
    for b in range(2):
        np.testing.assert_array_equal(out[b:b + 1], rope_rotate(x[b:b + 1], c[b], s[b]))


def test_synthetic_tables_are_pair_duplicated_and_flux_text_is_identity():
    cos, sin = syn.rope_tables(syn.flux_ids(512, 64), (16, 56, 56), 10000.0)
    assert cos.dtype == torch.float32 and cos.shape == (4608, 128)
    assert torch.equal(cos[:, 0::2], cos[:, 1::2]) and torch.equal(sin[:, 0::2], sin[:, 1::2])
    # text ids are (0,0,0): identity rotation; axis 0 id is 0 for every token: dims 0..15 identity
    assert torch.all(cos[:512] == 1) and torch.all(sin[:512] == 0)
    assert torch.all(cos[:, :16] == 1) and torch.all(sin[:, :16] == 0)


def test_f32_rotation_close_to_f64():
    rs = np.random.default_rng(8)
    x = rs.standard_normal((1, 2, 64, 64)).astype(np.float32)
    cos, sin = syn.rope_tables(np.arange(64), (64,), 10000.0)
    r32 = rope_rotate_f32(x, cos, sin)
    r64 = rope_rotate(x.astype(np.float64), cos, sin)
    assert r32.dtype == np.float32
    np.testing.assert_allclose(r32, r64, rtol=0, atol=4 * np.finfo(np.float32).eps * np.abs(x).max())


def _rot_f32_torch(x, c, s):
    """The fp32 rotation evaluated independently with torch float32 elementwise operations on
    the CPU: two products, each rounded to fp32, then their difference / sum, rounded once."""
    x = torch.as_tensor(np.asarray(x, dtype=np.float32))
    c = torch.as_tensor(np.asarray(c, dtype=np.float32))
    s = torch.as_tensor(np.asarray(s, dtype=np.float32))
    x0, x1 = x[..., 0::2], x[..., 1::2]
    c0, s0 = c[..., 0::2], s[..., 0::2]
    out = torch.empty_like(x)
    p0, p1 = torch.mul(x0, c0), torch.mul(x1, s0)
    out[..., 0::2] = torch.sub(p0, p1)
    p2, p3 = torch.mul(x0, s0), torch.mul(x1, c0)
    out[..., 1::2] = torch.add(p2, p3)
    return out.numpy()


def test_f32_rotation_bitwise_matches_torch_float32_ops():
    """rope_rotate_f32 decides the int8 codes, so its exact rounding is pinned, not only its
    closeness to float64: bit for bit against torch float32 elementwise ops."""
    rs = np.random.default_rng(81)
    x = rs.standard_normal((2, 3, 96, 128)).astype(np.float32) * rs.uniform(0.01, 50, (2, 3, 1, 1)).astype(np.float32)
    cos, sin = syn.rope_tables(syn.flux_ids(32, 8), (16, 56, 56), 10000.0)
    got = rope_rotate_f32(x, cos, sin)[0:2]
    ref = _rot_f32_torch(x, cos.numpy()[None, None], sin.numpy()[None, None])
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))


def test_f32_rotation_rounds_each_product_no_fma():
    """Inputs built so that one rounding of a fused multiply-add and two roundings of
    product-then-difference give different fp32 results:
      x0 = c = 1 + 2^-12: x0 c = 1 + 2^-11 + 2^-24 is a tie in fp32 and rounds to even,
      1 + 2^-11; x1 = 1 + 2^-11, s = 1.  Rounded products: x0 c - x1 s = 0 exactly, while a
      fused form would keep the 2^-24.  The second element: x0 s + x1 c with the same values
      = (1 + 2^-12) + (1 + 2^-11)(1 + 2^-12), product 1 + 2^-11 + 2^-12 + 2^-23 rounded
      to fp32 (exact: it has 24 significant bits), sum 2 + 2^-11 + 2^-11 + 2^-23, rounded
      to fp32 at spacing 2^-22: 2 + 2^-10 + 2^-23 is a tie, to even gives 2 + 2^-10."""
    a = np.float32(1 + 2.0 ** -12)
    b = np.float32(1 + 2.0 ** -11)
    x = np.array([[[[a, b]]]], dtype=np.float32)
    cos = np.array([[a, a]], dtype=np.float32)
    sin = np.array([[1.0, 1.0]], dtype=np.float32)
    got = rope_rotate_f32(x, cos, sin)[0, 0, 0]
    assert got[0] == np.float32(0.0)
    assert got[1] == np.float32(2 + 2.0 ** -10)
    # a fused evaluation differs on the first element
    fused0 = np.float32(float(a) * float(a) - float(b) * 1.0)
    assert fused0 != got[0]
