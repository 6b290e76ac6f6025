"""Pins of the RoPE oracle (CPU only), each against a fact that does not reuse its formula.

RoPE as in Su et al., RoFormer (2021): pair (x_{2i}, x_{2i+1}) of the row at position m is
rotated by m * theta_i, theta_i = base^(-2i/d).
"""
import numpy as np
import pytest
import scipy.linalg

from oracle import rope as R

RNG = np.random.default_rng(7)


def test_frequency_table_closed_values():
    """theta_0 = 1, theta at the middle pair = base^(-1/2), a constant ratio base^(-2/d)
    between neighbours, and the last pair's theta = base^(-(d-2)/d)."""
    for d, base in ((128, 10000.0), (64, 500000.0), (8, 4.0)):
        th = R.rope_frequencies(d, base)
        assert th.shape == (d // 2,)
        assert th[0] == 1.0
        np.testing.assert_allclose(th[d // 4], base ** -0.5, rtol=1e-15)
        np.testing.assert_allclose(th[1:] / th[:-1], base ** (-2.0 / d), rtol=1e-13)
        np.testing.assert_allclose(th[-1] * base, base ** (2.0 / d), rtol=1e-13)
    np.testing.assert_allclose(R.rope_frequencies(8, 10000.0), [1.0, 0.1, 0.01, 0.001], rtol=1e-15)


@pytest.mark.parametrize("d", [8, 64, 128])
def test_rope_is_complex_multiplication(d):
    """Pair i of row m, read as the complex number x_{2i} + i x_{2i+1}, is multiplied by
    exp(i m theta_i)."""
    x = RNG.standard_normal((2, 37, 3, d))
    y = R.apply_rope(x, 10000.0)
    th = R.rope_frequencies(d, 10000.0)
    z = (x[..., 0::2] + 1j * x[..., 1::2]) * np.exp(1j * np.arange(37)[None, :, None, None] * th)
    np.testing.assert_allclose(y[..., 0::2], z.real, atol=1e-12)
    np.testing.assert_allclose(y[..., 1::2], z.imag, atol=1e-12)


def test_rope_is_the_exponential_of_its_generator():
    """Brute force, d = 6: the row at position m is x exp(m J)^T with J block-diagonal,
    blocks [[0, -theta_i], [theta_i, 0]] (the rotation generator), via scipy's expm."""
    d, N, base = 6, 5, 100.0
    th = R.rope_frequencies(d, base)
    J = np.zeros((d, d))
    for i, t in enumerate(th):
        J[2 * i, 2 * i + 1], J[2 * i + 1, 2 * i] = -t, t
    x = RNG.standard_normal((1, N, 2, d))
    y = R.apply_rope(x, base)
    for m in range(N):
        Rm = scipy.linalg.expm(m * J)
        np.testing.assert_allclose(y[0, m], x[0, m] @ Rm.T, atol=1e-12)


def test_position_zero_is_identity_and_norms_are_kept():
    x = RNG.standard_normal((2, 50, 2, 64))
    y = R.apply_rope(x)
    np.testing.assert_array_equal(y[:, 0], x[:, 0])
    pn = lambda t: t[..., 0::2] ** 2 + t[..., 1::2] ** 2
    np.testing.assert_allclose(pn(y), pn(x), rtol=1e-12)
    assert np.abs(y[:, 1:] - x[:, 1:]).max() > 0.1


def test_scores_depend_only_on_relative_position():
    """<RoPE(q)_m, RoPE(k)_n> is a function of n - m alone, and equals <q, k> when m = n."""
    d, N = 64, 40
    a, b = RNG.standard_normal(d), RNG.standard_normal(d)
    x = np.zeros((1, N, 2, d))
    x[0, :, 0], x[0, :, 1] = a, b          # q = a and k = b at every position
    y = R.apply_rope(x)
    s = y[0, :, 0] @ y[0, :, 1].T          # s[m, n]
    for off in (-7, 0, 3, 11):
        diag = np.diagonal(s, offset=off)
        np.testing.assert_allclose(diag, diag[0], atol=1e-10)
    np.testing.assert_allclose(np.diagonal(s), a @ b, atol=1e-10)
    assert np.abs(s[0, 5] - s[5, 0]) > 1e-3   # not symmetric in m, n


def test_fused_prologue_is_the_composition():
    """quantize_rope_blocks = the block quantiser applied to RoPE(x): codes and descales equal,
    and scores of the dequantised values approximate RoPE attention scores."""
    import oracle
    x = RNG.standard_normal((1, 130, 2, 64)).astype(np.float32)
    for rotate in (False, True):
        c1, d1, y1 = oracle.quantize_rope_blocks(x, rotate, 99)
        c0, d0, y0 = oracle.quantize_blocks(R.apply_rope(x), rotate, 99)
        np.testing.assert_array_equal(c1, c0)
        np.testing.assert_array_equal(d1, d0)
    deq = oracle.dequantize_blocks(c1, d1)
    ref = R.apply_rope(x)
    s_deq = deq[0, :, 0] @ deq[0, :, 1].T
    s_ref = ref[0, :, 0] @ ref[0, :, 1].T
    assert np.abs(s_deq - s_ref).max() <= 0.05 * np.abs(s_ref).max()
