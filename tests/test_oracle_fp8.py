"""Pins for the FP8 oracle (CPU only): OCP e4m3 codec, rotation, SplitMix64, block quantiser."""
import numpy as np
import pytest
import scipy.linalg

import oracle

RNG = np.random.default_rng(99)


def test_e4m3_ocp_fixed_points():
    dec = oracle.e4m3_decode
    assert dec(0x7E) == 448.0 and dec(0xFE) == -448.0          # largest finite
    assert dec(0x08) == 2.0 ** -6                               # smallest normal
    assert dec(0x07) == 7 * 2.0 ** -9                           # largest subnormal
    assert dec(0x01) == 2.0 ** -9                               # smallest subnormal
    assert dec(0x38) == 1.0 and dec(0xB8) == -1.0               # exponent bias 7
    assert dec(0x00) == 0.0 and np.signbit(dec(0x80))
    assert np.isnan(dec(0x7F)) and np.isnan(dec(0xFF))
    assert np.isnan(dec(np.arange(256))).sum() == 2             # no infinities, two NaNs
    assert dec(0x78) == 256.0 and dec(0x57) == 15.0 and dec(0x70) == 128.0


def test_e4m3_positive_codes_are_strictly_increasing():
    v = oracle.e4m3_finite_values()
    assert len(v) == 127 and np.all(np.diff(v) > 0)


def test_e4m3_round_trip_all_codes():
    c = np.arange(256)
    v = oracle.e4m3_decode(c)
    ok = ~np.isnan(v)
    np.testing.assert_array_equal(oracle.e4m3_encode(v[ok]), c[ok])


def test_e4m3_midpoints_round_to_even_and_neighbours_to_nearest():
    v = oracle.e4m3_finite_values()
    for c in range(0x7E):
        mid = (v[c] + v[c + 1]) / 2
        even = c if c % 2 == 0 else c + 1
        assert oracle.e4m3_encode(mid) == even
        assert oracle.e4m3_encode(-mid) == even | 0x80
        eps = (v[c + 1] - v[c]) * 1e-6
        assert oracle.e4m3_encode(mid - eps) == c
        assert oracle.e4m3_encode(mid + eps) == c + 1


def test_e4m3_encode_is_nearest_by_brute_force():
    x = np.concatenate([RNG.standard_normal(4000) * s for s in (1e-3, 1e-1, 1, 30, 200)])
    codes = oracle.e4m3_encode(x)
    allv = oracle.e4m3_decode(np.arange(256))
    fin = np.where(np.isnan(allv), np.inf, allv)
    for xi, ci in zip(x, codes):
        best = np.abs(fin - xi).min()
        assert abs(allv[ci] - xi) == best


def test_e4m3_saturation():
    np.testing.assert_array_equal(oracle.e4m3_encode([449.0, 463.9, 464.0, 480.0, 1e9, -1e9, np.inf]),
                                  [0x7E, 0x7E, 0x7E, 0x7E, 0x7E, 0xFE, 0x7E])


def test_splitmix64_reference_outputs():
    # published first outputs of SplitMix64 seeded with 0
    assert oracle.splitmix64(0, 3) == [0xE220A8397B1DCDAF, 0x6E789E6AA1B965F4, 0x06C45D188009454F]


def test_signs_are_seed_dependent_and_mixed():
    s1, s2 = oracle.hadamard_signs(7, 128), oracle.hadamard_signs(8, 128)
    assert set(np.unique(s1)) == {-1.0, 1.0}
    assert 30 < (s1 > 0).sum() < 98
    assert np.any(s1 != s2)
    np.testing.assert_array_equal(s1, oracle.hadamard_signs(7, 128))


@pytest.mark.parametrize("d", [1, 2, 4, 64, 128, 256])
def test_sylvester_matches_scipy(d):
    np.testing.assert_array_equal(oracle.sylvester_hadamard(d), scipy.linalg.hadamard(d))


@pytest.mark.parametrize("d", [64, 128, 256])
def test_rotation_is_orthogonal_and_preserves_scores(d):
    m = oracle.rotation_matrix(d, seed=12345)
    np.testing.assert_allclose(m @ m.T, np.eye(d), atol=1e-12)
    q, k = RNG.standard_normal((20, d)), RNG.standard_normal((30, d))
    np.testing.assert_allclose((q @ m) @ (k @ m).T, q @ k.T, atol=1e-11)
    # it is not the identity and not a plain permutation
    assert np.abs(m).max() < 0.5


def _check_block_bounds(x, codes, descale, y):
    deq = oracle.dequantize_blocks(codes, descale)
    B, N, H, d = x.shape
    ds = np.transpose(descale.astype(np.float64)[:, :, np.arange(N) // 64], (0, 2, 1))[..., None]
    ay = np.abs(y)
    # half an e4m3 ulp: 2^-4 relative in the normal range, 2^-10 absolute (scaled) below it
    bound = np.maximum(ay * 2.0 ** -4, ds * 2.0 ** -10) * (1 + 1e-9)
    assert np.all(np.abs(deq - y) <= bound)
    for b in range(B):
        for h in range(H):
            for j in range(descale.shape[2]):
                tile = y[b, j * 64:(j + 1) * 64, h]
                amax = np.abs(tile).max()
                if amax == 0:
                    assert descale[b, h, j] == 1.0
                    assert np.all(codes[b, j * 64:(j + 1) * 64, h] & 0x7F == 0)
                    continue
                assert abs(descale[b, h, j] * 448.0 - amax) <= amax * 2.0 ** -22
                idx = np.unravel_index(np.abs(tile).argmax(), tile.shape)
                assert codes[b, j * 64:(j + 1) * 64, h][idx] & 0x7F == 0x7E


@pytest.mark.parametrize("rotate", [False, True])
def test_block_quantizer_bounds(rotate):
    x = RNG.standard_normal((2, 150, 3, 64))
    x[0, 3, 1, 5] = 40.0                      # an outlier
    x[1, 64:128, 2] = 0.0                     # an all-zero block
    codes, descale, y = oracle.quantize_blocks(x, rotate, seed=3)
    assert descale.shape == (2, 3, 3) and descale.dtype == np.float32
    if rotate:
        np.testing.assert_allclose(y, x @ oracle.rotation_matrix(64, 3), atol=1e-12)
    else:
        np.testing.assert_array_equal(y, x)
    _check_block_bounds(x, codes, descale, y)


@pytest.mark.parametrize("rotate", [False, True])
def test_per_tensor_quantizer(rotate):
    """One scale for the whole tensor: every element within half an e4m3 step of its value
    at that scale; only the tensor's largest element(s) reach the +-448 code; the descale
    is the largest of the block descales; power-of-two input scaling moves only the
    descale."""
    x = RNG.standard_normal((2, 150, 3, 64))
    x[1, 100, 2, 7] = -55.0                   # the tensor's outlier, in one block of one head
    x[0, 64:128, 1] = 0.0                     # an all-zero block keeps its codes at zero
    codes, descale, y = oracle.quantize_per_tensor(x, rotate, seed=5)
    assert descale.shape == (2, 3, 3) and descale.dtype == np.float32
    assert np.all(descale == descale.flat[0])
    ds = float(descale.flat[0])
    amax = np.abs(y).max()
    assert abs(ds * 448.0 - amax) <= amax * 2.0 ** -22
    deq = oracle.e4m3_decode(codes) * ds
    bound = np.maximum(np.abs(y) * 2.0 ** -4, ds * 2.0 ** -10) * (1 + 1e-9)
    assert np.all(np.abs(deq - y) <= bound)
    top = np.abs(y) == amax
    assert np.all(codes[top] & 0x7F == 0x7E)
    assert np.all(codes[~top] & 0x7F < 0x7E) or np.abs(y[~top]).max() * 448.0 / amax > 416.0
    assert np.all(codes[0, 64:128, 1] & 0x7F == 0)
    # the single descale is the largest descale of the blocks that are not all zero (an
    # all-zero block's own descale is 1 by definition)
    _, bds, _ = oracle.quantize_blocks(x, rotate, seed=5)
    nonzero = np.abs(y).reshape(2, 150, 3, 64).max(axis=3)
    nz = np.array([[[nonzero[b_, j * 64:(j + 1) * 64, h_].max() > 0 for j in range(3)] for h_ in range(3)]
                   for b_ in range(2)])
    assert ds == bds[nz].max() and not nz.all()
    # scaling the input by 2^-3 scales the descale by 2^-3 and keeps every code
    c2, d2, _ = oracle.quantize_per_tensor(x * 0.125, rotate, seed=5)
    np.testing.assert_array_equal(c2, codes)
    assert float(d2.flat[0]) == ds * 0.125


def test_per_tensor_equals_block_on_one_block():
    x = RNG.standard_normal((1, 50, 1, 128))
    for rotate in (False, True):
        c1, d1, _ = oracle.quantize_per_tensor(x, rotate, seed=9)
        c2, d2, _ = oracle.quantize_blocks(x, rotate, seed=9)
        np.testing.assert_array_equal(c1, c2)
        np.testing.assert_array_equal(d1, d2)
    # with several blocks they differ: small blocks keep finer codes under their own scale
    x = RNG.standard_normal((1, 128, 1, 64))
    x[0, 0, 0, 0] = 300.0
    c1, d1, y = oracle.quantize_per_tensor(x, False)
    c2, d2, _ = oracle.quantize_blocks(x, False)
    e1 = np.abs(oracle.dequantize_blocks(c1, d1) - y)[0, 64:].max()
    e2 = np.abs(oracle.dequantize_blocks(c2, d2) - y)[0, 64:].max()
    assert d1[0, 0, 1] > d2[0, 0, 1] and e1 > e2


def test_rotated_quantised_scores_track_exact_scores():
    x_q = RNG.standard_normal((1, 128, 1, 128))
    x_k = RNG.standard_normal((1, 128, 1, 128))
    q8, dq, _ = oracle.quantize_blocks(x_q, True, seed=11)
    k8, dk, _ = oracle.quantize_blocks(x_k, True, seed=11)
    qh = oracle.dequantize_blocks(q8, dq)[0, :, 0]
    kh = oracle.dequantize_blocks(k8, dk)[0, :, 0]
    exact = x_q[0, :, 0] @ x_k[0, :, 0].T
    err = qh @ kh.T - exact
    # each product term carries ~2*3.6% relative noise: rms error ~ 0.05*sqrt(d)
    assert np.sqrt((err ** 2).mean()) < 0.1 * np.sqrt(128)
    assert np.sqrt((err ** 2).mean()) > 1e-3            # it really was quantised
