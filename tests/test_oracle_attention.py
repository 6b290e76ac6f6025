"""Pins for the fp64 attention oracle (CPU only).

Each check compares the oracle with something other than itself: torch's fp64 CPU math
attention and autograd, scipy's logsumexp/softmax, finite differences, closed forms and
invariants that follow from the definition of softmax attention (Symbol Map of the page
"FlashAttention-3: Hopper Asynchrony and FP8 Attention").
"""
import numpy as np
import pytest
import scipy.special
import torch

import oracle

RNG = np.random.default_rng(1234)
SHAPES = [(1, 1, 1, 4), (2, 5, 2, 8), (1, 33, 3, 16), (2, 70, 1, 32)]


def _rand(*shape, scale=1.0):
    return RNG.standard_normal(shape) * scale


def _torch_attention(q, k, v, causal, scale):
    """torch fp64 math attention on [B, N, H, d] numpy inputs; returns O and LSE."""
    tq, tk, tv = (torch.from_numpy(x).permute(0, 2, 1, 3).contiguous() for x in (q, k, v))
    o = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=causal, scale=scale)
    s = scale * (tq @ tk.transpose(-1, -2).contiguous())
    if causal:
        n = s.shape[-1]
        s = s.masked_fill(torch.triu(torch.ones(n, n, dtype=torch.bool), 1), float("-inf"))
    return o.permute(0, 2, 1, 3).numpy(), torch.logsumexp(s, dim=-1).numpy()


@pytest.mark.parametrize("shape", SHAPES)
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("scale", [None, 0.37, 2.0])
def test_forward_matches_torch_math_attention(shape, causal, scale):
    q, k, v = _rand(*shape), _rand(*shape), _rand(*shape)
    sc = 1 / np.sqrt(shape[3]) if scale is None else scale
    o, lse = oracle.forward(q, k, v, causal, scale)
    o_t, lse_t = _torch_attention(q, k, v, causal, sc)
    np.testing.assert_allclose(o, o_t, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, lse_t, rtol=0, atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_lse_and_probs_match_scipy(causal):
    n, d = 40, 16
    q, k = _rand(n, d), _rand(n, d)
    sc = 0.3
    s = sc * q @ k.T
    if causal:
        s[np.triu_indices(n, 1)] = -np.inf
    _, lse = oracle.head_forward(q, k, _rand(n, d), causal, sc)
    np.testing.assert_allclose(lse, scipy.special.logsumexp(s, axis=1), atol=1e-12)
    np.testing.assert_allclose(oracle.head_probs(q, k, causal, sc), scipy.special.softmax(s, axis=1), atol=1e-14)


@pytest.mark.parametrize("causal", [False, True])
def test_rows_of_p_sum_to_one(causal):
    p = oracle.head_probs(_rand(50, 8, scale=3), _rand(50, 8, scale=3), causal, 1.0)
    np.testing.assert_allclose(p.sum(1), 1.0, atol=1e-14)
    if causal:
        assert np.all(p[np.triu_indices(50, 1)] == 0)


@pytest.mark.parametrize("causal", [False, True])
def test_constant_v_gives_constant_output(causal):
    n, d = 37, 8
    c = _rand(d)
    o, _ = oracle.head_forward(_rand(n, d, scale=2), _rand(n, d, scale=2), np.tile(c, (n, 1)), causal, 0.9)
    np.testing.assert_allclose(o, np.tile(c, (n, 1)), atol=1e-13)


def test_joint_key_value_permutation_leaves_noncausal_output_unchanged():
    n, d = 45, 16
    q, k, v = _rand(n, d), _rand(n, d), _rand(n, d)
    perm = RNG.permutation(n)
    o1, l1 = oracle.head_forward(q, k, v, False, 0.25)
    o2, l2 = oracle.head_forward(q, k[perm], v[perm], False, 0.25)
    np.testing.assert_allclose(o1, o2, atol=1e-13)
    np.testing.assert_allclose(l1, l2, atol=1e-13)
    # the causal output is NOT permutation invariant (guards against a dropped mask)
    o3, _ = oracle.head_forward(q, k[perm], v[perm], True, 0.25)
    o4, _ = oracle.head_forward(q, k, v, True, 0.25)
    assert np.abs(o3 - o4).max() > 1e-3


@pytest.mark.parametrize("jstar", [0, 7, 19])
def test_one_hot_scores_closed_form(jstar):
    n, d, alpha, scale = 20, 8, 3.0, 0.7
    q = np.zeros((n, d)); q[:, 0] = alpha
    k = _rand(n, d); k[:, 0] = 0.0; k[jstar, :] = 0.0; k[jstar, 0] = 1.0
    v = _rand(n, d)
    a = alpha * scale
    o, lse = oracle.head_forward(q, k, v, False, scale)
    den = np.exp(a) + n - 1
    np.testing.assert_allclose(lse, np.log(den), atol=1e-13)
    expect = (np.exp(a) * v[jstar] + v.sum(0) - v[jstar]) / den
    np.testing.assert_allclose(o, np.tile(expect, (n, 1)), atol=1e-13)


def test_scale_zero_is_uniform_average():
    n, d = 30, 8
    q, k, v = _rand(n, d), _rand(n, d), _rand(n, d)
    o, lse = oracle.head_forward(q, k, v, False, 0.0)
    np.testing.assert_allclose(o, np.tile(v.mean(0), (n, 1)), atol=1e-13)
    np.testing.assert_allclose(lse, np.log(n), atol=1e-13)
    o, lse = oracle.head_forward(q, k, v, True, 0.0)
    np.testing.assert_allclose(o, np.cumsum(v, 0) / np.arange(1, n + 1)[:, None], atol=1e-13)
    np.testing.assert_allclose(lse, np.log(np.arange(1, n + 1)), atol=1e-13)


def test_causal_first_row_and_single_token():
    n, d, sc = 12, 8, 0.45
    q, k, v = _rand(n, d), _rand(n, d), _rand(n, d)
    o, lse = oracle.head_forward(q, k, v, True, sc)
    np.testing.assert_allclose(o[0], v[0], atol=1e-14)
    np.testing.assert_allclose(lse[0], sc * q[0] @ k[0], atol=1e-14)
    o1, l1 = oracle.head_forward(q[:1], k[:1], v[:1], False, sc)
    np.testing.assert_allclose(o1[0], v[0], atol=1e-14)
    np.testing.assert_allclose(l1[0], sc * q[0] @ k[0], atol=1e-14)


def test_split_kv_lse_merge_identity():
    n, d, sc = 64, 16, 0.25
    q, k, v = _rand(n, d), _rand(n, d), _rand(n, d)
    cut = 23
    oa, la = oracle.head_forward(q, k[:cut], v[:cut], False, sc)
    ob, lb = oracle.head_forward(q, k[cut:], v[cut:], False, sc)
    o, lse = oracle.head_forward(q, k, v, False, sc)
    lm = np.logaddexp(la, lb)
    np.testing.assert_allclose(lse, lm, atol=1e-13)
    np.testing.assert_allclose(o, np.exp(la - lm)[:, None] * oa + np.exp(lb - lm)[:, None] * ob, atol=1e-13)


def test_forward_rows_matches_full():
    q, k, v = (_rand(1, 300, 2, 16) for _ in range(3))
    o, lse = oracle.forward(q, k, v, True, 0.3)
    rows = np.array([0, 5, 128, 299])
    o_r, l_r = oracle.forward_rows(q, k, v, 0, 1, rows, True, 0.3)
    np.testing.assert_allclose(o_r, o[0, rows, 1], atol=1e-14)
    np.testing.assert_allclose(l_r, lse[0, 1, rows], atol=1e-14)


def test_row_blocking_does_not_change_result(monkeypatch):
    q, k, v, do = (_rand(1, 90, 1, 8) for _ in range(4))
    o1, l1 = oracle.forward(q, k, v, True, 0.5)
    g1 = oracle.backward(q, k, v, do, True, 0.5)
    monkeypatch.setattr(oracle.attention, "ROW_BLOCK", 16)
    o2, l2 = oracle.forward(q, k, v, True, 0.5)
    g2 = oracle.backward(q, k, v, do, True, 0.5)
    np.testing.assert_allclose(o1, o2, atol=1e-14)
    np.testing.assert_allclose(l1, l2, atol=1e-14)
    for a, b in zip(g1, g2):
        np.testing.assert_allclose(a, b, atol=1e-13)


@pytest.mark.parametrize("shape", SHAPES)
@pytest.mark.parametrize("causal", [False, True])
def test_backward_matches_torch_autograd(shape, causal):
    q, k, v, do = (_rand(*shape) for _ in range(4))
    sc = 0.6
    tq, tk, tv = (torch.from_numpy(x).permute(0, 2, 1, 3).contiguous().requires_grad_(True) for x in (q, k, v))
    o = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=causal, scale=sc)
    o.backward(torch.from_numpy(do).permute(0, 2, 1, 3))
    dq, dk, dv = oracle.backward(q, k, v, do, causal, sc)
    for mine, ref in ((dq, tq.grad), (dk, tk.grad), (dv, tv.grad)):
        np.testing.assert_allclose(mine, ref.permute(0, 2, 1, 3).numpy(), atol=1e-12)


@pytest.mark.parametrize("n,d", [(1, 4), (3, 4), (8, 8)])
@pytest.mark.parametrize("causal", [False, True])
def test_backward_finite_differences(n, d, causal):
    q, k, v, do = (_rand(n, d) for _ in range(4))
    sc, h = 0.8, 1e-6
    dq, dk, dv = oracle.head_backward(q, k, v, do, causal, sc)

    def loss(qq, kk, vv):
        return float((oracle.head_forward(qq, kk, vv, causal, sc)[0] * do).sum())

    for which, grad in ((0, dq), (1, dk), (2, dv)):
        fd = np.empty_like(grad)
        for idx in np.ndindex(*grad.shape):
            args_p = [q.copy(), k.copy(), v.copy()]
            args_m = [q.copy(), k.copy(), v.copy()]
            args_p[which][idx] += h
            args_m[which][idx] -= h
            fd[idx] = (loss(*args_p) - loss(*args_m)) / (2 * h)
        err = np.abs(fd - grad).max() / max(np.abs(grad).max(), 1e-300)
        assert err <= 1e-6 or np.abs(grad).max() < 1e-12, (which, err)


@pytest.mark.parametrize("causal", [False, True])
def test_backward_invariants(causal):
    n, d = 60, 16
    q, k, v, do = (_rand(n, d) for _ in range(4))
    dq, dk, dv = oracle.head_backward(q, k, v, do, causal, 0.3)
    np.testing.assert_allclose(dk.sum(0), 0.0, atol=1e-12)          # softmax shift invariance
    np.testing.assert_allclose(dv.sum(0), do.sum(0), atol=1e-12)    # rows of P sum to one


def test_rowsum_identity_used_by_gradient_kernels():
    """sum_j P_ij dP_ij = dO_i . O_i: lets a kernel form D from dO and O alone."""
    n, d, sc = 50, 16, 0.4
    q, k, v, do = (_rand(n, d) for _ in range(4))
    for causal in (False, True):
        p = oracle.head_probs(q, k, causal, sc)
        o, _ = oracle.head_forward(q, k, v, causal, sc)
        np.testing.assert_allclose((p * (do @ v.T)).sum(1), (do * o).sum(1), atol=1e-12)


@pytest.mark.parametrize("hkv", [1, 2])
@pytest.mark.parametrize("causal", [False, True])
def test_grouped_kv_heads_match_torch(hkv, causal):
    """Grouped-query attention against torch's fp64 implementation (enable_gqa) and its
    autograd: forward O and the gradients of the shared key/value heads."""
    B, N, H, d, sc = 2, 37, 4, 8, 0.7
    q, do = _rand(B, N, H, d), _rand(B, N, H, d)
    k, v = _rand(B, N, hkv, d), _rand(B, N, hkv, d)
    tq, tk, tv = (torch.from_numpy(x).permute(0, 2, 1, 3).contiguous().requires_grad_(True) for x in (q, k, v))
    o_t = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=causal, scale=sc, enable_gqa=True)
    o_t.backward(torch.from_numpy(do).permute(0, 2, 1, 3))
    o, _ = oracle.forward(q, k, v, causal, sc)
    np.testing.assert_allclose(o, o_t.detach().permute(0, 2, 1, 3).numpy(), atol=1e-12)
    dq, dk, dv = oracle.backward(q, k, v, do, causal, sc)
    assert dk.shape == k.shape and dv.shape == v.shape
    for mine, ref in ((dq, tq.grad), (dk, tk.grad), (dv, tv.grad)):
        np.testing.assert_allclose(mine, ref.permute(0, 2, 1, 3).numpy(), atol=1e-12)


def test_grouped_kv_heads_finite_differences():
    """dK and dV of a key/value head shared by two query heads, by central differences of
    sum(dO o O) over all heads."""
    B, N, H, hkv, d, sc, h = 1, 5, 4, 2, 4, 0.8, 1e-6
    q, do = _rand(B, N, H, d), _rand(B, N, H, d)
    k, v = _rand(B, N, hkv, d), _rand(B, N, hkv, d)
    for causal in (False, True):
        _, dk, dv = oracle.backward(q, k, v, do, causal, sc)

        def loss(kk, vv):
            return float((oracle.forward(q, kk, vv, causal, sc)[0] * do).sum())

        for which, grad in ((0, dk), (1, dv)):
            fd = np.empty_like(grad)
            for idx in np.ndindex(*grad.shape):
                ap, am = [k.copy(), v.copy()], [k.copy(), v.copy()]
                ap[which][idx] += h
                am[which][idx] -= h
                fd[idx] = (loss(*ap) - loss(*am)) / (2 * h)
            assert np.abs(fd - grad).max() <= 1e-6 * np.abs(grad).max(), (causal, which)


CU = [0, 5, 5, 17, 18, 40]   # lengths 5, 0, 12, 1, 22


@pytest.mark.parametrize("causal", [False, True])
def test_varlen_sequences_are_isolated(causal):
    """Changing every other sequence's Q, K, V and dO leaves a sequence's O, L and gradients
    unchanged, and gradients never leak into another sequence's rows."""
    T, H, hkv, d = CU[-1], 4, 2, 8
    q, do = _rand(T, H, d), _rand(T, H, d)
    k, v = _rand(T, hkv, d), _rand(T, hkv, d)
    o, lse = oracle.forward_varlen(q, k, v, CU, causal, 0.6)
    g = oracle.backward_varlen(q, k, v, do, CU, causal, 0.6)
    s0, s1 = 5, 17
    outside = np.r_[0:s0, s1:T]
    q2, k2, v2, do2 = (x.copy() for x in (q, k, v, do))
    for x in (q2, k2, v2, do2):
        x[outside] = _rand(len(outside), *x.shape[1:])
    o2, lse2 = oracle.forward_varlen(q2, k2, v2, CU, causal, 0.6)
    g2 = oracle.backward_varlen(q2, k2, v2, do2, CU, causal, 0.6)
    np.testing.assert_array_equal(o[s0:s1], o2[s0:s1])
    np.testing.assert_array_equal(lse[:, s0:s1], lse2[:, s0:s1])
    for a, b in zip(g, g2):
        np.testing.assert_array_equal(a[s0:s1], b[s0:s1])
    # dO zero outside the sequence: no gradient anywhere outside it
    do3 = np.zeros_like(do)
    do3[s0:s1] = do[s0:s1]
    for x in oracle.backward_varlen(q, k, v, do3, CU, causal, 0.6):
        assert np.abs(x[outside]).max() == 0.0


def test_varlen_closed_forms():
    """scale = 0: each sequence's O is the (prefix) mean of its own V and L = log of the
    number of visible keys; causal: the first row of each sequence is its first V row; a
    one-token sequence has O = v and L = scale * q.k."""
    T, H, d = CU[-1], 2, 4
    q, k, v = _rand(T, H, d), _rand(T, H, d), _rand(T, H, d)
    for causal in (False, True):
        o, lse = oracle.forward_varlen(q, k, v, CU, causal, 0.0)
        for s0, s1 in zip(CU[:-1], CU[1:]):
            if s1 == s0:
                continue
            n = np.arange(1, s1 - s0 + 1)
            if causal:
                ref = np.cumsum(v[s0:s1], axis=0) / n[:, None, None]
                np.testing.assert_allclose(lse[:, s0:s1], np.broadcast_to(np.log(n), (H, s1 - s0)), atol=1e-14)
            else:
                ref = np.broadcast_to(v[s0:s1].mean(axis=0), v[s0:s1].shape)
                np.testing.assert_allclose(lse[:, s0:s1], np.log(s1 - s0), atol=1e-14)
            np.testing.assert_allclose(o[s0:s1], ref, atol=1e-14)
        oc, lc = oracle.forward_varlen(q, k, v, CU, causal, 0.9)
        for s0, s1 in zip(CU[:-1], CU[1:]):
            if s1 > s0 and (causal or s1 == s0 + 1):
                np.testing.assert_allclose(oc[s0], v[s0], atol=1e-14)
        # the one-token sequence (row 17): O = v and L = scale * q.k, per head
        np.testing.assert_allclose(lc[:, 17], 0.9 * np.einsum("hd,hd->h", q[17], k[17]), atol=1e-14)


def test_kv_head_mapping():
    assert [oracle.kv_head(h, 8, 2) for h in range(8)] == [0, 0, 0, 0, 1, 1, 1, 1]
    assert [oracle.kv_head(h, 4, 4) for h in range(4)] == [0, 1, 2, 3]
    with pytest.raises(ValueError):
        oracle.kv_head(0, 6, 4)


def test_flop_convention():
    assert oracle.flops_forward(2, 16, 8192, 128, False) == 4 * 2 * 16 * 8192 ** 2 * 128
    assert oracle.flops_forward(2, 16, 8192, 128, True) == 2 * 2 * 16 * 8192 ** 2 * 128
