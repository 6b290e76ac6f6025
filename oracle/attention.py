"""Exact attention in fp64, written as the plain definition (oracle; test infrastructure).

What is computed (page "FlashAttention-3: Hopper Asynchrony and FP8 Attention"):
  * Symbol Map: the score tile is Q_i K_j^T; P~ is the exponentiated score minus the row
    maximum; O_i is normalised by l_i at the end; the stored statistic is L_i = m_i + log(l_i).
  * The Core Idea: the FP16/BF16 output is the exact attention result, so the oracle is
    O = softmax(scale * Q K^T) V computed in one shot per row, with no online rescaling.
  * Deep Dive "Backward warp specialization": the backward recomputes S and P from L and
    forms dP, dS, dV, dK and dQ. The page names the quantities only; the formulas below are
    the analytic softmax gradient (dS = P o (dP - rowsum(P o dP))).

Readings where the pages are silent:
  * scale: the pages write S = Q K^T with no factor; the library takes an explicit scale
    (default 1/sqrt(d)) and both O and L are defined on the scaled scores.
  * log base of L: natural log, as written in the Symbol Map.
  * causal mask: key j is visible to query i iff j <= i (equal query and key lengths).
  * layout: tensors are [B, N, H, d] (token-major); L is [B, H, N].
  * variable-length batches (the enterprise post, "GPU Compatibility and Enablement Matrix",
    names variable-length sequence handling as a coming feature): sequences packed back to
    back, [T, heads, d], delimited by offsets cu_seqlens; each is an independent attention and
    L is [H, T].
  * grouped-query attention: the enterprise post ("FlashAttention 3 Hardware Acceleration",
    section "Runtime Kernel Selection") names the pattern without a formula. Reading: K and V
    may have Hkv heads, Hkv dividing H; query head h reads key/value head h // (H / Hkv); a
    shared head's dK, dV are the sums of the gradients through each of its query heads.

Row blocks below only bound memory: each row's softmax still sees its full key set at once,
and dK/dV sum over query rows block by block (the same sum, grouped).

Pins (tests/test_oracle_attention.py): torch's fp64 CPU math attention and autograd,
scipy's logsumexp/softmax, central finite differences, invariants (rows of P sum to 1,
constant V, key permutation, sum of dK = 0, sum of dV = sum of dO), closed forms (one-hot
scores, scale = 0, N = 1, causal row 0) and the split-KV log-sum-exp merge identity; for
grouped key/value heads, torch's fp64 grouped-query attention and its autograd, and central
finite differences through a shared head; for packed variable-length batches, isolation of
each sequence from the others' contents, and per-sequence closed forms (scale = 0 prefix
means, causal first rows).
"""
import numpy as np

ROW_BLOCK = 2048


def _f64(x):
    """Exact fp64 copy of an input given as numpy or torch (any float dtype)."""
    if hasattr(x, "detach"):
        x = x.detach().to("cpu")
        import torch
        x = x.to(torch.float64).numpy()
    return np.asarray(x, dtype=np.float64)


def _default_scale(d, scale):
    return 1.0 / np.sqrt(d) if scale is None else float(scale)


def _scores(qh, kh, rows, causal, scale):
    """scale * Q[rows] K^T with masked entries set to -inf (causal: key > query)."""
    s = scale * (qh[rows] @ kh.T)
    if causal:
        keys = np.arange(kh.shape[0])[None, :]
        s = np.where(keys > rows[:, None], -np.inf, s)
    return s


def head_probs(qh, kh, causal=False, scale=None, rows=None):
    """Normalised attention probabilities P = softmax(scale*Q K^T) for one head, rows given."""
    qh, kh = _f64(qh), _f64(kh)
    scale = _default_scale(qh.shape[1], scale)
    rows = np.arange(qh.shape[0]) if rows is None else np.asarray(rows)
    s = _scores(qh, kh, rows, causal, scale)
    m = s.max(axis=1, keepdims=True)
    e = np.exp(s - m)
    return e / e.sum(axis=1, keepdims=True)


def head_forward(qh, kh, vh, causal=False, scale=None, rows=None):
    """One head: qh [Nq, d], kh/vh [Nk, d]. Returns (O[rows] [len, d], L[rows] [len]).

    L_i = m_i + ln(l_i) with m_i the row maximum and l_i the max-subtracted sum of
    exponentials (Symbol Map); O = (exp(S - m) / l) V.
    """
    qh, kh, vh = _f64(qh), _f64(kh), _f64(vh)
    scale = _default_scale(qh.shape[1], scale)
    rows = np.arange(qh.shape[0]) if rows is None else np.asarray(rows)
    o = np.empty((len(rows), vh.shape[1]))
    lse = np.empty(len(rows))
    for r0 in range(0, len(rows), ROW_BLOCK):
        rr = rows[r0:r0 + ROW_BLOCK]
        s = _scores(qh, kh, rr, causal, scale)
        m = s.max(axis=1)
        e = np.exp(s - m[:, None])
        l = e.sum(axis=1)
        lse[r0:r0 + len(rr)] = m + np.log(l)
        o[r0:r0 + len(rr)] = (e / l[:, None]) @ vh
    return o, lse


def kv_head(h, H, Hkv):
    """Key/value head read by query head h when Hkv heads are shared by groups of H/Hkv
    consecutive query heads (grouped-query attention; Hkv = H is ordinary attention)."""
    if Hkv <= 0 or H % Hkv:
        raise ValueError(f"{H} query heads cannot be grouped over {Hkv} key/value heads")
    return h // (H // Hkv)


def forward(q, k, v, causal=False, scale=None):
    """Batched forward: q [B, N, H, d], k and v [B, N, Hkv, d] with Hkv dividing H (query
    head h attends to key/value head kv_head(h)). Returns O [B, N, H, d] and L [B, H, N]."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, N, H, d = q.shape
    Hkv = k.shape[2]
    o = np.empty((B, N, H, v.shape[3]))
    lse = np.empty((B, H, N))
    for b in range(B):
        for h in range(H):
            g = kv_head(h, H, Hkv)
            o[b, :, h], lse[b, h] = head_forward(q[b, :, h], k[b, :, g], v[b, :, g], causal, scale)
    return o, lse


def forward_rows(q, k, v, b, h, rows, causal=False, scale=None):
    """O and L for selected query rows of head (b, h); used for sampled checks at full size."""
    g = kv_head(h, q.shape[2], k.shape[2])
    return head_forward(q[b, :, h], k[b, :, g], v[b, :, g], causal, scale, rows=np.asarray(rows))


def head_backward(qh, kh, vh, doh, causal=False, scale=None):
    """Gradients of sum(dO o O) for one head. Returns (dQ, dK, dV), each [N, d] fp64.

    dV = P^T dO;  dP = dO V^T;  dS = P o (dP - rowsum(P o dP));  dQ = scale dS K;
    dK = scale dS^T Q. Masked entries have P = 0 and so dS = 0.
    """
    qh, kh, vh, doh = _f64(qh), _f64(kh), _f64(vh), _f64(doh)
    scale = _default_scale(qh.shape[1], scale)
    n = qh.shape[0]
    dq = np.empty_like(qh)
    dk = np.zeros_like(kh)
    dv = np.zeros_like(vh)
    for r0 in range(0, n, ROW_BLOCK):
        rr = np.arange(r0, min(n, r0 + ROW_BLOCK))
        s = _scores(qh, kh, rr, causal, scale)
        e = np.exp(s - s.max(axis=1, keepdims=True))
        p = e / e.sum(axis=1, keepdims=True)
        dp = doh[rr] @ vh.T
        ds = p * (dp - (p * dp).sum(axis=1, keepdims=True))
        dq[rr] = scale * (ds @ kh)
        dk += scale * (ds.T @ qh[rr])
        dv += p.T @ doh[rr]
    return dq, dk, dv


def backward(q, k, v, do, causal=False, scale=None):
    """Batched gradients; shapes as in forward. A shared key/value head collects the
    gradients of every query head that reads it. Returns fp64 (dQ, dK, dV)."""
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(do)
    B, N, H, d = q.shape
    Hkv = k.shape[2]
    dq, dk, dv = np.empty_like(q), np.zeros_like(k), np.zeros_like(v)
    for b in range(B):
        for h in range(H):
            g = kv_head(h, H, Hkv)
            dqh, dkh, dvh = head_backward(q[b, :, h], k[b, :, g], v[b, :, g], do[b, :, h], causal, scale)
            dq[b, :, h] = dqh
            dk[b, :, g] += dkh
            dv[b, :, g] += dvh
    return dq, dk, dv


def _spans(cu_seqlens):
    cu = [int(x) for x in np.asarray(cu_seqlens).reshape(-1)]
    if cu[0] != 0 or any(b < a for a, b in zip(cu, cu[1:])):
        raise ValueError("cu_seqlens must start at 0 and not decrease")
    return list(zip(cu[:-1], cu[1:]))


def forward_varlen(q, k, v, cu_seqlens, causal=False, scale=None):
    """Packed variable-length batch: q [T, H, d], k and v [T, Hkv, d]; sequence b is rows
    cu_seqlens[b] .. cu_seqlens[b+1]-1 and is an independent attention (the causal mask is
    within the sequence). Returns O [T, H, d] and L [H, T] in fp64."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    T, H, d = q.shape
    o = np.zeros((T, H, v.shape[2]))
    lse = np.zeros((H, T))
    for s0, s1 in _spans(cu_seqlens):
        if s1 > s0:
            ob, lb = forward(q[None, s0:s1], k[None, s0:s1], v[None, s0:s1], causal, scale)
            o[s0:s1], lse[:, s0:s1] = ob[0], lb[0]
    return o, lse


def backward_varlen(q, k, v, do, cu_seqlens, causal=False, scale=None):
    """Gradients of sum(dO o O) for a packed variable-length batch (shapes as in
    forward_varlen); returns fp64 (dQ, dK, dV)."""
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(do)
    dq, dk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    for s0, s1 in _spans(cu_seqlens):
        if s1 > s0:
            g = backward(q[None, s0:s1], k[None, s0:s1], v[None, s0:s1], do[None, s0:s1], causal, scale)
            dq[s0:s1], dk[s0:s1], dv[s0:s1] = (x[0] for x in g)
    return dq, dk, dv


def flops_forward(B, H, N, d, causal):
    """Forward FLOP convention: 4*B*H*N^2*d (two N x N x d products), halved when causal."""
    f = 4.0 * B * H * N * N * d
    return f / 2 if causal else f
