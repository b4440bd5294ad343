"""FAVOR+ attention oracle: plain, slow, float64, CPU only.

TEST INFRASTRUCTURE.  Only the test-suite, ``__graft_entry__.smoke()`` and the CPU-baseline
leg of ``bench.py`` may import or call this module.  The library's HIP path never does,
and this module shares no code with it (it takes every input, W included, as an array).

What it computes, and where that is defined
-------------------------------------------
Sources are the review pages of "Rethinking Attention with Performers" (Performer),
"KDEformer: Accelerating Transformers via Kernel Density Estimation" (KDEformer) and
"Fast Transformer Decoding: One Write-Head is All You Need" (MQA).

* Performer, sections "요약" and "ABSTRACT": softmax attention is estimated in linear
  space and time, with no sparsity or low-rank prior.
* Performer, section "제안 방법": attention is written in kernelised form and the softmax
  kernel exp(q.k) is approximated with positive random features, with orthogonal random
  features to cut the variance; the estimate of the attention matrix is (nearly)
  unbiased.  The page prints no formula.  The feature map used here is the positive one,
        phi(x) = exp(W x - |x|^2 / 2) / sqrt(m),       W of shape (m, d),
  chosen because for w ~ N(0, I_d) one has E[exp(w.z)] = exp(|z|^2 / 2), hence
  E[phi(x).phi(y)] = exp(x.y) (see ``tests/test_oracle.py`` for the pin).  A constant c
  subtracted inside the exponent cancels in the normalised output; the oracle uses c = 0
  (float64 needs no stabiliser) and exposes c only so the invariance can be tested.
* KDEformer, section "提出的方法": attention written as D^-1 A V with A the (unnormalised)
  attention matrix and D the diagonal of its row sums.  With A_hat = phi(Q) phi(K)^T the
  FAVOR+ output is D^-1 A_hat V.  ``favor_rows`` is that definition, row by row;
  ``favor_attention`` is the linear-order evaluation phi(Q) (phi(K)^T [V, 1]) that the
  Performer page's linear space/time claim rests on.  Both reach the same numbers up to
  float64 rounding (pinned by the associativity test).
* Causal (unidirectional) mode is not on the pages; the reading taken is the standard
  inclusive mask j <= i, evaluated as a left-to-right running sum of phi(k_j) [v_j, 1]^T.
* MQA, section "提出的方法": one K/V head may serve many query heads.  Query head hq reads
  kv head hq // (Hq / Hkv); the feature matrix is per kv head (Hw == Hkv) or shared
  (Hw == 1).

Shapes: Q (B, Hq, L, d), K and V (B, Hkv, L, d), W (Hw, m, d); out (B, Hq, L, d).
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "feature_map",
    "kv_summary",
    "favor_head",
    "favor_head_rows",
    "implied_attention",
    "favor_attention",
    "favor_rows",
    "softmax_head",
    "softmax_rows",
    "head_maps",
    "rowwise_rel_err",
    "relu_feature_map",
    "generalized_attention",
    "generalized_rows",
]

_F = np.float64


def feature_map(X, W, c=0.0):
    """Positive random features phi(x) = exp(W x - |x|^2/2 - c) / sqrt(m) (Performer, "제안 방법").

    X (..., d), W (m, d); c broadcastable to X[..., :1] (a stabiliser; 0 by default).
    Returns (..., m) float64.
    """
    X = np.asarray(X, dtype=_F)
    W = np.asarray(W, dtype=_F)
    m = W.shape[0]
    E = X @ W.T - 0.5 * np.sum(X * X, axis=-1, keepdims=True) - c
    if not np.all(np.abs(E) < 700.0):
        raise FloatingPointError("feature exponent outside the float64 exp range")
    return np.exp(E) / np.sqrt(m)


def kv_summary(phi_k, V):
    """S = phi(K)^T [V, 1]: returns (S_v (m, d), S_1 (m,)) (Performer, "제안 방법": linear order)."""
    V = np.asarray(V, dtype=_F)
    return phi_k.T @ V, phi_k.sum(axis=0)


def favor_head(q, k, v, W, causal=False, c_q=0.0, c_k=0.0):
    """FAVOR+ on one head in linear order.  q, k, v (L, d); W (m, d).  Returns (L, d) float64.

    Bidirectional: S = phi(K)^T [V, 1] once, then out_i = phi(q_i) S_v / phi(q_i) S_1.
    Causal: S accumulated left to right over positions j <= i (inclusive).
    """
    v = np.asarray(v, dtype=_F)
    pq = feature_map(q, W, c_q)
    pk = feature_map(k, W, c_k)
    if not causal:
        Sv, S1 = kv_summary(pk, v)
        return (pq @ Sv) / (pq @ S1)[:, None]
    L, d = v.shape
    m = pk.shape[1]
    Sv = np.zeros((m, d))
    S1 = np.zeros(m)
    out = np.empty((L, d))
    for i in range(L):
        Sv += np.outer(pk[i], v[i])
        S1 += pk[i]
        out[i] = (pq[i] @ Sv) / (pq[i] @ S1)
    return out


def implied_attention(q, k, W, causal=False):
    """A_hat = phi(Q) phi(K)^T (L x L), lower-triangular (j <= i) when causal."""
    A = feature_map(q, W) @ feature_map(k, W).T
    if causal:
        A = np.tril(A)
    return A


def favor_head_rows(q_rows, pos, k, v, W, causal=False):
    """Rows of D^-1 A_hat V for the query rows q_rows (n, d) sitting at positions pos (n,).

    The definition written out row by row: weights a_j = phi(q_i) . phi(k_j) over
    j <= pos_i (causal) or all j, then sum_j a_j v_j / sum_j a_j.
    """
    v = np.asarray(v, dtype=_F)
    pk = feature_map(k, W)
    pq = feature_map(q_rows, W)
    out = np.empty((len(pos), v.shape[1]))
    for r, i in enumerate(pos):
        n = int(i) + 1 if causal else len(v)
        a = pk[:n] @ pq[r]
        out[r] = (a @ v[:n]) / a.sum()
    return out


def head_maps(Hq, Hkv, Hw):
    """(kv head of each query head, W index of each kv head) (MQA page, "提出的方法")."""
    if Hq % Hkv != 0 or Hw not in (1, Hkv):
        raise ValueError("heads_q must be a multiple of heads_kv and heads_w in {1, heads_kv}")
    G = Hq // Hkv
    return [hq // G for hq in range(Hq)], [0 if Hw == 1 else h for h in range(Hkv)]


def favor_attention(Q, K, V, W, causal=False):
    """Full FAVOR+ output (B, Hq, L, d) float64, linear order, head by head."""
    B, Hq, L, d = Q.shape
    Hkv, Hw = K.shape[1], W.shape[0]
    kv_of, w_of = head_maps(Hq, Hkv, Hw)
    out = np.empty((B, Hq, L, d))
    for b in range(B):
        for hq in range(Hq):
            hk = kv_of[hq]
            out[b, hq] = favor_head(Q[b, hq], K[b, hk], V[b, hk], W[w_of[hk]], causal)
    return out


def favor_rows(Q, K, V, W, rows, causal=False):
    """FAVOR+ output at the listed rows (n, 3) of (b, hq, i), by the row definition."""
    B, Hq, L, d = Q.shape
    Hkv, Hw = K.shape[1], W.shape[0]
    kv_of, w_of = head_maps(Hq, Hkv, Hw)
    rows = np.asarray(rows)
    out = np.empty((len(rows), d))
    for (b, hk) in sorted({(int(r[0]), kv_of[int(r[1])]) for r in rows}):
        sel = [n for n, r in enumerate(rows) if int(r[0]) == b and kv_of[int(r[1])] == hk]
        qr = np.stack([Q[rows[n][0], rows[n][1], rows[n][2]] for n in sel])
        pos = [int(rows[n][2]) for n in sel]
        out[sel] = favor_head_rows(qr, pos, K[b, hk], V[b, hk], W[w_of[hk]], causal)
    return out


def favor_head_grads(q, k, v, W, dout, causal=False):
    """Gradients of sum(dout * out) for FAVOR+ on one head, out = favor_head(q, k, v, W, causal).

    Written out from the linear-order definition by the chain rule (the pages give no
    backward pass; W is a fixed input).  With phi = feature_map, S_v = phi(K)^T V,
    S_1 = phi(K)^T 1, D_i = phi(q_i) . S_1 and out_i = phi(q_i) S_v / D_i:
        g_i = dout_i / D_i,   h_i = -(dout_i . out_i) / D_i
        dphi(q_i) = S_v g_i + S_1 h_i
        dS_v = sum_i phi(q_i) g_i^T,   dS_1 = sum_i phi(q_i) h_i
        dphi(k_j) = dS_v v_j + dS_1,   dv_j = dS_v^T phi(k_j)
    and, since d phi(x)_f / dx = phi(x)_f (w_f - x),
        dx = W^T (dphi * phi) - x sum_f (dphi * phi)_f.
    Causal (inclusive mask): S_v, S_1 are the running sums over j <= i at query row i, and
    key row j receives dS_v, dS_1 summed over the query rows i >= j only; the first is a
    left-to-right sweep, the second a right-to-left one.  q has the length of k then.
    Returns (dq (Lq, d), dk (L, d), dv (L, d)) in float64.
    """
    q = np.asarray(q, dtype=_F)
    k = np.asarray(k, dtype=_F)
    v = np.asarray(v, dtype=_F)
    W = np.asarray(W, dtype=_F)
    dout = np.asarray(dout, dtype=_F)
    pq = feature_map(q, W)
    pk = feature_map(k, W)
    if not causal:
        Sv, S1 = kv_summary(pk, v)
        D = pq @ S1
        out = (pq @ Sv) / D[:, None]
        g = dout / D[:, None]
        h = -np.sum(dout * out, axis=1) / D
        dpq = g @ Sv.T + np.outer(h, S1)
        dSv = pq.T @ g
        dS1 = pq.T @ h
        dpk = v @ dSv.T + dS1[None, :]
        dv = pk @ dSv
    else:
        L, d = v.shape
        m = pk.shape[1]
        if len(q) != L:
            raise ValueError("causal: queries and keys must have the same length")
        g = np.empty((L, d))
        h = np.empty(L)
        dpq = np.empty((L, m))
        Sv = np.zeros((m, d))
        S1 = np.zeros(m)
        for i in range(L):  # left to right: the prefix summaries each query row sees
            Sv += np.outer(pk[i], v[i])
            S1 += pk[i]
            D = pq[i] @ S1
            out_i = (pq[i] @ Sv) / D
            g[i] = dout[i] / D
            h[i] = -(dout[i] @ out_i) / D
            dpq[i] = Sv @ g[i] + S1 * h[i]
        dpk = np.empty((L, m))
        dv = np.empty((L, d))
        dSv = np.zeros((m, d))
        dS1 = np.zeros(m)
        for j in range(L - 1, -1, -1):  # right to left: the query rows i >= j
            dSv += np.outer(pq[j], g[j])
            dS1 += pq[j] * h[j]
            dpk[j] = dSv @ v[j] + dS1
            dv[j] = dSv.T @ pk[j]

    def through_features(x, dphi, phi):
        t = dphi * phi
        return t @ W - x * t.sum(axis=1)[:, None]

    return through_features(q, dpq, pq), through_features(k, dpk, pk), dv


def favor_grads(Q, K, V, W, dOut, causal=False):
    """Gradients (dQ, dK, dV) of sum(dOut * favor_attention(Q, K, V, W, causal)), with the MQA
    head map: a kv head's dK and dV sum over the query heads that read it."""
    B, Hq, L, d = Q.shape
    Hkv, Hw = K.shape[1], W.shape[0]
    kv_of, w_of = head_maps(Hq, Hkv, Hw)
    G = Hq // Hkv
    dQ = np.empty(Q.shape)
    dK = np.zeros(K.shape)
    dV = np.zeros(V.shape)
    for b in range(B):
        for hk in range(Hkv):
            heads = [hq for hq in range(Hq) if kv_of[hq] == hk]
            assert G == len(heads)
            if causal:
                # each query head is its own sequence over the positions of the kv head
                for hq in heads:
                    dq, dk, dv = favor_head_grads(Q[b, hq], K[b, hk], V[b, hk], W[w_of[hk]], dOut[b, hq], True)
                    dQ[b, hq] = dq
                    dK[b, hk] += dk
                    dV[b, hk] += dv
                continue
            # the G query heads of a kv head form one longer query sequence over the same S
            q = np.concatenate([Q[b, hq] for hq in heads])
            do = np.concatenate([dOut[b, hq] for hq in heads])
            dq, dk, dv = favor_head_grads(q, K[b, hk], V[b, hk], W[w_of[hk]], do)
            for n, hq in enumerate(heads):
                dQ[b, hq] = dq[n * L:(n + 1) * L]
            dK[b, hk] += dk
            dV[b, hk] += dv
    return dQ, dK, dV


def relu_feature_map(X, W):
    """phi(x) = ReLU(W x) / sqrt(m): a non-negative random feature map for a kernel other than
    softmax (Performer page, "ABSTRACT": FAVOR+ also models kernelisable attention beyond
    softmax).  For w ~ N(0, I_d), m E[phi(x) . phi(y)] = E[ReLU(w.x) ReLU(w.y)], the
    first-order arc-cosine kernel |x||y| (sin t + (pi - t) cos t) / (2 pi), t the angle
    between x and y (pinned in tests/test_oracle.py)."""
    X = np.asarray(X, dtype=_F)
    W = np.asarray(W, dtype=_F)
    return np.maximum(X @ W.T, 0.0) / np.sqrt(W.shape[0])


def _ratio(num, den):
    # a row whose weights are all zero (possible with ReLU features) gets a zero output
    out = np.zeros_like(num)
    ok = den > 0
    out[ok] = num[ok] / den[ok, None]
    return out


def generalized_attention(Q, K, V, W, causal=False, fn="relu"):
    """D^-1 A V with A = phi(Q) phi(K)^T for the feature map `fn` (KDEformer page, "提出的方法":
    attention as D^-1 A V), evaluated in linear order phi(Q) (phi(K)^T [V, 1]) per head, the
    causal mask j <= i as a running sum.  (B, Hq, L, d) float64."""
    if fn != "relu":
        raise ValueError(fn)
    B, Hq, L, d = Q.shape
    Hkv, Hw = K.shape[1], W.shape[0]
    kv_of, w_of = head_maps(Hq, Hkv, Hw)
    out = np.empty((B, Hq, L, d))
    for b in range(B):
        for hq in range(Hq):
            hk = kv_of[hq]
            pq = relu_feature_map(Q[b, hq], W[w_of[hk]])
            pk = relu_feature_map(K[b, hk], W[w_of[hk]])
            v = np.asarray(V[b, hk], dtype=_F)
            if causal:  # left-to-right running sums over j <= i
                m = pk.shape[1]
                Sv, S1 = np.zeros((m, d)), np.zeros(m)
                num, den = np.empty((L, d)), np.empty(L)
                for i in range(L):
                    Sv += np.outer(pk[i], v[i])
                    S1 += pk[i]
                    num[i] = pq[i] @ Sv
                    den[i] = pq[i] @ S1
            else:
                num = pq @ (pk.T @ v)
                den = pq @ pk.sum(axis=0)
            out[b, hq] = _ratio(num, den)
    return out


def generalized_rows(Q, K, V, W, rows, causal=False, fn="relu"):
    """The same at the listed (b, hq, i) rows, by the row definition sum_j a_ij v_j / sum_j a_ij."""
    if fn != "relu":
        raise ValueError(fn)
    B, Hq, L, d = Q.shape
    Hkv, Hw = K.shape[1], W.shape[0]
    kv_of, w_of = head_maps(Hq, Hkv, Hw)
    out = np.empty((len(rows), d))
    for n, (b, hq, i) in enumerate(np.asarray(rows)):
        hk = kv_of[int(hq)]
        n_keys = int(i) + 1 if causal else L
        pk = relu_feature_map(K[b, hk, :n_keys], W[w_of[hk]])
        a = pk @ relu_feature_map(Q[b, hq, i][None, :], W[w_of[hk]])[0]
        s = a.sum()
        out[n] = (a @ np.asarray(V[b, hk, :n_keys], dtype=_F)) / s if s > 0 else 0.0
    return out


def softmax_head(q, k, v, causal=False):
    """Exact softmax attention softmax(q k^T) v on one head (no 1/sqrt(d): the data carry it)."""
    q, k, v = (np.asarray(t, dtype=_F) for t in (q, k, v))
    s = q @ k.T
    if causal:
        s = np.where(np.tril(np.ones(s.shape, dtype=bool)), s, -np.inf)
    s = s - s.max(axis=1, keepdims=True)
    p = np.exp(s)
    return (p @ v) / p.sum(axis=1, keepdims=True)


def softmax_rows(Q, K, V, rows, causal=False):
    """Exact softmax attention at listed rows (b, hq, i); kv head by the MQA head map."""
    B, Hq, L, d = Q.shape
    G = Hq // K.shape[1]
    out = np.empty((len(rows), d))
    for n, (b, hq, i) in enumerate(np.asarray(rows)):
        k = np.asarray(K[b, hq // G], dtype=_F)
        v = np.asarray(V[b, hq // G], dtype=_F)
        n_keys = int(i) + 1 if causal else L
        s = k[:n_keys] @ np.asarray(Q[b, hq, i], dtype=_F)
        p = np.exp(s - s.max())
        out[n] = (p @ v[:n_keys]) / p.sum()
    return out


def rowwise_rel_err(y, r):
    """max over rows of |y_i - r_i|_inf / |r_i|_inf (rows along the last axis)."""
    y = np.asarray(y, dtype=_F).reshape(-1, np.shape(y)[-1])
    r = np.asarray(r, dtype=_F).reshape(-1, np.shape(r)[-1])
    return float(np.max(np.max(np.abs(y - r), axis=1) / np.max(np.abs(r), axis=1)))
