"""Pins of the float64 oracle against what the pages and the mathematics fix.

None of these re-types an oracle formula and compares it with itself: each check is an
identity, a closed form, a special case that reduces to a textbook or library routine,
a statistical property, or brute force on tiny inputs.  ``test_planted_mistakes_fail``
shows that plausible slips in the feature map (a dropped norm term, a wrong sign, a
missing 1/sqrt(m), a transposed W) each break at least one pin.
"""
import math

import numpy as np
import pytest
import torch

import oracle.favor_oracle as O
from efficient_transformer_attention_favor_amd.inputs import iid_matrix, orf_matrix


def _rng(seed):
    return np.random.default_rng(seed)


def _small_inputs(L=24, d=8, scale=0.35, seed=0):
    r = _rng(seed)
    return (r.standard_normal((L, d)) * scale, r.standard_normal((L, d)) * scale,
            r.standard_normal((L, d)))


# ---------------------------------------------------------------- closed forms


def test_feature_map_closed_form_one_dimension():
    # d = 1, m = 1: phi(x) = exp(w x - x^2/2).  w = 0.5, x = 2 -> exp(1 - 2) = e^-1.
    phi = O.feature_map(np.array([[2.0]]), np.array([[0.5]]))
    assert phi.shape == (1, 1)
    assert abs(phi[0, 0] - math.exp(-1.0)) < 1e-15
    # m = 2 rows w = (0.5, -1): exp(1-2)/sqrt(2), exp(-2-2)/sqrt(2)
    phi = O.feature_map(np.array([[2.0]]), np.array([[0.5], [-1.0]]))
    assert np.allclose(phi[0], [math.exp(-1) / math.sqrt(2), math.exp(-4) / math.sqrt(2)], rtol=1e-15)


def test_two_key_closed_form():
    # One query, two keys, m = 1, d = 1, W = [[w]]: the weights are
    # exp(w k_j - k_j^2/2) (the query factor cancels), so
    # out = (a1 v1 + a2 v2) / (a1 + a2) with a_j = exp(w k_j - k_j^2 / 2).
    w, k1, k2, v1, v2 = 0.7, 0.3, -1.1, 2.0, -5.0
    a1, a2 = math.exp(w * k1 - k1 * k1 / 2), math.exp(w * k2 - k2 * k2 / 2)
    expect = (a1 * v1 + a2 * v2) / (a1 + a2)
    out = O.favor_head(np.array([[0.4]]), np.array([[k1], [k2]]), np.array([[v1], [v2]]),
                       np.array([[w]]))
    assert abs(out[0, 0] - expect) < 1e-14


def _unbiased_deviation(feature_fn, n_seeds=4000, m=16, d=8, orth=True, seed=1):
    """max over pairs of |mean_seeds(A_hat_ij) - exp(q_i.k_j)| / (5 * stderr + 0.02 exp(q.k))."""
    q, k, _ = _small_inputs(L=4, d=d, seed=seed)
    exact = np.exp(q @ k.T)
    acc = np.zeros_like(exact)
    acc2 = np.zeros_like(exact)
    r = _rng(seed + 100)
    for _ in range(n_seeds):
        W = orf_matrix(m, d, r) if orth else iid_matrix(m, d, r)
        A = feature_fn(q, W) @ feature_fn(k, W).T
        acc += A
        acc2 += A * A
    mean = acc / n_seeds
    var = acc2 / n_seeds - mean * mean
    stderr = np.sqrt(np.maximum(var, 0) / n_seeds)
    return float(np.max(np.abs(mean - exact) / (5 * stderr + 0.02 * exact)))


@pytest.mark.parametrize("orth", [True, False])
def test_kernel_estimate_unbiased(orth):
    # E_w[exp(w.z)] = exp(|z|^2/2) for w ~ N(0, I) gives E[phi(x).phi(y)] = exp(x.y):
    # the seed-mean of A_hat must approach exact exp(q.k) (Performer, "제안 방법" /
    # "주요 결과": unbiased estimation).  ORF rows are marginally N(0, I) as well.
    assert _unbiased_deviation(O.feature_map, orth=orth) < 1.0


def test_error_decays_like_inverse_sqrt_m():
    # Performer, "주요 결과": accurate approximation at practical feature counts; the
    # Monte-Carlo error of an unbiased estimator falls like 1/sqrt(m).
    # Small-norm inputs (|q|^2 ~ 0.5) keep the estimator in its asymptotic regime.
    q, k, v = _small_inputs(L=16, d=8, scale=0.25, seed=3)
    exact = O.softmax_head(q, k, v)
    ms = [16, 64, 256]
    errs = []
    r = _rng(7)
    for m in ms:
        e = []
        for _ in range(150):
            W = orf_matrix(m, 8, r)
            e.append(np.mean((O.favor_head(q, k, v, W) - exact) ** 2))
        errs.append(math.sqrt(np.mean(e)))
    slope = np.polyfit(np.log(ms), np.log(errs), 1)[0]
    assert -0.65 <= slope <= -0.35, (errs, slope)


def test_orthogonal_features_no_worse_than_iid():
    # Performer, "주요 결과": orthogonal random features lower the mean squared error.
    q, k, v = _small_inputs(L=16, d=8, seed=5)
    exact = O.softmax_head(q, k, v)
    r = _rng(11)
    mse = {True: [], False: []}
    for _ in range(200):
        for orth in (True, False):
            W = orf_matrix(16, 8, r) if orth else iid_matrix(16, 8, r)
            mse[orth].append(np.mean((O.favor_head(q, k, v, W) - exact) ** 2))
    assert np.mean(mse[True]) <= np.mean(mse[False]) * 1.05


def test_many_features_approach_softmax():
    # With many features the estimate sits close to exact softmax attention: RMS error
    # over 3 feature draws (the per-draw maximum is heavy-tailed, the RMS is not).
    q, k, v = _small_inputs(L=32, d=8, seed=9)
    for causal in (False, True):
        exact = O.softmax_head(q, k, v, causal)
        rms = [np.sqrt(np.mean((O.favor_head(q, k, v, orf_matrix(8192, 8, _rng(13 + s)), causal)
                                - exact) ** 2)) for s in range(3)]
        assert np.mean(rms) < 0.015, rms


# ---------------------------------------------------------------- identities


@pytest.mark.parametrize("causal", [False, True])
def test_associativity(causal):
    # Linear order phi(Q)(phi(K)^T [V,1]) equals the explicit D^-1 A_hat V
    # (KDEformer, "提出的方法" for the D^-1 A V notation; Performer "요약" for linear order).
    q, k, v = _small_inputs(L=40, d=8, seed=21)
    W = orf_matrix(16, 8, _rng(22))
    A = O.implied_attention(q, k, W, causal)
    explicit = (A @ v) / A.sum(axis=1, keepdims=True)
    linear = O.favor_head(q, k, v, W, causal)
    assert np.max(np.abs(explicit - linear)) < 1e-12 * np.max(np.abs(explicit))
    rows = O.favor_head_rows(q, np.arange(len(q)), k, v, W, causal)
    assert np.max(np.abs(rows - linear)) < 1e-12 * np.max(np.abs(explicit))


@pytest.mark.parametrize("causal", [False, True])
def test_row_stochastic(causal):
    q, k, v = _small_inputs(L=33, d=8, seed=31)
    W = orf_matrix(16, 8, _rng(32))
    A = O.implied_attention(q, k, W, causal)
    P = A / A.sum(axis=1, keepdims=True)
    assert np.allclose(P.sum(axis=1), 1.0, atol=1e-14)
    mask = np.tril(np.ones_like(P, dtype=bool)) if causal else np.ones_like(P, dtype=bool)
    assert np.all(P[mask] > 0) and np.all(P[~mask] == 0)
    ones = O.favor_head(q, k, np.ones_like(v), W, causal)
    assert np.allclose(ones, 1.0, atol=1e-13)
    out = O.favor_head(q, k, v, W, causal)
    for i in range(len(q)):
        n = i + 1 if causal else len(q)
        assert np.all(out[i] <= v[:n].max(axis=0) + 1e-12)
        assert np.all(out[i] >= v[:n].min(axis=0) - 1e-12)
    alpha, beta = -2.5, np.linspace(-1, 1, v.shape[1])
    aff = O.favor_head(q, k, alpha * v + beta, W, causal)
    assert np.allclose(aff, alpha * out + beta, atol=1e-12)


def test_causal_prefix_equivalence():
    # Causal output at i equals the bidirectional output on the prefix ending at i.
    q, k, v = _small_inputs(L=30, d=8, seed=41)
    W = orf_matrix(24, 8, _rng(42))
    causal = O.favor_head(q, k, v, W, causal=True)
    for i in [0, 1, 7, 15, 29]:
        bid = O.favor_head(q[: i + 1], k[: i + 1], v[: i + 1], W)
        assert np.max(np.abs(causal[i] - bid[i])) < 1e-12


def test_identical_keys_give_mean_of_values():
    r = _rng(51)
    q = r.standard_normal((20, 8)) * 0.4
    k = np.repeat(r.standard_normal((1, 8)) * 0.4, 20, axis=0)
    v = r.standard_normal((20, 8))
    W = orf_matrix(16, 8, _rng(52))
    assert np.allclose(O.favor_head(q, k, v, W), v.mean(axis=0), atol=1e-13)
    prefix_mean = np.cumsum(v, axis=0) / np.arange(1, 21)[:, None]
    assert np.allclose(O.favor_head(q, k, v, W, causal=True), prefix_mean, atol=1e-13)


def test_single_position_returns_value():
    r = _rng(61)
    q, k, v = r.standard_normal((1, 8)), r.standard_normal((1, 8)), r.standard_normal((1, 8))
    W = orf_matrix(16, 8, _rng(62))
    for causal in (False, True):
        assert np.allclose(O.favor_head(q, k, v, W, causal), v, atol=1e-15)


@pytest.mark.parametrize("causal", [False, True])
def test_stabiliser_cancels(causal):
    # Any per-query-row constant and any single key constant cancel in num / den.
    q, k, v = _small_inputs(L=25, d=8, seed=71)
    W = orf_matrix(16, 8, _rng(72))
    base = O.favor_head(q, k, v, W, causal)
    c_q = _rng(73).uniform(-20, 20, size=(25, 1))
    shifted = O.favor_head(q, k, v, W, causal, c_q=c_q, c_k=-13.0)
    assert np.max(np.abs(shifted - base)) < 1e-12


def test_permutation_equivariance():
    q, k, v = _small_inputs(L=28, d=8, seed=81)
    W = orf_matrix(16, 8, _rng(82))
    base = O.favor_head(q, k, v, W)
    pk = _rng(83).permutation(28)
    assert np.allclose(O.favor_head(q, k[pk], v[pk], W), base, atol=1e-13)
    pq = _rng(84).permutation(28)
    assert np.allclose(O.favor_head(q[pq], k, v, W), base[pq], atol=1e-13)


# ---------------------------------------------------------------- library routines


@pytest.mark.parametrize("causal", [False, True])
def test_softmax_matches_library(causal):
    q, k, v = _small_inputs(L=37, d=8, scale=1.0, seed=91)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q)[None], torch.from_numpy(k)[None], torch.from_numpy(v)[None],
        is_causal=causal, scale=1.0)[0].numpy()
    assert np.max(np.abs(O.softmax_head(q, k, v, causal) - ref)) < 1e-12
    Q, K, V = (t[None, None] for t in (q, k, v))
    rows = np.array([[0, 0, i] for i in (0, 5, 36)])
    assert np.max(np.abs(O.softmax_rows(Q, K, V, rows, causal) - ref[[0, 5, 36]])) < 1e-12


def test_feature_map_brute_force():
    # Element by element with math.exp, on a tiny input.
    r = _rng(101)
    X, W = r.standard_normal((3, 4)), r.standard_normal((5, 4))
    phi = O.feature_map(X, W)
    for i in range(3):
        n2 = sum(x * x for x in X[i])
        for f in range(5):
            e = sum(W[f, t] * X[i, t] for t in range(4)) - n2 / 2
            assert abs(phi[i, f] - math.exp(e) / math.sqrt(5)) < 1e-14 * max(1.0, phi[i, f])


def test_causal_brute_force_loops():
    # Pure-Python double loop over (i, j <= i) with the brute-force features.
    r = _rng(111)
    L, d, m = 6, 3, 4
    q, k, v = r.standard_normal((L, d)) * 0.5, r.standard_normal((L, d)) * 0.5, r.standard_normal((L, d))
    W = r.standard_normal((m, d))

    def phi(x):
        n2 = sum(t * t for t in x)
        return [math.exp(sum(W[f, t] * x[t] for t in range(d)) - n2 / 2) / math.sqrt(m) for f in range(m)]

    ref = np.zeros((L, d))
    for i in range(L):
        pq = phi(q[i])
        num, den = [0.0] * d, 0.0
        for j in range(i + 1):
            a = sum(x * y for x, y in zip(pq, phi(k[j])))
            den += a
            for t in range(d):
                num[t] += a * v[j, t]
        ref[i] = [x / den for x in num]
    assert np.max(np.abs(O.favor_head(q, k, v, W, causal=True) - ref)) < 1e-13


# ---------------------------------------------------------------- head layout


@pytest.mark.parametrize("Hq,Hkv,Hw", [(4, 2, 2), (4, 1, 1), (3, 3, 1), (6, 3, 3)])
@pytest.mark.parametrize("causal", [False, True])
def test_head_map_matches_expanded_heads(Hq, Hkv, Hw, causal):
    # MQA page, "提出的方法": shared K/V heads behave as if each query head had its own copy.
    r = _rng(121)
    B, L, d, m = 2, 9, 8, 16
    Q = r.standard_normal((B, Hq, L, d)) * 0.4
    K = r.standard_normal((B, Hkv, L, d)) * 0.4
    V = r.standard_normal((B, Hkv, L, d))
    W = np.stack([orf_matrix(m, d, r) for _ in range(Hw)])
    G = Hq // Hkv
    Kx, Vx = np.repeat(K, G, axis=1), np.repeat(V, G, axis=1)
    Wx = np.repeat(W, Hq if Hw == 1 else G, axis=0)
    ref = O.favor_attention(Q, Kx, Vx, Wx, causal)
    assert np.allclose(O.favor_attention(Q, K, V, W, causal), ref, atol=1e-14)
    rows = np.array([[b, h, i] for b in range(B) for h in range(Hq) for i in (0, 4, 8)])
    got = O.favor_rows(Q, K, V, W, rows, causal)
    want = np.stack([ref[b, h, i] for b, h, i in rows])
    assert np.max(np.abs(got - want)) < 1e-12


def test_head_map_rejects_bad_layouts():
    with pytest.raises(ValueError):
        O.head_maps(6, 4, 4)
    with pytest.raises(ValueError):
        O.head_maps(4, 2, 3)


# ---------------------------------------------------------------- pins have teeth


def test_planted_mistakes_fail():
    def no_norm(X, W, c=0.0):
        X, W = np.asarray(X, float), np.asarray(W, float)
        return np.exp(X @ W.T) / np.sqrt(W.shape[0])

    def wrong_sign(X, W, c=0.0):
        X, W = np.asarray(X, float), np.asarray(W, float)
        return np.exp(X @ W.T + 0.5 * np.sum(X * X, -1, keepdims=True)) / np.sqrt(W.shape[0])

    def no_scale(X, W, c=0.0):
        return O.feature_map(X, W) * np.sqrt(W.shape[0])

    for bad in (no_norm, wrong_sign, no_scale):
        assert _unbiased_deviation(bad, n_seeds=1000) > 1.0, bad.__name__

    # A transposed W (square case) is no longer a valid feature draw for the pinned
    # two-key closed form.
    w = np.array([[0.7, 0.1], [-0.2, 0.4]])
    q, k = np.array([[0.3, 0.2]]), np.array([[0.5, -0.1], [-0.4, 0.9]])
    v = np.array([[1.0, 0.0], [0.0, 1.0]])
    good = O.favor_head(q, k, v, w)
    bad = O.favor_head(q, k, v, w.T)
    a = np.exp(k @ w.T - 0.5 * np.sum(k * k, 1, keepdims=True)) * np.exp(q @ w.T)
    weights = a.sum(axis=1)
    assert np.allclose(good[0], weights / weights.sum(), atol=1e-14)
    assert not np.allclose(bad[0], weights / weights.sum(), atol=1e-6)


# ---- backward (gradients of sum(dout * out), bidirectional) --------------------------

def _loss(Q, K, V, W, dOut, causal=False):
    return float(np.sum(dOut * O.favor_attention(Q, K, V, W, causal)))


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("Hq,Hkv,Hw", [(1, 1, 1), (4, 2, 2), (4, 1, 1)])
def test_grads_match_central_differences(Hq, Hkv, Hw, causal):
    """Pin: the written-out gradients agree with central differences of the forward oracle
    along random directions (float64, step 1e-5: truncation error ~1e-10)."""
    rng = np.random.default_rng(11)
    B, L, d, m = 2, 7, 4, 12
    Q = rng.standard_normal((B, Hq, L, d)) * d ** -0.25
    K = rng.standard_normal((B, Hkv, L, d)) * d ** -0.25
    V = rng.standard_normal((B, Hkv, L, d))
    W = np.stack([orf_matrix(m, d, rng) for _ in range(Hw)])
    dOut = rng.standard_normal((B, Hq, L, d))
    dQ, dK, dV = O.favor_grads(Q, K, V, W, dOut, causal)
    eps = 1e-5
    for _ in range(3):
        uq, uk, uv = (rng.standard_normal(x.shape) for x in (Q, K, V))
        fd = (_loss(Q + eps * uq, K + eps * uk, V + eps * uv, W, dOut, causal)
              - _loss(Q - eps * uq, K - eps * uk, V - eps * uv, W, dOut, causal)) / (2 * eps)
        an = np.sum(dQ * uq) + np.sum(dK * uk) + np.sum(dV * uv)
        assert abs(fd - an) <= 1e-7 * max(1.0, abs(an))
    # each input separately, so a mistake in one gradient cannot hide behind another
    for which in range(3):
        u = [np.zeros_like(x) for x in (Q, K, V)]
        u[which] = rng.standard_normal(u[which].shape)
        fd = (_loss(Q + eps * u[0], K + eps * u[1], V + eps * u[2], W, dOut, causal)
              - _loss(Q - eps * u[0], K - eps * u[1], V - eps * u[2], W, dOut, causal)) / (2 * eps)
        an = np.sum((dQ, dK, dV)[which] * u[which])
        assert abs(fd - an) <= 1e-7 * max(1.0, abs(an))


def test_grad_of_values_is_the_attention_transpose():
    """dV = A_hat_norm^T dout, with A_hat_norm = D^-1 phi(Q) phi(K)^T (the output is linear in V)."""
    rng = np.random.default_rng(12)
    L, d, m = 9, 4, 16
    q, k, v = rng.standard_normal((3, L, d)) * 0.7
    W = orf_matrix(m, d, rng)
    dout = rng.standard_normal((L, d))
    A = O.implied_attention(q, k, W)
    A = A / A.sum(axis=1, keepdims=True)
    _, _, dv = O.favor_head_grads(q, k, v, W, dout)
    assert np.max(np.abs(dv - A.T @ dout)) < 1e-12


def test_grads_vanish_for_constant_values():
    """V = 1: the output is identically 1 whatever Q and K are, so dQ = dK = 0."""
    rng = np.random.default_rng(13)
    L, d, m = 6, 4, 8
    q, k = rng.standard_normal((2, L, d)) * 0.7
    W = orf_matrix(m, d, rng)
    dq, dk, _ = O.favor_head_grads(q, k, np.ones((L, d)), W, rng.standard_normal((L, d)))
    assert np.max(np.abs(dq)) < 1e-12 and np.max(np.abs(dk)) < 1e-12


def test_query_feature_gradient_is_orthogonal_to_the_features():
    """Scaling phi(q_i) leaves out_i unchanged, so sum_f dphi(q_i)_f phi(q_i)_f = 0: the
    identity that lets an implementation drop the -q * rowsum term of dq."""
    rng = np.random.default_rng(14)
    L, d, m = 8, 4, 16
    q, k, v = rng.standard_normal((3, L, d)) * 0.7
    W = orf_matrix(m, d, rng)
    dout = rng.standard_normal((L, d))
    pq, pk = O.feature_map(q, W), O.feature_map(k, W)
    Sv, S1 = O.kv_summary(pk, v)
    D = pq @ S1
    out = (pq @ Sv) / D[:, None]
    dpq = (dout / D[:, None]) @ Sv.T + np.outer(-np.sum(dout * out, axis=1) / D, S1)
    assert np.max(np.abs(np.sum(dpq * pq, axis=1))) < 1e-12
    dq, _, _ = O.favor_head_grads(q, k, v, W, dout)
    assert np.max(np.abs(dq - (dpq * pq) @ W)) < 1e-12


def test_causal_grads_of_values_are_the_masked_attention_transpose():
    """Causal: dV = A_norm^T dout with A_norm the row-normalised lower-triangular A_hat."""
    rng = np.random.default_rng(15)
    L, d, m = 9, 4, 16
    q, k, v = rng.standard_normal((3, L, d)) * 0.7
    W = orf_matrix(m, d, rng)
    dout = rng.standard_normal((L, d))
    A = O.implied_attention(q, k, W, causal=True)
    A = A / A.sum(axis=1, keepdims=True)
    _, _, dv = O.favor_head_grads(q, k, v, W, dout, causal=True)
    assert np.max(np.abs(dv - A.T @ dout)) < 1e-12


def test_causal_grads_last_row_equal_bidirectional():
    """The last query row sees every key, so with an upstream gradient on that row only the
    causal gradients are the bidirectional ones; with the upstream gradient on rows < t only,
    keys and values at positions >= t receive nothing."""
    rng = np.random.default_rng(16)
    L, d, m, t = 10, 4, 16, 6
    q, k, v = rng.standard_normal((3, L, d)) * 0.7
    W = orf_matrix(m, d, rng)
    dout = np.zeros((L, d))
    dout[-1] = rng.standard_normal(d)
    a = O.favor_head_grads(q, k, v, W, dout, causal=True)
    b = O.favor_head_grads(q, k, v, W, dout, causal=False)
    for x, y in zip(a, b):
        assert np.max(np.abs(x - y)) < 1e-12
    dout = rng.standard_normal((L, d))
    dout[t:] = 0
    _, dk, dv = O.favor_head_grads(q, k, v, W, dout, causal=True)
    assert np.all(dk[t:] == 0) and np.all(dv[t:] == 0)
    assert np.max(np.abs(dk[:t])) > 1e-3 and np.max(np.abs(dv[:t])) > 1e-3


def test_causal_grads_vanish_for_constant_values():
    """V = 1 gives out = 1 under the mask as well, so dQ = dK = 0."""
    rng = np.random.default_rng(17)
    L, d, m = 7, 4, 8
    q, k = rng.standard_normal((2, L, d)) * 0.7
    W = orf_matrix(m, d, rng)
    dq, dk, _ = O.favor_head_grads(q, k, np.ones((L, d)), W, rng.standard_normal((L, d)), causal=True)
    assert np.max(np.abs(dq)) < 1e-12 and np.max(np.abs(dk)) < 1e-12


# ---- generalised attention: ReLU random features ----------------------------------------

def test_relu_features_estimate_the_arc_cosine_kernel():
    """Pin: with many i.i.d. Gaussian features, phi(x) . phi(y) tends to the first-order
    arc-cosine kernel |x||y| (sin t + (pi - t) cos t) / (2 pi) (closed form of
    E[ReLU(w.x) ReLU(w.y)] for w ~ N(0, I))."""
    rng = np.random.default_rng(21)
    d, m = 3, 400_000
    W = rng.standard_normal((m, d))
    for _ in range(3):
        x, y = rng.standard_normal((2, d))
        est = float(O.relu_feature_map(x[None], W)[0] @ O.relu_feature_map(y[None], W)[0])
        t = np.arccos(np.clip(x @ y / np.linalg.norm(x) / np.linalg.norm(y), -1, 1))
        exact = np.linalg.norm(x) * np.linalg.norm(y) * (np.sin(t) + (np.pi - t) * np.cos(t)) / (2 * np.pi)
        # Monte Carlo error: std <= sqrt(3) |x||y| / sqrt(m) = 0.0027 |x||y|
        assert abs(est - exact) < 0.01 * np.linalg.norm(x) * np.linalg.norm(y)


@pytest.mark.parametrize("causal", [False, True])
def test_generalized_linear_order_equals_row_definition(causal):
    rng = np.random.default_rng(22)
    B, Hq, Hkv, L, d, m = 2, 4, 2, 33, 8, 32
    Q, K, V = rng.standard_normal((B, Hq, L, d)), rng.standard_normal((B, Hkv, L, d)), rng.standard_normal((B, Hkv, L, d))
    W = rng.standard_normal((Hkv, m, d))
    full = O.generalized_attention(Q, K, V, W, causal)
    rows = np.array([(b, h, i) for b in range(B) for h in range(Hq) for i in range(L)])
    by_row = O.generalized_rows(Q, K, V, W, rows, causal).reshape(full.shape)
    assert np.max(np.abs(full - by_row)) < 1e-12
    ones = O.generalized_attention(Q, K, np.ones_like(V), W, causal)
    assert np.max(np.abs(ones - 1)) < 1e-12


def test_generalized_zero_weights_give_zero_rows():
    """A query whose ReLU features are all zero has no weight on any key: its row is 0 (the
    reading for 0/0); a single position otherwise returns its value."""
    d, m = 4, 16
    rng = np.random.default_rng(23)
    W = np.abs(rng.standard_normal((1, m, d)))          # every row has positive entries
    Q = np.zeros((1, 1, 3, d))
    Q[0, 0, 0] = -1.0                                    # W q < 0 for every feature
    Q[0, 0, 1:] = np.abs(rng.standard_normal((2, d)))
    K = np.abs(rng.standard_normal((1, 1, 3, d)))
    V = rng.standard_normal((1, 1, 3, d))
    out = O.generalized_attention(Q, K, V, W)
    assert np.all(out[0, 0, 0] == 0) and np.all(np.abs(out[0, 0, 1:]) > 0)
    one = O.generalized_attention(Q[:, :, 1:2], K[:, :, :1], V[:, :, :1], W)
    assert np.max(np.abs(one[0, 0, 0] - V[0, 0, 0])) < 1e-12


# ---------------------------------------------------------------- the parity metric


def test_rowwise_rel_err_hand_computed_rows():
    """The pass/fail metric of every forward parity test: max over rows of
    |y_i - r_i|_inf / |r_i|_inf, each row against its own largest magnitude.  Values worked
    by hand; each case separates the metric from a plausible slip."""
    # row 0: |y - r|_inf = 1 over |r|_inf = 1 -> 1.0;  row 1: 10 / 20 -> 0.5.  Result 1.0.
    # The global ratio max|y - r| / max|r| (10 / 20 = 0.5) and the column-wise ratio
    # (column 1: 10 / 20 = 0.5) both miss row 0.
    assert O.rowwise_rel_err([[1.0, 2.0], [0.0, 10.0]], [[1.0, 1.0], [0.0, 20.0]]) == 1.0
    # a row with a smaller maximum than another: row 0 0.1 / 0.2 = 0.5, row 1 0.5 / 5.5;
    # normalising by the largest row maximum instead would give 0.1 / 5.5
    assert O.rowwise_rel_err([[0.1, 0.0], [5.0, 5.0]], [[0.2, 0.0], [5.0, 5.5]]) == 0.5
    # magnitudes, not signed values: |(-2) - (-4)| / |-4| = 0.5 (max(r) = 1 would give 2)
    assert O.rowwise_rel_err([[-2.0, 1.0]], [[-4.0, 1.0]]) == 0.5
    # the infinity norm of the difference, not its sum: |(0.3, -0.3)| -> 0.3 / 1
    assert abs(O.rowwise_rel_err([[1.3, -0.3]], [[1.0, 0.0]]) - 0.3) < 1e-15
    # exact agreement -> 0
    assert O.rowwise_rel_err([[3.0, -4.0]], [[3.0, -4.0]]) == 0.0


def test_rowwise_rel_err_rows_are_the_last_axis():
    """(B, H, L, d) arrays: a row is one d-vector, whatever the leading shape."""
    r = np.ones((2, 3, 4, 5))
    y = r.copy()
    y[1, 2, 3, 4] = 1.25                  # one entry of one row off by 0.25
    y[0, 0, 0, :] = 1.1                   # every entry of another row off by 0.1
    assert abs(O.rowwise_rel_err(y, r) - 0.25) < 1e-15
    r2 = r.copy()
    r2[1, 2, 3] = 100.0                   # the first row's own maximum now 100: 0.25 / 100 is
    y2 = y.copy()                         # no longer the worst, the 0.1 row is
    y2[1, 2, 3] = r2[1, 2, 3]
    y2[1, 2, 3, 4] = 100.25
    assert abs(O.rowwise_rel_err(y2, r2) - 0.1) < 1e-12
    # float32 and bf16-valued inputs are compared in float64
    assert O.rowwise_rel_err(np.float32([[1.0, 2.0]]), np.float64([[1.0, 2.0]])) == 0.0
