"""The seeded input generator: ORF structure, bf16 rounding, recipes, determinism."""
import math

import numpy as np
import pytest
import torch
from scipy.special import gammaln

from efficient_transformer_attention_favor_amd import inputs as I


def _chi_mean(d):
    return math.sqrt(2) * math.exp(gammaln((d + 1) / 2) - gammaln(d / 2))


@pytest.mark.parametrize("m,d", [(16, 8), (128, 64), (256, 128), (40, 16)])
def test_orf_blocks_orthogonal(m, d):
    W = I.orf_matrix(m, d, np.random.default_rng(0))
    assert W.shape == (m, d)
    for b0 in range(0, m, d):
        blk = W[b0:b0 + d]
        G = blk @ blk.T
        off = G - np.diag(np.diag(G))
        assert np.max(np.abs(off)) < 1e-12 * np.max(np.diag(G))


def test_orf_lengths_are_chi():
    d = 64
    W = I.orf_matrix(64 * 64, d, np.random.default_rng(1))
    n = np.linalg.norm(W, axis=1)
    # mean of chi(d) is sqrt(2) Gamma((d+1)/2) / Gamma(d/2) = 7.9688 for d = 64; its
    # variance is d - mean^2.
    mu = _chi_mean(d)
    sd = math.sqrt(d - mu * mu)
    assert abs(n.mean() - mu) < 5 * sd / math.sqrt(len(n))
    assert abs(n.std() - sd) < 0.1 * sd


def test_orf_rows_marginally_standard_normal():
    d = 8
    r = np.random.default_rng(2)
    rows = np.concatenate([I.orf_matrix(8, d, r) for _ in range(3000)])
    cov = rows.T @ rows / len(rows)
    assert np.max(np.abs(rows.mean(axis=0))) < 0.05
    assert np.max(np.abs(cov - np.eye(d))) < 0.06


def test_orf_deterministic():
    a = I.orf_matrix(32, 16, np.random.default_rng(5))
    b = I.orf_matrix(32, 16, np.random.default_rng(5))
    assert np.array_equal(a, b)


def test_bf16_rounding_matches_torch():
    r = np.random.default_rng(3)
    x = np.concatenate([r.standard_normal(100000).astype(np.float32) * 10,
                        np.array([0.0, -0.0, 1.0, 1.00390625, 1.01171875, 3.4e38, 1e-40], np.float32)])
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy()
    assert np.array_equal(I.round_to_bf16(x), ref)


def test_make_inputs_recipe_small():
    w = I.workload("c2_bidir_bf16").replace(name="tiny", batch=2, heads_q=4, heads_kv=2,
                                            heads_w=2, seq_len=300, num_features=128)
    Q, K, V, W = I.make_inputs(w, seed=0)
    assert Q.shape == (2, 4, 300, 64) and K.shape == (2, 2, 300, 64) and V.shape == K.shape
    assert W.shape == (2, 128, 64) and W.dtype == np.float32
    for t in (Q, K, V):
        assert np.array_equal(I.round_to_bf16(t), t)
    assert abs(Q.std() - 64 ** -0.25) < 0.01 and abs(V.std() - 1) < 0.02
    Q2, K2, V2, W2 = I.make_inputs(w, seed=0)
    assert all(np.array_equal(a, b) for a, b in ((Q, Q2), (K, K2), (V, V2), (W, W2)))
    Q3 = I.make_inputs(w, seed=1)[0]
    assert not np.array_equal(Q, Q3)


def test_heavy_rows():
    w = I.workload("c5_causal_long_bf16").replace(name="tiny_heavy", heads_q=2, heads_kv=2,
                                                  heads_w=2, seq_len=2000, num_features=64)
    Q, K, _, _ = I.make_inputs(w, seed=0)
    for X in (Q, K):
        n2 = np.sum(X.astype(np.float64) ** 2, axis=-1)
        heavy = n2 > 4 * math.sqrt(64)  # |x|^2 ~ sqrt(d) normally, ~9 sqrt(d) when heavy
        assert np.all(heavy.sum(axis=-1) == 100)


def test_workload_table():
    assert set(I.WORKLOADS) == {"c1_bidir_f32", "c2_bidir_bf16", "c3_causal_bf16",
                                "c4_mqa_bidir_bf16", "c5_causal_long_bf16"}
    c4 = I.workload("c4_mqa_bidir_bf16")
    assert (c4.heads_q, c4.heads_kv, c4.heads_w, c4.head_dim) == (16, 1, 1, 128)
    assert I.workload("c2_bidir_bf16").tokens == 8 * 8 * 4096


def test_sample_rows():
    w = I.workload("c5_causal_long_bf16")
    rows = I.sample_rows(w, 256)
    assert rows.shape[1] == 3 and len(rows) == 256
    assert (rows[:, 2] == 0).any() and (rows[:, 2] == w.seq_len - 1).any()
    assert np.all(rows[:, 1] < w.heads_q) and np.all(rows[:, 2] < w.seq_len)
