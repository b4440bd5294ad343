"""Pins of the seeded feature-matrix draw (oracle/feature_draw.py) against what fixes it
from outside: the generator's published known-answer vectors, the Gaussian distribution,
the QR factorisation (Gram-Schmidt is its Q up to column signs) and the row lengths."""
from pathlib import Path

import numpy as np
import pytest
from scipy import stats

import oracle.feature_draw as FD

GOLDEN = Path(__file__).parent / "golden" / "philox4x32_10_kat.txt"


def _kat_rows():
    for line in GOLDEN.read_text().splitlines():
        if line.strip() and not line.startswith("#"):
            yield [int(x, 16) for x in line.split()]


def test_philox_known_answers():
    rows = list(_kat_rows())
    assert len(rows) == 3
    for r in rows:
        out = FD.philox4x32_10(r[0:4], r[4:6])
        assert [int(x) for x in out] == r[6:10]


def test_philox_vectorised_matches_scalar():
    ctr = np.arange(5, dtype=np.uint64)
    vec = FD.philox4x32_10((ctr, 7, 0, 0), (3, 9))
    for i in range(5):
        one = FD.philox4x32_10((i, 7, 0, 0), (3, 9))
        assert [int(v[i]) for v in vec] == [int(x) for x in one]


def test_gaussian_stream_distribution():
    z = FD.gaussian_stream(1234, 0, 400_000)
    n = len(z)
    assert abs(z.mean()) < 5 / np.sqrt(n)
    assert abs(z.var() - 1) < 5 * np.sqrt(2 / n)
    assert stats.kstest(z, "norm").pvalue > 1e-4
    # the two numbers of one pair are uncorrelated
    assert abs(np.corrcoef(z[0::2], z[1::2])[0, 1]) < 5 / np.sqrt(n / 2)
    # fourth moment of N(0, 1) is 3
    assert abs(np.mean(z ** 4) - 3) < 0.1


def test_gaussian_stream_offsets_and_seeds():
    a = FD.gaussian_stream(7, 0, 100)
    assert np.array_equal(FD.gaussian_stream(7, 37, 20), a[37:57])
    assert not np.allclose(FD.gaussian_stream(8, 0, 100), a)
    big = (1 << 40) + 12345
    assert np.all(np.isfinite(FD.gaussian_stream(big, 1 << 33, 64)))


@pytest.mark.parametrize("m,d", [(64, 16), (40, 16), (48, 8)])
def test_orthogonal_draw_is_gram_schmidt(m, d):
    H, seed = 3, 99
    W = FD.draw_features(H, m, d, seed)
    G = FD.draw_features(H, m, d, seed, orthogonal=False)
    assert W.shape == (H, m, d) and G.shape == (H, m, d)
    nblk = (m + d - 1) // d
    for h in range(H):
        for b in range(nblk):
            rows = slice(b * d, min(m, (b + 1) * d))
            w, g = W[h, rows], G[h, rows]
            # lengths of the Gaussian rows
            assert np.allclose(np.linalg.norm(w, axis=1), np.linalg.norm(g, axis=1), rtol=1e-12)
            # orthogonal rows
            u = w / np.linalg.norm(w, axis=1)[:, None]
            assert np.max(np.abs(u @ u.T - np.eye(len(u)))) < 1e-12
            # Gram-Schmidt of the rows = Q of the QR factorisation of G^T, columns signed so
            # that R has a positive diagonal
            full = FD.gaussian_stream(seed, (h * nblk + b) * d * d, d * d).reshape(d, d)
            q, r = np.linalg.qr(full.T)
            q = q * np.sign(np.diag(r))[None, :]
            assert np.max(np.abs(u - q.T[:len(u)])) < 1e-10


def test_iid_draw_is_the_stream():
    H, m, d, seed = 2, 24, 8, 5
    G = FD.draw_features(H, m, d, seed, orthogonal=False)
    nblk = 3
    s = FD.gaussian_stream(seed, 0, H * nblk * d * d).reshape(H, nblk * d, d)
    assert np.array_equal(G, s[:, :m])


def test_truncated_last_block():
    W96 = FD.draw_features(1, 96, 64, 3)
    W128 = FD.draw_features(1, 128, 64, 3)
    assert np.array_equal(W96, W128[:, :96])


def test_orthogonal_rows_are_standard_gaussian():
    """Every ORF row is marginally N(0, I_d): entries with mean 0 and variance 1."""
    W = FD.draw_features(64, 64, 16, 11).reshape(-1)
    n = len(W)
    assert abs(W.mean()) < 5 / np.sqrt(n)
    assert abs(W.var() - 1) < 5 * np.sqrt(2 / n)
    assert stats.kstest(W, "norm").pvalue > 1e-4
