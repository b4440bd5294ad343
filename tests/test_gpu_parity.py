"""Parity of the HIP path (through the C ABI) with the float64 oracle.

Metric: row-wise relative error max_i |y_i - r_i|_inf / |r_i|_inf, the bar being 1e-4 for
float32 problems and 2e-2 for bf16 problems (bf16 inputs, float32 accumulation).  Small
shapes are compared in full (several tiles plus a ragged tail); the full-size workloads
on sampled rows that the oracle computes one by one.
"""
import sys

import numpy as np
import pytest
import torch

import oracle.favor_oracle as O
from efficient_transformer_attention_favor_amd import api
from efficient_transformer_attention_favor_amd import inputs as I

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-4, "bf16": 2e-2}


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _dev(x, dtype):
    return torch.from_numpy(np.ascontiguousarray(x)).to(device="cuda").to(dtype)


def _run(w, Q, K, V, W, chunk=0):
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    q, k, v = _dev(Q, dt), _dev(K, dt), _dev(V, dt)
    out = api.attn_fwd(q, k, v, _dev(W, torch.float32), causal=w.causal, chunk=chunk)
    torch.cuda.synchronize()
    return out


def _small(name, **kw):
    return I.workload(name).replace(name=f"{name}_small", **kw)


SMALL = [
    _small("c2_bidir_bf16", batch=1, heads_q=2, heads_kv=2, heads_w=2, seq_len=1000),
    _small("c2_bidir_bf16", batch=2, heads_q=1, heads_kv=1, heads_w=1, seq_len=1, num_features=64),
    _small("c2_bidir_bf16", batch=1, heads_q=1, heads_kv=1, heads_w=1, seq_len=31, num_features=64),
    _small("c2_bidir_bf16", batch=1, heads_q=1, heads_kv=1, heads_w=1, seq_len=64, num_features=192),
    _small("c2_bidir_bf16", batch=1, heads_q=1, heads_kv=1, heads_w=1, seq_len=300, num_features=512),
    _small("c2_bidir_bf16", batch=2, heads_q=6, heads_kv=2, heads_w=2, seq_len=129),
    _small("c4_mqa_bidir_bf16", batch=2, heads_q=4, heads_kv=1, heads_w=1, seq_len=777),
    # many kv heads, so one position range per head (the readout's ready LDS images)
    _small("c2_bidir_bf16", batch=8, heads_q=8, heads_kv=8, heads_w=8, seq_len=200),
    _small("c4_mqa_bidir_bf16", batch=64, heads_q=2, heads_kv=1, heads_w=1, seq_len=100),
    _small("c2_bidir_bf16", batch=32, heads_q=4, heads_kv=2, heads_w=1, seq_len=65, num_features=128),
    I.workload("c1_bidir_f32"),
    _small("c1_bidir_f32", batch=1, heads_q=2, heads_kv=1, heads_w=1, seq_len=333, head_dim=128,
           num_features=192),
    _small("c1_bidir_f32", batch=1, heads_q=1, heads_kv=1, heads_w=1, seq_len=70, num_features=320),
]


SMALL_CAUSAL = [
    _small("c3_causal_bf16", batch=1, heads_q=2, heads_kv=2, heads_w=2, seq_len=1000),
    _small("c3_causal_bf16", batch=2, heads_q=1, heads_kv=1, heads_w=1, seq_len=1, num_features=64),
    _small("c3_causal_bf16", batch=1, heads_q=1, heads_kv=1, heads_w=1, seq_len=33, num_features=128),
    _small("c3_causal_bf16", batch=2, heads_q=4, heads_kv=2, heads_w=2, seq_len=200),
    _small("c3_causal_bf16", batch=1, heads_q=2, heads_kv=1, heads_w=1, seq_len=300, head_dim=128),
    _small("c3_causal_bf16", batch=1, heads_q=1, heads_kv=1, heads_w=1, seq_len=270, head_dim=128),
    _small("c5_causal_long_bf16", batch=1, heads_q=2, heads_kv=2, heads_w=2, seq_len=700),
    _small("c3_causal_bf16", batch=1, heads_q=1, heads_kv=1, heads_w=1, seq_len=257, num_features=192),
    _small("c1_bidir_f32", causal=True, seq_len=257),
    _small("c1_bidir_f32", causal=True, batch=1, heads_q=2, heads_kv=1, heads_w=1, seq_len=100,
           head_dim=128, num_features=256),
    # d = 128 with m > 256: two launches over feature ranges [0, 256) and [256, m), the
    # second with (m - 256) / 32 waves, merged per row
    _small("c3_causal_bf16", batch=1, heads_q=2, heads_kv=1, heads_w=1, seq_len=301, head_dim=128,
           num_features=320),
    _small("c3_causal_bf16", batch=2, heads_q=2, heads_kv=2, heads_w=2, seq_len=95, head_dim=128,
           num_features=384),
    _small("c3_causal_bf16", batch=1, heads_q=1, heads_kv=1, heads_w=1, seq_len=160, head_dim=128,
           num_features=448),
    _small("c5_causal_long_bf16", batch=1, heads_q=4, heads_kv=1, heads_w=1, seq_len=513, head_dim=128),
    _small("c1_bidir_f32", causal=True, batch=1, heads_q=2, heads_kv=1, heads_w=1, seq_len=130,
           head_dim=128, num_features=384),
    _small("c1_bidir_f32", causal=True, batch=1, heads_q=1, heads_kv=1, heads_w=1, seq_len=67,
           head_dim=128, num_features=512),
]
SMALL = SMALL + SMALL_CAUSAL


@pytest.mark.parametrize("w", SMALL, ids=lambda w: f"{w.name}-L{w.seq_len}-d{w.head_dim}-m{w.num_features}")
def test_small_full_parity(w):
    _say(f"case {w}")
    Q, K, V, W = I.make_inputs(w, seed=0)
    y = _run(w, Q, K, V, W).float().cpu().numpy()
    ref = O.favor_attention(Q, K, V, W, causal=w.causal)
    err = O.rowwise_rel_err(y, ref)
    _say(f"  rowwise rel err {err:.3e}")
    assert np.isfinite(y).all()
    assert err < TOL[w.dtype]


@pytest.mark.parametrize("L", [777, 2900])
def test_causal_split_features_ragged(L):
    """d = 128 with m > 256 (two launches over feature ranges) with one and several segments
    and a ragged tail (its intra-chunk block is 32 positions)."""
    w = _small("c3_causal_bf16", batch=1, heads_q=2, heads_kv=1, heads_w=1, seq_len=L, head_dim=128,
               num_features=384)
    _say(f"case {w}")
    Q, K, V, W = I.make_inputs(w, seed=4)
    y = _run(w, Q, K, V, W, chunk=32).float().cpu().numpy()
    ref = O.favor_attention(Q, K, V, W, causal=True)
    assert O.rowwise_rel_err(y, ref) < TOL[w.dtype]


# intra-chunk blocks of 64-256 positions over feature counts that give 1, 2, 3 (of 4) and
# 8 waves, ragged tails, MQA groups; chunk 256 only up to m = 256
CHUNK_SHAPES = [
    (64, 64, 301, 1, 1), (128, 128, 700, 2, 2), (256, 192, 999, 4, 2), (64, 512, 640, 2, 1),
    (128, 512, 1001, 1, 1), (256, 256, 97, 2, 2), (128, 64, 1300, 3, 3),
    # shorter than one block, one position, one block and one more
    (32, 256, 1, 2, 2), (256, 256, 1, 1, 1), (64, 256, 31, 2, 1), (64, 128, 33, 1, 1), (256, 64, 33, 2, 2),
]


@pytest.mark.parametrize("chunk,m,L,hq,hkv", CHUNK_SHAPES,
                         ids=[f"C{c}-m{m}-L{L}-G{hq // hkv}" for c, m, L, hq, hkv in CHUNK_SHAPES])
def test_causal_intra_chunk_blocks(chunk, m, L, hq, hkv):
    w = _small("c3_causal_bf16", batch=1, heads_q=hq, heads_kv=hkv, heads_w=hkv, seq_len=L, num_features=m)
    _say(f"case {w} chunk={chunk}")
    Q, K, V, W = I.make_inputs(w, seed=6)
    y = _run(w, Q, K, V, W, chunk=chunk).float().cpu().numpy()
    ref = O.favor_attention(Q, K, V, W, causal=True)
    err = O.rowwise_rel_err(y, ref)
    _say(f"  rowwise rel err {err:.3e}")
    assert np.isfinite(y).all()
    assert err < TOL[w.dtype]


@pytest.mark.parametrize("chunk", [0, 32, 64, 128, 256])
def test_causal_chunk_sizes(chunk):
    w = _small("c3_causal_bf16", batch=1, heads_q=2, heads_kv=2, heads_w=2, seq_len=1111)
    _say(f"case {w} chunk={chunk}")
    Q, K, V, W = I.make_inputs(w, seed=1)
    y = _run(w, Q, K, V, W, chunk=chunk).float().cpu().numpy()
    ref = O.favor_attention(Q, K, V, W, causal=True)
    assert O.rowwise_rel_err(y, ref) < TOL[w.dtype]


def test_ones_values_give_ones():
    w = _small("c2_bidir_bf16", batch=1, heads_q=2, heads_kv=2, heads_w=2, seq_len=200)
    _say(f"case {w} V=1")
    Q, K, V, W = I.make_inputs(w, seed=3)
    y = _run(w, Q, K, np.ones_like(V), W).float().cpu().numpy()
    assert np.max(np.abs(y - 1.0)) < 1e-6


def test_deterministic_bits():
    w = _small("c2_bidir_bf16", batch=1, heads_q=2, heads_kv=2, heads_w=2, seq_len=1500)
    _say(f"case {w} determinism")
    Q, K, V, W = I.make_inputs(w, seed=5)
    a = _run(w, Q, K, V, W)
    b = _run(w, Q, K, V, W)
    assert torch.equal(a, b)


@pytest.mark.parametrize("name", ["c2_bidir_bf16", "c4_mqa_bidir_bf16", "c3_causal_bf16",
                                  "c5_causal_long_bf16"])
def test_full_size_sampled_rows(name):
    w = I.workload(name)
    _say(f"case {name} full size")
    Q, K, V, W = I.make_inputs(w, seed=0)
    y = _run(w, Q, K, V, W)
    rows = I.sample_rows(w, 256)
    got = torch.stack([y[b, h, i] for b, h, i in rows]).float().cpu().numpy()
    del y
    ref = O.favor_rows(Q, K, V, W, rows, causal=w.causal)
    err = O.rowwise_rel_err(got, ref)
    _say(f"  rowwise rel err over {len(rows)} rows {err:.3e}")
    assert err < TOL[w.dtype]


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_large_norm_inputs(causal, dtype):
    """Q and K scaled by 4 (exact in bf16): exponents spread over a range far beyond float32
    (|w.k| up to ~100 in log2 units), so the first block's stabilisers can be overtaken by
    later ones and the overflow fallback runs."""
    base = "c1_bidir_f32" if dtype == "f32" else "c2_bidir_bf16"
    w = _small(base, batch=1, heads_q=2, heads_kv=2, heads_w=2, seq_len=700, num_features=128, causal=causal)
    _say(f"case {w} x4")
    Q, K, V, W = I.make_inputs(w, seed=7)
    Q, K = Q * np.float32(4), K * np.float32(4)
    y = _run(w, Q, K, V, W).float().cpu().numpy()
    ref = O.favor_attention(Q, K, V, W, causal=causal)
    err = O.rowwise_rel_err(y, ref)
    _say(f"  rowwise rel err {err:.3e}")
    assert np.isfinite(y).all()
    assert err < TOL[w.dtype]


@pytest.mark.parametrize("base,kw,chunk", [
    ("c3_causal_bf16", dict(batch=1, heads_q=2, heads_kv=2, heads_w=2, seq_len=1000), 0),
    ("c3_causal_bf16", dict(batch=1, heads_q=2, heads_kv=1, heads_w=1, seq_len=301, head_dim=128), 0),
    ("c5_causal_long_bf16", dict(batch=1, heads_q=2, heads_kv=2, heads_w=2, seq_len=700, heavy_fraction=0.0), 0),
    ("c3_causal_bf16", dict(batch=1, heads_q=2, heads_kv=2, heads_w=2, seq_len=1000), 128),
    ("c5_causal_long_bf16", dict(batch=1, heads_q=2, heads_kv=2, heads_w=2, seq_len=700, heavy_fraction=0.0), 64),
    # one wave (m = 64); four waves of which the last has no features (m = 192)
    ("c3_causal_bf16", dict(batch=1, heads_q=1, heads_kv=1, heads_w=1, seq_len=500, num_features=64), 0),
    ("c3_causal_bf16", dict(batch=1, heads_q=2, heads_kv=1, heads_w=1, seq_len=650, num_features=192), 64),
    # d = 128 with m > 256: two launches over feature ranges, merged per row
    ("c3_causal_bf16", dict(batch=1, heads_q=2, heads_kv=1, heads_w=1, seq_len=700, head_dim=128, num_features=384), 0),
    # float32: one 32-feature tile per wave, two tiles per wave (m > 256), d = 128 split in two
    ("c1_bidir_f32", dict(heads_q=2, heads_kv=2, heads_w=2, seq_len=700, num_features=256, causal=True), 0),
    ("c1_bidir_f32", dict(heads_q=2, heads_kv=1, heads_w=1, seq_len=533, num_features=512, causal=True), 0),
    ("c1_bidir_f32", dict(heads_q=1, heads_kv=1, heads_w=1, seq_len=600, head_dim=128, num_features=128, causal=True), 0),
    ("c1_bidir_f32", dict(heads_q=2, heads_kv=1, heads_w=1, seq_len=417, head_dim=128, num_features=384, causal=True), 0),
], ids=["d64m256", "d128m256", "d64m512", "d64m256-C128", "d64m512-C64", "d64m64", "d64m192-C64", "d128m384",
        "f32-d64m256", "f32-d64m512", "f32-d128m128", "f32-d128m384"])
def test_causal_keys_far_apart(base, kw, chunk):
    """K scaled by 8 (exact in bf16): |k|^2 / 2 alone spreads the key exponents over hundreds
    of log2 units, so early queries whose keys all sit far below a later key of the same block
    (or of the sequence) must not lose their terms to underflow.  With intra-chunk blocks
    above 32 positions the stabilisers also move in the middle of a chunk.  Every causal
    kernel family is covered: bf16 d = 64 (by intra-chunk block), bf16 d = 128 (m <= 256 and
    the two-range split above), and float32."""
    w = _small(base, **kw)
    _say(f"case {w} K x8 chunk={chunk}")
    Q, K, V, W = I.make_inputs(w, seed=4)
    K = K * np.float32(8)
    y = _run(w, Q, K, V, W, chunk=chunk).float().cpu().numpy()
    ref = O.favor_attention(Q, K, V, W, causal=True)
    err = O.rowwise_rel_err(y, ref)
    _say(f"  rowwise rel err {err:.3e}")
    assert np.isfinite(y).all()
    assert err < TOL[w.dtype]
