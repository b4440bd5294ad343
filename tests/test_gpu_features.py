"""favor_features (the feature map alone) against the float64 oracle's feature map.

phi_gpu is compared element by element with the oracle's exp(W x - |x|^2/2 - c)/sqrt(m)
evaluated at the stabiliser c the library reports, and c itself with the oracle's maximum
exponent over the row (queries) or over the (batch, kv head) (keys).

Tolerances, from the arithmetic.  float32 problems accumulate the exponent in float32
over d products: 1e-4 relative covers it.  bf16 problems contract in fp16: Q and K convert
exactly, W * log2(e) is rounded to fp16 (relative error <= 2^-11 per entry), so the
exponent of feature f for row x is off by at most 2^-11 * sum_k |w_fk x_k| (natural-log
units) plus float32 accumulation; phi may differ by exp of that bound, which the test
computes element by element.  Values the oracle puts below 1e-30 are only checked to be
tiny.
"""
import sys

import numpy as np
import pytest
import torch

import oracle.favor_oracle as O
from efficient_transformer_attention_favor_amd import api
from efficient_transformer_attention_favor_amd import inputs as I

pytestmark = pytest.mark.gpu

RTOL_F32 = 1e-4
FP16_UNIT = 2.0 ** -11
CASES = [
    I.workload("c2_bidir_bf16").replace(name="feat_bf16", batch=2, heads_q=4, heads_kv=2, heads_w=2,
                                        seq_len=333),
    I.workload("c4_mqa_bidir_bf16").replace(name="feat_bf16_d128", batch=1, heads_q=2, heads_kv=1,
                                            heads_w=1, seq_len=100),
    I.workload("c5_causal_long_bf16").replace(name="feat_heavy", batch=1, heads_q=2, heads_kv=2,
                                              heads_w=2, seq_len=700),
    I.workload("c1_bidir_f32").replace(name="feat_f32", seq_len=257),
    I.workload("c1_bidir_f32").replace(name="feat_f32_d128", batch=1, heads_q=2, heads_kv=1, heads_w=1,
                                       seq_len=65, head_dim=128, num_features=192),
]


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _exponents(X, W, heads_kv_of):
    """Oracle exponents E[bh, i, f] = w_f.x - |x|^2/2 for every row (no stabiliser)."""
    B, H, L, d = X.shape
    out = np.empty((B, H, L, W.shape[1]))
    for b in range(B):
        for h in range(H):
            Wh = W[0 if W.shape[0] == 1 else heads_kv_of(h)]
            x = X[b, h].astype(np.float64)
            out[b, h] = np.log(O.feature_map(x, Wh) * np.sqrt(Wh.shape[0]))
    return out


def _abs_products(X, W, heads_kv_of):
    """sum_k |w_fk x_k| for every row and feature."""
    B, H, L, d = X.shape
    out = np.empty((B, H, L, W.shape[1]))
    for b in range(B):
        for h in range(H):
            Wh = W[0 if W.shape[0] == 1 else heads_kv_of(h)]
            out[b, h] = np.abs(X[b, h].astype(np.float64)) @ np.abs(Wh.astype(np.float64)).T
    return out


def _compare(phi, c, X, W, heads_kv_of, side, dtype):
    B, H, L, _ = X.shape
    m = W.shape[1]
    E = _exponents(X, W, heads_kv_of)
    if dtype == "f32":
        e_tol = np.full(E.shape, RTOL_F32)
    else:  # bound on the exponent error (natural-log units), plus float32 accumulation
        e_tol = FP16_UNIT * _abs_products(X, W, heads_kv_of) + 1e-5
    rtol = np.expm1(e_tol)
    phi = phi.reshape(B, H, L, m).astype(np.float64)
    if side == 0:
        c_ref = E.max(axis=-1)
        cb = c.reshape(B, H, L, 1).astype(np.float64)
    else:
        c_ref = E.max(axis=(-2, -1))
        cb = c.reshape(B, H, 1, 1).astype(np.float64)
    c_tol = e_tol.max(axis=-1) if side == 0 else e_tol.max(axis=(-2, -1))
    c_ratio = np.max(np.abs(c.reshape(c_ref.shape) - c_ref) / (c_tol * np.maximum(1.0, np.abs(c_ref))))
    ref = np.exp(E - cb) / np.sqrt(m)
    big = ref > 1e-30
    ratio = np.max(np.abs(phi[big] - ref[big]) / ref[big] / rtol[big])
    tiny_ok = np.all(np.abs(phi[~big]) < 1e-29)
    rel = np.max(np.abs(phi[big] - ref[big]) / ref[big])
    _say(f"  side {side}: phi rel err {rel:.2e} ({ratio:.2f} of its bound), c at {c_ratio:.2f} of its bound")
    assert np.isfinite(phi).all()
    assert tiny_ok
    assert ratio < 1.0
    assert c_ratio < 1.0


@pytest.mark.parametrize("w", CASES, ids=lambda w: w.name)
@pytest.mark.parametrize("side", [0, 1])
def test_features_match_oracle(w, side):
    _say(f"case {w} side {side}")
    Q, K, V, W = I.make_inputs(w, seed=2)
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    X = Q if side == 0 else K
    x = torch.from_numpy(X).cuda().to(dt)
    phi, c = api.features(x, torch.from_numpy(W).cuda(), side, w.heads_q, w.heads_kv)
    torch.cuda.synchronize()
    G = w.heads_q // w.heads_kv
    heads_kv_of = (lambda h: h // G) if side == 0 else (lambda h: h)
    _compare(phi.cpu().numpy(), c.cpu().numpy(), X, W, heads_kv_of, side, w.dtype)


def test_features_repeat_is_bitwise_equal():
    w = CASES[0]
    Q, K, V, W = I.make_inputs(w, seed=4)
    k = torch.from_numpy(K).cuda().to(torch.bfloat16)
    wd = torch.from_numpy(W).cuda()
    a = api.features(k, wd, 1, w.heads_q, w.heads_kv)
    b = api.features(k, wd, 1, w.heads_q, w.heads_kv)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])
