"""FAVOR+ against exact softmax attention, reported (not a pass criterion).

For every workload the GPU output on 256 sampled rows (all rows for the f32 workload) is
compared with exact softmax attention softmax(q K^T) V on the same inputs (the oracle's
``softmax_rows``), once with the orthogonal random features W of the workload and once
with an unstructured Gaussian W of the same shape (Performer page, "제안 방법" and
"주요 결과": orthogonal features lower the estimator's error).  The numbers are printed;
the only assertion is that they are finite.  (Row-wise relative error is large here: exact
softmax rows of these flat, long attentions are averages of many value rows and so small,
while the estimator's error scales with the value rows themselves; the relative Frobenius
error and the RMS error are printed next to it.)
"""
import sys

import numpy as np
import pytest
import torch

import oracle.favor_oracle as O
from efficient_transformer_attention_favor_amd import api
from efficient_transformer_attention_favor_amd import inputs as I

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _dev(x, dtype):
    return torch.from_numpy(np.ascontiguousarray(x)).to(device="cuda").to(dtype)


def _rows_out(w, Q, K, V, W, rows):
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    y = api.attn_fwd(_dev(Q, dt), _dev(K, dt), _dev(V, dt), _dev(W, torch.float32), causal=w.causal)
    torch.cuda.synchronize()
    got = torch.stack([y[b, h, i] for b, h, i in rows]).float().cpu().numpy()
    del y
    return got


def _iid(w):
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([0, 99] + [ord(c) for c in w.name])))
    return np.stack([I.iid_matrix(w.num_features, w.head_dim, rng) for _ in range(w.heads_w)]).astype(np.float32)


@pytest.mark.parametrize("name", ["c1_bidir_f32", "c2_bidir_bf16", "c3_causal_bf16", "c4_mqa_bidir_bf16",
                                  "c5_causal_long_bf16"])
def test_report_error_vs_softmax(name):
    w = I.workload(name)
    Q, K, V, W = I.make_inputs(w, seed=0)
    if w.batch * w.heads_q * w.seq_len <= 4096:
        rows = np.stack(np.unravel_index(np.arange(w.batch * w.heads_q * w.seq_len),
                                         (w.batch, w.heads_q, w.seq_len)), axis=1)
    else:
        rows = I.sample_rows(w, 256)
    exact = O.softmax_rows(Q, K, V, rows, causal=w.causal)
    res = {}
    for kind, Wk in (("orf", W), ("iid", _iid(w))):
        got = _rows_out(w, Q, K, V, Wk, rows)
        res[kind] = (O.rowwise_rel_err(got, exact), float(np.linalg.norm(got - exact) / np.linalg.norm(exact)),
                     float(np.sqrt(np.mean((got - exact) ** 2))))
    _say(f"  {name}: m={w.num_features}, {len(rows)} rows, exact output RMS {np.sqrt(np.mean(exact ** 2)):.3e}; "
         + "; ".join(f"{k}: row-wise rel {e:.3e}, Frobenius rel {f:.3e}, RMS {r:.3e}" for k, (e, f, r) in res.items()))
    for vals in res.values():
        assert all(np.isfinite(v) for v in vals)


def test_error_falls_with_features_and_orthogonal_rows_help():
    """At low temperature (Q and K scaled by 1/4, so the positive features' variance is
    small) the error against exact softmax falls like 1/sqrt(m) and orthogonal rows beat
    i.i.d. rows (Performer page, "제안 방법" and "주요 결과"), with W drawn on the device."""
    w = I.workload("c2_bidir_bf16").replace(name="approx_low_temp", batch=1, heads_q=4, heads_kv=4, heads_w=4)
    Q, K, V, _ = I.make_inputs(w, seed=0)
    Q, K = I.round_to_bf16(Q * 0.25), I.round_to_bf16(K * 0.25)  # exact in bf16 (power of two)
    rows = I.sample_rows(w, 256)
    exact = O.softmax_rows(Q, K, V, rows)
    q, k, v = (_dev(x, torch.bfloat16) for x in (Q, K, V))
    rms = {}
    for m in (64, 512):
        for orth in (True, False):
            errs = []
            for seed in range(4):
                Wd = api.draw_features(w.heads_w, m, w.head_dim, 100 * m + seed, orth)
                y = api.attn_fwd(q, k, v, Wd)
                got = torch.stack([y[b, h, i] for b, h, i in rows]).float().cpu().numpy()
                errs.append(np.sqrt(np.mean((got - exact) ** 2)))
            rms[(m, orth)] = float(np.mean(errs))
    _say(f"  RMS error vs softmax: {rms}")
    for orth in (True, False):
        assert rms[(512, orth)] < 0.5 * rms[(64, orth)]   # sqrt(8) = 2.8 expected
    assert rms[(64, True)] < rms[(64, False)] and rms[(512, True)] < rms[(512, False)]
