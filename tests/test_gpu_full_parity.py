"""Full-tensor parity of the benchmark workloads 2-4 with the float64 oracle.

Every output row of the c2 (bidirectional), c3 (causal, at each chunk size) and c4
(multi-query) workloads is compared with ``O.favor_attention`` on the same seeded inputs and
W.  The oracle runs block by block, one (batch, kv head) with its query heads at a time, so
host memory stays bounded; the GPU output is copied to the host once as bf16.  Metric:
row-wise relative error max_i |y_i - r_i|_inf / |r_i|_inf, bar 2e-2 (bf16 inputs, float32
accumulation).  The long causal workload c5 is checked on 256 sampled rows in
``test_gpu_parity.py``.
"""
import sys

import numpy as np
import pytest
import torch

import oracle.favor_oracle as O
from efficient_transformer_attention_favor_amd import api
from efficient_transformer_attention_favor_amd import inputs as I

pytestmark = pytest.mark.gpu

TOL = 2e-2


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _gpu_out(w, Q, K, V, W, chunk=0):
    q, k, v = (torch.from_numpy(x).cuda().to(torch.bfloat16) for x in (Q, K, V))
    y = api.attn_fwd(q, k, v, torch.from_numpy(W).cuda(), causal=w.causal, chunk=chunk)
    torch.cuda.synchronize()
    host = y.cpu()
    del q, k, v, y
    torch.cuda.empty_cache()
    return host


def _blocks(w):
    """(b, kv head, query-head slice, W index) of every block the oracle runs."""
    G = w.heads_q // w.heads_kv
    for b in range(w.batch):
        for hk in range(w.heads_kv):
            yield b, hk, slice(hk * G, (hk + 1) * G), (0 if w.heads_w == 1 else hk)


def _compare(w, Q, K, V, W, outs):
    """Row-wise relative error of each GPU output in `outs` against the oracle, block by block."""
    worst = [0.0] * len(outs)
    for b, hk, hs, wi in _blocks(w):
        ref = O.favor_attention(Q[b:b + 1, hs], K[b:b + 1, hk:hk + 1], V[b:b + 1, hk:hk + 1], W[wi:wi + 1],
                                causal=w.causal)
        for n, y in enumerate(outs):
            got = y[b:b + 1, hs].float().numpy()
            assert np.isfinite(got).all(), (b, hk)
            worst[n] = max(worst[n], O.rowwise_rel_err(got, ref))
    return worst


@pytest.mark.parametrize("name", ["c2_bidir_bf16", "c4_mqa_bidir_bf16"])
def test_full_tensor_bidirectional(name):
    w = I.workload(name)
    _say(f"case {name} full tensor")
    Q, K, V, W = I.make_inputs(w, seed=0)
    y = _gpu_out(w, Q, K, V, W)
    (err,) = _compare(w, Q, K, V, W, [y])
    _say(f"  {name}: row-wise relative error over all {w.batch * w.heads_q * w.seq_len} rows {err:.3e}")
    assert err < TOL


def test_full_tensor_causal_chunks():
    """c3 at the chunk sizes of its sweep (64, 128, 256) and the library default."""
    w = I.workload("c3_causal_bf16")
    chunks = [0, 64, 128, 256]
    _say(f"case c3_causal_bf16 full tensor, chunks {chunks}")
    Q, K, V, W = I.make_inputs(w, seed=0)
    outs = [_gpu_out(w, Q, K, V, W, chunk=c) for c in chunks]
    errs = _compare(w, Q, K, V, W, outs)
    for c, e in zip(chunks, errs):
        _say(f"  c3_causal_bf16 chunk {c}: row-wise relative error over all {w.batch * w.heads_q * w.seq_len} "
             f"rows {e:.3e}")
    assert max(errs) < TOL
