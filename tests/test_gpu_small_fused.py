"""Float32 bidirectional problems small enough to run as one launch (key-side units, a
grid-wide barrier on a tagged word in the workspace, then the readout), against the float64
oracle at the float32 bar (row-wise relative error 1e-4), and against themselves: repeated
calls on one workspace, a workspace holding arbitrary bytes, and graph replays (one launch
tag baked into the graph) must all give the same bits."""
import sys

import numpy as np
import pytest
import torch

import oracle.favor_oracle as O
from efficient_transformer_attention_favor_amd import _lib, api
from efficient_transformer_attention_favor_amd import inputs as I

pytestmark = pytest.mark.gpu

TOL = 1e-4


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _dev(x, dtype=torch.float32):
    return torch.from_numpy(np.ascontiguousarray(x)).to(device="cuda").to(dtype)


def _w(**kw):
    return I.workload("c1_bidir_f32").replace(name="c1_fused", **kw)


CASES = [
    _w(),                                                                    # c1 itself
    _w(seq_len=1),                                                           # one position
    _w(seq_len=200),                                                         # ragged tail
    _w(num_features=64, seq_len=300),                                        # two feature tiles: idle readout waves
    _w(num_features=320, seq_len=150),                                       # tiles beyond the waves
    _w(batch=2, heads_q=8, heads_kv=2, heads_w=1, seq_len=97),              # MQA groups, shared W
    _w(batch=1, heads_q=3, heads_kv=3, heads_w=3, seq_len=513, head_dim=128),
]


@pytest.mark.parametrize("w", CASES, ids=lambda w: f"B{w.batch}Hq{w.heads_q}Hkv{w.heads_kv}L{w.seq_len}d{w.head_dim}m{w.num_features}")
def test_one_launch_matches_oracle(w):
    Q, K, V, W = I.make_inputs(w, seed=3)
    q, k, v, wd = _dev(Q), _dev(K), _dev(V), _dev(W)
    p = api._problem(q, k, wd, False, 0)
    assert _lib.attn_fwd_launches(p) == 1
    _say(f"one launch {w}")
    out = api.attn_fwd(q, k, v, wd)
    torch.cuda.synchronize()
    err = O.rowwise_rel_err(out.cpu().numpy(), O.favor_attention(Q, K, V, W))
    _say(f"  row-wise relative error {err:.2e}")
    assert np.isfinite(out.cpu().numpy()).all() and err < TOL


def test_two_launches_past_the_limit():
    """More 32-row tiles than compute units: the key side and the readout as two kernels."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    L = 32 * (cus + 1)
    w = _w(seq_len=L, num_features=64)
    Q, K, V, W = I.make_inputs(w, seed=4)
    q, k, v, wd = _dev(Q), _dev(K), _dev(V), _dev(W)
    assert _lib.attn_fwd_launches(api._problem(q, k, wd, False, 0)) == 2
    _say(f"two launches, L = {L}")
    out = api.attn_fwd(q, k, v, wd)
    torch.cuda.synchronize()
    err = O.rowwise_rel_err(out.cpu().numpy(), O.favor_attention(Q, K, V, W))
    _say(f"  row-wise relative error {err:.2e}")
    assert err < TOL


def test_repeated_calls_and_stale_workspace_agree():
    """Back-to-back calls on one workspace (each a new barrier tag), then a workspace filled
    with arbitrary bytes (the barrier word included): every output has the same bits."""
    w = _w()
    Q, K, V, W = I.make_inputs(w, seed=5)
    q, k, v, wd = _dev(Q), _dev(K), _dev(V), _dev(W)
    p = api._problem(q, k, wd, False, 0)
    ws = torch.empty(_lib.workspace_bytes(p), dtype=torch.uint8, device="cuda")
    first = api.attn_fwd(q, k, v, wd, workspace=ws).clone()
    outs = [api.attn_fwd(q, k, v, wd, workspace=ws).clone() for _ in range(5)]
    torch.cuda.synchronize()
    for i, o in enumerate(outs):
        assert torch.equal(o, first), i
    for fill in (0, 255, 7):
        ws.fill_(fill)
        o = api.attn_fwd(q, k, v, wd, workspace=ws)
        torch.cuda.synchronize()
        _say(f"  workspace filled with {fill}: equal {torch.equal(o, first)}")
        assert torch.equal(o, first)
    ws.copy_(torch.randint(0, 256, ws.shape, dtype=torch.uint8, device="cuda"))
    o = api.attn_fwd(q, k, v, wd, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(o, first)
    err = O.rowwise_rel_err(first.cpu().numpy(), O.favor_attention(Q, K, V, W))
    assert err < TOL


def test_one_launch_graph_replays_match_eager():
    """A captured call keeps its launch tag on every replay: the barrier word left complete
    by one replay must start a new count on the next."""
    w = _w(batch=1, heads_q=2, heads_kv=1, heads_w=1, seq_len=400)
    Q, K, V, W = I.make_inputs(w, seed=6)
    q, k, v, wd = _dev(Q), _dev(K), _dev(V), _dev(W)
    p = api._problem(q, k, wd, False, 0)
    assert _lib.attn_fwd_launches(p) == 1
    ws = torch.empty(_lib.workspace_bytes(p), dtype=torch.uint8, device="cuda")
    out = torch.empty_like(q)
    eager = api.attn_fwd(q, k, v, wd, workspace=ws).clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        api.attn_fwd(q, k, v, wd, out=out, workspace=ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        api.attn_fwd(q, k, v, wd, out=out, workspace=ws)
    for i in range(4):
        out.fill_(7.0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        _say(f"  replay {i}: equal {torch.equal(out, eager)}")
        assert torch.equal(out, eager)
        other = api.attn_fwd(q, v, k, wd, workspace=ws)  # eager work on the same workspace in between
        torch.cuda.synchronize()
        del other


def test_barrier_that_gives_up_writes_nan_rows(monkeypatch):
    """The barrier's wait is bounded.  With the poll limit forced to zero from the host
    (FAVOR_BARRIER_POLLS_FOR_TESTS), workgroups that reach the barrier before the others give
    up at once: the kernel still finishes, and every output row is either all NaN (its
    workgroup gave up) or correct -- never silently wrong.  The next call on the same
    workspace, with the limit restored, is correct again."""
    w = _w()
    Q, K, V, W = I.make_inputs(w, seed=7)
    q, k, v, wd = _dev(Q), _dev(K), _dev(V), _dev(W)
    p = api._problem(q, k, wd, False, 0)
    assert _lib.attn_fwd_launches(p) == 1
    ws = torch.empty(_lib.workspace_bytes(p), dtype=torch.uint8, device="cuda")
    ref = O.favor_attention(Q, K, V, W)[0, 0]
    monkeypatch.setenv("FAVOR_BARRIER_POLLS_FOR_TESTS", "0")
    y = api.attn_fwd(q, k, v, wd, workspace=ws).cpu().numpy()[0, 0]
    torch.cuda.synchronize()
    nan_rows = np.isnan(y).all(axis=1)
    _say(f"  poll limit 0: {int(nan_rows.sum())} of {len(nan_rows)} rows NaN")
    assert nan_rows.any()  # the workgroups without a key-side unit arrive first and give up
    assert not np.isnan(y[~nan_rows]).any()
    if (~nan_rows).any():
        assert O.rowwise_rel_err(y[~nan_rows], ref[~nan_rows]) < TOL
    monkeypatch.delenv("FAVOR_BARRIER_POLLS_FOR_TESTS")
    y2 = api.attn_fwd(q, k, v, wd, workspace=ws).cpu().numpy()[0, 0]
    torch.cuda.synchronize()
    assert np.isfinite(y2).all() and O.rowwise_rel_err(y2, ref) < TOL
