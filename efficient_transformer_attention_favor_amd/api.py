"""Torch-tensor front end of the C ABI.

PyTorch provides device memory and the current stream; every step of the attention
runs in the library's HIP kernels.  Nothing here computes attention.
"""
from __future__ import annotations

import torch

from . import _lib

_DTYPES = {torch.float32: _lib.FAVOR_F32, torch.bfloat16: _lib.FAVOR_BF16}


def _keep_alive(stream, *tensors):
    """Tell the caching allocator that tensors allocated here are used on `stream` (which may
    not be the current stream), so their memory is not handed out again before the queued
    kernels have finished with it."""
    for t in tensors:
        if t is not None:
            t.record_stream(stream)


def _problem(Q, K, W, causal, chunk):
    if Q.dim() != 4 or K.dim() != 4 or W.dim() != 3:
        raise ValueError("expected Q, K, V of shape (B, H, L, d) and W of shape (Hw, m, d)")
    if Q.dtype not in _DTYPES:
        raise ValueError(f"unsupported dtype {Q.dtype}")
    B, Hq, L, d = Q.shape
    return _lib.problem(B, Hq, K.shape[1], W.shape[0], L, d, W.shape[1], _DTYPES[Q.dtype],
                        _lib.FAVOR_CAUSAL if causal else _lib.FAVOR_BIDIRECTIONAL, chunk)


def _check(Q, K, V, W):
    dev = Q.device
    if dev.type != "cuda":
        raise ValueError("tensors must be on the GPU")
    for name, t in (("K", K), ("V", V), ("W", W)):
        if t.device != dev:
            raise ValueError(f"{name} is on {t.device}, Q on {dev}")
    if K.dtype != Q.dtype or V.dtype != Q.dtype:
        raise ValueError("Q, K and V must share one dtype")
    if W.dtype != torch.float32:
        raise ValueError("W must be float32")
    if K.shape != V.shape or K.shape[0] != Q.shape[0] or K.shape[2:] != Q.shape[2:]:
        raise ValueError("K and V must be (B, Hkv, L, d) matching Q")
    if W.shape[2] != Q.shape[3]:
        raise ValueError("W must be (Hw, m, d)")
    for name, t in (("Q", Q), ("K", K), ("V", V), ("W", W)):
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")


def workspace_bytes(Q, K, W, causal=False, chunk=0) -> int:
    return _lib.workspace_bytes(_problem(Q, K, W, causal, chunk))


def attn_fwd(Q, K, V, W, causal=False, chunk=0, out=None, workspace=None, stream=None):
    """FAVOR+ attention forward; returns out (B, Hq, L, d) in Q's dtype."""
    _check(Q, K, V, W)
    p = _problem(Q, K, W, causal, chunk)
    nbytes = _lib.workspace_bytes(p)
    if nbytes == 0:
        st = _lib.attn_fwd(p, None, None, None, None, None, None, 0, None)
        raise _lib.FavorError(st, "favor_attn_fwd")
    own = []
    if out is None:
        out = torch.empty_like(Q)
        own.append(out)
    if workspace is None:
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=Q.device)
        own.append(workspace)
    if stream is None:
        stream = torch.cuda.current_stream(Q.device)
    st = _lib.attn_fwd(p, Q.data_ptr(), K.data_ptr(), V.data_ptr(), W.data_ptr(), out.data_ptr(),
                       workspace.data_ptr(), workspace.numel() * workspace.element_size(),
                       stream.cuda_stream)
    if st != _lib.FAVOR_OK:
        raise _lib.FavorError(st, "favor_attn_fwd")
    _keep_alive(stream, *own)
    return out


def attn_fwd_generalized(Q, K, V, W, fn="relu", causal=False, out=None, workspace=None, stream=None):
    """Kernelised attention D^-1 A V with A = phi(Q) phi(K)^T for the feature map `fn`
    ("relu": phi(x) = ReLU(W x) / sqrt(m)); returns out (B, Hq, L, d) in Q's dtype."""
    fns = {"relu": _lib.FAVOR_FEATURE_RELU}
    if fn not in fns:
        raise ValueError(f"unknown feature map {fn!r}")
    _check(Q, K, V, W)
    p = _problem(Q, K, W, causal, 0)
    nbytes = _lib.generalized_workspace_bytes(p, fns[fn])
    if nbytes == 0:
        st = _lib.attn_fwd_generalized(p, fns[fn], None, None, None, None, None, None, 0, None)
        raise _lib.FavorError(st, "favor_attn_fwd_generalized")
    own = []
    if out is None:
        out = torch.empty_like(Q)
        own.append(out)
    if workspace is None:
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=Q.device)
        own.append(workspace)
    if stream is None:
        stream = torch.cuda.current_stream(Q.device)
    st = _lib.attn_fwd_generalized(p, fns[fn], Q.data_ptr(), K.data_ptr(), V.data_ptr(), W.data_ptr(),
                                   out.data_ptr(), workspace.data_ptr(),
                                   workspace.numel() * workspace.element_size(), stream.cuda_stream)
    if st != _lib.FAVOR_OK:
        raise _lib.FavorError(st, "favor_attn_fwd_generalized")
    _keep_alive(stream, *own)
    return out


def features(X, W, side, heads_q, heads_kv, stream=None):
    """The feature map phi of the queries (side 0) or keys (side 1) of X (B, H, L, d).

    Returns (phi (rows, m) float32, c) with c the natural-log stabiliser per row (side 0)
    or per (batch, kv head) (side 1).
    """
    if X.dim() != 4 or W.dim() != 3 or X.dtype not in _DTYPES or W.dtype != torch.float32:
        raise ValueError("expected X (B, H, L, d) in float32/bfloat16 and W (Hw, m, d) float32")
    if X.device.type != "cuda" or W.device != X.device or not (X.is_contiguous() and W.is_contiguous()):
        raise ValueError("X and W must be contiguous tensors on one GPU")
    B, H, L, d = X.shape
    if side not in (0, 1) or H != (heads_q if side == 0 else heads_kv):
        raise ValueError("side 0 takes X with heads_q heads, side 1 with heads_kv heads")
    m = W.shape[1]
    dtype = _DTYPES[X.dtype]
    p = _lib.problem(B, heads_q, heads_kv, W.shape[0], L, d, m, dtype, _lib.FAVOR_BIDIRECTIONAL)
    rows = B * H * L
    phi = torch.empty((rows, m), dtype=torch.float32, device=X.device)
    c = torch.empty((rows if side == 0 else B * heads_kv,), dtype=torch.float32, device=X.device)
    if stream is None:
        stream = torch.cuda.current_stream(X.device)
    st = _lib.features(p, side, X.data_ptr(), W.data_ptr(), phi.data_ptr(), c.data_ptr(),
                       stream.cuda_stream)
    if st != _lib.FAVOR_OK:
        raise _lib.FavorError(st, "favor_features")
    _keep_alive(stream, phi, c)
    return phi, c


def _decode_problem(q, k, W):
    if q.dim() != 3 or k.dim() != 3 or W.dim() != 3 or q.dtype not in _DTYPES:
        raise ValueError("expected q (B, Hq, d), k and v (B, Hkv, d) in float32/bfloat16, W (Hw, m, d)")
    B, Hq, d = q.shape
    return _lib.problem(B, Hq, k.shape[1], W.shape[0], 1, d, W.shape[1], _DTYPES[q.dtype],
                        _lib.FAVOR_CAUSAL, 0)


def decode_state(q, k, W):
    """A zero (empty) decoding state for queries like q (B, Hq, d) and keys like k (B, Hkv, d)."""
    nbytes = _lib.decode_state_bytes(_decode_problem(q, k, W))
    if nbytes == 0:
        raise ValueError("unsupported decoding problem")
    return torch.zeros(nbytes // 4, dtype=torch.float32, device=q.device)


def decode_prefill(K, V, W, heads_q, state=None, stream=None):
    """The decoding state after the prompt K, V (B, Hkv, L, d): favor_decode_prefill.  Returns
    the state (float32, the layout of decode_state), ready for attn_decode."""
    if K.dim() != 4 or V.shape != K.shape or K.dtype not in _DTYPES or V.dtype != K.dtype:
        raise ValueError("expected K, V (B, Hkv, L, d) of one dtype (float32/bfloat16)")
    if W.dtype != torch.float32 or W.dim() != 3 or any(not t.is_contiguous() for t in (K, V, W)):
        raise ValueError("W must be a contiguous float32 (Hw, m, d); K, V contiguous")
    B, Hkv, L, d = K.shape
    p = _lib.problem(B, heads_q, Hkv, W.shape[0], L, d, W.shape[1], _DTYPES[K.dtype], _lib.FAVOR_CAUSAL, 0)
    one = _lib.problem(B, heads_q, Hkv, W.shape[0], 1, d, W.shape[1], _DTYPES[K.dtype], _lib.FAVOR_CAUSAL, 0)
    nbytes, sbytes = _lib.decode_prefill_workspace_bytes(p), _lib.decode_state_bytes(one)
    if nbytes == 0 or sbytes == 0:
        raise ValueError("unsupported prefill problem")
    own = []
    if state is None:
        state = torch.empty(sbytes // 4, dtype=torch.float32, device=K.device)
        own.append(state)
    elif state.dtype != torch.float32 or state.numel() * 4 < sbytes or not state.is_contiguous():
        raise ValueError("state must be a contiguous float32 tensor of favor_decode_state_bytes()")
    ws = torch.empty(nbytes, dtype=torch.uint8, device=K.device)
    if stream is None:
        stream = torch.cuda.current_stream(K.device)
    st = _lib.decode_prefill(p, K.data_ptr(), V.data_ptr(), W.data_ptr(), state.data_ptr(), ws.data_ptr(), nbytes,
                             stream.cuda_stream)
    if st != _lib.FAVOR_OK:
        raise _lib.FavorError(st, "favor_decode_prefill")
    _keep_alive(stream, ws, *own)
    return state


def attn_decode(q, k, v, W, state, out=None, stream=None):
    """One causal decoding step: adds position (k, v) to `state` (from decode_state, updated
    in place) and returns out (B, Hq, d) = the new position's attention output."""
    if q.device.type != "cuda" or any(t.device != q.device for t in (k, v, W, state)):
        raise ValueError("tensors must be on one GPU")
    if k.dtype != q.dtype or v.dtype != q.dtype or W.dtype != torch.float32 or state.dtype != torch.float32:
        raise ValueError("q, k, v share one dtype; W and the state are float32")
    if k.shape != v.shape or k.shape[0] != q.shape[0] or k.shape[2] != q.shape[2] or W.shape[2] != q.shape[2]:
        raise ValueError("k and v must be (B, Hkv, d) matching q, W (Hw, m, d)")
    for name, t in (("q", q), ("k", k), ("v", v), ("W", W), ("state", state)):
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    p = _decode_problem(q, k, W)
    if state.numel() * 4 < _lib.decode_state_bytes(p):
        raise ValueError("state is smaller than favor_decode_state_bytes()")
    own = []
    if out is None:
        out = torch.empty_like(q)
        own.append(out)
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    st = _lib.attn_decode(p, q.data_ptr(), k.data_ptr(), v.data_ptr(), W.data_ptr(), state.data_ptr(),
                          out.data_ptr(), stream.cuda_stream)
    if st != _lib.FAVOR_OK:
        raise _lib.FavorError(st, "favor_attn_decode")
    _keep_alive(stream, *own)
    return out


def attn_bwd(Q, K, V, W, dout, causal=False, workspace=None, stream=None):
    """Gradients (dQ, dK, dV) of sum(dout * attn_fwd(Q, K, V, W, causal)); W fixed."""
    _check(Q, K, V, W)
    if dout.shape != Q.shape or dout.dtype != Q.dtype or dout.device != Q.device or not dout.is_contiguous():
        raise ValueError("dout must be a contiguous tensor like Q")
    p = _problem(Q, K, W, causal, 0)
    nbytes = _lib.bwd_workspace_bytes(p)
    if nbytes == 0:
        st = _lib.attn_bwd(p, None, None, None, None, None, None, None, None, None, 0, None)
        raise _lib.FavorError(st, "favor_attn_bwd")
    own = []
    if workspace is None:
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=Q.device)
        own.append(workspace)
    if stream is None:
        stream = torch.cuda.current_stream(Q.device)
    dQ, dK, dV = torch.empty_like(Q), torch.empty_like(K), torch.empty_like(V)
    st = _lib.attn_bwd(p, Q.data_ptr(), K.data_ptr(), V.data_ptr(), W.data_ptr(), dout.data_ptr(), dQ.data_ptr(),
                       dK.data_ptr(), dV.data_ptr(), workspace.data_ptr(),
                       workspace.numel() * workspace.element_size(), stream.cuda_stream)
    if st != _lib.FAVOR_OK:
        raise _lib.FavorError(st, "favor_attn_bwd")
    _keep_alive(stream, dQ, dK, dV, *own)
    return dQ, dK, dV


def draw_features(heads_w, num_features, head_dim, seed, orthogonal=True, device="cuda", stream=None):
    """W [heads_w][num_features][head_dim] float32 drawn on the device from `seed`
    (orthogonal random features, or i.i.d. Gaussian rows with orthogonal=False)."""
    W = torch.empty((heads_w, num_features, head_dim), dtype=torch.float32, device=device)
    if stream is None:
        stream = torch.cuda.current_stream(W.device)
    st = _lib.draw_features(heads_w, num_features, head_dim, int(seed), orthogonal, W.data_ptr(), stream.cuda_stream)
    if st != _lib.FAVOR_OK:
        raise _lib.FavorError(st, "favor_draw_features")
    _keep_alive(stream, W)
    return W


class _FavorAttention(torch.autograd.Function):
    """favor_attn_fwd forward, favor_attn_bwd backward (W is a fixed input: no gradient)."""

    @staticmethod
    def forward(ctx, Q, K, V, W, causal):
        ctx.causal = causal
        ctx.save_for_backward(Q, K, V, W)
        return attn_fwd(Q, K, V, W, causal=causal)

    @staticmethod
    def backward(ctx, dout):
        Q, K, V, W = ctx.saved_tensors
        dQ, dK, dV = attn_bwd(Q, K, V, W, dout.contiguous(), causal=ctx.causal)
        return dQ, dK, dV, None, None


def favor_attention(Q, K, V, W, causal=False):
    """FAVOR+ attention as a differentiable op: out = attn_fwd(Q, K, V, W, causal), with the
    gradients of Q, K and V from favor_attn_bwd (W gets none)."""
    return _FavorAttention.apply(Q, K, V, W, causal)
