"""ctypes binding of libfavor.so (argument marshalling only).

The shared library is built in-tree next to this file (see ``build.py``).  There is no
fallback: if the library is missing, loading raises.
"""
from __future__ import annotations

import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libfavor.so")

FAVOR_OK = 0
FAVOR_ERR_INVALID_ARG = 1
FAVOR_ERR_UNSUPPORTED = 2
FAVOR_ERR_WORKSPACE = 3
FAVOR_ERR_HIP = 4

FAVOR_F32 = 0
FAVOR_BF16 = 1
FAVOR_BIDIRECTIONAL = 0
FAVOR_CAUSAL = 1

FAVOR_FWD_KERNELS = 3
FAVOR_NOALLOC_SCRATCH_BYTES = 64 << 20
FAVOR_FEATURE_RELU = 1

EXPORTED = ("favor_workspace_bytes", "favor_attn_fwd", "favor_attn_fwd_timed", "favor_features",
            "favor_decode_state_bytes", "favor_attn_decode", "favor_bwd_workspace_bytes", "favor_attn_bwd",
            "favor_draw_features", "favor_generalized_workspace_bytes", "favor_attn_fwd_generalized",
            "favor_decode_prefill_workspace_bytes", "favor_decode_prefill",
            "favor_attn_fwd_noalloc", "favor_attn_fwd_launches", "favor_status_string", "favor_abi_version")


class FavorProblem(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "batch", "heads_q", "heads_kv", "heads_w", "seq_len", "head_dim", "num_features",
        "dtype", "mode", "chunk")]


class FavorError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"{what}: {status_string(status)} (status {status})")
        self.status = status


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded library; raises OSError if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise OSError(f"{LIB_PATH} is missing: build it with "
                          "`python -m efficient_transformer_attention_favor_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        P = ctypes.POINTER(FavorProblem)
        vp = ctypes.c_void_p
        L.favor_workspace_bytes.argtypes = [P]
        L.favor_workspace_bytes.restype = ctypes.c_size_t
        L.favor_attn_fwd_launches.argtypes = [P]
        L.favor_attn_fwd_launches.restype = ctypes.c_int32
        L.favor_attn_fwd.argtypes = [P, vp, vp, vp, vp, vp, vp, ctypes.c_size_t, vp]
        L.favor_attn_fwd.restype = ctypes.c_int
        L.favor_attn_fwd_timed.argtypes = [P, vp, vp, vp, vp, vp, vp, ctypes.c_size_t, vp,
                                           ctypes.POINTER(ctypes.c_void_p), ctypes.c_int32]
        L.favor_attn_fwd_timed.restype = ctypes.c_int
        L.favor_attn_fwd_noalloc.argtypes = [P, vp, vp, vp, vp, vp, vp]
        L.favor_attn_fwd_noalloc.restype = ctypes.c_int
        L.favor_features.argtypes = [P, ctypes.c_int32, vp, vp, vp, vp, vp]
        L.favor_features.restype = ctypes.c_int
        L.favor_decode_state_bytes.argtypes = [P]
        L.favor_decode_state_bytes.restype = ctypes.c_size_t
        L.favor_attn_decode.argtypes = [P, vp, vp, vp, vp, vp, vp, vp]
        L.favor_attn_decode.restype = ctypes.c_int
        L.favor_bwd_workspace_bytes.argtypes = [P]
        L.favor_bwd_workspace_bytes.restype = ctypes.c_size_t
        L.favor_attn_bwd.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_size_t, vp]
        L.favor_attn_bwd.restype = ctypes.c_int
        L.favor_decode_prefill_workspace_bytes.argtypes = [P]
        L.favor_decode_prefill_workspace_bytes.restype = ctypes.c_size_t
        L.favor_decode_prefill.argtypes = [P, vp, vp, vp, vp, vp, ctypes.c_size_t, vp]
        L.favor_decode_prefill.restype = ctypes.c_int
        L.favor_generalized_workspace_bytes.argtypes = [P, ctypes.c_int32]
        L.favor_generalized_workspace_bytes.restype = ctypes.c_size_t
        L.favor_attn_fwd_generalized.argtypes = [P, ctypes.c_int32, vp, vp, vp, vp, vp, vp, ctypes.c_size_t, vp]
        L.favor_attn_fwd_generalized.restype = ctypes.c_int
        L.favor_draw_features.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_uint64,
                                          ctypes.c_int32, vp, vp]
        L.favor_draw_features.restype = ctypes.c_int
        L.favor_status_string.argtypes = [ctypes.c_int]
        L.favor_status_string.restype = ctypes.c_char_p
        L.favor_abi_version.argtypes = []
        L.favor_abi_version.restype = ctypes.c_int32
        _lib = L
    return _lib


def status_string(status: int) -> str:
    return lib().favor_status_string(int(status)).decode()


def problem(batch, heads_q, heads_kv, heads_w, seq_len, head_dim, num_features, dtype, mode,
            chunk=0) -> FavorProblem:
    return FavorProblem(batch, heads_q, heads_kv, heads_w, seq_len, head_dim, num_features,
                        dtype, mode, chunk)


def _ref(p):
    return None if p is None else ctypes.byref(p)


def workspace_bytes(p: FavorProblem) -> int:
    return int(lib().favor_workspace_bytes(_ref(p)))


def attn_fwd_launches(p: FavorProblem) -> int:
    return int(lib().favor_attn_fwd_launches(_ref(p)))


def attn_fwd(p: FavorProblem, q, k, v, w, out, workspace, workspace_nbytes, stream) -> int:
    return int(lib().favor_attn_fwd(_ref(p), q, k, v, w, out, workspace,
                                    ctypes.c_size_t(workspace_nbytes), stream))


def attn_fwd_timed(p: FavorProblem, q, k, v, w, out, workspace, workspace_nbytes, stream,
                   events) -> int:
    arr = (ctypes.c_void_p * len(events))(*events) if events is not None else None
    return int(lib().favor_attn_fwd_timed(_ref(p), q, k, v, w, out, workspace,
                                          ctypes.c_size_t(workspace_nbytes), stream, arr,
                                          0 if events is None else len(events)))


def attn_fwd_noalloc(p: FavorProblem, q, k, v, w, out, stream) -> int:
    return int(lib().favor_attn_fwd_noalloc(_ref(p), q, k, v, w, out, stream))


def features(p: FavorProblem, side, x, w, phi_out, c_out, stream) -> int:
    return int(lib().favor_features(_ref(p), int(side), x, w, phi_out, c_out, stream))


def decode_state_bytes(p: FavorProblem) -> int:
    return int(lib().favor_decode_state_bytes(_ref(p)))


def attn_decode(p: FavorProblem, q, k, v, w, state, out, stream) -> int:
    return int(lib().favor_attn_decode(_ref(p), q, k, v, w, state, out, stream))


def bwd_workspace_bytes(p: FavorProblem) -> int:
    return int(lib().favor_bwd_workspace_bytes(_ref(p)))


def attn_bwd(p: FavorProblem, q, k, v, w, dout, dq, dk, dv, workspace, workspace_nbytes, stream) -> int:
    return int(lib().favor_attn_bwd(_ref(p), q, k, v, w, dout, dq, dk, dv, workspace,
                                    ctypes.c_size_t(workspace_nbytes), stream))


def decode_prefill_workspace_bytes(p: FavorProblem) -> int:
    return lib().favor_decode_prefill_workspace_bytes(_ref(p))


def decode_prefill(p: FavorProblem, k, v, w, state, workspace, workspace_nbytes, stream) -> int:
    return lib().favor_decode_prefill(_ref(p), k, v, w, state, workspace, workspace_nbytes, stream)


def generalized_workspace_bytes(p: FavorProblem, fn) -> int:
    return lib().favor_generalized_workspace_bytes(_ref(p), fn)


def attn_fwd_generalized(p: FavorProblem, fn, q, k, v, w, out, workspace, workspace_nbytes, stream) -> int:
    return lib().favor_attn_fwd_generalized(_ref(p), fn, q, k, v, w, out, workspace, workspace_nbytes, stream)


def draw_features(heads_w, num_features, head_dim, seed, orthogonal, w, stream) -> int:
    return lib().favor_draw_features(heads_w, num_features, head_dim, seed, int(orthogonal), w, stream)


def abi_version() -> int:
    return int(lib().favor_abi_version())
