"""C ABI: the library loads, exports what include/favor.h declares, and rejects bad
arguments before touching the GPU (these calls never reach a HIP API)."""
import ctypes
import os
import re

import pytest

from efficient_transformer_attention_favor_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_symbols():
    text = open(os.path.join(ROOT, "include", "favor.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(favor_[a-z_]+)\s*\(", text)))


def test_header_declares_the_binding_exports():
    assert _declared_symbols() == sorted(_lib.EXPORTED)


def test_library_exports_every_declared_symbol():
    L = _lib.lib()
    for name in _declared_symbols():
        assert hasattr(L, name), name
    assert _lib.abi_version() == 1


def _p(**kw):
    base = dict(batch=2, heads_q=4, heads_kv=2, heads_w=2, seq_len=100, head_dim=64,
                num_features=128, dtype=_lib.FAVOR_BF16, mode=_lib.FAVOR_BIDIRECTIONAL, chunk=0)
    base.update(kw)
    return _lib.problem(**base)


BAD = [
    (dict(batch=0), _lib.FAVOR_ERR_INVALID_ARG),
    (dict(seq_len=0), _lib.FAVOR_ERR_INVALID_ARG),
    (dict(heads_q=3), _lib.FAVOR_ERR_INVALID_ARG),          # not a multiple of heads_kv
    (dict(heads_w=3), _lib.FAVOR_ERR_INVALID_ARG),          # neither 1 nor heads_kv
    (dict(head_dim=32), _lib.FAVOR_ERR_UNSUPPORTED),
    (dict(head_dim=96), _lib.FAVOR_ERR_UNSUPPORTED),
    (dict(num_features=96), _lib.FAVOR_ERR_UNSUPPORTED),
    (dict(num_features=576), _lib.FAVOR_ERR_UNSUPPORTED),
    (dict(dtype=7), _lib.FAVOR_ERR_UNSUPPORTED),
    (dict(mode=2), _lib.FAVOR_ERR_UNSUPPORTED),
    (dict(mode=_lib.FAVOR_CAUSAL, chunk=48), _lib.FAVOR_ERR_UNSUPPORTED),
    # intra-chunk blocks above 32 positions: bf16 d = 64 only, 256 up to m = 256
    (dict(mode=_lib.FAVOR_CAUSAL, chunk=64, head_dim=128), _lib.FAVOR_ERR_UNSUPPORTED),
    (dict(mode=_lib.FAVOR_CAUSAL, chunk=128, dtype=_lib.FAVOR_F32), _lib.FAVOR_ERR_UNSUPPORTED),
    (dict(mode=_lib.FAVOR_CAUSAL, chunk=256, num_features=320), _lib.FAVOR_ERR_UNSUPPORTED),
    (dict(batch=1 << 12, heads_q=1 << 8, heads_kv=1 << 8, heads_w=1, seq_len=1 << 14),
     _lib.FAVOR_ERR_UNSUPPORTED),                           # more than 2^31 elements
    (dict(batch=1 << 12, heads_q=1 << 4, heads_kv=1 << 4, heads_w=1, seq_len=1),
     _lib.FAVOR_ERR_UNSUPPORTED),                           # more than 65535 (batch, head) pairs
    (dict(batch=1, heads_q=1, heads_kv=1, heads_w=1, seq_len=1 << 24, head_dim=64),
     _lib.FAVOR_ERR_UNSUPPORTED),                           # one bf16 head of 2^31 bytes
]


GOOD_CAUSAL_CHUNKS = [
    dict(chunk=0, head_dim=128), dict(chunk=32, dtype=_lib.FAVOR_F32), dict(chunk=64),
    dict(chunk=128, num_features=512), dict(chunk=256, num_features=256),
]


@pytest.mark.parametrize("kw", GOOD_CAUSAL_CHUNKS)
def test_causal_chunk_values_accepted(kw):
    assert _lib.workspace_bytes(_p(mode=_lib.FAVOR_CAUSAL, **kw)) > 0


@pytest.mark.parametrize("kw,status", BAD)
def test_invalid_problems_rejected(kw, status):
    p = _p(**kw)
    assert _lib.workspace_bytes(p) == 0
    assert _lib.attn_fwd(p, 8, 8, 8, 8, 8, 256, 1 << 30, None) == status
    assert _lib.features(p, 0, 8, 8, 8, 8, None) == status


def test_null_pointers_and_workspace():
    p = _p()
    need = _lib.workspace_bytes(p)
    assert need > 0 and need % 256 == 0
    assert _lib.attn_fwd(p, None, 8, 8, 8, 8, 256, need, None) == _lib.FAVOR_ERR_INVALID_ARG
    assert _lib.attn_fwd(p, 8, 8, 8, 8, None, 256, need, None) == _lib.FAVOR_ERR_INVALID_ARG
    assert _lib.attn_fwd(p, 8, 8, 8, 8, 8, None, need, None) == _lib.FAVOR_ERR_WORKSPACE
    assert _lib.attn_fwd(p, 8, 8, 8, 8, 8, 256, need - 1, None) == _lib.FAVOR_ERR_WORKSPACE
    assert _lib.attn_fwd(p, 8, 8, 8, 8, 8, 260, need, None) == _lib.FAVOR_ERR_WORKSPACE  # misaligned
    assert _lib.features(p, 2, 8, 8, 8, 8, None) == _lib.FAVOR_ERR_INVALID_ARG
    assert _lib.features(p, 0, None, 8, 8, 8, None) == _lib.FAVOR_ERR_INVALID_ARG
    assert _lib.attn_fwd(None, 8, 8, 8, 8, 8, 256, need, None) == _lib.FAVOR_ERR_INVALID_ARG


def test_workspace_grows_with_problem():
    small = _lib.workspace_bytes(_p(seq_len=64))
    big = _lib.workspace_bytes(_p(seq_len=8192))
    causal = _lib.workspace_bytes(_p(mode=_lib.FAVOR_CAUSAL, seq_len=8192, chunk=64))
    assert 0 < small <= big and causal > 0


@pytest.mark.parametrize("m", [320, 512])
def test_causal_wide_head_workspace_holds_row_partials(m):
    """Causal d = 128 with m > 256 runs its chunk kernel as two launches over feature ranges,
    the first writing a float32 partial of d + 4 values per output row: the workspace must
    hold those B Hq L rows besides the segment summaries and their prefixes."""
    # 16 query heads on one kv head: the summaries of one segment are small next to the
    # row partials, so a layout without them falls short
    B, Hq, Hkv, L, d = 2, 16, 1, 1000, 128
    p = _p(batch=B, heads_q=Hq, heads_kv=Hkv, heads_w=Hkv, seq_len=L, head_dim=d, num_features=m,
           mode=_lib.FAVOR_CAUSAL, chunk=0)
    partials = 4 * B * Hq * L * (d + 4)
    one_segment = 4 * (d + 1) * m * B * Hkv  # summaries (and again prefixes) of one segment
    assert 2 * 4 * one_segment + 64 * 1024 < partials
    assert _lib.workspace_bytes(p) >= partials + 2 * one_segment


def test_status_strings():
    for s in range(5):
        assert isinstance(_lib.status_string(s), str) and _lib.status_string(s)
    assert _lib.status_string(99) == "unknown status"


def test_decode_validation():
    """favor_attn_decode takes causal problems of one position; its state size is the
    summaries [B*Hkv][m][d+1] plus a stabiliser and a count per slice of m/8 features,
    256-byte aligned."""
    p = _p(mode=_lib.FAVOR_CAUSAL, seq_len=1, chunk=48)  # the chunk is ignored when decoding
    n = _lib.decode_state_bytes(p)
    assert n == ((2 * 2 * 128 * 65 + 2 * 2 * 8 * 2) * 4 + 255) // 256 * 256
    assert _lib.decode_state_bytes(_p(seq_len=1)) == 0                       # bidirectional
    assert _lib.decode_state_bytes(_p(mode=_lib.FAVOR_CAUSAL, seq_len=2)) == 0
    assert _lib.attn_decode(_p(seq_len=1), 8, 8, 8, 8, 256, 8, None) == _lib.FAVOR_ERR_INVALID_ARG
    assert _lib.attn_decode(_p(mode=_lib.FAVOR_CAUSAL, seq_len=3), 8, 8, 8, 8, 256, 8, None) == \
        _lib.FAVOR_ERR_INVALID_ARG
    assert _lib.attn_decode(_p(mode=_lib.FAVOR_CAUSAL, seq_len=1, head_dim=32), 8, 8, 8, 8, 256, 8, None) == \
        _lib.FAVOR_ERR_UNSUPPORTED
    for i in range(6):
        args = [8, 8, 8, 8, 256, 8]
        args[i] = None
        assert _lib.attn_decode(p, *args, None) == _lib.FAVOR_ERR_INVALID_ARG
    assert _lib.attn_decode(None, 8, 8, 8, 8, 256, 8, None) == _lib.FAVOR_ERR_INVALID_ARG


def test_backward_validation():
    p = _p()
    need = _lib.bwd_workspace_bytes(p)
    assert need > 0 and need % 256 == 0
    causal = _p(mode=_lib.FAVOR_CAUSAL)
    cneed = _lib.bwd_workspace_bytes(causal)
    assert cneed > need and cneed % 256 == 0
    assert _lib.attn_bwd(causal, *([8] * 8), 256, cneed - 1, None) == _lib.FAVOR_ERR_WORKSPACE
    assert _lib.bwd_workspace_bytes(_p(head_dim=32)) == 0
    assert _lib.attn_bwd(_p(head_dim=32), *([8] * 8), 256, need, None) == _lib.FAVOR_ERR_UNSUPPORTED
    assert _lib.attn_bwd(_p(mode=_lib.FAVOR_CAUSAL, chunk=48), *([8] * 8), 256, cneed, None) == \
        _lib.FAVOR_ERR_UNSUPPORTED
    assert _lib.attn_bwd(None, *([8] * 8), 256, need, None) == _lib.FAVOR_ERR_INVALID_ARG
    for i in range(8):
        args = [8] * 8
        args[i] = None
        assert _lib.attn_bwd(p, *args, 256, need, None) == _lib.FAVOR_ERR_INVALID_ARG
    assert _lib.attn_bwd(p, *([8] * 8), None, need, None) == _lib.FAVOR_ERR_WORKSPACE
    assert _lib.attn_bwd(p, *([8] * 8), 256, need - 1, None) == _lib.FAVOR_ERR_WORKSPACE
    assert _lib.attn_bwd(p, *([8] * 8), 260, need, None) == _lib.FAVOR_ERR_WORKSPACE
    assert _lib.bwd_workspace_bytes(_p(seq_len=4096)) > need


def test_draw_features_validation():
    L = _lib
    assert L.draw_features(1, 64, 64, 0, True, None, None) == L.FAVOR_ERR_INVALID_ARG
    assert L.draw_features(0, 64, 64, 0, True, 256, None) == L.FAVOR_ERR_INVALID_ARG
    assert L.draw_features(1, 0, 64, 0, True, 256, None) == L.FAVOR_ERR_INVALID_ARG
    assert L.draw_features(1, 64, 0, 0, True, 256, None) == L.FAVOR_ERR_INVALID_ARG
    assert L.draw_features(1, 64, 64, 0, 2, 256, None) == L.FAVOR_ERR_INVALID_ARG
    assert L.draw_features(1, 64, 129, 0, True, 256, None) == L.FAVOR_ERR_UNSUPPORTED
    assert L.draw_features(65537, 64, 64, 0, True, 256, None) == L.FAVOR_ERR_INVALID_ARG


def test_generalized_validation():
    L = _lib
    p = _p()
    need = L.generalized_workspace_bytes(p, L.FAVOR_FEATURE_RELU)
    assert need > 0 and need % 256 == 0
    assert L.generalized_workspace_bytes(p, 0) == 0 and L.generalized_workspace_bytes(p, 7) == 0
    causal = _p(mode=L.FAVOR_CAUSAL)
    assert L.generalized_workspace_bytes(causal, L.FAVOR_FEATURE_RELU) > 0
    assert L.attn_fwd_generalized(p, 0, 8, 8, 8, 8, 8, 256, need, None) == L.FAVOR_ERR_UNSUPPORTED
    assert L.attn_fwd_generalized(None, 1, 8, 8, 8, 8, 8, 256, need, None) == L.FAVOR_ERR_INVALID_ARG
    for i in range(5):
        args = [8] * 5
        args[i] = None
        assert L.attn_fwd_generalized(p, 1, *args, 256, need, None) == L.FAVOR_ERR_INVALID_ARG
    assert L.attn_fwd_generalized(p, 1, *([8] * 5), 256, need - 1, None) == L.FAVOR_ERR_WORKSPACE
    assert L.attn_fwd_generalized(p, 1, *([8] * 5), 260, need, None) == L.FAVOR_ERR_WORKSPACE
    assert L.attn_fwd_generalized(_p(head_dim=32), 1, *([8] * 5), 256, need, None) == L.FAVOR_ERR_UNSUPPORTED


def test_decode_prefill_validation():
    L = _lib
    causal = _p(mode=L.FAVOR_CAUSAL, seq_len=300)
    need = L.decode_prefill_workspace_bytes(causal)
    assert need > 0 and need % 256 == 0
    assert L.decode_prefill_workspace_bytes(_p(seq_len=300)) == 0            # bidirectional
    assert L.decode_prefill(_p(seq_len=300), 8, 8, 8, 256, 256, need, None) == L.FAVOR_ERR_INVALID_ARG
    assert L.decode_prefill(None, 8, 8, 8, 256, 256, need, None) == L.FAVOR_ERR_INVALID_ARG
    for i in range(4):
        args = [8, 8, 8, 256]
        args[i] = None
        assert L.decode_prefill(causal, *args, 256, need, None) == L.FAVOR_ERR_INVALID_ARG
    assert L.decode_prefill(causal, 8, 8, 8, 256, 256, need - 1, None) == L.FAVOR_ERR_WORKSPACE
    assert L.decode_prefill(causal, 8, 8, 8, 256, None, need, None) == L.FAVOR_ERR_WORKSPACE
    assert L.decode_prefill(_p(mode=L.FAVOR_CAUSAL, head_dim=32), 8, 8, 8, 256, 256, need, None) == \
        L.FAVOR_ERR_UNSUPPORTED


def test_noalloc_rejects_before_any_hip_call():
    """favor_attn_fwd_noalloc validates the problem, the pointers and the scratch limit before
    it touches the GPU (these calls return without a device)."""
    ok = _p()
    fake = 256  # never dereferenced: every call below fails validation first
    assert _lib.attn_fwd_noalloc(_p(batch=0), fake, fake, fake, fake, fake, None) == _lib.FAVOR_ERR_INVALID_ARG
    assert _lib.attn_fwd_noalloc(_p(head_dim=32), fake, fake, fake, fake, fake, None) == _lib.FAVOR_ERR_UNSUPPORTED
    assert _lib.attn_fwd_noalloc(ok, None, fake, fake, fake, fake, None) == _lib.FAVOR_ERR_INVALID_ARG
    assert _lib.attn_fwd_noalloc(ok, fake, fake, fake, fake, None, None) == _lib.FAVOR_ERR_INVALID_ARG
    # a problem whose workspace is larger than the library's scratch array
    big = _p(batch=64, heads_q=16, heads_kv=16, heads_w=1, seq_len=8192, num_features=512,
             mode=_lib.FAVOR_CAUSAL)
    assert _lib.workspace_bytes(big) > _lib.FAVOR_NOALLOC_SCRATCH_BYTES
    assert _lib.attn_fwd_noalloc(big, fake, fake, fake, fake, fake, None) == _lib.FAVOR_ERR_WORKSPACE


def test_fwd_launch_count_query():
    """favor_attn_fwd_launches: 0 for an invalid problem, 4 / 6 kernels for causal problems,
    1 or 2 for float32 bidirectional ones (1 only where a device reports enough compute
    units), 2 for bf16 bidirectional ones."""
    assert _lib.attn_fwd_launches(None) == 0
    assert _lib.attn_fwd_launches(_p(head_dim=32)) == 0
    assert _lib.attn_fwd_launches(_p(mode=_lib.FAVOR_CAUSAL)) == 4
    assert _lib.attn_fwd_launches(_p(mode=_lib.FAVOR_CAUSAL, head_dim=128, num_features=384)) == 6
    assert _lib.attn_fwd_launches(_p(dtype=_lib.FAVOR_BF16)) == 2
    assert _lib.attn_fwd_launches(_p(dtype=_lib.FAVOR_F32, seq_len=1024)) in (1, 2)
