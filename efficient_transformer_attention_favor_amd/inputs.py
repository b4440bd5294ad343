"""Seeded synthetic inputs for FAVOR+ attention: Q, K, V and the random-feature matrix W.

This module holds input generation only -- none of the attention arithmetic.  The
library takes W as a host-generated input, so a caller needs a generator for it; the
test-suite and the benchmark draw the same seeded inputs for the HIP path and for the
CPU oracle from here.

W follows the orthogonal random features of "Rethinking Attention with Performers"
(section "제안 방법", orthogonal random features, ORF): per block of d rows, a d x d
standard Gaussian matrix whose rows are orthonormalised by Gram-Schmidt and then each
rescaled by a chi(d)-distributed length, so that every row is marginally N(0, I_d) while
rows inside one block are exactly orthogonal.  The pages name the construction but not
its details; the reading taken here (modified Gram-Schmidt, rows in order; each row
rescaled by the length of the same row of the block's original Gaussian matrix, which is
chi(d) and independent of the orthonormalised direction) is recorded with the other
readings of the pages in the design notes.

Q, K ~ N(0,1) * d^(-1/4) and V ~ N(0,1), drawn in float32 and rounded to the device
dtype with round-to-nearest-even; the arrays returned hold exactly the device values.
"""
from __future__ import annotations

import dataclasses
import numpy as np

__all__ = [
    "Workload",
    "WORKLOADS",
    "orf_matrix",
    "iid_matrix",
    "round_to_bf16",
    "make_inputs",
    "workload",
]


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even); returns float32 holding bf16 values."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    bits = x.view(np.uint32)
    rounding = ((bits >> 16) & np.uint32(1)) + np.uint32(0x7FFF)
    out = ((bits + rounding) & np.uint32(0xFFFF0000)).astype(np.uint32)
    return out.view(np.float32)


def orf_matrix(m: int, d: int, rng: np.random.Generator) -> np.ndarray:
    """Orthogonal random feature matrix W of shape (m, d), float64.

    ceil(m/d) independent blocks; block rows are orthonormalised by modified Gram-Schmidt
    (in row order) and rescaled by the lengths of the original Gaussian rows.  The last
    block is truncated when d does not divide m.
    """
    blocks = []
    for _ in range((m + d - 1) // d):
        g = rng.standard_normal((d, d))
        lengths = np.sqrt(np.sum(g * g, axis=1))
        q = g.copy()
        for i in range(d):
            for j in range(i):
                q[i] -= np.dot(q[i], q[j]) * q[j]
            q[i] /= np.sqrt(np.dot(q[i], q[i]))
        blocks.append(q * lengths[:, None])
    return np.concatenate(blocks, axis=0)[:m]


def iid_matrix(m: int, d: int, rng: np.random.Generator) -> np.ndarray:
    """Unstructured Gaussian feature matrix (rows i.i.d. N(0, I_d)), float64."""
    return rng.standard_normal((m, d))


@dataclasses.dataclass(frozen=True)
class Workload:
    """Shape, dtype, mode and distribution recipe of one synthetic FAVOR+ workload."""

    name: str
    batch: int
    heads_q: int
    heads_kv: int
    heads_w: int
    seq_len: int
    head_dim: int
    num_features: int
    dtype: str  # "f32" or "bf16"
    causal: bool
    heavy_fraction: float = 0.0  # fraction of Q/K rows scaled by heavy_scale
    heavy_scale: float = 3.0
    sampled_rows: int = 0  # >0: parity on this many sampled output rows

    @property
    def tokens(self) -> int:
        return self.batch * self.heads_q * self.seq_len

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


# The five synthetic workloads (sizes, dtypes, layouts and distributions of the
# benchmark configurations).  W is redrawn per kv-head index where heads_w == heads_kv,
# shared by all heads where heads_w == 1.
WORKLOADS = {
    "c1_bidir_f32": Workload("c1_bidir_f32", 1, 1, 1, 1, 1024, 64, 128, "f32", False),
    "c2_bidir_bf16": Workload("c2_bidir_bf16", 8, 8, 8, 8, 4096, 64, 256, "bf16", False),
    "c3_causal_bf16": Workload("c3_causal_bf16", 4, 12, 12, 12, 8192, 64, 256, "bf16", True),
    "c4_mqa_bidir_bf16": Workload("c4_mqa_bidir_bf16", 16, 16, 1, 1, 16384, 128, 256, "bf16", False),
    "c5_causal_long_bf16": Workload(
        "c5_causal_long_bf16", 1, 8, 8, 8, 65536, 64, 512, "bf16", True,
        heavy_fraction=0.05, heavy_scale=3.0, sampled_rows=256),
}


def workload(name: str) -> Workload:
    return WORKLOADS[name]


def _rng(seed: int, tag: str, index: int) -> np.random.Generator:
    key = [int(seed), index] + [ord(c) for c in tag]
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(key)))


def _heavy_rows(x: np.ndarray, frac: float, scale: float, rng: np.random.Generator) -> None:
    """Scale round(frac*L) distinct rows of every (b, h) slice of x in place."""
    if frac <= 0.0:
        return
    B, H, L, _ = x.shape
    n = int(round(frac * L))
    for b in range(B):
        for h in range(H):
            rows = rng.choice(L, size=n, replace=False)
            x[b, h, rows, :] *= np.float32(scale)


def make_inputs(w: Workload, seed: int = 0):
    """Seeded inputs of workload w.

    Returns (Q, K, V, W): Q (B, Hq, L, d), K and V (B, Hkv, L, d) as float32 arrays whose
    values are exactly representable in w.dtype, and W (Hw, m, d) float32.
    """
    B, Hq, Hkv, L, d, m = w.batch, w.heads_q, w.heads_kv, w.seq_len, w.head_dim, w.num_features
    scale = np.float32(d ** -0.25)
    Q = _rng(seed, w.name + "/Q", 0).standard_normal((B, Hq, L, d), dtype=np.float32)
    Q *= scale
    K = _rng(seed, w.name + "/K", 1).standard_normal((B, Hkv, L, d), dtype=np.float32)
    K *= scale
    V = _rng(seed, w.name + "/V", 2).standard_normal((B, Hkv, L, d), dtype=np.float32)
    _heavy_rows(Q, w.heavy_fraction, w.heavy_scale, _rng(seed, w.name + "/heavyQ", 3))
    _heavy_rows(K, w.heavy_fraction, w.heavy_scale, _rng(seed, w.name + "/heavyK", 4))
    if w.dtype == "bf16":
        Q, K, V = round_to_bf16(Q), round_to_bf16(K), round_to_bf16(V)
    Ws = np.stack([orf_matrix(m, d, _rng(seed, w.name + "/W", 100 + h)) for h in range(w.heads_w)])
    return Q, K, V, Ws.astype(np.float32)


def sample_rows(w: Workload, n: int, seed: int = 0) -> np.ndarray:
    """n distinct (b, hq, i) output rows to check at full size; always includes i = 0 and i = L-1."""
    rng = _rng(seed, w.name + "/rows", 7)
    total = w.batch * w.heads_q * w.seq_len
    flat = rng.choice(total, size=min(n, total), replace=False)
    rows = np.stack(np.unravel_index(flat, (w.batch, w.heads_q, w.seq_len)), axis=1)
    rows[0] = (0, 0, 0)
    if len(rows) > 1:
        rows[1] = (w.batch - 1, w.heads_q - 1, w.seq_len - 1)
    return np.unique(rows, axis=0)
