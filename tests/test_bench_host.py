"""Host-side checks of the measurement code (no GPU): the algorithmic work bench.py divides
by matches the hand-computed totals of the workloads, and the single-GPU guard."""
import subprocess
import sys
from pathlib import Path

import pytest

ROOT = Path(__file__).resolve().parents[1]
sys.path.insert(0, str(ROOT))

import bench  # noqa: E402
from efficient_transformer_attention_favor_amd import inputs as I  # noqa: E402

# (algorithmic GFLOP, MB): (B Hq + B Hkv)(2 L d m + 2 L m (d+1)) and
# e L d (2 B Hq + 2 B Hkv) + 4 Hw m d -- Q, K, V read once, out written once, W once
TOTALS = {
    "c1_bidir_f32": (0.0676, 1.08),
    "c2_bidir_bf16": (34.63, 134.7),
    "c3_causal_bf16": (51.94, 202.1),
    "c4_mqa_bidir_bf16": (586.4, 2281.8),
    "c5_causal_long_bf16": (138.5, 269.5),
}


@pytest.mark.parametrize("name", sorted(TOTALS))
def test_algorithmic_work_matches_totals(name):
    w = I.workload(name)
    work = bench.algorithmic_work(w)
    B, Hq, Hkv, L, d, m = w.batch, w.heads_q, w.heads_kv, w.seq_len, w.head_dim, w.num_features
    side = 2 * L * d * m + 2 * L * m * (d + 1)
    flops = sum(f for _, f in work.values())
    if w.causal:  # the chunk kernel recomputes the key features; count them once
        flops -= B * Hkv * side
    gflop, mb = TOTALS[name]
    assert abs(flops / 1e9 - gflop) <= 5e-3 * gflop  # the totals are printed to 3-4 digits
    e = 2 if w.dtype == "bf16" else 4
    total_bytes = e * L * d * (2 * B * Hq + 2 * B * Hkv) + 4 * w.heads_w * m * d
    assert abs(total_bytes / 1e6 - mb) <= 5e-3 * mb
    # every kernel's bytes include what it must read: K, V (key side), Q and out (readout)
    kv = work[bench.KERNELS[w.causal][0]][0]
    assert kv >= e * 2 * B * Hkv * L * d
    last = work[bench.KERNELS[w.causal][2]][0]
    assert last >= e * 2 * B * Hq * L * d


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, str(ROOT / "bench.py"), "--gpus", "2"], capture_output=True, text=True,
                       timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_traffic_only_for_the_profiled_setting(tmp_path, monkeypatch):
    """A committed traffic summary is used for its workload at the chunk it was taken with,
    and only while the kernel sources hash to its digest."""
    prof = tmp_path / "profiles"
    prof.mkdir()
    rec = {"workload": "c3_causal_bf16", "source_sha256": bench.source_digest(),
           "traffic_bytes": {"causal_chunk": 123}}
    (prof / "x_c3_causal_bf16_traffic.txt").write_text("json: " + __import__("json").dumps(rec) + "\n")
    digest = bench.source_digest()
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "source_digest", lambda: digest)
    assert bench.measured_traffic("c3_causal_bf16", "causal_chunk") == 123
    assert bench.measured_traffic("c3_causal_bf16", "causal_chunk", 64) is None
    assert bench.measured_traffic("c5_causal_long_bf16", "causal_chunk") is None
    rec["source_sha256"] = "0" * 64
    (prof / "x_c3_causal_bf16_traffic.txt").write_text("json: " + __import__("json").dumps(rec) + "\n")
    assert bench.measured_traffic("c3_causal_bf16", "causal_chunk") is None


@pytest.mark.parametrize("name", ["c1_bidir_f32", "c2_bidir_bf16"])
def test_one_launch_slot_carries_the_whole_call(name):
    """A call the library runs as one launch is timed as one slot; its algorithmic bytes and
    flops are those of the whole call (Q, K, V read once, out written once, W; both sides'
    feature maps and contractions)."""
    w = I.workload(name)
    work = bench.algorithmic_work(w, fused=True)
    assert list(work) == [bench.FUSED_NAME]
    assert work[bench.FUSED_NAME] == bench.call_work(w)
