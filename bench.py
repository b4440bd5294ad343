#!/usr/bin/env python3
"""Throughput of the FAVOR+ forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--also all|LIST]

One step is one favor_attn_fwd call (every kernel of the path) over one batch of seeded
synthetic input already resident in HBM.  W untimed warm-up steps, then exactly K timed
steps between a synchronize on each side.  The headline workload is the largest one (the
multi-query c4); the others, and the causal chunk sweep, follow under "also", each timed
the same way.  Prints one JSON line:
  value          tokens/s = batch * heads_q * seq_len / step time
  roofline       for the kernel with the longest duration: its algorithmic bytes or flops
                 per launch over its duration.  The duration is the kernel's share of the
                 plain-call step time, split in the ratio of per-kernel intervals that a
                 second pass measures with HIP events recorded by the library between its
                 kernels on its own stream (event_ms: the marked interval itself)
  roofline_call  the whole call: its algorithmic bytes and flops against the step time
  cpu_baseline   the float64 CPU oracle timed on this host on a bounded sample of the same
                 workload (whole (batch, head) slices), scaled to tokens/s
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "FAVOR+ attention fwd tokens/s (B*H*L/s) and % MFMA/HBM roofline, 1 GPU"
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E
PEAK_TFLOPS = {"bf16": 2500.0, "f32": 157.3}   # dense MFMA
# Kernel slots of one call (the bidirectional path has no middle kernel; a small float32
# call that runs as one launch fills the first slot only).
FUSED_NAME = "small_fused"
KERNELS = {
    False: ("kv_summary", None, "readout"),
    True: ("kv_summary", "causal_scan", "causal_chunk"),
}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


class HipEvents:
    """hipEvent_t handles through the HIP runtime (the library records them on its stream)."""

    def __init__(self):
        self.rt = ctypes.CDLL("libamdhip64.so")
        self.rt.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.rt.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                ctypes.c_void_p]
        self.rt.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def create(self, n):
        out = []
        for _ in range(n):
            e = ctypes.c_void_p()
            if self.rt.hipEventCreate(ctypes.byref(e)) != 0:
                raise RuntimeError("hipEventCreate failed")
            out.append(e.value)
        return out

    def elapsed_ms(self, a, b):
        ms = ctypes.c_float()
        if self.rt.hipEventElapsedTime(ctypes.byref(ms), ctypes.c_void_p(a), ctypes.c_void_p(b)) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return ms.value

    def destroy(self, evs):
        for e in evs:
            self.rt.hipEventDestroy(ctypes.c_void_p(e))


def algorithmic_work(w, fused=False):
    """Per-kernel algorithmic bytes and flops of one call (what FAVOR+ itself must move and do).

    Bytes: Q, K, V read once and out written once, plus W (and S where a kernel reads the
    finished summary).  Flops: 2 L d m for a feature map plus 2 L m (d+1) for the summary
    (keys) or the readout (queries), per head.  The combine and scan kernels do only
    implementation work (merging position-range partials) and get none.
    """
    e = 2 if w.dtype == "bf16" else 4
    B, Hq, Hkv, Hw, L, d, m = (w.batch, w.heads_q, w.heads_kv, w.heads_w, w.seq_len, w.head_dim,
                               w.num_features)
    side = 2 * L * d * m + 2 * L * m * (d + 1)
    w_bytes = 4 * Hw * m * d
    s_bytes = 4 * B * Hkv * m * (d + 1)
    k_bytes = 2 * e * B * Hkv * L * d
    q_bytes = 2 * e * B * Hq * L * d
    names = KERNELS[w.causal]
    if fused:  # one launch: the whole call's reads, writes and flops
        return {FUSED_NAME: (k_bytes + q_bytes + w_bytes, B * Hkv * side + B * Hq * side)}
    if not w.causal:
        return {names[0]: (k_bytes + w_bytes, B * Hkv * side),
                names[2]: (q_bytes + w_bytes + s_bytes, B * Hq * side)}
    return {names[0]: (k_bytes + w_bytes, B * Hkv * side), names[1]: (0, 0),
            names[2]: (q_bytes + k_bytes + w_bytes, B * Hq * side + B * Hkv * side)}


def call_work(w):
    """Algorithmic bytes and flops of one whole favor_attn_fwd call: Q, K, V read once, out
    written once and W; the feature maps of Q and K (2 L d m per head) and the summary and
    readout contractions (2 L m (d+1) per head)."""
    e = 2 if w.dtype == "bf16" else 4
    B, Hq, Hkv, Hw, L, d, m = (w.batch, w.heads_q, w.heads_kv, w.heads_w, w.seq_len, w.head_dim,
                               w.num_features)
    nbytes = e * L * d * (2 * B * Hq + 2 * B * Hkv) + 4 * Hw * m * d
    flops = (B * Hq + B * Hkv) * (2 * L * d * m + 2 * L * m * (d + 1))
    return nbytes, flops


def kernel_names(w, p=None):
    """Names of the kernel slots of one call (None for an empty slot).  A call the library
    runs as one launch (small float32 bidirectional problems) fills the first slot only."""
    if p is not None and not w.causal:
        from efficient_transformer_attention_favor_amd import _lib
        if _lib.attn_fwd_launches(p) == 1:
            return (FUSED_NAME, None, None)
    return KERNELS[w.causal]


# The sources the forward kernels (favor_attn_fwd) are built from.
FORWARD_SOURCES = ("favor_device.hpp", "favor_kernels.hip", "favor_causal.hip", "favor_small.hip", "favor_ops.hpp",
                   "favor_plan.cpp", "favor_plan.hpp")


def source_digest():
    """SHA-256 over the forward kernels' sources (identifies the kernels counters were taken on)."""
    import hashlib
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "efficient_transformer_attention_favor_amd", "csrc")
    for name in sorted(FORWARD_SOURCES):
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()


def measured_traffic(workload, kernel, chunk=0):
    """HBM bytes per launch of `kernel` from the committed rocprofv3 FETCH_SIZE/WRITE_SIZE summary
    for this workload at this chunk setting (the summaries are taken at the default, 0), or None
    if there is none or the kernels changed since it was taken."""
    import glob
    for path in glob.glob(os.path.join(ROOT, "profiles", f"*_{workload}_traffic.txt")):
        with open(path) as f:
            for line in f:
                if line.startswith("json: "):
                    rec = json.loads(line[6:])
                    if (rec.get("workload") == workload and rec.get("chunk", 0) == chunk
                            and rec.get("source_sha256") == source_digest()):
                        return rec["traffic_bytes"].get(kernel)
    return None


def cpu_baseline(w, Q, K, V, W, min_s=10.0):
    """The float64 oracle on whole (batch, head) slices, cycling over the workload's slices
    until at least min_s seconds have passed (a bounded sample; at most one extra slice)."""
    from threadpoolctl import threadpool_info

    import oracle.favor_oracle as O

    threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    G = w.heads_q // w.heads_kv
    total = w.batch * w.heads_q
    t0 = time.perf_counter()
    heads = 0
    while time.perf_counter() - t0 < min_s:
        b, hq = divmod(heads % total, w.heads_q)
        hk = hq // G
        Wh = W[0 if w.heads_w == 1 else hk]
        O.favor_head(Q[b, hq], K[b, hk], V[b, hk], Wh, causal=w.causal)
        heads += 1
    secs = time.perf_counter() - t0
    # the same oracle with one BLAS thread, on a shorter sample
    from threadpoolctl import threadpool_limits
    with threadpool_limits(limits=1):
        t1 = time.perf_counter()
        n1 = 0
        while time.perf_counter() - t1 < max(1.0, min_s / 4):
            b, hq = divmod(n1 % total, w.heads_q)
            hk = hq // G
            O.favor_head(Q[b, hq], K[b, hk], V[b, hk], W[0 if w.heads_w == 1 else hk], causal=w.causal)
            n1 += 1
        s1 = time.perf_counter() - t1
    return {"value": heads * w.seq_len / secs, "unit": "tokens/s", "cores": threads,
            "kind": "oracle",
            "sample": f"{heads} (batch, head) slices of L={w.seq_len} ({heads / total:.2f} passes over the "
                      f"workload's {total}), float64 NumPy, {secs:.1f} s on the host CPU",
            "single_thread": {"value": n1 * w.seq_len / s1, "cores": 1,
                              "sample": f"{n1} slices, {s1:.1f} s with one BLAS thread"},
            "cpu": _cpu_model()}


def cpu_backward_baseline(w, Q, K, V, W, dO, min_s=10.0):
    """The oracle's gradients on whole kv-head slices (a kv head with its query heads),
    cycling over the workload's slices until at least min_s seconds have passed."""
    from threadpoolctl import threadpool_info

    import oracle.favor_oracle as O

    threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    G = w.heads_q // w.heads_kv
    total = w.batch * w.heads_kv
    t0 = time.perf_counter()
    n = 0
    while time.perf_counter() - t0 < min_s:
        b, hk = divmod(n % total, w.heads_kv)
        sl = (slice(b, b + 1), slice(hk * G, (hk + 1) * G))
        Wh = W[0 if w.heads_w == 1 else hk][None]
        O.favor_grads(Q[sl], K[b:b + 1, hk:hk + 1], V[b:b + 1, hk:hk + 1], Wh, dO[sl], causal=w.causal)
        n += 1
    secs = time.perf_counter() - t0
    return {"value": n * G * w.seq_len / secs, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"{n} kv-head slices ({G} query heads each) of L={w.seq_len}, float64 NumPy, "
                      f"{secs:.1f} s on the host CPU", "cpu": _cpu_model()}


def cpu_generalized_baseline(w, Q, K, V, W, min_s=10.0):
    """The oracle's ReLU attention on whole (batch, query head) slices, cycling until at least
    min_s seconds have passed."""
    from threadpoolctl import threadpool_info

    import oracle.favor_oracle as O

    threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    G = w.heads_q // w.heads_kv
    total = w.batch * w.heads_q
    t0 = time.perf_counter()
    n = 0
    while time.perf_counter() - t0 < min_s:
        b, hq = divmod(n % total, w.heads_q)
        hk = hq // G
        Wh = W[0 if w.heads_w == 1 else hk][None]
        O.generalized_attention(Q[b:b + 1, hq:hq + 1], K[b:b + 1, hk:hk + 1], V[b:b + 1, hk:hk + 1], Wh,
                                causal=w.causal)
        n += 1
    secs = time.perf_counter() - t0
    return {"value": n * w.seq_len / secs, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"{n} (batch, head) slices of L={w.seq_len}, float64 NumPy, {secs:.1f} s on the host CPU",
            "cpu": _cpu_model()}


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="c4_mqa_bidir_bf16",
                    help="the workload of the headline line (default: the largest, multi-query c4)")
    ap.add_argument("--also", default="all",
                    help="other workloads timed in the same run, reported under 'also': 'all' (every other "
                         "workload; causal ones at the default chunk and 64, 128, 256), a comma-separated list, "
                         "or '' for none")
    ap.add_argument("--chunk", type=int, default=0, help="causal chunk (0 = library default)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=10.0, help="seconds of oracle time (at least)")
    ap.add_argument("--copy-probe-mb", type=int, default=0,
                    help="after the timed steps, one device copy of this many MiB (counter calibration)")
    ap.add_argument("--out", default="", help="also append the JSON line to this file")
    ap.add_argument("--decode", action="store_true",
                    help="time favor_attn_decode (one new position per head per step) on the workload's "
                         "head layout instead of the forward pass")
    ap.add_argument("--prefill", type=int, default=256, help="positions decoded before timing (--decode)")
    ap.add_argument("--backward", action="store_true",
                    help="time favor_attn_bwd (gradients of Q, K, V) instead of the forward")
    ap.add_argument("--generalized", default="", choices=["", "relu"],
                    help="time favor_attn_fwd_generalized with this feature map instead of the softmax forward")
    ap.add_argument("--approx-study", action="store_true",
                    help="error of FAVOR+ against exact softmax over feature counts and seeds, orthogonal vs "
                         "i.i.d. features drawn on the device (favor_draw_features); no timing")
    ap.add_argument("--seeds", type=int, default=8, help="feature draws per setting (--approx-study)")
    ap.add_argument("--qk-scale", type=float, default=1.0,
                    help="multiply the workload's Q and K by this factor (--approx-study; 1 = the workload)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only: the library has no multi-GPU path "
              f"(asked for --gpus {args.gpus}, WORLD_SIZE {world}).", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from efficient_transformer_attention_favor_amd import _lib, api
    from efficient_transformer_attention_favor_amd import inputs as I

    w = I.workload(args.workload)
    log(f"workload {w}")
    if args.decode:
        return decode_main(args, w)
    if args.backward:
        return backward_main(args, w)
    if args.approx_study:
        return approx_study(args, w)
    if args.generalized:
        return generalized_main(args, w)
    Q, K, V, W = I.make_inputs(w, seed=0)
    res = forward_record(w, Q, K, V, W, args.chunk, args.steps, args.warmup, graph=True,
                         copy_probe_mb=args.copy_probe_mb)
    if not args.no_cpu_baseline:
        log("timing the CPU oracle ...")
        res["cpu_baseline"] = cpu_baseline(w, Q, K, V, W, args.cpu_budget)
    del Q, K, V, W
    res["launch_floor_us"] = launch_floor_us()
    if args.also:
        # the other benchmark workloads (and the causal chunk sweep) in the same run, each
        # timed the same way on its own inputs; keys are workload names (with the chunk)
        also = {}
        for name, chunk in _also_list(args.also, w.name, args.chunk):
            wa = I.workload(name)
            log(f"also: {name} chunk {chunk}")
            Qa, Ka, Va, Wa = I.make_inputs(wa, seed=0)
            rec = forward_record(wa, Qa, Ka, Va, Wa, chunk, args.steps, args.warmup, graph=name.startswith("c1"))
            del Qa, Ka, Va, Wa
            keep = ("value", "ms_per_step", "dtype", "config", "roofline", "roofline_call", "kernels",
                    "graph_ms_per_step")
            also[f"{name}" + (f"/chunk{chunk}" if wa.causal else "")] = {k: rec[k] for k in keep if k in rec}
        res["also"] = also
    line = json.dumps(res)
    print(line, flush=True)
    if args.out:
        with open(args.out, "a") as f:
            f.write(line + "\n")


def launch_floor_us(n=2000):
    """Microseconds per launch of a one-element fill kernel issued back to back on the current
    stream: the floor under any kernel of a call (a call with k kernels costs at least k of
    these)."""
    import torch
    x = torch.zeros(1, device="cuda")
    for _ in range(50):
        x.fill_(1.0)
    torch.cuda.synchronize()
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record()
    for _ in range(n):
        x.fill_(1.0)
    e.record()
    torch.cuda.synchronize()
    return round(s.elapsed_time(e) / n * 1e3, 3)


def _also_list(spec, main_name, main_chunk):
    """(workload, chunk) pairs of --also: 'all' = every other workload, causal ones at the
    library default and at intra-chunk blocks 64, 128, 256 (256 where the problem has at most
    256 features); else a comma-separated list of names."""
    from efficient_transformer_attention_favor_amd import inputs as I

    names = sorted(I.WORKLOADS) if spec == "all" else [n for n in spec.split(",") if n]
    out = []
    for n in names:
        w = I.workload(n)
        # the 256-position intra-chunk block is built up to 256 features
        chunks = [c for c in (0, 64, 128, 256) if c < 256 or w.num_features <= 256] if w.causal else [0]
        for c in chunks:
            if (n, c) != (main_name, main_chunk):
                out.append((n, c))
    return out


def forward_record(w, Q, K, V, W, chunk, steps, warmup, graph=False, copy_probe_mb=0):
    """Time `steps` plain favor_attn_fwd calls on workload w (inputs resident in HBM) and
    return the JSON record: tokens/s, the whole-call roofline fraction, and per-kernel
    durations from a second pass whose calls record HIP events between the kernels."""
    import numpy as np
    import torch

    from efficient_transformer_attention_favor_amd import _lib, api

    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    dev = torch.device("cuda:0")
    q, k, v = (torch.from_numpy(x).to(dev).to(dt) for x in (Q, K, V))
    wd = torch.from_numpy(W).to(dev)
    out = torch.empty_like(q)
    p = api._problem(q, k, wd, w.causal, chunk)
    nbytes = _lib.workspace_bytes(p)
    if nbytes == 0:
        raise _lib.FavorError(_lib.attn_fwd(p, None, None, None, None, None, None, 0, None), "favor_attn_fwd")
    ws = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)
    ptrs = (q.data_ptr(), k.data_ptr(), v.data_ptr(), wd.data_ptr(), out.data_ptr(), ws.data_ptr())

    def step():
        st = _lib.attn_fwd(p, *ptrs, nbytes, stream.cuda_stream)
        if st != _lib.FAVOR_OK:
            raise _lib.FavorError(st, "favor_attn_fwd")

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()

    # Timed region: exactly `steps` plain calls between a synchronize on each side.
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_host = time.perf_counter()
    start.record(stream)
    for _ in range(steps):
        step()
    end.record(stream)
    torch.cuda.synchronize()
    t_host = time.perf_counter() - t_host
    ms_step = start.elapsed_time(end) / steps

    # The same calls captured in one HIP graph and replayed (launch overhead removed; the
    # library allocates nothing and issues no memset, so it captures as is).  Reported beside
    # the plain-call figure, not instead of it.
    graph_ms = None
    if graph:
        try:
            side = torch.cuda.Stream()
            side.wait_stream(stream)
            with torch.cuda.stream(side):
                st = _lib.attn_fwd(p, *ptrs, nbytes, side.cuda_stream)
            stream.wait_stream(side)
            torch.cuda.synchronize()
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                cap = torch.cuda.current_stream(dev)
                for _ in range(steps):
                    st = _lib.attn_fwd(p, *ptrs, nbytes, cap.cuda_stream)
            if st == _lib.FAVOR_OK:
                g.replay()
                torch.cuda.synchronize()
                g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                g0.record(stream)
                g.replay()
                g1.record(stream)
                torch.cuda.synchronize()
                graph_ms = g0.elapsed_time(g1) / steps
            del g
        except RuntimeError as e:  # capture unavailable: report the plain figure only
            log(f"graph timing skipped: {e}")

    # Per-kernel durations: `steps` more calls with the library recording HIP events between
    # its kernels on its own stream (outside the timed region above).
    hev = HipEvents()
    nk = _lib.FAVOR_FWD_KERNELS
    evs = [hev.create(nk + 1) for _ in range(steps)]
    for i in range(steps):
        st = _lib.attn_fwd_timed(p, *ptrs, nbytes, stream.cuda_stream, evs[i])
        if st != _lib.FAVOR_OK:
            raise _lib.FavorError(st, "favor_attn_fwd_timed")
    torch.cuda.synchronize()
    names = kernel_names(w, p)
    samples = {n: [hev.elapsed_ms(e[j], e[j + 1]) for e in evs] for j, n in enumerate(names) if n is not None}
    for e in evs:
        hev.destroy(e)

    if copy_probe_mb > 0:
        n = copy_probe_mb * (1 << 20)
        src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        log(f"copy probe: {n} bytes device-to-device")

    work = algorithmic_work(w, fused=names[0] == FUSED_NAME)
    peak_tf = PEAK_TFLOPS[w.dtype]
    kms = {n: float(np.mean(v)) for n, v in samples.items()}
    ev_total = sum(kms.values())
    kernels = {}
    for n in kms:
        b, f = work.get(n, (0, 0))
        # event markers between kernels add a gap to each interval: the kernel's share of the
        # plain (unmarked) call time, split in the ratio of the marked intervals
        t = ms_step * kms[n] / ev_total * 1e-3
        kernels[n] = {"ms": round(t * 1e3, 5), "event_ms": round(kms[n], 5),
                      "event_median_ms": round(float(np.median(samples[n])), 5),
                      "event_min_ms": round(float(np.min(samples[n])), 5),
                      "alg_bytes": b, "alg_flops": f,
                      "GB/s": round(b / t / 1e9, 1) if b else None,
                      "TFLOP/s": round(f / t / 1e12, 2) if f else None}
    dom = max(kms, key=lambda n: kms[n])
    b, f = work.get(dom, (0, 0))
    t_dom = kernels[dom]["ms"] * 1e-3
    if b / (PEAK_HBM_GBS * 1e9) >= f / (peak_tf * 1e12):
        roof = {"kernel": dom, "bound": "hbm", "achieved": round(b / t_dom / 1e9, 1), "peak": PEAK_HBM_GBS,
                "unit": "GB/s"}
    else:
        roof = {"kernel": dom, "bound": "mfma", "achieved": round(f / t_dom / 1e12, 2), "peak": peak_tf,
                "unit": "TFLOP/s"}
    roof["frac"] = round(roof["achieved"] / roof["peak"], 4)
    roof["traffic"] = measured_traffic(w.name, dom, chunk)
    roof["per_launch"] = {"alg_bytes": b, "alg_flops": f, "avg_ms": round(t_dom * 1e3, 5),
                          "event_ms": round(kms[dom], 5)}
    # the whole call against the roofline of its algorithmic work (Q, K, V read once, out
    # written once, W; the feature maps, the summary and the readout flops)
    cb, cf = call_work(w)
    t_call = ms_step * 1e-3
    t_roof = max(cb / (PEAK_HBM_GBS * 1e9), cf / (peak_tf * 1e12))
    call = {"bound": "hbm" if cb / (PEAK_HBM_GBS * 1e9) >= cf / (peak_tf * 1e12) else "mfma",
            "alg_bytes": cb, "alg_flops": cf, "GB/s": round(cb / t_call / 1e9, 1),
            "TFLOP/s": round(cf / t_call / 1e12, 2), "roofline_ms": round(t_roof * 1e3, 5),
            "frac": round(t_roof / t_call, 4)}

    tokens = w.batch * w.heads_q * w.seq_len
    return {
        "metric": METRIC,
        "value": round(tokens / (ms_step * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded Gaussian Q, K, V; orthogonal random features W)",
        "config": {"workload": w.name, "batch": w.batch, "heads_q": w.heads_q, "heads_kv": w.heads_kv,
                   "heads_w": w.heads_w, "seq_len": w.seq_len, "head_dim": w.head_dim,
                   "num_features": w.num_features, "mode": "causal" if w.causal else "bidirectional",
                   "chunk": chunk, "parallelism": "single GPU"},
        "roofline": roof,
        "roofline_call": call,
        "kernels": kernels,
        "graph_ms_per_step": round(graph_ms, 5) if graph_ms is not None else None,
        "host_wall_s": round(t_host, 4),
    }


def decode_main(args, w0):
    """Decoding: the state holds --prefill positions (one favor_decode_prefill call, timed on
    its own as prefill_ms), then each step adds one position per (batch, kv head) and answers
    every query head.  Algorithmic bytes per step: the state read and written once (float32
    [B*Hkv][m][d+1]), W, and the new q, k, v and out rows."""
    import numpy as np
    import torch

    from efficient_transformer_attention_favor_amd import _lib, api
    from efficient_transformer_attention_favor_amd import inputs as I

    n_pos = args.prefill + args.warmup + args.steps
    w = w0.replace(seq_len=n_pos, causal=True)
    Q, K, V, W = I.make_inputs(w, seed=0)
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    dev = torch.device("cuda:0")
    # position-major copies so that one position's rows are contiguous
    qs, ks, vs = (torch.from_numpy(np.ascontiguousarray(x.transpose(2, 0, 1, 3))).to(dev).to(dt) for x in (Q, K, V))
    wd = torch.from_numpy(W).to(dev)
    state = api.decode_state(qs[0], ks[0], wd)
    prefill_ms = None
    if args.prefill > 0:
        kp, vp = (torch.from_numpy(np.ascontiguousarray(x[:, :, :args.prefill])).to(dev).to(dt) for x in (K, V))
        api.decode_prefill(kp, vp, wd, w.heads_q, state=state)  # untimed first call
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        api.decode_prefill(kp, vp, wd, w.heads_q, state=state)
        e1.record()
        torch.cuda.synchronize()
        prefill_ms = round(e0.elapsed_time(e1), 5)
        del kp, vp
    out = torch.empty_like(qs[0])
    p = api._decode_problem(qs[0], ks[0], wd)
    stream = torch.cuda.current_stream(dev)

    def step(t):
        st = _lib.attn_decode(p, qs[t].data_ptr(), ks[t].data_ptr(), vs[t].data_ptr(), wd.data_ptr(),
                              state.data_ptr(), out.data_ptr(), stream.cuda_stream)
        if st != _lib.FAVOR_OK:
            raise _lib.FavorError(st, "favor_attn_decode")

    for t in range(args.prefill, args.prefill + args.warmup):
        step(t)
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    t0 = args.prefill + args.warmup
    start.record(stream)
    for t in range(t0, t0 + args.steps):
        step(t)
    end.record(stream)
    torch.cuda.synchronize()
    ms_step = start.elapsed_time(end) / args.steps

    e = 2 if w.dtype == "bf16" else 4
    B, Hq, Hkv, d, m = w.batch, w.heads_q, w.heads_kv, w.head_dim, w.num_features
    alg_bytes = 2 * 4 * B * Hkv * m * (d + 1) + 4 * w.heads_w * m * d + e * d * (2 * B * Hq + 2 * B * Hkv)
    achieved = alg_bytes / (ms_step * 1e-3) / 1e9
    res = {
        "metric": "FAVOR+ causal decode step tokens/s (B*Hq new positions per step), 1 GPU",
        "value": round(B * Hq / (ms_step * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded Gaussian q, k, v; orthogonal random features W)",
        "config": {"workload": f"{w0.name} head layout, decode after {args.prefill} positions", "batch": B,
                   "heads_q": Hq, "heads_kv": Hkv, "heads_w": w.heads_w, "head_dim": d, "num_features": m,
                   "mode": "causal decode", "parallelism": "single GPU", "prefill_ms": prefill_ms},
        "roofline": {"kernel": "decode_update+decode_readout", "bound": "hbm", "achieved": round(achieved, 1),
                     "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4),
                     "traffic": None, "per_launch": {"alg_bytes": alg_bytes, "avg_ms": round(ms_step, 5)}},
    }
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_decode_baseline(w, Q, K, V, W, args)
    line = json.dumps(res)
    print(line, flush=True)
    if args.out:
        with open(args.out, "a") as f:
            f.write(line + "\n")


def backward_main(args, w):
    """Gradients of the forward in the workload's mode: one step = one favor_attn_bwd call on
    an upstream gradient of the output's shape (inputs resident).  Algorithmic flops: the
    feature maps of Q and K, S, phi(Q) S, dphi(Q), dS, dphi(K), and the three products with W
    and dS that give dQ, dK, dV (the same count for both modes, as for the forward; the
    causal chunk products execute more, reported as exec_flops); they run as float32 MFMAs,
    so the roofline is the float32 matrix peak."""
    import numpy as np
    import torch

    from efficient_transformer_attention_favor_amd import _lib, api
    from efficient_transformer_attention_favor_amd import inputs as I

    Q, K, V, W = I.make_inputs(w, seed=0)
    dO = np.random.default_rng(0).standard_normal(Q.shape).astype(np.float32)
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    dev = torch.device("cuda:0")
    q, k, v, do = (torch.from_numpy(x).to(dev).to(dt) for x in (Q, K, V, dO))
    wd = torch.from_numpy(W).to(dev)
    p = api._problem(q, k, wd, w.causal, 0)
    nbytes = _lib.bwd_workspace_bytes(p)
    ws = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    stream = torch.cuda.current_stream(dev)
    ptrs = (q.data_ptr(), k.data_ptr(), v.data_ptr(), wd.data_ptr(), do.data_ptr(), dq.data_ptr(), dk.data_ptr(),
            dv.data_ptr(), ws.data_ptr())

    def step():
        st = _lib.attn_bwd(p, *ptrs, nbytes, stream.cuda_stream)
        if st != _lib.FAVOR_OK:
            raise _lib.FavorError(st, "favor_attn_bwd")

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for _ in range(args.steps):
        step()
    end.record(stream)
    torch.cuda.synchronize()
    ms_step = start.elapsed_time(end) / args.steps

    e = 2 if w.dtype == "bf16" else 4
    B, Hq, Hkv, L, d, m = w.batch, w.heads_q, w.heads_kv, w.seq_len, w.head_dim, w.num_features
    Rq, Rk = B * Hq * L, B * Hkv * L
    flops = 2 * m * ((Rq + Rk) * d + Rk * (d + 1) + 3 * Rq * (d + 1) + Rq * d + Rk * (d + 1) + 2 * Rk * d)
    exec_flops = flops
    if w.causal:
        C = 64
        Lp = (L + C - 1) // C * C
        Qp, Kp = B * Hq * Lp, B * Hkv * Lp
        d1 = d + 1
        exec_flops = 2 * ((Rq + Rk) * d * m + Kp * m * d1 + Qp * C * m + Qp * C * d1 + Qp * m * d1 + Qp * C * d1
                          + Qp * C * m + Qp * d1 * m + Qp * m * d + Qp * m * d1 + Kp * d1 * m + Qp * C * m
                          + Kp * m * d + Kp * m * d + Qp * C * d)
    alg_bytes = e * d * (3 * Rq + 4 * Rk) + 4 * w.heads_w * m * d
    achieved = flops / (ms_step * 1e-3) / 1e12
    res = {
        "metric": "FAVOR+ attention bwd (dQ, dK, dV) tokens/s (B*H*L/s), 1 GPU",
        "value": round(Rq / (ms_step * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic (seeded Gaussian Q, K, V and upstream gradient; orthogonal random features W)",
        "config": {"workload": f"{w.name} backward", "batch": B, "heads_q": Hq, "heads_kv": Hkv,
                   "heads_w": w.heads_w, "seq_len": L, "head_dim": d, "num_features": m,
                   "input_dtype": w.dtype, "mode": f"{'causal' if w.causal else 'bidirectional'} backward",
                   "parallelism": "single GPU"},
        "roofline": {"kernel": "favor_attn_bwd (all kernels)", "bound": "mfma", "achieved": round(achieved, 2),
                     "peak": PEAK_TFLOPS["f32"], "unit": "TFLOP/s", "frac": round(achieved / PEAK_TFLOPS["f32"], 4),
                     "traffic": None, "per_launch": {"alg_flops": flops, "exec_flops": exec_flops, "alg_bytes": alg_bytes,
                                                     "avg_ms": round(ms_step, 5)}},
    }
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_backward_baseline(w, Q, K, V, W, dO,
                                                    min_s=args.cpu_budget)
    line = json.dumps(res)
    print(line, flush=True)
    if args.out:
        with open(args.out, "a") as f:
            f.write(line + "\n")


def generalized_main(args, w):
    """Kernelised attention with the ReLU feature map (favor_attn_fwd_generalized): one step =
    one call on the workload (inputs resident).  Algorithmic flops as for the softmax forward
    (features of Q and K, S, phi(Q) S).  The kernels run MFMA in the input's precision (bf16:
    fp16 W contraction, bf16 products), so the roofline is that dtype's matrix peak."""
    import numpy as np
    import torch

    from efficient_transformer_attention_favor_amd import _lib, api
    from efficient_transformer_attention_favor_amd import inputs as I

    Q, K, V, W = I.make_inputs(w, seed=0)
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    dev = torch.device("cuda:0")
    q, k, v = (torch.from_numpy(x).to(dev).to(dt) for x in (Q, K, V))
    wd = torch.from_numpy(W).to(dev)
    p = api._problem(q, k, wd, w.causal, 0)
    fn = _lib.FAVOR_FEATURE_RELU
    nbytes = _lib.generalized_workspace_bytes(p, fn)
    ws = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    out = torch.empty_like(q)
    stream = torch.cuda.current_stream(dev)
    ptrs = (q.data_ptr(), k.data_ptr(), v.data_ptr(), wd.data_ptr(), out.data_ptr(), ws.data_ptr())

    def step():
        st = _lib.attn_fwd_generalized(p, fn, *ptrs, nbytes, stream.cuda_stream)
        if st != _lib.FAVOR_OK:
            raise _lib.FavorError(st, "favor_attn_fwd_generalized")

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for _ in range(args.steps):
        step()
    end.record(stream)
    torch.cuda.synchronize()
    ms_step = start.elapsed_time(end) / args.steps
    B, Hq, Hkv, L, d, m = w.batch, w.heads_q, w.heads_kv, w.seq_len, w.head_dim, w.num_features
    Rq, Rk = B * Hq * L, B * Hkv * L
    flops = 2 * m * ((Rq + Rk) * d + (Rq + Rk) * (d + 1))
    achieved = flops / (ms_step * 1e-3) / 1e12
    cdt = w.dtype
    res = {
        "metric": "kernelised attention (ReLU random features) fwd tokens/s (B*H*L/s), 1 GPU",
        "value": round(Rq / (ms_step * 1e-3), 1), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_step, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": cdt,
        "data": "synthetic (seeded Gaussian Q, K, V; orthogonal random features W)",
        "config": {"workload": f"{w.name} relu features", "batch": B, "heads_q": Hq, "heads_kv": Hkv,
                   "heads_w": w.heads_w, "seq_len": L, "head_dim": d, "num_features": m,
                   "input_dtype": w.dtype, "mode": "causal" if w.causal else "bidirectional",
                   "parallelism": "single GPU"},
        "roofline": {"kernel": "favor_attn_fwd_generalized (all kernels)", "bound": "mfma",
                     "achieved": round(achieved, 2), "peak": PEAK_TFLOPS[cdt], "unit": "TFLOP/s",
                     "frac": round(achieved / PEAK_TFLOPS[cdt], 4), "traffic": None,
                     "per_launch": {"alg_flops": flops, "avg_ms": round(ms_step, 5)}},
    }
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_generalized_baseline(w, Q, K, V, W, min_s=args.cpu_budget)
    line = json.dumps(res)
    print(line, flush=True)
    if args.out:
        with open(args.out, "a") as f:
            f.write(line + "\n")


def approx_study(args, w):
    """Error of FAVOR+ against exact softmax attention over the feature count m and args.seeds
    draws of W, orthogonal vs i.i.d. rows, both drawn on the device from consecutive seeds
    (Performer page, "제안 방법" and "주요 결과": orthogonal features lower the estimator's
    error).  Inputs: the workload's Q, K, V (Q and K times --qk-scale, which sets the kernel's
    temperature and so the features' variance); 256 sampled query rows; exact softmax on those
    rows in float32 on the GPU.  Metric per setting: RMS over the sampled rows' entries of
    (FAVOR+ - softmax), mean and standard deviation over the draws; and the relative mean
    squared error of the kernel estimate phi(q) . phi(k) against exp(q . k) on 256 queries x
    1024 keys of the first head (favor_features, stabilisers added back).  One JSON line."""
    import numpy as np
    import torch

    from efficient_transformer_attention_favor_amd import api
    from efficient_transformer_attention_favor_amd import inputs as I

    Q, K, V, _ = I.make_inputs(w, seed=0)
    Q, K = Q * args.qk_scale, K * args.qk_scale
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    dev = torch.device("cuda:0")
    q, k, v = (torch.from_numpy(x).to(dev).to(dt) for x in (Q, K, V))
    rows = I.sample_rows(w, 256)
    G = w.heads_q // w.heads_kv
    exact = []
    for b, h, i in rows:  # softmax(q_i K^T) V on the (masked) keys, float32
        n = int(i) + 1 if w.causal else w.seq_len
        kk = k[b, h // G, :n].float()
        s = kk @ q[b, h, i].float()
        exact.append(torch.softmax(s, dim=0) @ v[b, h // G, :n].float())
    exact = torch.stack(exact)
    bi, hi, ii = (torch.as_tensor(rows[:, j], device=dev) for j in range(3))
    qs, ks = q[:1, :1, :256].contiguous(), k[:1, :1, :1024].contiguous()
    kexact = torch.exp(qs[0, 0].double() @ ks[0, 0].double().T)

    def kernel_rel_mse(Wd):
        pq, cq = api.features(qs, Wd[:1].contiguous(), 0, 1, 1)
        pk, ck = api.features(ks, Wd[:1].contiguous(), 1, 1, 1)
        est = (pq.double() @ pk.double().T) * torch.exp(cq.double()[:, None] + ck.double()[0])
        return float(torch.mean(((est - kexact) / kexact) ** 2))

    table = []
    for m in (64, 128, 256, 512):
        entry = {"m": m}
        for kind, orth in (("orf", True), ("iid", False)):
            errs, kmse = [], []
            for sd in range(args.seeds):
                Wd = api.draw_features(w.heads_w, m, w.head_dim, 1000 * m + sd, orth)
                y = api.attn_fwd(q, k, v, Wd, causal=w.causal)
                got = y[bi, hi, ii].float()
                errs.append(float(torch.sqrt(torch.mean((got - exact) ** 2))))
                kmse.append(kernel_rel_mse(Wd))
                del y
            entry[f"{kind}_rms"] = round(float(np.mean(errs)), 6)
            entry[f"{kind}_std"] = round(float(np.std(errs)), 6)
            entry[f"{kind}_kernel_rel_mse"] = round(float(np.mean(kmse)), 6)
        entry["orf_over_iid"] = round(entry["orf_rms"] / entry["iid_rms"], 4)
        log(f"m={m}: {entry}")
        table.append(entry)
    res = {
        "metric": "FAVOR+ RMS error vs exact softmax attention (256 sampled rows)",
        "unit": "RMS", "higher_is_better": False, "seeds": args.seeds, "dtype": w.dtype,
        "data": "synthetic (seeded Gaussian Q, K, V; W drawn on the device by favor_draw_features)",
        "config": {"workload": w.name, "batch": w.batch, "heads_q": w.heads_q, "heads_kv": w.heads_kv,
                   "heads_w": w.heads_w, "seq_len": w.seq_len, "head_dim": w.head_dim,
                   "mode": "causal" if w.causal else "bidirectional", "qk_scale": args.qk_scale},
        "table": table,
    }
    line = json.dumps(res)
    print(line, flush=True)
    if args.out:
        with open(args.out, "a") as f:
            f.write(line + "\n")


def cpu_decode_baseline(w, Q, K, V, W, args, min_s=5.0):
    """The oracle's feature map and summary update, one position at a time on the host."""
    import numpy as np
    from threadpoolctl import threadpool_info

    import oracle.favor_oracle as O

    threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    G = w.heads_q // w.heads_kv
    B, Hkv, d, m = w.batch, w.heads_kv, w.head_dim, w.num_features
    S = np.zeros((B, Hkv, m, d + 1))
    t0 = time.perf_counter()
    steps = 0
    for t in range(w.seq_len):
        for b in range(B):
            for h in range(Hkv):
                Wh = W[0 if w.heads_w == 1 else h]
                pk = O.feature_map(K[b, h, t:t + 1], Wh)[0]
                S[b, h] += np.outer(pk, np.append(V[b, h, t].astype(np.float64), 1.0))
                pq = O.feature_map(Q[b, h * G:(h + 1) * G, t], Wh)
                _ = (pq @ S[b, h, :, :d]) / (pq @ S[b, h, :, d])[:, None]
        steps += 1
        if time.perf_counter() - t0 >= min_s:
            break
    secs = time.perf_counter() - t0
    return {"value": steps * w.batch * w.heads_q / secs, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"{steps} decode steps of {w.batch * w.heads_q} heads, float64 NumPy, {secs:.1f} s",
            "cpu": _cpu_model()}


if __name__ == "__main__":
    main()
