#!/usr/bin/env python3
"""Throughput of the sparse-query denoising step on one MI355X.

Workload (default): the 64-step denoising loop of one bf16 GQA attention layer
(B = 8 sequences of S = 2048, hidden 4096, 32 query / 8 KV heads of 128): the
locked fraction rises linearly from 0 to 95 % over the steps, the unlocked
positions of each sequence are a fixed random permutation's first M_t
entries, and the hidden states are redrawn every step.  One denoising step =
compaction of the unlocked positions (given scores) -> Q/K/V of those rows
with K/V scatter into the 2048-slot cache -> partial attention of their
queries over all keys with the context scattered into the cached
activations.  One bench step = one pass of the whole 64-step loop.

Metric: selected-query tokens per second (rows recomputed over the loop / loop
time), and the partial attention's TFLOP/s against the bf16 MFMA peak.  All
inputs (64 distinct hidden-state tensors, 8.6 GB, more than the 256 MB
Infinity Cache) are resident in HBM before timing; the loop is one captured
HIP graph replayed between two HIP events.  The dominant kernel's mean launch
duration is measured live the same way (its 64 launches of one loop in one
graph).  The fp64 CPU oracle is timed on a bounded sample of the same loop as
a reported baseline.

Prints one JSON line.
"""
import argparse
import re
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_HBM = 8.0e12      # MI355X HBM3E, bytes/s
PEAK_BF16 = 2.5e15     # MI355X dense bf16 MFMA, flop/s
# ceiling measured on this GPU at the start of the run (measured_ceilings):
# "mfma_bf16" flop/s of the library's MFMA-loop probe.  HBM fractions are
# reported against the published 8 TB/s only.
MEASURED = {}


def of_measured(rate, key):
    """rate as a fraction of the ceiling measured on this GPU (None if not measured)."""
    return rate / MEASURED[key] if MEASURED.get(key) else None


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20, help="timed passes of the 64-step loop")
    ap.add_argument("--warmup", type=int, default=3, help="untimed passes of the loop before timing")
    ap.add_argument("--sets", type=int, default=4, help="rotating input sets of the one-layer step extra")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the dominant-kernel measurements of the other four workloads")
    ap.add_argument("--only-extras", action="store_true", help="measure only the other workloads")
    ap.add_argument("--hbm-ceiling", action="store_true",
                    help="measure a plain streaming read and a 1 GiB copy (the reference for the "
                         "FETCH_SIZE / WRITE_SIZE byte counters) and exit")
    ap.add_argument("--kernel-only", choices=KERNEL_ONLY,
                    help="run ten eager calls of one dominant kernel's library call and exit "
                         "(a short program for rocprofv3 counter passes)")
    return ap.parse_args()


def source_digest(*names):
    """Digest of the kernel sources with comments and whitespace removed, so
    that a comment edit does not orphan the committed counter summary."""
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "sparse_query_attention_dlm_amd", "csrc", n), encoding="utf-8") as f:
            src = f.read()
        src = re.sub(r"/\*.*?\*/", " ", src, flags=re.S)
        src = re.sub(r"//[^\n]*", " ", src)
        h.update("".join(src.split()).encode())
    return h.hexdigest()[:16]


def committed_traffic(kernel_key, digest):
    """HBM bytes per launch from the committed rocprofv3 PMC summary, or None
    when the summary is missing or was taken on a different kernel source."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(path) as f:
            rec = json.load(f).get(kernel_key)
    except (OSError, ValueError):
        return None
    if not rec or rec.get("source_digest") != digest:
        return None
    return rec.get("bytes_per_launch")


class StepSet:
    """Device-resident inputs, caches and outputs of one rotating input set."""

    def __init__(self, dlm, W, shape, r, max_rows):
        import torch
        inp = W.cosine_step_inputs(shape, seed=shape.seed + 1000 * r)
        s = shape
        bf = torch.bfloat16
        up = lambda a: torch.from_numpy(a).to("cuda").to(bf)
        self.cur, self.prev, self.w = up(inp.cur), up(inp.prev), up(inp.w_qkv)
        B, S = s.B, s.S
        self.kc = torch.zeros(B, S, s.Hkv, s.hd, dtype=bf, device="cuda")
        self.vc = torch.zeros_like(self.kc)
        self.out = torch.zeros(B, S, s.Hq * s.hd, dtype=bf, device="cuda")
        self.q = torch.zeros(max_rows, s.Hq, s.hd, dtype=bf, device="cuda")
        self.o = torch.zeros_like(self.q)
        self.lse = torch.zeros(max_rows, s.Hq, dtype=torch.float32, device="cuda")
        self.idx = torch.zeros(B * S, dtype=torch.int32, device="cuda")
        self.counts = torch.zeros(B, dtype=torch.int32, device="cuda")
        self.offsets = torch.zeros(B + 1, dtype=torch.int32, device="cuda")
        self.ws_sel = torch.zeros(dlm.dlm_select_workspace_size(dlm.DLM_SCORE_COSINE, B, S),
                                  dtype=torch.uint8, device="cuda")
        self.ws_attn = torch.zeros(dlm.dlm_partial_attn_workspace_size(dlm.DLM_BF16, max_rows, B, S, s.Hq, s.Hkv, s.hd),
                                   dtype=torch.uint8, device="cuda")
        self.ws_qkv = torch.zeros(dlm.dlm_gather_qkv_workspace_size(dlm.DLM_BF16, max_rows, s.D, s.Hq, s.Hkv, s.hd),
                                  dtype=torch.uint8, device="cuda")
        # cache state of the previous step: a full pass (every row selected) on prev
        all_rows = torch.zeros(B, S, dtype=torch.float32, device="cuda")
        dlm.dlm_saliency_select(dlm.DLM_SCORE_GIVEN, all_rows, None, lo=0, hi=S, threshold=0.5,
                                idx=self.idx, counts=self.counts, offsets=self.offsets)
        dlm.dlm_gather_qkv_scatter_kv(self.prev, self.idx, self.offsets, B * S, self.w, s.Hq, s.Hkv,
                                      s.hd, self.q, self.kc, self.vc, workspace=self.ws_qkv)
        dlm.dlm_partial_attn(self.q, self.idx, self.offsets, B * S, self.kc, self.vc,
                             1.0 / math.sqrt(s.hd), self.o, self.lse, out_cache=self.out,
                             workspace=self.ws_attn)


class LockLoop:
    """Device-resident state of the 64-step GQA lock loop: the Q/K/V weights,
    one hidden-state tensor per step (8.6 GB in all), each step's given scores
    (0 = unlocked) and its own selection buffers, the caches and the output
    buffers.  Each step passes its exact unlocked count as the row bound (the
    host knows the lock schedule)."""

    def __init__(self, dlm, W):
        import torch
        sh = W.GQA_LOCK_LOOP
        self.dlm, self.sh = dlm, sh
        B, S, D, Hq, Hkv, hd, T = sh.B, sh.S, sh.D, sh.Hq, sh.Hkv, sh.hd, sh.steps
        self.N = (Hq + 2 * Hkv) * hd
        self.scale = 1.0 / math.sqrt(hd)
        self.w = _gen((self.N, D), 601, scale=sh.w_std)
        self.xs = [_gen((B, S, D), 1000 + t) for t in range(T)]
        g = torch.Generator(device="cuda")
        g.manual_seed(604)
        perms = torch.stack([torch.randperm(S, generator=g, device="cuda") for _ in range(B)])
        self.sc, self.n = [], []
        for t in range(T):
            m = W.unlocked_count(S, t, T, sh.lock_max)
            s_t = torch.ones(B, S, dtype=torch.float32, device="cuda")
            s_t.scatter_(1, perms[:, :m], 0.0)
            self.sc.append(s_t)
            self.n.append(B * m)
        bf = torch.bfloat16
        self.kc = torch.zeros(B, S, Hkv, hd, dtype=bf, device="cuda")
        self.vc = torch.zeros_like(self.kc)
        self.out = torch.zeros(B, S, Hq * hd, dtype=bf, device="cuda")
        self.q = torch.zeros(B * S, Hq, hd, dtype=bf, device="cuda")
        self.o = torch.zeros_like(self.q)
        self.lse = torch.zeros(B * S, Hq, dtype=torch.float32, device="cuda")
        self.idx = torch.zeros(T, B * S, dtype=torch.int32, device="cuda")
        self.counts = torch.zeros(T, B, dtype=torch.int32, device="cuda")
        self.offsets = torch.zeros(T, B + 1, dtype=torch.int32, device="cuda")
        self.wsa = torch.zeros(dlm.dlm_partial_attn_workspace_size(dlm.DLM_BF16, B * S, B, S, Hq, Hkv, hd),
                               dtype=torch.uint8, device="cuda")
        self.wsq = torch.zeros(max(16, dlm.dlm_gather_qkv_workspace_size(dlm.DLM_BF16, B * S, D, Hq, Hkv, hd)),
                               dtype=torch.uint8, device="cuda")

    def select(self, t):
        self.dlm.dlm_saliency_select(self.dlm.DLM_SCORE_GIVEN, self.sc[t], None, lo=0, hi=self.sh.S, threshold=0.5,
                                     idx=self.idx[t], counts=self.counts[t], offsets=self.offsets[t])

    def qkv(self, t):
        sh = self.sh
        self.dlm.dlm_gather_qkv_scatter_kv(self.xs[t], self.idx[t], self.offsets[t], self.n[t], self.w, sh.Hq,
                                           sh.Hkv, sh.hd, self.q, self.kc, self.vc, workspace=self.wsq)

    def attn(self, t):
        self.dlm.dlm_partial_attn(self.q, self.idx[t], self.offsets[t], self.n[t], self.kc, self.vc, self.scale,
                                  self.o, self.lse, out_cache=self.out, workspace=self.wsa)

    def loop(self):
        for t in range(self.sh.steps):
            self.select(t)
            self.qkv(t)
            self.attn(t)

    def qkv_flops(self, t):
        return 2.0 * self.n[t] * self.sh.D * self.N

    def attn_flops(self, t):
        sh = self.sh
        return 4.0 * self.n[t] * sh.S * sh.hd * sh.Hq


def main():
    a = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if a.gpus != 1 or world != 1:
        print(f"bench.py measures a single GPU; this build has no multi-GPU path "
              f"(asked for --gpus {a.gpus}, WORLD_SIZE {world}).", file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    from sparse_query_attention_dlm_amd import binding as dlm
    from sparse_query_attention_dlm_amd import workloads as W

    torch.cuda.set_device(0)
    if a.hbm_ceiling:
        print(json.dumps(hbm_ceiling()), flush=True)
        return
    if a.kernel_only:
        print(json.dumps(kernel_only(dlm, W, a.kernel_only)), flush=True)
        return
    if a.only_extras:
        ceil = measured_ceilings(dlm)
        res = {}
        for name, fn in EXTRAS:
            print(f"[bench]   {name}", file=sys.stderr, flush=True)
            res[name] = fn(dlm, W, a)
            torch.cuda.empty_cache()
        print(json.dumps({"measured_ceilings": ceil, "other_workloads": res}), flush=True)
        return
    print("[bench] measuring the MFMA ceiling", file=sys.stderr, flush=True)
    ceilings = measured_ceilings(dlm)
    sh = W.GQA_LOCK_LOOP
    T = sh.steps
    print(f"[bench] building the {sh.name} state (64 hidden-state tensors)", file=sys.stderr, flush=True)
    L = LockLoop(dlm, W)
    torch.cuda.synchronize()

    # eager pass (the reference for the graph replays)
    L.loop()
    torch.cuda.synchronize()
    n_last = L.n[-1]
    ref_o = L.o[:n_last].clone()
    ref_out = L.out.clone()
    # the whole loop in one HIP graph: a replay is one bench step
    capture_stream = torch.cuda.Stream()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=capture_stream):
        L.loop()
    torch.cuda.synchronize()
    graph.replay()
    torch.cuda.synchronize()
    assert torch.equal(L.o[:n_last], ref_o) and torch.equal(L.out, ref_out), "graph replay differs from the eager loop"
    for t in range(T):
        assert int(L.offsets[t, -1].item()) == L.n[t]
    # the warm-up runs right before the timed steps, so the chip enters them
    # at the clock it holds under this load
    print(f"[bench] warmup {a.warmup} loops", file=sys.stderr, flush=True)
    for _ in range(max(1, a.warmup)):
        graph.replay()

    print(f"[bench] timing {a.steps} loops", file=sys.stderr, flush=True)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record()
    for _ in range(a.steps):
        graph.replay()
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    step_gpu_ms = e0.elapsed_time(e1) / a.steps
    ms_per_step = wall * 1e3 / a.steps
    rows = sum(L.n)
    value = rows / (ms_per_step / 1e3)

    # Stage durations over one loop: each stage's 64 calls (one per denoising
    # step, each with its own row count) captured back to back in one HIP
    # graph, replayed for ~30 ms so the clock settles under that stage, then
    # three replays timed between two HIP events on the launch stream.  The
    # Q/K/V call is one GEMM launch (plus a split-K pass that exits at once
    # unless the device split K), so its mean is the dominant kernel's mean
    # launch duration.
    print("[bench] stage timing", file=sys.stderr, flush=True)
    stage_ms = {}
    for name, fn in (("select", L.select), ("qkv", L.qkv), ("attn", L.attn)):
        rot = iter(range(1 << 30))
        stage_ms[name] = _graph_time(lambda: fn(next(rot) % T), T) * T  # ms per loop
    qkv_flops = sum(L.qkv_flops(t) for t in range(T))
    attn_flops = sum(L.attn_flops(t) for t in range(T))
    qkv_rate = qkv_flops / (stage_ms["qkv"] / 1e3)
    attn_rate = attn_flops / (stage_ms["attn"] / 1e3)
    # per-step breakdown at the first, middle and last step
    per = {}
    for t in (0, T // 2, T - 1):
        L.select(t)
        tq = _time(lambda: L.qkv(t), 5)
        ta = _time(lambda: L.attn(t), 5)
        per[f"t{t}"] = {"rows": L.n[t], "qkv_ms": tq, "qkv_TFLOPs": L.qkv_flops(t) / tq / 1e9,
                        "qkv_frac": L.qkv_flops(t) / (tq / 1e3) / PEAK_BF16,
                        "attn_ms": ta, "attn_TFLOPs": L.attn_flops(t) / ta / 1e9,
                        "attn_frac": L.attn_flops(t) / (ta / 1e3) / PEAK_BF16}
    digest = source_digest("gemm.hip", "common.hpp")
    traffic = committed_traffic("gemm_qkv_lock_loop", digest)
    D, N = sh.D, L.N

    out = {
        "metric": "selected-query tokens/s per denoise step",
        "value": value,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) hidden states redrawn every step, N(0,1/64) weights; random init, no checkpoint)",
        "config": {"workload": sh.name + " lock loop", "B": sh.B, "S": sh.S, "D": D, "Hq": sh.Hq, "Hkv": sh.Hkv,
                   "hd": sh.hd, "denoising_steps_per_bench_step": T, "locked_fraction": "0 -> 95 % linear",
                   "rows_per_loop": rows, "rows_first_last_step": [L.n[0], L.n[-1]],
                   "row_bound": "exact count per step",
                   "launch": "the 64-step loop (192 library calls) as one hip graph per bench step"},
        "step_gpu_ms": step_gpu_ms,
        "partial_attn": {"TFLOP/s": attn_rate / 1e12, "frac_of_peak_bf16": attn_rate / PEAK_BF16,
                         "frac_of_measured_mfma": of_measured(attn_rate, "mfma_bf16"),
                         "ms_per_loop": stage_ms["attn"], "flop_per_loop": attn_flops},
        "stages_ms_per_loop": stage_ms,
        "stage_timing": f"one HIP graph of the stage's {T} calls of a loop, replayed for ~30 ms, then 3 replays between two HIP events",
        "roofline": {"kernel": "gemm_dual_kernel, 256 x 256 tiles (128 x 128 at the last step): gathered Q/K/V + K/V scatter",
                     "bound": "mfma", "achieved": qkv_rate / 1e12, "peak": PEAK_BF16 / 1e12, "unit": "TFLOP/s",
                     "frac": qkv_rate / PEAK_BF16, "traffic": traffic,
                     "algorithmic_flop_per_launch": qkv_flops / T,
                     "mean_launch_ms": stage_ms["qkv"] / T,
                     "frac_of_measured_mfma": of_measured(qkv_rate, "mfma_bf16")},
        "loop_frac_of_peak_bf16": (qkv_flops + attn_flops) / (step_gpu_ms / 1e3) / PEAK_BF16,
        "per_step": per,
        "measured_ceilings": ceilings,
    }
    del graph, L
    torch.cuda.empty_cache()
    if not a.no_extras:
        print("[bench] other workloads", file=sys.stderr, flush=True)
        out["other_workloads"] = {}
        for name, fn in EXTRAS:
            print(f"[bench]   {name}", file=sys.stderr, flush=True)
            out["other_workloads"][name] = fn(dlm, W, a)
            torch.cuda.empty_cache()
    if not a.no_cpu_baseline:
        print("[bench] cpu baseline (oracle)", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(W, a.cpu_seconds)
    print(json.dumps(out), flush=True)


def extra_one_layer_step(dlm, W, a):
    """The one-layer bf16 step (B = 1, S = 1024, hidden 4096, 32 x 128 heads,
    102 of 1024 rows selected by cosine < 0.95): select -> Q/K/V + scatter ->
    partial attention + scatter, with the loose row bound B*S (the host does
    not know the count).  Rotating input sets (hidden states, weights, caches)
    larger than twice the Infinity Cache; one HIP graph per round of the sets.
    HBM-bound at this size: the Q/K/V GEMM streams its 100.7 MB of weights."""
    import numpy as np
    import torch
    sh = W.BF16_S1024
    B, S, s = sh.B, sh.S, sh
    max_rows = B * S
    scale = 1.0 / math.sqrt(sh.hd)
    sets = [StepSet(dlm, W, sh, r, max_rows) for r in range(a.sets)]
    torch.cuda.synchronize()

    def stages(st):
        return [
            lambda: dlm.dlm_saliency_select(dlm.DLM_SCORE_COSINE, st.cur, st.prev, lo=0, hi=S,
                                            threshold=sh.tau, idx=st.idx, counts=st.counts,
                                            offsets=st.offsets, workspace=st.ws_sel),
            lambda: dlm.dlm_gather_qkv_scatter_kv(st.cur, st.idx, st.offsets, max_rows, st.w, s.Hq,
                                                  s.Hkv, s.hd, st.q, st.kc, st.vc, workspace=st.ws_qkv),
            lambda: dlm.dlm_partial_attn(st.q, st.idx, st.offsets, max_rows, st.kc, st.vc, scale,
                                         st.o, st.lse, out_cache=st.out, workspace=st.ws_attn),
        ]

    for st in sets:
        for f in stages(st):
            f()
    torch.cuda.synchronize()
    n_sel = int(sets[0].offsets[-1].item())
    step_ms = _graph_time(lambda: [f() for st in sets for f in stages(st)], 1) / len(sets)
    names = ["select", "qkv", "attn"]
    stage_ms = []
    for k in range(3):
        rot = iter(range(1 << 30))
        stage_ms.append(_graph_time(lambda: stages(sets[next(rot) % a.sets])[k](), 100))
    D, N = sh.D, (s.Hq + 2 * s.Hkv) * s.hd
    qkv_bytes = N * D * 2 + n_sel * D * 2 + n_sel * N * 2
    sel_bytes = 2 * B * S * D * 2
    # the K/V cache read once; the selected rows' Q read, their O and output-cache rows written
    attn_bytes = 2 * B * S * s.Hkv * s.hd * 2 + 3 * n_sel * s.Hq * s.hd * 2
    attn_flops = 4.0 * n_sel * S * s.hd * s.Hq
    achieved = qkv_bytes / (stage_ms[1] / 1e3)
    digest = source_digest("gemm.hip", "common.hpp")
    return {"workload": sh.name + " cosine-select step", "n_selected": n_sel, "max_rows_bound": max_rows,
            "step_ms": step_ms, "tokens_per_s": n_sel / (step_ms / 1e3),
            "stages_ms": dict(zip(names, stage_ms)),
            "roofline": {"kernel": "gemm_dual_kernel, weight-streaming body: 48 weight rows x 128 tokens per tile",
                         "bound": "hbm", "achieved": achieved / 1e9, "peak": PEAK_HBM / 1e9, "unit": "GB/s",
                         "frac": achieved / PEAK_HBM, "algorithmic_bytes": qkv_bytes,
                         "traffic": committed_traffic("gemm_qkv_bf16_s1024", digest)},
            "select": {"GB/s": sel_bytes / (stage_ms[0] / 1e3) / 1e9, "frac": sel_bytes / (stage_ms[0] / 1e3) / PEAK_HBM},
            "attn": {"GB/s": attn_bytes / (stage_ms[2] / 1e3) / 1e9, "frac": attn_bytes / (stage_ms[2] / 1e3) / PEAK_HBM,
                     "TFLOP/s": attn_flops / (stage_ms[2] / 1e3) / 1e12, "algorithmic_bytes": attn_bytes}}


# ---------------------------------------------------------------------------
# dominant kernels of the other workloads (colsum, LM head, lock loop, tiny fp32)
# ---------------------------------------------------------------------------
def _gen(shape, seed, scale=1.0, dtype=None):
    import torch
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    t = torch.randn(shape, generator=g, device="cuda", dtype=torch.float32)
    if scale != 1.0:
        t.mul_(scale)
    return t.to(dtype or torch.bfloat16)


def queue_warm(fn, ms=30.0):
    """Queue about `ms` of GPU time of real calls of fn (never fewer than one)
    without waiting, so that calls the host enqueues next run back to back on
    a GPU that is already at the clock it holds under this load.  (A GPU spin
    kernel would also keep the queue full, but the chip lowers its clock
    during a spin and the first milliseconds after it run up to 20 % slower.)"""
    import torch
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    a.record()
    fn()
    b.record()
    torch.cuda.synchronize()
    one = max(a.elapsed_time(b), 1e-3)
    for _ in range(int(min(4000, max(1, math.ceil(ms / one))))):
        fn()


GRAPH_BELOW_MS = 0.15  # calls shorter than this are timed as a captured graph


def _graph_time(fn, reps, warm_ms=30.0):
    """Mean GPU time (ms) per call of `reps` back-to-back calls of fn captured
    in one HIP graph.  For calls shorter than the host's launch time the host
    cannot stay ahead of the GPU; one graph launch submits them all.  The
    graph is replayed for about warm_ms first (the clock settles under this
    exact load), then three replays are timed between two HIP events."""
    import torch
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=torch.cuda.Stream()):
        for _ in range(reps):
            fn()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    g.replay()
    b.record()
    torch.cuda.synchronize()
    for _ in range(int(min(1000, max(1, math.ceil(warm_ms / max(a.elapsed_time(b), 1e-3)))))):
        g.replay()
    a.record()
    for _ in range(3):
        g.replay()
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) / (3 * reps)


def _time(fn, reps, warmup=2, graph=True):
    """Mean GPU time (ms) of fn over `reps` back-to-back calls.  Calls of
    GRAPH_BELOW_MS or more: each between two HIP events on the current
    stream, behind a queue of warm-up calls.  Shorter calls (graph=True):
    captured in a HIP graph, see _graph_time."""
    import torch
    for _ in range(warmup):
        fn()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    a.record()
    fn()
    b.record()
    torch.cuda.synchronize()
    if graph and a.elapsed_time(b) < GRAPH_BELOW_MS:
        return _graph_time(fn, reps)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    queue_warm(fn)
    for a, b in ev:
        a.record()
        fn()
        b.record()
    torch.cuda.synchronize()
    return sum(a.elapsed_time(b) for a, b in ev) / reps


def _packed_rows(rows_per_b):
    """(idx, offsets) device tensors from a list of sorted int64 device tensors."""
    import torch
    counts = torch.tensor([r.numel() for r in rows_per_b], dtype=torch.int64)
    offsets = torch.zeros(len(rows_per_b) + 1, dtype=torch.int32)
    offsets[1:] = torch.cumsum(counts, 0).to(torch.int32)
    return torch.cat(rows_per_b).to(torch.int32).contiguous(), offsets.cuda()


def extra_colsum(dlm, W, a=None):
    """Attention over the masked region + column sums + top-64 (B=4, S=4096)."""
    import torch
    sh = W.COLSUM_TOP64
    B, S, nq, Hq, Hkv, hd = sh.B, sh.S, sh.S - sh.prompt, sh.Hq, sh.Hkv, sh.hd
    n = B * nq
    q = _gen((n, Hq, hd), 401)
    k = _gen((B, S, Hkv, hd), 402)
    v = _gen((B, S, Hkv, hd), 403)
    idx, offsets = _packed_rows([torch.arange(sh.prompt, S, device="cuda") for _ in range(B)])
    o = torch.empty_like(q)
    lse = torch.empty(n, Hq, dtype=torch.float32, device="cuda")
    wsa = torch.zeros(dlm.dlm_partial_attn_workspace_size(dlm.DLM_BF16, n, B, S, Hq, Hkv, hd), dtype=torch.uint8, device="cuda")
    colsum = torch.empty(B, S, dtype=torch.float32, device="cuda")
    ti = torch.empty(B, sh.k, dtype=torch.int32, device="cuda")
    tv = torch.empty(B, sh.k, dtype=torch.float32, device="cuda")
    wsc = torch.zeros(dlm.dlm_attn_colsum_workspace_size(B, S, Hkv), dtype=torch.uint8, device="cuda")
    scale = 1.0 / math.sqrt(hd)
    attn = lambda: dlm.dlm_partial_attn(q, idx, offsets, n, k, v, scale, o, lse, workspace=wsa)
    col = lambda: dlm.dlm_attn_colsum(q, offsets, n, k, lse, scale, colsum, sh.prompt, S, sh.k,
                                      topk_idx=ti, topk_val=tv, workspace=wsc)
    # block-wise variant: sums and top-64 over a 1024-key sub-block of the masked region
    colw = lambda: dlm.dlm_attn_colsum(q, offsets, n, k, lse, scale, colsum, sh.prompt, sh.prompt + 1024, sh.k,
                                       topk_idx=ti, topk_val=tv, workspace=wsc, window_only=True)
    t_attn = _time(attn, 10)
    t_col = _time(col, 10)
    t_colw = _time(colw, 10)
    f_attn = 4.0 * n * S * hd * Hq
    f_col = 2.0 * n * S * hd * Hq
    return {"workload": sh.name, "n_selected": n,
            "partial_attn": {"ms": t_attn, "TFLOP/s": f_attn / t_attn / 1e9, "frac": f_attn / (t_attn / 1e3) / PEAK_BF16,
                             "frac_of_measured_mfma": of_measured(f_attn / (t_attn / 1e3), "mfma_bf16")},
            "colsum_topk": {"ms": t_col, "TFLOP/s": f_col / t_col / 1e9, "frac": f_col / (t_col / 1e3) / PEAK_BF16,
                            "frac_of_measured_mfma": of_measured(f_col / (t_col / 1e3), "mfma_bf16")},
            "tokens_per_s": n / ((t_attn + t_col) / 1e3),
            "colsum_topk_window_1024_keys": {"ms": t_colw, "TFLOP/s": f_col / 4 / t_colw / 1e9}}


KERNEL_ONLY = ("attn_colsum_top64", "attn_lock_t0", "qkv_lock_t0", "lmhead_lsp", "step_s1024")


def kernel_only(dlm, W, which, calls=10):
    """Ten eager calls of one library call, for counter passes: the partial
    attention of the column-sum workload (B=4, S=4096, the 3072 masked rows of
    each sequence, 32 x 128 heads) or of the lock loop's first step (B=8,
    S=2048, every row, 32 query over 8 KV heads); the lock loop's first-step
    Q/K/V GEMM (16,384 rows, K=4096, N=6144); the confidence LM head of the
    LSP workload (3,680 rows, V=32768); or the one-layer step (B=1, S=1024,
    hidden 4096, 32 x 128 heads: cosine select, Q/K/V + K/V scatter, partial
    attention + output scatter, loose row bound 1024) over four rotating
    input sets.  Inputs are seeded N(0,1)."""
    import torch
    if which == "step_s1024":
        sh = W.BF16_S1024
        max_rows = sh.B * sh.S
        scale = 1.0 / math.sqrt(sh.hd)
        sets = [StepSet(dlm, W, sh, r, max_rows) for r in range(4)]
        rot = iter(range(1 << 30))

        def call():
            st = sets[next(rot) % len(sets)]
            dlm.dlm_saliency_select(dlm.DLM_SCORE_COSINE, st.cur, st.prev, lo=0, hi=sh.S, threshold=sh.tau,
                                    idx=st.idx, counts=st.counts, offsets=st.offsets, workspace=st.ws_sel)
            dlm.dlm_gather_qkv_scatter_kv(st.cur, st.idx, st.offsets, max_rows, st.w, sh.Hq, sh.Hkv, sh.hd,
                                          st.q, st.kc, st.vc, workspace=st.ws_qkv)
            dlm.dlm_partial_attn(st.q, st.idx, st.offsets, max_rows, st.kc, st.vc, scale, st.o, st.lse,
                                 out_cache=st.out, workspace=st.ws_attn)
        call()
        torch.cuda.synchronize()
        n = int(sets[0].offsets[-1].item())
        N = (sh.Hq + 2 * sh.Hkv) * sh.hd
        flops = 2.0 * n * sh.D * N + 4.0 * n * sh.S * sh.hd * sh.Hq
    elif which.startswith("attn"):
        sh = W.COLSUM_TOP64 if which == "attn_colsum_top64" else W.GQA_LOCK_LOOP
        B, S, Hq, Hkv, hd = sh.B, sh.S, sh.Hq, sh.Hkv, sh.hd
        lo = sh.prompt if which == "attn_colsum_top64" else 0
        n = B * (S - lo)
        q = _gen((n, Hq, hd), 411)
        k = _gen((B, S, Hkv, hd), 412)
        v = _gen((B, S, Hkv, hd), 413)
        idx, offsets = _packed_rows([torch.arange(lo, S, device="cuda") for _ in range(B)])
        o = torch.empty_like(q)
        lse = torch.empty(n, Hq, dtype=torch.float32, device="cuda")
        ws = torch.zeros(dlm.dlm_partial_attn_workspace_size(dlm.DLM_BF16, n, B, S, Hq, Hkv, hd),
                         dtype=torch.uint8, device="cuda")
        scale = 1.0 / math.sqrt(hd)
        call = lambda: dlm.dlm_partial_attn(q, idx, offsets, n, k, v, scale, o, lse, workspace=ws)
        flops = 4.0 * n * S * hd * Hq
    elif which == "qkv_lock_t0":
        sh = W.GQA_LOCK_LOOP
        B, S, D, Hq, Hkv, hd = sh.B, sh.S, sh.D, sh.Hq, sh.Hkv, sh.hd
        N, n = (Hq + 2 * Hkv) * hd, B * S
        x = _gen((B, S, D), 421)
        w = _gen((N, D), 422, scale=sh.w_std)
        idx, offsets = _packed_rows([torch.arange(0, S, device="cuda") for _ in range(B)])
        q = torch.empty(n, Hq, hd, dtype=torch.bfloat16, device="cuda")
        kc = torch.zeros(B, S, Hkv, hd, dtype=torch.bfloat16, device="cuda")
        vc = torch.zeros_like(kc)
        ws = torch.zeros(max(16, dlm.dlm_gather_qkv_workspace_size(dlm.DLM_BF16, n, D, Hq, Hkv, hd)),
                         dtype=torch.uint8, device="cuda")
        call = lambda: dlm.dlm_gather_qkv_scatter_kv(x, idx, offsets, n, w, Hq, Hkv, hd, q, kc, vc, workspace=ws)
        flops = 2.0 * n * D * N
    else:
        sh = W.LSP_COMMIT
        B, S, D, V = sh.B, sh.S, sh.D, sh.V
        na = int(math.floor(sh.active_frac * (S - sh.prompt)))
        h = _gen((B, S, D), 431)
        w = _gen((V, D), 432, scale=sh.w_std)
        g = torch.Generator(device="cuda")
        g.manual_seed(433)
        rows = [torch.sort(torch.randperm(S - sh.prompt, generator=g, device="cuda")[:na])[0] + sh.prompt
                for _ in range(B)]
        eidx, eoff = _packed_rows(rows)
        n = int(eidx.numel())
        scores = torch.zeros(B, S, dtype=torch.float32, device="cuda")
        argmax = torch.full((B, S), -1, dtype=torch.int32, device="cuda")
        idx = torch.empty(B * S, dtype=torch.int32, device="cuda")
        counts = torch.empty(B, dtype=torch.int32, device="cuda")
        offsets = torch.empty(B + 1, dtype=torch.int32, device="cuda")
        ws = torch.zeros(dlm.dlm_select_workspace_size(dlm.DLM_SCORE_CONFIDENCE, B, S, V, n), dtype=torch.uint8,
                         device="cuda")
        call = lambda: dlm.dlm_saliency_select(dlm.DLM_SCORE_CONFIDENCE, h, w, lo=sh.prompt, hi=S,
                                               threshold=sh.conf, idx=idx, counts=counts, offsets=offsets,
                                               scores=scores, argmax=argmax, eval_idx=eidx, eval_offsets=eoff,
                                               max_eval=n, workspace=ws)
        flops = 2.0 * n * D * V
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    call()
    torch.cuda.synchronize()
    e0.record()
    for _ in range(calls):
        call()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / calls
    return {"kernel_only": which, "rows": n, "ms_per_call": ms, "TFLOP/s": flops / ms / 1e9}


def extra_lsp(dlm, W, a=None):
    """Confidence select (LM head over 230 active rows per sequence) + stable prefix (B=16)."""
    import torch
    sh = W.LSP_COMMIT
    B, S, D, V = sh.B, sh.S, sh.D, sh.V
    S_gen = S - sh.prompt
    na = int(math.floor(sh.active_frac * S_gen))
    h = _gen((B, S, D), 501)
    w = _gen((V, D), 502, scale=sh.w_std)
    g = torch.Generator(device="cuda")
    g.manual_seed(503)
    rows = [torch.sort(torch.randperm(S_gen, generator=g, device="cuda")[:na])[0] + sh.prompt for _ in range(B)]
    eidx, eoff = _packed_rows(rows)
    n = int(eidx.numel())
    scores = torch.zeros(B, S, dtype=torch.float32, device="cuda")
    argmax = torch.full((B, S), -1, dtype=torch.int32, device="cuda")
    ring = torch.full((B, S_gen, sh.W), -1, dtype=torch.int32, device="cuda")
    com = torch.zeros(B, dtype=torch.int32, device="cuda")
    idx = torch.empty(B * S, dtype=torch.int32, device="cuda")
    counts = torch.empty(B, dtype=torch.int32, device="cuda")
    offsets = torch.empty(B + 1, dtype=torch.int32, device="cuda")
    ws = torch.zeros(dlm.dlm_select_workspace_size(dlm.DLM_SCORE_CONFIDENCE, B, S, V, n), dtype=torch.uint8, device="cuda")
    conf = lambda: dlm.dlm_saliency_select(dlm.DLM_SCORE_CONFIDENCE, h, w, lo=sh.prompt, hi=S,
                                           threshold=sh.conf, idx=idx, counts=counts, offsets=offsets,
                                           scores=scores, argmax=argmax, eval_idx=eidx,
                                           eval_offsets=eoff, max_eval=n, workspace=ws)
    step = [0]

    def prefix():
        dlm.dlm_stable_prefix(argmax, scores, sh.prompt, S, ring, step[0], sh.conf, com)
        step[0] += 1
    # the margin variant: the same LM-head pass scoring top-1 minus top-2, then
    # the adaptive-threshold commit from a fresh frontier (restored each call)
    margin = torch.zeros(B, S, dtype=torch.float32, device="cuda")
    mar = lambda: dlm.dlm_saliency_select(dlm.DLM_SCORE_MARGIN, h, w, lo=sh.prompt, hi=S, threshold=0.0, idx=idx,
                                          counts=counts, offsets=offsets, scores=margin, argmax=argmax,
                                          eval_idx=eidx, eval_offsets=eoff, max_eval=n, workspace=ws)
    com2 = torch.zeros(B, dtype=torch.int32, device="cuda")
    tau = torch.empty(B, dtype=torch.float32, device="cuda")

    def adaptive():
        com2.zero_()
        dlm.dlm_lsp_adaptive_commit(margin, sh.prompt, S, com2, 0.25, 0.5, tau=tau)
    t_conf = _time(conf, 10)
    t_pre = _time(prefix, 10)
    t_mar = _time(mar, 10)
    t_ad = _time(adaptive, 10)
    f = 2.0 * n * D * V
    return {"workload": sh.name, "n_selected": n,
            "confidence_lm_head": {"ms": t_conf, "TFLOP/s": f / t_conf / 1e9, "frac": f / (t_conf / 1e3) / PEAK_BF16,
                                   "frac_of_measured_mfma": of_measured(f / (t_conf / 1e3), "mfma_bf16")},
            "stable_prefix": {"ms": t_pre},
            "tokens_per_s": n / ((t_conf + t_pre) / 1e3),
            "margin_lm_head": {"ms": t_mar, "TFLOP/s": f / t_mar / 1e9, "frac": f / (t_mar / 1e3) / PEAK_BF16},
            "adaptive_commit": {"ms": t_ad, "note": "includes a 64-byte frontier reset"}}


def extra_tiny(dlm, W, a=None):
    """The tiny fp32 layer (S=128, hidden 256): step latency."""
    import torch
    sh = W.TINY_FP32
    inp = W.cosine_step_inputs(sh)
    f = lambda a: torch.from_numpy(a).cuda()
    cur, prev, wq, wo = f(inp.cur), f(inp.prev), f(inp.w_qkv), f(inp.w_o)
    B, S = sh.B, sh.S
    kc = torch.zeros(B, S, sh.Hkv, sh.hd, device="cuda")
    vc = torch.zeros_like(kc)
    out = torch.zeros(B, S, sh.D, device="cuda")
    q = torch.empty(B * S, sh.Hq, sh.hd, device="cuda")
    o = torch.empty_like(q)
    lse = torch.empty(B * S, sh.Hq, device="cuda")
    idx = torch.empty(B * S, dtype=torch.int32, device="cuda")
    counts = torch.empty(B, dtype=torch.int32, device="cuda")
    offsets = torch.empty(B + 1, dtype=torch.int32, device="cuda")
    ws = torch.zeros(dlm.dlm_select_workspace_size(dlm.DLM_SCORE_COSINE, B, S), dtype=torch.uint8, device="cuda")
    mr = B * S

    def step():
        dlm.dlm_saliency_select(dlm.DLM_SCORE_COSINE, cur, prev, lo=0, hi=S, threshold=sh.tau, idx=idx,
                                counts=counts, offsets=offsets, workspace=ws)
        dlm.dlm_gather_qkv_scatter_kv(cur, idx, offsets, mr, wq, sh.Hq, sh.Hkv, sh.hd, q, kc, vc)
        dlm.dlm_partial_attn(q, idx, offsets, mr, kc, vc, 1.0 / math.sqrt(sh.hd), o, lse, w_o=wo,
                             out_cache=out)
    step()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    t = _time(g.replay, 50, warmup=5, graph=False)
    n = int(offsets[-1].item())
    return {"workload": sh.name, "n_selected": n, "step_us": t * 1e3, "tokens_per_s": n / (t / 1e3)}


def hbm_ceiling():
    """Measured HBM ceilings on this GPU: a streaming read (torch sum over 2 GiB,
    more than the Infinity Cache) and a plain 1 GiB device copy."""
    import torch
    n = (2 << 30) // 4
    x = torch.ones(n, dtype=torch.float32, device="cuda")
    y = torch.empty(n // 2, dtype=torch.float32, device="cuda")
    t_sum = _time(lambda: x.sum(), 10)
    t_copy = _time(lambda: y.copy_(x[: n // 2]), 10)
    return {"stream_read_GBps": n * 4 / t_sum / 1e6, "copy_1GiB_GBps_read_plus_write": 2 * (n // 2) * 4 / t_copy / 1e6,
            "copy_bytes_each_way": (n // 2) * 4}


def mfma_ceiling(dlm, grid=512, iters=2000):
    """Measured bf16 MFMA ceiling: the library's MFMA-loop probe (eight
    independent 32x32x16 chains per wave on registers, no memory traffic)."""
    import torch
    sink = torch.empty(grid * 256, dtype=torch.float32, device="cuda")
    t = _time(lambda: dlm.dlm_probe_mfma_bf16(iters, grid, sink), 5)
    flops = grid * 4 * iters * 8 * 32768
    return {"mfma_bf16_TFLOPs": flops / (t / 1e3) / 1e12,
            "mfma_probe": f"{grid} workgroups x 4 waves x {iters} rounds of 8 independent 32x32x16 bf16 MFMAs"}


def measured_ceilings(dlm):
    """The MFMA ceiling measured on this GPU (the library's probe); also fills
    MEASURED for the frac_of_measured_mfma figures.  HBM figures are reported
    against the published 8 TB/s only (hbm_ceiling() is the copy kernel of
    known size that the byte counters are scaled by, run with --hbm-ceiling)."""
    import torch
    c = mfma_ceiling(dlm)
    torch.cuda.empty_cache()
    MEASURED["mfma_bf16"] = c["mfma_bf16_TFLOPs"] * 1e12
    return c


def extra_select_b8(dlm, W, a=None):
    """Not a configuration of the pages: the C2 cosine select at B = 8 (134 MB
    per call, two rotating input sets of 268 MB, more than the Infinity
    Cache), the asymptote of the select kernel's HBM rate."""
    import torch
    B, S, D = 8, 1024, 4096
    sets = [(_gen((B, S, D), 601 + 2 * r, dtype=torch.bfloat16), _gen((B, S, D), 602 + 2 * r, dtype=torch.bfloat16))
            for r in range(2)]
    idx = torch.empty(B * S, dtype=torch.int32, device="cuda")
    counts = torch.empty(B, dtype=torch.int32, device="cuda")
    offsets = torch.empty(B + 1, dtype=torch.int32, device="cuda")
    ws = torch.zeros(dlm.dlm_select_workspace_size(dlm.DLM_SCORE_COSINE, B, S, 0, 0), dtype=torch.uint8, device="cuda")
    calls = [lambda c=c, p=p: dlm.dlm_saliency_select(dlm.DLM_SCORE_COSINE, c, p, lo=0, hi=S, threshold=0.95, idx=idx,
                                                      counts=counts, offsets=offsets, workspace=ws) for c, p in sets]
    state = {"i": 0}

    def call():
        calls[state["i"] % 2]()
        state["i"] += 1
    t = _time(call, 20)
    nbytes = 2 * B * S * D * 2
    return {"workload": "bf16_select_b8_s1024_d4096 (not a configuration of the pages)", "ms": t,
            "GB/s": nbytes / (t / 1e3) / 1e9, "frac": nbytes / (t / 1e3) / PEAK_HBM}


def extra_dv_update(dlm, W, a=None):
    """The non-salient value-change update (DyLLM's non-salient path) on two
    shapes: the bf16 one-layer step (1024 positions, 32 x 128 heads, 102
    salient) and a mid-loop step of the GQA lock loop (B = 8, S = 2048, 32 / 8
    heads, half the positions unlocked).  Rotating input sets larger than the
    Infinity Cache.  Algorithmic bytes: the stable rows' query, LSE and output
    (read and written) plus the salient rows' K_old, V_old and new V."""
    import torch
    out = {}
    for name, B, S, Hq, Hkv, hd, n_b, nsets in (("bf16_s1024_32x128_102_salient", 1, 1024, 32, 32, 128, 102, 12),
                                                ("gqa_b8_s2048_32q8kv_half_unlocked", 8, 2048, 32, 8, 128, 1024, 2)):
        g = torch.Generator(device="cuda")
        g.manual_seed(700)
        rows = [torch.sort(torch.randperm(S, device="cuda", generator=g)[:n_b]).values for _ in range(B)]
        idx, offsets = _packed_rows(rows)
        n = B * n_b
        sets = []
        for r in range(nsets):
            q = _gen((B, S, Hq, hd), 710 + 5 * r, dtype=torch.bfloat16)
            lse = torch.full((B, S, Hq), 7.0, dtype=torch.float32, device="cuda")
            o = _gen((B, S, Hq, hd), 711 + 5 * r, dtype=torch.bfloat16)
            ko = _gen((n, Hkv, hd), 712 + 5 * r, dtype=torch.bfloat16)
            vo = _gen((n, Hkv, hd), 713 + 5 * r, dtype=torch.bfloat16)
            v = _gen((B, S, Hkv, hd), 714 + 5 * r, dtype=torch.bfloat16)
            sets.append((q, lse, ko, vo, v, o))
        calls = [lambda st=st: dlm.dlm_nonsalient_dv_update(st[0], st[1], idx, offsets, n, st[2], st[3], st[4],
                                                            1.0 / math.sqrt(hd), st[5]) for st in sets]
        state = {"i": 0}

        def call():
            calls[state["i"] % nsets]()
            state["i"] += 1
        t = _time(call, 24)
        stable = B * S - n
        nbytes = stable * Hq * (3 * hd * 2 + 4) + 3 * n * Hkv * hd * 2
        flops = 4.0 * (S - n_b) * n_b * hd * Hq * B
        out[name] = {"ms": t, "GB/s": nbytes / (t / 1e3) / 1e9, "frac": nbytes / (t / 1e3) / PEAK_HBM,
                     "TFLOP/s": flops / t / 1e9, "algorithmic_bytes": nbytes}
    return out


def extra_salient_ffn(dlm, W, a=None):
    """The salient-row SwiGLU FFN (D = 4096, F = 12288) on the one-layer step's
    102 selected rows (weight-stream bound: 2F.D + D.F bf16 weights per call,
    two rotating weight sets larger than the Infinity Cache) and on 2048
    selected rows (matrix-core bound)."""
    import torch
    D, F = 4096, 12288
    out = {}
    for name, B, S, n_b, nsets in (("bf16_s1024_102_rows", 1, 1024, 102, 2), ("bf16_b2_s1024_2048_rows", 2, 1024, 1024, 1)):
        g = torch.Generator(device="cuda")
        g.manual_seed(800)
        rows = [torch.sort(torch.randperm(S, device="cuda", generator=g)[:n_b]).values for _ in range(B)]
        idx, offsets = _packed_rows(rows)
        n = B * n_b
        x = _gen((B, S, D), 801, dtype=torch.bfloat16)
        cache = _gen((B, S, D), 802, dtype=torch.bfloat16)
        wsets = [(_gen((2 * F, D), 803 + 2 * r, 1 / 64, torch.bfloat16), _gen((D, F), 804 + 2 * r, 1 / 110, torch.bfloat16))
                 for r in range(nsets)]
        ws = torch.zeros(dlm.dlm_salient_ffn_workspace_size(dlm.DLM_BF16, n, D, F), dtype=torch.uint8, device="cuda")
        calls = [lambda w=w: dlm.dlm_salient_ffn(x, idx, offsets, n, w[0], w[1], cache, workspace=ws) for w in wsets]
        state = {"i": 0}

        def call():
            calls[state["i"] % nsets]()
            state["i"] += 1
        t = _time(call, 10)
        flops = 2.0 * n * D * 3 * F
        nbytes = 3 * F * D * 2 + n * D * 2 * 2 + n * F * 2 * 2
        out[name] = {"ms": t, "TFLOP/s": flops / t / 1e9, "frac_mfma": flops / (t / 1e3) / PEAK_BF16,
                     "GB/s": nbytes / (t / 1e3) / 1e9, "frac_hbm": nbytes / (t / 1e3) / PEAK_HBM,
                     "algorithmic_bytes": nbytes}
    return out


def extra_kl_lock(dlm, W, a=None):
    """SureLock's lock criterion at the confidence workload's size (B = 16,
    S = 1024, D = 4096, V = 32768, 230 evaluated positions per sequence): the
    two-step LM head (both steps' logits of every evaluated position in one
    pass over W_lm, 2 x 2 n D V flop), the KL merge and the per-sequence lock
    decision with the 50th-percentile gate."""
    import torch
    sh = W.LSP_COMMIT
    B, S, D, V = sh.B, sh.S, sh.D, sh.V
    S_gen = S - sh.prompt
    na = int(math.floor(sh.active_frac * S_gen))
    hc, hp = _gen((B, S, D), 511), _gen((B, S, D), 512)
    w = _gen((V, D), 513, scale=sh.w_std)
    g = torch.Generator(device="cuda")
    g.manual_seed(514)
    rows = [torch.sort(torch.randperm(S_gen, generator=g, device="cuda")[:na])[0] + sh.prompt for _ in range(B)]
    eidx, eoff = _packed_rows(rows)
    n = int(eidx.numel())
    kl = torch.zeros(B, S, dtype=torch.float32, device="cuda")
    mp = torch.zeros_like(kl)
    am = torch.zeros(B, S, dtype=torch.int32, device="cuda")
    lk = torch.zeros_like(kl)
    ws = torch.zeros(dlm.dlm_kl_lock_workspace_size(B, S, V, n), dtype=torch.uint8, device="cuda")
    call = lambda: dlm.dlm_kl_lock(hc, hp, w, eidx, eoff, n, 0.05, kl, mp, am, lk, gate_q=0.5, workspace=ws)
    t = _time(call, 10)
    f = 2.0 * 2.0 * n * D * V
    return {"workload": sh.name + " two-step KL lock", "n_evaluated": n, "ms": t, "TFLOP/s": f / t / 1e9,
            "frac": f / (t / 1e3) / PEAK_BF16, "tokens_per_s": n / (t / 1e3)}


def extra_scatter_rows(dlm, W, a=None):
    """The output-row scatter at the GQA loop's middle step (t = 32: 8480 of
    16384 rows of B = 8, S = 2048, rows of 32 x 128 bf16 = 8 KB): the packed
    rows are read and written into the [B, S, 4096] cache with dlm_scatter_rows.
    Two rotating sets (row blocks, caches and positions; 2 x 412 MB, more than
    the Infinity Cache).  Algorithmic bytes: 2 x n x 8 KB."""
    import torch
    sh = W.GQA_LOCK_LOOP
    B, S, Hq, hd = sh.B, sh.S, sh.Hq, sh.hd
    m = W.unlocked_count(S, 32, sh.steps, sh.lock_max)
    sets = []
    for r in range(2):
        g = torch.Generator(device="cuda")
        g.manual_seed(900 + r)
        rows = [torch.sort(torch.randperm(S, generator=g, device="cuda")[:m])[0] for _ in range(B)]
        idx, off = _packed_rows(rows)
        n = int(idx.numel())
        sets.append((idx, off, n, _gen((n, Hq * hd), 910 + r), _gen((B, S, Hq * hd), 920 + r)))
    calls = [lambda st=st: dlm.dlm_scatter_rows(st[3], st[0], st[1], st[2], st[4]) for st in sets]
    state = {"i": 0}

    def call():
        calls[state["i"] % 2]()
        state["i"] += 1
    t = _time(call, 20)
    n = sets[0][2]
    nbytes = 2 * n * Hq * hd * 2
    return {"workload": sh.name + " output rows of step t = 32", "rows": n, "row_bytes": Hq * hd * 2, "ms": t,
            "GB/s": nbytes / (t / 1e3) / 1e9, "frac": nbytes / (t / 1e3) / PEAK_HBM, "algorithmic_bytes": nbytes}


EXTRAS = (("one_layer_step_bf16_s1024", extra_one_layer_step), ("tiny_fp32", extra_tiny),
          ("colsum_top64", extra_colsum), ("lsp_commit", extra_lsp), ("kl_lock", extra_kl_lock),
          ("select_b8_asymptote", extra_select_b8), ("scatter_rows", extra_scatter_rows),
          ("nonsalient_dv_update", extra_dv_update), ("salient_ffn", extra_salient_ffn))


def cpu_baseline(W, seconds):
    """The fp64 oracle (untuned) on the same workload: denoising steps of the
    64-step GQA lock loop at full size, from the last step backwards
    (t = 63, 62, ...), until about `seconds` of oracle time.  Each step is the
    oracle's compaction, Q/K/V with K/V scatter, partial attention and output
    scatter; input generation is not timed.  The oracle's cost per recomputed
    row is about the same at every step (Q/K/V and attention both scale with
    the row count), so rows per second over the sample stand for the loop."""
    import numpy as np
    from oracle import dlm_oracle as O
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:
        threads = len(os.sched_getaffinity(0))
    inp = W.lock_loop_inputs(W.GQA_LOCK_LOOP)
    s = inp.shape
    scale = 1.0 / math.sqrt(s.hd)
    rng = np.random.default_rng(99)
    kc = rng.standard_normal((s.B, s.S, s.Hkv, s.hd))
    vc = rng.standard_normal((s.B, s.S, s.Hkv, s.hd))
    out = np.zeros((s.B, s.S, s.Hq * s.hd))
    rows, spent, steps = 0, 0.0, []
    for t in range(s.steps - 1, -1, -1):
        sc, x = inp.unlocked_scores(t), inp.hidden(t)
        t0 = time.perf_counter()
        idx, _, off = O.compact(sc, 0, s.S, 0.5)
        q, kc, vc = O.qkv_project_scatter(x, idx, off, inp.w_qkv, s.Hq, s.Hkv, s.hd, kc, vc)
        o, _ = O.partial_attention(q, idx, off, kc, vc, s.Hq, s.Hkv, scale)
        out = O.output_scatter(o, idx, off, out)
        spent += time.perf_counter() - t0
        rows += int(off[-1])
        steps.append(t)
        if spent >= seconds:
            break
    return {"value": rows / spent, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"{len(steps)} full-size oracle steps (t = {steps[0]} down to {steps[-1]}) of the "
                      f"{s.name} loop, {rows} rows, {spent:.1f} s of fp64 NumPy"}


if __name__ == "__main__":
    main()
