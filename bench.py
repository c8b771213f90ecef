"""Benchmark: per-layer sparse decode steps/s and achieved HBM bandwidth on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-sweep] [--no-cpu]

Workload (the headline line): a Llama-3.1-8B-shaped attention layer in bf16 -- B=1, 32
query heads, 8 KV heads, D=128, d'=32, L=32768 cached tokens, 1% heavy-hitter keys --
decoded with the raw TokenButler scorer, a fixed_50pc budget (top 50% of tokens) plus
sink 4 and window 64.  One step is one pass of the whole hot path for one layer:
project the appended token's key to K_imp, score all L tokens, select, attend over the
selected set.  Eight independent layer replicas (1.15 GiB of K/V/K_imp) are cycled so
that the 256 MB Infinity Cache cannot serve a step from the previous one.

Timing: W warm-up steps, then exactly K steps replayed from one captured HIP graph,
bracketed by torch.cuda.synchronize().  Per-call durations: where the runtime accepts
event-record nodes inside a captured graph, every call of the timed graph is bracketed by
them; ROCm refuses those, and then each call kind is timed with events on the launch
stream around a graph of K back-to-back calls of that kind (score and select as a pair,
since they hand over the first-digit histogram).  The roofline object uses the attention
call (split kernel + merge kernel), the dominant one: it moves ~79% of a step's
algorithmic bytes.

Extra fields: the same step at L = 128K and 256K (2 replicas each), and the CPU oracle
timed on a bounded sample of the same workload (one thread).  Inputs are seeded and
synthetic; nothing is read from disk except profiles/traffic_*.json (rocprof counters
recorded for the current kernel source, else traffic is null).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "sparse decode steps/s per layer at 32K–256K ctx; achieved HBM GB/s vs peak"
HBM_PEAK_GBS = 8000.0


def log(*a):
    print(*a, file=sys.stderr, flush=True)


class Layer:
    """Device buffers of one layer replica and the calls of one decode step."""

    def __init__(self, w, layer: int, L: int, device: str):
        import torch
        import synthetic
        import query_aware_sparse_imp_amd as qa
        self.qa, self.w, self.L = qa, w, L
        t0 = time.time()
        inp = synthetic.decode_layer(w, layer, L=L)
        self.host = inp
        self.k = inp["k_cache"].to(device)
        self.v = inp["v_cache"].to(device)
        self.q = inp["q"].to(device)
        self.wk = inp["w_k"].to(device)
        self.qi = inp["q_imp"].to(device)
        self.kimp = torch.empty(w.B, w.Hkv, L, w.dprime, dtype=w.dtype, device=device)
        qa.butler_project_keys(self.k, self.wk, self.kimp, 0, L)      # setup, untimed
        self.cap = w.cap(L)
        self.scores = torch.empty(w.B, w.Hkv, 1, L, dtype=torch.float32, device=device)
        self.idx = torch.empty(w.B, w.Hkv, 1, self.cap, dtype=torch.int32, device=device)
        self.count = torch.empty(w.B, w.Hkv, 1, dtype=torch.int32, device=device)
        # first-digit histogram handed from the scorer to the selection (kept zeroed by it)
        self.hist = torch.zeros(w.B, w.Hkv, 1, 2048, dtype=torch.int32, device=device)
        self.out = torch.empty(w.B, w.Hq, 1, w.D, dtype=torch.float32, device=device)
        log(f"  layer replica {layer} at L={L} ready in {time.time() - t0:.1f}s")

    def free(self):
        """Drop the device buffers (the host copy of the inputs stays)."""
        for name in ("k", "v", "q", "wk", "qi", "kimp", "scores", "idx", "count", "hist", "out"):
            setattr(self, name, None)

    def calls(self):
        qa, w, L = self.qa, self.w, self.L
        return [
            ("project", lambda: qa.butler_project_keys(self.k, self.wk, self.kimp, L - 1, 1)),
            ("score", lambda: qa.butler_score(qa.BUTLER_SCORE_RAW, self.qi, self.kimp,
                                              self.scores, Hkv=w.Hkv, L=L,
                                              radix_hist=self.hist)),
            ("select", lambda: qa.butler_select_topk(self.scores, w.budget_num, w.budget_den,
                                                     w.n_sink, w.n_window, self.count,
                                                     idx=self.idx, radix_hist=self.hist)),
            ("attn", lambda: qa.butler_sparse_decode_attn(self.q, self.k, self.v, self.out,
                                                          L=L, idx=self.idx, count=self.count,
                                                          softmax_scale=w.scale)),
        ]

    def algorithmic_bytes(self):
        """Bytes a step must move: the K_imp stream, the new key row and its K_imp row,
        the selected K and V rows, the index list written and read back, q and out."""
        w = self.w
        n_sel = int(self.count.sum().item())
        elt = 2 if w.dtype.itemsize == 2 else 4
        kimp = w.B * w.Hkv * self.L * w.dprime * elt
        proj = w.B * w.Hkv * (w.D + w.dprime) * elt + w.D * w.dprime * elt
        gather = n_sel * 2 * w.D * elt
        idx = n_sel * 4 * 2
        qo = w.B * w.Hq * w.D * (elt + 4)
        attn = gather + n_sel * 4 + qo
        return {"step": kimp + proj + gather + idx + qo, "attn": attn, "n_sel": n_sel}


def run_config(w, L, replicas, steps, warmup, device):
    import torch
    layers = [Layer(w, r, L, device) for r in range(replicas)]
    # eager warm-up: allocates every workspace before capture
    for lay in layers:
        for _, fn in lay.calls():
            fn()
    torch.cuda.synchronize()

    names = [n for n, _ in layers[0].calls()]

    def capture(nsteps, with_events):
        g = torch.cuda.CUDAGraph()
        evs = []
        with torch.cuda.graph(g):
            for s in range(nsteps):
                lay = layers[s % replicas]
                for name, fn in lay.calls():
                    if with_events:
                        e0 = torch.cuda.Event(enable_timing=True, external=True)
                        e1 = torch.cuda.Event(enable_timing=True, external=True)
                        e0.record()
                        fn()
                        e1.record()
                        evs.append((name, e0, e1))
                    else:
                        fn()
        return g, evs

    method = "graph-events"
    try:
        g_warm, _ = capture(max(warmup, 1), False)
        g_timed, evs = capture(steps, True)
    except Exception as exc:  # event nodes not capturable: time kernels by further graphs
        log(f"  external events in capture failed ({exc}); timing kernels per graph")
        method = "per-call-graphs"
        g_warm, _ = capture(max(warmup, 1), False)
        g_timed, evs = capture(steps, False)

    g_warm.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    g_timed.replay()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    elapsed = t1 - t0
    ab = [lay.algorithmic_bytes() for lay in layers]   # counts of the last timed steps

    per_kernel = {}
    if method == "graph-events":
        for name, e0, e1 in evs:
            per_kernel.setdefault(name, []).append(e0.elapsed_time(e1) * 1e3)   # us
    else:
        # Events around a graph of `steps` back-to-back calls of one kind.  The scorer and
        # the selection share the first-digit histogram (the scorer fills it, the selection
        # empties it), so they are timed together as one pair.
        groups = {"project": ["project"], "score+select": ["score", "select"], "attn": ["attn"]}
        for gname, members in groups.items():
            gk = torch.cuda.CUDAGraph()
            with torch.cuda.graph(gk):
                for s in range(steps):
                    calls = dict(layers[s % replicas].calls())
                    for m in members:
                        calls[m]()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            gk.replay()
            b.record()
            torch.cuda.synchronize()
            per_kernel[gname] = [a.elapsed_time(b) * 1e3 / steps]
    avg_us = {k: sum(v) / len(v) for k, v in per_kernel.items()}
    step_bytes = sum(a["step"] for a in ab) / len(ab)
    attn_bytes = sum(a["attn"] for a in ab) / len(ab)
    n_sel = sum(a["n_sel"] for a in ab) / len(ab)
    ms = elapsed * 1e3 / steps
    return {
        "L": L, "replicas": replicas, "steps": steps, "ms_per_step": ms,
        "steps_per_s": steps / elapsed, "timing": method,
        "kernel_us": {k: round(v, 3) for k, v in avg_us.items()},
        "step_bytes": step_bytes, "attn_bytes": attn_bytes, "selected_per_step": n_sel,
        "step_GBps": step_bytes / (ms * 1e-3) / 1e9,
        "attn_GBps": attn_bytes / (avg_us["attn"] * 1e-6) / 1e9,
    }, layers


def traffic_record(kernel_file: str, name: str):
    """rocprof FETCH_SIZE + WRITE_SIZE per launch recorded for the current source of the
    kernel, scaled by the copy-kernel calibration; None when absent or stale."""
    path = os.path.join(ROOT, "profiles", f"traffic_{name}.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    src = open(os.path.join(ROOT, "query_aware_sparse_imp_amd", "csrc", kernel_file), "rb").read()
    if rec.get("source_sha256") != hashlib.sha256(src).hexdigest():
        return None
    return rec.get("bytes_per_launch")


def cpu_baseline(layer, budget_s: float = 12.0):
    """The oracle's per-layer decode step on the host (one thread), on a bounded sample:
    as many whole steps of the same layer as fit in ~budget_s seconds (at least 2)."""
    import numpy as np
    from threadpoolctl import threadpool_limits
    import oracle
    w, inp, L = layer.w, layer.host, layer.L
    f64 = lambda t: t.float().double().numpy()
    k, v = f64(inp["k_cache"]), f64(inp["v_cache"])
    q = f64(inp["q"])[:, :, 0]
    wk = f64(inp["w_k"])
    qi = f64(inp["q_imp"])[:, :, 0, 0]
    with threadpool_limits(1):
        kimp = oracle.project_keys(k[:, :, :L - 1], wk, "bf16")
        n, t0 = 0, time.perf_counter()
        while True:
            new = oracle.project_keys(k[:, :, L - 1:L], wk, "bf16")
            kimp_all = np.concatenate([kimp, new], axis=2)
            oracle.decode_layer_step(q=q, k_cache=k, v_cache=v, L=L, num=w.budget_num,
                                     den=w.budget_den, n_sink=w.n_sink, n_window=w.n_window,
                                     scale=w.scale, Hkv=w.Hkv, mode="raw", q_imp_slot=qi,
                                     kimp=kimp_all)
            n += 1
            el = time.perf_counter() - t0
            if (el >= budget_s and n >= 2) or el > 3 * budget_s:
                break
    return {"value": n / el, "unit": "steps/s", "cores": 1, "kind": "oracle",
            "sample": f"{n} whole per-layer decode steps (project new key, score, select, "
                      f"attend; 8 KV heads, L={L}) of one layer replica, numpy float64, "
                      f"{el:.1f} s"}


def main(argv=None) -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=400)
    ap.add_argument("--warmup", type=int, default=40)
    ap.add_argument("--no-sweep", action="store_true")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--L", type=int, default=None)
    ap.add_argument("--copy-cal", action="store_true",
                    help="run a 256 MiB device copy first (HBM counter calibration)")
    a = ap.parse_args(argv)
    if a.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        return 2

    import torch
    import synthetic
    torch.cuda.set_device(0)
    dev = "cuda:0"
    w = synthetic.WORKLOADS[2]
    L = a.L or w.L
    if a.copy_cal:
        # a plain copy of known size: its FETCH_SIZE / WRITE_SIZE counters scale the
        # counters of the attention kernel to bytes
        src = torch.randn(64 * 1024 * 1024, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    log(f"[bench] {w.name}: L={L}, 8 replicas, steps={a.steps}, warmup={a.warmup}")
    head, layers = run_config(w, L, 8, a.steps, a.warmup, dev)
    host0 = layers[0]
    log(f"[bench] headline: {json.dumps(head)}")

    sweep = []
    if not a.no_sweep:
        for Ls in (131072, 262144):
            for lay in layers:
                if lay is not host0:
                    lay.free()
            layers = []
            torch.cuda.empty_cache()
            log(f"[bench] sweep L={Ls}")
            r, layers = run_config(w, Ls, 2, max(a.steps // 4, 20), max(a.warmup // 4, 4), dev)
            sweep.append({k: r[k] for k in ("L", "steps_per_s", "ms_per_step", "step_GBps",
                                            "attn_GBps", "kernel_us", "timing")})
            sweep[-1]["step_frac_of_hbm_peak"] = r["step_GBps"] / HBM_PEAK_GBS
            log(f"[bench] sweep result: {json.dumps(sweep[-1])}")
        for lay in layers:
            lay.free()
        layers = None

    cpu = None
    if not a.no_cpu:
        log("[bench] cpu baseline (oracle)")
        cpu = cpu_baseline(host0)
        log(f"[bench] cpu baseline: {json.dumps(cpu)}")

    attn_us = head["kernel_us"]["attn"]
    achieved = head["attn_bytes"] / (attn_us * 1e-6) / 1e9
    traffic = traffic_record("attn.hip", "attn_decode_L32768")
    line = {
        "metric": METRIC,
        "value": head["steps_per_s"],
        "unit": "steps/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"llama3.1-8b-shaped attention layer decode, L={L}",
                   "B": w.B, "Hq": w.Hq, "Hkv": w.Hkv, "D": w.D, "dprime": w.dprime,
                   "L": L, "scorer": "raw", "budget": f"{w.budget_num}/{w.budget_den}",
                   "sink": w.n_sink, "window": w.n_window, "layer_replicas": 8,
                   "parallelism": "none (1 GPU)"},
        "roofline": {"bound": "hbm", "kernel": "sparse decode attention call: attn_mfma_kernel + attn_merge_kernel",
                     "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": traffic,
                     "algorithmic_bytes_per_launch": head["attn_bytes"],
                     "avg_launch_us": attn_us, "timing": head["timing"]},
        "step_hbm": {"algorithmic_bytes": head["step_bytes"], "GB/s": head["step_GBps"],
                     "frac": head["step_GBps"] / HBM_PEAK_GBS},
        "kernel_us": head["kernel_us"],
        "sweep": sweep,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
