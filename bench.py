"""Benchmark of the per-layer cached denoising step on one MI355X.

A step is one pass of the whole hot path over one batch of synthetic input: fused refresh
(gather + QKV projection + RoPE + K/V scatter), block attention over the whole cache with the
column attention mass, and the drift check with the tracking update (FP8 caches have no drift
check).  Inputs are resident in HBM before timing starts; the cache and weights of several layer
instances are rotated so the 256 MB Infinity Cache cannot serve repeats.

Default workload: the LLaDA-8B-shaped bf16 layer, B=1, hidden 4096, 32 heads x 128, S=1024
(512 prompt + 512 response), 32 refreshed rows per step.

Prints one JSON line (metric, value in refreshed tokens/s, roofline of the dominant kernel,
the CPU oracle's rate on a bounded sample of the same workload).
"""
from __future__ import annotations

import argparse
import dataclasses
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

import synth  # noqa: E402

HBM_PEAK_GBS = 8000.0
MFMA_PEAK_TFLOPS = {"bf16": 2500.0, "f32": 157.3}
RIDGE = {"bf16": 2500e12 / 8000e9, "f32": 157.3e12 / 8000e9}
MALL_BYTES = 256 << 20
METRIC = "refreshed tokens/sec per layer step (QKV+RoPE+cache write+attn); % MFMA/HBM peak"


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def source_sha() -> str:
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "diffusion_kv_cache_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(f.encode() + fh.read())
    return h.hexdigest()[:16]


def work_model(wl):
    """Algorithmic bytes and flops per call (what the method must move / compute)."""
    B, n, H, Hq, Hkv, D, S = (wl.batch, wl.n_refresh, wl.hidden, wl.q_heads, wl.kv_heads,
                              wl.head_dim, wl.seq)
    M, N = B * n, wl.n_cols
    act = 4 if wl.act == "f32" else 2
    kv = {"f32": 4, "bf16": 2, "fp8": 1}[wl.cache]
    scales = 2 * 4 if wl.cache == "fp8" else 0
    refresh = dict(bytes=M * H * act + N * H * act + M * Hq * D * act + 2 * M * Hkv * D * kv
                   + M * Hkv * scales + M * 4,
                   flops=2 * M * N * H)
    attention = dict(bytes=2 * B * n * Hq * D * act + 2 * B * Hkv * S * D * kv
                     + B * Hkv * S * scales + B * Hq * n * 4,
                     flops=4 * B * Hq * n * S * D)
    tracking = wl.cache != "fp8"
    if tracking:  # mass pass re-reads K per head group and writes the mass
        attention["flops"] += 2 * B * Hq * n * S * D
        attention["bytes"] += B * Hq * S * 4
    k = wl.track_k
    drift = dict(bytes=(B * Hq * k * 2 * D * kv) * 3 + B * Hq * S * 4 + B * Hq * k * 8,
                 flops=6 * B * Hq * k * 2 * D)
    return {"refresh": refresh, "attention": attention, "drift": drift if tracking else None}


def roofline_entry(name, w, us, dtype):
    ai = w["flops"] / w["bytes"]
    if ai >= RIDGE[dtype]:
        achieved = w["flops"] / (us * 1e-6) / 1e12
        peak = MFMA_PEAK_TFLOPS[dtype]
        return {"kernel": name, "bound": "mfma", "achieved": round(achieved, 2), "peak": peak,
                "unit": "TFLOP/s", "frac": round(achieved / peak, 4),
                "algorithmic_flops": w["flops"], "avg_us": round(us, 3)}
    achieved = w["bytes"] / (us * 1e-6) / 1e9
    return {"kernel": name, "bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
            "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
            "algorithmic_bytes": w["bytes"], "avg_us": round(us, 3)}


def measured_traffic(workload: str, kernel: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it was taken on
    the current kernel sources."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    e = t.get(workload, {}).get(kernel)
    if not e or e.get("source_sha") != source_sha():
        return None
    return e.get("bytes_per_launch")


class Layer:
    def __init__(self, dkv, torch, wl, w, h_prev, idx_t):
        self.cache = dkv.Cache(wl.batch, wl.kv_heads, wl.seq, wl.head_dim,
                               {"f32": dkv.DLLM_F32, "bf16": dkv.DLLM_BF16,
                                "fp8": dkv.DLLM_FP8_E4M3}[wl.cache])
        self.w = w.clone()
        dev = h_prev.device
        all_rows = torch.arange(wl.seq, dtype=torch.int32, device=dev).repeat(wl.batch, 1)
        q_all = torch.empty((wl.batch, wl.seq, wl.q_heads, wl.head_dim), dtype=h_prev.dtype,
                            device=dev)
        dkv.dllm_refresh_qkv_rope_scatter(self.cache, h_prev, all_rows, self.w, wl.q_heads,
                                          wl.rope_base, q_all)
        del q_all
        k = wl.track_k
        self.track = wl.cache != "fp8"
        if self.track:
            tdt = torch.float32 if wl.cache == "f32" else torch.bfloat16
            self.T = torch.full((wl.batch, wl.q_heads, k), -1, dtype=torch.int32, device=dev)
            self.buf = torch.zeros((wl.batch, wl.q_heads, k, 2, wl.head_dim), dtype=tdt, device=dev)


def run(args):
    import torch

    import diffusion_kv_cache_amd as dkv

    wl = synth.WORKLOADS[args.config]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    act = torch.float32 if wl.act == "f32" else torch.bfloat16
    log(f"[bench] workload {wl.name}: {wl.description}")
    t0 = time.time()
    inp = synth.make_inputs(wl)
    log(f"[bench] inputs generated in {time.time() - t0:.1f}s")
    h_prev = torch.from_numpy(inp.hidden_prev).to(dev).to(act)
    h_cur = h_prev.clone()
    idx_t = torch.from_numpy(inp.idx).to(dev)
    h_cur[torch.arange(wl.batch, device=dev)[:, None], idx_t.long()] = \
        torch.from_numpy(inp.new_rows).to(dev).to(act)
    w = torch.from_numpy(inp.w).to(dev).to(act)
    B, n, S, Hq, D, k = wl.batch, wl.n_refresh, wl.seq, wl.q_heads, wl.head_dim, wl.track_k
    M = B * n

    per_layer = w.numel() * w.element_size() + dkv.dllm_cache_bytes(
        dkv.CacheDesc(B, wl.kv_heads, S, D, {"f32": 0, "bf16": 1, "fp8": 2}[wl.cache],
                      D if wl.cache == "fp8" else 0))
    L = args.layers or max(3, math.ceil(3 * MALL_BYTES / per_layer))
    log(f"[bench] {L} layer instances x {per_layer / 2**20:.1f} MiB")
    layers = [Layer(dkv, torch, wl, w, h_prev, idx_t) for _ in range(L)]

    q = torch.empty((B, n, Hq, D), dtype=act, device=dev)
    out = torch.empty_like(q)
    lse = torch.empty((B, Hq, n), dtype=torch.float32, device=dev)
    mass = torch.empty((B, Hq, S), dtype=torch.float32, device=dev)
    sigma = torch.empty((B, Hq), dtype=torch.float32, device=dev)
    refresh = torch.empty((B,), dtype=torch.uint8, device=dev)
    rws_bytes = dkv.dllm_refresh_workspace_bytes(layers[0].cache, wl.hidden,
                                                 dkv.DLLM_F32 if wl.act == "f32" else dkv.DLLM_BF16,
                                                 n, Hq)
    rws = torch.empty(rws_bytes, dtype=torch.uint8, device=dev) if rws_bytes else None
    ws = torch.empty(max(1, dkv.dllm_attention_workspace_bytes(layers[0].cache, Hq, n)),
                     dtype=torch.uint8, device=dev)
    scale = 1.0 / math.sqrt(D)
    track = layers[0].track

    # Previous step (untimed, on H_prev): the tracking sets come from its attention mass.
    for ly in layers:
        if track:
            dkv.dllm_refresh_qkv_rope_scatter(ly.cache, h_prev, idx_t, ly.w, Hq, wl.rope_base, q,
                                              rws)
            dkv.dllm_block_attention(ly.cache, q, Hq, scale, out, lse, mass, ws)
            dkv.dllm_drift_check(ly.cache, Hq, k, wl.gamma, ly.T, ly.buf, mass, sigma, refresh)
    torch.cuda.synchronize()

    names = ["refresh", "attention"] + (["drift"] if track else [])
    calls = {
        "refresh": lambda ly: dkv.dllm_refresh_qkv_rope_scatter(ly.cache, h_cur, idx_t, ly.w, Hq,
                                                                wl.rope_base, q, rws),
        "attention": lambda ly: dkv.dllm_block_attention(ly.cache, q, Hq, scale, out, lse,
                                                         mass if track else None, ws),
        "drift": lambda ly: dkv.dllm_drift_check(ly.cache, Hq, k, wl.gamma, ly.T, ly.buf, mass,
                                                 sigma, refresh),
    }

    def step(ly):
        for nm in names:
            calls[nm](ly)

    for s in range(args.warmup):
        step(layers[s % L])
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record()
    for s in range(args.steps):
        step(layers[(args.warmup + s) % L])
    end.record()
    torch.cuda.synchronize()
    total_ms = start.elapsed_time(end)
    ms_per_step = total_ms / args.steps
    value = M / (ms_per_step * 1e-3)

    # Average duration of each call: the call alone, `burst` times back to back on the launch
    # stream (layers rotating as in the steps), between two events.  Events between the calls
    # of a step would each add a bubble of a few microseconds to the timeline they measure.
    # A spin kernel ahead of the first event keeps the GPU busy while the host enqueues the
    # burst, so host-side launch cost does not show in the interval (short calls would
    # otherwise be timed at the rate the host issues them).
    burst = max(10, args.steps)
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    torch.cuda._sleep(1 << 20)
    e1.record()
    torch.cuda.synchronize()
    spin_per_ms = (1 << 20) / e0.elapsed_time(e1)
    per = {}
    for nm in names:
        t0 = time.perf_counter()
        for r in range(burst):
            calls[nm](layers[r % L])
        host_ms = (time.perf_counter() - t0) * 1e3
        torch.cuda.synchronize()
        torch.cuda._sleep(int(spin_per_ms * (2.0 * host_ms + 0.2)))
        e0.record()
        for r in range(burst):
            calls[nm](layers[r % L])
        e1.record()
        torch.cuda.synchronize()
        per[nm] = e0.elapsed_time(e1) / burst * 1e3
    log(f"[bench] {args.steps} steps: {ms_per_step * 1e3:.1f} us/step; per call (us, {burst} back to "
        f"back): " + ", ".join(f"{k_}={v:.1f}" for k_, v in per.items()))

    works = work_model(wl)
    dtype = "f32" if wl.act == "f32" else "bf16"
    entries = {nm: roofline_entry(nm, works[nm], per[nm], dtype) for nm in names}
    for nm, e in entries.items():
        log(f"[bench] {nm}: {e['achieved']} {e['unit']} ({100 * e['frac']:.1f}% of {e['bound']} peak)")
    dom = max(names, key=lambda nm: per[nm])
    roof = dict(entries[dom])
    roof["traffic"] = measured_traffic(wl.name, dom)

    result = {
        "metric": METRIC, "value": round(value, 1), "unit": "refreshed tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32" if wl.act == "f32" else "bf16",
        "data": "synthetic (seeded, shaped like the workload; random-init weights)",
        "config": {"workload": f"{wl.name}: {wl.description}", "global_batch": B, "seq_len": S,
                   "refreshed_per_seq": n, "hidden": wl.hidden, "q_heads": Hq,
                   "kv_heads": wl.kv_heads, "head_dim": D, "cache_dtype": wl.cache,
                   "tracking": track, "layer_instances": L, "parallelism": "none (1 GPU)"},
        "per_call_us": {k_: round(v, 2) for k_, v in per.items()},
        "per_call_back_to_back": burst,
        "rooflines": entries,
        "roofline": roof,
    }
    del layers
    torch.cuda.empty_cache()
    if args.copy_calibration:
        # A plain device copy of known size, so HBM byte counters read under a profiler can be
        # scaled by what they report for a copy (reads = writes = the buffer size).
        nb = args.copy_calibration << 20
        src = torch.empty(nb, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        result["copy_calibration_bytes"] = nb
        del src, dst
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(wl, inp, args.cpu_budget)
    print(json.dumps(result), flush=True)


def cpu_baseline(wl, inp, budget_s: float):
    """The CPU oracle (fp64, plain loops) timed on this host's cores on a bounded sample of the
    same workload: the cached step of the first `nb` sequences (prefill untimed)."""
    cores = len(os.sched_getaffinity(0))
    os.environ["OMP_NUM_THREADS"] = str(cores)
    import oracle

    nb = {"c1": 1, "c2": 1, "c3": 2, "c4": 1, "c5": 1}.get(wl.name, 1)
    ws = dataclasses.replace(wl, batch=nb)
    sub = synth.Inputs(ws, inp.w, inp.hidden_prev[:nb], inp.new_rows[:nb], inp.idx[:nb])
    h_cur = sub.hidden_cur()
    t0 = time.time()
    cache = oracle.prefill(ws, sub.hidden_prev, sub.w)
    track = wl.cache != "fp8"
    if track:  # previous step's tracking set (untimed)
        qp = oracle.queries(ws, sub.hidden_prev, sub.w, sub.idx)
        _, _, mp = oracle.attend(ws, qp, cache, want_mass=True)
        T, buf = oracle.track(cache, mp, ws.track_k)
    log(f"[cpu] oracle setup {time.time() - t0:.1f}s on {cores} threads")
    runs, t_total = 0, 0.0
    while runs == 0 or t_total < budget_s / 2:
        t0 = time.time()
        oracle.refresh_rows(cache, h_cur, sub.w, sub.idx)
        q = oracle.queries(ws, h_cur, sub.w, sub.idx)
        _, _, m = oracle.attend(ws, q, cache, want_mass=track)
        if track:
            oracle.drift(buf, T, cache.k, cache.v, float(np.float32(ws.gamma)))
            oracle.track(cache, m, ws.track_k)
        t_total += time.time() - t0
        runs += 1
    rate = runs * nb * wl.n_refresh / t_total
    log(f"[cpu] {runs} oracle step(s) in {t_total:.2f}s: {rate:.1f} tokens/s")
    return {"value": round(rate, 2), "unit": "refreshed tokens/s", "cores": cores,
            "kind": "oracle",
            "sample": f"cached step (refresh + attention{' + mass + drift + top-k' if track else ''})"
                      f" of {nb} of {wl.batch} sequence(s), {runs} run(s), prefill untimed, "
                      f"fp64 C oracle with OpenMP"}


def main():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", default="c2", choices=sorted(synth.WORKLOADS))
    ap.add_argument("--layers", type=int, default=0, help="layer instances to rotate (0: auto)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=20.0)
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MiB",
                    help="after timing, run a plain device copy of this size (counter scaling)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU: the library has no multi-GPU path; each GPU serves its own sequences (--gpus {args.gpus} "
              f"requested).", file=sys.stderr)
        sys.exit(2)
    run(args)


if __name__ == "__main__":
    main()
