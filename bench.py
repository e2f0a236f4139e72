"""Benchmark of the per-layer cached denoising step on one MI355X.

A step is one pass of the whole hot path over one batch of synthetic input: fused refresh
(gather + QKV projection + RoPE + K/V scatter), block attention over the whole cache with the
column attention mass, and the drift check with the tracking update, its decision taken in the
same launch (the long-context FP8 workload names no drift test, so its step has none).  Inputs
are resident in HBM before timing starts; the cache and weights of several layer instances are
rotated so the 256 MB Infinity Cache cannot serve repeats.

Default workload: the LLaDA-8B-shaped bf16 layer, B=1, hidden 4096, 32 heads x 128, S=1024
(512 prompt + 512 response), 32 refreshed rows per step.

Prints one JSON line (metric, value in refreshed tokens/s, roofline of the dominant kernel,
the CPU oracle's rate on a bounded sample of the same workload).  The other workloads (batched,
GQA scattered refresh with drift, long-context FP8) are measured in the same run and reported
under "configs", each with its step time, rate and per-call rooflines.
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
MFMA_PEAK_TFLOPS = {"bf16": 2500.0, "f32": 157.3, "fp8": 5000.0}
RIDGE = {"bf16": 2500e12 / 8000e9, "f32": 157.3e12 / 8000e9, "fp8": 5000e12 / 8000e9}
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


def measure(args, wl):
    """Time K steps of workload `wl` (after W warm-up steps) and each call of the step alone;
    returns the per-workload record and the host inputs (for the CPU baseline)."""
    import torch

    import diffusion_kv_cache_amd as dkv

    dev = torch.device("cuda:0")
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
    dws = dkv.drift_workspace(B, dev) if track else None  # decision in the drift launch

    # Previous step (untimed, on H_prev): the tracking sets come from its attention mass.
    for ly in layers:
        if track:
            dkv.dllm_refresh_qkv_rope_scatter(ly.cache, h_prev, idx_t, ly.w, Hq, wl.rope_base, q,
                                              rws)
            dkv.dllm_block_attention(ly.cache, q, Hq, scale, out, lse, mass, ws)
            dkv.dllm_drift_check(ly.cache, Hq, k, wl.gamma, ly.T, ly.buf, mass, sigma, refresh,
                                 dws)
    torch.cuda.synchronize()

    names = ["refresh", "attention"] + (["drift"] if track else [])
    calls = {
        "refresh": lambda ly: dkv.dllm_refresh_qkv_rope_scatter(ly.cache, h_cur, idx_t, ly.w, Hq,
                                                                wl.rope_base, q, rws),
        "attention": lambda ly: dkv.dllm_block_attention(ly.cache, q, Hq, scale, out, lse,
                                                         mass if track else None, ws),
        "drift": lambda ly: dkv.dllm_drift_check(ly.cache, Hq, k, wl.gamma, ly.T, ly.buf, mass,
                                                 sigma, refresh, dws),
    }

    def step(ly):
        for nm in names:
            calls[nm](ly)

    t0 = time.perf_counter()
    for s_ in range(args.warmup):
        step(layers[s_ % L])
    host_step_ms = (time.perf_counter() - t0) * 1e3 / max(1, args.warmup)
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    per_ms = spin_rate(torch)
    # The K steps are timed between two events on the launch stream.  A spin kernel ahead of
    # the first event keeps the GPU busy while Python enqueues the steps (about as long as the
    # GPU runs them on the small workloads), so the interval is the GPU's, not the launcher's.
    # The rate with the launcher in the loop is timed first and reported beside it.
    def timed_steps(spin_len_ms):
        if spin_len_ms:
            torch.cuda._sleep(int(per_ms * spin_len_ms))
        start.record()
        for s_ in range(args.steps):
            step(layers[(args.warmup + s_) % L])
        end.record()
        torch.cuda.synchronize()
        return start.elapsed_time(end) / args.steps
    ms_per_step_host = timed_steps(0.0)
    ms_per_step = timed_steps(spin_ms(host_step_ms * args.steps, ms_per_step_host * args.steps))
    value = M / (ms_per_step * 1e-3)

    # Average duration of each call: the call alone, `burst` times back to back on the launch
    # stream (layers rotating as in the steps), between two events.  Events between the calls
    # of a step would each add a bubble of a few microseconds to the timeline they measure.
    # A spin kernel ahead of the first event keeps the GPU busy while the host enqueues the
    # burst, so host-side launch cost does not show in the interval (short calls would
    # otherwise be timed at the rate the host issues them).
    burst = max(10, args.steps)
    per = {nm: burst_us(torch, calls[nm], burst, layers) for nm in names}
    log(f"[bench] {wl.name}: {args.steps} steps: {ms_per_step * 1e3:.1f} us/step "
        f"({ms_per_step_host * 1e3:.1f} with the Python launcher in the loop, "
        f"{host_step_ms * 1e3:.1f} us of host time per step); per call (us, "
        f"{burst} back to back): " + ", ".join(f"{k_}={v:.1f}" for k_, v in per.items()))

    works = work_model(wl)
    dtype = "f32" if wl.act == "f32" else "bf16"
    entries = {nm: roofline_entry(nm, works[nm], per[nm], dtype) for nm in names}
    for nm, e in entries.items():
        log(f"[bench] {wl.name} {nm}: {e['achieved']} {e['unit']} ({100 * e['frac']:.1f}% of "
            f"{e['bound']} peak)")
    dom = max(names, key=lambda nm: per[nm])
    roof = dict(entries[dom])
    roof["traffic"] = measured_traffic(wl.name, dom)
    for nm, e in entries.items():
        e["traffic"] = measured_traffic(wl.name, nm)
    rec = {
        "value": round(value, 1), "unit": "refreshed tokens/s",
        "ms_per_step": round(ms_per_step, 5),
        "ms_per_step_with_launcher": round(ms_per_step_host, 5),
        "workload": f"{wl.name}: {wl.description}",
        "global_batch": B, "seq_len": S, "refreshed_per_seq": n, "hidden": wl.hidden,
        "q_heads": Hq, "kv_heads": wl.kv_heads, "head_dim": D, "cache_dtype": wl.cache,
        "tracking": track, "layer_instances": L,
        "per_call_us": {k_: round(v, 2) for k_, v in per.items()},
        "per_call_back_to_back": burst,
        "rooflines": entries,
        "roofline": roof,
    }
    del layers
    torch.cuda.empty_cache()
    return rec, inp


def spin_ms(host_ms: float, gpu_ms: float) -> float:
    """Length of the spin kernel queued ahead of a timed region whose host enqueue takes host_ms
    and whose GPU work takes about gpu_ms: a 0.5 ms head start, plus twice the time by which the
    host would fall behind the GPU.  Where the host enqueues faster than the GPU runs, the
    spin stays short: a long near-idle spin lets the chip lower its clocks, and the work after
    it then starts slow (measured: 2-3% on the MFMA-bound workloads)."""
    return 0.5 + 2.0 * max(0.0, host_ms - 0.5 * gpu_ms)


def spin_rate(torch):
    """Spin-kernel cycles per millisecond on this GPU."""
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    torch.cuda._sleep(1 << 20)
    e1.record()
    torch.cuda.synchronize()
    return (1 << 20) / e0.elapsed_time(e1)


def burst_us(torch, fn, count, layers):
    """Average duration of fn(layer), `count` calls back to back with the layers rotating,
    between two events on the launch stream; a spin kernel ahead of the first event keeps the
    GPU busy while the host enqueues (host launch cost stays out of the interval)."""
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    per_ms = spin_rate(torch)
    t0 = time.perf_counter()
    e0.record()
    for r in range(count):
        fn(layers[r % len(layers)])
    e1.record()
    host_ms = (time.perf_counter() - t0) * 1e3
    torch.cuda.synchronize()
    gpu_ms = e0.elapsed_time(e1)                 # with the launcher in the loop: an upper bound
    torch.cuda._sleep(int(per_ms * spin_ms(host_ms, gpu_ms)))
    e0.record()
    for r in range(count):
        fn(layers[r % len(layers)])
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / count * 1e3


def measure_facache(args, wl):
    """FACache attention of every row (first layer of a block step) on the workload's shape,
    the block being the refreshed rows: the build step, a reuse step, and plain attention of
    every row for comparison."""
    import torch

    import diffusion_kv_cache_amd as dkv

    dev = torch.device("cuda:0")
    B, n, S, Hq, Hkv, D = wl.batch, wl.n_refresh, wl.seq, wl.q_heads, wl.kv_heads, wl.head_dim
    inp = synth.make_inputs(wl)
    h_prev = torch.from_numpy(inp.hidden_prev).to(dev).to(torch.bfloat16)
    w = torch.from_numpy(inp.w).to(dev).to(torch.bfloat16)
    idx = torch.from_numpy(inp.idx).to(dev)
    starts = idx[:, 0].contiguous()
    all_rows = torch.arange(S, dtype=torch.int32, device=dev).repeat(B, 1)
    state_bytes = B * Hq * S * (D + 2) * 4
    per = 2 * B * Hkv * S * D * 2 + 2 * B * S * Hq * D * 2 + state_bytes
    L = max(3, math.ceil(3 * MALL_BYTES / per))

    class FL:
        pass

    layers = []
    for _ in range(L):
        ly = FL()
        ly.cache = dkv.Cache(B, Hkv, S, D, dkv.DLLM_BF16)
        ly.q_all = torch.empty((B, S, Hq, D), dtype=torch.bfloat16, device=dev)
        dkv.dllm_refresh_qkv_rope_scatter(ly.cache, h_prev, all_rows, w, Hq, wl.rope_base, ly.q_all)
        ly.q_blk = ly.q_all[:, wl.block_start:wl.block_start + n].contiguous()
        ly.state = torch.empty((state_bytes // 4,), dtype=torch.float32, device=dev)
        ly.out = torch.empty((B, S, Hq, D), dtype=torch.bfloat16, device=dev)
        ly.lse = torch.empty((B, Hq, S), dtype=torch.float32, device=dev)
        dkv.dllm_facache_attention(ly.cache, ly.q_all, ly.q_blk, starts, Hq, 1 / math.sqrt(D),
                                   ly.state, True, ly.out, ly.lse)
        layers.append(ly)
    ws = torch.empty(max(1, dkv.dllm_attention_workspace_bytes(layers[0].cache, Hq, S)),
                     dtype=torch.uint8, device=dev)
    scale = 1 / math.sqrt(D)
    calls = {
        "build": lambda ly: dkv.dllm_facache_attention(ly.cache, ly.q_all, ly.q_blk, starts, Hq,
                                                       scale, ly.state, True, ly.out, ly.lse),
        "reuse": lambda ly: dkv.dllm_facache_attention(ly.cache, ly.q_all, ly.q_blk, starts, Hq,
                                                       scale, ly.state, False, ly.out, ly.lse),
        "plain_all_rows": lambda ly: dkv.dllm_block_attention(ly.cache, ly.q_all, Hq, scale,
                                                              ly.out, ly.lse, None, ws),
    }
    for fn in calls.values():
        for r in range(3):
            fn(layers[r % L])
    torch.cuda.synchronize()
    count = max(10, args.steps)
    us = {k_: burst_us(torch, fn, count, layers) for k_, fn in calls.items()}
    q_out = 2 * B * S * Hq * D * 2 + B * Hq * S * 4          # every row's Q in, output + lse out
    kv = 2 * B * Hkv * S * D * 2
    st_inv = B * Hq * (S - n) * (D + 2) * 4                   # the invariant rows' state
    works = {
        "plain_all_rows": dict(bytes=q_out + kv, flops=4 * B * Hq * S * S * D),
        "build": dict(bytes=q_out + kv + st_inv, flops=4 * B * Hq * S * S * D),
        "reuse": dict(bytes=q_out + kv + st_inv + B * n * Hq * D * 2,
                      flops=4 * B * Hq * n * S * D + 4 * B * Hq * (S - n) * n * D),
    }
    entries = {k_: roofline_entry(k_, works[k_], us[k_], "bf16") for k_ in calls}
    log(f"[bench] facache on {wl.name}: " + ", ".join(f"{k_}={v:.1f} us" for k_, v in us.items()))
    del layers
    torch.cuda.empty_cache()
    return {"workload": f"{wl.name} shape, every row's attention, block = the refreshed rows",
            "layer_instances": L, "per_call_us": {k_: round(v, 2) for k_, v in us.items()},
            "per_call_back_to_back": count, "rooflines": entries,
            "reuse_speedup_vs_plain": round(us["plain_all_rows"] / us["reuse"], 3)}


def measure_schedule(args):
    """One denoising step over L synthetic layers of the GQA workload's shape under the
    Elastic-Cache layer schedule with the similarity-chosen partial refresh: per layer, one
    call (similarity choice -> row schedule -> variable-length refresh -> attention with mass
    -> drift test -> feature copy), every decision on the device.  Each sequence's states move
    from a planted layer on, so the drift fires there and the later layers of that sequence
    refresh every row.  Beside it, the same layers with every row recomputed (refresh and
    attention of all S rows), the step that caching replaces."""
    import torch

    import diffusion_kv_cache_amd as dkv

    dev = torch.device("cuda:0")
    base = synth.WORKLOADS["c4"]
    L = args.schedule_layers
    wl = dataclasses.replace(base, name="schedule", seed=2001)
    triggers = [1, L, 2, L, 3, L, L, 1][:wl.batch]
    B, S, H, Hq, Hkv, D = wl.batch, wl.seq, wl.hidden, wl.q_heads, wl.kv_heads, wl.head_dim
    window, k_sel, k_track = wl.window, wl.subset, wl.track_k
    log(f"[bench] schedule: {L} layers of the {base.name} shape, triggers {triggers}")
    t0 = time.time()
    st = synth.layer_stack(wl, L, triggers, window)
    log(f"[bench] schedule inputs generated in {time.time() - t0:.1f}s")
    bf = torch.bfloat16
    cap = B * S
    scale = 1.0 / math.sqrt(D)
    all_rows = torch.arange(S, dtype=torch.int32, device=dev).repeat(B, 1)
    rows0 = torch.from_numpy(np.stack([np.arange(w0, w0 + window) for w0 in st.window_start])
                             .astype(np.int32)).to(dev)
    ws_d = torch.from_numpy(st.window_start).to(dev)
    q_all = torch.empty((B, S, Hq, D), dtype=bf, device=dev)
    out_all = torch.empty_like(q_all)
    lse_all = torch.empty((B, Hq, S), dtype=torch.float32, device=dev)
    layers = []
    for l in range(L):
        ly = {"cache": dkv.Cache(B, Hkv, S, D, dkv.DLLM_BF16),
              "w": torch.from_numpy(st.w[l]).to(dev).to(bf),
              "hcur": torch.from_numpy(st.hidden_cur[l]).to(dev).to(bf)}
        hp = torch.from_numpy(st.hidden_prev[l]).to(dev).to(bf)
        dkv.dllm_refresh_qkv_rope_scatter(ly["cache"], hp, all_rows, ly["w"], Hq, wl.rope_base,
                                          q_all)
        q0 = torch.empty((B, window, Hq, D), dtype=bf, device=dev)
        dkv.dllm_refresh_qkv_rope_scatter(ly["cache"], hp, rows0, ly["w"], Hq, wl.rope_base, q0)
        mass0 = torch.empty((B, Hq, S), dtype=torch.float32, device=dev)
        dkv.dllm_block_attention(ly["cache"], q0, Hq, scale, torch.empty_like(q0),
                                 torch.empty((B, Hq, window), dtype=torch.float32, device=dev),
                                 mass0)
        ly["T"] = torch.full((B, Hq, k_track), -1, dtype=torch.int32, device=dev)
        ly["buf"] = torch.zeros((B, Hq, k_track, 2, D), dtype=bf, device=dev)
        dkv.dllm_drift_check(ly["cache"], Hq, k_track, wl.gamma, ly["T"], ly["buf"], mass0,
                             torch.empty((B, Hq), dtype=torch.float32, device=dev),
                             torch.empty((B,), dtype=torch.uint8, device=dev))
        ly["feat"] = hp
        ly["snap"] = {k_: v.clone() for k_, v in (("k", ly["cache"].k), ("v", ly["cache"].v),
                                                   ("T", ly["T"]), ("buf", ly["buf"]),
                                                   ("feat", ly["feat"]))}
        layers.append(ly)
    torch.cuda.synchronize()
    full = torch.zeros((B,), dtype=torch.uint8, device=dev)
    decision = torch.zeros((B,), dtype=torch.uint8, device=dev)
    o = dict(step_rows=torch.empty((B, window + k_sel), dtype=torch.int32, device=dev),
             rows=torch.empty((cap,), dtype=torch.int32, device=dev),
             q=torch.empty((cap, Hq, D), dtype=bf, device=dev),
             out=torch.empty((cap, Hq, D), dtype=bf, device=dev),
             lse=None, attn_mass=torch.empty((B, Hq, S), dtype=torch.float32, device=dev),
             sigma=torch.empty((B, Hq), dtype=torch.float32, device=dev))
    ws = torch.empty(dkv.dllm_layer_step_workspace_bytes(layers[0]["cache"], H, Hq),
                     dtype=torch.uint8, device=dev)
    cus = torch.empty((L, B + 1), dtype=torch.int32, device=dev)

    def restore():
        for ly in layers:
            ly["cache"].k.copy_(ly["snap"]["k"])
            ly["cache"].v.copy_(ly["snap"]["v"])
            ly["T"].copy_(ly["snap"]["T"])
            ly["buf"].copy_(ly["snap"]["buf"])
            ly["feat"].copy_(ly["snap"]["feat"])
        full.zero_()
        decision.zero_()

    def step():
        for l, ly in enumerate(layers):
            dkv.dllm_elastic_layer_step(
                ly["cache"], hidden_cur=ly["hcur"], hidden_feat=ly["feat"], w_qkv=ly["w"],
                window_start=ws_d, track_idx=ly["T"], track_buf=ly["buf"], full=full,
                decision=decision, num_q_heads=Hq, lo=wl.prompt, window=window,
                k_select=k_sel, k_track=k_track, rope_base=wl.rope_base, softmax_scale=scale,
                gamma=wl.gamma, workspace=ws, cu_rows=cus[l], **o)

    def full_recompute():
        for ly in layers:
            dkv.dllm_refresh_qkv_rope_scatter(ly["cache"], ly["hcur"], all_rows, ly["w"], Hq,
                                              wl.rope_base, q_all)
            dkv.dllm_block_attention(ly["cache"], q_all, Hq, scale, out_all, lse_all, None)

    reps = max(3, min(args.steps, 10))
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    times = []
    for r in range(reps + 1):
        restore()
        torch.cuda.synchronize()
        e0.record()
        step()
        e1.record()
        torch.cuda.synchronize()
        if r:
            times.append(e0.elapsed_time(e1) * 1e3)
    rows_per_layer = [int(x) for x in cus[:, -1].cpu().tolist()]
    full_flags = full.cpu().tolist()
    us = float(np.median(times))
    full_recompute()
    torch.cuda.synchronize()
    ftimes = []
    for _ in range(reps):
        e0.record()
        full_recompute()
        e1.record()
        torch.cuda.synchronize()
        ftimes.append(e0.elapsed_time(e1) * 1e3)
    fus = float(np.median(ftimes))
    restore()
    log(f"[bench] schedule: {us:.1f} us/step over {L} layers, rows per layer {rows_per_layer}; "
        f"every row recomputed: {fus:.1f} us")
    del layers
    torch.cuda.empty_cache()
    return {"workload": f"{L} synthetic layers of the {base.name} shape ({base.description}); "
                        f"per step window {window} + {k_sel} least-similar response rows + "
                        f"tracked rows, every row after a drift; states move from layers "
                        f"{triggers}",
            "layers": L, "us_per_step": round(us, 1), "refreshed_rows_per_layer": rows_per_layer,
            "refreshed_tokens_per_s": round(sum(rows_per_layer) / (us * 1e-6), 1),
            "full_after_step": full_flags,
            "every_row_recomputed_us": round(fus, 1),
            "speedup_vs_every_row": round(fus / us, 3), "repeats": reps}


def measure_fp8_linear(args):
    """The per-group FP8 linear layer (FFN Gate-Up and FF-Out, LaCache Methodology 2) on the
    refreshed rows of the LLaDA-8B-shaped (hidden 4096, FFN 12288) and Dream-7B-shaped
    (hidden 3584, FFN 18944) steps, beside torch's bf16 matmul of the same shape."""
    import torch

    import diffusion_kv_cache_amd as dkv

    dev = torch.device("cuda:0")
    shapes = [("c2 rows, LLaDA gate-up", 32, 2 * 12288, 4096),
              ("c2 rows, LLaDA ff-out", 32, 4096, 12288),
              ("c3 rows, LLaDA gate-up", 1024, 2 * 12288, 4096),
              ("c3 rows, LLaDA ff-out", 1024, 4096, 12288),
              ("c4 rows, Dream gate-up", 2304, 2 * 18944, 3584),
              ("c4 rows, Dream ff-out", 2304, 3584, 18944)]
    out = {}
    g = torch.Generator(device=dev)
    g.manual_seed(3)
    for name, M, N, K in shapes:
        inst = max(2, math.ceil(3 * MALL_BYTES / (N * K)))
        x = (torch.randn((M, K), generator=g, device=dev)).to(torch.bfloat16)
        ws = []
        for _ in range(inst):
            w = (torch.randn((N, K), generator=g, device=dev) * 0.02).to(torch.bfloat16)
            wc = torch.empty((N, K), dtype=torch.uint8, device=dev)
            sc = torch.empty((N // 128, K // 128), dtype=torch.float32, device=dev)
            dkv.dllm_fp8_quantize_weight(w, wc, sc)
            ws.append((wc, sc, w if inst * N * K * 2 < (8 << 30) else None))
        y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
        wsp = torch.empty(dkv.dllm_fp8_linear_workspace_bytes(M, N, K), dtype=torch.uint8,
                          device=dev)
        fp8 = lambda t: dkv.dllm_fp8_linear(x, t[0], t[1], y, wsp)       # noqa: E731
        bf16 = lambda t: torch.matmul(x, t[2].t(), out=y)               # noqa: E731
        for _ in range(3):
            fp8(ws[0])
            bf16(ws[0])
        torch.cuda.synchronize()
        count = max(10, args.steps)
        us8 = burst_us(torch, fp8, count, ws)
        us16 = burst_us(torch, bf16, count, ws)
        w8 = dict(bytes=M * K * 2 + N * K + (N // 128) * (K // 128) * 4 + M * N * 2,
                  flops=2 * M * N * K)
        out[name] = {"M": M, "N": N, "K": K, "fp8_us": round(us8, 2),
                     "bf16_matmul_us": round(us16, 2), "speedup_vs_bf16": round(us16 / us8, 3),
                     "roofline": roofline_entry("fp8_linear", w8, us8, "fp8")}
        log(f"[bench] fp8 linear {name} (M={M} N={N} K={K}): {us8:.1f} us, bf16 matmul "
            f"{us16:.1f} us; {out[name]['roofline']['achieved']} {out[name]['roofline']['unit']}")
        del ws, x, y, wsp
        torch.cuda.empty_cache()
    return out


def measure_unfused_and_hbm_paths(args):
    """The fused refresh beside its unfused form (gather + GEMM, then the rotary kernel, then
    the row scatter: the four-kernel pipeline the fused call replaces, Flash-dLLM news summary,
    memory paragraph) on the c2, c3 and c4 shapes; the row scatter's own HBM rate (c3); and the
    drift check batched over 28 layers of the GQA shape in one launch (28 x 8 sequences)."""
    import torch

    import diffusion_kv_cache_amd as dkv

    dev = torch.device("cuda:0")
    bf = torch.bfloat16
    ab = {}
    scatter = None
    for name in ("c2", "c3", "c4"):
        wl = synth.WORKLOADS[name]
        inp = synth.make_inputs(wl)
        B, n, S, H, Hq, Hkv, D = (wl.batch, wl.n_refresh, wl.seq, wl.hidden, wl.q_heads,
                                  wl.kv_heads, wl.head_dim)
        M, N = B * n, wl.n_cols
        h = torch.from_numpy(inp.hidden_cur()).to(dev).to(bf)
        idx = torch.from_numpy(inp.idx).to(dev)
        bidx = torch.arange(B, device=dev)[:, None]
        pos = idx.reshape(-1).contiguous()
        L = max(3, math.ceil(3 * MALL_BYTES / (N * H * 2 + 2 * B * Hkv * S * D * 2)))
        layers = []
        for _ in range(L):
            c = dkv.Cache(B, Hkv, S, D, dkv.DLLM_BF16)
            w = torch.from_numpy(inp.w).to(dev).to(bf)
            layers.append((c, w))
        q = torch.empty((B, n, Hq, D), dtype=bf, device=dev)
        rws_bytes = dkv.dllm_refresh_workspace_bytes(layers[0][0], H, dkv.DLLM_BF16, n, Hq)
        rws = torch.empty(rws_bytes, dtype=torch.uint8, device=dev) if rws_bytes else None
        y = torch.empty((M, N), dtype=bf, device=dev)

        def fused(ly):
            dkv.dllm_refresh_qkv_rope_scatter(ly[0], h, idx, ly[1], Hq, wl.rope_base, q, rws)

        def unfused(ly):
            x = h[bidx, idx.long()].reshape(M, H)
            torch.matmul(x, ly[1].t(), out=y)
            dkv.dllm_rope_rows(y, Hq + Hkv, D, pos, wl.rope_base)
            dkv.dllm_scatter_kv_rows(ly[0], y, Hq * D, (Hq + Hkv) * D, idx)

        def scat(ly):
            dkv.dllm_scatter_kv_rows(ly[0], y, Hq * D, (Hq + Hkv) * D, idx)

        for fn in (fused, unfused):
            for r in range(3):
                fn(layers[r % L])
        torch.cuda.synchronize()
        count = max(10, args.steps)
        uf, uu = burst_us(torch, fused, count, layers), burst_us(torch, unfused, count, layers)
        ab[name] = {"rows": M, "fused_us": round(uf, 2), "unfused_us": round(uu, 2),
                    "fused_speedup": round(uu / uf, 3)}
        log(f"[bench] {name} refresh: fused {uf:.1f} us, unfused (gather + GEMM + rope + "
            f"scatter) {uu:.1f} us")
        if name == "c3":
            us = burst_us(torch, scat, count, layers)
            byts = 2 * M * Hkv * D * 2 * 2 + M * 4           # K, V rows read from y and written
            scatter = {"workload": "c3 rows (1024 rows x 2 x 32 heads x 128, bf16)",
                       "us": round(us, 2), "algorithmic_bytes": byts,
                       "achieved_GBs": round(byts / (us * 1e-6) / 1e9, 1),
                       "frac": round(byts / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)}
            log(f"[bench] row scatter (c3): {us:.1f} us, {scatter['achieved_GBs']} GB/s")
        del layers, h, y
        torch.cuda.empty_cache()

    # the drift check batched over 28 layers of the GQA shape: 28 x 8 sequences in one launch,
    # on a bf16 cache and on an FP8 cache (codes and one scale per row)
    wl = synth.WORKLOADS["c4"]
    Lyr = 28
    Bb, Hq, Hkv, S, D, k = wl.batch * Lyr, wl.q_heads, wl.kv_heads, wl.seq, wl.head_dim, wl.track_k
    drift_b = {}
    for kv, tag in ((dkv.DLLM_BF16, "bf16"), (dkv.DLLM_FP8_E4M3, "fp8")):
        c = dkv.Cache(Bb, Hkv, S, D, kv)
        g = torch.Generator(device=dev)
        g.manual_seed(5)
        if kv == dkv.DLLM_BF16:
            c.k.copy_(torch.randn(c.k.shape, generator=g, device=dev).to(bf))
            c.v.copy_(torch.randn(c.v.shape, generator=g, device=dev).to(bf))
            buf = torch.zeros((Bb, Hq, k, 2, D), dtype=bf, device=dev)
            row_bytes = D * 2
        else:
            c.k.copy_(torch.randint(0, 0x7f, c.k.shape, generator=g, device=dev, dtype=torch.uint8))
            c.v.copy_(torch.randint(0, 0x7f, c.v.shape, generator=g, device=dev, dtype=torch.uint8))
            c.k_scale.fill_(0.01)
            c.v_scale.fill_(0.02)
            buf = torch.zeros(dkv.track_buffer_bytes(c, Hq, k),
                              dtype=torch.uint8, device=dev)
            row_bytes = D + 4
        masses = [torch.rand((Bb, Hq, S), generator=g, device=dev) for _ in range(3)]
        T = torch.full((Bb, Hq, k), -1, dtype=torch.int32, device=dev)
        sig = torch.empty((Bb, Hq), dtype=torch.float32, device=dev)
        dec = torch.empty((Bb,), dtype=torch.uint8, device=dev)
        dws = dkv.drift_workspace(Bb, dev)
        dkv.dllm_drift_check(c, Hq, k, wl.gamma, T, buf, masses[0], sig, dec, dws)
        torch.cuda.synchronize()
        it = [0]

        def drift(_):
            it[0] += 1
            dkv.dllm_drift_check(c, Hq, k, wl.gamma, T, buf, masses[it[0] % 3], sig, dec, dws)

        us = burst_us(torch, drift, max(10, args.steps), [None])
        byts = Bb * Hq * (3 * k * 2 * row_bytes + S * 4 + k * 8)
        drift_b[tag] = {"workload": f"{Lyr} layers x B=8 of the GQA shape (28 query heads, "
                                   f"S=2048, k=32), {tag} cache, in one launch",
                        "us": round(us, 2), "algorithmic_bytes": byts,
                        "achieved_GBs": round(byts / (us * 1e-6) / 1e9, 1),
                        "frac": round(byts / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)}
        log(f"[bench] drift batched over {Lyr} layers ({tag}): {us:.1f} us, "
            f"{drift_b[tag]['achieved_GBs']} GB/s")
        del c, masses, T, buf
        torch.cuda.empty_cache()
    # attainable rates beside the datasheet peaks: a device copy, a read-only stream, and a loop
    # of independent MFMAs on register operands
    nb = 1 << 30
    src = torch.empty(nb, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    cp_us = burst_us(torch, lambda _: dst.copy_(src), 10, [None])
    rwg = 4096
    rout = torch.empty(rwg, dtype=torch.int32, device=dev)
    rd_us = burst_us(torch, lambda _: dkv.dllm_read_rate_probe(src, rwg, rout), 10, [None])
    del src, dst, rout
    wgs, iters = 256 * 8, 2048
    out = torch.empty(wgs * 4, dtype=torch.float32, device=dev)
    attain = {"copy_GBs": round(2 * nb / (cp_us * 1e-6) / 1e9, 1),
              "read_GBs": round(nb / (rd_us * 1e-6) / 1e9, 1)}
    for kind, name, tile, flops in ((dkv.DLLM_BF16, "bf16_16x16x32", 16, 2 * 16 * 16 * 32 * 8),
                                    (dkv.DLLM_BF16, "bf16_32x32x16", 32, 2 * 32 * 32 * 16 * 4),
                                    (dkv.DLLM_FP8_E4M3, "fp8_16x16x128", 16, 2 * 16 * 16 * 128 * 8),
                                    (dkv.DLLM_FP8_E4M3, "fp8_32x32x64", 32, 2 * 32 * 32 * 64 * 4)):
        dkv.dllm_mfma_rate_probe(kind, tile, wgs, 16, out)
        us = burst_us(torch, lambda _: dkv.dllm_mfma_rate_probe(kind, tile, wgs, iters, out), 5,
                      [None])
        tf = wgs * 4 * iters * flops / (us * 1e-6) / 1e12
        attain[f"mfma_{name}_TFLOPs"] = round(tf, 1)
        attain[f"mfma_{name}_frac_of_peak"] = round(tf / MFMA_PEAK_TFLOPS[name[:4].rstrip("_")], 4)
    log("[bench] attainable: copy {} GB/s, read {} GB/s; ".format(attain["copy_GBs"], attain["read_GBs"]) +
        ", ".join(f"{k[5:-7]} {v} TFLOP/s" for k, v in attain.items() if k.endswith("TFLOPs")))
    return ab, {"row_scatter": scatter, "drift_batched": drift_b, "attainable": attain}


def run(args):
    import torch

    wl = synth.WORKLOADS[args.config]
    torch.cuda.set_device(torch.device("cuda:0"))
    head, inp = measure(args, wl)
    others = {}
    for name in [c for c in args.also.split(",") if c and c != args.config]:
        rec, _ = measure(args, synth.WORKLOADS[name])
        others[name] = rec

    result = {
        "metric": METRIC, "value": head["value"], "unit": head["unit"],
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "ms_per_step_with_launcher": head["ms_per_step_with_launcher"],
        "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32" if wl.act == "f32" else "bf16",
        "data": "synthetic (seeded, shaped like the workload; random-init weights)",
        "config": {"workload": head["workload"], "global_batch": head["global_batch"],
                   "seq_len": head["seq_len"], "refreshed_per_seq": head["refreshed_per_seq"],
                   "hidden": head["hidden"], "q_heads": head["q_heads"],
                   "kv_heads": head["kv_heads"], "head_dim": head["head_dim"],
                   "cache_dtype": head["cache_dtype"], "tracking": head["tracking"],
                   "layer_instances": head["layer_instances"], "parallelism": "none (1 GPU)"},
        "per_call_us": head["per_call_us"],
        "per_call_back_to_back": head["per_call_back_to_back"],
        "rooflines": head["rooflines"],
        "roofline": head["roofline"],
    }
    if others:
        # the other workloads, measured the same way in the same run (not the headline)
        result["configs"] = others
    if not args.no_facache and wl.cache == "bf16":
        result["facache"] = measure_facache(args, wl)
    if args.schedule_layers > 0:
        result["layer_schedule"] = measure_schedule(args)
    if not args.no_fp8_linear:
        result["fp8_linear"] = measure_fp8_linear(args)
    if not args.no_unfused:
        result["unfused_refresh"], result["hbm_paths"] = measure_unfused_and_hbm_paths(args)
    if args.copy_calibration:
        # A plain device copy of known size, so HBM byte counters read under a profiler can be
        # scaled by what they report for a copy (reads = writes = the buffer size).
        dev = torch.device("cuda:0")
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


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


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
    # Three runs, each repeating the cached step for a third of the budget; the median rate
    # is reported.
    rates, total_runs = [], 0
    for _ in range(3):
        runs, t_total = 0, 0.0
        while runs == 0 or t_total < budget_s / 3:
            t0 = time.time()
            oracle.refresh_rows(cache, h_cur, sub.w, sub.idx)
            q = oracle.queries(ws, h_cur, sub.w, sub.idx)
            _, _, m = oracle.attend(ws, q, cache, want_mass=track)
            if track:
                oracle.drift(buf, T, cache.k, cache.v, float(np.float32(ws.gamma)))
                oracle.track(cache, m, ws.track_k)
            t_total += time.time() - t0
            runs += 1
        rates.append(runs * nb * wl.n_refresh / t_total)
        total_runs += runs
    rate = float(np.median(rates))
    log(f"[cpu] {total_runs} oracle step(s) in 3 runs: " + ", ".join(f"{r:.1f}" for r in rates)
        + f" tokens/s; median {rate:.1f}")
    return {"value": round(rate, 2), "unit": "refreshed tokens/s", "cores": cores,
            "kind": "oracle", "cpu_model": cpu_model(),
            "runs_tokens_per_s": [round(r, 2) for r in rates],
            "sample": f"cached step (refresh + attention{' + mass + drift + top-k' if track else ''})"
                      f" of {nb} of {wl.batch} sequence(s), median of 3 runs ({total_runs} steps "
                      f"in all), prefill untimed, fp64 C oracle with OpenMP"}


def main():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", default="c2", choices=sorted(synth.WORKLOADS),
                    help="the headline workload of the JSON line")
    ap.add_argument("--also", default="c3,c4,c5",
                    help="other workloads measured in the same run, reported under 'configs' "
                         "(comma-separated; '' for none)")
    ap.add_argument("--layers", type=int, default=0, help="layer instances to rotate (0: auto)")
    ap.add_argument("--no-facache", action="store_true",
                    help="skip the FACache measurement (every row's attention with cached "
                         "statistics of the invariant rows)")
    ap.add_argument("--schedule-layers", type=int, default=4,
                    help="layers of the Elastic-Cache schedule section (0: skip it)")
    ap.add_argument("--no-fp8-linear", action="store_true",
                    help="skip the per-group FP8 linear layer section")
    ap.add_argument("--no-unfused", action="store_true",
                    help="skip the unfused-refresh comparison and the HBM-path section")
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
