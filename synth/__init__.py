"""Seeded synthetic inputs for the per-layer cached denoising step.

This module is shared by the CPU oracle (``oracle/``), the HIP library's tests and the
benchmark. It draws random numbers and lays out index lists; it holds none of the step's
arithmetic (no projection, rotation, attention, quantisation or drift test).

Recipe (one per workload, all seeded):

* generator ``numpy.random.Generator(PCG64(SeedSequence(seed)))`` with spawned child streams
  ``[W, H_prev, H_new, window, subset, mix]``;
* normals are drawn in fp32; for bf16 workloads they are rounded to bf16 (round to nearest
  even) on the host, so both sides consume exactly the same values;
* weights ``W_qkv ~ N(0, 0.02)`` with rows ordered Q heads | K heads | V heads; hidden states
  ``~ N(0, 1)``;
* ``H_cur`` equals ``H_prev`` except on the refreshed rows, which are redrawn, or for the
  scattered-refresh workload mixed as ``alpha_b * H_prev + sqrt(1 - alpha_b^2) * eps`` with
  ``alpha_b = 0.99`` on even sequences and ``0.0`` on odd ones, so that both drift decisions
  occur.

The shapes mirror the 7-8B diffusion-LLM workloads that the pages measure: LLaDA-8B geometry
(hidden 4096, 32 heads x 128), Dream-7B geometry (hidden 3584, 28 query / 4 KV heads x 128),
generation lengths 256/512 and long contexts of 2048+ tokens.  No item of any evaluation set is
used; these arrays stand in for them.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

F32, BF16, FP8 = "f32", "bf16", "fp8"


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    hidden: int
    q_heads: int
    kv_heads: int
    head_dim: int
    seq: int
    prompt: int
    act: str            # "f32" or "bf16": hidden states, weights, Q and attention output
    cache: str          # "f32", "bf16" or "fp8"
    refresh: str        # "block" or "window+subset"
    block_start: int = 0
    block_len: int = 32
    window: int = 32
    subset: int = 0
    rope_base: float = 10000.0
    gamma: float = 0.9
    track_k: int = 32
    seed: int = 1000
    description: str = ""

    @property
    def n_cols(self) -> int:
        return (self.q_heads + 2 * self.kv_heads) * self.head_dim

    @property
    def n_refresh(self) -> int:
        if self.refresh == "block":
            return self.block_len
        return self.window + self.subset


# The five workloads.  Index i is seeded with 1000 + i + 1.
WORKLOADS = {
    "c1": Workload("c1", 1, 256, 4, 4, 64, 128, 64, F32, F32, "block", block_start=64,
                   block_len=16, seed=1001,
                   description="tiny fp32 layer: B=1 H=256 4x64 S=128 (64+64) block 16 at 64"),
    "c2": Workload("c2", 1, 4096, 32, 32, 128, 1024, 512, BF16, BF16, "block", block_start=512,
                   block_len=32, seed=1002,
                   description="LLaDA-8B-shaped layer, bf16: B=1 H=4096 32x128 S=1024 (512+512) "
                               "block 32 at 512"),
    "c3": Workload("c3", 32, 4096, 32, 32, 128, 768, 256, BF16, BF16, "block", block_start=256,
                   block_len=32, seed=1003,
                   description="batched bf16: B=32 H=4096 32x128 S=768 (256+512) block 32 at 256"),
    "c4": Workload("c4", 8, 3584, 28, 4, 128, 2048, 1024, BF16, BF16, "window+subset",
                   window=32, subset=256, seed=1004,
                   description="Dream-7B-like GQA bf16: B=8 H=3584 28/4x128 S=2048 (1024+1024); "
                               "window 32 + random 25% of response rows; drift top-32, gamma 0.9"),
    "c5": Workload("c5", 8, 4096, 32, 32, 128, 4096, 2048, BF16, FP8, "block", block_start=2048,
                   block_len=32, seed=1005,
                   description="long-context FP8 cache: B=8 H=4096 32x128 S=4096 (2048+2048) "
                               "block 32 at 2048; e4m3 K/V + fp32 scale per 128-group"),
}


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to the nearest bf16 (ties to even); returns fp32 holding bf16 values.

    Input preparation only: inputs are finite normals.
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = (u + np.uint32(0x7FFF) + lsb) & np.uint32(0xFFFF0000)
    return r.view(np.float32)


@dataclasses.dataclass
class Inputs:
    wl: Workload
    w: np.ndarray            # [N, H] float32 (bf16-valued for bf16 workloads)
    hidden_prev: np.ndarray  # [B, S, H] float32
    new_rows: np.ndarray     # [B, n, H] float32: H_cur at the refreshed rows
    idx: np.ndarray          # [B, n] int32, sorted, unique

    def hidden_cur(self) -> np.ndarray:
        h = self.hidden_prev.copy()
        for b in range(self.wl.batch):
            h[b, self.idx[b]] = self.new_rows[b]
        return h


def _normal(rng: np.random.Generator, shape, std: float, act: str) -> np.ndarray:
    x = rng.standard_normal(shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    return round_to_bf16(x) if act == BF16 else x


def refresh_rows(wl: Workload, rng_window: np.random.Generator,
                 rng_subset: np.random.Generator) -> np.ndarray:
    """The refresh (= query) index list [B, n], sorted and unique per sequence."""
    B = wl.batch
    if wl.refresh == "block":
        row = np.arange(wl.block_start, wl.block_start + wl.block_len, dtype=np.int32)
        return np.tile(row, (B, 1))
    resp = wl.seq - wl.prompt
    out = np.empty((B, wl.window + wl.subset), dtype=np.int32)
    for b in range(B):
        w0 = wl.prompt + int(rng_window.integers(0, resp - wl.window + 1))
        win = np.arange(w0, w0 + wl.window)
        rest = np.setdiff1d(np.arange(wl.prompt, wl.seq), win)
        pick = rng_subset.choice(rest, size=wl.subset, replace=False)
        out[b] = np.sort(np.concatenate([win, pick])).astype(np.int32)
    return out


def make_inputs(wl: Workload) -> Inputs:
    ss = np.random.SeedSequence(wl.seed)
    r_w, r_hp, r_hn, r_win, r_sub, r_mix = [np.random.Generator(np.random.PCG64(c))
                                            for c in ss.spawn(6)]
    B, S, H = wl.batch, wl.seq, wl.hidden
    w = _normal(r_w, (wl.n_cols, H), 0.02, wl.act)
    hidden_prev = _normal(r_hp, (B, S, H), 1.0, wl.act)
    idx = refresh_rows(wl, r_win, r_sub)
    n = idx.shape[1]
    if wl.refresh == "block":
        new_rows = _normal(r_hn, (B, n, H), 1.0, wl.act)
    else:
        eps = r_mix.standard_normal((B, n, H), dtype=np.float32)
        new_rows = np.empty((B, n, H), dtype=np.float32)
        for b in range(B):
            alpha = np.float32(0.99 if b % 2 == 0 else 0.0)
            beta = np.float32(math.sqrt(1.0 - float(alpha) ** 2))
            new_rows[b] = alpha * hidden_prev[b, idx[b]] + beta * eps[b]
        if wl.act == BF16:
            new_rows = round_to_bf16(new_rows)
    return Inputs(wl, w, hidden_prev, new_rows, idx)


def custom(name: str = "custom", *, batch=1, hidden=256, q_heads=4, kv_heads=4, head_dim=64,
           seq=128, prompt=64, act=BF16, cache=BF16, refresh="block", block_start=64,
           block_len=16, window=8, subset=8, seed=7, **kw) -> Workload:
    """A workload of arbitrary (small) shape for tests."""
    return Workload(name, batch, hidden, q_heads, kv_heads, head_dim, seq, prompt, act, cache,
                    refresh, block_start=block_start, block_len=block_len, window=window,
                    subset=subset, seed=seed, **kw)


def uniform_mass(rng: np.random.Generator, shape, ties: int = 0) -> np.ndarray:
    """Non-negative fp32 'attention mass' arrays for stage-wise top-k tests.

    With ``ties`` > 0, that many values per row are copied from other positions so the
    (value desc, index asc) tie-break is exercised.
    """
    a = rng.random(shape, dtype=np.float32)
    if ties:
        rows = a.reshape(-1, shape[-1])
        for r in rows:
            src = rng.integers(0, r.size, size=ties)
            dst = rng.integers(0, r.size, size=ties)
            r[dst] = r[src]
    return a


def small_integer_grid(rng: np.random.Generator, shape) -> np.ndarray:
    """Entries in {-2..2} * 2^-4: every fp32 partial sum of their products is exact."""
    return (rng.integers(-2, 3, size=shape).astype(np.float32) * np.float32(1.0 / 16.0))


@dataclasses.dataclass
class LayerStack:
    """Seeded inputs of a step over L synthetic layers (one weight matrix and one pair of
    hidden-state arrays per layer; no layer feeds the next)."""
    wl: Workload
    w: list                  # L x [N, H] float32
    hidden_prev: list        # L x [B, S, H] float32: the states the caches were built from
    hidden_cur: list         # L x [B, S, H] float32: this step's states
    window_start: np.ndarray  # [B] int32: first row of each sequence's window
    triggers: np.ndarray     # [B] int32: first layer whose states move (L = none)


def layer_stack(wl: Workload, layers: int, triggers, window: int) -> LayerStack:
    """Every row of layer l of sequence b is mixed as alpha * H_prev + sqrt(1 - alpha^2) * eps
    with alpha = 0.99 before triggers[b] and 0.0 from that layer on, so the drift test at
    layer triggers[b] sees a clear change and the earlier ones do not.  Window starts are
    uniform over the response rows."""
    ss = np.random.SeedSequence(wl.seed)
    streams = [np.random.Generator(np.random.PCG64(c)) for c in ss.spawn(3 * layers + 1)]
    B, S, H = wl.batch, wl.seq, wl.hidden
    trig = np.asarray(triggers, np.int32)
    assert trig.shape == (B,)
    ws = streams[-1].integers(wl.prompt, S - window + 1, size=B).astype(np.int32)
    w, hp, hc = [], [], []
    for l in range(layers):
        r_w, r_h, r_e = streams[3 * l: 3 * l + 3]
        w.append(_normal(r_w, (wl.n_cols, H), 0.02, wl.act))
        prev = _normal(r_h, (B, S, H), 1.0, wl.act)
        eps = r_e.standard_normal((B, S, H), dtype=np.float32)
        cur = np.empty_like(prev)
        for b in range(B):
            alpha = np.float32(0.99 if l < trig[b] else 0.0)
            beta = np.float32(math.sqrt(1.0 - float(alpha) ** 2))
            cur[b] = alpha * prev[b] + beta * eps[b]
        if wl.act == BF16:
            cur = round_to_bf16(cur)
        hp.append(prev)
        hc.append(cur)
    return LayerStack(wl, w, hp, hc, ws, trig)
