"""Helpers for the GPU parity tests: run the HIP path through the C ABI on seeded inputs and
compute what the oracle says for the same inputs.  Nothing here computes the method's
arithmetic; the oracle (``oracle``) and the library (``diffusion_kv_cache_amd``) do."""
from __future__ import annotations

import math
import sys

import numpy as np
import torch

import oracle
import synth

ACT_TORCH = {"f32": torch.float32, "bf16": torch.bfloat16}


def say(msg: str):
    print(msg, flush=True)
    sys.stdout.flush()


def dkv():
    import diffusion_kv_cache_amd as m
    return m


def kv_code(name: str) -> int:
    m = dkv()
    return {"f32": m.DLLM_F32, "bf16": m.DLLM_BF16, "fp8": m.DLLM_FP8_E4M3}[name]


def to_dev(x: np.ndarray, dtype) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x)).to("cuda").to(dtype).contiguous()


def poison_(t: torch.Tensor, seed: int):
    """Fill a uint8 device tensor with seeded random bytes."""
    g = np.random.default_rng(seed)
    t.copy_(torch.from_numpy(g.integers(0, 256, t.numel(), dtype=np.uint8)).to(t.device))


class GpuLayer:
    """One layer on the GPU: the cache (with guard bands) and the layer's weights."""

    def __init__(self, wl, w: np.ndarray, guard: int = 4096, seed: int = 99):
        m = dkv()
        self.wl = wl
        self.act = ACT_TORCH[wl.act]
        self.cache = m.Cache(wl.batch, wl.kv_heads, wl.seq, wl.head_dim, kv_code(wl.cache),
                             guard=guard)
        poison_(self.cache.storage, seed)
        self.w = to_dev(w, self.act)

    def guards_intact(self, snapshot: torch.Tensor) -> bool:
        c = self.cache
        a, b = c.region_offset, c.region_offset + c.region.numel()
        return bool(torch.equal(c.storage[:a], snapshot[:a]) and torch.equal(c.storage[b:], snapshot[b:]))

    def refresh(self, hidden: torch.Tensor, idx: np.ndarray) -> torch.Tensor:
        m = dkv()
        wl = self.wl
        idx_t = torch.from_numpy(np.ascontiguousarray(idx, dtype=np.int32)).cuda()
        q = torch.empty((wl.batch, idx.shape[1], wl.q_heads, wl.head_dim), dtype=self.act,
                        device="cuda")
        m.dllm_refresh_qkv_rope_scatter(self.cache, hidden, idx_t, self.w, wl.q_heads,
                                        wl.rope_base, q)
        return q

    def prefill(self, hidden: torch.Tensor) -> torch.Tensor:
        idx = np.tile(np.arange(self.wl.seq, dtype=np.int32), (self.wl.batch, 1))
        return self.refresh(hidden, idx)

    def attention(self, q: torch.Tensor, want_mass: bool = False):
        m = dkv()
        wl = self.wl
        out = torch.empty_like(q)
        lse = torch.empty((wl.batch, wl.q_heads, q.shape[1]), dtype=torch.float32, device="cuda")
        mass = torch.empty((wl.batch, wl.q_heads, wl.seq), dtype=torch.float32,
                           device="cuda") if want_mass else None
        m.dllm_block_attention(self.cache, q, wl.q_heads, 1.0 / math.sqrt(wl.head_dim), out,
                               lse, mass)
        return out, lse, mass

    def kv_host(self):
        """(k, v) as float64 numpy [B,Hkv,S,D] of the stored values (fp8: decoded codes x
        scale via the oracle's codec, i.e. the values the cache represents)."""
        c = self.cache
        if self.wl.cache == "fp8":
            ks = c.k_scale.cpu().numpy().astype(np.float64)[..., None]
            vs = c.v_scale.cpu().numpy().astype(np.float64)[..., None]
            return (oracle.e4m3_decode(c.k.cpu().numpy()) * ks,
                    oracle.e4m3_decode(c.v.cpu().numpy()) * vs)
        return (c.k.float().cpu().numpy().astype(np.float64),
                c.v.float().cpu().numpy().astype(np.float64))


def slice_rel_err(gpu: np.ndarray, ref: np.ndarray, keep_axes) -> float:
    """max over slices (the axes in keep_axes) of max|gpu - ref| / max|ref|."""
    gpu = np.asarray(gpu, np.float64)
    ref = np.asarray(ref, np.float64)
    red = tuple(a for a in range(ref.ndim) if a not in keep_axes)
    num = np.abs(gpu - ref).max(axis=red)
    den = np.abs(ref).max(axis=red)
    den = np.where(den == 0, 1.0, den)
    return float((num / den).max())


def e4m3_step_distance(a: np.ndarray, b: np.ndarray) -> int:
    """Largest distance between two e4m3 code arrays in sign-magnitude order."""
    def ordinal(c):
        c = c.astype(np.int32)
        mag = c & 0x7F
        return np.where(c & 0x80, -mag, mag)
    return int(np.abs(ordinal(a) - ordinal(b)).max()) if a.size else 0
