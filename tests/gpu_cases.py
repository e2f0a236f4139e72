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


def run_workload_gpu(wl, inp, snapshot_prefill: bool = True):
    """The bench's launch sequence on one layer: prefill(H_prev); previous step (refresh of
    R from H_prev, attention with mass, drift check from an empty tracking set); current step
    (refresh of R from H_cur, attention with mass, drift check).  Returns host copies."""
    m = dkv()
    act = ACT_TORCH[wl.act]
    B, n, S, Hq, D, k = wl.batch, wl.n_refresh, wl.seq, wl.q_heads, wl.head_dim, wl.track_k
    track = wl.cache != "fp8"
    say(f"[{wl.name}] gpu prefill")
    h_prev = to_dev(inp.hidden_prev, act)
    layer = GpuLayer(wl, inp.w, guard=0)
    layer.prefill(h_prev)
    torch.cuda.synchronize()
    res = {}
    if snapshot_prefill:
        res["region_prefill"] = layer.cache.region.clone()
    idx_t = torch.from_numpy(inp.idx).cuda()
    h_cur = h_prev.clone()
    h_cur[torch.arange(B, device="cuda")[:, None], idx_t.long()] = to_dev(inp.new_rows, act)
    scale = 1.0 / math.sqrt(D)
    q = torch.empty((B, n, Hq, D), dtype=act, device="cuda")
    out = torch.empty_like(q)
    lse = torch.empty((B, Hq, n), dtype=torch.float32, device="cuda")
    mass = torch.empty((B, Hq, S), dtype=torch.float32, device="cuda")
    sigma = torch.empty((B, Hq), dtype=torch.float32, device="cuda")
    refresh = torch.empty((B,), dtype=torch.uint8, device="cuda")
    if track:
        tdt = torch.float32 if wl.cache == "f32" else torch.bfloat16
        T = torch.full((B, Hq, k), -1, dtype=torch.int32, device="cuda")
        buf = torch.zeros((B, Hq, k, 2, D), dtype=tdt, device="cuda")
        say(f"[{wl.name}] gpu previous step")
        m.dllm_refresh_qkv_rope_scatter(layer.cache, h_prev, idx_t, layer.w, Hq, wl.rope_base, q)
        m.dllm_block_attention(layer.cache, q, Hq, scale, out, lse, mass)
        m.dllm_drift_check(layer.cache, Hq, k, wl.gamma, T, buf, mass, sigma, refresh)
        torch.cuda.synchronize()
        res["mass_prev"] = mass.cpu().numpy()
        res["T_prev"] = T.cpu().numpy()
    say(f"[{wl.name}] gpu step")
    m.dllm_refresh_qkv_rope_scatter(layer.cache, h_cur, idx_t, layer.w, Hq, wl.rope_base, q)
    m.dllm_block_attention(layer.cache, q, Hq, scale, out, lse, mass if track else None)
    if track:
        # the step takes the decision in the same launch, as the bench does
        dws = m.drift_workspace(B)
        m.dllm_drift_check(layer.cache, Hq, k, wl.gamma, T, buf, mass, sigma, refresh, dws)
    torch.cuda.synchronize()
    if track:
        assert not dws.any(), "drift workspace not left zero"
    res.update(layer=layer, q=q.float().cpu().numpy(), out=out.float().cpu().numpy(),
               lse=lse.cpu().numpy())
    if track:
        res.update(mass=mass.cpu().numpy(), sigma=sigma.cpu().numpy(),
                   refresh=refresh.cpu().numpy(), T=T.cpu().numpy())
    return res


def topk_margin(a: np.ndarray, k: int) -> np.ndarray:
    """Relative gap between the k-th and (k+1)-th largest values of each row of a [..., S]."""
    s = -np.sort(-a, axis=-1)
    if a.shape[-1] <= k:
        return np.full(a.shape[:-1], np.inf)
    return (s[..., k - 1] - s[..., k]) / np.maximum(np.abs(s[..., k - 1]), 1e-300)


def elem_rel_err(gpu: np.ndarray, ref: np.ndarray, keep_axes, floor: float = 1e-2) -> float:
    """Elementwise relative error with a floor, reported beside slice_rel_err: max over
    elements of |gpu - ref| / max(|ref|, floor * max|ref| of the element's slice)."""
    gpu = np.asarray(gpu, np.float64)
    ref = np.asarray(ref, np.float64)
    red = tuple(a for a in range(ref.ndim) if a not in keep_axes)
    den = np.maximum(np.abs(ref), floor * np.abs(ref).max(axis=red, keepdims=True))
    den = np.where(den == 0, 1.0, den)
    return float((np.abs(gpu - ref) / den).max())


# FP8 cache bar.  Near zero one e4m3 step (2^-9 of the row scale) is smaller than the rounding
# error of the fp32 projection over H terms, so a code is compared as the correct rounding of
# SOME value within delta of the oracle's exact value, delta being a first-order bound on that
# fp32 error, element by element:
#   delta = depth(H) * 2^-24 * sum_k |x_k| |w_k|,   depth(H) = H / 128 + 11,
# the number of roundings along the kernel's fixed reduction order (each product of two bf16
# values is exact in fp32): at most 6 inside one 32-deep MFMA, H/128 - 1 chained MFMAs per
# quarter of H, 4 partition adds, and 2 for the rotation; for K the rotation mixes the pair
# (i, i + D/2), so the two elements' sums are added.  The encoder itself is pinned bit for
# bit by the codec sweep (test_fp8_codec_matches_oracle), where RNE ties and saturation are
# exercised directly.
def fp8_depth(hidden: int) -> int:
    return hidden // 128 + 11


def kv_abs_sums(wl, x_rows: np.ndarray, w: np.ndarray, part: str, heads=None) -> np.ndarray:
    """sum_k |x_k| |w_k| per element of the K or V rows of x_rows [R, H], as [R, nh, D]; for K
    the two members of each rotation pair are added."""
    nh = wl.kv_heads if heads is None else len(heads)
    a = oracle.linear(np.abs(x_rows), np.abs(w), oracle.head_rows(wl, part, heads))
    a = a.reshape(len(x_rows), nh, wl.head_dim)
    if part == "k":
        a = a + np.roll(a, wl.head_dim // 2, axis=-1)
    return a


def fp8_delta(wl, x_rows: np.ndarray, w: np.ndarray, part: str, heads=None) -> np.ndarray:
    return fp8_depth(wl.hidden) * 2.0 ** -24 * kv_abs_sums(wl, x_rows, w, part, heads)


def e4m3_halfstep(mag: np.ndarray) -> np.ndarray:
    """Half the e4m3 step at magnitude `mag` (in units of the scale)."""
    e = np.floor(np.log2(np.maximum(mag, 2.0 ** -6)))
    return 2.0 ** (np.minimum(e, 8) - 3) / 2


def check_fp8_rows(codes: np.ndarray, scales: np.ndarray, exact: np.ndarray, ocodes: np.ndarray,
                   delta: np.ndarray):
    """codes [..., D] uint8 and scales [...] from the GPU; exact [..., D] float64 values before
    quantisation, ocodes the oracle's codes and delta [..., D] the fp32 error bound above.
    Asserts that every decoded GPU value lies within half an e4m3 step (at the bound's edge)
    plus delta of the exact value; returns the number of codes more than one step from the
    oracle's."""
    s = scales.astype(np.float64)[..., None]
    deq = oracle.e4m3_decode(codes) * s
    bound = (e4m3_halfstep((np.abs(exact) + delta) / np.where(s == 0, 1, s)) * s + delta)
    bad = np.abs(deq - exact) > bound * (1 + 1e-12)
    if bad.any():
        idx = np.argwhere(bad)[:4]
        sc = np.broadcast_to(s, exact.shape)
        detail = "; ".join(
            f"at {tuple(int(v) for v in i)}: exact {exact[tuple(i)]:.9g} decoded {deq[tuple(i)]:.9g} "
            f"scale {sc[tuple(i)]:.6g} code {int(codes[tuple(i)])} oracle code {int(ocodes[tuple(i)])} "
            f"delta {delta[tuple(i)]:.3g} excess/delta "
            f"{(abs(deq[tuple(i)] - exact[tuple(i)]) - (bound[tuple(i)] - delta[tuple(i)])) / delta[tuple(i)]:.3g}"
            for i in idx)
        raise AssertionError(f"{int(bad.sum())} FP8 codes off by more than the bound: {detail}")
    def ordinal(c):
        c = c.astype(np.int32)
        return np.where(c & 0x80, -(c & 0x7F), c & 0x7F)
    return int((np.abs(ordinal(codes) - ordinal(ocodes)) > 1).sum())
