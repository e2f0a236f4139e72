"""Variable-length batches through the C ABI against the oracle: packed refreshed rows with
per-sequence row counts (one sequence without rows), then attention of the packed queries over
each sequence's own key length.

Bars: K/V rows <= 1e-2 max relative error per (b, head) slice against the oracle and bit for
bit equal to what a full refresh of every row stores; rows outside the refresh lists
untouched (bitwise); packed queries <= 1e-2; attention output <= 2e-2 per (sequence, head)
slice, log-sum-exp <= 1e-2 absolute, column mass <= 2e-2 and exactly 0 at and past each
sequence's length; the same without the mass (split merge by its own kernel).
"""
import math

import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_cases import ACT_TORCH, GpuLayer, say, slice_rel_err, to_dev

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # collected on CPU-only hosts, never run there
    pytest.skip("needs a GPU", allow_module_level=True)

import diffusion_kv_cache_amd as dkv  # noqa: E402

C = synth.custom
CASES = {
    # uneven counts, one empty sequence, lengths down to a single key (split-K refresh: 54 rows)
    "g1_d128_uneven": (C(batch=4, hidden=256, q_heads=2, kv_heads=2, head_dim=128, seq=100,
                         prompt=0, block_start=0, block_len=32, seed=81),
                       [5, 0, 17, 32], [100, 40, 77, 1]),
    # GQA 4, D = 64, FP8 cache; 96 rows: the tiled GEMM refresh
    "gqa4_d64_fp8": (C(batch=3, hidden=256, q_heads=8, kv_heads=2, head_dim=64, seq=90,
                       prompt=0, block_start=0, block_len=40, seed=82, cache="fp8"),
                     [40, 17, 39], [90, 33, 60]),
    # one head, long rows: the attention splits keys (mass pass merges the splits)
    "splits_long": (C(batch=2, hidden=256, q_heads=1, kv_heads=1, head_dim=128, seq=3000,
                      prompt=0, block_start=0, block_len=40, seed=83),
                    [40, 3], [3000, 1500]),
    # GQA 7 with many rows: 128-row query tiles of different counts per sequence
    "gqa7_many_rows": (C(batch=2, hidden=256, q_heads=7, kv_heads=1, head_dim=128, seq=600,
                         prompt=0, block_start=0, block_len=100, seed=84),
                       [100, 23], [600, 300]),
}


def _lists(rng, S, counts):
    return [np.sort(rng.choice(S, size=c, replace=False)).astype(np.int32) for c in counts]


@pytest.mark.parametrize("name", list(CASES))
def test_varlen_refresh_and_attention(name):
    wl, counts, lens = CASES[name]
    say(f"[varlen] {name} counts {counts} lens {lens}")
    B, S, Hq, D = wl.batch, wl.seq, wl.q_heads, wl.head_dim
    inp = synth.make_inputs(wl)
    rng = np.random.default_rng(len(name))
    lists = _lists(rng, S, counts)
    cu = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    T = int(cu[-1])
    idx = np.concatenate(lists).astype(np.int32)
    h_prev = inp.hidden_prev
    h_cur = h_prev.copy()
    for b in range(B):
        h_cur[b, lists[b]] = synth.round_to_bf16(
            rng.standard_normal((counts[b], wl.hidden)).astype(np.float32))
    act = ACT_TORCH[wl.act]

    layer = GpuLayer(wl, inp.w)
    layer.prefill(to_dev(h_prev, act))
    q = torch.empty((T, Hq, D), dtype=act, device="cuda")
    cu_d = torch.from_numpy(cu).cuda()
    dkv.dllm_refresh_qkv_rope_scatter_varlen(layer.cache, to_dev(h_cur, act),
                                             torch.from_numpy(idx).cuda(), cu_d, max(counts),
                                             layer.w, Hq, wl.rope_base, q)
    full = GpuLayer(wl, inp.w)
    full.prefill(to_dev(h_cur, act))
    torch.cuda.synchronize()
    # every row now equals a full refresh of h_cur: the refreshed rows bit for bit (the
    # projection's reduction order does not depend on the row set), the others untouched
    views = ["k", "v"] + (["k_scale", "v_scale"] if wl.cache == "fp8" else [])
    for name in views:
        assert torch.equal(getattr(layer.cache, name), getattr(full.cache, name)), name

    cache_o = oracle.prefill(wl, h_prev, inp.w)
    for b in range(B):
        if counts[b]:
            oracle.refresh_rows(cache_o, h_cur, inp.w, [lists[b]] * B, batches=[b])
    kg, vg = layer.kv_host()
    for b in range(B):
        rows = lists[b]
        if not len(rows):
            continue
        if wl.cache == "fp8":
            # e4m3 keeps 3 mantissa bits: within half a step (2^-4 relative) of the exact value
            for got, ref in ((kg, cache_o.k_exact), (vg, cache_o.v_exact)):
                assert slice_rel_err(got[b][:, rows], ref[b][:, rows], (0,)) <= 2 ** -4 + 1e-2
        else:
            for got, ref in ((kg, cache_o.k), (vg, cache_o.v)):
                assert slice_rel_err(got[b][:, rows], ref[b][:, rows], (0,)) <= 1e-2
    q_ref = np.zeros((T, Hq, D))
    for b in range(B):
        if counts[b]:
            q_ref[cu[b]:cu[b + 1]] = oracle.queries(wl, h_cur, inp.w, np.stack([lists[b]] * B),
                                                    batches=[b])[b]
    qg = q.float().cpu().numpy()
    for b in range(B):
        if counts[b]:
            assert slice_rel_err(qg[cu[b]:cu[b + 1]], q_ref[cu[b]:cu[b + 1]], (1,)) <= 1e-2

    lens_d = torch.tensor(lens, dtype=torch.int32, device="cuda")
    out = torch.empty_like(q)
    lse = torch.empty((T * Hq,), dtype=torch.float32, device="cuda")
    mass = torch.full((B, Hq, S), float("nan"), dtype=torch.float32, device="cuda")
    scale = 1.0 / math.sqrt(D)
    dkv.dllm_block_attention_varlen(layer.cache, q, Hq, cu_d, lens_d, max(counts), scale, out,
                                    lse, mass)
    torch.cuda.synchronize()
    kq, vq = layer.kv_host()                                   # the values the cache stores
    o_ref, l_ref, m_ref = oracle.attention_varlen(qg, kq, vq, scale, cu, lens, True)
    og = out.float().cpu().numpy()
    mg = mass.cpu().numpy()
    for b in range(B):
        if counts[b]:
            e = slice_rel_err(og[cu[b]:cu[b + 1]], o_ref[cu[b]:cu[b + 1]], (1,))
            say(f"  sequence {b}: {counts[b]} rows, {lens[b]} keys, out err {e:.2e}")
            assert e <= 2e-2
        assert slice_rel_err(mg[b][:, :lens[b]], m_ref[b][:, :lens[b]], (0,)) <= 2e-2
        assert not mg[b][:, lens[b]:].any()
    np.testing.assert_allclose(lse.cpu().numpy(), l_ref, rtol=0, atol=1e-2)
    # without the mass
    out2 = torch.empty_like(q)
    dkv.dllm_block_attention_varlen(layer.cache, q, Hq, cu_d, lens_d, max(counts), scale, out2)
    torch.cuda.synchronize()
    o2 = out2.float().cpu().numpy()
    for b in range(B):
        if counts[b]:
            assert slice_rel_err(o2[cu[b]:cu[b + 1]], o_ref[cu[b]:cu[b + 1]], (1,)) <= 2e-2


def test_varlen_debug_mode_rejects_broken_offsets():
    wl, counts, _ = CASES["g1_d128_uneven"]
    inp = synth.make_inputs(wl)
    layer = GpuLayer(wl, inp.w)
    h = to_dev(inp.hidden_prev, torch.bfloat16)
    idx = torch.arange(10, dtype=torch.int32, device="cuda")
    q = torch.empty((10, wl.q_heads, wl.head_dim), dtype=torch.bfloat16, device="cuda")
    bad = torch.tensor([0, 4, 3, 8, 10], dtype=torch.int32, device="cuda")   # not monotone
    prev = dkv.dllm_set_options(dkv.DLLM_OPT_DEBUG)
    try:
        with pytest.raises(dkv.DllmError) as e:
            dkv.dllm_refresh_qkv_rope_scatter_varlen(layer.cache, h, idx, bad, 6, layer.w,
                                                     wl.q_heads, wl.rope_base, q)
        assert "offsets" in str(e.value)
        good = torch.tensor([0, 4, 4, 8, 10], dtype=torch.int32, device="cuda")
        dkv.dllm_refresh_qkv_rope_scatter_varlen(layer.cache, h, idx, good, 4, layer.w,
                                                 wl.q_heads, wl.rope_base, q)
        torch.cuda.synchronize()
    finally:
        dkv.dllm_set_options(prev)


def test_varlen_debug_mode_rejects_broken_key_counts():
    wl, counts, lens = CASES["g1_d128_uneven"]
    inp = synth.make_inputs(wl)
    layer = GpuLayer(wl, inp.w)
    layer.prefill(to_dev(inp.hidden_prev, torch.bfloat16))
    T = sum(counts)
    q = torch.zeros((T, wl.q_heads, wl.head_dim), dtype=torch.bfloat16, device="cuda")
    out = torch.empty_like(q)
    cu = torch.tensor(np.concatenate([[0], np.cumsum(counts)]), dtype=torch.int32, device="cuda")
    prev = dkv.dllm_set_options(dkv.DLLM_OPT_DEBUG)
    try:
        for bad in ([100, 40, 0, 1], [100, 40, 77, wl.seq + 1]):
            with pytest.raises(dkv.DllmError) as e:
                dkv.dllm_block_attention_varlen(layer.cache, q, wl.q_heads, cu,
                                                torch.tensor(bad, dtype=torch.int32,
                                                             device="cuda"),
                                                max(counts), 0.1, out)
            assert "sequence" in str(e.value)
        with pytest.raises(dkv.DllmError):                     # max_rows below a count
            dkv.dllm_block_attention_varlen(layer.cache, q, wl.q_heads, cu,
                                            torch.tensor(lens, dtype=torch.int32, device="cuda"),
                                            max(counts) - 1, 0.1, out)
        dkv.dllm_block_attention_varlen(layer.cache, q, wl.q_heads, cu,
                                        torch.tensor(lens, dtype=torch.int32, device="cuda"),
                                        max(counts), 0.1, out)
        torch.cuda.synchronize()
    finally:
        dkv.dllm_set_options(prev)
