"""FACache attention (cached softmax statistics of the invariant rows) through the C ABI
against the oracle, on a build step and a reuse step of the same block.

Bars: attention output of every row <= 2e-2 max relative error per (b, head) slice and
log-sum-exp <= 1e-2 absolute against full attention over all keys; the kept state of every
invariant row, as its normalised output O~ / l (<= 2e-2 per slice) and log-sum-exp (<= 1e-2
absolute), against the oracle's state over the invariant keys; the reuse step's output also
against the library's plain attention of every row; the block rows of the query cache equal
this step's block queries bit for bit.  The state is filled with NaN before the build step,
so a read of a state row the build step did not write shows up in the outputs.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_cases import GpuLayer, say, slice_rel_err, to_dev

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # collected on CPU-only hosts, never run there
    pytest.skip("needs a GPU", allow_module_level=True)

import diffusion_kv_cache_amd as dkv  # noqa: E402

CASES = {
    # blocks at different, unaligned rows per sequence
    "g1_d128_two_starts": dict(B=2, Hq=2, Hkv=2, D=128, S=300, n=32, starts=[100, 7]),
    # GQA (4 query heads per KV head), a block that ends the sequence, ragged last tiles
    "gqa4_d64_block_at_end": dict(B=1, Hq=8, Hkv=2, D=64, S=257, n=20, starts=[237]),
    # one-row blocks at the first and the last row
    "n1_first_and_last_row": dict(B=2, Hq=4, Hkv=4, D=128, S=96, n=1, starts=[0, 95]),
    # the whole sequence is the block: no invariant rows, nothing kept
    "whole_sequence_block": dict(B=1, Hq=2, Hkv=1, D=64, S=40, n=40, starts=[0]),
    # a longer sequence, GQA 7, D = 128: several key tiles per key group in phase U
    "gqa7_d128_long": dict(B=1, Hq=7, Hkv=1, D=128, S=1100, n=32, starts=[530]),
}


def _replace_block(h, idx, rng):
    h = h.copy()
    for b in range(h.shape[0]):
        h[b, idx[b]] = synth.round_to_bf16(rng.standard_normal((idx.shape[1], h.shape[2]))
                                           .astype(np.float32))
    return h


@pytest.mark.parametrize("name", list(CASES))
def test_facache_build_and_reuse_steps(name):
    p = CASES[name]
    B, Hq, Hkv, D, S, n = p["B"], p["Hq"], p["Hkv"], p["D"], p["S"], p["n"]
    say(f"[facache] {name}")
    wl = synth.custom(batch=B, hidden=256, q_heads=Hq, kv_heads=Hkv, head_dim=D, seq=S,
                      prompt=0, block_start=0, block_len=n, seed=70 + len(name))
    inp = synth.make_inputs(wl)
    starts = np.array(p["starts"], np.int32)
    idx = np.stack([np.arange(s, s + n, dtype=np.int32) for s in starts])
    rng = np.random.default_rng(7 + len(name))
    h0 = inp.hidden_prev
    h1 = _replace_block(h0, idx, rng)
    h2 = _replace_block(h1, idx, rng)
    scale = 1.0 / math.sqrt(D)
    all_rows = np.tile(np.arange(S, dtype=np.int32), (B, 1))

    layer = GpuLayer(wl, inp.w)
    q_cache = layer.prefill(to_dev(h0, torch.bfloat16))
    st_bytes = dkv.dllm_facache_state_bytes(layer.cache, Hq)
    assert st_bytes == B * Hq * S * (D + 2) * 4
    state = torch.full((st_bytes // 4,), float("nan"), dtype=torch.float32, device="cuda")
    bs = torch.from_numpy(starts).cuda()
    out = torch.empty((B, S, Hq, D), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((B, Hq, S), dtype=torch.float32, device="cuda")

    cache_o = oracle.prefill(wl, h0, inp.w)
    for step, h in ((1, h1), (2, h2)):
        q_blk = layer.refresh(to_dev(h, torch.bfloat16), idx)
        dkv.dllm_facache_attention(layer.cache, q_cache, q_blk, bs, Hq, scale, state,
                                   step == 1, out, lse)
        torch.cuda.synchronize()
        for b in range(B):
            assert torch.equal(q_cache[b, starts[b]:starts[b] + n], q_blk[b])
        cache_o = oracle.refresh_rows(cache_o, h, inp.w, idx)
        q_all = oracle.queries(wl, h, inp.w, all_rows)
        ref_out, ref_lse, (m, ll, o), inv = oracle.facache_reference(wl, q_all, cache_o, starts)
        og = out.float().cpu().numpy()
        e_out = slice_rel_err(og, ref_out, (0, 2))
        e_lse = float(np.abs(lse.cpu().numpy() - ref_lse).max())
        say(f"  step {step} ({'build' if step == 1 else 'reuse'}): out {e_out:.2e}, lse {e_lse:.2e}")
        assert e_out <= 2e-2 and e_lse <= 1e-2
        if step == 1 and inv.any():
            st = state.cpu().numpy()
            so = st[:B * Hq * S * D].reshape(B, Hq, S, D)
            sml = st[B * Hq * S * D:].reshape(B, Hq, S, 2)
            for b in range(B):
                rows = np.flatnonzero(inv[b])
                gpu_norm = so[b][:, rows] / sml[b][:, rows, 1:2]          # Hq, R, D
                ref_norm = (o[b][rows] / ll[b].T[rows][..., None]).transpose(1, 0, 2)
                assert slice_rel_err(gpu_norm, ref_norm, (0,)) <= 2e-2
                gpu_lse = (sml[b][:, rows, 0] + np.log2(sml[b][:, rows, 1])) * math.log(2)
                ref_l = m[b][:, rows] + np.log(ll[b][:, rows])
                assert float(np.abs(gpu_lse - ref_l).max()) <= 1e-2
                blk = np.flatnonzero(~inv[b])                              # never written
                assert np.isnan(so[b][:, blk]).all() and np.isnan(sml[b][:, blk]).all()
    # the reuse step against the library's plain attention of every row
    plain = torch.empty_like(out)
    dkv.dllm_block_attention(layer.cache, q_cache, Hq, scale, plain)
    torch.cuda.synchronize()
    assert slice_rel_err(out.float().cpu().numpy(), plain.float().cpu().numpy(), (0, 2)) <= 2e-2


def test_facache_rejects_bad_arguments():
    cache = dkv.Cache(1, 2, 64, 128, dkv.DLLM_FP8_E4M3)
    q = torch.zeros((1, 64, 2, 128), dtype=torch.bfloat16, device="cuda")
    qb = torch.zeros((1, 8, 2, 128), dtype=torch.bfloat16, device="cuda")
    bs = torch.zeros((1,), dtype=torch.int32, device="cuda")
    st = torch.zeros((dkv.dllm_facache_state_bytes(cache, 2) // 4,), dtype=torch.float32,
                     device="cuda")
    with pytest.raises(dkv.DllmError) as e:
        dkv.dllm_facache_attention(cache, q, qb, bs, 2, 0.1, st, True, torch.empty_like(q))
    assert e.value.status == dkv.DLLM_EUNSUPPORTED
