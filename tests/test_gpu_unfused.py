"""The unfused refresh (gather + GEMM, then the rotary kernel, then the row scatter) through the
C ABI against the oracle: K/V rows and queries <= 1e-2 per (b, head) slice of the fp64 result
(bf16 GEMM output rounding, then the rotation in fp32), every other cache row and the guard
bands untouched bit for bit, and debug mode rejecting a bad index list before the scatter."""
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
    "d128_gqa": synth.custom(batch=2, hidden=512, q_heads=4, kv_heads=2, head_dim=128, seq=100,
                             prompt=40, block_start=41, block_len=20, seed=71),
    "d64_scattered": synth.custom(batch=3, hidden=256, q_heads=6, kv_heads=3, head_dim=64,
                                  seq=90, prompt=40, refresh="window+subset", window=6,
                                  subset=9, seed=72),
}


@pytest.mark.parametrize("name", list(CASES))
def test_unfused_refresh_matches_oracle(name):
    wl = CASES[name]
    say(f"[unfused] {name}")
    B, n, Hq, Hkv, D = wl.batch, wl.n_refresh, wl.q_heads, wl.kv_heads, wl.head_dim
    inp = synth.make_inputs(wl)
    h_cur = inp.hidden_cur()
    layer = GpuLayer(wl, inp.w)
    snap = layer.cache.storage.clone()
    hid = to_dev(h_cur, torch.bfloat16)
    idx = torch.from_numpy(inp.idx).cuda()
    x = hid[torch.arange(B, device="cuda")[:, None], idx.long()].reshape(B * n, wl.hidden)
    y = torch.matmul(x, layer.w.t().contiguous())             # [B n, N] bf16
    pos = idx.reshape(-1).contiguous()
    dkv.dllm_rope_rows(y, Hq + Hkv, D, pos, wl.rope_base)
    dkv.dllm_scatter_kv_rows(layer.cache, y, Hq * D, (Hq + Hkv) * D, idx)
    torch.cuda.synchronize()
    cache_o = oracle.refresh_rows(oracle.Cache(wl), h_cur, inp.w, inp.idx)
    kg, vg = layer.kv_host()
    rows = np.zeros((B, wl.seq), bool)
    for b in range(B):
        rows[b, inp.idx[b]] = True
        r = inp.idx[b]
        assert slice_rel_err(kg[b][:, r], cache_o.k[b][:, r], (0,)) <= 1e-2
        assert slice_rel_err(vg[b][:, r], cache_o.v[b][:, r], (0,)) <= 1e-2
    q_ref = oracle.queries(wl, h_cur, inp.w, inp.idx)
    qg = y[:, :Hq * D].float().cpu().numpy().reshape(B, n, Hq, D)
    for b in range(B):
        assert slice_rel_err(qg[b], q_ref[b], (1,)) <= 1e-2
    # every byte outside the refreshed rows is as it was (poisoned rows and guard bands)
    st = layer.cache.storage
    kview = layer.cache.k.view(torch.uint8).reshape(B, Hkv, wl.seq, -1)
    vview = layer.cache.v.view(torch.uint8).reshape(B, Hkv, wl.seq, -1)
    changed = ~torch.eq(st, snap)
    written = torch.zeros_like(changed)
    k_off = layer.cache.k.data_ptr() - st.data_ptr()
    v_off = layer.cache.v.data_ptr() - st.data_ptr()
    row_b = D * 2
    for b in range(B):
        for g in range(Hkv):
            for p in inp.idx[b]:
                for off in (k_off, v_off):
                    o = off + ((b * Hkv + g) * wl.seq + int(p)) * row_b
                    written[o:o + row_b] = True
    assert not (changed & ~written).any()
    del kview, vview


def test_unfused_scatter_debug_mode_rejects_a_bad_list():
    wl = CASES["d128_gqa"]
    inp = synth.make_inputs(wl)
    layer = GpuLayer(wl, inp.w)
    n = wl.n_refresh
    y = torch.zeros((wl.batch * n, wl.n_cols), dtype=torch.bfloat16, device="cuda")
    bad = torch.from_numpy(inp.idx.copy()).cuda()
    bad[1, 3] = wl.seq + 5
    prev = dkv.dllm_set_options(dkv.DLLM_OPT_DEBUG)
    try:
        with pytest.raises(dkv.DllmError) as e:
            dkv.dllm_scatter_kv_rows(layer.cache, y, wl.q_heads * wl.head_dim,
                                     (wl.q_heads + wl.kv_heads) * wl.head_dim, bad)
        assert "outside" in str(e.value)
    finally:
        dkv.dllm_set_options(prev)


@pytest.mark.parametrize("words,wgs", [(0, 4), (4 * 1000003, 37), (4 * 1024 * 64, 8)])
def test_read_rate_probe_reads_every_word_once(words, wgs):
    """The XOR of the per-workgroup folds equals the XOR of every 32-bit word of the buffer
    (a ragged tail, more workgroups than chunks, and the empty buffer)."""
    g = torch.Generator().manual_seed(words + wgs)
    host = torch.randint(-2**31, 2**31 - 1, (words,), dtype=torch.int32, generator=g)
    buf = host.cuda()
    out = torch.full((wgs,), 12345, dtype=torch.int32, device="cuda")
    dkv.dllm_read_rate_probe(buf, wgs, out)
    torch.cuda.synchronize()
    folds = out.cpu().numpy().view(np.uint32)
    want = np.bitwise_xor.reduce(host.numpy().view(np.uint32)) if words else np.uint32(0)
    assert np.bitwise_xor.reduce(folds) == want
    if words == 0:
        assert not folds.any()


def test_read_rate_probe_rejects_bad_arguments():
    out = torch.zeros(4, dtype=torch.int32, device="cuda")
    buf = torch.zeros(64, dtype=torch.uint8, device="cuda")
    with pytest.raises(dkv.DllmError):
        dkv.dllm_read_rate_probe(buf[:60], 4, out)          # not a multiple of 16 bytes
    with pytest.raises(dkv.DllmError):
        dkv.dllm_read_rate_probe(buf[4:52], 4, out)         # not 16-byte aligned
    with pytest.raises(dkv.DllmError):
        dkv.dllm_read_rate_probe(buf, 0, out)               # out shape does not match


def test_mfma_rate_probe_runs_and_writes_every_wave():
    for kind in (dkv.DLLM_BF16, dkv.DLLM_FP8_E4M3):
        for tile in (16, 32):
            out = torch.full((8 * 4,), 12345.0, dtype=torch.float32, device="cuda")
            dkv.dllm_mfma_rate_probe(kind, tile, 8, 4, out)
            torch.cuda.synchronize()
            assert not torch.eq(out, 12345.0).any()
    with pytest.raises(dkv.DllmError):
        dkv.dllm_mfma_rate_probe(dkv.DLLM_F32, 16, 8, 4, out)
    with pytest.raises(dkv.DllmError):
        dkv.dllm_mfma_rate_probe(dkv.DLLM_BF16, 8, 8, 4, out)
