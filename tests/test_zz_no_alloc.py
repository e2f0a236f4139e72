"""The allocation-free attention call (library-owned scratch instead of a caller workspace)
against the workspace call on the same inputs, twice in a row on one GPU: a split-key shape
with the mass pass and no lse (both live in the scratch), then a smaller shape whose
scratch use is a prefix of the first call's."""
import math

import numpy as np
import pytest
import torch

import synth
from gpu_cases import GpuLayer, say, to_dev

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # collected on CPU-only hosts, never run there
    pytest.skip("needs a GPU", allow_module_level=True)

import diffusion_kv_cache_amd as dkv  # noqa: E402

C = synth.custom
CASES = [
    # B = 1, 32 heads of 128, S = 1024: four key splits, so partials go to the scratch
    C(batch=1, hidden=256, q_heads=32, kv_heads=32, head_dim=128, seq=1024, prompt=512,
      block_start=512, block_len=32, seed=61),
    # smaller: GQA, fewer rows and keys
    C(batch=1, hidden=256, q_heads=8, kv_heads=2, head_dim=64, seq=300, prompt=150,
      block_start=151, block_len=9, seed=62),
]


def _layer(wl):
    inp = synth.make_inputs(wl)
    layer = GpuLayer(wl, inp.w)
    layer.prefill(to_dev(inp.hidden_prev, layer.act))
    q = layer.refresh(to_dev(inp.hidden_cur(), layer.act), inp.idx)
    return layer, q


def test_noalloc_attention_matches_workspace_call_twice():
    layers = [_layer(wl) for wl in CASES]
    torch.cuda.synchronize()
    for call, (wl, (layer, q)) in enumerate(zip(CASES, layers)):
        say(f"[noalloc attention] call {call}: B={wl.batch} Hq={wl.q_heads} S={wl.seq} "
            f"n={wl.n_refresh}")
        need = dkv.dllm_attention_workspace_bytes(layer.cache, wl.q_heads, wl.n_refresh)
        assert 0 < need <= dkv.DLLM_NOALLOC_SCRATCH_BYTES
        scale = 1.0 / math.sqrt(wl.head_dim)
        ref_out, ref_lse, ref_mass = layer.attention(q, want_mass=True)
        out = torch.empty_like(q)
        mass = torch.empty_like(ref_mass)
        lse = torch.empty_like(ref_lse) if call == 1 else None
        dkv.dllm_block_attention_noalloc(layer.cache, q, wl.q_heads, scale, out, lse, mass)
        torch.cuda.synchronize()
        # same kernels and launch plan as the workspace call: identical bits
        assert torch.equal(out, ref_out)
        assert torch.equal(mass, ref_mass)
        if lse is not None:
            assert torch.equal(lse, ref_lse)
        # and without the mass (split merge by its own kernel, log-sum-exp in the scratch)
        out2 = torch.empty_like(q)
        dkv.dllm_block_attention_noalloc(layer.cache, q, wl.q_heads, scale, out2)
        torch.cuda.synchronize()
        assert torch.equal(out2, ref_out)


def test_noalloc_rejects_shapes_beyond_its_scratch():
    # 65536 keys of 8 query heads per KV head, 1024 rows: far more split state than 32 MiB
    cache = dkv.Cache(1, 1, 65536, 128, dkv.DLLM_BF16)
    need = dkv.dllm_attention_workspace_bytes(cache, 8, 1024)
    assert need > dkv.DLLM_NOALLOC_SCRATCH_BYTES
    q = torch.zeros((1, 1024, 8, 128), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(dkv.DllmError) as e:
        dkv.dllm_block_attention_noalloc(cache, q, 8, 0.1, torch.empty_like(q))
    assert e.value.status == dkv.DLLM_ESIZE
