"""Per-group FP8 linear layer through the C ABI against the oracle: weight and activation
codes and scales bit for bit (the same fp32 decisions on both sides), and the layer's output
elementwise within |dy| <= 2^-8 |y| + 2^-14 sum_k |x_k w_k| of the fp64 result on the same
codes, on shapes that take the 64 x 64 and the 128 x 128 tiles, with and without the split
over k, and ragged row counts.  The bar: rounding the output to bf16 moves it by at most half
a unit in the last of its 8 significant bits, 2^-8 of its magnitude; the e4m3 products are
exact in fp32 and the fp32 sums over a 128-group and over the K / 128 groups add at most
about (128 + K / 128) 2^-24 of sum |x_k w_k|, far inside 2^-14 of it.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_cases import say, to_dev

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # collected on CPU-only hosts, never run there
    pytest.skip("needs a GPU", allow_module_level=True)

import diffusion_kv_cache_amd as dkv  # noqa: E402

BF = torch.bfloat16

# M, N, K: small tiles with splits / without, 128 tiles with splits / without, ragged M
CASES = {
    "m1_split": (1, 256, 1024),
    "m32_split": (32, 1024, 512),
    "m17_nosplit": (17, 32768, 256),
    "m100_split": (100, 1024, 1024),
    "m300_ragged": (300, 512, 768),
    "m1024_nosplit": (1024, 8192, 512),
}


def _inputs(M, N, K, seed):
    r = np.random.default_rng(seed)
    x = synth.round_to_bf16((r.standard_normal((M, K)) *
                             np.exp(r.uniform(-3, 3, size=(M, 1)))).astype(np.float32))
    w = synth.round_to_bf16((r.standard_normal((N, K)) * 0.02 *
                             np.exp(r.uniform(-2, 2, size=(N // 128, 1, K // 128, 1)))
                             .repeat(128, 1).repeat(128, 3).reshape(N, K)).astype(np.float32))
    x[0, :128] = 0.0                               # a zero group: scale 1, codes 0
    return x, w


@pytest.mark.parametrize("name", list(CASES))
def test_fp8_linear_matches_oracle(name):
    M, N, K = CASES[name]
    say(f"[fp8 linear] {name}: M={M} N={N} K={K}")
    x, w = _inputs(M, N, K, len(name))
    wd, xd = to_dev(w, BF), to_dev(x, BF)
    wc = torch.empty((N, K), dtype=torch.uint8, device="cuda")
    ws = torch.empty((N // 128, K // 128), dtype=torch.float32, device="cuda")
    dkv.dllm_fp8_quantize_weight(wd, wc, ws)
    pitch = M + 5
    xc = torch.empty((M, K), dtype=torch.uint8, device="cuda")
    xs = torch.full((K // 128, pitch), float("nan"), dtype=torch.float32, device="cuda")
    dkv.dllm_fp8_quantize_activations(xd, xc, xs)
    y = torch.full((M, N), float("nan"), dtype=BF, device="cuda")
    dkv.dllm_fp8_linear(xd, wc, ws, y)
    torch.cuda.synchronize()
    rwc, rws = oracle.fp8_quantize_blocks(w)
    rxc, rxs = oracle.fp8_quantize_groups(x)
    np.testing.assert_array_equal(ws.cpu().numpy(), rws)
    np.testing.assert_array_equal(wc.cpu().numpy(), rwc)
    np.testing.assert_array_equal(xs.cpu().numpy()[:, :M], rxs.T)
    assert not xs.cpu().numpy()[:, M:].any()
    np.testing.assert_array_equal(xc.cpu().numpy(), rxc)
    rows = np.arange(M) if M <= 128 else np.unique(
        np.concatenate([np.arange(8), np.random.default_rng(1).choice(M, 56), [M - 1]]))
    ref = oracle.fp8_linear(rxc[rows], rxs[rows], rwc, rws)
    mag = oracle.fp8_linear(oracle.e4m3_encode(np.abs(oracle.e4m3_decode(rxc[rows]))), rxs[rows],
                            oracle.e4m3_encode(np.abs(oracle.e4m3_decode(rwc))), rws)
    got = y.float().cpu().numpy()[rows]
    bound = 2.0 ** -8 * np.abs(ref) + 2.0 ** -14 * mag
    err = np.abs(got - ref)
    worst = float((err / np.maximum(bound, 1e-30)).max())
    i = np.unravel_index(np.argmax(err / np.maximum(bound, 1e-30)), err.shape)
    say(f"  max |dy| / bound = {worst:.3f} at ref {ref[i]:.6g} got {got[i]:.6g} mag {mag[i]:.6g}; "
        f"max |dy| / mag {float((err / mag).max()):.2e}, max rel {float((err / np.abs(ref).max()).max()):.2e}")
    assert np.isfinite(got).all()
    assert (err <= bound).all()
