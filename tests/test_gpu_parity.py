"""GPU parity: the HIP path, called through the C ABI, against the CPU oracle on the same
seeded inputs, at sizes that span several tiles and ragged tails.

Bars: K/V rows written to the cache <= 1e-2 max relative error per (b, head) slice; FP8 codes
each the correct rounding of a value within the fp32 projection's error bound of the oracle's
exact value (codes more than one e4m3 step from the oracle's at most 1 in 10^4; scales
<= 1e-2); attention output <= 2e-2; untouched rows, guard bands and index outputs bit-exact;
drift decisions exact (away from |sigma - gamma| < 1e-5).
"""
import math

import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_cases import (ACT_TORCH, GpuLayer, check_fp8_rows, elem_rel_err, fp8_delta, say,
                       slice_rel_err, to_dev)

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # collected on CPU-only hosts, never run there
    pytest.skip("needs a GPU", allow_module_level=True)

import diffusion_kv_cache_amd as dkv  # noqa: E402

C = synth.custom
REFRESH_CASES = {
    "skinny_bf16_d128": C(batch=1, hidden=512, q_heads=4, kv_heads=4, head_dim=128, seq=96,
                          prompt=48, block_start=50, block_len=20, seed=11),
    "skinny_gqa_d64_scattered": C(batch=3, hidden=256, q_heads=6, kv_heads=2, head_dim=64,
                                  seq=130, prompt=60, refresh="window+subset", window=5,
                                  subset=7, seed=12),
    "tiled64_bf16_ragged": C(batch=2, hidden=512, q_heads=4, kv_heads=2, head_dim=128, seq=200,
                             prompt=100, block_start=101, block_len=37, seed=13),
    "tiled_bk32_h256": C(batch=2, hidden=256, q_heads=2, kv_heads=2, head_dim=128, seq=90,
                         prompt=40, block_start=41, block_len=40, seed=14),
    "fp8_tiled_d128": C(batch=2, hidden=512, q_heads=4, kv_heads=2, head_dim=128, seq=150,
                        prompt=70, cache="fp8", block_start=71, block_len=33, seed=15),
    "fp8_d64_scattered": C(batch=2, hidden=256, q_heads=6, kv_heads=2, head_dim=64, seq=100,
                           prompt=50, cache="fp8", refresh="window+subset", window=4, subset=9,
                           seed=16),
    "f32_d64": C(batch=2, hidden=256, q_heads=4, kv_heads=4, head_dim=64, seq=70, prompt=30,
                 act="f32", cache="f32", block_start=31, block_len=9, seed=17),
    "splitk_fp8_h768_m64": C(batch=4, hidden=768, q_heads=6, kv_heads=3, head_dim=128, seq=64,
                             prompt=30, cache="fp8", block_start=40, block_len=16, seed=21),
    "splitk_bf16_h768_d64": C(batch=1, hidden=768, q_heads=3, kv_heads=1, head_dim=64, seq=90,
                              prompt=40, block_start=45, block_len=45, seed=22),
    "f32_d128_gqa": C(batch=1, hidden=512, q_heads=4, kv_heads=2, head_dim=128, seq=40,
                      prompt=20, act="f32", cache="f32", block_start=3, block_len=30, seed=18),
    # more split-K shapes: GQA with D = 64 over a scattered set, 129 query heads of 64, and
    # 33 + 33 + 33 heads of 128
    "splitk_gqa_d64": C(batch=2, hidden=512, q_heads=6, kv_heads=2, head_dim=64, seq=80,
                        prompt=40, refresh="window+subset", window=5, subset=8, seed=23),
    "splitk_d64_129_heads": C(batch=1, hidden=256, q_heads=129, kv_heads=1, head_dim=64,
                              seq=40, prompt=20, block_start=21, block_len=7, seed=24),
    "splitk_d128_33_heads": C(batch=2, hidden=256, q_heads=33, kv_heads=33, head_dim=128,
                              seq=48, prompt=24, block_start=24, block_len=16, seed=25),
    # a hidden size past the split-K limit: ten rows through the tiled GEMM
    "gemm_few_rows_h8448": C(batch=1, hidden=8448, q_heads=1, kv_heads=1, head_dim=64,
                              seq=40, prompt=20, block_start=20, block_len=10, seed=26),
    # the largest hidden size of the split-K path (its LDS slice is largest here)
    "splitk_h8192_m64": C(batch=2, hidden=8192, q_heads=1, kv_heads=1, head_dim=128, seq=48,
                          prompt=16, block_start=16, block_len=32, seed=28),
    # 256 rows, D = 128: the sixteen-wave GEMM form, two row tiles
    "gemm_wide_m256_fp8": C(batch=8, hidden=512, q_heads=2, kv_heads=2, head_dim=128, seq=64,
                            prompt=32, cache="fp8", block_start=32, block_len=32, seed=27),
}


def _rows_mask(wl, idx):
    mask = np.zeros((wl.batch, wl.seq), bool)
    for b in range(wl.batch):
        mask[b, idx[b]] = True
    return mask


@pytest.mark.parametrize("name", list(REFRESH_CASES))
def test_refresh_parity_and_untouched_rows(name):
    wl = REFRESH_CASES[name]
    say(f"[refresh parity] {name} M={wl.batch * wl.n_refresh}")
    inp = synth.make_inputs(wl)
    h_cur = inp.hidden_cur()
    layer = GpuLayer(wl, inp.w)
    c = layer.cache
    before = {k: t.clone() for k, t in (("k", c.k), ("v", c.v), ("ks", c.k_scale),
                                         ("vs", c.v_scale)) if t is not None}
    snap = c.storage.clone()
    q = layer.refresh(to_dev(h_cur, layer.act), inp.idx)   # on the poisoned cache
    torch.cuda.synchronize()
    assert layer.guards_intact(snap)

    mask = _rows_mask(wl, inp.idx)                          # [B, S]
    for key, t in (("k", c.k), ("v", c.v), ("ks", c.k_scale), ("vs", c.v_scale)):
        if t is None:
            continue
        as_int = {torch.bfloat16: torch.int16, torch.float32: torch.int32,
                  torch.uint8: torch.uint8}[t.dtype]        # bitwise: the poison holds NaNs
        now = t.cpu().view(as_int)
        old = before[key].cpu().view(as_int)
        m = torch.from_numpy(mask)[:, None, :].expand(now.shape[:3])
        assert torch.equal(now[~m], old[~m]), f"{key}: a row outside the refresh set changed"

    ref = oracle.refresh_rows(oracle.Cache(wl), h_cur, inp.w, inp.idx)
    qref = oracle.queries(wl, h_cur, inp.w, inp.idx)
    kg, vg = layer.kv_host()
    for b in range(wl.batch):
        rows = inp.idx[b]
        if wl.cache != "fp8":
            assert slice_rel_err(kg[b][:, rows], ref.k[b][:, rows], (0,)) <= 1e-2
            assert slice_rel_err(vg[b][:, rows], ref.v[b][:, rows], (0,)) <= 1e-2
            say(f"  b={b} elementwise (floor 1e-2): K {elem_rel_err(kg[b][:, rows], ref.k[b][:, rows], (0,)):.2e} "
                f"V {elem_rel_err(vg[b][:, rows], ref.v[b][:, rows], (0,)):.2e}")
        else:  # one e4m3 step near amax is 1/14 of the row's range: the bar is on codes
            for nm in ("k", "v"):
                gc = getattr(c, nm).cpu().numpy()[b][:, rows]
                gs = getattr(c, nm + "_scale").cpu().numpy()[b][:, rows]
                delta = fp8_delta(wl, h_cur[b, rows], inp.w, nm).transpose(1, 0, 2)
                far = check_fp8_rows(gc, gs, getattr(ref, nm + "_exact")[b][:, rows],
                                     getattr(ref, nm + "_codes")[b][:, rows], delta)
                assert far <= gc.size // 10000
                np.testing.assert_allclose(gs, getattr(ref, nm + "_scale")[b][:, rows], rtol=1e-2)
    qg = q.float().cpu().numpy()
    assert slice_rel_err(qg, qref, (0, 2)) <= 1e-2


@pytest.mark.parametrize("name", ["skinny_bf16_d128", "skinny_gqa_d64_scattered",
                                  "tiled64_bf16_ragged", "fp8_tiled_d128", "f32_d64",
                                  "f32_d128_gqa", "splitk_fp8_h768_m64", "splitk_bf16_h768_d64",
                                  "splitk_gqa_d64", "splitk_d64_129_heads",
                                  "splitk_d128_33_heads", "splitk_h8192_m64",
                                  "gemm_few_rows_h8448",
                                  "gemm_wide_m256_fp8"])
def test_step_reproduces_full_refresh_bitwise(name):
    """Cached step (prefill on H_prev, refresh of R on H_cur) stores exactly what a full
    refresh on H_cur stores -- on the GPU too, whichever kernel each call picks."""
    wl = REFRESH_CASES[name]
    say(f"[step == full refresh] {name}")
    inp = synth.make_inputs(wl)
    h_prev = to_dev(inp.hidden_prev, ACT_TORCH[wl.act])
    h_cur = to_dev(inp.hidden_cur(), ACT_TORCH[wl.act])
    full = GpuLayer(wl, inp.w)
    q_full = full.prefill(h_cur)
    step = GpuLayer(wl, inp.w)
    step.prefill(h_prev)
    q_step = step.refresh(h_cur, inp.idx)
    torch.cuda.synchronize()
    assert torch.equal(full.cache.region, step.cache.region)
    for b in range(wl.batch):
        assert torch.equal(q_full[b, torch.from_numpy(inp.idx[b]).long().cuda()], q_step[b])


@pytest.mark.parametrize("name", ["skinny_bf16_d128", "fp8_tiled_d128"])
def test_gemm_wide_offsets_match(name):
    """The refresh GEMM's 64-bit operand addressing (taken for operands of 4 GB or more)
    stores exactly what the 32-bit-offset form stores."""
    wl = REFRESH_CASES[name]
    say(f"[wide offsets] {name}")
    inp = synth.make_inputs(wl)
    h_prev = to_dev(inp.hidden_prev, ACT_TORCH[wl.act])
    base = GpuLayer(wl, inp.w)
    q_base = base.prefill(h_prev)
    prev = dkv.dllm_set_options(dkv.DLLM_OPT_WIDE_OFFSETS)
    try:
        wide = GpuLayer(wl, inp.w)
        q_wide = wide.prefill(h_prev)
        torch.cuda.synchronize()
    finally:
        dkv.dllm_set_options(prev)
    assert torch.equal(base.cache.region, wide.cache.region)
    assert torch.equal(q_base, q_wide)


def test_tiled128_prefill_matches_oracle_and_step():
    """A prefill large enough for the 128-row tiles, against the oracle and against a
    step on the small-M kernel (bitwise)."""
    wl = C(batch=2, hidden=256, q_heads=32, kv_heads=8, head_dim=128, seq=704, prompt=352,
           block_start=400, block_len=24, seed=19)
    say("[tiled128 prefill]")
    inp = synth.make_inputs(wl)
    h_cur = inp.hidden_cur()
    full = GpuLayer(wl, inp.w)
    q_full = full.prefill(to_dev(h_cur, torch.bfloat16))
    torch.cuda.synchronize()
    kg, vg = full.kv_host()
    ref = oracle.prefill(wl, h_cur, inp.w, batches=[1])
    assert slice_rel_err(kg[1], ref.k[1], (0,)) <= 1e-2
    assert slice_rel_err(vg[1], ref.v[1], (0,)) <= 1e-2
    all_rows = np.tile(np.arange(wl.seq, dtype=np.int32), (wl.batch, 1))
    qref = oracle.queries(wl, h_cur, inp.w, all_rows, batches=[0], q_heads=[0, 17, 31])
    qg = q_full.float().cpu().numpy()[0][:, [0, 17, 31]]
    assert slice_rel_err(qg, qref[0], (1,)) <= 1e-2
    step = GpuLayer(wl, inp.w)
    step.prefill(to_dev(inp.hidden_prev, torch.bfloat16))
    step.refresh(to_dev(h_cur, torch.bfloat16), inp.idx)
    torch.cuda.synchronize()
    assert torch.equal(full.cache.region, step.cache.region)


@pytest.mark.parametrize("n_rows", [20, 160])
def test_exact_values_on_integer_grid(n_rows):
    """Entries in {-2..2}/16 make every fp32 and fp64 partial sum exact, so the V rows (never
    rotated) must match the oracle bit for bit whatever the summation order: this pins the
    gather, the head split and the scatter."""
    wl = C(batch=2, hidden=512, q_heads=4, kv_heads=2, head_dim=128, seq=200, prompt=10,
           block_start=11, block_len=n_rows, seed=20)
    say(f"[integer grid] n={n_rows}")
    rng = np.random.default_rng(5)
    hidden = synth.small_integer_grid(rng, (wl.batch, wl.seq, wl.hidden))
    w = synth.small_integer_grid(rng, (wl.n_cols, wl.hidden))
    idx = np.tile(np.arange(11, 11 + n_rows, dtype=np.int32), (wl.batch, 1))
    idx[1] += 3
    layer = GpuLayer(wl, w)
    layer.refresh(to_dev(hidden, torch.bfloat16), idx)
    torch.cuda.synchronize()
    ref = oracle.refresh_rows(oracle.Cache(wl), hidden, w, idx)
    vg = layer.cache.v.float().cpu().numpy().astype(np.float64)
    for b in range(wl.batch):
        np.testing.assert_array_equal(vg[b][:, idx[b]], ref.v[b][:, idx[b]])


ATT_CASES = {
    "bf16_g1_splits": C(batch=1, hidden=256, q_heads=2, kv_heads=2, head_dim=128, seq=1000,
                        prompt=500, block_start=500, block_len=20, seed=31),
    # 8192 keys over two heads: 64 key splits, more than one merge batch
    "bf16_many_splits": C(batch=1, hidden=256, q_heads=2, kv_heads=2, head_dim=128, seq=8192,
                          prompt=4096, block_start=4096, block_len=20, seed=41),
    # FP8 cache, 8192 keys of one head: 32 key splits
    "fp8_many_splits": C(batch=1, hidden=256, q_heads=1, kv_heads=1, head_dim=128, seq=8192,
                         prompt=4096, cache="fp8", block_start=4096, block_len=20, seed=42),
    "bf16_g7_qt128_ragged": C(batch=2, hidden=256, q_heads=7, kv_heads=1, head_dim=128, seq=300,
                              prompt=150, refresh="window+subset", window=8, subset=72, seed=32),
    "bf16_g3_qt64_d64": C(batch=2, hidden=256, q_heads=6, kv_heads=2, head_dim=64, seq=257,
                          prompt=128, block_start=130, block_len=15, seed=33),
    "bf16_s17": C(batch=2, hidden=256, q_heads=2, kv_heads=1, head_dim=128, seq=17, prompt=8,
                  block_start=8, block_len=9, seed=34),
    "bf16_s1": C(batch=1, hidden=256, q_heads=2, kv_heads=2, head_dim=64, seq=1, prompt=0,
                 block_start=0, block_len=1, seed=35),
    "fp8_g1": C(batch=2, hidden=512, q_heads=4, kv_heads=4, head_dim=128, seq=333, prompt=200,
                cache="fp8", block_start=200, block_len=33, seed=36),
    "fp8_d64_g2_splits": C(batch=1, hidden=256, q_heads=4, kv_heads=2, head_dim=64, seq=900,
                           prompt=450, cache="fp8", block_start=450, block_len=16, seed=37),
    "f32_d64": C(batch=2, hidden=256, q_heads=4, kv_heads=2, head_dim=64, seq=77, prompt=40,
                 act="f32", cache="f32", block_start=41, block_len=9, seed=38),
    # one case per remaining (cache dtype, packed query tile, head dim) kernel instance
    "bf16_g4_qt64_d128": C(batch=2, hidden=256, q_heads=8, kv_heads=2, head_dim=128, seq=410,
                           prompt=200, block_start=203, block_len=40, seed=39),
    "bf16_g8_qt128_d64": C(batch=1, hidden=256, q_heads=8, kv_heads=1, head_dim=64, seq=333,
                           prompt=160, block_start=161, block_len=70, seed=40),
    "fp8_g1_qt32": C(batch=2, hidden=512, q_heads=4, kv_heads=4, head_dim=128, seq=611,
                     prompt=300, cache="fp8", block_start=301, block_len=20, seed=41),
    "fp8_g8_qt128": C(batch=1, hidden=256, q_heads=8, kv_heads=1, head_dim=128, seq=290,
                      prompt=150, cache="fp8", block_start=150, block_len=64, seed=42),
    "fp8_d64_g4_qt64": C(batch=2, hidden=256, q_heads=8, kv_heads=2, head_dim=64, seq=520,
                         prompt=260, cache="fp8", block_start=263, block_len=20, seed=43),
    "fp8_d64_g8_qt128": C(batch=1, hidden=256, q_heads=8, kv_heads=1, head_dim=64, seq=300,
                          prompt=150, cache="fp8", block_start=151, block_len=70, seed=44),
    # one query head per KV head, n <= 32, heads enough not to split keys (B * Hkv >= 512):
    # attention and mass in one launch -- ragged last key tile, a wave without tiles (3 tiles
    # for 4 waves), a single key
    "fused_d128_ragged": C(batch=16, hidden=256, q_heads=32, kv_heads=32, head_dim=128, seq=300,
                           prompt=150, block_start=151, block_len=20, seed=46),
    "fused_d64_three_tiles": C(batch=16, hidden=256, q_heads=32, kv_heads=32, head_dim=64,
                               seq=70, prompt=30, block_start=32, block_len=32, seed=47),
    "fused_s1": C(batch=16, hidden=256, q_heads=32, kv_heads=32, head_dim=64, seq=1, prompt=0,
                  block_start=0, block_len=1, seed=48),
    # few heads (the keys are split; the mass pass merges the splits), ragged last key tile
    "few_heads_d128_ragged": C(batch=2, hidden=256, q_heads=16, kv_heads=16, head_dim=128, seq=1000,
                            prompt=500, block_start=501, block_len=24, seed=50),
    # more than six key tiles per wave: scores not kept in registers, K read in both passes
    "fused_d128_two_k_passes": C(batch=16, hidden=256, q_heads=32, kv_heads=32, head_dim=128,
                                 seq=900, prompt=450, block_start=451, block_len=24, seed=49),
    # n * G = 8800 packed rows: more log-sum-exp values than the mass pass stages in LDS
    "bf16_mass_rows_over_lds": C(batch=1, hidden=256, q_heads=8, kv_heads=1, head_dim=64,
                                 seq=1100, prompt=0, block_start=0, block_len=1100, seed=45),
}


@pytest.mark.parametrize("name", list(ATT_CASES))
def test_attention_parity(name):
    wl = ATT_CASES[name]
    say(f"[attention parity] {name}")
    inp = synth.make_inputs(wl)
    h_cur = inp.hidden_cur()
    layer = GpuLayer(wl, inp.w)
    layer.prefill(to_dev(inp.hidden_prev, layer.act))
    q = layer.refresh(to_dev(h_cur, layer.act), inp.idx)
    out, lse, mass = layer.attention(q, want_mass=True)
    torch.cuda.synchronize()

    cache = oracle.refresh_rows(oracle.prefill(wl, inp.hidden_prev, inp.w), h_cur, inp.w, inp.idx)
    qref = oracle.queries(wl, h_cur, inp.w, inp.idx)
    o_ref, l_ref, m_ref = oracle.attend(wl, qref, cache, want_mass=True)
    assert slice_rel_err(out.float().cpu().numpy(), o_ref, (0, 2)) <= 2e-2
    np.testing.assert_allclose(lse.cpu().numpy(), l_ref, rtol=0, atol=1e-2)
    assert slice_rel_err(mass.cpu().numpy(), m_ref, (0, 1)) <= 2e-2
    # each query's probabilities sum to one: every head's mass sums to n
    np.testing.assert_allclose(mass.sum(-1).cpu().numpy(), wl.n_refresh, rtol=1e-3)
    # without the mass the key splits are merged by their own kernel
    out2, lse2, _ = layer.attention(q, want_mass=False)
    torch.cuda.synchronize()
    assert slice_rel_err(out2.float().cpu().numpy(), o_ref, (0, 2)) <= 2e-2
    np.testing.assert_allclose(lse2.cpu().numpy(), l_ref, rtol=0, atol=1e-2)
    if wl.seq == 1:
        vg = layer.cache.v.float()
        for h in range(wl.q_heads):
            assert torch.equal(out[0, 0, h].float(), vg[0, h // (wl.q_heads // wl.kv_heads), 0])


DRIFT_CASES = {
    "bf16_gqa": dict(B=3, Hq=6, Hkv=2, S=300, D=128, k=32, dt="bf16"),
    "bf16_k64_d64": dict(B=2, Hq=4, Hkv=4, S=500, D=64, k=64, dt="bf16"),
    "bf16_S_below_k": dict(B=2, Hq=2, Hkv=1, S=20, D=128, k=32, dt="bf16"),
    "f32": dict(B=2, Hq=4, Hkv=2, S=50, D=64, k=8, dt="f32"),
    # rows past 4096 keys: further rounds of mass loads and of the selection walk
    "bf16_long_S": dict(B=2, Hq=2, Hkv=2, S=6000, D=64, k=32, dt="bf16"),
    # a long row that is not a multiple of 4 (scalar mass loads), GQA
    "bf16_long_ragged_gqa": dict(B=2, Hq=4, Hkv=2, S=4099, D=128, k=32, dt="bf16"),
    # degenerate budgets: one tracked token; exactly as many positions as the budget
    "bf16_k1": dict(B=2, Hq=2, Hkv=1, S=100, D=128, k=1, dt="bf16"),
    "bf16_S_equals_k": dict(B=2, Hq=2, Hkv=2, S=32, D=64, k=32, dt="bf16"),
    # the largest row and budget the tracking update takes (S = 16384, k = 64)
    "bf16_max_S_max_k": dict(B=2, Hq=2, Hkv=2, S=16384, D=64, k=64, dt="bf16"),
}


def _drift_inputs(p, seed):
    rng = np.random.default_rng(seed)
    B, Hq, Hkv, S, D, k = p["B"], p["Hq"], p["Hkv"], p["S"], p["D"], p["k"]
    G = Hq // Hkv
    kc = rng.standard_normal((B, Hkv, S, D)).astype(np.float32)
    vc = rng.standard_normal((B, Hkv, S, D)).astype(np.float32)
    if p["dt"] == "bf16":
        kc, vc = synth.round_to_bf16(kc), synth.round_to_bf16(vc)
    T = -np.ones((B, Hq, k), np.int32)
    buf = np.zeros((B, Hq, k, 2, D), np.float32)
    for b in range(B):
        for h in range(Hq):
            if b == 0 and h == 0:
                continue                                   # empty tracking set
            take = min(k, S) - (3 if (b, h) == (1, 1) and min(k, S) > 3 else 0)
            pos = np.sort(rng.choice(S, size=take, replace=False)).astype(np.int32)
            T[b, h, :take] = pos
            alpha = rng.uniform(0.3, 1.0)
            g = h // G
            for t, j in enumerate(pos):
                noise = rng.standard_normal((2, D)).astype(np.float32)
                rows = np.stack([kc[b, g, j], vc[b, g, j]])
                buf[b, h, t] = alpha * rows + math.sqrt(1 - alpha * alpha) * noise
    if p["dt"] == "bf16":
        buf = synth.round_to_bf16(buf)
    mass = synth.uniform_mass(rng, (B, Hq, S), ties=S // 5)
    mass[0, 1, :] = 0.25                                   # all tied: lowest positions win
    if S > k:                                              # exactly k values in [4, 8): the
        big = rng.choice(S, size=k, replace=False)         # leading byte alone decides
        mass[1, 0, :] = rng.uniform(0.0, 1.0, S).astype(np.float32)
        mass[1, 0, big] = rng.uniform(4.0, 8.0, k).astype(np.float32)
    return kc, vc, T, buf, mass


@pytest.mark.parametrize("name", list(DRIFT_CASES))
@pytest.mark.parametrize("update", [True, False])
@pytest.mark.parametrize("same_launch", [False, True])
def test_drift_stagewise(name, update, same_launch):
    """Drift test and tracking update on identical seeded inputs: sigma to fp32 rounding of
    the fp64 value, decisions and the new tracking set exactly, buffer refilled bitwise.
    same_launch: the decision taken in the drift kernel through a workspace (left zero, and
    right again on a second call) instead of by the second kernel."""
    p = DRIFT_CASES[name]
    say(f"[drift] {name} update={update} same_launch={same_launch}")
    B, Hq, Hkv, S, D, k = p["B"], p["Hq"], p["Hkv"], p["S"], p["D"], p["k"]
    kc, vc, T, buf, mass = _drift_inputs(p, 40 + len(name))
    tdt = torch.bfloat16 if p["dt"] == "bf16" else torch.float32
    cache = dkv.Cache(B, Hkv, S, D, dkv.DLLM_BF16 if p["dt"] == "bf16" else dkv.DLLM_F32)
    cache.k.copy_(torch.from_numpy(kc).to(tdt))
    cache.v.copy_(torch.from_numpy(vc).to(tdt))
    T_d = torch.from_numpy(T).cuda()
    buf_d = torch.from_numpy(buf).to(tdt).cuda()
    mass_d = torch.from_numpy(mass).cuda()
    sigma = torch.empty((B, Hq), dtype=torch.float32, device="cuda")
    refresh = torch.empty((B,), dtype=torch.uint8, device="cuda")
    gamma = float(np.float32(0.9))
    dws = dkv.drift_workspace(B) if same_launch else None
    dkv.dllm_drift_check(cache, Hq, k, gamma, T_d, buf_d, mass_d if update else None, sigma,
                         refresh, dws)
    torch.cuda.synchronize()
    if same_launch:
        assert not dws.any()

    s_ref, r_ref = oracle.drift(buf.astype(np.float64), T, kc.astype(np.float64),
                                vc.astype(np.float64), gamma)
    np.testing.assert_allclose(sigma.cpu().numpy(), s_ref, rtol=0, atol=2e-7)
    assert s_ref[0, 0] == 1.0 and sigma[0, 0].item() == 1.0
    margin = np.abs(s_ref.min(axis=1) - gamma)
    decided = margin >= 1e-5
    np.testing.assert_array_equal(refresh.cpu().numpy()[decided], r_ref[decided])
    assert (sigma.cpu().numpy() < gamma).any(axis=1).astype(np.uint8).tolist() == \
        refresh.cpu().numpy().tolist()
    if same_launch:
        # a second call on the same workspace (inputs now the updated set and buffer)
        sigma2 = torch.empty_like(sigma)
        refresh2 = torch.full_like(refresh, 7)
        dkv.dllm_drift_check(cache, Hq, k, gamma, T_d.clone(), buf_d.clone(), None, sigma2,
                             refresh2, dws)
        torch.cuda.synchronize()
        assert not dws.any()
        assert (sigma2.cpu().numpy() < gamma).any(axis=1).astype(np.uint8).tolist() == \
            refresh2.cpu().numpy().tolist()
    if not update:
        assert torch.equal(T_d.cpu(), torch.from_numpy(T))
        return
    T_ref = oracle.topk(mass.astype(np.float64), k)
    np.testing.assert_array_equal(T_d.cpu().numpy(), T_ref)
    assert list(T_d[0, 1, :min(k, S)].cpu().numpy()) == list(range(min(k, S)))
    G = Hq // Hkv
    bg = buf_d.float().cpu().numpy()
    for b in range(B):
        for h in range(Hq):
            for t in range(k):
                j = T_ref[b, h, t]
                if j < 0:
                    assert not bg[b, h, t].any()
                else:
                    np.testing.assert_array_equal(bg[b, h, t, 0], kc[b, h // G, j])
                    np.testing.assert_array_equal(bg[b, h, t, 1], vc[b, h // G, j])


DRIFT_FP8_CASES = {
    "fp8_gqa": dict(B=3, Hq=6, Hkv=2, S=300, D=128, k=32),
    "fp8_d64_k64": dict(B=2, Hq=4, Hkv=4, S=500, D=64, k=64),
    "fp8_S_below_k": dict(B=2, Hq=2, Hkv=1, S=20, D=128, k=32),
    # rows past 4096 keys (64 mass values per thread), k = 1
    "fp8_long_k1": dict(B=2, Hq=2, Hkv=2, S=6000, D=128, k=1),
}


@pytest.mark.parametrize("name", list(DRIFT_FP8_CASES))
@pytest.mark.parametrize("update", [True, False])
@pytest.mark.parametrize("same_launch", [False, True])
def test_drift_fp8(name, update, same_launch):
    """Drift test on an FP8 cache: the tracked rows are E4M3 codes with one fp32 scale per
    row, compared as code * scale in fp64 (the oracle's drift on the decoded values); the new
    set exact, the buffer refilled with the cache's codes and scales bitwise."""
    p = DRIFT_FP8_CASES[name]
    say(f"[drift fp8] {name} update={update} same_launch={same_launch}")
    B, Hq, Hkv, S, D, k = p["B"], p["Hq"], p["Hkv"], p["S"], p["D"], p["k"]
    G = Hq // Hkv
    rng = np.random.default_rng(90 + len(name))
    kcod, ksc, kdq = oracle.fp8_quantize_rows(rng.standard_normal((B, Hkv, S, D)) * 0.7)
    vcod, vsc, vdq = oracle.fp8_quantize_rows(rng.standard_normal((B, Hkv, S, D)) * 1.3)
    T = -np.ones((B, Hq, k), np.int32)
    rows = np.zeros((B, Hq, k, 2, D))
    for b in range(B):
        for h in range(Hq):
            if b == 0 and h == 0:
                continue                                   # empty tracking set
            take = min(k, S) - (1 if (b, h) == (1, 1) and min(k, S) > 1 else 0)
            pos = np.sort(rng.choice(S, size=take, replace=False)).astype(np.int32)
            T[b, h, :take] = pos
            alpha = rng.uniform(0.3, 1.0)
            for t, j in enumerate(pos):
                base = np.stack([kdq[b, h // G, j], vdq[b, h // G, j]])
                rows[b, h, t] = alpha * base + math.sqrt(1 - alpha * alpha) * \
                    rng.standard_normal((2, D))
    bcod, bsc, bdq = oracle.fp8_quantize_rows(rows)
    bdq[T < 0] = 0.0
    mass = synth.uniform_mass(rng, (B, Hq, S), ties=S // 5)

    cache = dkv.Cache(B, Hkv, S, D, dkv.DLLM_FP8_E4M3)
    cache.k.copy_(torch.from_numpy(kcod))
    cache.v.copy_(torch.from_numpy(vcod))
    cache.k_scale.copy_(torch.from_numpy(ksc))
    cache.v_scale.copy_(torch.from_numpy(vsc))
    nb = dkv.track_buffer_bytes(cache, Hq, k)
    ncod = B * Hq * k * 2 * D
    assert nb == ncod + B * Hq * k * 2 * 4
    buf_d = torch.zeros(nb, dtype=torch.uint8, device="cuda")
    buf_d[:ncod].copy_(torch.from_numpy(bcod.reshape(-1)))
    buf_d[ncod:].view(torch.float32).copy_(torch.from_numpy(bsc.reshape(-1)))
    T_d = torch.from_numpy(T).cuda()
    mass_d = torch.from_numpy(mass).cuda()
    sigma = torch.empty((B, Hq), dtype=torch.float32, device="cuda")
    refresh = torch.empty((B,), dtype=torch.uint8, device="cuda")
    gamma = float(np.float32(0.9))
    dws = dkv.drift_workspace(B) if same_launch else None
    dkv.dllm_drift_check(cache, Hq, k, gamma, T_d, buf_d, mass_d if update else None, sigma,
                         refresh, dws)
    torch.cuda.synchronize()
    if same_launch:
        assert not dws.any()

    s_ref, r_ref = oracle.drift(bdq, T, kdq, vdq, gamma)
    np.testing.assert_allclose(sigma.cpu().numpy(), s_ref, rtol=0, atol=2e-7)
    assert sigma[0, 0].item() == 1.0
    decided = np.abs(s_ref.min(axis=1) - gamma) >= 1e-5
    np.testing.assert_array_equal(refresh.cpu().numpy()[decided], r_ref[decided])
    assert (sigma.cpu().numpy() < gamma).any(axis=1).astype(np.uint8).tolist() == \
        refresh.cpu().numpy().tolist()
    if not update:
        assert torch.equal(T_d.cpu(), torch.from_numpy(T))
        assert torch.equal(buf_d[:ncod].cpu(), torch.from_numpy(bcod.reshape(-1)))
        return
    T_ref = oracle.topk(mass.astype(np.float64), k)
    np.testing.assert_array_equal(T_d.cpu().numpy(), T_ref)
    codes = buf_d[:ncod].cpu().numpy().reshape(B, Hq, k, 2, D)
    scales = buf_d[ncod:].view(torch.float32).cpu().numpy().reshape(B, Hq, k, 2)
    for b in range(B):
        for h in range(Hq):
            for t in range(k):
                j = T_ref[b, h, t]
                if j < 0:
                    assert not codes[b, h, t].any() and not scales[b, h, t].any()
                else:
                    np.testing.assert_array_equal(codes[b, h, t, 0], kcod[b, h // G, j])
                    np.testing.assert_array_equal(codes[b, h, t, 1], vcod[b, h // G, j])
                    assert scales[b, h, t, 0] == ksc[b, h // G, j]
                    assert scales[b, h, t, 1] == vsc[b, h // G, j]


@pytest.mark.parametrize("scale", [1.0, 0.0123, 3.7])
def test_fp8_codec_matches_oracle(scale):
    say(f"[fp8 codec] scale={scale}")
    vals = oracle.e4m3_decode(np.arange(256, dtype=np.uint8))
    fin = vals[~np.isnan(vals)]
    mids = (np.sort(fin)[:-1] + np.sort(fin)[1:]) / 2
    sweep = np.linspace(-500, 500, 400_001)
    tiny = np.linspace(-0.02, 0.02, 20_001)
    special = np.array([0.0, -0.0, np.inf, -np.inf, np.nan, 448.0, 464.0, -464.0, 1e30])
    x = np.concatenate([fin, mids, sweep, tiny, special]) * scale
    x32 = x.astype(np.float32)
    xd = torch.from_numpy(x32).cuda()
    codes = torch.empty(x32.shape, dtype=torch.uint8, device="cuda")
    dec = torch.empty(x32.shape, dtype=torch.float32, device="cuda")
    dkv.dllm_fp8_e4m3_roundtrip(xd, scale, codes, dec)
    torch.cuda.synchronize()
    q32 = (x32 / np.float32(scale)).astype(np.float32)
    want = oracle.e4m3_encode(q32.astype(np.float64))
    got = codes.cpu().numpy()
    np.testing.assert_array_equal(got, want)
    want_dec = (oracle.e4m3_decode(want).astype(np.float32) * np.float32(scale)).astype(np.float32)
    np.testing.assert_array_equal(dec.cpu().numpy(), want_dec)


def test_zero_rows_is_a_no_op():
    wl = REFRESH_CASES["tiled64_bf16_ragged"]
    inp = synth.make_inputs(wl)
    layer = GpuLayer(wl, inp.w)
    snap = layer.cache.storage.clone()
    idx = np.zeros((wl.batch, 0), np.int32)
    q = layer.refresh(to_dev(inp.hidden_prev, torch.bfloat16), idx)
    torch.cuda.synchronize()
    assert q.numel() == 0 and torch.equal(snap, layer.cache.storage)


def test_debug_mode_rejects_bad_index_lists():
    """Debug mode: index lists are checked by a device pass before the refresh launches."""
    wl = REFRESH_CASES["skinny_bf16_d128"]
    inp = synth.make_inputs(wl)
    layer = GpuLayer(wl, inp.w)
    h = to_dev(inp.hidden_prev, torch.bfloat16)
    prev = dkv.dllm_set_options(dkv.DLLM_OPT_DEBUG)
    try:
        _debug_rejections(layer, h, inp, wl)
    finally:
        dkv.dllm_set_options(prev)


def _debug_rejections(layer, h, inp, wl):
    unsorted = inp.idx.copy()
    unsorted[0, [0, 1]] = unsorted[0, [1, 0]]          # in range: harmless if not checked
    with pytest.raises(dkv.DllmError) as e:
        layer.refresh(h, unsorted)
    assert e.value.status == dkv.DLLM_EINVAL
    dup = inp.idx.copy()
    dup[0, 1] = dup[0, 0]
    with pytest.raises(dkv.DllmError):
        layer.refresh(h, dup)
    oob = inp.idx.copy()
    oob[0, -1] = wl.seq                                 # rejected before launching
    with pytest.raises(dkv.DllmError) as e:
        layer.refresh(h, oob)
    assert "outside" in str(e.value)
    neg = inp.idx.copy()
    neg[0, 0] = -1
    with pytest.raises(dkv.DllmError):
        layer.refresh(h, neg)
    layer.refresh(h, inp.idx)                           # a valid list still runs
    torch.cuda.synchronize()


def test_binding_rejects_mismatched_tensors():
    wl = REFRESH_CASES["skinny_bf16_d128"]
    inp = synth.make_inputs(wl)
    layer = GpuLayer(wl, inp.w)
    h = to_dev(inp.hidden_prev, torch.bfloat16)
    with pytest.raises(dkv.DllmError):
        layer.refresh(h[:, :-1].contiguous(), inp.idx)          # wrong S
    q = torch.empty((wl.batch, wl.n_refresh, wl.q_heads, wl.head_dim), dtype=torch.bfloat16,
                    device="cuda")
    with pytest.raises(dkv.DllmError):
        dkv.dllm_block_attention(layer.cache, q, wl.q_heads, 0.1, q[:, :1].contiguous())
