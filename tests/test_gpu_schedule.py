"""The layer schedule on the device through the C ABI, against the oracle: the similarity
choice of the step rows (cosines to 1e-12, chosen rows exact, ties to the lower row), the
per-layer row schedule and the feature-row copy (exact), and a step over four synthetic layers
checked stage by stage (each stage's oracle fed the GPU's inputs to that stage): decisions,
row sets, tracked sets and copies exact, cache rows <= 1e-2 and bit for bit those of a full
refresh, attention <= 2e-2, sigma <= 2e-6; the drift fires at the planted layers only.
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

BF, F32 = torch.bfloat16, torch.float32


def _features(rng, B, S, H, act):
    """Current features and cached ones that moved by a per-row random amount."""
    cur = rng.standard_normal((B, S, H)).astype(np.float32)
    alpha = rng.uniform(-0.2, 1.0, size=(B, S, 1)).astype(np.float32)
    cached = alpha * cur + np.sqrt(1 - alpha ** 2) * rng.standard_normal((B, S, H)).astype(
        np.float32)
    if act == "bf16":
        cur, cached = synth.round_to_bf16(cur), synth.round_to_bf16(cached)
    return cur, cached


SELECT_CASES = {
    "bf16_s600": (4, 600, 512, "bf16", 300, 16, 64),
    "f32_s3000": (2, 3000, 256, "f32", 1000, 32, 500),
    "bf16_s8192_nowindow": (2, 8192, 64, "bf16", 0, 0, 100),
    "window_only": (3, 200, 128, "bf16", 50, 20, 0),
}


@pytest.mark.parametrize("name", list(SELECT_CASES))
def test_similarity_select_matches_oracle(name):
    B, S, H, act, lo, window, k = SELECT_CASES[name]
    say(f"[select] {name}")
    rng = np.random.default_rng(len(name) + 7)
    cur, cached = _features(rng, B, S, H, act)
    ws = rng.integers(0, S - window + 1, size=B).astype(np.int32)
    dt = BF if act == "bf16" else F32
    idx = torch.full((B, window + k), -5, dtype=torch.int32, device="cuda")
    sim = torch.full((B, S), float("nan"), dtype=torch.float64, device="cuda")
    dkv.dllm_similarity_select(to_dev(cur, dt), to_dev(cached, dt), lo,
                               torch.from_numpy(ws).cuda() if window else None, window, k, idx,
                               sim)
    # without sim_out (the workspace holds the similarities)
    idx2 = torch.full_like(idx, -5)
    dkv.dllm_similarity_select(to_dev(cur, dt), to_dev(cached, dt), lo,
                               torch.from_numpy(ws).cuda() if window else None, window, k, idx2)
    torch.cuda.synchronize()
    ref_idx, ref_sim = oracle.similarity_select(cur, cached, lo, ws, window, k)
    got = sim.cpu().numpy()
    np.testing.assert_allclose(got[:, lo:], ref_sim[:, lo:], rtol=0, atol=1e-12)
    assert np.isnan(got[:, :lo]).all()                 # rows below lo are not written
    np.testing.assert_array_equal(idx.cpu().numpy(), ref_idx)
    np.testing.assert_array_equal(idx2.cpu().numpy(), ref_idx)


def test_similarity_select_ties_go_to_the_lower_row():
    B, S, H, lo, window, k = 2, 300, 128, 40, 10, 2
    rng = np.random.default_rng(5)
    cur, cached = _features(rng, B, S, H, "bf16")
    ws = np.array([100, 200], np.int32)
    _, sim = oracle.similarity_select(cur, cached, lo, ws, window, k)
    expect = []
    for b in range(B):
        win = set(range(ws[b], ws[b] + window))
        cand = [j for j in range(lo, S) if j not in win]
        j1 = min(cand, key=lambda j: sim[b, j])
        others = [j for j in (lo + 1, S - 1, (j1 + lo) // 2 + 1) if j != j1 and j not in win][:2]
        for j2 in others:                              # exact copies: equal cosines both sides
            cur[b, j2], cached[b, j2] = cur[b, j1], cached[b, j1]
        expect.append(sorted(win | set(sorted([j1] + others)[:k])))
    idx = torch.empty((B, window + k), dtype=torch.int32, device="cuda")
    dkv.dllm_similarity_select(to_dev(cur, BF), to_dev(cached, BF), lo,
                               torch.from_numpy(ws).cuda(), window, k, idx)
    torch.cuda.synchronize()
    ref_idx, _ = oracle.similarity_select(cur, cached, lo, ws, window, k)
    assert [list(r) for r in ref_idx] == expect
    np.testing.assert_array_equal(idx.cpu().numpy(), ref_idx)


SCHED_CASES = {
    "s1500_mixed_flags": (5, 1500, 40, 24, True),
    "s300_no_flags": (3, 300, 17, 0, False),
    "s32768_max": (2, 32768, 100, 64, True),
}


@pytest.mark.parametrize("name", list(SCHED_CASES))
def test_schedule_rows_and_copy_match_oracle(name):
    B, S, n, m, flags = SCHED_CASES[name]
    say(f"[schedule] {name}")
    rng = np.random.default_rng(len(name))
    idx = rng.integers(-3, S + 3, size=(B, n)).astype(np.int32)      # out-of-range: skipped
    tracked = rng.integers(-1, S, size=(B, m)).astype(np.int32) if m else None
    if m:
        tracked[:, 1::3] = tracked[:, ::3][:, :tracked[:, 1::3].shape[1]]   # duplicates
        tracked[:, -2:] = -1
    full_in = np.array([1, 0, 0, 0, 0][:B], np.uint8) if flags else None
    decision = np.array([0, 0, 1, 0, 1][:B], np.uint8) if flags else None
    cap = B * S
    rows = torch.full((cap,), -7, dtype=torch.int32, device="cuda")
    cu = torch.empty((B + 1,), dtype=torch.int32, device="cuda")
    full_out = torch.full((B,), 9, dtype=torch.uint8, device="cuda")
    dev = (lambda a: None if a is None else torch.from_numpy(a).cuda())
    dkv.dllm_schedule_rows(S, dev(idx), dev(tracked), dev(full_in), dev(decision), full_out,
                           rows, cu)
    torch.cuda.synchronize()
    ok_idx = np.where((idx >= 0) & (idx < S), idx, -1)
    full = None
    if flags:
        full = (full_in | decision).astype(bool)
    tr = np.concatenate([ok_idx, tracked], 1) if m else ok_idx
    ref_rows, ref_cu = oracle.schedule_rows(S, np.zeros((B, 0), np.int32), tr, full)
    got_cu = cu.cpu().numpy()
    np.testing.assert_array_equal(got_cu, ref_cu)
    got = rows.cpu().numpy()
    np.testing.assert_array_equal(got[:ref_cu[-1]], ref_rows)
    assert (got[ref_cu[-1]:] == -7).all()
    np.testing.assert_array_equal(full_out.cpu().numpy(),
                                  full.astype(np.uint8) if flags else np.zeros(B, np.uint8))
    # the feature copy of those rows
    H = 64
    src = torch.randn((B, S, H), device="cuda").to(BF)
    dst = torch.randn((B, S, H), device="cuda").to(BF)
    expect = dst.clone()
    for b in range(B):
        r = torch.from_numpy(ref_rows[ref_cu[b]:ref_cu[b + 1]]).long().cuda()
        expect[b, r] = src[b, r]
    dkv.dllm_copy_rows_varlen(src, dst, rows, cu)
    torch.cuda.synchronize()
    assert torch.equal(dst, expect)


def test_four_layer_schedule_stage_by_stage():
    L, triggers = 4, [1, 4, 2]
    wl = synth.custom(batch=3, hidden=256, q_heads=4, kv_heads=2, head_dim=128, seq=256,
                      prompt=128, seed=91, track_k=8)
    window, k_sel, k_track, gamma = 8, 24, wl.track_k, wl.gamma
    st = synth.layer_stack(wl, L, triggers, window)
    B, S, Hq, D, lo = wl.batch, wl.seq, wl.q_heads, wl.head_dim, wl.prompt
    scale = 1.0 / math.sqrt(D)
    cap = B * S
    rows0 = np.stack([np.arange(s, s + window) for s in st.window_start]).astype(np.int32)
    ws_d = torch.from_numpy(st.window_start).cuda()
    layers = []
    for l in range(L):
        say(f"[schedule] layer {l}: prefill and previous step")
        g = GpuLayer(wl, st.w[l], guard=0)
        hp = to_dev(st.hidden_prev[l], BF)
        g.prefill(hp)
        q0 = g.refresh(hp, rows0)
        _, _, mass0 = g.attention(q0, want_mass=True)
        T = torch.full((B, Hq, k_track), -1, dtype=torch.int32, device="cuda")
        buf = torch.zeros((B, Hq, k_track, 2, D), dtype=BF, device="cuda")
        sig = torch.empty((B, Hq), dtype=F32, device="cuda")
        dec = torch.empty((B,), dtype=torch.uint8, device="cuda")
        dkv.dllm_drift_check(g.cache, Hq, k_track, gamma, T, buf, mass0, sig, dec)
        layers.append(dict(g=g, feat=hp.clone(), T=T, buf=buf, hcur=to_dev(st.hidden_cur[l], BF)))
    full = torch.zeros((B,), dtype=torch.uint8, device="cuda")
    decision = torch.zeros((B,), dtype=torch.uint8, device="cuda")
    out_t = dict(step_rows=torch.empty((B, window + k_sel), dtype=torch.int32, device="cuda"),
                 rows=torch.empty((cap,), dtype=torch.int32, device="cuda"),
                 cu_rows=torch.empty((B + 1,), dtype=torch.int32, device="cuda"),
                 q=torch.empty((cap, Hq, D), dtype=BF, device="cuda"),
                 out=torch.empty((cap, Hq, D), dtype=BF, device="cuda"),
                 lse=torch.empty((cap * Hq,), dtype=F32, device="cuda"),
                 attn_mass=torch.empty((B, Hq, S), dtype=F32, device="cuda"),
                 sigma=torch.empty((B, Hq), dtype=F32, device="cuda"))
    decisions = []
    for l in range(L):
        say(f"[schedule] layer {l}: step")
        ly = layers[l]
        g = ly["g"]
        before = dict(feat=ly["feat"].float().cpu().numpy(), T=ly["T"].cpu().numpy(),
                      buf=ly["buf"].float().cpu().numpy().astype(np.float64),
                      full=full.cpu().numpy().copy(), dec=decision.cpu().numpy().copy(),
                      k=g.cache.k.clone(), v=g.cache.v.clone())
        dkv.dllm_elastic_layer_step(
            g.cache, hidden_cur=ly["hcur"], hidden_feat=ly["feat"], w_qkv=g.w,
            window_start=ws_d, track_idx=ly["T"], track_buf=ly["buf"], full=full,
            decision=decision, num_q_heads=Hq, lo=lo, window=window, k_select=k_sel,
            k_track=k_track, rope_base=wl.rope_base, softmax_scale=scale, gamma=gamma, **out_t)
        torch.cuda.synchronize()
        h_cur = st.hidden_cur[l]
        # 1. step rows from the features the GPU held before this layer
        R = out_t["step_rows"].cpu().numpy()
        ref_R, _ = oracle.similarity_select(h_cur, before["feat"], lo, st.window_start, window,
                                            k_sel)
        np.testing.assert_array_equal(R, ref_R)
        # 2. flags and the row schedule
        fl = (before["full"] | before["dec"]).astype(bool)
        np.testing.assert_array_equal(full.cpu().numpy(), fl.astype(np.uint8))
        rows, cu = out_t["rows"].cpu().numpy(), out_t["cu_rows"].cpu().numpy()
        ref_rows, ref_cu = oracle.schedule_rows(S, R, before["T"].reshape(B, -1), fl)
        np.testing.assert_array_equal(cu, ref_cu)
        np.testing.assert_array_equal(rows[:cu[-1]], ref_rows)
        # 3. cache rows: those of a full refresh of h_cur, bit for bit; the rest unchanged
        full_g = GpuLayer(wl, st.w[l], guard=0)
        full_g.prefill(ly["hcur"])
        torch.cuda.synchronize()
        cache_o = oracle.prefill(wl, h_cur, st.w[l])
        kg, vg = g.kv_host()
        for b in range(B):
            r = torch.from_numpy(rows[cu[b]:cu[b + 1]]).long().cuda()
            keep = torch.ones(S, dtype=torch.bool, device="cuda")
            keep[r] = False
            assert torch.equal(g.cache.k[b][:, r], full_g.cache.k[b][:, r])
            assert torch.equal(g.cache.v[b][:, r], full_g.cache.v[b][:, r])
            assert torch.equal(g.cache.k[b][:, keep], before["k"][b][:, keep])
            rn = rows[cu[b]:cu[b + 1]]
            assert slice_rel_err(kg[b][:, rn], cache_o.k[b][:, rn], (0,)) <= 1e-2
            assert slice_rel_err(vg[b][:, rn], cache_o.v[b][:, rn], (0,)) <= 1e-2
        # 4. attention of the refreshed rows' queries
        T_rows = int(cu[-1])
        qg = out_t["q"][:T_rows].float().cpu().numpy()
        o_ref, l_ref, m_ref = oracle.attention_varlen(qg, kg, vg, scale, cu, np.full(B, S), True)
        og = out_t["out"][:T_rows].float().cpu().numpy()
        for b in range(B):
            assert slice_rel_err(og[cu[b]:cu[b + 1]], o_ref[cu[b]:cu[b + 1]], (1,)) <= 2e-2
        np.testing.assert_allclose(out_t["lse"][:T_rows * Hq].cpu().numpy(), l_ref, rtol=0,
                                   atol=1e-2)
        mg = out_t["attn_mass"].cpu().numpy()
        assert slice_rel_err(mg, m_ref, (0, 1)) <= 2e-2
        # 5. drift test of the previous tracked rows against the cache now, tracking update
        s_ref, d_ref = oracle.drift(before["buf"], before["T"], kg, vg, gamma)
        np.testing.assert_allclose(out_t["sigma"].cpu().numpy(), s_ref, rtol=0, atol=2e-6)
        np.testing.assert_array_equal(decision.cpu().numpy(), d_ref)
        np.testing.assert_array_equal(ly["T"].cpu().numpy(), oracle.topk(mg, k_track))
        decisions.append(decision.cpu().numpy().copy())
        say(f"  rows per sequence {np.diff(cu).tolist()}, sigma min "
            f"{out_t['sigma'].cpu().numpy().min(axis=1).round(3).tolist()}, "
            f"decision {decisions[-1].tolist()}")
        # 6. feature rows
        fg = ly["feat"].float().cpu().numpy()
        for b in range(B):
            rn = rows[cu[b]:cu[b + 1]]
            keep = np.setdiff1d(np.arange(S), rn)
            np.testing.assert_array_equal(fg[b, rn], h_cur[b, rn])
            np.testing.assert_array_equal(fg[b, keep], before["feat"][b, keep])
    # the drift fires at the planted layers: sequence 0 at layer 1 (and after), 2 at 2, 1 never
    dec = np.stack(decisions)
    assert dec[0].tolist() == [0, 0, 0]
    assert dec[1].tolist() == [1, 0, 0] and dec[2].tolist()[2] == 1
    assert not dec[:, 1].any()
