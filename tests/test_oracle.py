"""Pins of the CPU oracle against what the pages and the mathematics fix (no GPU).

Each test checks the oracle against something other than itself: a library routine (torch's
fp64 scaled-dot-product attention, torch's bf16 / e4m3fn casts, numpy integer matmul, complex
multiplication), a closed form, an invariant, or brute force on tiny inputs.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
import synth

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def rng(seed=0):
    return np.random.default_rng(seed)


# ---------------------------------------------------------------- storage rounding ------

def test_bf16_matches_torch_cast_on_fp32_inputs():
    x = rng(1).standard_normal(200_000).astype(np.float32) * np.float32(3.0)
    x = np.concatenate([x, np.float32([1e-39, -3e-40, 3.3e38, 1.0, -0.0])])
    want = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    got = oracle.round_storage(x.astype(np.float64), "bf16")
    np.testing.assert_array_equal(got, want)


def test_bf16_ties_to_even_and_overflow():
    r = oracle.round_bf16_scalar
    assert r(1 + 2 ** -8) == 1.0                      # halfway, even neighbour is 1
    assert r(1 + 3 * 2 ** -8) == 1 + 2 ** -6          # halfway, even neighbour is up
    assert r(1 + 2 ** -8 + 2 ** -30) == 1 + 2 ** -7   # just above halfway rounds up
    assert r(2 ** -133) == 2 ** -133                  # smallest subnormal
    assert r(2 ** -134) == 0.0                        # tie with zero -> even (zero)
    assert math.isinf(r(2.0 ** 128 * (1 - 2 ** -9)))  # above max + half ulp -> inf
    assert r(-2.5) == -2.5


# ---------------------------------------------------------------- e4m3 codec ------------

def _gold_e4m3():
    with open(os.path.join(GOLD, "e4m3_ocp.json")) as f:
        return json.load(f)


def test_e4m3_decode_matches_spec_table():
    g = _gold_e4m3()
    for code, val in g["codes"].items():
        got = oracle.e4m3_decode([int(code, 16)])[0]
        assert got == val and math.copysign(1, got) == math.copysign(1, val), code
    for code in g["nan_codes"]:
        assert math.isnan(oracle.e4m3_decode([int(code, 16)])[0])


def test_e4m3_all_codes_match_torch_and_reencode():
    codes = np.arange(256, dtype=np.uint8)
    got = oracle.e4m3_decode(codes)
    want = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    np.testing.assert_array_equal(np.isnan(got), np.isnan(want))
    fin = ~np.isnan(got)
    np.testing.assert_array_equal(got[fin], want[fin])
    # every finite code re-encodes to itself (the two zeros keep their sign)
    np.testing.assert_array_equal(oracle.e4m3_encode(got[fin]), codes[fin])
    # positive codes are monotone in value
    pos = got[:0x7F]
    assert np.all(np.diff(pos) > 0)


def test_e4m3_encode_matches_torch_in_range():
    x = rng(2).uniform(-464, 464, 300_000).astype(np.float32)
    x = np.concatenate([x, rng(3).standard_normal(100_000).astype(np.float32) * 0.01])
    want = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = oracle.e4m3_encode(x.astype(np.float64))
    np.testing.assert_array_equal(got, want)


def test_e4m3_midpoints_ties_to_even_and_saturation():
    vals = oracle.e4m3_decode(np.arange(0, 0x7F, dtype=np.uint8))
    mids = (vals[:-1] + vals[1:]) / 2
    codes = oracle.e4m3_encode(mids)
    even = np.where(np.arange(0, 0x7E) % 2 == 0, np.arange(0, 0x7E), np.arange(1, 0x7F))
    np.testing.assert_array_equal(codes, even.astype(np.uint8))
    sat = oracle.e4m3_encode([449.0, 1e9, np.inf, -1e9, -np.inf, 464.0, 480.0])
    np.testing.assert_array_equal(sat, [0x7E, 0x7E, 0x7E, 0xFE, 0xFE, 0x7E, 0x7E])


def test_fp8_rows_scale_and_error_bound():
    x = rng(4).standard_normal((500, 128)) * rng(5).uniform(0.01, 10, (500, 1))
    x[7] = 0.0
    codes, scales, deq = oracle.fp8_quantize_rows(x)
    amax = np.abs(x).max(axis=1)
    want_scale = (amax.astype(np.float32) / np.float32(448.0)).astype(np.float32)
    want_scale[7] = 1.0
    np.testing.assert_array_equal(scales, want_scale)
    # the largest element of each non-zero row lands on +-448
    top = np.abs(oracle.e4m3_decode(codes)).max(axis=1)
    assert np.all(top[np.arange(500) != 7] == 448.0)
    assert np.all(codes[7] == 0)
    # |x - deq| <= half an e4m3 step: 2^-4 relative in the normal range, 2^-10 * scale below
    err = np.abs(deq - x)
    bound = np.maximum(np.abs(x) * 2.0 ** -4, scales[:, None].astype(np.float64) * 2.0 ** -10)
    assert np.all(err <= bound * (1 + 1e-9))


# ---------------------------------------------------------------- rotary embedding ------

def test_rope_position_zero_is_identity():
    x = rng(6).standard_normal((3, 2, 64))
    np.testing.assert_array_equal(oracle.rope(x, [0, 0, 0], 10000.0), x)


def test_rope_matches_complex_rotation():
    """Rotate-half RoPE equals multiplying z_i = x_i + i x_{i+D/2} by exp(i pos theta_i)."""
    D = 128
    x = rng(7).standard_normal((5, 3, D))
    pos = np.array([1, 17, 500, 2047, 4095], np.int32)
    got = oracle.rope(x, pos, 10000.0)
    theta = 10000.0 ** (-2.0 * np.arange(D // 2) / D)
    z = x[..., :D // 2] + 1j * x[..., D // 2:]
    zr = z * np.exp(1j * pos[:, None, None] * theta[None, None, :])
    want = np.concatenate([zr.real, zr.imag], axis=-1)
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-12)


def test_rope_unit_vectors_closed_form_and_pair_norms():
    D = 64
    pos = np.array([3], np.int32)
    for i in (0, 5, 31):
        e = np.zeros((1, 1, D))
        e[0, 0, i] = 1.0
        y = oracle.rope(e, pos, 10000.0)[0, 0]
        th = 10000.0 ** (-2.0 * i / D)
        assert y[i] == pytest.approx(math.cos(3 * th), abs=1e-15)
        assert y[i + D // 2] == pytest.approx(math.sin(3 * th), abs=1e-15)
    # component 0 turns by exactly pos radians
    e = np.zeros((1, 1, D)); e[0, 0, 0] = 1.0
    y = oracle.rope(e, np.array([1000], np.int32), 10000.0)[0, 0]
    assert y[0] == math.cos(1000.0) and y[D // 2] == math.sin(1000.0)
    x = rng(8).standard_normal((4, 2, D))
    y = oracle.rope(x, np.array([5, 99, 1234, 7], np.int32), 10000.0)
    n0 = x[..., :D // 2] ** 2 + x[..., D // 2:] ** 2
    n1 = y[..., :D // 2] ** 2 + y[..., D // 2:] ** 2
    np.testing.assert_allclose(n1, n0, rtol=1e-12)


def test_rope_scores_depend_on_relative_position_only():
    D = 128
    q = rng(9).standard_normal((1, 1, D))
    k = rng(10).standard_normal((1, 1, D))
    s = []
    for p, pk in ((10, 3), (107, 100), (2007, 2000)):
        qr = oracle.rope(q, np.array([p], np.int32), 10000.0)
        kr = oracle.rope(k, np.array([pk], np.int32), 10000.0)
        s.append(float((qr * kr).sum()))
    assert s[0] == pytest.approx(s[1], rel=1e-10) and s[0] == pytest.approx(s[2], rel=1e-10)


# ---------------------------------------------------------------- projection ------------

def test_linear_exact_on_small_integer_grid():
    r = rng(11)
    x = synth.small_integer_grid(r, (9, 256))
    w = synth.small_integer_grid(r, (40, 256))
    rows = np.array([3, 0, 39, 17, 17], np.int32)
    got = oracle.linear(x, w, rows)
    xi = (x * 16).astype(np.int64)
    wi = (w * 16).astype(np.int64)
    want = (xi @ wi[rows].T).astype(np.float64) / 256.0
    np.testing.assert_array_equal(got, want)


def test_qkv_head_layout_q_then_k_then_v():
    """With W = I (H = N) the projection returns the hidden dims of each head's slot."""
    wl = synth.custom(hidden=(4 + 2 * 2) * 16, q_heads=4, kv_heads=2, head_dim=16, seq=8,
                      prompt=4, act="f32", cache="f32")
    H = wl.hidden
    w = np.eye(H, dtype=np.float32)
    x = rng(12).standard_normal((3, H)).astype(np.float32)
    pos = np.zeros(3, np.int32)   # rotation at position 0 is the identity
    q = oracle.qkv_rows(x, pos, w, wl, "q")
    k = oracle.qkv_rows(x, pos, w, wl, "k")
    v = oracle.qkv_rows(x, pos, w, wl, "v")
    np.testing.assert_array_equal(q.reshape(3, -1), x[:, :64])
    np.testing.assert_array_equal(k.reshape(3, -1), x[:, 64:96])
    np.testing.assert_array_equal(v.reshape(3, -1), x[:, 96:128])
    k1 = oracle.qkv_rows(x, pos, w, wl, "k", heads=[1])
    np.testing.assert_array_equal(k1[:, 0], x[:, 80:96])


# ---------------------------------------------------------------- attention -------------

def _torch_sdpa(q, k, v, scale):
    """Library attention in fp64: q [B,n,Hq,D], k/v [B,Hkv,S,D] (KV head h // G)."""
    B, n, Hq, D = q.shape
    G = Hq // k.shape[1]
    qt = torch.from_numpy(q).permute(0, 2, 1, 3)                    # B Hq n D
    kt = torch.from_numpy(k).repeat_interleave(G, dim=1)
    vt = torch.from_numpy(v).repeat_interleave(G, dim=1)
    out = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, scale=scale)
    logits = (qt @ kt.transpose(-1, -2).contiguous()) * scale
    lse = torch.logsumexp(logits, dim=-1)
    mass = torch.softmax(logits, dim=-1).sum(dim=2)                 # B Hq S
    return out.permute(0, 2, 1, 3).numpy(), lse.numpy(), mass.numpy()


@pytest.mark.parametrize("B,n,Hq,Hkv,S,D", [(1, 3, 2, 2, 5, 4), (2, 4, 6, 2, 17, 8),
                                            (1, 1, 7, 1, 1, 4), (2, 5, 4, 4, 33, 16)])
def test_attention_matches_library_sdpa(B, n, Hq, Hkv, S, D):
    r = rng(13 + S)
    q = r.standard_normal((B, n, Hq, D))
    k = r.standard_normal((B, Hkv, S, D))
    v = r.standard_normal((B, Hkv, S, D))
    out, lse, mass = oracle.attention(q, k, v, 1 / math.sqrt(D), True, True)
    o2, l2, m2 = _torch_sdpa(q, k, v, 1 / math.sqrt(D))
    np.testing.assert_allclose(out, o2, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(lse, l2, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(mass, m2, rtol=1e-12, atol=1e-13)
    # every query's probabilities sum to one, so each head's mass sums to n
    np.testing.assert_allclose(mass.sum(-1), n, rtol=1e-12)


def test_attention_special_cases():
    r = rng(14)
    D = 8
    v = r.standard_normal((1, 1, 6, D))
    k = r.standard_normal((1, 1, 6, D))
    # one key: the output is that key's value row, lse is the single logit
    q = r.standard_normal((1, 2, 1, D))
    out, lse, _ = oracle.attention(q, k[:, :, :1], v[:, :, :1], 0.5)
    np.testing.assert_array_equal(out[0, :, 0], np.repeat(v[0, 0, :1], 2, axis=0))
    np.testing.assert_allclose(lse[0, 0], 0.5 * (q[0, :, 0] @ k[0, 0, 0]), rtol=1e-14)
    # zero query: uniform weights, the output is the mean of V and lse = log S
    out, lse, _ = oracle.attention(np.zeros((1, 1, 1, D)), k, v, 0.3)
    np.testing.assert_allclose(out[0, 0, 0], v[0, 0].mean(0), rtol=1e-13, atol=1e-15)
    assert lse[0, 0, 0] == pytest.approx(math.log(6), rel=1e-14)
    # one dominant logit selects its value row
    kd = np.zeros((1, 1, 6, D)); kd[0, 0, 4, 0] = 1.0
    qd = np.zeros((1, 1, 1, D)); qd[0, 0, 0, 0] = 200.0
    out, _, _ = oracle.attention(qd, kd, v, 1.0)
    np.testing.assert_allclose(out[0, 0, 0], v[0, 0, 4], rtol=1e-12, atol=1e-60)


def test_attention_split_merge_identity():
    """Online-softmax state merge (the FACache identity): partials over disjoint key sets,
    combined with their log-sum-exp, equal the unsplit result."""
    r = rng(15)
    q = r.standard_normal((1, 3, 2, 16))
    k = r.standard_normal((1, 2, 40, 16))
    v = r.standard_normal((1, 2, 40, 16))
    full, lse, _ = oracle.attention(q, k, v, 0.25)
    parts = [(0, 7), (7, 31), (31, 40)]
    outs, lses = [], []
    for a, b in parts:
        o, l, _ = oracle.attention(q, k[:, :, a:b], v[:, :, a:b], 0.25)
        outs.append(o)
        lses.append(l)
    L = np.stack(lses)                                  # P B H n
    m = L.max(0)
    wts = np.exp(L - m)                                 # P B H n
    merged = sum(w.transpose(0, 2, 1)[..., None] * o for w, o in zip(wts, outs))
    merged /= wts.sum(0).transpose(0, 2, 1)[..., None]
    np.testing.assert_allclose(merged, full, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(m + np.log(wts.sum(0)), lse, rtol=1e-13)


def test_attention_varlen_reduces_to_the_fixed_batch_and_ignores_keys_past_the_length():
    """Variable-length batches: equal row counts and full lengths give the fixed-batch
    attention (packed rows, lse and mass in the same layout); a sequence's keys at and past
    its length change nothing, and get no mass."""
    r = rng(18)
    B, n, Hq, Hkv, S, D = 3, 4, 4, 2, 21, 8
    q = r.standard_normal((B, n, Hq, D))
    k = r.standard_normal((B, Hkv, S, D))
    v = r.standard_normal((B, Hkv, S, D))
    cu = np.arange(B + 1) * n
    full, lse, mass = oracle.attention(q, k, v, 0.3, True, True)
    o2, l2, m2 = oracle.attention_varlen(q.reshape(B * n, Hq, D), k, v, 0.3, cu, [S] * B, True)
    np.testing.assert_array_equal(o2, full.reshape(B * n, Hq, D))
    np.testing.assert_array_equal(l2, lse.reshape(-1))
    np.testing.assert_array_equal(m2, mass)
    # uneven counts (one empty sequence) and lengths; keys past each length redrawn
    cu = np.array([0, 3, 3, 7])
    lens = [21, 9, 1]
    qp = r.standard_normal((7, Hq, D))
    o3, l3, m3 = oracle.attention_varlen(qp, k, v, 0.3, cu, lens, True)
    k2, v2 = k.copy(), v.copy()
    for b, L in enumerate(lens):
        k2[b, :, L:] = 50 * r.standard_normal(k2[b, :, L:].shape)
        v2[b, :, L:] = 50 * r.standard_normal(v2[b, :, L:].shape)
    o4, l4, m4 = oracle.attention_varlen(qp, k2, v2, 0.3, cu, lens, True)
    np.testing.assert_array_equal(o3, o4)
    np.testing.assert_array_equal(l3, l4)
    np.testing.assert_array_equal(m3, m4)
    assert not m3[1].any()                                   # no rows: no mass
    assert not m3[2, :, 1:].any() and np.allclose(m3[2, :, 0], 4)   # one key takes it all
    np.testing.assert_allclose(o3[3:7, :, :], np.repeat(v[2:3, :, 0], 2, axis=1)
                               .repeat(4, axis=0).reshape(4, Hq, D), rtol=1e-14)


@pytest.mark.parametrize("B,n,Hq,Hkv,S,D", [(1, 3, 2, 2, 9, 4), (2, 4, 6, 2, 33, 8)])
def test_attention_state_matches_library_softmax_on_the_kept_keys(B, n, Hq, Hkv, S, D):
    """FACache state over a key subset: o_tilde / l is the library attention over the kept
    keys only, and m + log l their log-sum-exp; m is the largest kept logit."""
    r = rng(16 + S)
    q = r.standard_normal((B, n, Hq, D))
    k = r.standard_normal((B, Hkv, S, D))
    v = r.standard_normal((B, Hkv, S, D))
    keep = r.random((B, S)) < 0.6
    keep[:, 0] = True
    m, ll, o = oracle.attention_state(q, k, v, 0.4, keep)
    G = Hq // Hkv
    for b in range(B):
        ks, vs = k[b:b + 1, :, keep[b]], v[b:b + 1, :, keep[b]]
        o2, l2, _ = _torch_sdpa(q[b:b + 1], ks, vs, 0.4)
        np.testing.assert_allclose(o[b] / ll[b].transpose(1, 0)[..., None], o2[0], rtol=1e-12,
                                   atol=1e-13)
        np.testing.assert_allclose(m[b] + np.log(ll[b]), l2[0], rtol=1e-12)
        logits = np.einsum("nhd,hsd->hns", q[b], np.repeat(ks[0], G, axis=0)) * 0.4
        np.testing.assert_allclose(m[b], logits.max(-1), rtol=1e-14)


def test_attention_state_of_a_partition_merges_to_full_attention():
    """The FACache identity on the state itself: the states over the invariant keys and over
    the block keys, merged with their maxima, reproduce full attention; all keys kept gives
    full attention directly; no key kept gives (-inf, 0, 0)."""
    r = rng(17)
    B, n, Hq, Hkv, S, D = 2, 5, 4, 2, 70, 16
    q = r.standard_normal((B, n, Hq, D))
    k = r.standard_normal((B, Hkv, S, D))
    v = r.standard_normal((B, Hkv, S, D))
    full, lse, _ = oracle.attention(q, k, v, 0.25)
    blk = np.zeros((B, S), bool)
    blk[0, 20:52] = True
    blk[1, 38:70] = True
    mu, lu, ou = oracle.attention_state(q, k, v, 0.25, ~blk)
    mg, lg, og = oracle.attention_state(q, k, v, 0.25, blk)
    mm = np.maximum(mu, mg)
    wu, wg = np.exp(mu - mm), np.exp(mg - mm)              # B Hq n
    den = (lu * wu + lg * wg).transpose(0, 2, 1)[..., None]
    merged = (ou * wu.transpose(0, 2, 1)[..., None] + og * wg.transpose(0, 2, 1)[..., None]) / den
    np.testing.assert_allclose(merged, full, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(mm + np.log(lu * wu + lg * wg), lse, rtol=1e-13)
    ma, la, oa = oracle.attention_state(q, k, v, 0.25, np.ones((B, S), bool))
    np.testing.assert_allclose(oa / la.transpose(0, 2, 1)[..., None], full, rtol=1e-12, atol=1e-14)
    m0, l0, o0 = oracle.attention_state(q, k, v, 0.25, np.zeros((B, S), bool))
    assert np.all(m0 == -np.inf) and not l0.any() and not o0.any()


# ---------------------------------------------------------------- top-k + drift ----------

def test_topk_brute_force_with_ties():
    r = rng(16)
    a = synth.uniform_mass(r, (6, 300), ties=40).astype(np.float64)
    a[0, :] = 0.5                                        # all tied: lowest indices win
    T = oracle.topk(a, 32)
    for p in range(6):
        order = sorted(range(300), key=lambda j: (-a[p, j], j))[:32]
        assert list(T[p]) == sorted(order)
    assert list(T[0]) == list(range(32))
    # fewer candidates than slots: all of them, then -1
    T2 = oracle.topk(a[:, :5], 8)
    assert list(T2[1]) == [0, 1, 2, 3, 4, -1, -1, -1]


def _drift_case(u_rows, w_rows, D):
    """One (b, h): tracking buffer rows u and cache rows w at positions 0..k-1."""
    k = len(u_rows)
    buf = np.zeros((1, 1, k, 2, D))
    kc = np.zeros((1, 1, k, D)); vc = np.zeros((1, 1, k, D))
    for t in range(k):
        buf[0, 0, t, 0], buf[0, 0, t, 1] = u_rows[t][:D], u_rows[t][D:]
        kc[0, 0, t], vc[0, 0, t] = w_rows[t][:D], w_rows[t][D:]
    T = np.arange(k, dtype=np.int32).reshape(1, 1, k)
    return buf, T, kc, vc


def test_drift_cosine_closed_forms():
    r = rng(17)
    D = 8
    u = [r.standard_normal(2 * D) for _ in range(3)]
    for w, want in ((u, 1.0), ([-x for x in u], -1.0), ([3.5 * x for x in u], 1.0)):
        s, ref = oracle.drift(*_drift_case(u, w, D), gamma=0.9)
        assert s[0, 0] == pytest.approx(want, abs=4e-16)
    # orthogonal
    e1 = np.zeros(2 * D); e1[0] = 1
    e2 = np.zeros(2 * D); e2[D + 1] = 2
    s, _ = oracle.drift(*_drift_case([e1], [e2], D), gamma=0.9)
    assert s[0, 0] == 0.0
    # rotation by angle t in one plane: cosine = cos t
    for t in (0.1, 0.45102681, 1.3):
        a = np.zeros(2 * D); a[2] = 1.0
        b = np.zeros(2 * D); b[2] = math.cos(t); b[D + 3] = math.sin(t)
        s, _ = oracle.drift(*_drift_case([a], [b], D), gamma=0.9)
        assert s[0, 0] == pytest.approx(math.cos(t), abs=1e-15)


def test_drift_decision_rules():
    D = 4
    # sigma exactly gamma does not refresh (strict <); just below does
    a = np.zeros(2 * D); a[0] = 1.0
    g = 0.75
    b = np.zeros(2 * D); b[0] = g; b[1] = math.sqrt(1 - g * g)
    s, ref = oracle.drift(*_drift_case([a], [b], D), gamma=g)
    assert s[0, 0] == g and ref[0] == 0
    s, ref = oracle.drift(*_drift_case([a], [b], D), gamma=np.nextafter(g, 1))
    assert ref[0] == 1
    # empty tracking set -> sigma 1; zero rows: equal -> 1, different -> 0
    buf, T, kc, vc = _drift_case([a], [b], D)
    s, ref = oracle.drift(buf, -np.ones_like(T), kc, vc, 0.9)
    assert s[0, 0] == 1.0 and ref[0] == 0
    z = np.zeros(2 * D)
    s, _ = oracle.drift(*_drift_case([z], [z], D), gamma=0.9)
    assert s[0, 0] == 1.0
    s, _ = oracle.drift(*_drift_case([z], [a], D), gamma=0.9)
    assert s[0, 0] == 0.0


def test_drift_min_over_heads_and_gqa_rows():
    """Two query heads share KV head 0; one drifts. The decision is the minimum."""
    D, S = 4, 6
    r = rng(18)
    kc = r.standard_normal((1, 1, S, D)); vc = r.standard_normal((1, 1, S, D))
    T = np.array([[[1, 4], [0, 5]]], np.int32)          # [B=1, Hq=2, k=2]
    buf = np.zeros((1, 2, 2, 2, D))
    for h in range(2):
        for t in range(2):
            buf[0, h, t, 0] = kc[0, 0, T[0, h, t]]
            buf[0, h, t, 1] = vc[0, 0, T[0, h, t]]
    buf[0, 1] *= -1.0                                   # head 1's saved rows point away
    s, ref = oracle.drift(buf, T, kc, vc, 0.9)
    assert s[0, 0] == pytest.approx(1.0, abs=1e-15) and s[0, 1] == pytest.approx(-1.0, abs=1e-15)
    assert ref[0] == 1


# ---------------------------------------------------------------- lossless memoisation --

@pytest.mark.parametrize("cache_dtype,act", [("f32", "f32"), ("bf16", "bf16"), ("fp8", "bf16")])
def test_cached_step_equals_full_recompute_bitwise(cache_dtype, act):
    """LaCache's lossless state memoisation: with unchanged inputs outside the refresh set,
    prefill(H_prev) + refresh(R) gives exactly prefill(H_cur), and so does attention."""
    wl = synth.custom(batch=2, hidden=128, q_heads=4, kv_heads=2, head_dim=16, seq=40, prompt=20,
                      act=act, cache=cache_dtype, refresh="window+subset", window=4, subset=6,
                      seed=21)
    inp = synth.make_inputs(wl)
    h_cur = inp.hidden_cur()
    assert not np.array_equal(h_cur, inp.hidden_prev)
    cached = oracle.refresh_rows(oracle.prefill(wl, inp.hidden_prev, inp.w), h_cur, inp.w, inp.idx)
    full = oracle.prefill(wl, h_cur, inp.w)
    for name in ("k", "v") + (("k_codes", "v_codes", "k_scale", "v_scale")
                              if cache_dtype == "fp8" else ()):
        np.testing.assert_array_equal(getattr(cached, name), getattr(full, name))
    q = oracle.queries(wl, h_cur, inp.w, inp.idx)
    o1, l1, m1 = oracle.attend(wl, q, cached, want_mass=True)
    o2, l2, m2 = oracle.attend(wl, q, full, want_mass=True)
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(m1, m2)


def test_refresh_leaves_other_rows_untouched():
    wl = synth.custom(batch=2, hidden=64, q_heads=2, kv_heads=2, head_dim=8, seq=24, prompt=12,
                      act="bf16", cache="bf16", block_start=13, block_len=5, seed=22)
    inp = synth.make_inputs(wl)
    before = oracle.prefill(wl, inp.hidden_prev, inp.w)
    after = oracle.refresh_rows(before.copy(), inp.hidden_cur(), inp.w, inp.idx)
    mask = np.ones(wl.seq, bool)
    mask[inp.idx[0]] = False
    np.testing.assert_array_equal(after.k[:, :, mask], before.k[:, :, mask])
    np.testing.assert_array_equal(after.v[:, :, mask], before.v[:, :, mask])
    assert not np.array_equal(after.k[:, :, ~mask], before.k[:, :, ~mask])


# ---------------------------------------------------------------- page constants --------

def test_workloads_use_the_pages_constants():
    with open(os.path.join(GOLD, "page_constants.json")) as f:
        g = json.load(f)
    for wl in synth.WORKLOADS.values():
        assert wl.gamma == g["drift_gamma"]["value"]
        assert wl.track_k == g["tracking_budget"]["value"]
    lo, hi = g["window_beta_range"]["value"]
    assert lo <= synth.WORKLOADS["c4"].window <= hi
    assert synth.WORKLOADS["c5"].head_dim == g["fp8_group"]["value"][1]


def test_drift_reads_the_query_heads_kv_group():
    """Hq=4 over Hkv=2: heads 0,1 read KV head 0 and heads 2,3 read KV head 1.  Buffers saved
    from the right group give sigma 1 on every head; a wrong head mapping would not."""
    D, S = 4, 5
    r = rng(19)
    kc = r.standard_normal((1, 2, S, D)); vc = r.standard_normal((1, 2, S, D))
    T = np.array([[[0, 3], [1, 2], [4, 0], [2, 3]]], np.int32)
    buf = np.zeros((1, 4, 2, 2, D))
    for h in range(4):
        for t in range(2):
            buf[0, h, t, 0] = kc[0, h // 2, T[0, h, t]]
            buf[0, h, t, 1] = vc[0, h // 2, T[0, h, t]]
    s, ref = oracle.drift(buf, T, kc, vc, 0.9)
    np.testing.assert_allclose(s, 1.0, atol=1e-15)
    assert ref[0] == 0
    # the tracking refill reads the same rows
    wl = synth.custom(batch=1, q_heads=4, kv_heads=2, head_dim=D, seq=S, act="f32", cache="f32")
    c = oracle.Cache(wl)
    c.k[:], c.v[:] = kc, vc
    mass = r.random((1, 4, S))
    T2, buf2 = oracle.track(c, mass, 2)
    for h in range(4):
        for t in range(2):
            np.testing.assert_array_equal(buf2[0, h, t, 0], kc[0, h // 2, T2[0, h, t]])


def test_step_uses_absolute_row_positions():
    """With every hidden row equal, the logit of query row p against key row j depends only
    on p - j, so the log-probability profiles of two queries are shifts of each other.
    Rotating by the slot index instead of the row position breaks this."""
    S = D = 16
    wl = synth.custom(batch=1, hidden=32, q_heads=1, kv_heads=1, head_dim=D, seq=S, prompt=4,
                      act="f32", cache="f32", block_start=5, block_len=2, seed=23)
    inp = synth.make_inputs(wl)
    x = np.tile(inp.hidden_prev[0, :1], (S, 1))[None]
    idx = np.array([[5, 9]], np.int32)
    cache = oracle.prefill(wl, x, inp.w)
    cache.v[:] = np.eye(S)[None, None]                  # out[i][j] = p_ij
    q = oracle.queries(wl, x, inp.w, idx)
    out, _, _ = oracle.attend(wl, q, cache)
    lp = np.log(out[0, :, 0])                           # [2, S]
    d = 9 - 5
    a = lp[0, 0:S - d] - lp[0, 0]
    b = lp[1, d:S] - lp[1, d]
    np.testing.assert_allclose(a, b, rtol=0, atol=2e-5)


# ---------------------------------------------------------------- similarity refresh ----

def test_feature_similarity_closed_forms():
    """Cosine of planted pairs: x = e1, y = cos(t) e1 + sin(t) e2 gives cos(t); scaling either
    row keeps it; the negation gives -1; zero rows follow the drift test's convention."""
    H = 6
    t = np.linspace(0.0, math.pi, 9)
    x = np.zeros((1, 9, H)); y = np.zeros((1, 9, H))
    x[0, :, 0] = 1.0
    y[0, :, 0], y[0, :, 1] = np.cos(t), np.sin(t)
    np.testing.assert_allclose(oracle.feature_similarity(x, y)[0], np.cos(t), atol=1e-15)
    np.testing.assert_allclose(oracle.feature_similarity(3.0 * x, 0.5 * y)[0], np.cos(t),
                               atol=1e-15)
    r = rng(40).standard_normal((2, 5, H))
    np.testing.assert_allclose(oracle.feature_similarity(r, -2.0 * r), -1.0, atol=1e-15)
    z = np.zeros((1, 3, H)); o = np.ones((1, 3, H))
    np.testing.assert_array_equal(oracle.feature_similarity(z, z), 1.0)
    np.testing.assert_array_equal(oracle.feature_similarity(z, o), 0.0)
    np.testing.assert_array_equal(oracle.feature_similarity(o, z), 0.0)
    # the inner product runs over the feature axis, row by row
    a = rng(41).standard_normal((2, 4, H)); bb = rng(42).standard_normal((2, 4, H))
    for b in range(2):
        for s in range(4):
            ref = a[b, s] @ bb[b, s] / (np.linalg.norm(a[b, s]) * np.linalg.norm(bb[b, s]))
            assert abs(oracle.feature_similarity(a, bb)[b, s] - ref) < 1e-14


def test_similarity_select_planted_angles_window_and_ties():
    """Planted angles: row j of the response turned by t_j; the k most-turned rows outside
    the window are chosen, the window always, ties go to the lower position; nothing below
    lo is ever chosen by similarity."""
    B, S, H, lo, window, k = 2, 24, 4, 8, 3, 5
    r = rng(43)
    t = np.zeros((B, S))
    t[:, lo:] = r.uniform(0, 3.0, size=(B, S - lo))
    t[:, :lo] = 3.1                                   # prompt rows moved most, yet not eligible
    t[1, lo:] = 1.0                                   # sequence 1: one clear top row, then
    t[1, 15] = 2.9                                    # a three-way tie that the cut splits
    t[1, 20] = t[1, 21] = t[1, 22] = 2.5
    x = np.zeros((B, S, H)); y = np.zeros((B, S, H))
    x[..., 0] = 1.0
    y[..., 0], y[..., 1] = np.cos(t), np.sin(t)
    ws = np.array([10, 10])
    idx, sim = oracle.similarity_select(x, y, lo, ws, window, k)
    idx3, _ = oracle.similarity_select(x, y, lo, ws, window, 3)
    assert list(idx3[1]) == [10, 11, 12, 15, 20, 21]
    for b in range(B):
        win = set(range(ws[b], ws[b] + window))
        cand = [j for j in range(lo, S) if j not in win]
        brute = sorted(cand, key=lambda j: (-t[b, j], j))[:k]
        assert list(idx[b]) == sorted(win | set(brute))
        chosen = [j for j in idx[b] if j not in win]
        rest = [j for j in cand if j not in chosen]
        assert max(sim[b, chosen]) <= min(sim[b, rest])


def test_schedule_rows_union_full_and_empty_slots():
    S = 30
    idx = np.array([[3, 7, 20], [5, 6, 7], [0, 29, 1]], np.int32)
    tracked = np.array([[7, 2, -1, 20, 25], [-1, -1, -1, -1, -1], [29, 29, 0, 15, 3]], np.int32)
    full = np.array([False, False, True])
    rows, cu = oracle.schedule_rows(S, idx, tracked, full)
    assert list(cu) == [0, 5, 8, 38]
    assert list(rows[0:5]) == [2, 3, 7, 20, 25]
    assert list(rows[5:8]) == [5, 6, 7]
    assert list(rows[8:]) == list(range(S))
    rows2, cu2 = oracle.schedule_rows(S, idx, None, None)
    assert list(cu2) == [0, 3, 6, 9] and list(rows2) == [3, 7, 20, 5, 6, 7, 0, 1, 29]


def _stack_case(layers=3, triggers=(1, 3), gamma=0.9):
    wl = synth.custom(batch=2, hidden=64, q_heads=2, kv_heads=1, head_dim=16, seq=40, prompt=16,
                      act="bf16", cache="bf16", seed=44, gamma=gamma, track_k=4)
    return wl, synth.layer_stack(wl, layers, list(triggers), window=4)


def test_layer_schedule_triggers_where_the_states_move_and_refreshes_deeper_layers():
    """Sequence 0's states move from layer 1 on, sequence 1's never (trigger = L): the drift
    test fires at layer 1 for sequence 0 only (the tracked rows were recomputed, so sigma
    measures the change: about 0.99 before, about 0 at the trigger), and layer 2 then
    recomputes every row of sequence 0, leaving exactly a full recompute from its states."""
    wl, st = _stack_case()
    L, B, S = 3, wl.batch, wl.seq
    rows0 = np.stack([np.arange(s, s + 4) for s in st.window_start])
    states = [oracle.schedule_prepare(wl, st.w[l], st.hidden_prev[l], rows0, wl.track_k)
              for l in range(L)]
    full = np.zeros(B, bool)
    recs = []
    for l in range(L):
        rec = oracle.schedule_layer(states[l], st.hidden_cur[l], full, wl.prompt, st.window_start,
                                    4, 6, wl.gamma)
        recs.append(rec)
        full = rec["full_next"]
    assert list(recs[0]["decision"]) == [0, 0]
    assert list(recs[1]["decision"])[0] == 1 and recs[1]["decision"][1] == 0
    assert recs[0]["sigma"].min() > 0.95 and recs[1]["sigma"][0].max() < 0.5
    assert list(recs[2]["cu"][1:2]) == [S]                     # sequence 0: every row
    full2 = oracle.prefill(wl, st.hidden_cur[2], st.w[2])
    np.testing.assert_array_equal(states[2].cache.k[0], full2.k[0])
    np.testing.assert_array_equal(states[2].cache.v[0], full2.v[0])
    np.testing.assert_array_equal(states[2].feat[0], st.hidden_cur[2][0])
    # sequence 1 at layer 2 refreshed its window, the chosen rows and its tracked rows only
    r1 = recs[2]["rows"][recs[2]["cu"][1]:]
    prev = oracle.prefill(wl, st.hidden_prev[2], st.w[2])
    other = np.setdiff1d(np.arange(S), r1)
    np.testing.assert_array_equal(states[2].cache.k[1][:, other], prev.k[1][:, other])
    np.testing.assert_array_equal(states[2].cache.k[1][:, r1], full2.k[1][:, r1])
    assert set(recs[2]["T_prev"][1].ravel()) <= set(r1)


def test_layer_schedule_threshold_extremes():
    """gamma below -1 never fires (no deeper full refresh); gamma above 1 fires at the first
    layer for every sequence, so every later layer recomputes all rows."""
    for gamma, expect in ((-2.0, 0), (2.0, 1)):
        wl, st = _stack_case(layers=2, triggers=(2, 2), gamma=gamma)
        rows0 = np.stack([np.arange(s, s + 4) for s in st.window_start])
        states = [oracle.schedule_prepare(wl, st.w[l], st.hidden_prev[l], rows0, wl.track_k)
                  for l in range(2)]
        full = np.zeros(wl.batch, bool)
        rec0 = oracle.schedule_layer(states[0], st.hidden_cur[0], full, wl.prompt,
                                     st.window_start, 4, 6, gamma)
        assert list(rec0["decision"]) == [expect] * wl.batch
        rec1 = oracle.schedule_layer(states[1], st.hidden_cur[1], rec0["full_next"], wl.prompt,
                                     st.window_start, 4, 6, gamma)
        sizes = np.diff(rec1["cu"])
        assert (sizes == wl.seq).all() == bool(expect)


# ---------------------------------------------------------------- per-group FP8 linear --

def test_fp8_group_codes_are_torch_casts_of_the_fp32_quotient():
    """Each code is the nearest-even e4m3 of the fp32 quotient x / scale (torch's
    float8_e4m3fn cast as the independent encoder); the group's largest magnitude maps to 448
    and a zero group keeps scale 1 with zero codes."""
    r = rng(60)
    x = synth.round_to_bf16(r.standard_normal((5, 512)).astype(np.float32) *
                            np.float32(3.0))
    x[2, 128:256] = 0.0
    codes, scales = oracle.fp8_quantize_groups(x)
    assert scales.shape == (5, 4) and scales.dtype == np.float32
    g = x.reshape(5, 4, 128)
    amax = np.abs(g).max(-1)
    np.testing.assert_array_equal(scales[amax > 0], (amax / np.float32(448))[amax > 0])
    assert scales[2, 1] == 1.0 and not codes[2, 128:256].any()
    q = torch.from_numpy(g / scales[..., None]).clamp(-448, 448)
    ref = q.to(torch.float8_e4m3fn).view(torch.uint8).numpy().reshape(5, 512)
    np.testing.assert_array_equal(codes, ref)
    dec = oracle.e4m3_decode(codes).reshape(5, 4, 128)
    big = np.abs(g).argmax(-1)
    for m in range(5):
        for kb in range(4):
            if amax[m, kb] > 0:
                assert abs(dec[m, kb, big[m, kb]]) == 448.0


def test_fp8_block_scales_sit_on_their_128x128_block():
    """A single large weight raises the scale of its own 128 x 128 block only (rows = output
    features, columns = input features; a transposed or mis-strided block map fails)."""
    r = rng(61)
    w = r.standard_normal((256, 384)).astype(np.float32) * np.float32(0.02)
    base_codes, base = oracle.fp8_quantize_blocks(w)
    w2 = w.copy()
    w2[130, 300] = 5.0                                  # block (1, 2)
    codes2, s2 = oracle.fp8_quantize_blocks(w2)
    changed = s2 != base
    assert changed.sum() == 1 and changed[1, 2]
    assert s2[1, 2] == np.float32(5.0) / np.float32(448)
    assert oracle.e4m3_decode(codes2[130:131, 300:301])[0, 0] == 448.0
    np.testing.assert_array_equal(codes2[:128], base_codes[:128])
    np.testing.assert_array_equal(codes2[128:, :256], base_codes[128:, :256])


def test_fp8_linear_is_an_integer_matmul_with_group_and_block_scales():
    """Codes of small integers with unit scales make the layer an exact integer matmul
    (numpy int64); doubling one activation group's scale adds exactly that group's share, and
    doubling one weight block's scale that block's share (scale placement, no transposition)."""
    r = rng(62)
    M, N, K = 3, 256, 384
    xi = r.integers(-8, 9, size=(M, K))
    wi = r.integers(-8, 9, size=(N, K))
    xc = oracle.e4m3_encode(xi.astype(np.float64))
    wc = oracle.e4m3_encode(wi.astype(np.float64))
    sx = np.ones((M, K // 128), np.float32)
    sw = np.ones((N // 128, K // 128), np.float32)
    y = oracle.fp8_linear(xc, sx, wc, sw)
    np.testing.assert_array_equal(y, (xi @ wi.T).astype(np.float64))
    sx2 = sx.copy(); sx2[1, 2] = 2.0
    part = xi[1, 256:384] @ wi[:, 256:384].T
    d = oracle.fp8_linear(xc, sx2, wc, sw) - y
    np.testing.assert_array_equal(d[1], part)
    assert not d[[0, 2]].any()
    sw2 = sw.copy(); sw2[1, 0] = 2.0
    d2 = oracle.fp8_linear(xc, sx, wc, sw2) - y
    np.testing.assert_array_equal(d2[:, 128:256], xi[:, :128] @ wi[128:256, :128].T)
    assert not d2[:, :128].any()
