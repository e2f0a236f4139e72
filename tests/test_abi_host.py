"""The C-ABI library loads, exports every symbol its header declares, and rejects bad
arguments on the host (no kernel is launched by any call here)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dllm_cache.h")

dkv = pytest.importorskip("diffusion_kv_cache_amd")


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"DLLM_API\s+[\w\s\*]*?\b(dllm_\w+)\s*\(", text)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for want in ("dllm_cache_bytes", "dllm_cache_alloc", "dllm_refresh_qkv_rope_scatter",
                 "dllm_attention_workspace_bytes", "dllm_block_attention", "dllm_drift_check",
                 "dllm_last_error"):
        assert want in names
    assert set(names) == set(dkv.EXPORTS)


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(dkv.LIB_PATH)
    for name in declared_functions():
        assert hasattr(lib, name), name


def _desc(B=1, Hkv=4, S=128, D=64, dt=dkv.DLLM_BF16, group=0):
    return dkv.CacheDesc(B, Hkv, S, D, dt, group)


def test_cache_bytes_layout():
    d = _desc(B=2, Hkv=3, S=100, D=128, dt=dkv.DLLM_BF16)
    kv = 2 * 3 * 100 * 128 * 2
    assert dkv.dllm_cache_bytes(d) == 2 * ((kv + 255) // 256 * 256)
    d8 = _desc(B=2, Hkv=3, S=100, D=128, dt=dkv.DLLM_FP8_E4M3, group=128)
    kv8 = (2 * 3 * 100 * 128 + 255) // 256 * 256
    sc = (2 * 3 * 100 * 4 + 255) // 256 * 256
    assert dkv.dllm_cache_bytes(d8) == 2 * kv8 + 2 * sc
    assert dkv.dllm_cache_bytes(_desc(D=96)) == 0


def _alloc(d, base, nbytes):
    c = dkv.CCache()
    st = dkv.lib.dllm_cache_alloc(ctypes.byref(d), ctypes.c_void_p(base), nbytes, ctypes.byref(c))
    return st, c


def test_cache_alloc_carves_regions_without_touching_memory():
    d = _desc(B=2, Hkv=2, S=64, D=128, dt=dkv.DLLM_FP8_E4M3, group=128)
    need = dkv.dllm_cache_bytes(d)
    base = 1 << 40                                   # never dereferenced
    st, c = _alloc(d, base, need)
    assert st == dkv.DLLM_OK
    assert c.k == base and c.v == base + 2 * 2 * 64 * 128
    assert c.k_scale == c.v + 2 * 2 * 64 * 128 and c.v_scale == c.k_scale + 1024
    st, _ = _alloc(d, base, need - 1)
    assert st == dkv.DLLM_ESIZE and "needs" in dkv.dllm_last_error()
    st, _ = _alloc(d, base + 16, need)
    assert st == dkv.DLLM_EINVAL
    st, _ = _alloc(_desc(D=128, dt=dkv.DLLM_FP8_E4M3, group=64), base, 1 << 30)
    assert st == dkv.DLLM_EUNSUPPORTED
    st, _ = _alloc(_desc(B=0), base, 1 << 30)
    assert st == dkv.DLLM_EINVAL
    st, _ = _alloc(_desc(D=80), base, 1 << 30)
    assert st == dkv.DLLM_EUNSUPPORTED


def _fake_cache(dt=dkv.DLLM_BF16, D=128, Hkv=4, S=64):
    d = _desc(B=2, Hkv=Hkv, S=S, D=D, dt=dt, group=D if dt == dkv.DLLM_FP8_E4M3 else 0)
    st, c = _alloc(d, 1 << 40, dkv.dllm_cache_bytes(d))
    assert st == 0
    return c


P = ctypes.c_void_p
ADDR = P(1 << 41)


def _refresh(c, H=256, act=dkv.DLLM_BF16, n=4, hq=4, base=10000.0, hidden=ADDR, q_out=ADDR,
             ws=ADDR, ws_bytes=1 << 30):
    return dkv.lib.dllm_refresh_qkv_rope_scatter(ctypes.byref(c), hidden, H, act, ADDR, n, ADDR,
                                                 hq, base, q_out, ws, ws_bytes, None)


def test_refresh_rejects_bad_arguments_on_host():
    c = _fake_cache()
    assert _refresh(c, H=200) == dkv.DLLM_EUNSUPPORTED             # H % 256
    assert _refresh(c, hq=6) == dkv.DLLM_EINVAL                    # Hq % Hkv
    assert _refresh(c, n=65) == dkv.DLLM_EINVAL                    # n > S
    assert _refresh(c, n=-1) == dkv.DLLM_EINVAL
    assert _refresh(c, act=dkv.DLLM_F32) == dkv.DLLM_EUNSUPPORTED  # fp32 act, bf16 cache
    assert _refresh(c, act=7) == dkv.DLLM_EINVAL
    assert _refresh(c, base=0.0) == dkv.DLLM_EINVAL
    assert _refresh(c, hidden=None) == dkv.DLLM_EINVAL
    assert _refresh(c, q_out=P((1 << 41) + 8)) == dkv.DLLM_EINVAL  # misaligned
    assert _refresh(c, n=0) == dkv.DLLM_OK                         # nothing to do, no launch
    assert dkv.lib.dllm_refresh_qkv_rope_scatter(None, ADDR, 256, 1, ADDR, 4, ADDR, 4, 1e4, ADDR,
                                                 None, 0, None) == dkv.DLLM_EINVAL
    # small bf16 steps split K over workgroups and need 4 fp32 partials per output
    L = dkv.lib
    need = L.dllm_refresh_workspace_bytes(ctypes.byref(c.desc), 256, dkv.DLLM_BF16, 4, 4)
    assert need == 4 * (2 * 4) * ((4 + 2 * 4) * 128) * 4
    assert _refresh(c, ws_bytes=need - 1) == dkv.DLLM_ESIZE
    assert _refresh(c, ws=None, ws_bytes=need) == dkv.DLLM_EINVAL
    # large steps and fp32 run as one fused kernel: no workspace
    assert L.dllm_refresh_workspace_bytes(ctypes.byref(c.desc), 256, dkv.DLLM_BF16, 64, 4) == 0
    assert L.dllm_refresh_workspace_bytes(ctypes.byref(c.desc), 256, dkv.DLLM_F32, 4, 4) == 0
    assert L.dllm_refresh_workspace_bytes(ctypes.byref(c.desc), 256, dkv.DLLM_BF16, 4, 5) == 0


def test_attention_and_drift_reject_bad_arguments_on_host():
    c = _fake_cache()
    L = dkv.lib
    need = L.dllm_attention_workspace_bytes(ctypes.byref(c.desc), 4, 8)
    assert need > 0
    att = lambda **kw: L.dllm_block_attention(
        ctypes.byref(c), kw.get("q", ADDR), kw.get("act", 1), kw.get("hq", 4), kw.get("n", 8),
        kw.get("scale", 0.088), ADDR, None, None, ADDR, kw.get("ws", need), None)
    assert att(ws=need - 1) == dkv.DLLM_ESIZE
    assert att(hq=5) == dkv.DLLM_EINVAL
    assert att(scale=0.0) == dkv.DLLM_EINVAL
    assert att(act=dkv.DLLM_F32) == dkv.DLLM_EUNSUPPORTED
    assert att(q=None) == dkv.DLLM_EINVAL
    assert att(n=0) == dkv.DLLM_OK
    dr = lambda cc, **kw: L.dllm_drift_check(ctypes.byref(cc), kw.get("hq", 4), kw.get("k", 32),
                                             0.9, ADDR, ADDR, None, ADDR, ADDR, kw.get("w"),
                                             kw.get("wb", 0), None)
    assert dr(c, k=0) == dkv.DLLM_EINVAL and dr(c, k=65) == dkv.DLLM_EINVAL
    assert dr(c, hq=3) == dkv.DLLM_EINVAL
    # FP8 caches are tracked too: the buffer holds the codes, then one fp32 scale per row
    f8 = _fake_cache(dt=dkv.DLLM_FP8_E4M3)
    assert dr(f8, k=0) == dkv.DLLM_EINVAL
    for dt, per in ((dkv.DLLM_F32, 64 * 4), (dkv.DLLM_BF16, 64 * 2), (dkv.DLLM_FP8_E4M3, 64 + 4)):
        dd = _desc(B=3, D=64, dt=dt, group=64 if dt == dkv.DLLM_FP8_E4M3 else 0)
        assert L.dllm_track_buffer_bytes(ctypes.byref(dd), 5, 7) == 3 * 5 * 7 * 2 * per
    assert L.dllm_track_buffer_bytes(ctypes.byref(_desc()), 0, 7) == 0
    # the decision's workspace: one 128-byte line per sequence, 8-byte aligned
    dws = L.dllm_drift_workspace_bytes(c.desc.batch)
    assert dws == 128 * c.desc.batch and L.dllm_drift_workspace_bytes(0) == 0
    assert dr(c, k=0, w=ADDR, wb=dws) == dkv.DLLM_EINVAL
    assert dr(c, w=ADDR, wb=dws - 1) == dkv.DLLM_ESIZE
    assert dr(c, w=P((1 << 41) + 4), wb=dws) == dkv.DLLM_EINVAL
    # the allocation-free call validates the same way, and refuses shapes beyond its scratch
    na = lambda cc, **kw: L.dllm_block_attention_noalloc(
        ctypes.byref(cc), kw.get("q", ADDR), 1, kw.get("hq", 4), kw.get("n", 8), 0.088, ADDR,
        None, None, None)
    assert na(c, hq=5) == dkv.DLLM_EINVAL and na(c, q=None) == dkv.DLLM_EINVAL
    assert na(c, n=0) == dkv.DLLM_OK
    big = _fake_cache(S=65536, Hkv=1)
    assert L.dllm_attention_workspace_bytes(ctypes.byref(big.desc), 8, 1024) > \
        dkv.DLLM_NOALLOC_SCRATCH_BYTES
    assert na(big, hq=8, n=1024) == dkv.DLLM_ESIZE and "scratch" in dkv.dllm_last_error()
    assert L.dllm_fp8_e4m3_roundtrip(ADDR, 10, ctypes.c_float(0.0), ADDR, None, None) == dkv.DLLM_EINVAL
    assert L.dllm_fp8_e4m3_roundtrip(ADDR, 0, ctypes.c_float(1.0), ADDR, None, None) == dkv.DLLM_OK


def test_options_switch_round_trips():
    """dllm_set_options replaces the process-wide switches and returns the previous value;
    unknown bits are dropped."""
    prev = dkv.dllm_set_options(dkv.DLLM_OPT_DEBUG | 0x100)
    try:
        assert dkv.dllm_set_options(dkv.DLLM_OPT_WIDE_OFFSETS) == dkv.DLLM_OPT_DEBUG
        assert dkv.dllm_set_options(0) == dkv.DLLM_OPT_WIDE_OFFSETS
    finally:
        dkv.dllm_set_options(prev)


def test_schedule_calls_reject_bad_arguments_on_host():
    lib = dkv.lib
    F = ctypes.c_void_p(1 << 40)                     # never dereferenced
    EINVAL, ESIZE, EUNS = dkv.DLLM_EINVAL, dkv.DLLM_ESIZE, dkv.DLLM_EUNSUPPORTED
    sel = lib.dllm_similarity_select
    # B, S, H, act, cur, cached, lo, window_start, window, k, idx_out, sim_out, ws, ws_bytes, s
    assert sel(2, 9000, 64, dkv.DLLM_BF16, F, F, 0, F, 4, 4, F, F, F, 1 << 30, None) == EUNS
    assert sel(2, 100, 60, dkv.DLLM_BF16, F, F, 0, F, 4, 4, F, F, F, 1 << 30, None) == EINVAL
    assert sel(2, 100, 64, dkv.DLLM_BF16, F, F, 50, F, 20, 31, F, F, F, 1 << 30, None) == EINVAL
    assert sel(2, 100, 64, dkv.DLLM_BF16, F, F, 100, F, 0, 0, F, F, F, 1 << 30, None) == EINVAL
    assert sel(2, 100, 64, dkv.DLLM_BF16, F, F, 0, None, 4, 4, F, F, F, 1 << 30, None) == EINVAL
    assert sel(2, 100, 64, dkv.DLLM_BF16, F, F, 0, F, 4, 4, F, None, F, 100, None) == ESIZE
    assert sel(2, 100, 64, dkv.DLLM_BF16, F, F, 0, F, 0, 0, F, None, None, 0, None) == dkv.DLLM_OK
    assert lib.dllm_similarity_select_workspace_bytes(2, 100) == 2 * 100 * 8
    sch = lib.dllm_schedule_rows
    need = lib.dllm_schedule_rows_workspace_bytes(3, 50)
    assert need >= 3 * 50 * 4 + 3 * 4
    # B, S, idx, n, tracked, m, full_in, decision, full_out, rows, cap, cu, ws, ws_bytes, s
    assert sch(3, 50, F, 4, F, 8, F, F, F, F, 149, F, F, need, None) == ESIZE
    assert sch(3, 50, F, 4, F, 8, F, F, F, F, 150, F, F, need - 1, None) == ESIZE
    assert sch(3, 50, None, 4, F, 8, F, F, F, F, 150, F, F, need, None) == EINVAL
    assert sch(3, 50, F, 4, None, 8, F, F, F, F, 150, F, F, need, None) == EINVAL
    assert sch(3, 40000, F, 4, F, 8, F, F, F, F, 3 * 40000, F, F, 1 << 30, None) == EUNS
    assert sch(3, 50, F, 4, F, 8, F, F, F, F, 150, F, ctypes.c_void_p((1 << 40) + 8), need,
               None) == EINVAL                       # workspace not 256-byte aligned
    cp = lib.dllm_copy_rows_varlen
    assert cp(2, 10, 24, F, F, F, F, 20, None) == EINVAL
    assert cp(2, 10, 32, None, F, F, F, 20, None) == EINVAL
    assert cp(2, 10, 32, F, F, F, F, 0, None) == dkv.DLLM_OK


def test_probes_reject_bad_arguments_on_host():
    lib = dkv.lib
    F = ctypes.c_void_p(1 << 40)                     # never dereferenced
    EINVAL = dkv.DLLM_EINVAL
    rd = lib.dllm_read_rate_probe
    # buf, bytes, workgroups, out, stream
    assert rd(F, 15, 4, F, None) == EINVAL                      # not a multiple of 16
    assert rd(F, -16, 4, F, None) == EINVAL
    assert rd(None, 16, 4, F, None) == EINVAL
    assert rd(ctypes.c_void_p((1 << 40) + 8), 16, 4, F, None) == EINVAL   # misaligned
    assert rd(F, 16, 0, F, None) == EINVAL
    assert rd(F, 16, 4, None, None) == EINVAL
    mp = lib.dllm_mfma_rate_probe
    assert mp(dkv.DLLM_F32, 16, 4, 4, F, None) == EINVAL
    assert mp(dkv.DLLM_BF16, 8, 4, 4, F, None) == EINVAL
    assert mp(dkv.DLLM_BF16, 16, 0, 4, F, None) == EINVAL
    assert mp(dkv.DLLM_BF16, 16, 4, 4, None, None) == EINVAL
