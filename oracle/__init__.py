"""CPU oracle for the per-layer cached denoising step (plain C in fp64, ctypes binding).

TEST INFRASTRUCTURE.  Only ``tests/``, the smoke check in ``__graft_entry__`` and the
benchmark's ``cpu_baseline`` leg import this package.  It shares no code with the HIP library
(``diffusion_kv_cache_amd``) and neither side imports the other; the only common module is the
seeded input generator ``synth``.

The low-level routines live in ``oracle.c`` (each cites the passage it follows).  This module
composes them into the step the pages describe:

* O1/O2  project the refreshed hidden rows and rotate q and k (``qkv_rows``);
* O3     prefill: fill every cache row from the previous hidden states (``prefill``);
* O4     cached step: recompute only the refresh rows from the current hidden states and
         overwrite those cache rows, leaving every other row as it was (``cached_step``)
         -- LaCache's lossless state memoisation: reusing rows whose inputs did not change
         gives exactly the full recompute (LaCache Technical Summary, Methodology 1);
* O5/O6  attention of the refreshed rows' queries over the whole cache, log-sum-exp and the
         column attention mass (``attention``);
* O8-O10 top-k tracking set, drift test and tracking-buffer refill (``drift``, ``topk``,
         ``track``), after Elastic-Cache's core idea;
* O11-O14 the partial refresh chosen by feature similarity (dLLM-Cache abstract) and one layer
         of the Elastic-Cache layer schedule (``feature_similarity``, ``similarity_select``,
         ``schedule_rows``, ``schedule_layer``).

"Storage" rounding: the cache holds K/V in its own dtype (fp32, bf16, or e4m3 codes with one
fp32 scale per 128-value row) and Q is handed to attention in the activation dtype.  The oracle
computes in fp64 and rounds exactly where the method stores a value.
"""
from __future__ import annotations

import ctypes
import math
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

ROUND_MODE = {"f64": 0, "f32": 1, "bf16": 2}


def build(force: bool = False) -> str:
    """Compile oracle.c with the host C compiler (no HIP headers, no fused multiply-add)."""
    if force or not os.path.exists(_LIB_PATH) or \
            os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        tmp = _LIB_PATH + ".tmp"
        subprocess.check_call(["gcc", "-std=c11", "-O2", "-ffp-contract=off", "-fno-fast-math",
                               "-fopenmp", "-fPIC", "-shared", _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is None:
        build()
        lib = ctypes.CDLL(_LIB_PATH)
        P = ctypes.c_void_p
        i64, i32, f64 = ctypes.c_int64, ctypes.c_int, ctypes.c_double
        lib.orc_round_bf16.restype = f64
        lib.orc_round_bf16.argtypes = [f64]
        lib.orc_round.argtypes = [P, i64, i32]
        lib.orc_e4m3_decode.restype = f64
        lib.orc_e4m3_decode.argtypes = [ctypes.c_uint8]
        lib.orc_e4m3_encode.restype = ctypes.c_uint8
        lib.orc_e4m3_encode.argtypes = [f64]
        lib.orc_e4m3_encode_array.argtypes = [P, i64, P]
        lib.orc_e4m3_decode_array.argtypes = [P, i64, P]
        lib.orc_fp8_quantize_rows.argtypes = [P, i64, i32, P, P, P]
        lib.orc_linear.argtypes = [P, i64, i64, P, P, i64, P]
        lib.orc_rope_rows.argtypes = [P, i64, i32, i32, P, f64]
        lib.orc_attention.argtypes = [P, P, P, i32, i32, i32, i32, i32, i32, f64, P, P, P]
        lib.orc_attention_state.argtypes = [P, P, P, P, i32, i32, i32, i32, i32, i32, f64, P, P,
                                            P]
        lib.orc_topk.argtypes = [P, i64, i32, i32, P]
        lib.orc_drift.argtypes = [P, P, P, P, i32, i32, i32, i32, i32, i32, f64, P, P]
        _lib = lib
    return _lib


def _p(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p) if a is not None else None


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


# ------------------------------------------------------------------------------------------
# Low-level routines
# ------------------------------------------------------------------------------------------

def round_bf16_scalar(x: float) -> float:
    return _load().orc_round_bf16(float(x))


def round_storage(x: np.ndarray, mode: str) -> np.ndarray:
    """Copy of x (float64) rounded to fp32 / bf16 (round to nearest even)."""
    y = _c(x, np.float64).copy()
    _load().orc_round(_p(y), y.size, ROUND_MODE[mode])
    return y


def e4m3_encode(x) -> np.ndarray:
    x = _c(x, np.float64)
    out = np.empty(x.shape, np.uint8)
    _load().orc_e4m3_encode_array(_p(x), x.size, _p(out))
    return out


def e4m3_decode(codes) -> np.ndarray:
    c = _c(codes, np.uint8)
    out = np.empty(c.shape, np.float64)
    _load().orc_e4m3_decode_array(_p(c), c.size, _p(out))
    return out


def fp8_quantize_rows(x: np.ndarray):
    """x: [..., G] float64 -> (codes uint8 [..., G], scales float32 [...], dequant float64)."""
    x = _c(x, np.float64)
    G = x.shape[-1]
    rows = x.size // G
    codes = np.empty(x.shape, np.uint8)
    scales = np.empty(x.shape[:-1], np.float32)
    deq = np.empty(x.shape, np.float64)
    _load().orc_fp8_quantize_rows(_p(x), rows, G, _p(codes), _p(scales), _p(deq))
    return codes, scales, deq


def linear(x: np.ndarray, w: np.ndarray, wrows) -> np.ndarray:
    """y[r, j] = sum_k x[r, k] w[wrows[j], k] (fp64, ascending k)."""
    x = _c(x, np.float32)
    w = _c(w, np.float32)
    wrows = _c(wrows, np.int32)
    R, H = x.shape
    assert w.shape[1] == H and (wrows.size == 0 or (wrows.min() >= 0 and wrows.max() < w.shape[0]))
    y = np.empty((R, wrows.size), np.float64)
    _load().orc_linear(_p(x), R, H, _p(w), _p(wrows), wrows.size, _p(y))
    return y


def rope(x: np.ndarray, pos, base: float) -> np.ndarray:
    """Rotate-half rotary embedding of x: [R, nh, D] at positions pos: [R] (returns a copy)."""
    y = _c(x, np.float64).copy()
    pos = _c(pos, np.int32)
    R, nh, D = y.shape
    assert pos.shape == (R,) and D % 2 == 0
    _load().orc_rope_rows(_p(y), R, nh, D, _p(pos), float(base))
    return y


def attention(q, k, v, scale: float, want_lse=True, want_mass=False):
    """q: [B, n, Hq, D]; k, v: [B, Hkv, S, D] -> (out [B,n,Hq,D], lse [B,Hq,n], mass [B,Hq,S])."""
    q = _c(q, np.float64)
    k = _c(k, np.float64)
    v = _c(v, np.float64)
    B, n, Hq, D = q.shape
    _, Hkv, S, _ = k.shape
    assert k.shape == v.shape == (B, Hkv, S, D) and Hq % Hkv == 0 and S >= 1
    out = np.empty_like(q)
    lse = np.empty((B, Hq, n), np.float64) if want_lse else None
    mass = np.empty((B, Hq, S), np.float64) if want_mass else None
    _load().orc_attention(_p(q), _p(k), _p(v), B, n, Hq, Hkv, S, D, float(scale), _p(out),
                          _p(lse), _p(mass))
    return out, lse, mass


def attention_varlen(q, k, v, scale: float, cu, lens, want_mass=False):
    """Attention of a variable-length batch (Elastic-Cache card, deployment notes: variable-
    length sequences concatenated): q [T, Hq, D] packed rows, rows cu[b] .. cu[b+1] belonging
    to sequence b, which attends to the first lens[b] rows of k[b], v[b] ([B, Hkv, S, D]).
    Returns out [T, Hq, D], lse [T * Hq] (sequence b's block at cu[b] * Hq laid out [Hq][rows])
    and mass [B, Hq, S] (0 at and past lens[b])."""
    q = _c(q, np.float64)
    B, Hkv, S, D = k.shape
    T, Hq, _ = q.shape
    out = np.zeros((T, Hq, D))
    lse = np.zeros(T * Hq)
    mass = np.zeros((B, Hq, S)) if want_mass else None
    for b in range(B):
        r0, r1, L = int(cu[b]), int(cu[b + 1]), int(lens[b])
        if r1 == r0:
            continue
        o, ls, m = attention(q[None, r0:r1], k[b:b + 1, :, :L], v[b:b + 1, :, :L], scale, True,
                             want_mass)
        out[r0:r1] = o[0]
        lse[r0 * Hq:r1 * Hq] = ls[0].reshape(-1)
        if want_mass:
            mass[b, :, :L] = m[0]
    return out, lse, mass


def attention_state(q, k, v, scale: float, keep):
    """Online-softmax state over the keys kept by keep [B, S] (bool): q [B, n, Hq, D], k, v
    [B, Hkv, S, D] -> (m [B, Hq, n], l [B, Hq, n], o_tilde [B, n, Hq, D]), natural log."""
    q = _c(q, np.float64)
    k = _c(k, np.float64)
    v = _c(v, np.float64)
    B, n, Hq, D = q.shape
    _, Hkv, S, _ = k.shape
    keep = _c(np.asarray(keep, dtype=bool).astype(np.uint8), np.uint8)
    assert keep.shape == (B, S) and k.shape == v.shape == (B, Hkv, S, D) and Hq % Hkv == 0
    m = np.empty((B, Hq, n), np.float64)
    ll = np.empty((B, Hq, n), np.float64)
    o = np.empty_like(q)
    _load().orc_attention_state(_p(q), _p(k), _p(v), _p(keep), B, n, Hq, Hkv, S, D, float(scale),
                                _p(m), _p(ll), _p(o))
    return m, ll, o


def topk(a: np.ndarray, k: int) -> np.ndarray:
    """a: [..., S] -> [..., k] int32: the k largest by (value desc, index asc), index-sorted."""
    a = _c(a, np.float64)
    S = a.shape[-1]
    P = a.size // S if S else 0
    T = np.empty(a.shape[:-1] + (k,), np.int32)
    _load().orc_topk(_p(a), P, S, k, _p(T))
    return T


def drift(buf, T, kc, vc, gamma: float):
    """buf: [B,Hq,k,2,D], T: [B,Hq,k], kc/vc: [B,Hkv,S,D] -> (sigma [B,Hq], refresh [B] uint8)."""
    buf = _c(buf, np.float64)
    T = _c(T, np.int32)
    kc = _c(kc, np.float64)
    vc = _c(vc, np.float64)
    B, Hq, k = T.shape
    _, Hkv, S, D = kc.shape
    assert buf.shape == (B, Hq, k, 2, D) and vc.shape == kc.shape
    sigma = np.empty((B, Hq), np.float64)
    refresh = np.empty((B,), np.uint8)
    _load().orc_drift(_p(buf), _p(T), _p(kc), _p(vc), B, Hq, Hkv, S, D, k, float(gamma),
                      _p(sigma), _p(refresh))
    return sigma, refresh


# ------------------------------------------------------------------------------------------
# The step, composed
# ------------------------------------------------------------------------------------------

def head_rows(wl, part: str, heads=None) -> np.ndarray:
    """Rows of W_qkv ([Q heads | K heads | V heads] x D) for the given heads of one part."""
    D = wl.head_dim
    base = {"q": 0, "k": wl.q_heads, "v": wl.q_heads + wl.kv_heads}[part]
    count = wl.q_heads if part == "q" else wl.kv_heads
    heads = range(count) if heads is None else heads
    return np.concatenate([np.arange((base + h) * D, (base + h + 1) * D) for h in heads]) \
        .astype(np.int32) if len(heads) else np.zeros(0, np.int32)


def qkv_rows(x_rows: np.ndarray, pos, w: np.ndarray, wl, part: str, heads=None) -> np.ndarray:
    """O1 + O2: the given part ('q', 'k' or 'v') of rows x_rows [R, H] at positions pos [R],
    as [R, nheads, D] float64; q and k rotated, v as projected."""
    count = wl.q_heads if part == "q" else wl.kv_heads
    nh = count if heads is None else len(heads)
    y = linear(x_rows, w, head_rows(wl, part, heads)).reshape(len(x_rows), nh, wl.head_dim)
    if part in ("q", "k"):
        y = rope(y, pos, wl.rope_base)
    return y


def store_rows(x: np.ndarray, dtype: str):
    """Round K/V rows [..., D] as the cache stores them.  Returns (values, codes, scales);
    codes/scales are None except for the fp8 cache."""
    if dtype == "fp8":
        codes, scales, deq = fp8_quantize_rows(x)
        return deq, codes, scales
    return round_storage(x, dtype), None, None


class Cache:
    """K and V [B, Hkv, S, D] as stored (float64 holding storage values), plus, for the fp8
    cache, the codes, the scales and the exact values before quantisation."""

    def __init__(self, wl):
        B, Hkv, S, D = wl.batch, wl.kv_heads, wl.seq, wl.head_dim
        self.wl = wl
        self.k = np.zeros((B, Hkv, S, D))
        self.v = np.zeros((B, Hkv, S, D))
        if wl.cache == "fp8":
            self.k_codes = np.zeros((B, Hkv, S, D), np.uint8)
            self.v_codes = np.zeros((B, Hkv, S, D), np.uint8)
            self.k_scale = np.zeros((B, Hkv, S), np.float32)
            self.v_scale = np.zeros((B, Hkv, S), np.float32)
            self.k_exact = np.zeros((B, Hkv, S, D))
            self.v_exact = np.zeros((B, Hkv, S, D))

    def copy(self):
        c = Cache.__new__(Cache)
        c.__dict__ = {k: (v.copy() if isinstance(v, np.ndarray) else v)
                      for k, v in self.__dict__.items()}
        return c

    def write_rows(self, b: int, rows, kx: np.ndarray, vx: np.ndarray):
        """Write K/V rows for sequence b at positions rows; kx/vx: [R, Hkv, D] float64."""
        rows = np.asarray(rows)
        for name, x in (("k", kx), ("v", vx)):
            vals, codes, scales = store_rows(x, self.wl.cache)
            getattr(self, name)[b][:, rows] = vals.transpose(1, 0, 2)
            if codes is not None:
                getattr(self, name + "_codes")[b][:, rows] = codes.transpose(1, 0, 2)
                getattr(self, name + "_scale")[b][:, rows] = scales.T
                getattr(self, name + "_exact")[b][:, rows] = x.transpose(1, 0, 2)


def refresh_rows(cache: Cache, hidden: np.ndarray, w: np.ndarray, idx, batches=None,
                 kv_heads=None):
    """O4: recompute the K/V rows idx[b] of every sequence from hidden [B, S, H] and write
    them into the cache.  Every other row is left as it is."""
    wl = cache.wl
    batches = range(wl.batch) if batches is None else batches
    for b in batches:
        rows = np.asarray(idx[b], dtype=np.int32)
        x = hidden[b, rows]
        kx = qkv_rows(x, rows, w, wl, "k", kv_heads)
        vx = qkv_rows(x, rows, w, wl, "v", kv_heads)
        if kv_heads is not None and len(kv_heads) != wl.kv_heads:
            full_k = np.zeros((len(rows), wl.kv_heads, wl.head_dim))
            full_v = np.zeros_like(full_k)
            full_k[:, list(kv_heads)] = kx
            full_v[:, list(kv_heads)] = vx
            kx, vx = full_k, full_v
        cache.write_rows(b, rows, kx, vx)
    return cache


def prefill(wl, hidden: np.ndarray, w: np.ndarray, batches=None, kv_heads=None) -> Cache:
    """O3: fill every cache row from hidden [B, S, H] (the first step of a block)."""
    cache = Cache(wl)
    all_rows = np.tile(np.arange(wl.seq, dtype=np.int32), (wl.batch, 1))
    return refresh_rows(cache, hidden, w, all_rows, batches, kv_heads)


def queries(wl, hidden: np.ndarray, w: np.ndarray, idx, batches=None, q_heads=None):
    """Q of the refreshed rows, [B, n, Hq, D], rounded to the activation dtype."""
    B, n = idx.shape
    nh = wl.q_heads if q_heads is None else len(q_heads)
    q = np.zeros((B, n, nh, wl.head_dim))
    batches = range(B) if batches is None else batches
    for b in batches:
        rows = np.asarray(idx[b], dtype=np.int32)
        q[b] = qkv_rows(hidden[b, rows], rows, w, wl, "q", q_heads)
    return round_storage(q, wl.act)


def attend(wl, q: np.ndarray, cache: Cache, want_mass=False):
    """O5/O6 over the stored cache values: (out, lse, mass); out is left in float64."""
    return attention(q, cache.k, cache.v, 1.0 / math.sqrt(wl.head_dim), True, want_mass)


def facache_reference(wl, q_all: np.ndarray, cache: Cache, block_start):
    """What a FACache attention step must give for query rows of every position: the
    attention output and log-sum-exp of every row over all keys (the plain definition), and,
    for the rows outside each sequence's block [block_start[b], + n), the online-softmax
    state over the keys outside the block (LaCache Technical Summary, Methodology 1).
    q_all: [B, S, Hq, D].  Returns out [B,S,Hq,D], lse [B,Hq,S], (m, l, o_tilde) as in
    attention_state and the invariant-row mask [B, S]."""
    B, S, n = wl.batch, wl.seq, wl.n_refresh
    out, lse, _ = attend(wl, q_all, cache)
    inv = np.ones((B, S), bool)
    for b in range(B):
        inv[b, block_start[b]:block_start[b] + n] = False
    m, ll, o = attention_state(q_all, cache.k, cache.v, 1.0 / math.sqrt(wl.head_dim), inv)
    return out, lse, (m, ll, o), inv


def track(cache: Cache, mass: np.ndarray, k: int):
    """O8 + O10: T = top-k of the mass per (b, h); buffer = the cache rows at T, [B,Hq,k,2,D]."""
    wl = cache.wl
    T = topk(mass, k)
    B, Hq = T.shape[:2]
    G = wl.q_heads // wl.kv_heads
    buf = np.zeros((B, Hq, k, 2, wl.head_dim))
    for b in range(B):
        for h in range(Hq):
            for t in range(k):
                j = T[b, h, t]
                if j >= 0:
                    buf[b, h, t, 0] = cache.k[b, h // G, j]
                    buf[b, h, t, 1] = cache.v[b, h // G, j]
    return T, buf


# ------------------------------------------------------------------------------------------
# Partial refresh chosen by feature similarity (dLLM-Cache) and the layer schedule
# (Elastic-Cache)
# ------------------------------------------------------------------------------------------

def feature_similarity(h_cur: np.ndarray, h_cached: np.ndarray) -> np.ndarray:
    """O11: cosine of every row's current input feature with the feature its cache rows were
    last computed from (dLLM-Cache record, abstract: partial response updates guided by
    feature similarity).  [B, S, H] x [B, S, H] -> [B, S] fp64: <x, y> / (|x| |y|); two zero
    rows -> 1, exactly one zero row -> 0 (the drift test's convention)."""
    x = _c(h_cur, np.float64)
    y = _c(h_cached, np.float64)
    assert x.shape == y.shape and x.ndim == 3
    dot = np.einsum("bsh,bsh->bs", x, y)
    nx = np.sqrt(np.einsum("bsh,bsh->bs", x, x))
    ny = np.sqrt(np.einsum("bsh,bsh->bs", y, y))
    zx, zy = nx == 0, ny == 0
    with np.errstate(invalid="ignore", divide="ignore"):
        sim = dot / (nx * ny)
    return np.where(zx & zy, 1.0, np.where(zx | zy, 0.0, sim))


def similarity_select(h_cur, h_cached, lo: int, window_start, window: int, k: int):
    """O12: the rows a sequence refreshes at this step: its window rows [ws_b, ws_b + window)
    (Elastic-Cache core idea: the live tokens near the decoding position), plus the k rows of
    the response [lo, S) outside that window whose features moved most, i.e. the k lowest
    cosines of O11 (ties: lower position first; dLLM-Cache abstract).  Returns
    (idx [B, window + k] int32 ascending, sim [B, S])."""
    sim = feature_similarity(h_cur, h_cached)
    B, S = sim.shape
    ws = np.zeros(B, np.int64) if window_start is None else np.asarray(window_start)
    out = np.empty((B, window + k), np.int32)
    for b in range(B):
        win = set(range(int(ws[b]), int(ws[b]) + window))
        cand = [j for j in range(lo, S) if j not in win]
        assert len(cand) >= k
        chosen = sorted(cand, key=lambda j: (sim[b, j], j))[:k]
        out[b] = sorted(win | set(chosen))
    return out, sim


def schedule_rows(S: int, idx, tracked, full):
    """O13: rows each sequence refreshes at one layer of the Elastic-Cache schedule (card,
    core idea): every row when its drift test fired at an earlier layer of this step
    (recomputation from layer l + 1 to L), otherwise its step rows idx[b] together with its
    tracked positions (tracked[b], -1 = empty slot), so that the drift test compares rows
    computed at this step.  Returns (rows [T] int32, each sequence's rows ascending and
    packed in sequence order, cu [B + 1] int32)."""
    idx = np.asarray(idx)
    B = idx.shape[0]
    parts = []
    for b in range(B):
        if full is not None and full[b]:
            parts.append(np.arange(S, dtype=np.int32))
            continue
        s = set(int(j) for j in np.asarray(idx[b]).ravel())
        if tracked is not None:
            s |= set(int(j) for j in np.asarray(tracked[b]).ravel() if j >= 0)
        parts.append(np.array(sorted(s), dtype=np.int32))
    cu = np.zeros(B + 1, np.int32)
    cu[1:] = np.cumsum([len(p) for p in parts])
    rows = np.concatenate(parts).astype(np.int32) if parts else np.zeros(0, np.int32)
    return rows, cu


class LayerState:
    """One layer of the schedule: its workload geometry, weights, cache, cached input features
    ([B, S, H], the rows' inputs when their cache rows were last computed), tracked positions
    [B, Hq, k] and tracking buffer [B, Hq, k, 2, D]."""

    def __init__(self, wl, w, cache, feat, T, buf):
        self.wl, self.w, self.cache, self.feat, self.T, self.buf = wl, w, cache, feat, T, buf


def schedule_prepare(wl, w: np.ndarray, h_prev: np.ndarray, rows0, k_track: int) -> LayerState:
    """A layer before the step: prefill from h_prev, then the previous step (rows0 [B, n]
    refreshed from the same states, their attention with mass) sets the tracked positions and
    the tracking buffer from that mass."""
    cache = prefill(wl, h_prev, w)
    rows0 = np.asarray(rows0, np.int32)
    q = queries(wl, h_prev, w, rows0)
    _, _, mass = attend(wl, q, cache, want_mass=True)
    T, buf = track(cache, mass, k_track)
    return LayerState(wl, w, cache, np.array(h_prev, np.float64), T, buf)


def schedule_layer(st: LayerState, h_cur: np.ndarray, full, lo: int, window_start, window: int,
                   k_select: int, gamma: float):
    """O14: one layer of one denoising step under the Elastic-Cache schedule with a
    similarity-chosen partial refresh.  full [B] (bool): the sequences whose drift test fired
    at an earlier layer of this step.  In order:
      1. step rows R_b: window plus the k_select least similar response rows (O12);
      2. refreshed rows: all rows of a full sequence, else R_b with the tracked positions (O13);
      3. their K/V rows recomputed from h_cur into the cache, their queries formed (O1-O4);
      4. attention of those queries over each sequence's whole cache, with mass (O5/O6);
      5. drift test of the previous tracked rows against the cache now (O9), then the
         tracking update from this mass (O8/O10);
      6. the refreshed rows' cached features become h_cur's;
      7. full_next = full or the drift decision (Elastic-Cache: recompute from l + 1 to L).
    Returns a dict of every intermediate; st is updated in place."""
    wl = st.wl
    B, S, Hq, D = wl.batch, wl.seq, wl.q_heads, wl.head_dim
    R, sim = similarity_select(h_cur, st.feat, lo, window_start, window, k_select)
    rows, cu = schedule_rows(S, R, st.T.reshape(B, -1), full)
    q = np.zeros((int(cu[-1]), Hq, D))
    for b in range(B):
        r = rows[cu[b]:cu[b + 1]]
        if len(r):
            refresh_rows(st.cache, h_cur, st.w, [r] * B, batches=[b])
            q[cu[b]:cu[b + 1]] = round_storage(qkv_rows(h_cur[b, r], r, st.w, wl, "q"), wl.act)
    lens = np.full(B, S, np.int32)
    out, lse, mass = attention_varlen(q, st.cache.k, st.cache.v, 1.0 / math.sqrt(D), cu, lens,
                                      True)
    sigma, decision = drift(st.buf, st.T, st.cache.k, st.cache.v, gamma)
    T_prev = st.T
    st.T, st.buf = track(st.cache, mass, st.T.shape[-1])
    for b in range(B):
        r = rows[cu[b]:cu[b + 1]]
        st.feat[b, r] = h_cur[b, r]
    full_next = np.asarray(full, bool) | decision.astype(bool)
    return dict(R=R, sim=sim, rows=rows, cu=cu, q=q, out=out, lse=lse, mass=mass, sigma=sigma,
                decision=decision, T_prev=T_prev, full_next=full_next)


# ------------------------------------------------------------------------------------------
# Per-group FP8 linear layer (LaCache Technical Summary, Methodology 2)
# ------------------------------------------------------------------------------------------

FP8_GROUP = 128


def _e4m3_of_fp32_quotient(x32: np.ndarray, scale32: np.ndarray) -> np.ndarray:
    """Codes e4m3(fp32(x / scale)): the quotient rounded to fp32 first (IEEE division), the
    precision the kernel forms it in, since it decides the code."""
    q = (x32 / scale32).astype(np.float32)
    return e4m3_encode(q.astype(np.float64))


def fp8_quantize_groups(x: np.ndarray):
    """O15: activations [M, K] -> (codes uint8 [M, K], scales fp32 [M, K / 128]): one scale
    per 1 x 128 group (LaCache Methodology 2, granularity): scale = fp32(amax) / 448 in fp32
    (a zero group: 1), code = e4m3(x / scale)."""
    x32 = _c(x, np.float32)
    M, K = x32.shape
    assert K % FP8_GROUP == 0
    g = x32.reshape(M, K // FP8_GROUP, FP8_GROUP)
    amax = np.abs(g).max(axis=-1)
    scale = np.where(amax == 0, np.float32(1.0), amax / np.float32(448.0)).astype(np.float32)
    codes = _e4m3_of_fp32_quotient(g, scale[..., None]).reshape(M, K)
    return codes, scale


def fp8_quantize_blocks(w: np.ndarray):
    """O16: weights [N, K] -> (codes uint8 [N, K], scales fp32 [N / 128, K / 128]): one scale
    per 128 x 128 block (LaCache Methodology 2, granularity), same rule as O15 over the
    block."""
    w32 = _c(w, np.float32)
    N, K = w32.shape
    assert N % FP8_GROUP == 0 and K % FP8_GROUP == 0
    blk = w32.reshape(N // FP8_GROUP, FP8_GROUP, K // FP8_GROUP, FP8_GROUP)
    amax = np.abs(blk).max(axis=(1, 3))
    scale = np.where(amax == 0, np.float32(1.0), amax / np.float32(448.0)).astype(np.float32)
    codes = _e4m3_of_fp32_quotient(blk, scale[:, None, :, None]).reshape(N, K)
    return codes, scale


def fp8_linear(x_codes, x_scales, w_codes, w_scales) -> np.ndarray:
    """O17: y = dequant(x) dequant(w)^T in fp64, with dequant(x)[m, k] =
    decode(x_codes[m, k]) * x_scales[m, k / 128] and dequant(w)[n, k] =
    decode(w_codes[n, k]) * w_scales[n / 128, k / 128]: the linear layer the per-group FP8
    GEMM computes (LaCache Methodology 2).  [M, K] x [N, K] -> [M, N]."""
    xd = e4m3_decode(x_codes) * np.repeat(np.asarray(x_scales, np.float64), FP8_GROUP, axis=1)
    ws = np.repeat(np.repeat(np.asarray(w_scales, np.float64), FP8_GROUP, axis=0), FP8_GROUP,
                   axis=1)
    wd = e4m3_decode(w_codes) * ws
    return xd @ wd.T
