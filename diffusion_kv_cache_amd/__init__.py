"""Python binding of libdllm_cache.so: the per-layer cached denoising step on MI355X.

Argument marshalling only: every step runs in the library's HIP kernels.  PyTorch supplies
device memory and the stream (``torch.cuda.current_stream()`` unless one is given).  The
functions carry the C names of ``include/dllm_cache.h``; each raises ``DllmError`` with the
library's message when the call returns an error.

There is no fallback: importing this package on a machine without the built library raises
``ImportError``; calling it without a GPU fails in the HIP runtime.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libdllm_cache.so")

DLLM_OK, DLLM_EINVAL, DLLM_ESIZE, DLLM_EUNSUPPORTED, DLLM_ELAUNCH = 0, 1, 2, 3, 4
DLLM_F32, DLLM_BF16, DLLM_FP8_E4M3 = 0, 1, 2
STATUS_NAMES = {0: "DLLM_OK", 1: "DLLM_EINVAL", 2: "DLLM_ESIZE", 3: "DLLM_EUNSUPPORTED",
                4: "DLLM_ELAUNCH"}
EXPORTS = ("dllm_cache_bytes", "dllm_cache_alloc", "dllm_refresh_qkv_rope_scatter",
           "dllm_refresh_workspace_bytes", "dllm_attention_workspace_bytes",
           "dllm_block_attention", "dllm_track_buffer_bytes", "dllm_drift_workspace_bytes",
           "dllm_drift_check",
           "dllm_fp8_e4m3_roundtrip",
           "dllm_set_options", "dllm_block_attention_noalloc", "dllm_facache_state_bytes",
           "dllm_facache_attention", "dllm_refresh_qkv_rope_scatter_varlen",
           "dllm_attention_varlen_workspace_bytes", "dllm_block_attention_varlen",
           "dllm_similarity_select_workspace_bytes", "dllm_similarity_select",
           "dllm_schedule_rows_workspace_bytes", "dllm_schedule_rows", "dllm_copy_rows_varlen",
           "dllm_layer_step_workspace_bytes", "dllm_elastic_layer_step",
           "dllm_fp8_quantize_weight", "dllm_fp8_quantize_activations",
           "dllm_fp8_linear_workspace_bytes", "dllm_fp8_linear", "dllm_rope_rows",
           "dllm_scatter_kv_rows", "dllm_mfma_rate_probe", "dllm_read_rate_probe", "dllm_last_error")
DLLM_OPT_DEBUG, DLLM_OPT_WIDE_OFFSETS = 1, 2
DLLM_NOALLOC_SCRATCH_BYTES = 32 << 20

_TORCH_DTYPE = {DLLM_F32: torch.float32, DLLM_BF16: torch.bfloat16, DLLM_FP8_E4M3: torch.uint8}
_DTYPE_CODE = {torch.float32: DLLM_F32, torch.bfloat16: DLLM_BF16}


class DllmError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {msg}")
        self.status = status


class CacheDesc(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32),
                ("max_seq", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("kv_dtype", ctypes.c_int32), ("group_size", ctypes.c_int32)]


class LayerStep(ctypes.Structure):
    """The C struct dllm_layer_step (device pointers and sizes)."""
    _fields_ = [(name, ctypes.c_void_p) for name in (
        "hidden_cur", "hidden_feat", "w_qkv", "window_start", "track_idx", "track_buf", "full",
        "decision", "step_rows", "rows", "cu_rows", "q", "out", "lse", "attn_mass", "sigma")] + \
        [(name, ctypes.c_int32) for name in (
            "hidden_size", "num_q_heads", "lo", "window", "k_select", "k_track")] + \
        [(name, ctypes.c_float) for name in ("rope_base", "softmax_scale", "gamma")]


class CCache(ctypes.Structure):
    _fields_ = [("desc", CacheDesc), ("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
                ("k_scale", ctypes.c_void_p), ("v_scale", ctypes.c_void_p)]


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run python -m diffusion_kv_cache_amd.build")
    lib = ctypes.CDLL(LIB_PATH)
    P, i32, i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
    lib.dllm_cache_bytes.restype = ctypes.c_size_t
    lib.dllm_cache_bytes.argtypes = [ctypes.POINTER(CacheDesc)]
    lib.dllm_cache_alloc.restype = i32
    lib.dllm_cache_alloc.argtypes = [ctypes.POINTER(CacheDesc), P, ctypes.c_size_t,
                                     ctypes.POINTER(CCache)]
    lib.dllm_refresh_qkv_rope_scatter.restype = i32
    lib.dllm_refresh_qkv_rope_scatter.argtypes = [ctypes.POINTER(CCache), P, i32, i32, P, i32, P,
                                                  i32, ctypes.c_float, P, P, ctypes.c_size_t, P]
    lib.dllm_refresh_workspace_bytes.restype = ctypes.c_size_t
    lib.dllm_refresh_workspace_bytes.argtypes = [ctypes.POINTER(CacheDesc), i32, i32, i32, i32]
    lib.dllm_attention_workspace_bytes.restype = ctypes.c_size_t
    lib.dllm_attention_workspace_bytes.argtypes = [ctypes.POINTER(CacheDesc), i32, i32]
    lib.dllm_block_attention.restype = i32
    lib.dllm_block_attention.argtypes = [ctypes.POINTER(CCache), P, i32, i32, i32, ctypes.c_float,
                                         P, P, P, P, ctypes.c_size_t, P]
    lib.dllm_block_attention_noalloc.restype = i32
    lib.dllm_block_attention_noalloc.argtypes = [ctypes.POINTER(CCache), P, i32, i32, i32,
                                                 ctypes.c_float, P, P, P, P]
    lib.dllm_facache_state_bytes.restype = ctypes.c_size_t
    lib.dllm_facache_state_bytes.argtypes = [ctypes.POINTER(CacheDesc), i32]
    lib.dllm_facache_attention.restype = i32
    lib.dllm_facache_attention.argtypes = [ctypes.POINTER(CCache), P, P, P, i32, i32, ctypes.c_float,
                                           P, i32, P, P, P]
    lib.dllm_refresh_qkv_rope_scatter_varlen.restype = i32
    lib.dllm_refresh_qkv_rope_scatter_varlen.argtypes = [ctypes.POINTER(CCache), P, i32, i32, P, P,
                                                         i32, i32, P, i32, ctypes.c_float, P, P,
                                                         ctypes.c_size_t, P]
    lib.dllm_attention_varlen_workspace_bytes.restype = ctypes.c_size_t
    lib.dllm_attention_varlen_workspace_bytes.argtypes = [ctypes.POINTER(CacheDesc), i32, i32, i32]
    lib.dllm_block_attention_varlen.restype = i32
    lib.dllm_block_attention_varlen.argtypes = [ctypes.POINTER(CCache), P, i32, i32, P, P, i32,
                                                i32, ctypes.c_float, P, P, P, P, ctypes.c_size_t,
                                                P]
    lib.dllm_similarity_select_workspace_bytes.restype = ctypes.c_size_t
    lib.dllm_similarity_select_workspace_bytes.argtypes = [i32, i32]
    lib.dllm_similarity_select.restype = i32
    lib.dllm_similarity_select.argtypes = [i32, i32, i32, i32, P, P, i32, P, i32, i32, P, P, P,
                                           ctypes.c_size_t, P]
    lib.dllm_schedule_rows_workspace_bytes.restype = ctypes.c_size_t
    lib.dllm_schedule_rows_workspace_bytes.argtypes = [i32, i32]
    lib.dllm_schedule_rows.restype = i32
    lib.dllm_schedule_rows.argtypes = [i32, i32, P, i32, P, i32, P, P, P, P, i32, P, P,
                                       ctypes.c_size_t, P]
    lib.dllm_copy_rows_varlen.restype = i32
    lib.dllm_copy_rows_varlen.argtypes = [i32, i32, i32, P, P, P, P, i32, P]
    lib.dllm_layer_step_workspace_bytes.restype = ctypes.c_size_t
    lib.dllm_layer_step_workspace_bytes.argtypes = [ctypes.POINTER(CacheDesc), i32, i32]
    lib.dllm_elastic_layer_step.restype = i32
    lib.dllm_elastic_layer_step.argtypes = [ctypes.POINTER(CCache), ctypes.POINTER(LayerStep), P,
                                            ctypes.c_size_t, P]
    lib.dllm_fp8_quantize_weight.restype = i32
    lib.dllm_fp8_quantize_weight.argtypes = [P, i32, i32, P, P, P]
    lib.dllm_fp8_quantize_activations.restype = i32
    lib.dllm_fp8_quantize_activations.argtypes = [P, i32, i32, P, P, i32, P]
    lib.dllm_fp8_linear_workspace_bytes.restype = ctypes.c_size_t
    lib.dllm_fp8_linear_workspace_bytes.argtypes = [i32, i32, i32]
    lib.dllm_fp8_linear.restype = i32
    lib.dllm_fp8_linear.argtypes = [P, i32, i32, P, P, i32, P, P, ctypes.c_size_t, P]
    lib.dllm_rope_rows.restype = i32
    lib.dllm_rope_rows.argtypes = [P, i32, i32, i32, i32, P, ctypes.c_float, P]
    lib.dllm_scatter_kv_rows.restype = i32
    lib.dllm_scatter_kv_rows.argtypes = [ctypes.POINTER(CCache), P, i32, i32, i32, P, i32, P]
    lib.dllm_mfma_rate_probe.restype = i32
    lib.dllm_mfma_rate_probe.argtypes = [i32, i32, i32, i32, P, P]
    lib.dllm_read_rate_probe.restype = i32
    lib.dllm_read_rate_probe.argtypes = [P, i64, i32, P, P]
    lib.dllm_drift_check.restype = i32
    lib.dllm_track_buffer_bytes.restype = ctypes.c_size_t
    lib.dllm_track_buffer_bytes.argtypes = [ctypes.POINTER(CacheDesc), i32, i32]
    lib.dllm_drift_workspace_bytes.restype = ctypes.c_size_t
    lib.dllm_drift_workspace_bytes.argtypes = [i32]
    lib.dllm_drift_check.argtypes = [ctypes.POINTER(CCache), i32, i32, ctypes.c_float, P, P, P, P,
                                     P, P, ctypes.c_size_t, P]
    lib.dllm_fp8_e4m3_roundtrip.restype = i32
    lib.dllm_fp8_e4m3_roundtrip.argtypes = [P, i64, ctypes.c_float, P, P, P]
    lib.dllm_set_options.restype = i32
    lib.dllm_set_options.argtypes = [i32]
    lib.dllm_last_error.restype = ctypes.c_char_p
    lib.dllm_last_error.argtypes = []
    return lib


lib = _load()


def _check(status: int):
    if status != DLLM_OK:
        raise DllmError(status, lib.dllm_last_error().decode())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _scratch(nbytes: int, device, stream):
    """A workspace allocated here for one call.  The caching allocator ties a block to the
    stream current at allocation, so the block is recorded on the launch stream too: it is
    not handed out again before the library's kernels there are done with it."""
    t = torch.empty(nbytes, dtype=torch.uint8, device=device)
    if stream is not None:
        t.record_stream(stream)
    return t


class Cache:
    """One layer's flat K/V cache in a single torch allocation, with the C descriptor.

    ``k``, ``v`` are [B, Hkv, S, D] views (uint8 codes for FP8), ``k_scale``/``v_scale``
    [B, Hkv, S] fp32 views (FP8 only).  The memory is uninitialised until a refresh over all
    rows fills it."""

    def __init__(self, batch, num_kv_heads, max_seq, head_dim, kv_dtype, device="cuda",
                 guard: int = 0):
        """``guard`` extra bytes (rounded up to 256) are kept on both sides of the region
        inside ``storage``, so tests can check that nothing is written outside it."""
        self.desc = CacheDesc(batch, num_kv_heads, max_seq, head_dim, kv_dtype,
                              head_dim if kv_dtype == DLLM_FP8_E4M3 else 0)
        nbytes = dllm_cache_bytes(self.desc)
        if nbytes == 0:
            raise DllmError(DLLM_EINVAL, lib.dllm_last_error().decode())
        guard = (guard + 255) // 256 * 256
        self.storage = torch.empty(nbytes + 2 * guard + 256, dtype=torch.uint8, device=device)
        off = (-self.storage.data_ptr()) % 256 + guard
        self.region_offset = off
        self.region = self.storage[off:off + nbytes]
        self.c = CCache()
        _check(lib.dllm_cache_alloc(ctypes.byref(self.desc), _ptr(self.region), nbytes,
                                    ctypes.byref(self.c)))
        shape = (batch, num_kv_heads, max_seq, head_dim)
        rows = batch * num_kv_heads * max_seq
        dt = _TORCH_DTYPE[kv_dtype]
        esz = torch.empty(0, dtype=dt).element_size()
        base = self.region.data_ptr()
        self.k = self._view(self.c.k - base, rows * head_dim * esz, dt, shape)
        self.v = self._view(self.c.v - base, rows * head_dim * esz, dt, shape)
        self.k_scale = self.v_scale = None
        if kv_dtype == DLLM_FP8_E4M3:
            self.k_scale = self._view(self.c.k_scale - base, rows * 4, torch.float32, shape[:3])
            self.v_scale = self._view(self.c.v_scale - base, rows * 4, torch.float32, shape[:3])

    def _view(self, off, nbytes, dtype, shape):
        return self.region[off:off + nbytes].view(dtype).view(shape)

    @property
    def kv_dtype(self):
        return self.desc.kv_dtype


def dllm_cache_bytes(desc: CacheDesc) -> int:
    return lib.dllm_cache_bytes(ctypes.byref(desc))


def _expect(t: torch.Tensor, name: str, shape, dtype):
    if t is None:
        raise DllmError(DLLM_EINVAL, f"{name} is required")
    if tuple(t.shape) != tuple(shape) or t.dtype != dtype or not t.is_contiguous() \
            or t.device.type != "cuda":
        raise DllmError(DLLM_EINVAL, f"{name}: expected contiguous cuda {dtype} {tuple(shape)}, "
                                     f"got {t.device} {t.dtype} {tuple(t.shape)}")


def dllm_refresh_workspace_bytes(cache: Cache, hidden_size: int, act_dtype: int, n: int,
                                 num_q_heads: int) -> int:
    return lib.dllm_refresh_workspace_bytes(ctypes.byref(cache.desc), hidden_size, act_dtype, n,
                                            num_q_heads)


def dllm_refresh_qkv_rope_scatter(cache: Cache, hidden: torch.Tensor, refresh_idx: torch.Tensor,
                                  w_qkv: torch.Tensor, num_q_heads: int, rope_base: float,
                                  q_out: torch.Tensor, workspace=None, stream=None):
    """hidden [B,S,H], refresh_idx [B,n] int32, w_qkv [(Hq+2Hkv)D, H], q_out [B,n,Hq,D];
    workspace a uint8 device tensor (allocated here when None and needed)."""
    d = cache.desc
    if hidden.dtype not in _DTYPE_CODE:
        raise DllmError(DLLM_EINVAL, f"hidden dtype {hidden.dtype}")
    act = _DTYPE_CODE[hidden.dtype]
    H = hidden.shape[-1]
    n = refresh_idx.shape[1] if refresh_idx.dim() == 2 else -1
    _expect(hidden, "hidden", (d.batch, d.max_seq, H), hidden.dtype)
    _expect(refresh_idx, "refresh_idx", (d.batch, n), torch.int32)
    _expect(w_qkv, "w_qkv", ((num_q_heads + 2 * d.num_kv_heads) * d.head_dim, H), hidden.dtype)
    _expect(q_out, "q_out", (d.batch, n, num_q_heads, d.head_dim), hidden.dtype)
    if workspace is None:
        need = dllm_refresh_workspace_bytes(cache, H, act, n, num_q_heads)
        workspace = _scratch(need, hidden.device, stream) if need else None
    ws_bytes = 0 if workspace is None else workspace.numel()
    _check(lib.dllm_refresh_qkv_rope_scatter(
        ctypes.byref(cache.c), _ptr(hidden), H, act, _ptr(refresh_idx), n,
        _ptr(w_qkv), num_q_heads, float(rope_base), _ptr(q_out), _ptr(workspace), ws_bytes,
        _stream(stream)))


def dllm_refresh_qkv_rope_scatter_varlen(cache: Cache, hidden: torch.Tensor,
                                         refresh_idx: torch.Tensor, cu_rows: torch.Tensor,
                                         max_rows: int, w_qkv: torch.Tensor, num_q_heads: int,
                                         rope_base: float, q_out: torch.Tensor, workspace=None,
                                         stream=None):
    """Packed rows of a variable-length batch: refresh_idx [T] int32, cu_rows [B+1] int32
    (device), q_out [T, Hq, D]; T = cu_rows[B] = refresh_idx.numel()."""
    d = cache.desc
    if hidden.dtype not in _DTYPE_CODE:
        raise DllmError(DLLM_EINVAL, f"hidden dtype {hidden.dtype}")
    act = _DTYPE_CODE[hidden.dtype]
    H = hidden.shape[-1]
    T = refresh_idx.numel()
    _expect(hidden, "hidden", (d.batch, d.max_seq, H), hidden.dtype)
    _expect(refresh_idx, "refresh_idx", (T,), torch.int32)
    _expect(cu_rows, "cu_rows", (d.batch + 1,), torch.int32)
    _expect(w_qkv, "w_qkv", ((num_q_heads + 2 * d.num_kv_heads) * d.head_dim, H), hidden.dtype)
    _expect(q_out, "q_out", (T, num_q_heads, d.head_dim), hidden.dtype)
    if workspace is None:
        need = _refresh_ws_for_rows(cache, H, act, T, num_q_heads)
        workspace = _scratch(need, hidden.device, stream) if need else None
    ws_bytes = 0 if workspace is None else workspace.numel()
    _check(lib.dllm_refresh_qkv_rope_scatter_varlen(
        ctypes.byref(cache.c), _ptr(hidden), H, act, _ptr(refresh_idx), _ptr(cu_rows), T,
        int(max_rows), _ptr(w_qkv), num_q_heads, float(rope_base), _ptr(q_out),
        _ptr(workspace), ws_bytes, _stream(stream)))


def _refresh_ws_for_rows(cache: Cache, H: int, act: int, rows: int, num_q_heads: int) -> int:
    """Workspace of a refresh of `rows` rows in all (what a one-sequence batch of that many
    rows needs)."""
    d = cache.desc
    one = CacheDesc(1, d.num_kv_heads, max(d.max_seq, rows), d.head_dim, d.kv_dtype, d.group_size)
    return lib.dllm_refresh_workspace_bytes(ctypes.byref(one), H, act, rows, num_q_heads)


def dllm_attention_varlen_workspace_bytes(cache: Cache, num_q_heads: int, total_rows: int,
                                          max_rows: int) -> int:
    return lib.dllm_attention_varlen_workspace_bytes(ctypes.byref(cache.desc), num_q_heads,
                                                     total_rows, max_rows)


def dllm_block_attention_varlen(cache: Cache, q: torch.Tensor, num_q_heads: int,
                                cu_rows: torch.Tensor, seq_lens: torch.Tensor, max_rows: int,
                                softmax_scale: float, out: torch.Tensor, lse=None, attn_mass=None,
                                workspace=None, stream=None):
    """q, out [T, Hq, D] bf16 (packed rows), cu_rows [B+1] int32, seq_lens [B] int32 or None,
    lse [T * Hq] fp32 or None, attn_mass [B, Hq, S] fp32 or None."""
    d = cache.desc
    T = q.shape[0] if q.dim() == 3 else -1
    if q.dtype not in _DTYPE_CODE:
        raise DllmError(DLLM_EINVAL, f"q dtype {q.dtype}")
    _expect(q, "q", (T, num_q_heads, d.head_dim), q.dtype)
    _expect(out, "out", (T, num_q_heads, d.head_dim), q.dtype)
    _expect(cu_rows, "cu_rows", (d.batch + 1,), torch.int32)
    if seq_lens is not None:
        _expect(seq_lens, "seq_lens", (d.batch,), torch.int32)
    if lse is not None:
        _expect(lse, "lse", (T * num_q_heads,), torch.float32)
    if attn_mass is not None:
        _expect(attn_mass, "attn_mass", (d.batch, num_q_heads, d.max_seq), torch.float32)
    if workspace is None:
        workspace = _scratch(max(1, dllm_attention_varlen_workspace_bytes(cache, num_q_heads, T,
                                                                          max_rows)),
                             q.device, stream)
    _check(lib.dllm_block_attention_varlen(
        ctypes.byref(cache.c), _ptr(q), _DTYPE_CODE[q.dtype], num_q_heads, _ptr(cu_rows),
        _ptr(seq_lens), T, int(max_rows), float(softmax_scale), _ptr(out), _ptr(lse),
        _ptr(attn_mass), _ptr(workspace), workspace.numel(), _stream(stream)))


def dllm_attention_workspace_bytes(cache: Cache, num_q_heads: int, n: int) -> int:
    return lib.dllm_attention_workspace_bytes(ctypes.byref(cache.desc), num_q_heads, n)


def dllm_block_attention(cache: Cache, q: torch.Tensor, num_q_heads: int, softmax_scale: float,
                         out: torch.Tensor, lse=None, attn_mass=None, workspace=None,
                         stream=None):
    """q, out [B,n,Hq,D]; lse [B,Hq,n] fp32 or None; attn_mass [B,Hq,S] fp32 or None;
    workspace a uint8 device tensor (allocated here when None)."""
    d = cache.desc
    if q.dtype not in _DTYPE_CODE or q.dim() != 4:
        raise DllmError(DLLM_EINVAL, f"q: expected [B,n,Hq,D] fp32/bf16, got {q.dtype} {tuple(q.shape)}")
    n = q.shape[1]
    act = _DTYPE_CODE[q.dtype]
    _expect(q, "q", (d.batch, n, num_q_heads, d.head_dim), q.dtype)
    _expect(out, "out", (d.batch, n, num_q_heads, d.head_dim), q.dtype)
    if lse is not None:
        _expect(lse, "lse", (d.batch, num_q_heads, n), torch.float32)
    if attn_mass is not None:
        _expect(attn_mass, "attn_mass", (d.batch, num_q_heads, d.max_seq), torch.float32)
    if workspace is None:
        workspace = _scratch(max(1, dllm_attention_workspace_bytes(cache, num_q_heads, n)),
                             q.device, stream)
    _check(lib.dllm_block_attention(
        ctypes.byref(cache.c), _ptr(q), act, num_q_heads, n, float(softmax_scale), _ptr(out),
        _ptr(lse), _ptr(attn_mass), _ptr(workspace), workspace.numel(), _stream(stream)))


def dllm_block_attention_noalloc(cache: Cache, q: torch.Tensor, num_q_heads: int,
                                 softmax_scale: float, out: torch.Tensor, lse=None,
                                 attn_mass=None, stream=None):
    """dllm_block_attention without a workspace: the library's per-GPU scratch serves instead
    (calls that overlap on one GPU race)."""
    d = cache.desc
    if q.dtype not in _DTYPE_CODE or q.dim() != 4:
        raise DllmError(DLLM_EINVAL, f"q: expected [B,n,Hq,D] fp32/bf16, got {q.dtype} {tuple(q.shape)}")
    n = q.shape[1]
    _expect(q, "q", (d.batch, n, num_q_heads, d.head_dim), q.dtype)
    _expect(out, "out", (d.batch, n, num_q_heads, d.head_dim), q.dtype)
    if lse is not None:
        _expect(lse, "lse", (d.batch, num_q_heads, n), torch.float32)
    if attn_mass is not None:
        _expect(attn_mass, "attn_mass", (d.batch, num_q_heads, d.max_seq), torch.float32)
    _check(lib.dllm_block_attention_noalloc(
        ctypes.byref(cache.c), _ptr(q), _DTYPE_CODE[q.dtype], num_q_heads, n,
        float(softmax_scale), _ptr(out), _ptr(lse), _ptr(attn_mass), _stream(stream)))


def dllm_facache_state_bytes(cache: Cache, num_q_heads: int) -> int:
    return lib.dllm_facache_state_bytes(ctypes.byref(cache.desc), num_q_heads)


def dllm_facache_attention(cache: Cache, q_cache: torch.Tensor, q_block: torch.Tensor,
                           block_start: torch.Tensor, num_q_heads: int, softmax_scale: float,
                           fa_state: torch.Tensor, build: bool, out: torch.Tensor, lse=None,
                           stream=None):
    """q_cache [B,S,Hq,D] bf16 (in/out), q_block [B,n,Hq,D] bf16, block_start [B] int32,
    fa_state a float32 tensor of dllm_facache_state_bytes(...) bytes, out [B,S,Hq,D] bf16,
    lse [B,Hq,S] fp32 or None."""
    d = cache.desc
    B, S, D = d.batch, d.max_seq, d.head_dim
    n = q_block.shape[1] if q_block.dim() == 4 else -1
    _expect(q_cache, "q_cache", (B, S, num_q_heads, D), torch.bfloat16)
    _expect(q_block, "q_block", (B, n, num_q_heads, D), torch.bfloat16)
    _expect(block_start, "block_start", (B,), torch.int32)
    _expect(out, "out", (B, S, num_q_heads, D), torch.bfloat16)
    if lse is not None:
        _expect(lse, "lse", (B, num_q_heads, S), torch.float32)
    need = dllm_facache_state_bytes(cache, num_q_heads)
    if fa_state.dtype != torch.float32 or not fa_state.is_contiguous() or \
            fa_state.numel() * 4 < need or fa_state.device.type != "cuda":
        raise DllmError(DLLM_EINVAL, f"fa_state: expected a contiguous cuda float32 tensor of at "
                                     f"least {need} bytes")
    _check(lib.dllm_facache_attention(
        ctypes.byref(cache.c), _ptr(q_cache), _ptr(q_block), _ptr(block_start), n, num_q_heads,
        float(softmax_scale), _ptr(fa_state), int(bool(build)), _ptr(out), _ptr(lse),
        _stream(stream)))


def track_buffer_bytes(cache: Cache, num_q_heads: int, k: int) -> int:
    """Bytes of dllm_drift_check's tracking buffer for this cache (FP8: codes, then scales)."""
    return int(lib.dllm_track_buffer_bytes(ctypes.byref(cache.desc), num_q_heads, k))


def drift_workspace(batch: int, device="cuda") -> torch.Tensor:
    """A zero-filled workspace for dllm_drift_check's decision in the same launch (every call
    leaves it zero; calls that share it must not overlap)."""
    n = int(lib.dllm_drift_workspace_bytes(batch))
    return torch.zeros(max(n, 8) // 8, dtype=torch.int64, device=device)


def dllm_drift_check(cache: Cache, num_q_heads: int, k: int, gamma: float,
                     track_idx: torch.Tensor, track_buf: torch.Tensor, attn_mass, sigma_out,
                     refresh_out, workspace=None, stream=None):
    """track_idx [B,Hq,k] int32 (in/out), track_buf [B,Hq,k,2,D] cache dtype (in/out; FP8
    caches: flat uint8 of track_buffer_bytes, codes then row scales), attn_mass [B,Hq,S] fp32
    or None, sigma_out [B,Hq] fp32, refresh_out [B] uint8,
    workspace from drift_workspace(B) or None (the decision by a second kernel)."""
    d = cache.desc
    B, Hq = d.batch, num_q_heads
    _expect(track_idx, "track_idx", (B, Hq, k), torch.int32)
    if d.kv_dtype == DLLM_FP8_E4M3:
        _expect(track_buf, "track_buf", (track_buffer_bytes(cache, Hq, k),), torch.uint8)
    else:
        _expect(track_buf, "track_buf", (B, Hq, k, 2, d.head_dim), _TORCH_DTYPE[d.kv_dtype])
    if attn_mass is not None:
        _expect(attn_mass, "attn_mass", (B, Hq, d.max_seq), torch.float32)
    _expect(sigma_out, "sigma_out", (B, Hq), torch.float32)
    _expect(refresh_out, "refresh_out", (B,), torch.uint8)
    ws_bytes = 0
    if workspace is not None:
        if not workspace.is_cuda or not workspace.is_contiguous():
            raise DllmError(DLLM_EINVAL, "workspace: contiguous device tensor")
        ws_bytes = workspace.numel() * workspace.element_size()
    _check(lib.dllm_drift_check(
        ctypes.byref(cache.c), num_q_heads, k, float(gamma), _ptr(track_idx), _ptr(track_buf),
        _ptr(attn_mass), _ptr(sigma_out), _ptr(refresh_out), _ptr(workspace), ws_bytes,
        _stream(stream)))


def dllm_similarity_select(hidden_cur: torch.Tensor, hidden_cached: torch.Tensor, lo: int,
                           window_start, window: int, k: int, idx_out: torch.Tensor,
                           sim_out=None, workspace=None, stream=None):
    """hidden_cur, hidden_cached [B, S, H] (bf16 or fp32), window_start [B] int32 or None,
    idx_out [B, window + k] int32, sim_out [B, S] fp64 or None."""
    if hidden_cur.dim() != 3 or hidden_cur.dtype not in _DTYPE_CODE:
        raise DllmError(DLLM_EINVAL, "hidden_cur: [B, S, H] bf16 or fp32")
    B, S, H = hidden_cur.shape
    _expect(hidden_cur, "hidden_cur", (B, S, H), hidden_cur.dtype)
    _expect(hidden_cached, "hidden_cached", (B, S, H), hidden_cur.dtype)
    if window_start is not None:
        _expect(window_start, "window_start", (B,), torch.int32)
    _expect(idx_out, "idx_out", (B, window + k), torch.int32)
    if sim_out is not None:
        _expect(sim_out, "sim_out", (B, S), torch.float64)
    elif workspace is None:
        workspace = _scratch(lib.dllm_similarity_select_workspace_bytes(B, S), hidden_cur.device,
                             stream)
    ws_bytes = 0 if workspace is None else workspace.numel()
    _check(lib.dllm_similarity_select(B, S, H, _DTYPE_CODE[hidden_cur.dtype], _ptr(hidden_cur),
                                      _ptr(hidden_cached), lo, _ptr(window_start), window, k,
                                      _ptr(idx_out), _ptr(sim_out), _ptr(workspace), ws_bytes,
                                      _stream(stream)))


def dllm_schedule_rows(max_seq: int, idx: torch.Tensor, tracked, full_in, decision, full_out,
                       rows_out: torch.Tensor, cu_out: torch.Tensor, workspace=None,
                       stream=None):
    """idx [B, n] int32, tracked [B, ...] int32 or None, full_in / decision / full_out [B]
    uint8 or None, rows_out [capacity >= B * S] int32, cu_out [B + 1] int32."""
    B = idx.shape[0]
    n = idx.numel() // B if B else 0
    _expect(idx, "idx", (B, n), torch.int32)
    m = 0
    if tracked is not None:
        m = tracked.numel() // B
        _expect(tracked.view(B, m), "tracked", (B, m), torch.int32)
    for name, t in (("full_in", full_in), ("decision", decision), ("full_out", full_out)):
        if t is not None:
            _expect(t, name, (B,), torch.uint8)
    if rows_out.dim() != 1:
        raise DllmError(DLLM_EINVAL, "rows_out must be 1-D")
    _expect(rows_out, "rows_out", (rows_out.numel(),), torch.int32)
    _expect(cu_out, "cu_out", (B + 1,), torch.int32)
    if workspace is None:
        workspace = _scratch(lib.dllm_schedule_rows_workspace_bytes(B, max_seq) + 256,
                             idx.device, stream)
    base = (-workspace.data_ptr()) % 256
    ws = workspace[base:]
    _check(lib.dllm_schedule_rows(B, max_seq, _ptr(idx), n, _ptr(tracked), m, _ptr(full_in),
                                  _ptr(decision), _ptr(full_out), _ptr(rows_out), rows_out.numel(),
                                  _ptr(cu_out), _ptr(ws), ws.numel(), _stream(stream)))


def dllm_copy_rows_varlen(src: torch.Tensor, dst: torch.Tensor, rows: torch.Tensor,
                          cu_rows: torch.Tensor, stream=None):
    """src, dst [B, S, ...] (same shape and dtype), rows [capacity] int32, cu_rows [B + 1]."""
    if src.dim() < 2:
        raise DllmError(DLLM_EINVAL, "src must be [B, S, ...]")
    B, S = src.shape[:2]
    _expect(src, "src", tuple(src.shape), src.dtype)
    _expect(dst, "dst", tuple(src.shape), src.dtype)
    _expect(rows, "rows", (rows.numel(),), torch.int32)
    _expect(cu_rows, "cu_rows", (B + 1,), torch.int32)
    row_bytes = src[0, 0].numel() * src.element_size()
    _check(lib.dllm_copy_rows_varlen(B, S, row_bytes, _ptr(src), _ptr(dst), _ptr(rows),
                                     _ptr(cu_rows), rows.numel(), _stream(stream)))


def dllm_layer_step_workspace_bytes(cache: Cache, hidden_size: int, num_q_heads: int) -> int:
    return lib.dllm_layer_step_workspace_bytes(ctypes.byref(cache.desc), hidden_size, num_q_heads)


def dllm_elastic_layer_step(cache: Cache, *, hidden_cur, hidden_feat, w_qkv, window_start,
                            track_idx, track_buf, full, decision, step_rows, rows, cu_rows, q,
                            out, lse, attn_mass, sigma, num_q_heads: int, lo: int, window: int,
                            k_select: int, k_track: int, rope_base: float, softmax_scale: float,
                            gamma: float, workspace=None, stream=None):
    """One layer of the schedule (see the header for the six stages).  Shapes (S, B from the
    cache, cap = B * S): hidden_cur / hidden_feat [B, S, H] bf16, w_qkv [N, H] bf16,
    window_start [B] int32, track_idx [B, Hq, k_track] int32, track_buf [B, Hq, k_track, 2, D]
    bf16, full / decision [B] uint8, step_rows [B, window + k_select] int32, rows [cap] int32,
    cu_rows [B + 1] int32, q / out [cap, Hq, D] bf16, lse [cap * Hq] fp32 or None,
    attn_mass [B, Hq, S] fp32, sigma [B, Hq] fp32."""
    d = cache.desc
    B, S, D, Hq = d.batch, d.max_seq, d.head_dim, num_q_heads
    H = hidden_cur.shape[-1]
    cap = B * S
    bf = torch.bfloat16
    _expect(hidden_cur, "hidden_cur", (B, S, H), bf)
    _expect(hidden_feat, "hidden_feat", (B, S, H), bf)
    _expect(w_qkv, "w_qkv", ((Hq + 2 * d.num_kv_heads) * D, H), bf)
    if window_start is not None:
        _expect(window_start, "window_start", (B,), torch.int32)
    _expect(track_idx, "track_idx", (B, Hq, k_track), torch.int32)
    _expect(track_buf, "track_buf", (B, Hq, k_track, 2, D), bf)
    _expect(full, "full", (B,), torch.uint8)
    _expect(decision, "decision", (B,), torch.uint8)
    _expect(step_rows, "step_rows", (B, window + k_select), torch.int32)
    _expect(rows, "rows", (cap,), torch.int32)
    _expect(cu_rows, "cu_rows", (B + 1,), torch.int32)
    _expect(q, "q", (cap, Hq, D), bf)
    _expect(out, "out", (cap, Hq, D), bf)
    if lse is not None:
        _expect(lse, "lse", (cap * Hq,), torch.float32)
    _expect(attn_mass, "attn_mass", (B, Hq, S), torch.float32)
    _expect(sigma, "sigma", (B, Hq), torch.float32)
    if workspace is None:
        need = dllm_layer_step_workspace_bytes(cache, H, Hq)
        if need == 0:
            raise DllmError(DLLM_EINVAL, "invalid layer step shape")
        workspace = _scratch(need, hidden_cur.device, stream)
    a = LayerStep()
    for name, t in (("hidden_cur", hidden_cur), ("hidden_feat", hidden_feat), ("w_qkv", w_qkv),
                    ("window_start", window_start), ("track_idx", track_idx),
                    ("track_buf", track_buf), ("full", full), ("decision", decision),
                    ("step_rows", step_rows), ("rows", rows), ("cu_rows", cu_rows), ("q", q),
                    ("out", out), ("lse", lse), ("attn_mass", attn_mass), ("sigma", sigma)):
        setattr(a, name, None if t is None else t.data_ptr())
    a.hidden_size, a.num_q_heads, a.lo, a.window = H, Hq, lo, window
    a.k_select, a.k_track = k_select, k_track
    a.rope_base, a.softmax_scale, a.gamma = rope_base, softmax_scale, gamma
    _check(lib.dllm_elastic_layer_step(ctypes.byref(cache.c), ctypes.byref(a), _ptr(workspace),
                                       workspace.numel(), _stream(stream)))


def dllm_fp8_quantize_weight(w: torch.Tensor, codes: torch.Tensor, scales: torch.Tensor,
                             stream=None):
    """w [N, K] bf16 -> codes [N, K] uint8, scales [N / 128, K / 128] fp32."""
    N, K = w.shape
    _expect(w, "w", (N, K), torch.bfloat16)
    _expect(codes, "codes", (N, K), torch.uint8)
    _expect(scales, "scales", (N // 128, K // 128), torch.float32)
    _check(lib.dllm_fp8_quantize_weight(_ptr(w), N, K, _ptr(codes), _ptr(scales),
                                        _stream(stream)))


def dllm_fp8_quantize_activations(x: torch.Tensor, codes: torch.Tensor, scales_t: torch.Tensor,
                                  stream=None):
    """x [M, K] bf16 -> codes [M, K] uint8, scales_t [K / 128, pitch] fp32 (pitch >= M)."""
    M, K = x.shape
    _expect(x, "x", (M, K), torch.bfloat16)
    _expect(codes, "codes", (M, K), torch.uint8)
    pitch = scales_t.shape[-1]
    _expect(scales_t, "scales_t", (K // 128, pitch), torch.float32)
    _check(lib.dllm_fp8_quantize_activations(_ptr(x), M, K, _ptr(codes), _ptr(scales_t), pitch,
                                             _stream(stream)))


def dllm_fp8_linear_workspace_bytes(M: int, N: int, K: int) -> int:
    return lib.dllm_fp8_linear_workspace_bytes(M, N, K)


def dllm_fp8_linear(x: torch.Tensor, w_codes: torch.Tensor, w_scales: torch.Tensor,
                    y: torch.Tensor, workspace=None, stream=None):
    """x [M, K] bf16, w_codes [N, K] uint8, w_scales [N / 128, K / 128] fp32, y [M, N] bf16."""
    M, K = x.shape
    N = w_codes.shape[0]
    _expect(x, "x", (M, K), torch.bfloat16)
    _expect(w_codes, "w_codes", (N, K), torch.uint8)
    _expect(w_scales, "w_scales", (N // 128, K // 128), torch.float32)
    _expect(y, "y", (M, N), torch.bfloat16)
    if workspace is None:
        need = dllm_fp8_linear_workspace_bytes(M, N, K)
        workspace = _scratch(max(1, need), x.device, stream)
    _check(lib.dllm_fp8_linear(_ptr(x), M, K, _ptr(w_codes), _ptr(w_scales), N, _ptr(y),
                               _ptr(workspace), workspace.numel(), _stream(stream)))


def dllm_rope_rows(y: torch.Tensor, heads: int, head_dim: int, pos: torch.Tensor,
                   rope_base: float, stream=None):
    """y [M, ld] bf16 (rotated in place), pos [M] int32."""
    M, ld = y.shape
    _expect(y, "y", (M, ld), torch.bfloat16)
    _expect(pos, "pos", (M,), torch.int32)
    _check(lib.dllm_rope_rows(_ptr(y), M, ld, heads, head_dim, _ptr(pos), float(rope_base),
                              _stream(stream)))


def dllm_scatter_kv_rows(cache: Cache, y: torch.Tensor, k_col: int, v_col: int,
                         refresh_idx: torch.Tensor, stream=None):
    """y [B * n, ld] bf16, refresh_idx [B, n] int32."""
    d = cache.desc
    n = refresh_idx.shape[1]
    _expect(refresh_idx, "refresh_idx", (d.batch, n), torch.int32)
    _expect(y, "y", (d.batch * n, y.shape[1]), torch.bfloat16)
    _check(lib.dllm_scatter_kv_rows(ctypes.byref(cache.c), _ptr(y), y.shape[1], k_col, v_col,
                                    _ptr(refresh_idx), n, _stream(stream)))


def dllm_mfma_rate_probe(kind: int, tile: int, workgroups: int, iters: int, out: torch.Tensor,
                         stream=None):
    """out [workgroups * 4] fp32; tile 16 or 32."""
    _expect(out, "out", (workgroups * 4,), torch.float32)
    _check(lib.dllm_mfma_rate_probe(kind, tile, workgroups, iters, _ptr(out), _stream(stream)))


def dllm_read_rate_probe(buf: torch.Tensor, workgroups: int, out: torch.Tensor, stream=None):
    """Reads every byte of the contiguous device tensor buf once; out [workgroups] int32 gets
    the XOR of the 32-bit words each workgroup read."""
    if not buf.is_contiguous() or buf.device.type != "cuda":
        raise DllmError(DLLM_EINVAL, "buf: expected a contiguous cuda tensor")
    _expect(out, "out", (workgroups,), torch.int32)
    _check(lib.dllm_read_rate_probe(_ptr(buf), buf.numel() * buf.element_size(), workgroups,
                                    _ptr(out), _stream(stream)))


def dllm_fp8_e4m3_roundtrip(x: torch.Tensor, scale: float, codes: torch.Tensor,
                            decoded=None, stream=None):
    _expect(x, "x", tuple(x.shape), torch.float32)
    _expect(codes, "codes", tuple(x.shape), torch.uint8)
    if decoded is not None:
        _expect(decoded, "decoded", tuple(x.shape), torch.float32)
    _check(lib.dllm_fp8_e4m3_roundtrip(_ptr(x), x.numel(), float(scale), _ptr(codes),
                                       _ptr(decoded), _stream(stream)))


def dllm_set_options(flags: int) -> int:
    """Replace the process-wide DLLM_OPT_* switches; returns the previous value."""
    return lib.dllm_set_options(int(flags))


def dllm_last_error() -> str:
    return lib.dllm_last_error().decode()
