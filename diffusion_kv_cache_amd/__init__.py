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
           "dllm_block_attention", "dllm_drift_check", "dllm_fp8_e4m3_roundtrip",
           "dllm_last_error")

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
    lib.dllm_drift_check.restype = i32
    lib.dllm_drift_check.argtypes = [ctypes.POINTER(CCache), i32, i32, ctypes.c_float, P, P, P, P,
                                     P, P]
    lib.dllm_fp8_e4m3_roundtrip.restype = i32
    lib.dllm_fp8_e4m3_roundtrip.argtypes = [P, i64, ctypes.c_float, P, P, P]
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
        workspace = torch.empty(need, dtype=torch.uint8, device=hidden.device) if need else None
    ws_bytes = 0 if workspace is None else workspace.numel()
    _check(lib.dllm_refresh_qkv_rope_scatter(
        ctypes.byref(cache.c), _ptr(hidden), H, act, _ptr(refresh_idx), n,
        _ptr(w_qkv), num_q_heads, float(rope_base), _ptr(q_out), _ptr(workspace), ws_bytes,
        _stream(stream)))


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
        workspace = torch.empty(max(1, dllm_attention_workspace_bytes(cache, num_q_heads, n)),
                                dtype=torch.uint8, device=q.device)
    _check(lib.dllm_block_attention(
        ctypes.byref(cache.c), _ptr(q), act, num_q_heads, n, float(softmax_scale), _ptr(out),
        _ptr(lse), _ptr(attn_mass), _ptr(workspace), workspace.numel(), _stream(stream)))


def dllm_drift_check(cache: Cache, num_q_heads: int, k: int, gamma: float,
                     track_idx: torch.Tensor, track_buf: torch.Tensor, attn_mass, sigma_out,
                     refresh_out, stream=None):
    """track_idx [B,Hq,k] int32 (in/out), track_buf [B,Hq,k,2,D] cache dtype (in/out),
    attn_mass [B,Hq,S] fp32 or None, sigma_out [B,Hq] fp32, refresh_out [B] uint8."""
    d = cache.desc
    B, Hq = d.batch, num_q_heads
    _expect(track_idx, "track_idx", (B, Hq, k), torch.int32)
    _expect(track_buf, "track_buf", (B, Hq, k, 2, d.head_dim), _TORCH_DTYPE[d.kv_dtype])
    if attn_mass is not None:
        _expect(attn_mass, "attn_mass", (B, Hq, d.max_seq), torch.float32)
    _expect(sigma_out, "sigma_out", (B, Hq), torch.float32)
    _expect(refresh_out, "refresh_out", (B,), torch.uint8)
    _check(lib.dllm_drift_check(
        ctypes.byref(cache.c), num_q_heads, k, float(gamma), _ptr(track_idx), _ptr(track_buf),
        _ptr(attn_mass), _ptr(sigma_out), _ptr(refresh_out), _stream(stream)))


def dllm_fp8_e4m3_roundtrip(x: torch.Tensor, scale: float, codes: torch.Tensor,
                            decoded=None, stream=None):
    _expect(x, "x", tuple(x.shape), torch.float32)
    _expect(codes, "codes", tuple(x.shape), torch.uint8)
    if decoded is not None:
        _expect(decoded, "decoded", tuple(x.shape), torch.float32)
    _check(lib.dllm_fp8_e4m3_roundtrip(_ptr(x), x.numel(), float(scale), _ptr(codes),
                                       _ptr(decoded), _stream(stream)))


def dllm_last_error() -> str:
    return lib.dllm_last_error().decode()
