"""Paged-attention decode for MI355X (gfx950): Python binding of libpagedkv.so.

Argument marshalling only: every operation runs in the library's HIP kernels,
on torch's current HIP stream unless ``stream`` is given.  Functions mirror
the C entry points of include/pagedkv.h without the ``pkv_`` prefix.  There is
no CPU fallback: if the library is missing or cannot be loaded, every call
raises.

Tensors are torch tensors on the GPU, contiguous, with these dtypes:

* q / key / value / out: float32, float16 or bfloat16;
* k_cache / v_cache: the same dtype as q, or uint8 (or float8_e4m3fn) holding
  OCP E4M3FN bytes, or int8, with one fp32 scale per pool;
* slot_mapping, block_tables, context_lens, pairs, cu_lens: int32.

8-bit pools take ``k_scale`` / ``v_scale`` as one number per pool, or as one
scale per head: a float32 device tensor of H values (or a host array, which
is copied to the device on the current stream), which routes the call to the
library's ``*_head_scales`` entry point.
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional

import numpy as np
import torch

_PKG_DIR = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG_DIR, "libpagedkv.so")

PKV_OK, PKV_ERR_INVALID_ARG, PKV_ERR_UNSUPPORTED, PKV_ERR_WORKSPACE, PKV_ERR_HIP, PKV_ERR_DEVICE_CHECK = range(6)
# bits of the mask pkv_check_step_inputs reports (pkv_check_bit)
(PKV_CHECK_CONTEXT_LEN, PKV_CHECK_BLOCK_ID, PKV_CHECK_SLOT_RANGE, PKV_CHECK_SLOT_DUP, PKV_CHECK_PAIR_RANGE,
 PKV_CHECK_PAIR_OVERLAP, PKV_CHECK_APPEND_SLOT, PKV_CHECK_SHARED_WRITE) = (1 << i for i in range(8))
PKV_F32, PKV_F16, PKV_BF16, PKV_FP8_E4M3, PKV_INT8 = range(5)

_DTYPE_CODE = {torch.float32: PKV_F32, torch.float16: PKV_F16, torch.bfloat16: PKV_BF16,
               torch.uint8: PKV_FP8_E4M3, torch.float8_e4m3fn: PKV_FP8_E4M3, torch.int8: PKV_INT8}

EXPORTS = ("pkv_status_string", "pkv_version", "pkv_reshape_and_cache", "pkv_reshape_and_cache_head_scales",
           "pkv_decode_workspace_bytes",
           "pkv_paged_attention_decode_head_scales",
           "pkv_paged_attention_decode_partitions_head_scales", "pkv_paged_attention_decode_merge_head_scales",
           "pkv_paged_attention_decode_append_head_scales", "pkv_paged_attention_decode_append_partitions_head_scales",
           "pkv_paged_attention_prefill_head_scales", "pkv_paged_attention_prefill_append_head_scales",
           "pkv_paged_attention_decode", "pkv_paged_attention_decode_static", "pkv_paged_attention_decode_partitions",
           "pkv_paged_attention_decode_grouped", "pkv_paged_attention_decode_grouped_partitions",
           "pkv_paged_attention_decode_merge",
           "pkv_paged_attention_decode_append", "pkv_paged_attention_decode_append_partitions",
           "pkv_paged_attention_prefill", "pkv_paged_attention_prefill_append", "pkv_copy_blocks", "pkv_swap_blocks", "pkv_gather_kv", "pkv_decode_graph_create",
           "pkv_decode_graph_launch", "pkv_decode_graph_destroy", "pkv_stream_read", "pkv_check_workspace_bytes",
           "pkv_check_step_inputs")


class PagedKVError(RuntimeError):
    """A libpagedkv call returned a non-OK status."""

    def __init__(self, func: str, status: int):
        self.status = status
        super().__init__(f"{func}: {status_string(status)} (status {status})")


_lib_handle: Optional[ctypes.CDLL] = None


class _DecodeStep(ctypes.Structure):
    """Mirror of pkv_decode_step (include/pagedkv.h)."""
    _fields_ = [("k_cache", ctypes.c_void_p), ("v_cache", ctypes.c_void_p), ("key", ctypes.c_void_p),
                ("value", ctypes.c_void_p), ("slot_mapping", ctypes.c_void_p), ("copy_pairs", ctypes.c_void_p),
                ("num_pairs", ctypes.c_int32), ("q", ctypes.c_void_p), ("out", ctypes.c_void_p),
                ("block_tables", ctypes.c_void_p), ("context_lens", ctypes.c_void_p), ("workspace", ctypes.c_void_p),
                ("workspace_bytes", ctypes.c_size_t), ("S", ctypes.c_int32), ("H", ctypes.c_int32),
                ("D", ctypes.c_int32), ("BS", ctypes.c_int32), ("MB", ctypes.c_int32), ("NB", ctypes.c_int32),
                ("scale", ctypes.c_float), ("k_scale", ctypes.c_float), ("v_scale", ctypes.c_float),
                ("q_dtype", ctypes.c_int), ("cache_dtype", ctypes.c_int), ("append", ctypes.c_int32),
                ("k_scales", ctypes.c_void_p), ("v_scales", ctypes.c_void_p)]


def _declare(lib: ctypes.CDLL) -> None:
    vp, i32, f32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_float, ctypes.c_size_t
    lib.pkv_status_string.argtypes = [ctypes.c_int]
    lib.pkv_status_string.restype = ctypes.c_char_p
    lib.pkv_version.argtypes = []
    lib.pkv_version.restype = ctypes.c_int
    lib.pkv_reshape_and_cache.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, ctypes.c_int,
                                          ctypes.c_int, f32, f32, vp]
    lib.pkv_reshape_and_cache.restype = ctypes.c_int
    lib.pkv_reshape_and_cache_head_scales.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, ctypes.c_int,
                                                      ctypes.c_int, vp, vp, vp]
    lib.pkv_reshape_and_cache_head_scales.restype = ctypes.c_int
    for name in ("pkv_paged_attention_decode_head_scales", "pkv_paged_attention_decode_partitions_head_scales"):
        fn = getattr(lib, name)
        fn.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, f32, ctypes.c_int, ctypes.c_int, vp, vp,
                       vp, sz, vp]
        fn.restype = ctypes.c_int
    lib.pkv_paged_attention_decode_merge_head_scales.argtypes = [vp, vp, i32, i32, i32, i32, i32, ctypes.c_int,
                                                                 ctypes.c_int, vp, vp, sz, vp]
    lib.pkv_paged_attention_decode_merge_head_scales.restype = ctypes.c_int
    for name in ("pkv_paged_attention_decode_append_head_scales",
                 "pkv_paged_attention_decode_append_partitions_head_scales"):
        fn = getattr(lib, name)
        fn.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, f32, ctypes.c_int,
                       ctypes.c_int, vp, vp, vp, sz, vp]
        fn.restype = ctypes.c_int
    lib.pkv_paged_attention_prefill_head_scales.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32,
                                                            i32, i32, f32, ctypes.c_int, ctypes.c_int, vp, vp, vp]
    lib.pkv_paged_attention_prefill_head_scales.restype = ctypes.c_int
    lib.pkv_paged_attention_prefill_append_head_scales.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, i32, i32,
                                                                   i32, i32, i32, i32, i32, i32, f32, ctypes.c_int,
                                                                   ctypes.c_int, vp, vp, vp]
    lib.pkv_paged_attention_prefill_append_head_scales.restype = ctypes.c_int
    lib.pkv_decode_workspace_bytes.argtypes = [i32, i32, i32, i32, i32]
    lib.pkv_decode_workspace_bytes.restype = sz
    for name in ("pkv_paged_attention_decode", "pkv_paged_attention_decode_partitions"):
        fn = getattr(lib, name)
        fn.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, f32, ctypes.c_int, ctypes.c_int, f32, f32,
                       vp, sz, vp]
        fn.restype = ctypes.c_int
    lib.pkv_paged_attention_decode_static.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, f32,
                                                      ctypes.c_int, ctypes.c_int, f32, f32, vp]
    lib.pkv_paged_attention_decode_static.restype = ctypes.c_int
    for name in ("pkv_paged_attention_decode_grouped", "pkv_paged_attention_decode_grouped_partitions"):
        fn = getattr(lib, name)
        fn.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, f32, ctypes.c_int,
                       ctypes.c_int, i32, vp, sz, vp]
        fn.restype = ctypes.c_int
    lib.pkv_paged_attention_decode_merge.argtypes = [vp, vp, i32, i32, i32, i32, i32, ctypes.c_int, ctypes.c_int, f32,
                                                     vp, sz, vp]
    lib.pkv_paged_attention_decode_merge.restype = ctypes.c_int
    for name in ("pkv_paged_attention_decode_append", "pkv_paged_attention_decode_append_partitions"):
        fn = getattr(lib, name)
        fn.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, f32, ctypes.c_int,
                       ctypes.c_int, f32, f32, vp, sz, vp]
        fn.restype = ctypes.c_int
    lib.pkv_paged_attention_prefill.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32, i32,
                                                f32, ctypes.c_int, ctypes.c_int, f32, f32, vp]
    lib.pkv_paged_attention_prefill.restype = ctypes.c_int
    lib.pkv_paged_attention_prefill_append.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32,
                                                       i32, i32, i32, f32, ctypes.c_int, ctypes.c_int, f32, f32, vp]
    lib.pkv_paged_attention_prefill_append.restype = ctypes.c_int
    lib.pkv_copy_blocks.argtypes = [vp, vp, vp, i32, i32, i32, i32, i32, ctypes.c_int, vp]
    lib.pkv_copy_blocks.restype = ctypes.c_int
    lib.pkv_swap_blocks.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, ctypes.c_int, vp]
    lib.pkv_swap_blocks.restype = ctypes.c_int
    lib.pkv_gather_kv.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, ctypes.c_int, vp]
    lib.pkv_gather_kv.restype = ctypes.c_int
    lib.pkv_decode_graph_create.argtypes = [ctypes.POINTER(_DecodeStep), ctypes.POINTER(ctypes.c_void_p)]
    lib.pkv_decode_graph_create.restype = ctypes.c_int
    lib.pkv_decode_graph_launch.argtypes = [vp, vp]
    lib.pkv_decode_graph_launch.restype = ctypes.c_int
    lib.pkv_decode_graph_destroy.argtypes = [vp]
    lib.pkv_decode_graph_destroy.restype = ctypes.c_int
    lib.pkv_stream_read.argtypes = [vp, sz, vp, vp]
    lib.pkv_stream_read.restype = ctypes.c_int
    lib.pkv_check_workspace_bytes.argtypes = [i32, i32]
    lib.pkv_check_workspace_bytes.restype = sz
    lib.pkv_check_step_inputs.argtypes = [vp, vp, i32, i32, vp, i32, vp, i32, i32, i32, i32, vp, sz,
                                          ctypes.POINTER(ctypes.c_uint32), vp]
    lib.pkv_check_step_inputs.restype = ctypes.c_int


def lib() -> ctypes.CDLL:
    """The loaded libpagedkv.so; raises if it has not been built."""
    global _lib_handle
    if _lib_handle is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m paged_kv_cache_423_amd.build` "
                               "(there is no fallback path)")
        handle = ctypes.CDLL(LIB_PATH)
        _declare(handle)
        _lib_handle = handle
    return _lib_handle


def loaded_path() -> str:
    lib()
    return LIB_PATH


def status_string(status: int) -> str:
    return lib().pkv_status_string(int(status)).decode()


def version() -> int:
    return int(lib().pkv_version())


# ------------------------------------------------------------------ helpers

def _ptr(t: Optional[torch.Tensor]):
    # a plain int: every entry point declares its pointer arguments c_void_p
    return None if t is None else t.data_ptr()


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _dev(name: str, t: torch.Tensor, dtype=None, ndim=None) -> None:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on the GPU (got {t.device})")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype} (got {t.dtype})")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dimensions (got {t.dim()})")


def _code(name: str, t: torch.Tensor) -> int:
    if t.dtype not in _DTYPE_CODE:
        raise ValueError(f"{name}: unsupported dtype {t.dtype}")
    return _DTYPE_CODE[t.dtype]


def _check(func: str, status: int) -> None:
    if status != PKV_OK:
        raise PagedKVError(func, status)


class PreparedCall:
    """One library call with its arguments checked and marshalled once.

    Calling it launches the same kernels again on the same buffers, whose
    contents may change between calls (slots, tables, lengths, new tokens),
    on the stream fixed when it was prepared (the one given, else the
    current one then).  It holds references to the tensors it was built
    from, so that their memory outlives it.  The functions that accept
    ``prepare=True`` return one instead of calling."""

    __slots__ = ("_fn", "_args", "_name", "_keep")

    def __init__(self, name: str, args, keep):
        self._fn = getattr(lib(), name)
        self._args = tuple(args)
        self._name = name
        self._keep = keep

    def __call__(self) -> None:
        st = self._fn(*self._args)
        if st != PKV_OK:
            raise PagedKVError(self._name, st)


def _invoke(name: str, args, prepare: bool, keep):
    """Call ``name`` with ``args`` now, or return it as a PreparedCall."""
    if prepare:
        return PreparedCall(name, args, keep)
    _check(name, getattr(lib(), name)(*args))
    return None


def _is_per_head(x) -> bool:
    if isinstance(x, (float, int)):
        return False
    return (isinstance(x, torch.Tensor) and x.dim() == 1) or (not isinstance(x, torch.Tensor) and np.ndim(x) == 1)


def _head_scales(k_scale, v_scale, H: int, device, stream):
    """None for per-pool scales (two numbers); else the per-head scales as two
    contiguous float32 [H] tensors on ``device``.  Host arrays are copied on
    the current stream, so they are refused when the call names another."""
    per_head = (_is_per_head(k_scale), _is_per_head(v_scale))
    if not any(per_head):
        return None
    if not all(per_head):
        raise ValueError("k_scale and v_scale must both be per-pool numbers or both per-head arrays")
    out = []
    for name, x in (("k_scale", k_scale), ("v_scale", v_scale)):
        if not isinstance(x, torch.Tensor) or x.device.type != "cuda":
            if stream is not None:
                raise ValueError(f"{name}: pass per-head scales as a device tensor when giving a stream")
            x = torch.as_tensor(np.asarray(x, dtype=np.float32), device=device)
        if x.dtype != torch.float32 or x.shape != (H,) or x.device != torch.device(device):
            raise ValueError(f"{name}: per-head scales must be float32 [{H}] on {device}")
        out.append(x.contiguous())
    return out


# ------------------------------------------------------------------ API

def reshape_and_cache(key: torch.Tensor, value: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                      slot_mapping: torch.Tensor, k_scale: float = 1.0, v_scale: float = 1.0, *,
                      stream=None, prepare: bool = False) -> Optional[PreparedCall]:
    """Write key/value [T, H, D] into the pools [NB, H, BS, D] at slot_mapping [T]
    (slot = block * BS + offset; negative = skip).  8-bit pools store
    E4M3(x / scale) or INT8(x / scale), with the pool's or the head's scale."""
    for n, t in (("key", key), ("value", value)):
        _dev(n, t, ndim=3)
    for n, t in (("k_cache", k_cache), ("v_cache", v_cache)):
        _dev(n, t, ndim=4)
    _dev("slot_mapping", slot_mapping, torch.int32, 1)
    T, H, D = key.shape
    NB, Hc, BS, Dc = k_cache.shape
    if value.shape != key.shape or v_cache.shape != k_cache.shape or (Hc, Dc) != (H, D) \
            or slot_mapping.shape[0] != T or value.dtype != key.dtype or v_cache.dtype != k_cache.dtype:
        raise ValueError("reshape_and_cache: shapes or dtypes disagree")
    hs = _head_scales(k_scale, v_scale, H, key.device, stream)
    keep = (key, value, k_cache, v_cache, slot_mapping, hs)
    if hs is not None:
        return _invoke("pkv_reshape_and_cache_head_scales",
                       (_ptr(key), _ptr(value), _ptr(k_cache), _ptr(v_cache), _ptr(slot_mapping), T, H, D, BS, NB,
                        _code("key", key), _code("k_cache", k_cache), _ptr(hs[0]), _ptr(hs[1]), _stream(stream)),
                       prepare, keep)
    return _invoke("pkv_reshape_and_cache",
                   (_ptr(key), _ptr(value), _ptr(k_cache), _ptr(v_cache), _ptr(slot_mapping), T, H, D, BS, NB,
                    _code("key", key), _code("k_cache", k_cache), float(k_scale), float(v_scale), _stream(stream)),
                   prepare, keep)


_WS_BYTES = {}


def decode_workspace_bytes(S: int, H: int, D: int, BS: int, MB: int) -> int:
    key = (int(S), int(H), int(D), int(BS), int(MB))
    n = _WS_BYTES.get(key)
    if n is None:
        n = _WS_BYTES[key] = int(lib().pkv_decode_workspace_bytes(*key))
    return n


def alloc_decode_workspace(S: int, H: int, D: int, BS: int, MB: int, device="cuda") -> Optional[torch.Tensor]:
    """A device buffer big enough for paged_attention_decode (None if none is needed)."""
    nbytes = decode_workspace_bytes(S, H, D, BS, MB)
    return torch.empty(nbytes, dtype=torch.uint8, device=device) if nbytes else None


def _decode_args(out, q, k_cache, v_cache, block_tables, context_lens, workspace):
    _dev("out", out, q.dtype, 3)
    _dev("q", q, ndim=3)
    for n, t in (("k_cache", k_cache), ("v_cache", v_cache)):
        _dev(n, t, ndim=4)
    _dev("block_tables", block_tables, torch.int32, 2)
    _dev("context_lens", context_lens, torch.int32, 1)
    S, H, D = q.shape
    NB, Hc, BS, Dc = k_cache.shape
    MB = block_tables.shape[1]
    if out.shape != q.shape or v_cache.shape != k_cache.shape or (Hc, Dc) != (H, D) \
            or block_tables.shape[0] != S or context_lens.shape[0] != S or v_cache.dtype != k_cache.dtype:
        raise ValueError("paged_attention_decode: shapes or dtypes disagree")
    need = decode_workspace_bytes(S, H, D, BS, MB)
    if need and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    if workspace is not None:
        _dev("workspace", workspace)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    return S, H, D, BS, MB, NB, workspace, ws_bytes


def paged_attention_decode(out: torch.Tensor, q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                           block_tables: torch.Tensor, context_lens: torch.Tensor, scale: float,
                           k_scale: float = 1.0, v_scale: float = 1.0, *, workspace: Optional[torch.Tensor] = None,
                           stream=None, prepare: bool = False):
    """out[s, h] = softmax(scale * q[s, h] . K_s^T) V_s over the n_s = context_lens[s]
    tokens that block_tables[s] maps; returns ``out`` (a PreparedCall with
    ``prepare=True``)."""
    S, H, D, BS, MB, NB, workspace, ws_bytes = _decode_args(out, q, k_cache, v_cache, block_tables, context_lens,
                                                            workspace)
    hs = _head_scales(k_scale, v_scale, H, q.device, stream)
    keep = (out, q, k_cache, v_cache, block_tables, context_lens, workspace, hs)
    if hs is not None:
        call = _invoke("pkv_paged_attention_decode_head_scales",
                       (_ptr(out), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_tables), _ptr(context_lens), S,
                        H, D, BS, MB, NB, float(scale), _code("q", q), _code("k_cache", k_cache), _ptr(hs[0]),
                        _ptr(hs[1]), _ptr(workspace), ws_bytes, _stream(stream)), prepare, keep)
    else:
        call = _invoke("pkv_paged_attention_decode",
                       (_ptr(out), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_tables), _ptr(context_lens), S,
                        H, D, BS, MB, NB, float(scale), _code("q", q), _code("k_cache", k_cache), float(k_scale),
                        float(v_scale), _ptr(workspace), ws_bytes, _stream(stream)), prepare, keep)
    return call if prepare else out


# bytes of the decode workspace paged_attention_decode_static holds on each GPU
STATIC_WORKSPACE_BYTES = 16 << 20


def paged_attention_decode_static(out: torch.Tensor, q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                                  block_tables: torch.Tensor, context_lens: torch.Tensor, scale: float,
                                  k_scale: float = 1.0, v_scale: float = 1.0, *, stream=None) -> torch.Tensor:
    """paged_attention_decode without a caller workspace and without any
    allocation: the partition partials go to a buffer of
    STATIC_WORKSPACE_BYTES the library holds on each GPU (larger needs raise
    PKV_ERR_WORKSPACE).  Calls that overlap on one GPU race; calls ordered
    on one stream do not.  Returns ``out``."""
    _dev("out", out, q.dtype, 3)
    _dev("q", q, ndim=3)
    for n, t in (("k_cache", k_cache), ("v_cache", v_cache)):
        _dev(n, t, ndim=4)
    _dev("block_tables", block_tables, torch.int32, 2)
    _dev("context_lens", context_lens, torch.int32, 1)
    S, H, D = q.shape
    NB, Hc, BS, Dc = k_cache.shape
    MB = block_tables.shape[1]
    if out.shape != q.shape or v_cache.shape != k_cache.shape or (Hc, Dc) != (H, D) \
            or block_tables.shape[0] != S or context_lens.shape[0] != S or v_cache.dtype != k_cache.dtype:
        raise ValueError("paged_attention_decode_static: shapes or dtypes disagree")
    st = lib().pkv_paged_attention_decode_static(_ptr(out), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_tables),
                                                 _ptr(context_lens), S, H, D, BS, MB, NB, float(scale), _code("q", q),
                                                 _code("k_cache", k_cache), float(k_scale), float(v_scale),
                                                 _stream(stream))
    _check("pkv_paged_attention_decode_static", st)
    return out


def _grouped_call(func, out, q, k_cache, v_cache, block_tables, context_lens, scale, group_size, key, value,
                  slot_mapping, workspace, stream, prepare=False):
    S, H, D, BS, MB, NB, workspace, ws_bytes = _decode_args(out, q, k_cache, v_cache, block_tables, context_lens,
                                                            workspace)
    given = [t is not None for t in (key, value, slot_mapping)]
    if any(given) and not all(given):
        raise ValueError(f"{func}: give key, value and slot_mapping together (or none)")
    if all(given):
        for n, t in (("key", key), ("value", value)):
            _dev(n, t, q.dtype, 3)
        _dev("slot_mapping", slot_mapping, torch.int32, 1)
        if key.shape != q.shape or value.shape != q.shape or slot_mapping.shape[0] != S:
            raise ValueError(f"{func}: key, value and slot_mapping must hold one token per sequence")
    keep = (out, q, key, value, k_cache, v_cache, slot_mapping, block_tables, context_lens, workspace)
    return _invoke(func, (_ptr(out), _ptr(q), _ptr(key), _ptr(value), _ptr(k_cache), _ptr(v_cache),
                          _ptr(slot_mapping), _ptr(block_tables), _ptr(context_lens), S, H, D, BS, MB, NB,
                          float(scale), _code("q", q), _code("k_cache", k_cache), int(group_size), _ptr(workspace),
                          ws_bytes, _stream(stream)), prepare, keep)


def paged_attention_decode_grouped(out, q, k_cache, v_cache, block_tables, context_lens, scale: float,
                                   group_size: int, *, key=None, value=None, slot_mapping=None,
                                   workspace: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """paged_attention_decode (with key / value / slot_mapping:
    paged_attention_decode_append) for a batch whose sequences come in groups
    of ``group_size`` consecutive ones that may share blocks: a block every
    sequence of a group maps is read once per chunk of at most four of them
    (with key / value / slot_mapping the same kernel stores the step's
    tokens).  Bitwise equal to
    the per-sequence decode; 16-bit and f32 pools.  Returns ``out``."""
    _grouped_call("pkv_paged_attention_decode_grouped", out, q, k_cache, v_cache, block_tables, context_lens, scale,
                  group_size, key, value, slot_mapping, workspace, stream)
    return out


def paged_attention_decode_grouped_partitions(out, q, k_cache, v_cache, block_tables, context_lens, scale: float,
                                              group_size: int, *, key=None, value=None, slot_mapping=None,
                                              workspace: Optional[torch.Tensor] = None, stream=None,
                                              prepare: bool = False) -> Optional[PreparedCall]:
    """First phase of paged_attention_decode_grouped (paged_attention_decode_merge completes it)."""
    return _grouped_call("pkv_paged_attention_decode_grouped_partitions", out, q, k_cache, v_cache, block_tables,
                         context_lens, scale, group_size, key, value, slot_mapping, workspace, stream, prepare)


def paged_attention_decode_partitions(out, q, k_cache, v_cache, block_tables, context_lens, scale: float,
                                      k_scale: float = 1.0, v_scale: float = 1.0, *, workspace: torch.Tensor,
                                      stream=None, prepare: bool = False) -> Optional[PreparedCall]:
    """First phase of the decode (see paged_attention_decode_merge)."""
    S, H, D, BS, MB, NB, workspace, ws_bytes = _decode_args(out, q, k_cache, v_cache, block_tables, context_lens,
                                                            workspace)
    hs = _head_scales(k_scale, v_scale, H, q.device, stream)
    keep = (out, q, k_cache, v_cache, block_tables, context_lens, workspace, hs)
    if hs is not None:
        return _invoke("pkv_paged_attention_decode_partitions_head_scales",
                       (_ptr(out), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_tables), _ptr(context_lens), S,
                        H, D, BS, MB, NB, float(scale), _code("q", q), _code("k_cache", k_cache), _ptr(hs[0]),
                        _ptr(hs[1]), _ptr(workspace), ws_bytes, _stream(stream)), prepare, keep)
    return _invoke("pkv_paged_attention_decode_partitions",
                   (_ptr(out), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_tables), _ptr(context_lens), S, H,
                    D, BS, MB, NB, float(scale), _code("q", q), _code("k_cache", k_cache), float(k_scale),
                    float(v_scale), _ptr(workspace), ws_bytes, _stream(stream)), prepare, keep)


def _append_call(func, out, q, key, value, k_cache, v_cache, slot_mapping, block_tables, context_lens, scale,
                 k_scale, v_scale, workspace, stream, prepare=False):
    S, H, D, BS, MB, NB, workspace, ws_bytes = _decode_args(out, q, k_cache, v_cache, block_tables, context_lens,
                                                            workspace)
    for n, t in (("key", key), ("value", value)):
        _dev(n, t, q.dtype, 3)
    _dev("slot_mapping", slot_mapping, torch.int32, 1)
    if key.shape != q.shape or value.shape != q.shape or slot_mapping.shape[0] != S:
        raise ValueError(f"{func}: key, value and slot_mapping must hold one token per sequence")
    hs = _head_scales(k_scale, v_scale, H, q.device, stream)
    if hs is not None:
        func += "_head_scales"
        ks, vs = _ptr(hs[0]), _ptr(hs[1])
    else:
        ks, vs = float(k_scale), float(v_scale)
    keep = (out, q, key, value, k_cache, v_cache, slot_mapping, block_tables, context_lens, workspace, hs)
    return _invoke(func, (_ptr(out), _ptr(q), _ptr(key), _ptr(value), _ptr(k_cache), _ptr(v_cache),
                          _ptr(slot_mapping), _ptr(block_tables), _ptr(context_lens), S, H, D, BS, MB, NB,
                          float(scale), _code("q", q), _code("k_cache", k_cache), ks, vs, _ptr(workspace), ws_bytes,
                          _stream(stream)), prepare, keep)


def paged_attention_decode_append(out, q, key, value, k_cache, v_cache, slot_mapping, block_tables, context_lens,
                                  scale: float, k_scale: float = 1.0, v_scale: float = 1.0, *,
                                  workspace: Optional[torch.Tensor] = None, stream=None, prepare: bool = False):
    """A decode step's cache write and decode in one pass: key/value [S, H, D]
    (one new token per sequence, at slot_mapping[s], the slot of position
    context_lens[s] - 1) go into the pools, then out = the decode over the
    updated pools.  Bitwise equal to reshape_and_cache followed by
    paged_attention_decode; returns ``out`` (a PreparedCall with
    ``prepare=True``)."""
    call = _append_call("pkv_paged_attention_decode_append", out, q, key, value, k_cache, v_cache, slot_mapping,
                        block_tables, context_lens, scale, k_scale, v_scale, workspace, stream, prepare)
    return call if prepare else out


def paged_attention_decode_append_partitions(out, q, key, value, k_cache, v_cache, slot_mapping, block_tables,
                                             context_lens, scale: float, k_scale: float = 1.0, v_scale: float = 1.0,
                                             *, workspace: Optional[torch.Tensor], stream=None,
                                             prepare: bool = False) -> Optional[PreparedCall]:
    """First phase of paged_attention_decode_append (paged_attention_decode_merge completes it)."""
    return _append_call("pkv_paged_attention_decode_append_partitions", out, q, key, value, k_cache, v_cache,
                        slot_mapping, block_tables, context_lens, scale, k_scale, v_scale, workspace, stream, prepare)


def paged_attention_decode_merge(out, context_lens, block_size: int, max_blocks_per_seq: int, cache_dtype,
                                 v_scale: float = 1.0, *, workspace: Optional[torch.Tensor], stream=None,
                                 prepare: bool = False):
    """Second phase: merge the partitions the first phase left in ``workspace``.
    ``cache_dtype`` is the pools' torch dtype; returns ``out`` (a PreparedCall
    with ``prepare=True``)."""
    _dev("out", out, ndim=3)
    _dev("context_lens", context_lens, torch.int32, 1)
    S, H, D = out.shape
    if workspace is not None:
        _dev("workspace", workspace)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    if _is_per_head(v_scale):
        vs = _head_scales(v_scale, v_scale, H, out.device, stream)[1]
        call = _invoke("pkv_paged_attention_decode_merge_head_scales",
                       (_ptr(out), _ptr(context_lens), S, H, D, int(block_size), int(max_blocks_per_seq),
                        _code("out", out), _DTYPE_CODE[cache_dtype], _ptr(vs), _ptr(workspace), ws_bytes,
                        _stream(stream)), prepare, (out, context_lens, vs, workspace))
    else:
        call = _invoke("pkv_paged_attention_decode_merge",
                       (_ptr(out), _ptr(context_lens), S, H, D, int(block_size), int(max_blocks_per_seq),
                        _code("out", out), _DTYPE_CODE[cache_dtype], float(v_scale), _ptr(workspace), ws_bytes,
                        _stream(stream)), prepare, (out, context_lens, workspace))
    return call if prepare else out


def paged_attention_prefill(out: torch.Tensor, q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                            block_tables: torch.Tensor, context_lens: torch.Tensor, cu_q_lens: torch.Tensor,
                            max_q_len: int, scale: float, k_scale: float = 1.0, v_scale: float = 1.0, *,
                            stream=None, prepare: bool = False):
    """Causal attention of each sequence's new tokens over its paged cache.

    q / out [Tq, H, D] (float16 or bfloat16) hold the new tokens of all
    sequences packed by ``cu_q_lens`` [S + 1]; new token i of sequence s sits
    at position context_lens[s] - q_s + i and sees positions up to its own.
    The pools hold q's dtype, or E4M3 (uint8) / INT8 (int8) bytes of value /
    scale with ``k_scale`` / ``v_scale``.  ``max_q_len`` is the largest q_s.
    Returns ``out`` (a PreparedCall with ``prepare=True``)."""
    _dev("out", out, q.dtype, 3)
    _dev("q", q, ndim=3)
    for n, t in (("k_cache", k_cache), ("v_cache", v_cache)):
        _dev(n, t, ndim=4)
    if v_cache.dtype != k_cache.dtype:
        raise ValueError("paged_attention_prefill: the pools' dtypes differ")
    _dev("block_tables", block_tables, torch.int32, 2)
    _dev("context_lens", context_lens, torch.int32, 1)
    _dev("cu_q_lens", cu_q_lens, torch.int32, 1)
    Tq, H, D = q.shape
    NB, Hc, BS, Dc = k_cache.shape
    S, MB = block_tables.shape
    if out.shape != q.shape or v_cache.shape != k_cache.shape or (Hc, Dc) != (H, D) \
            or context_lens.shape[0] != S or cu_q_lens.shape[0] != S + 1:
        raise ValueError("paged_attention_prefill: shapes disagree")
    hs = _head_scales(k_scale, v_scale, H, q.device, stream)
    keep = (out, q, k_cache, v_cache, block_tables, context_lens, cu_q_lens, hs)
    if hs is not None:
        call = _invoke("pkv_paged_attention_prefill_head_scales",
                       (_ptr(out), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_tables), _ptr(context_lens),
                        _ptr(cu_q_lens), S, Tq, int(max_q_len), H, D, BS, MB, NB, float(scale), _code("q", q),
                        _code("k_cache", k_cache), _ptr(hs[0]), _ptr(hs[1]), _stream(stream)), prepare, keep)
    else:
        call = _invoke("pkv_paged_attention_prefill",
                       (_ptr(out), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_tables), _ptr(context_lens),
                        _ptr(cu_q_lens), S, Tq, int(max_q_len), H, D, BS, MB, NB, float(scale), _code("q", q),
                        _code("k_cache", k_cache), float(k_scale), float(v_scale), _stream(stream)), prepare, keep)
    return call if prepare else out


def paged_attention_prefill_append(out, q, key, value, k_cache, v_cache, slot_mapping, block_tables, context_lens,
                                   cu_q_lens, max_q_len: int, scale: float, k_scale: float = 1.0,
                                   v_scale: float = 1.0, *, stream=None, prepare: bool = False):
    """A prompt step's cache write and prompt attention in one pass: key/value
    [Tq, H, D] (the new tokens, packed like q) go to slot_mapping [Tq] (the
    slots of their positions) and are attended with the cached context.
    Bitwise equal to reshape_and_cache followed by paged_attention_prefill;
    returns ``out`` (a PreparedCall with ``prepare=True``)."""
    _dev("out", out, q.dtype, 3)
    _dev("q", q, ndim=3)
    for n, t in (("key", key), ("value", value)):
        _dev(n, t, q.dtype, 3)
    for n, t in (("k_cache", k_cache), ("v_cache", v_cache)):
        _dev(n, t, ndim=4)
    if v_cache.dtype != k_cache.dtype:
        raise ValueError("paged_attention_prefill_append: the pools' dtypes differ")
    for n, t in (("slot_mapping", slot_mapping), ("context_lens", context_lens), ("cu_q_lens", cu_q_lens)):
        _dev(n, t, torch.int32, 1)
    _dev("block_tables", block_tables, torch.int32, 2)
    Tq, H, D = q.shape
    NB, Hc, BS, Dc = k_cache.shape
    S, MB = block_tables.shape
    if out.shape != q.shape or key.shape != q.shape or value.shape != q.shape or v_cache.shape != k_cache.shape \
            or (Hc, Dc) != (H, D) or slot_mapping.shape[0] != Tq or context_lens.shape[0] != S \
            or cu_q_lens.shape[0] != S + 1:
        raise ValueError("paged_attention_prefill_append: shapes disagree")
    hs = _head_scales(k_scale, v_scale, H, q.device, stream)
    func = "pkv_paged_attention_prefill_append" + ("_head_scales" if hs is not None else "")
    ks, vs = (_ptr(hs[0]), _ptr(hs[1])) if hs is not None else (float(k_scale), float(v_scale))
    keep = (out, q, key, value, k_cache, v_cache, slot_mapping, block_tables, context_lens, cu_q_lens, hs)
    call = _invoke(func, (_ptr(out), _ptr(q), _ptr(key), _ptr(value), _ptr(k_cache), _ptr(v_cache),
                          _ptr(slot_mapping), _ptr(block_tables), _ptr(context_lens), _ptr(cu_q_lens), S, Tq,
                          int(max_q_len), H, D, BS, MB, NB, float(scale), _code("q", q), _code("k_cache", k_cache),
                          ks, vs, _stream(stream)), prepare, keep)
    return call if prepare else out


def copy_blocks(k_cache: torch.Tensor, v_cache: torch.Tensor, pairs: torch.Tensor, *, stream=None,
                prepare: bool = False) -> Optional[PreparedCall]:
    """For each (src, dst) row of pairs [N, 2], block dst of both pools becomes a copy of block src."""
    for n, t in (("k_cache", k_cache), ("v_cache", v_cache)):
        _dev(n, t, ndim=4)
    _dev("pairs", pairs, torch.int32, 2)
    if pairs.shape[1] != 2 or v_cache.shape != k_cache.shape or v_cache.dtype != k_cache.dtype:
        raise ValueError("copy_blocks: pairs must be [N, 2] and the pools must match")
    NB, H, BS, D = k_cache.shape
    return _invoke("pkv_copy_blocks", (_ptr(k_cache), _ptr(v_cache), _ptr(pairs), pairs.shape[0], H, D, BS, NB,
                                       _code("k_cache", k_cache), _stream(stream)), prepare, (k_cache, v_cache, pairs))


def check_workspace_bytes(num_blocks: int, block_size: int) -> int:
    return int(lib().pkv_check_workspace_bytes(int(num_blocks), int(block_size)))


def check_step_inputs(block_tables: Optional[torch.Tensor], context_lens: Optional[torch.Tensor], block_size: int,
                      num_blocks: int, slot_mapping: Optional[torch.Tensor] = None,
                      pairs: Optional[torch.Tensor] = None, append: bool = False,
                      workspace: Optional[torch.Tensor] = None, *, stream=None) -> int:
    """Check one step's index inputs on the device; returns the violation mask
    (0 = well formed; bits PKV_CHECK_*).  Synchronises the stream.  A
    workspace of check_workspace_bytes(num_blocks, block_size) bytes is
    allocated through torch when none is given."""
    S, MB = 0, 1
    if block_tables is not None:
        _dev("block_tables", block_tables, torch.int32, 2)
        _dev("context_lens", context_lens, torch.int32, 1)
        S, MB = block_tables.shape
        if context_lens.shape[0] != S:
            raise ValueError("check_step_inputs: one context length per table row")
    T = 0
    if slot_mapping is not None:
        _dev("slot_mapping", slot_mapping, torch.int32, 1)
        T = slot_mapping.shape[0]
    N = 0
    if pairs is not None:
        _dev("pairs", pairs, torch.int32, 2)
        if pairs.shape[1] != 2:
            raise ValueError("check_step_inputs: pairs must be [N, 2]")
        N = pairs.shape[0]
    need = check_workspace_bytes(num_blocks, block_size)
    if workspace is None:
        dev = next(t.device for t in (block_tables, slot_mapping, pairs) if t is not None) \
            if any(t is not None for t in (block_tables, slot_mapping, pairs)) else torch.device("cuda")
        workspace = torch.empty(max(need, 4), dtype=torch.uint8, device=dev)
    _dev("workspace", workspace)
    mask = ctypes.c_uint32(0)
    st = lib().pkv_check_step_inputs(_ptr(block_tables), _ptr(context_lens), S, MB, _ptr(slot_mapping), T,
                                     _ptr(pairs), N, int(block_size), int(num_blocks), 1 if append else 0,
                                     _ptr(workspace), workspace.numel() * workspace.element_size(),
                                     ctypes.byref(mask), _stream(stream))
    if st not in (PKV_OK, PKV_ERR_DEVICE_CHECK):
        raise PagedKVError("pkv_check_step_inputs", st)
    return int(mask.value)


def swap_blocks(dst_k_cache: torch.Tensor, dst_v_cache: torch.Tensor, src_k_cache: torch.Tensor,
                src_v_cache: torch.Tensor, pairs: torch.Tensor, *, stream=None) -> None:
    """For each (src, dst) row of pairs [N, 2], block dst of the destination
    pools becomes a copy of block src of the source pools.  Either side may
    live in pinned host memory (``pin_memory=True``), the swap space; pairs
    may be on the GPU or pinned.  Synchronise the stream before reading a
    host destination."""
    for n, t in (("dst_k_cache", dst_k_cache), ("dst_v_cache", dst_v_cache), ("src_k_cache", src_k_cache),
                 ("src_v_cache", src_v_cache), ("pairs", pairs)):
        if not isinstance(t, torch.Tensor) or not t.is_contiguous():
            raise ValueError(f"{n} must be a contiguous torch.Tensor")
        if t.device.type != "cuda" and not t.is_pinned():
            raise ValueError(f"{n} must be on the GPU or in pinned host memory")
    if pairs.dtype != torch.int32 or pairs.dim() != 2 or pairs.shape[1] != 2:
        raise ValueError("pairs must be int32 [N, 2]")
    if dst_k_cache.shape != dst_v_cache.shape or src_k_cache.shape != src_v_cache.shape \
            or dst_k_cache.shape[1:] != src_k_cache.shape[1:] or dst_k_cache.dim() != 4 \
            or len({dst_k_cache.dtype, dst_v_cache.dtype, src_k_cache.dtype, src_v_cache.dtype}) != 1:
        raise ValueError("swap_blocks: pools differ in block shape or dtype")
    NBd, H, BS, D = dst_k_cache.shape
    NBs = src_k_cache.shape[0]
    st = lib().pkv_swap_blocks(_ptr(dst_k_cache), _ptr(dst_v_cache), _ptr(src_k_cache), _ptr(src_v_cache),
                               _ptr(pairs), pairs.shape[0], H, D, BS, NBs, NBd, _code("k_cache", dst_k_cache),
                               _stream(stream))
    _check("pkv_swap_blocks", st)


def gather_kv(k_out: torch.Tensor, v_out: torch.Tensor, cu_lens: torch.Tensor, k_cache: torch.Tensor,
              v_cache: torch.Tensor, block_tables: torch.Tensor, context_lens: torch.Tensor, *, stream=None) -> None:
    """Contiguous copy of each sequence's K/V rows: k_out[cu_lens[s] + t] = token t of sequence s."""
    for n, t in (("k_out", k_out), ("v_out", v_out)):
        _dev(n, t, k_cache.dtype, 3)
    for n, t in (("k_cache", k_cache), ("v_cache", v_cache)):
        _dev(n, t, ndim=4)
    _dev("cu_lens", cu_lens, torch.int32, 1)
    _dev("block_tables", block_tables, torch.int32, 2)
    _dev("context_lens", context_lens, torch.int32, 1)
    NB, H, BS, D = k_cache.shape
    S, MB = block_tables.shape
    if cu_lens.shape[0] != S + 1 or context_lens.shape[0] != S or k_out.shape != v_out.shape \
            or k_out.shape[1:] != (H, D):
        raise ValueError("gather_kv: shapes disagree")
    st = lib().pkv_gather_kv(_ptr(k_out), _ptr(v_out), _ptr(cu_lens), _ptr(k_cache), _ptr(v_cache),
                             _ptr(block_tables), _ptr(context_lens), S, H, D, BS, MB, NB, _code("k_cache", k_cache),
                             _stream(stream))
    _check("pkv_gather_kv", st)


def stream_read(buf: torch.Tensor, sink: torch.Tensor, nbytes: Optional[int] = None, *, stream=None) -> None:
    """Read-only bandwidth probe: reads the first nbytes (default: all) of the
    contiguous device buffer buf once with the decode's 16-byte non-temporal
    loads.  sink is a one-element int32 / uint32 device tensor that the probe
    writes only when one lane's XOR of what it read equals 0x9e3779b9."""
    if not (buf.is_cuda and buf.is_contiguous()):
        raise ValueError("stream_read: buf must be a contiguous device tensor")
    if not (sink.is_cuda and sink.numel() >= 1 and sink.element_size() == 4):
        raise ValueError("stream_read: sink must be a device tensor of 4-byte elements")
    total = buf.numel() * buf.element_size()
    n = total if nbytes is None else int(nbytes)
    if n < 0 or n > total:
        raise ValueError(f"stream_read: {n} bytes requested from a buffer of {total}")
    _check("pkv_stream_read", lib().pkv_stream_read(_ptr(buf), n, _ptr(sink), _stream(stream)))


class DecodeGraph:
    """The decode step captured into a HIP graph over fixed buffers.

    The graph records: copy_blocks(k_cache, v_cache, copy_pairs) when
    copy_pairs has rows, reshape_and_cache(key, value, ..., slot_mapping),
    and the decode of q into out.  Every tensor given here must stay alive
    and in place while the graph exists (this object keeps references);
    ``launch()`` replays the step on their current contents.  Batch slots
    without a sequence carry slot -1 and context length 0; unused copy
    pairs carry ids outside the pool.  With ``append`` the cache write and
    the decode are recorded as paged_attention_decode_append (each slot must
    then be the slot of its sequence's last position).  Per-head scales
    (float32 [H] device tensors) are read at every replay."""

    def __init__(self, k_cache, v_cache, key, value, slot_mapping, q, out, block_tables, context_lens, scale: float,
                 k_scale: float = 1.0, v_scale: float = 1.0, *, copy_pairs: Optional[torch.Tensor] = None,
                 workspace: Optional[torch.Tensor] = None, append: bool = False):
        for n, t in (("key", key), ("value", value), ("q", q), ("out", out)):
            _dev(n, t, q.dtype, 3)
        for n, t in (("k_cache", k_cache), ("v_cache", v_cache)):
            _dev(n, t, k_cache.dtype, 4)
        _dev("slot_mapping", slot_mapping, torch.int32, 1)
        _dev("block_tables", block_tables, torch.int32, 2)
        _dev("context_lens", context_lens, torch.int32, 1)
        S, H, D = q.shape
        NB, Hc, BS, Dc = k_cache.shape
        MB = block_tables.shape[1]
        if key.shape != q.shape or value.shape != q.shape or out.shape != q.shape or (Hc, Dc) != (H, D) \
                or v_cache.shape != k_cache.shape or slot_mapping.shape[0] != S or block_tables.shape[0] != S \
                or context_lens.shape[0] != S:
            raise ValueError("DecodeGraph: shapes disagree")
        npairs = 0
        if copy_pairs is not None:
            _dev("copy_pairs", copy_pairs, torch.int32, 2)
            if copy_pairs.shape[1] != 2:
                raise ValueError("copy_pairs must be [N, 2]")
            npairs = copy_pairs.shape[0]
        need = decode_workspace_bytes(S, H, D, BS, MB)
        if need and workspace is None:
            workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
        ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
        hs = _head_scales(k_scale, v_scale, H, q.device, None)
        self._keep = (k_cache, v_cache, key, value, slot_mapping, q, out, block_tables, context_lens, copy_pairs,
                      workspace, hs)
        self.workspace = workspace
        st = _DecodeStep(k_cache.data_ptr(), v_cache.data_ptr(), key.data_ptr(), value.data_ptr(),
                         slot_mapping.data_ptr(), None if copy_pairs is None else copy_pairs.data_ptr(), npairs,
                         q.data_ptr(), out.data_ptr(), block_tables.data_ptr(), context_lens.data_ptr(),
                         None if workspace is None else workspace.data_ptr(), ws_bytes, S, H, D, BS, MB, NB,
                         float(scale), 1.0 if hs else float(k_scale), 1.0 if hs else float(v_scale), _code("q", q),
                         _code("k_cache", k_cache), 1 if append else 0,
                         hs[0].data_ptr() if hs else None, hs[1].data_ptr() if hs else None)
        handle = ctypes.c_void_p()
        with torch.cuda.device(q.device):
            _check("pkv_decode_graph_create", lib().pkv_decode_graph_create(ctypes.byref(st), ctypes.byref(handle)))
        self._handle = handle

    def launch(self, stream=None) -> None:
        if not self._handle:
            raise RuntimeError("DecodeGraph has been destroyed")
        _check("pkv_decode_graph_launch", lib().pkv_decode_graph_launch(self._handle, _stream(stream)))

    def destroy(self) -> None:
        if self._handle:
            lib().pkv_decode_graph_destroy(self._handle)
            self._handle = ctypes.c_void_p()

    def __del__(self):
        try:
            self.destroy()
        except Exception:
            pass


__all__ = ["LIB_PATH", "EXPORTS", "PagedKVError", "lib", "loaded_path", "status_string", "version",
           "reshape_and_cache", "decode_workspace_bytes", "alloc_decode_workspace", "paged_attention_decode",
           "STATIC_WORKSPACE_BYTES", "paged_attention_decode_static", "paged_attention_decode_grouped",
           "paged_attention_decode_grouped_partitions",
           "paged_attention_decode_partitions", "paged_attention_decode_merge", "paged_attention_decode_append",
           "paged_attention_decode_append_partitions",
           "paged_attention_prefill", "paged_attention_prefill_append", "copy_blocks", "swap_blocks", "gather_kv", "stream_read", "DecodeGraph",
           "check_workspace_bytes", "check_step_inputs",
           "PKV_OK", "PKV_ERR_INVALID_ARG", "PKV_ERR_UNSUPPORTED", "PKV_ERR_WORKSPACE", "PKV_ERR_HIP",
           "PKV_ERR_DEVICE_CHECK", "PKV_CHECK_CONTEXT_LEN", "PKV_CHECK_BLOCK_ID", "PKV_CHECK_SLOT_RANGE",
           "PKV_CHECK_SLOT_DUP", "PKV_CHECK_PAIR_RANGE", "PKV_CHECK_PAIR_OVERLAP", "PKV_CHECK_APPEND_SLOT",
           "PKV_CHECK_SHARED_WRITE",
           "PKV_F32", "PKV_F16", "PKV_BF16", "PKV_FP8_E4M3", "PKV_INT8"]
