"""Python binding of libpadecode.so (ctypes): argument marshalling only.

Every step of the decode runs in the HIP library; this module reads shapes
and dtypes off torch tensors, fills ``pa_dims_t`` and calls the C ABI on the
current torch stream. There is no fallback: a missing library or a non-zero
status raises.
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libpadecode.so")

PA_OK, PA_ERR_NULL, PA_ERR_SHAPE, PA_ERR_UNSUPPORTED, PA_ERR_ALIGN, PA_ERR_WORKSPACE, PA_ERR_HIP = range(7)
PA_DTYPE_F32, PA_DTYPE_BF16, PA_DTYPE_FP8_E5M2, PA_DTYPE_FP8_E4M3, PA_DTYPE_INT4 = 0, 1, 2, 3, 4
KERNELS = {"auto": 0, "valu": 1, "mfma": 2}
KERNEL_NAMES = {v: k for k, v in KERNELS.items()}
SCHEDULES = {"auto": 0, "grid": 1, "queue": 2}
SCHEDULE_NAMES = {v: k for k, v in SCHEDULES.items()}

# Symbols declared in include/pa_decode.h and include/pa_cache.h.
EXPORTED = ("pa_decode", "pa_decode_ws", "pa_decode_ws_timed", "pa_decode_noalloc", "pa_decode_workspace_bytes",
            "pa_decode_plan", "pa_status_str", "pa_version", "pa_cache_append", "pa_cache_copy_blocks", "pa_read_probe")
NOALLOC_SCRATCH_BYTES = 128 << 20   # PA_NOALLOC_SCRATCH_BYTES


class PaDims(ctypes.Structure):
    _fields_ = [("num_seqs", ctypes.c_int32), ("num_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("num_blocks", ctypes.c_int32), ("block_size", ctypes.c_int32),
                ("max_blocks_per_seq", ctypes.c_int32), ("q_dtype", ctypes.c_int32),
                ("kv_dtype", ctypes.c_int32), ("k_scale", ctypes.c_float), ("v_scale", ctypes.c_float),
                ("max_seq_len", ctypes.c_int32), ("partition_tokens", ctypes.c_int32),
                ("kernel", ctypes.c_int32), ("q_len", ctypes.c_int32), ("schedule", ctypes.c_int32),
                ("waves_per_item", ctypes.c_int32), ("k_block_scales", ctypes.c_void_p),
                ("v_block_scales", ctypes.c_void_p)]


class PaPlan(ctypes.Structure):
    _fields_ = [("kernel", ctypes.c_int32), ("partition_tokens", ctypes.c_int32),
                ("max_partitions", ctypes.c_int32), ("grid_workgroups", ctypes.c_int32),
                ("reduce_workgroups", ctypes.c_int32), ("schedule", ctypes.c_int32),
                ("waves_per_item", ctypes.c_int32), ("pad", ctypes.c_int32),
                ("workspace_bytes", ctypes.c_size_t)]


class PagedAttentionError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(msg)
        self.status = status


_lib = None


def load_library(path: Optional[str] = None) -> ctypes.CDLL:
    """Load the HIP library (built by ``python -m paged_kv_cache_220_amd.build``)."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise RuntimeError(f"{p} is missing: build the HIP library first "
                           f"(python -m paged_kv_cache_220_amd.build); there is no CPU fallback")
    lib = ctypes.CDLL(p)
    vp, i32, f32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_float, ctypes.c_size_t
    dims_p = ctypes.POINTER(PaDims)
    common = [vp, vp, vp, vp, vp, i32, f32, vp, dims_p]
    lib.pa_decode.argtypes = common + [vp]
    lib.pa_decode.restype = ctypes.c_int
    lib.pa_decode_ws.argtypes = common + [vp, sz, vp]
    lib.pa_decode_ws.restype = ctypes.c_int
    lib.pa_decode_ws_timed.argtypes = common + [vp, sz, vp, vp, vp, vp]
    lib.pa_decode_ws_timed.restype = ctypes.c_int
    lib.pa_decode_noalloc.argtypes = common + [vp]
    lib.pa_decode_noalloc.restype = ctypes.c_int
    lib.pa_decode_workspace_bytes.argtypes = [dims_p, i32, ctypes.POINTER(ctypes.c_int)]
    lib.pa_decode_workspace_bytes.restype = sz
    lib.pa_decode_plan.argtypes = [dims_p, i32, ctypes.POINTER(PaPlan)]
    lib.pa_decode_plan.restype = ctypes.c_int
    lib.pa_status_str.argtypes = [ctypes.c_int]
    lib.pa_status_str.restype = ctypes.c_char_p
    lib.pa_version.argtypes = []
    lib.pa_version.restype = ctypes.c_int
    lib.pa_cache_append.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, dims_p, vp]
    lib.pa_cache_append.restype = ctypes.c_int
    lib.pa_cache_copy_blocks.argtypes = [vp, vp, vp, vp, i32, i32, dims_p, vp]
    lib.pa_cache_copy_blocks.restype = ctypes.c_int
    lib.pa_read_probe.argtypes = [vp, sz, vp, vp]
    lib.pa_read_probe.restype = ctypes.c_int
    if path is None:
        _lib = lib
    return lib


def status_str(status: int) -> str:
    return load_library().pa_status_str(status).decode()


def _check(rc: int):
    if rc != PA_OK:
        raise PagedAttentionError(rc, status_str(rc))


_TORCH_DTYPES = {torch.float32: PA_DTYPE_F32, torch.bfloat16: PA_DTYPE_BF16}
_KV_NAMES = {"f32": PA_DTYPE_F32, "bf16": PA_DTYPE_BF16, "e5m2": PA_DTYPE_FP8_E5M2, "e4m3": PA_DTYPE_FP8_E4M3,
             "int4": PA_DTYPE_INT4}


def _kv_dtype_code(t: torch.Tensor, kv_dtype: Optional[str]) -> int:
    if kv_dtype is not None:
        return _KV_NAMES[kv_dtype]
    if t.dtype == torch.float8_e5m2:
        return PA_DTYPE_FP8_E5M2
    if t.dtype == torch.float8_e4m3fn:
        return PA_DTYPE_FP8_E4M3
    if t.dtype == torch.uint8:
        return PA_DTYPE_INT4          # packed int4 codes, two tokens per byte
    if t.dtype in _TORCH_DTYPES:
        return _TORCH_DTYPES[t.dtype]
    raise TypeError(f"unsupported KV cache dtype {t.dtype}; pass kv_dtype for raw byte views")


_KV_ELEM_BYTES = {PA_DTYPE_F32: 4, PA_DTYPE_BF16: 2, PA_DTYPE_FP8_E5M2: 1, PA_DTYPE_FP8_E4M3: 1, PA_DTYPE_INT4: 1}


def _tokens_per_row(k_cache: torch.Tensor, kv_code: int) -> int:
    """Tokens per block from the cache's last axis; the tensor's element size
    must be that of the cache type (one byte holds two int4 tokens), so the
    library's byte arithmetic matches the tensor's extent."""
    if k_cache.element_size() != _KV_ELEM_BYTES[kv_code]:
        _shape_error(f"a {k_cache.element_size()}-byte cache element does not hold the KV dtype {kv_code}")
    return k_cache.shape[3] * (2 if kv_code == PA_DTYPE_INT4 else 1)


def _scale_ptr(t: Optional[torch.Tensor], k_cache: torch.Tensor, name: str):
    """Device pointer of a [num_blocks, num_kv_heads] float32 scale array, or None."""
    if t is None:
        return None
    if t.dtype != torch.float32 or not t.is_contiguous() or t.device != k_cache.device:
        raise ValueError(f"{name}: contiguous float32 on the caches' device expected")
    if tuple(t.shape) != (k_cache.shape[0], k_cache.shape[1]):
        raise ValueError(f"{name}: shape [num_blocks, num_kv_heads] expected")
    return t.data_ptr()


def make_dims(q: torch.Tensor, k_cache: torch.Tensor, block_tables: torch.Tensor, *,
              kv_dtype: Optional[str] = None, max_seq_len: int = 0, partition_tokens: int = 0,
              kernel: str = "auto", k_scale: float = 1.0, v_scale: float = 1.0,
              schedule: str = "auto", waves_per_item: int = 0,
              k_block_scales: Optional[torch.Tensor] = None,
              v_block_scales: Optional[torch.Tensor] = None) -> PaDims:
    if q.dim() not in (3, 4) or k_cache.dim() != 4 or block_tables.dim() != 2:
        raise ValueError("q [S,H,D] or [S,q_len,H,D], k_cache [NB,Hkv,D,bs], block_tables [S,max_blocks] expected")
    if q.dtype not in _TORCH_DTYPES:
        raise TypeError(f"unsupported q dtype {q.dtype}")
    if q.dim() == 4:
        S, QL, H, D = q.shape
    else:
        (S, H, D), QL = q.shape, 1
    kv_code = _kv_dtype_code(k_cache, kv_dtype)
    NB = k_cache.shape[0]
    return PaDims(num_seqs=S, num_heads=H, head_dim=D, num_blocks=NB, block_size=_tokens_per_row(k_cache, kv_code),
                  max_blocks_per_seq=block_tables.shape[1], q_dtype=_TORCH_DTYPES[q.dtype],
                  kv_dtype=kv_code, k_scale=k_scale, v_scale=v_scale,
                  max_seq_len=max_seq_len, partition_tokens=partition_tokens, kernel=KERNELS[kernel], q_len=QL,
                  schedule=SCHEDULES[schedule], waves_per_item=waves_per_item,
                  k_block_scales=_scale_ptr(k_block_scales, k_cache, "k_block_scales"),
                  v_block_scales=_scale_ptr(v_block_scales, k_cache, "v_block_scales"))


def plan(dims: PaDims, num_kv_heads: int) -> dict:
    p = PaPlan()
    _check(load_library().pa_decode_plan(ctypes.byref(dims), num_kv_heads, ctypes.byref(p)))
    return dict(kernel=KERNEL_NAMES[p.kernel], partition_tokens=p.partition_tokens,
                max_partitions=p.max_partitions, grid_workgroups=p.grid_workgroups,
                reduce_workgroups=p.reduce_workgroups, workspace_bytes=p.workspace_bytes,
                schedule=SCHEDULE_NAMES[p.schedule], waves_per_item=p.waves_per_item)


def workspace_bytes(dims: PaDims, num_kv_heads: int) -> int:
    st = ctypes.c_int(0)
    n = load_library().pa_decode_workspace_bytes(ctypes.byref(dims), num_kv_heads, ctypes.byref(st))
    _check(st.value)
    return int(n)


def _shape_error(msg: str):
    """PA_ERR_SHAPE raised by the binding: the C ABI sees sizes, not tensors, so
    the agreement between the tensors and the sizes passed on is checked here."""
    raise PagedAttentionError(PA_ERR_SHAPE, f"PA_ERR_SHAPE: {msg}")


def _check_decode_shapes(q, k_cache, block_tables, seq_lens, num_kv_heads):
    """The tensor shapes pa_decode relies on (they size every device access):
    k_cache [num_blocks, num_kv_heads, head_dim, block_size (int4: block_size / 2 bytes)],
    q [S, H, head_dim] or [S, q_len, H, head_dim], block_tables [S, max_blocks], seq_lens [S]."""
    if q.dim() not in (3, 4) or k_cache.dim() != 4 or block_tables.dim() != 2:
        _shape_error("q [S,H,D] or [S,q_len,H,D], k_cache [NB,Hkv,D,bs], block_tables [S,max_blocks] expected")
    S, D = q.shape[0], q.shape[-1]
    if int(num_kv_heads) != k_cache.shape[1]:
        _shape_error(f"num_kv_heads {num_kv_heads} differs from the cache's KV-head axis {k_cache.shape[1]}")
    if k_cache.shape[2] != D:
        _shape_error(f"the cache's head_dim {k_cache.shape[2]} differs from q's {D}")
    if block_tables.shape[0] != S:
        _shape_error(f"block_tables has {block_tables.shape[0]} rows for {S} sequences")
    if seq_lens.dim() != 1 or seq_lens.numel() != S:
        _shape_error(f"seq_lens has shape {tuple(seq_lens.shape)} for {S} sequences")


def _validate_tensors(q, k_cache, v_cache, block_tables, seq_lens, out, num_kv_heads):
    dev = q.device
    _check_decode_shapes(q, k_cache, block_tables, seq_lens, num_kv_heads)
    if out.shape != q.shape:
        _shape_error(f"out has shape {tuple(out.shape)}, q {tuple(q.shape)}")
    if v_cache.shape != k_cache.shape:
        _shape_error(f"v_cache has shape {tuple(v_cache.shape)}, k_cache {tuple(k_cache.shape)}")
    if dev.type != "cuda":
        raise ValueError("pa_decode runs on the GPU: q must be a cuda tensor")
    for name, t in (("q", q), ("k_cache", k_cache), ("v_cache", v_cache), ("block_tables", block_tables),
                    ("seq_lens", seq_lens), ("out", out)):
        if t.device != dev:
            raise ValueError(f"{name} is on {t.device}, q on {dev}")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    if block_tables.dtype != torch.int32 or seq_lens.dtype != torch.int32:
        raise TypeError("block_tables and seq_lens must be int32")
    if out.shape != q.shape or out.dtype != q.dtype:
        raise ValueError("out must have q's shape and dtype")
    if v_cache.shape != k_cache.shape or v_cache.dtype != k_cache.dtype:
        raise ValueError("v_cache must match k_cache")


def pa_decode(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor, block_tables: torch.Tensor,
              seq_lens: torch.Tensor, num_kv_heads: int, scale: float, out: Optional[torch.Tensor] = None, *,
              kv_dtype: Optional[str] = None, max_seq_len: int = 0, partition_tokens: int = 0,
              kernel: str = "auto", k_scale: float = 1.0, v_scale: float = 1.0, schedule: str = "auto",
              waves_per_item: int = 0, workspace: Optional[torch.Tensor] = None, events=None,
              k_block_scales: Optional[torch.Tensor] = None,
              v_block_scales: Optional[torch.Tensor] = None) -> torch.Tensor:
    """PagedAttention decode through the C ABI; returns `out`.

    q may be [S, H, D] (one query per sequence) or [S, q_len, H, D] (the last
    q_len positions of each sequence, causally masked).

    `workspace` (uint8 cuda tensor) selects ``pa_decode_ws``; without it the
    library takes its workspace from the stream-ordered allocator.
    `events` = (start, mid, end) raw hipEvent_t handles selects ``pa_decode_ws_timed``.
    """
    if out is None:
        out = torch.empty_like(q)
    _validate_tensors(q, k_cache, v_cache, block_tables, seq_lens, out, num_kv_heads)
    dims = make_dims(q, k_cache, block_tables, kv_dtype=kv_dtype, max_seq_len=max_seq_len,
                     partition_tokens=partition_tokens, kernel=kernel, k_scale=k_scale, v_scale=v_scale,
                     schedule=schedule, waves_per_item=waves_per_item, k_block_scales=k_block_scales,
                     v_block_scales=v_block_scales)
    lib = load_library()
    stream = ctypes.c_void_p(torch.cuda.current_stream(q.device).cuda_stream)
    args = (ctypes.c_void_p(q.data_ptr()), ctypes.c_void_p(k_cache.data_ptr()),
            ctypes.c_void_p(v_cache.data_ptr()), ctypes.c_void_p(block_tables.data_ptr()),
            ctypes.c_void_p(seq_lens.data_ptr()), ctypes.c_int32(num_kv_heads), ctypes.c_float(scale),
            ctypes.c_void_p(out.data_ptr()), ctypes.byref(dims))
    if workspace is None and events is None:
        rc = lib.pa_decode(*args, stream)
    else:
        if workspace is None:
            raise ValueError("events need a caller workspace")
        if workspace.device != q.device or workspace.dtype != torch.uint8:
            raise ValueError("workspace must be a uint8 tensor on q's device")
        ws = (ctypes.c_void_p(workspace.data_ptr()), ctypes.c_size_t(workspace.numel()))
        if events is None:
            rc = lib.pa_decode_ws(*args, *ws, stream)
        else:
            ev = [ctypes.c_void_p(e) if e else None for e in events]
            rc = lib.pa_decode_ws_timed(*args, *ws, stream, *ev)
    _check(rc)
    return out


def pa_decode_noalloc(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor, block_tables: torch.Tensor,
                      seq_lens: torch.Tensor, num_kv_heads: int, scale: float, out: torch.Tensor, *,
                      kv_dtype: Optional[str] = None, max_seq_len: int = 0, partition_tokens: int = 0,
                      kernel: str = "auto", k_scale: float = 1.0, v_scale: float = 1.0, schedule: str = "auto",
                      waves_per_item: int = 0, k_block_scales: Optional[torch.Tensor] = None,
                      v_block_scales: Optional[torch.Tensor] = None) -> torch.Tensor:
    """``pa_decode_noalloc``: decode without any allocation, the workspace taken
    from the library's fixed per-GPU scratch array (NOALLOC_SCRATCH_BYTES). The
    caller passes `out`; calls that may overlap on one GPU must be ordered."""
    _validate_tensors(q, k_cache, v_cache, block_tables, seq_lens, out, num_kv_heads)
    dims = make_dims(q, k_cache, block_tables, kv_dtype=kv_dtype, max_seq_len=max_seq_len,
                     partition_tokens=partition_tokens, kernel=kernel, k_scale=k_scale, v_scale=v_scale,
                     schedule=schedule, waves_per_item=waves_per_item, k_block_scales=k_block_scales,
                     v_block_scales=v_block_scales)
    stream = ctypes.c_void_p(torch.cuda.current_stream(q.device).cuda_stream)
    _check(load_library().pa_decode_noalloc(
        ctypes.c_void_p(q.data_ptr()), ctypes.c_void_p(k_cache.data_ptr()), ctypes.c_void_p(v_cache.data_ptr()),
        ctypes.c_void_p(block_tables.data_ptr()), ctypes.c_void_p(seq_lens.data_ptr()), ctypes.c_int32(num_kv_heads),
        ctypes.c_float(scale), ctypes.c_void_p(out.data_ptr()), ctypes.byref(dims), stream))
    return out


class DecodeCall:
    """One pa_decode_ws / pa_decode_ws_timed call with its arguments checked and
    marshalled once, for loops that repeat the same call (the tensors are kept
    alive by this object; the stream is the current one at construction)."""

    def __init__(self, q, k_cache, v_cache, block_tables, seq_lens, num_kv_heads, scale, out, *,
                 workspace=None, kv_dtype=None, max_seq_len=0, partition_tokens=0, kernel="auto",
                 k_scale=1.0, v_scale=1.0, schedule="auto", waves_per_item=0, k_block_scales=None,
                 v_block_scales=None):
        _validate_tensors(q, k_cache, v_cache, block_tables, seq_lens, out, num_kv_heads)
        self.dims = make_dims(q, k_cache, block_tables, kv_dtype=kv_dtype, max_seq_len=max_seq_len,
                              partition_tokens=partition_tokens, kernel=kernel, k_scale=k_scale, v_scale=v_scale,
                              schedule=schedule, waves_per_item=waves_per_item,
                              k_block_scales=k_block_scales, v_block_scales=v_block_scales)
        self._scales = (k_block_scales, v_block_scales)   # keep the tensors alive with the pointers
        if workspace is None:
            workspace = alloc_workspace(self.dims, num_kv_heads, q.device)
        self._keep = (q, k_cache, v_cache, block_tables, seq_lens, out, workspace)
        self._lib = load_library()
        self._args = (ctypes.c_void_p(q.data_ptr()), ctypes.c_void_p(k_cache.data_ptr()),
                      ctypes.c_void_p(v_cache.data_ptr()), ctypes.c_void_p(block_tables.data_ptr()),
                      ctypes.c_void_p(seq_lens.data_ptr()), ctypes.c_int32(num_kv_heads), ctypes.c_float(scale),
                      ctypes.c_void_p(out.data_ptr()), ctypes.byref(self.dims),
                      ctypes.c_void_p(workspace.data_ptr()), ctypes.c_size_t(workspace.numel()),
                      ctypes.c_void_p(torch.cuda.current_stream(q.device).cuda_stream))

    def __call__(self, events=None):
        if events is None:
            rc = self._lib.pa_decode_ws(*self._args)
        else:
            rc = self._lib.pa_decode_ws_timed(*self._args, *[ctypes.c_void_p(e) if e else None for e in events])
        if rc != PA_OK:
            _check(rc)


def alloc_workspace(dims: PaDims, num_kv_heads: int, device) -> torch.Tensor:
    n = workspace_bytes(dims, num_kv_heads)
    # torch's caching allocator hands out 512-byte aligned blocks
    return torch.empty(max(n, 256), dtype=torch.uint8, device=device)


def _cache_dims(k_cache: torch.Tensor, block_tables: Optional[torch.Tensor], kv_dtype: Optional[str],
                k_scale: float, v_scale: float, k_block_scales=None, v_block_scales=None) -> PaDims:
    NB, _, D, _ = k_cache.shape
    kv_code = _kv_dtype_code(k_cache, kv_dtype)
    S, MB = (block_tables.shape if block_tables is not None else (1, 1))
    return PaDims(num_seqs=S, num_heads=k_cache.shape[1], head_dim=D, num_blocks=NB,
                  block_size=_tokens_per_row(k_cache, kv_code), max_blocks_per_seq=MB, q_dtype=PA_DTYPE_BF16,
                  kv_dtype=kv_code, k_scale=k_scale, v_scale=v_scale, max_seq_len=0, partition_tokens=0, kernel=0,
                  q_len=0, schedule=0, k_block_scales=_scale_ptr(k_block_scales, k_cache, "k_block_scales"),
                  v_block_scales=_scale_ptr(v_block_scales, k_cache, "v_block_scales"))


def pa_cache_append(k_new: torch.Tensor, v_new: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                    block_tables: torch.Tensor, token_seq: torch.Tensor, token_pos: torch.Tensor, *,
                    kv_dtype: Optional[str] = None, k_scale: float = 1.0, v_scale: float = 1.0,
                    k_block_scales: Optional[torch.Tensor] = None,
                    v_block_scales: Optional[torch.Tensor] = None) -> None:
    """Write new tokens' K/V ([num_tokens, num_kv_heads, head_dim]) into the paged caches in place."""
    for name, t in (("k_new", k_new), ("v_new", v_new), ("k_cache", k_cache), ("v_cache", v_cache),
                    ("block_tables", block_tables), ("token_seq", token_seq), ("token_pos", token_pos)):
        if t.device != k_cache.device or not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous on the caches' device")
    if k_new.dtype not in _TORCH_DTYPES or v_new.dtype != k_new.dtype or k_new.shape != v_new.shape:
        raise TypeError("k_new / v_new: same shape, float32 or bfloat16")
    if token_seq.dtype != torch.int32 or token_pos.dtype != torch.int32 or block_tables.dtype != torch.int32:
        raise TypeError("block_tables, token_seq and token_pos must be int32")
    if k_new.dim() != 3 or k_cache.dim() != 4 or block_tables.dim() != 2:
        _shape_error("k_new [num_tokens, num_kv_heads, head_dim], k_cache [NB, Hkv, D, bs], "
                     "block_tables [S, max_blocks] expected")
    if v_cache.shape != k_cache.shape or v_cache.dtype != k_cache.dtype:
        _shape_error("v_cache must match k_cache")
    n, hkv, d = k_new.shape
    if (hkv, d) != (k_cache.shape[1], k_cache.shape[2]):
        _shape_error(f"k_new rows are [{hkv}, {d}], the cache holds [{k_cache.shape[1]}, {k_cache.shape[2]}] "
                     f"(num_kv_heads, head_dim)")
    if token_seq.dim() != 1 or token_pos.dim() != 1 or token_seq.numel() != n or token_pos.numel() != n:
        _shape_error(f"token_seq {tuple(token_seq.shape)} and token_pos {tuple(token_pos.shape)} must both "
                     f"have num_tokens = {n} entries")
    if k_cache.device.type != "cuda":
        raise ValueError("pa_cache_append runs on the GPU: the caches must be cuda tensors")
    dims = _cache_dims(k_cache, block_tables, kv_dtype, k_scale, v_scale, k_block_scales, v_block_scales)
    stream = ctypes.c_void_p(torch.cuda.current_stream(k_cache.device).cuda_stream)
    rc = load_library().pa_cache_append(
        ctypes.c_void_p(k_new.data_ptr()), ctypes.c_void_p(v_new.data_ptr()), ctypes.c_void_p(k_cache.data_ptr()),
        ctypes.c_void_p(v_cache.data_ptr()), ctypes.c_void_p(block_tables.data_ptr()),
        ctypes.c_void_p(token_seq.data_ptr()), ctypes.c_void_p(token_pos.data_ptr()), n, hkv,
        _TORCH_DTYPES[k_new.dtype], ctypes.byref(dims), stream)
    _check(rc)


def pa_cache_copy_blocks(k_cache: torch.Tensor, v_cache: torch.Tensor, src_blocks: torch.Tensor,
                         dst_blocks: torch.Tensor, *, kv_dtype: Optional[str] = None,
                         k_block_scales: Optional[torch.Tensor] = None,
                         v_block_scales: Optional[torch.Tensor] = None) -> None:
    """Copy physical blocks src_blocks[i] -> dst_blocks[i] in both caches (in place), and
    their per-block scales when given."""
    for name, t in (("k_cache", k_cache), ("v_cache", v_cache), ("src_blocks", src_blocks), ("dst_blocks", dst_blocks)):
        if t.device != k_cache.device or not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous on the caches' device")
    if src_blocks.dtype != torch.int32 or dst_blocks.dtype != torch.int32:
        raise TypeError("src_blocks / dst_blocks must be int32")
    if src_blocks.dim() != 1 or src_blocks.shape != dst_blocks.shape:
        _shape_error(f"src_blocks {tuple(src_blocks.shape)} and dst_blocks {tuple(dst_blocks.shape)} must be "
                     f"1-D of the same length")
    if k_cache.dim() != 4 or v_cache.shape != k_cache.shape or v_cache.dtype != k_cache.dtype:
        _shape_error("k_cache [NB, Hkv, D, bs] and a v_cache of the same shape and dtype expected")
    if k_cache.device.type != "cuda":
        raise ValueError("pa_cache_copy_blocks runs on the GPU: the caches must be cuda tensors")
    dims = _cache_dims(k_cache, None, kv_dtype, 1.0, 1.0, k_block_scales, v_block_scales)
    stream = ctypes.c_void_p(torch.cuda.current_stream(k_cache.device).cuda_stream)
    rc = load_library().pa_cache_copy_blocks(
        ctypes.c_void_p(k_cache.data_ptr()), ctypes.c_void_p(v_cache.data_ptr()),
        ctypes.c_void_p(src_blocks.data_ptr()), ctypes.c_void_p(dst_blocks.data_ptr()), src_blocks.numel(),
        k_cache.shape[1], ctypes.byref(dims), stream)
    _check(rc)


PROBE_SINK_WORDS = 4096      # PA_PROBE_SINK_WORDS
PROBE_CHUNK_BYTES = 32768    # PA_PROBE_CHUNK_BYTES


def pa_read_probe(buf: torch.Tensor, sink: torch.Tensor, stream=None) -> int:
    """Stream every byte of `buf` once (128-bit non-temporal loads), nothing else.

    Measurement only: its rate is the read ceiling the decode kernels are compared with.
    `buf` is any contiguous device tensor whose byte size is a multiple of 16; `sink` a
    device tensor of PROBE_SINK_WORDS 32-bit words. Workgroup w stores the XOR of the words it
    read in sink[w]; returns the number of workgroups n, so the XOR of sink[:n] is the XOR of
    all of buf's 32-bit words.
    """
    if not buf.is_contiguous() or not sink.is_contiguous() or sink.numel() < PROBE_SINK_WORDS \
            or sink.element_size() != 4:
        raise ValueError(f"pa_read_probe: contiguous buf and a {PROBE_SINK_WORDS}-word 32-bit sink expected")
    if buf.device != sink.device:
        raise ValueError("pa_read_probe: buf and sink must be on the same device")
    if stream is None:
        stream = torch.cuda.current_stream(buf.device).cuda_stream
    nbytes = buf.numel() * buf.element_size()
    _check(load_library().pa_read_probe(ctypes.c_void_p(buf.data_ptr()), nbytes,
                                        ctypes.c_void_p(sink.data_ptr()), ctypes.c_void_p(stream)))
    return min(-(-nbytes // PROBE_CHUNK_BYTES), PROBE_SINK_WORDS)
