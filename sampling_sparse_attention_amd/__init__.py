"""SANTA decode-step attention on MI355X (gfx950): Python binding of libsanta.

Every call is marshalled straight into the C ABI declared in
``include/santa.h`` (same names, same arguments); all of the computation runs
in the library's HIP kernels.  PyTorch only provides device memory and the
current stream.  If ``libsanta.so`` has not been built the import still works
but every entry point raises: there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

__all__ = [
    "MODE_MULTINOMIAL", "MODE_STRATIFIED", "MODE_SYSTEMATIC", "Shape", "WorkspaceLayout",
    "SantaError", "library", "library_path", "make_shape", "santa_workspace_layout_query",
    "santa_workspace_size", "santa_workspace_init", "santa_decode_path", "santa_decode",
    "santa_score_pass", "santa_sample_pass", "santa_decode_flash", "decode", "allocate_workspace",
    "workspace_error",
    "EXPORTED_SYMBOLS",
]

MODE_MULTINOMIAL = 0
MODE_STRATIFIED = 1
MODE_SYSTEMATIC = 2
DTYPE_BF16 = 0
DTYPE_F32 = 1

EXPORTED_SYMBOLS = (
    "santa_abi_version", "santa_status_string", "santa_last_error",
    "santa_workspace_layout_query", "santa_workspace_size", "santa_workspace_init",
    "santa_decode_path", "santa_decode", "santa_score_pass", "santa_sample_pass", "santa_decode_flash",
)
PATH_FUSED = 1
PATH_TWO_KERNELS = 2

_PKG_DIR = os.path.dirname(os.path.abspath(__file__))
library_path = os.path.join(_PKG_DIR, "libsanta.so")


class Shape(ctypes.Structure):
    """Mirror of ``santa_shape``."""
    _fields_ = [
        ("batch", ctypes.c_int32), ("num_q_heads", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
        ("max_seq_len", ctypes.c_int32), ("page_size", ctypes.c_int32),
        ("pages_per_seq", ctypes.c_int32), ("num_pages", ctypes.c_int32),
        ("dtype", ctypes.c_int32), ("split_size", ctypes.c_int32),
        ("kv_stride_seq", ctypes.c_int64), ("kv_stride_tok", ctypes.c_int64),
        ("kv_stride_head", ctypes.c_int64),
    ]


class WorkspaceLayout(ctypes.Structure):
    """Mirror of ``santa_workspace_layout``."""
    _fields_ = [
        ("total_bytes", ctypes.c_size_t), ("sync_offset", ctypes.c_size_t),
        ("barrier_offset", ctypes.c_size_t), ("accum_offset", ctypes.c_size_t),
        ("flash_offset", ctypes.c_size_t),
        ("records_offset", ctypes.c_size_t), ("stash_offset", ctypes.c_size_t),
        ("stash_row_bytes", ctypes.c_size_t), ("targets_offset", ctypes.c_size_t),
        ("split_size", ctypes.c_int32), ("num_splits", ctypes.c_int32),
    ]


class SantaError(RuntimeError):
    def __init__(self, status: int, where: str, detail: str):
        super().__init__(f"{where}: {detail} (status {status})")
        self.status = status


_lib = None


def library() -> ctypes.CDLL:
    """The loaded libsanta.so; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(library_path):
            raise ImportError(f"{library_path} is missing: build it with "
                              "`python -m sampling_sparse_attention_amd.build`")
        lib = ctypes.CDLL(library_path)
        vp, i32, u64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_uint64, ctypes.c_size_t
        lib.santa_abi_version.restype = i32
        lib.santa_status_string.restype = ctypes.c_char_p
        lib.santa_status_string.argtypes = [ctypes.c_int]
        lib.santa_last_error.restype = ctypes.c_char_p
        lib.santa_workspace_layout_query.restype = ctypes.c_int
        lib.santa_workspace_layout_query.argtypes = [ctypes.POINTER(Shape), i32, i32,
                                                     ctypes.POINTER(WorkspaceLayout)]
        lib.santa_workspace_size.restype = ctypes.c_int
        lib.santa_workspace_size.argtypes = [ctypes.POINTER(Shape), i32, i32, ctypes.POINTER(sz)]
        lib.santa_workspace_init.restype = ctypes.c_int
        lib.santa_workspace_init.argtypes = [vp, sz, vp]
        lib.santa_decode_path.restype = i32
        lib.santa_decode_path.argtypes = [ctypes.POINTER(Shape), i32, i32]
        for name in ("santa_decode", "santa_score_pass", "santa_sample_pass", "santa_decode_flash"):
            fn = getattr(lib, name)
            fn.restype = ctypes.c_int
            fn.argtypes = [ctypes.POINTER(Shape), vp, vp, vp, vp, vp, i32, i32, u64, vp, vp, vp, sz, vp]
        _lib = lib
    return _lib


def _check(status: int, where: str) -> None:
    if status != 0:
        lib = library()
        detail = lib.santa_last_error().decode() or lib.santa_status_string(status).decode()
        raise SantaError(status, where, detail)


def make_shape(q: torch.Tensor, k_cache: torch.Tensor, block_table: Optional[torch.Tensor] = None,
               max_seq_len: Optional[int] = None, split_size: int = 0) -> Shape:
    """``santa_shape`` of torch tensors: q ``[B, Hq, d]``; a contiguous cache
    ``[B, n_max, Hkv, d]`` or, with ``block_table [B, pages_per_seq]``, a paged
    cache ``[num_pages, page_size, Hkv, d]``."""
    B, Hq, d = q.shape
    if block_table is None:
        _, n_max, Hkv, _ = k_cache.shape
        page_size, pages_per_seq, num_pages = 0, 0, 0
    else:
        num_pages, page_size, Hkv, _ = k_cache.shape
        pages_per_seq = block_table.shape[1]
        n_max = pages_per_seq * page_size
    if max_seq_len is not None:
        n_max = max_seq_len
    dtype = {torch.bfloat16: DTYPE_BF16, torch.float32: DTYPE_F32}.get(q.dtype, -1)
    st = k_cache.stride()
    return Shape(B, Hq, Hkv, d, n_max, page_size, pages_per_seq, num_pages, dtype, split_size,
                 st[0], st[1], st[2])


def santa_workspace_layout_query(shape: Shape, num_samples: int, mode: int) -> WorkspaceLayout:
    out = WorkspaceLayout()
    _check(library().santa_workspace_layout_query(ctypes.byref(shape), num_samples, mode,
                                                  ctypes.byref(out)), "santa_workspace_layout_query")
    return out


def santa_workspace_size(shape: Shape, num_samples: int, mode: int) -> int:
    out = ctypes.c_size_t()
    _check(library().santa_workspace_size(ctypes.byref(shape), num_samples, mode, ctypes.byref(out)),
           "santa_workspace_size")
    return out.value


def santa_workspace_init(workspace: torch.Tensor, stream=None) -> None:
    """Zero-fills a workspace on the device (``santa_workspace_init``)."""
    _check(library().santa_workspace_init(_ptr(workspace), workspace.numel() * workspace.element_size(),
                                          _stream_handle(stream)), "santa_workspace_init")


def santa_decode_path(shape: Shape, num_samples: int, mode: int) -> int:
    """1: ``santa_decode`` runs one fused kernel; 2: the score pass then the sample pass."""
    r = library().santa_decode_path(ctypes.byref(shape), num_samples, mode)
    if r < 0:
        _check(-r, "santa_decode_path")
    return r


def allocate_workspace(shape: Shape, num_samples: int, mode: int, device) -> torch.Tensor:
    """A workspace of the size the problem needs, initialised by ``santa_workspace_init``."""
    n = santa_workspace_size(shape, num_samples, mode)
    ws = torch.empty(max(n, 256), dtype=torch.uint8, device=device)
    santa_workspace_init(ws)
    return ws


def workspace_error(workspace: torch.Tensor) -> int:
    """The workspace's error word (nonzero: a bounded wait of a decode call gave up).
    Reads device memory: synchronises with the current stream."""
    return int(workspace[0:4].view(torch.int32).item())


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream_handle(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _call(name, shape, q, k_cache, v_cache, seq_lens, block_table, num_samples, mode, seed, o, idx,
          workspace, stream):
    fn = getattr(library(), name)
    _check(fn(ctypes.byref(shape), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(seq_lens),
              _ptr(block_table), int(num_samples), int(mode), ctypes.c_uint64(seed & (2 ** 64 - 1)),
              _ptr(o), _ptr(idx), _ptr(workspace), workspace.numel() * workspace.element_size(),
              _stream_handle(stream)), name)


def santa_decode(shape, q, k_cache, v_cache, seq_lens, block_table, num_samples, mode, seed, o, idx,
                 workspace, stream=None) -> None:
    """One SANTA decode step (``santa_decode`` of the C ABI)."""
    _call("santa_decode", shape, q, k_cache, v_cache, seq_lens, block_table, num_samples, mode,
          seed, o, idx, workspace, stream)


def santa_decode_flash(shape, q, k_cache, v_cache, seq_lens, block_table, num_samples, mode, seed, o, idx,
                       workspace, stream=None) -> None:
    """One S^2ANTA-flash decode step (``santa_decode_flash`` of the C ABI)."""
    _call("santa_decode_flash", shape, q, k_cache, v_cache, seq_lens, block_table, num_samples, mode,
          seed, o, idx, workspace, stream)


def santa_score_pass(shape, q, k_cache, v_cache, seq_lens, block_table, num_samples, mode, seed, o,
                     idx, workspace, stream=None) -> None:
    """First half of a decode step (``santa_score_pass`` of the C ABI)."""
    _call("santa_score_pass", shape, q, k_cache, v_cache, seq_lens, block_table, num_samples, mode,
          seed, o, idx, workspace, stream)


def santa_sample_pass(shape, q, k_cache, v_cache, seq_lens, block_table, num_samples, mode, seed, o,
                      idx, workspace, stream=None) -> None:
    """Second half of a decode step (``santa_sample_pass`` of the C ABI)."""
    _call("santa_sample_pass", shape, q, k_cache, v_cache, seq_lens, block_table, num_samples, mode,
          seed, o, idx, workspace, stream)


def decode(q, k_cache, v_cache, seq_lens, block_table=None, num_samples=256,
           mode=MODE_SYSTEMATIC, seed=0, *, max_seq_len=None, split_size=0, o=None, idx=None,
           workspace=None, stream=None):
    """Convenience wrapper: allocates ``o``, ``idx`` and the workspace with torch
    when not given, then calls ``santa_decode``.  Returns ``(o, idx)``."""
    shape = make_shape(q, k_cache, block_table, max_seq_len, split_size)
    B, Hq, d = q.shape
    if o is None:
        o = torch.empty((B, Hq, d), dtype=torch.float32, device=q.device)
    if idx is None:
        idx = torch.empty((B, Hq, num_samples), dtype=torch.int32, device=q.device)
    if workspace is None:
        workspace = allocate_workspace(shape, num_samples, mode, q.device)
    santa_decode(shape, q, k_cache, v_cache, seq_lens, block_table, num_samples, mode, seed, o, idx,
                 workspace, stream)
    return o, idx
