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
    "workspace_error", "validate", "Args", "santa_decode_args", "santa_workspace_status",
    "ALGO_PROP", "ALGO_FLASH", "FLAG_TWO_KERNEL", "santa_decode_noalloc", "santa_noalloc_init",
    "santa_noalloc_status", "santa_noalloc_scratch_bytes", "santa_decode_topk",
    "KtLayout", "santa_decode_bernoulli", "PPTable", "santa_pp_num_teams", "allocate_pp_table",
    "santa_pp_build", "santa_pp_workspace_size", "santa_pp_decode", "EXPORTED_SYMBOLS",
]

MODE_MULTINOMIAL = 0
MODE_STRATIFIED = 1
MODE_SYSTEMATIC = 2
DTYPE_BF16 = 0
DTYPE_F32 = 1
_DTYPE_CODE = {torch.bfloat16: DTYPE_BF16, torch.float32: DTYPE_F32}

EXPORTED_SYMBOLS = (
    "santa_abi_version", "santa_status_string", "santa_last_error",
    "santa_workspace_layout_query", "santa_workspace_size", "santa_workspace_init",
    "santa_decode_path", "santa_decode", "santa_score_pass", "santa_sample_pass", "santa_decode_flash",
    "santa_decode_args", "santa_workspace_status",
    "santa_noalloc_scratch_bytes", "santa_noalloc_init", "santa_decode_noalloc", "santa_noalloc_status",
    "santa_decode_topk", "santa_decode_bernoulli",
    "santa_pp_num_teams", "santa_pp_build", "santa_pp_workspace_size", "santa_pp_decode",
)
ALGO_PROP = 0
ALGO_FLASH = 1
FLAG_TWO_KERNEL = 1
PATH_FUSED = 1
PATH_TWO_KERNELS = 2
PATH_FUSED_TICKETS = 3

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


class Args(ctypes.Structure):
    """Mirror of ``santa_args``."""
    _fields_ = [
        ("shape", Shape), ("q", ctypes.c_void_p), ("k_cache", ctypes.c_void_p), ("v_cache", ctypes.c_void_p),
        ("seq_lens", ctypes.c_void_p), ("block_table", ctypes.c_void_p), ("num_samples", ctypes.c_int32),
        ("mode", ctypes.c_int32), ("seed", ctypes.c_uint64), ("o", ctypes.c_void_p), ("idx", ctypes.c_void_p),
        ("workspace", ctypes.c_void_p), ("workspace_bytes", ctypes.c_size_t), ("algorithm", ctypes.c_int32),
        ("flags", ctypes.c_uint32),
    ]


class KtLayout(ctypes.Structure):
    """Mirror of ``santa_kt_layout``."""
    _fields_ = [("stride_seq", ctypes.c_int64), ("stride_head", ctypes.c_int64), ("stride_feat", ctypes.c_int64)]


class PPTable(ctypes.Structure):
    """Mirror of ``santa_pp_table``."""
    _fields_ = [("packed_k", ctypes.c_void_p), ("packed_v", ctypes.c_void_p), ("rep_k", ctypes.c_void_p),
                ("team_start", ctypes.c_void_p), ("perm", ctypes.c_void_p)]


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
        lib.santa_decode_args.restype = ctypes.c_int
        lib.santa_decode_args.argtypes = [ctypes.POINTER(Args), vp]
        lib.santa_workspace_status.restype = ctypes.c_int
        lib.santa_workspace_status.argtypes = [vp, sz, vp, ctypes.POINTER(ctypes.c_uint32)]
        lib.santa_decode_topk.restype = ctypes.c_int
        lib.santa_decode_topk.argtypes = [ctypes.POINTER(Shape), vp, vp, vp, vp, vp, i32, vp, vp, vp, sz, vp]
        lib.santa_noalloc_scratch_bytes.restype = sz
        lib.santa_decode_bernoulli.restype = ctypes.c_int
        lib.santa_decode_bernoulli.argtypes = [ctypes.POINTER(Shape), vp, vp, ctypes.POINTER(KtLayout), vp, vp,
                                               i32, i32, u64, i32, vp, vp, vp, vp, sz, vp]
        lib.santa_pp_num_teams.restype = i32
        lib.santa_pp_num_teams.argtypes = [i32, i32, i32]
        lib.santa_pp_build.restype = ctypes.c_int
        lib.santa_pp_build.argtypes = [ctypes.POINTER(Shape), vp, vp, i32, i32, i32, ctypes.POINTER(PPTable), vp]
        lib.santa_pp_workspace_size.restype = ctypes.c_int
        lib.santa_pp_workspace_size.argtypes = [ctypes.POINTER(Shape), i32, i32, i32, i32, ctypes.POINTER(sz)]
        lib.santa_pp_decode.restype = ctypes.c_int
        lib.santa_pp_decode.argtypes = [ctypes.POINTER(Shape), vp, vp, vp, vp, i32, i32, i32, ctypes.POINTER(PPTable),
                                        i32, u64, vp, vp, vp, vp, sz, vp]
        lib.santa_noalloc_scratch_bytes.argtypes = []
        lib.santa_noalloc_init.restype = ctypes.c_int
        lib.santa_noalloc_init.argtypes = [vp]
        lib.santa_noalloc_status.restype = ctypes.c_int
        lib.santa_noalloc_status.argtypes = [vp, ctypes.POINTER(ctypes.c_uint32)]
        lib.santa_decode_noalloc.restype = ctypes.c_int
        lib.santa_decode_noalloc.argtypes = [ctypes.POINTER(Shape), vp, vp, vp, vp, vp, i32, i32, u64, vp, vp, vp]
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
    dtype = _DTYPE_CODE.get(q.dtype, -1)
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
    """1: ``santa_decode`` runs one fused kernel with every workgroup resident; 3: the fused
    kernel with items taken in start order (one group resident at a time); 2: the score
    pass then the sample pass."""
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


def validate(shape: Shape, q, k_cache, v_cache, seq_lens, block_table, num_samples, o, idx, workspace) -> None:
    """Checks that the tensors match ``shape`` and the layouts of ``include/santa.h``
    before anything reaches the library (the kernels trust the pointers they get:
    a cache of another dtype or stride would be read out of bounds).  Raises
    ``ValueError``."""
    def need(cond, msg):
        if not cond:
            raise ValueError(msg)

    tensors = {"q": q, "k_cache": k_cache, "v_cache": v_cache, "seq_lens": seq_lens, "o": o, "idx": idx}
    if workspace is not None:
        tensors["workspace"] = workspace
    if block_table is not None:
        tensors["block_table"] = block_table
    for name, t in tensors.items():
        need(isinstance(t, torch.Tensor), f"{name} must be a torch.Tensor")
    devices = {t.device for t in tensors.values()}
    need(len(devices) == 1, f"all tensors must be on one device (got {sorted(map(str, devices))})")
    need(q.dim() == 3 and q.is_contiguous(), "q must be a contiguous [B, Hq, d] tensor")
    B, Hq, d = q.shape
    need(q.dtype in _DTYPE_CODE, f"q must be bfloat16 or float32 (got {q.dtype})")
    need(shape.dtype == _DTYPE_CODE[q.dtype], "shape.dtype does not match q.dtype")
    need((shape.batch, shape.num_q_heads, shape.head_dim) == (B, Hq, d),
         f"shape (batch {shape.batch}, heads {shape.num_q_heads}, head_dim {shape.head_dim}) "
         f"does not match q {tuple(q.shape)}")
    need(k_cache.dtype == q.dtype and v_cache.dtype == q.dtype,
         f"k_cache and v_cache must have q's dtype {q.dtype} (got {k_cache.dtype}, {v_cache.dtype})")
    need(k_cache.dim() == 4, "k_cache must be 4-D ([B, n_max, Hkv, d] or [pages, page_size, Hkv, d])")
    need(v_cache.shape == k_cache.shape, f"v_cache shape {tuple(v_cache.shape)} differs from k_cache "
                                         f"{tuple(k_cache.shape)}")
    need(v_cache.stride() == k_cache.stride(), f"v_cache strides {v_cache.stride()} differ from k_cache "
                                               f"{k_cache.stride()}")
    need(k_cache.stride(-1) == 1, "the head dimension of the caches must be contiguous (stride 1)")
    need(k_cache.shape[2] == shape.num_kv_heads and k_cache.shape[3] == d,
         f"cache KV heads / head_dim {tuple(k_cache.shape[2:])} do not match the shape "
         f"({shape.num_kv_heads}, {d})")
    need(tuple(k_cache.stride()[:3]) == (shape.kv_stride_seq, shape.kv_stride_tok, shape.kv_stride_head),
         "shape's KV strides do not match k_cache.stride()")
    if shape.page_size == 0:
        need(block_table is None, "block_table given for a contiguous cache (shape.page_size == 0)")
        need(k_cache.shape[0] >= B and k_cache.shape[1] >= shape.max_seq_len,
             f"contiguous cache {tuple(k_cache.shape[:2])} smaller than (batch {B}, max_seq_len "
             f"{shape.max_seq_len})")
    else:
        need(block_table is not None, "a paged cache (shape.page_size > 0) needs block_table")
        need(block_table.dtype == torch.int32 and block_table.dim() == 2 and block_table.is_contiguous(),
             "block_table must be a contiguous int32 [B, pages_per_seq] tensor")
        need(tuple(block_table.shape) == (B, shape.pages_per_seq),
             f"block_table shape {tuple(block_table.shape)} is not (batch {B}, pages_per_seq "
             f"{shape.pages_per_seq})")
        need(k_cache.shape[0] == shape.num_pages and k_cache.shape[1] == shape.page_size,
             f"paged cache {tuple(k_cache.shape[:2])} is not (num_pages {shape.num_pages}, page_size "
             f"{shape.page_size})")
    need(seq_lens.dtype == torch.int32 and tuple(seq_lens.shape) == (B,) and seq_lens.is_contiguous(),
         "seq_lens must be a contiguous int32 [B] tensor")
    need(o.dtype == torch.float32 and tuple(o.shape) == (B, Hq, d) and o.is_contiguous(),
         "o must be a contiguous float32 [B, Hq, d] tensor")
    need(idx.dtype == torch.int32 and tuple(idx.shape) == (B, Hq, num_samples) and idx.is_contiguous(),
         f"idx must be a contiguous int32 [B, Hq, {num_samples}] tensor")
    need(workspace is None or workspace.is_contiguous(), "workspace must be contiguous")


def _call(name, shape, q, k_cache, v_cache, seq_lens, block_table, num_samples, mode, seed, o, idx,
          workspace, stream):
    validate(shape, q, k_cache, v_cache, seq_lens, block_table, num_samples, o, idx, workspace)
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


def santa_decode_args(shape, q, k_cache, v_cache, seq_lens, block_table, num_samples, mode, seed, o, idx,
                      workspace, algorithm=ALGO_PROP, flags=0, stream=None) -> None:
    """One decode step through the struct entry point (``santa_decode_args`` of the C ABI)."""
    validate(shape, q, k_cache, v_cache, seq_lens, block_table, num_samples, o, idx, workspace)
    a = Args(shape, q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(), seq_lens.data_ptr(),
             None if block_table is None else block_table.data_ptr(), int(num_samples), int(mode),
             seed & (2 ** 64 - 1), o.data_ptr(), idx.data_ptr(), workspace.data_ptr(),
             workspace.numel() * workspace.element_size(), int(algorithm), int(flags))
    _check(library().santa_decode_args(ctypes.byref(a), _stream_handle(stream)), "santa_decode_args")


def santa_workspace_status(workspace: torch.Tensor, stream=None) -> int:
    """The workspace's error word through the C ABI (``santa_workspace_status``); waits
    for the stream's enqueued work."""
    out = ctypes.c_uint32()
    _check(library().santa_workspace_status(_ptr(workspace), workspace.numel() * workspace.element_size(),
                                            _stream_handle(stream), ctypes.byref(out)), "santa_workspace_status")
    return out.value


def santa_decode_topk(shape, q, k_cache, v_cache, seq_lens, block_table, k, o, idx, workspace,
                      stream=None) -> None:
    """Top-k attention at budget k (``santa_decode_topk`` of the C ABI); the workspace is
    ``santa_workspace_size(shape, k, MODE_SYSTEMATIC)`` bytes."""
    validate(shape, q, k_cache, v_cache, seq_lens, block_table, k, o, idx, workspace)
    _check(library().santa_decode_topk(ctypes.byref(shape), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(seq_lens),
                                       _ptr(block_table), int(k), _ptr(o), _ptr(idx), _ptr(workspace),
                                       workspace.numel() * workspace.element_size(), _stream_handle(stream)),
           "santa_decode_topk")


def santa_decode_bernoulli(shape, q, k_t, v_cache, seq_lens, num_samples, mode, seed, num_bernoulli, o, idx,
                           feature_counts, workspace, stream=None) -> None:
    """Bernoulli qK^T with the mean group query, then SANTA (``santa_decode_bernoulli``
    of the C ABI).  ``k_t`` is K transposed, ``[B, Hkv, d, >= n_max]`` with tokens
    contiguous; ``shape`` describes the contiguous token-major ``v_cache``;
    ``feature_counts`` is a uint8 ``[B, Hkv, d]`` output."""
    validate(shape, q, v_cache, v_cache, seq_lens, None, num_samples, o, idx, workspace)
    B, Hq, d = q.shape
    if not isinstance(k_t, torch.Tensor) or k_t.device != q.device or k_t.dtype != q.dtype:
        raise ValueError("k_t must be a tensor of q's dtype on q's device")
    if k_t.dim() != 4 or k_t.stride(-1) != 1:
        raise ValueError("k_t must be a [B, Hkv, d, tokens] tensor with tokens contiguous")
    if k_t.shape[0] < B or k_t.shape[1] != shape.num_kv_heads or k_t.shape[2] != d or \
            k_t.shape[3] < shape.max_seq_len:
        raise ValueError(f"k_t shape {tuple(k_t.shape)} does not cover (batch {B}, Hkv {shape.num_kv_heads}, "
                         f"d {d}, max_seq_len {shape.max_seq_len})")
    if not isinstance(feature_counts, torch.Tensor) or feature_counts.dtype != torch.uint8 or \
            tuple(feature_counts.shape) != (B, shape.num_kv_heads, d) or not feature_counts.is_contiguous() or \
            feature_counts.device != q.device:
        raise ValueError(f"feature_counts must be a contiguous uint8 [{B}, {shape.num_kv_heads}, {d}] tensor")
    st = k_t.stride()
    kt = KtLayout(st[0], st[1], st[2])
    _check(library().santa_decode_bernoulli(ctypes.byref(shape), _ptr(q), _ptr(k_t), ctypes.byref(kt),
                                            _ptr(v_cache), _ptr(seq_lens), int(num_samples), int(mode),
                                            ctypes.c_uint64(seed & (2 ** 64 - 1)), int(num_bernoulli), _ptr(o),
                                            _ptr(idx), _ptr(feature_counts), _ptr(workspace),
                                            workspace.numel() * workspace.element_size(), _stream_handle(stream)),
           "santa_decode_bernoulli")


def santa_pp_num_teams(N: int, P: int, R: int) -> int:
    """Teams of a prompt of N tokens, contiguous parents of P, at most R teams each (-1: invalid)."""
    return int(library().santa_pp_num_teams(int(N), int(P), int(R)))


def allocate_pp_table(shape: Shape, N: int, P: int, R: int, dtype: torch.dtype, device) -> dict:
    """The device arrays of a SANTA++ team table (``santa_pp_table``) for ``shape``."""
    M = santa_pp_num_teams(N, P, R)
    if M < 1:
        raise ValueError(f"invalid team parameters N={N}, P={P}, R={R}")
    B, Hkv, d = shape.batch, shape.num_kv_heads, shape.head_dim
    return {"packed_k": torch.empty((B, Hkv, N, d), dtype=dtype, device=device),
            "packed_v": torch.empty((B, Hkv, N, d), dtype=dtype, device=device),
            "rep_k": torch.empty((B, Hkv, M, d), dtype=dtype, device=device),
            "team_start": torch.empty((B, Hkv, M + 1), dtype=torch.int32, device=device),
            "perm": torch.empty((B, Hkv, N), dtype=torch.int32, device=device),
            "N": N, "P": P, "R": R, "M": M}


def _pp_table(shape: Shape, table: dict, dtype, device) -> PPTable:
    B, Hkv, d = shape.batch, shape.num_kv_heads, shape.head_dim
    N, M = table["N"], table["M"]
    want = {"packed_k": ((B, Hkv, N, d), dtype), "packed_v": ((B, Hkv, N, d), dtype),
            "rep_k": ((B, Hkv, M, d), dtype), "team_start": ((B, Hkv, M + 1), torch.int32),
            "perm": ((B, Hkv, N), torch.int32)}
    for name, (shp, dt) in want.items():
        t = table[name]
        if not isinstance(t, torch.Tensor) or tuple(t.shape) != shp or t.dtype != dt or not t.is_contiguous() \
                or t.device != device:
            raise ValueError(f"team table {name} must be a contiguous {dt} {shp} tensor on {device}")
    return PPTable(*(table[name].data_ptr() for name in ("packed_k", "packed_v", "rep_k", "team_start", "perm")))


def santa_pp_build(shape, k_cache, v_cache, table: dict, stream=None) -> None:
    """Builds the SANTA++ team table from the first ``table["N"]`` rows of every
    sequence (``santa_pp_build`` of the C ABI)."""
    if k_cache.dtype not in _DTYPE_CODE or v_cache.dtype != k_cache.dtype or v_cache.stride() != k_cache.stride() \
            or v_cache.shape != k_cache.shape or k_cache.stride(-1) != 1 or k_cache.dim() != 4:
        raise ValueError("k_cache and v_cache must be [B, n_max, Hkv, d] of one dtype and layout")
    if shape.dtype != _DTYPE_CODE[k_cache.dtype] or tuple(k_cache.stride()[:3]) != \
            (shape.kv_stride_seq, shape.kv_stride_tok, shape.kv_stride_head):
        raise ValueError("shape does not describe k_cache")
    if k_cache.shape[0] < shape.batch or k_cache.shape[1] < shape.max_seq_len:
        raise ValueError("k_cache is smaller than the shape")
    tb = _pp_table(shape, table, k_cache.dtype, k_cache.device)
    _check(library().santa_pp_build(ctypes.byref(shape), _ptr(k_cache), _ptr(v_cache), int(table["N"]),
                                    int(table["P"]), int(table["R"]), ctypes.byref(tb), _stream_handle(stream)),
           "santa_pp_build")


def santa_pp_workspace_size(shape: Shape, N: int, P: int, R: int, K: int) -> int:
    out = ctypes.c_size_t()
    _check(library().santa_pp_workspace_size(ctypes.byref(shape), int(N), int(P), int(R), int(K), ctypes.byref(out)),
           "santa_pp_workspace_size")
    return out.value


def santa_pp_decode(shape, q, k_cache, v_cache, seq_lens, table: dict, K, seed, o, teams, corr, workspace,
                    stream=None) -> None:
    """One SANTA++ decode step (``santa_pp_decode`` of the C ABI): ``o`` [B, Hq, d],
    ``teams`` [B, Hq, K + 1] int32 (selected teams ascending, then the threshold
    team), ``corr`` [B, Hq, K] fp32 inclusion corrections."""
    validate(shape, q, k_cache, v_cache, seq_lens, None, int(K) + 1, o, teams, workspace)
    B, Hq, _ = q.shape
    if not isinstance(corr, torch.Tensor) or corr.dtype != torch.float32 or tuple(corr.shape) != (B, Hq, int(K)) \
            or not corr.is_contiguous() or corr.device != q.device:
        raise ValueError(f"corr must be a contiguous float32 [{B}, {Hq}, {K}] tensor on q's device")
    tb = _pp_table(shape, table, q.dtype, q.device)
    _check(library().santa_pp_decode(ctypes.byref(shape), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(seq_lens),
                                     int(table["N"]), int(table["P"]), int(table["R"]), ctypes.byref(tb), int(K),
                                     ctypes.c_uint64(seed & (2 ** 64 - 1)), _ptr(o), _ptr(teams), _ptr(corr),
                                     _ptr(workspace), workspace.numel() * workspace.element_size(),
                                     _stream_handle(stream)), "santa_pp_decode")


def santa_noalloc_scratch_bytes() -> int:
    """Bytes of the library's no-allocation scratch array."""
    return int(library().santa_noalloc_scratch_bytes())


def santa_noalloc_init(stream=None) -> None:
    """Zero-fills the current device's scratch array (``santa_noalloc_init``)."""
    _check(library().santa_noalloc_init(_stream_handle(stream)), "santa_noalloc_init")


def santa_decode_noalloc(shape, q, k_cache, v_cache, seq_lens, block_table, num_samples, mode, seed, o, idx,
                         stream=None) -> None:
    """``santa_decode`` on the library's own scratch array, allocating nothing
    (``santa_decode_noalloc`` of the C ABI)."""
    validate(shape, q, k_cache, v_cache, seq_lens, block_table, num_samples, o, idx, None)
    _check(library().santa_decode_noalloc(ctypes.byref(shape), _ptr(q), _ptr(k_cache), _ptr(v_cache),
                                          _ptr(seq_lens), _ptr(block_table), int(num_samples), int(mode),
                                          ctypes.c_uint64(seed & (2 ** 64 - 1)), _ptr(o), _ptr(idx),
                                          _stream_handle(stream)), "santa_decode_noalloc")


def santa_noalloc_status(stream=None) -> int:
    """The error word of the current device's scratch array (synchronises the stream)."""
    out = ctypes.c_uint32()
    _check(library().santa_noalloc_status(_stream_handle(stream), ctypes.byref(out)), "santa_noalloc_status")
    return out.value


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
