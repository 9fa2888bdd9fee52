"""ctypes binding of libdsa: argument marshalling only.

Every function here has the name of the C entry point it calls, checks the
torch tensors it is given (device, dtype, contiguity, shape), passes their
data pointers and torch's current HIP stream, and raises on a non-OK status.
All arithmetic happens in the HIP kernels behind the C ABI.  If libdsa.so is
missing the first call raises: there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
import threading
from typing import List, Optional, Sequence

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libdsa.so")

DSA_OK, DSA_ERR_INVALID_ARG, DSA_ERR_UNSUPPORTED, DSA_ERR_WORKSPACE, DSA_ERR_HIP = 0, -1, -2, -3, -4
DSA_F32, DSA_BF16, DSA_FP8_E4M3FN = 0, 1, 2
DSA_TOPK_MAX = 2048
DSA_MAX_SHARED_LAYERS = 8

EXPORTS = ("dsa_index_k_cache_write", "dsa_index_q_quant", "dsa_index_front_end", "dsa_index_scores", "dsa_topk_workspace_size", "dsa_topk", "dsa_index_topk",
           "dsa_index_scores_hist", "dsa_topk_after_hist", "sparse_mla_workspace_size",
           "sparse_mla_decode", "sparse_mla_prefill", "sparse_mla_decode_shared", "sparse_mla_decode_no_alloc",
           "dsa_gather_ceiling", "dsa_read_ceiling", "dsa_last_error",
           "dsa_abi_version")


class DsaError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__("libdsa status %d: %s" % (status, message))
        self.status = status


class dsa_layout(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("total_q", ctypes.c_int32), ("max_ctx", ctypes.c_int64),
                ("kv_indptr", ctypes.c_void_p), ("q_indptr", ctypes.c_void_p),
                ("block_table", ctypes.c_void_p), ("block_table_stride", ctypes.c_int32),
                ("page_size", ctypes.c_int32), ("cache_rows", ctypes.c_int64)]


class dsa_mla_layer(ctypes.Structure):
    _fields_ = [("q", ctypes.c_void_p), ("kv", ctypes.c_void_p), ("kv_scale", ctypes.c_float),
                ("out", ctypes.c_void_p), ("lse", ctypes.c_void_p)]


_lock = threading.Lock()
_lib = None


def load_library(path: str = LIB_PATH):
    """Load libdsa.so (raises if it has not been built)."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(path):
            raise RuntimeError("libdsa.so not found at %s: build it with "
                               "`python -m deepseek_sparse_mla_amd.build`" % path)
        lib = ctypes.CDLL(path)
        P, I, L, F, S = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t
        LP = ctypes.POINTER(dsa_layout)
        lib.dsa_index_scores.argtypes = [LP, I, I, I, P, P, P, I, P, L, P, L, P, L, P]
        lib.dsa_index_k_cache_write.argtypes = [L, I, P, L, P, P, L, I, P, P, L, P, L, L, P]
        lib.dsa_index_q_quant.argtypes = [L, I, I, P, L, P, P, L, I, P, P, P]
        lib.dsa_index_front_end.argtypes = [L, I, I, P, L, P, L, P, P, L, I, P, P, L, P, L, L, P, P, P]
        lib.dsa_topk_workspace_size.argtypes = [LP, L, I]
        lib.dsa_topk_workspace_size.restype = S
        lib.dsa_topk.argtypes = [LP, P, L, I, P, P, S, P]
        lib.dsa_index_topk.argtypes = [LP, I, I, I, P, P, P, I, P, L, P, L, P, L, I, P, P, S, P]
        lib.dsa_index_scores_hist.argtypes = [LP, I, I, I, P, P, P, I, P, L, P, L, P, L, I, P, S,
                                              ctypes.POINTER(ctypes.c_int), P]
        lib.dsa_topk_after_hist.argtypes = [LP, P, L, I, P, P, S, I, P]
        lib.sparse_mla_workspace_size.argtypes = [LP, I, I, I, I, I]
        lib.sparse_mla_workspace_size.restype = S
        mla = [LP, I, I, I, F, I, P, I, P, F, P, I, I, P, P, P, S, P]
        lib.sparse_mla_decode.argtypes = mla
        lib.sparse_mla_prefill.argtypes = mla
        lib.sparse_mla_decode_no_alloc.argtypes = mla[:15] + [P]
        lib.sparse_mla_decode_shared.argtypes = [LP, I, I, I, F, I, I, I, I,
                                                 ctypes.POINTER(dsa_mla_layer), P, I, P, S, P]
        lib.dsa_gather_ceiling.argtypes = [P, L, I, P, L, I, P, P]
        lib.dsa_read_ceiling.argtypes = [P, L, P, L, L, I, I, P, P]
        for f in (lib.dsa_index_k_cache_write, lib.dsa_index_q_quant, lib.dsa_index_front_end,
                  lib.dsa_index_scores, lib.dsa_topk, lib.dsa_index_topk, lib.dsa_index_scores_hist,
                  lib.dsa_topk_after_hist, lib.sparse_mla_decode, lib.sparse_mla_prefill,
                  lib.sparse_mla_decode_shared, lib.sparse_mla_decode_no_alloc, lib.dsa_gather_ceiling, lib.dsa_read_ceiling,
                  lib.dsa_abi_version):
            f.restype = I
        lib.dsa_last_error.restype = ctypes.c_char_p
        lib.dsa_last_error.argtypes = []
        lib.dsa_abi_version.argtypes = []
        _lib = lib
        return lib


def _check(lib, st: int):
    if st != DSA_OK:
        raise DsaError(st, lib.dsa_last_error().decode())


def _dt(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return DSA_F32
    if t.dtype == torch.bfloat16:
        return DSA_BF16
    if t.dtype in (torch.uint8, torch.float8_e4m3fn):
        return DSA_FP8_E4M3FN
    raise TypeError("unsupported dtype %s" % t.dtype)


def _dev(t: Optional[torch.Tensor], name: str, dtype=None, contiguous=True):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("%s must be a device tensor" % name)
    if dtype is not None and t.dtype not in (dtype if isinstance(dtype, tuple) else (dtype,)):
        raise TypeError("%s must have dtype %s, got %s" % (name, dtype, t.dtype))
    if contiguous and not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    return t.data_ptr()


def _stream(stream) -> int:
    if stream is None:
        stream = torch.cuda.current_stream()
    return int(stream.cuda_stream)


class Layout:
    """Ragged layout (mirrors dsa_layout); tensors stay referenced while the object lives.

    Paged caches: block_table int32 [B, pages] of physical page ids, page_size tokens per
    page, cache_rows rows in every per-token cache; top-k then returns physical rows and
    sparse MLA reads them."""

    def __init__(self, kv_indptr: torch.Tensor, q_indptr: Optional[torch.Tensor], total_q: int,
                 max_ctx: int, block_table: Optional[torch.Tensor] = None, page_size: int = 0,
                 cache_rows: int = 0):
        _dev(kv_indptr, "kv_indptr", torch.int64)
        _dev(q_indptr, "q_indptr", torch.int32)
        _dev(block_table, "block_table", torch.int32)
        self.kv_indptr = kv_indptr
        self.q_indptr = q_indptr
        self.block_table = block_table
        self.batch = kv_indptr.numel() - 1
        self.total_q = int(total_q)
        self.max_ctx = int(max_ctx)
        if block_table is not None and (block_table.dim() != 2 or block_table.shape[0] != self.batch):
            raise ValueError("block_table must be [batch, pages]")
        self.c = dsa_layout(self.batch, self.total_q, self.max_ctx, kv_indptr.data_ptr(),
                            q_indptr.data_ptr() if q_indptr is not None else None,
                            block_table.data_ptr() if block_table is not None else None,
                            int(block_table.shape[1]) if block_table is not None else 0,
                            int(page_size), int(cache_rows))

    @staticmethod
    def of_case(case) -> "Layout":
        return Layout(case.kv_indptr, case.q_indptr, case.T, case.max_ctx)


def _rope_args(positions, cos_sin, n):
    if cos_sin is None:
        return None, None, 0
    if positions is None or positions.numel() != n:
        raise ValueError("rope needs one int64 position per row")
    if cos_sin.dim() != 2 or cos_sin.shape[1] != 64:
        raise ValueError("cos_sin must be [rows, 64] (32 cos then 32 sin)")
    return (_dev(positions, "positions", torch.int64), _dev(cos_sin, "cos_sin", torch.float32),
            cos_sin.shape[0])


def _row_stride_bytes(x: torch.Tensor, name: str) -> int:
    if x.stride(-1) != 1 or (x.dim() == 3 and x.shape[1] > 1 and x.stride(1) != x.shape[2]):
        raise ValueError("%s must have unit stride inside a row" % name)
    return x.stride(0) * x.element_size()


def dsa_index_k_cache_write(k: torch.Tensor, slots: torch.Tensor, cache: torch.Tensor,
                            cache_scale: torch.Tensor, positions: Optional[torch.Tensor] = None,
                            cos_sin: Optional[torch.Tensor] = None, rope_off: int = 0,
                            cache_row_stride: Optional[int] = None, cache_scale_stride: int = 1,
                            cache_rows: Optional[int] = None, stream=None) -> None:
    """Rope (optional) + fp8 quantise k [n, 128] (bf16 / fp32, rows may be strided) into cache
    rows slots[r] (negative = skip).  cache: uint8 [rows, 128] codes plane (or a raw byte buffer
    with cache_row_stride and cache_rows given); cache_scale: fp32 with cache_scale_stride."""
    lib = load_library()
    n = k.shape[0]
    if k.shape[-1] != 128:
        raise ValueError("index keys are 128 wide")
    if cache_row_stride is None:
        cache_row_stride = cache.stride(0) * cache.element_size()
    if cache_rows is None:
        cache_rows = cache.shape[0]
    if slots.numel() != n:
        raise ValueError("slots must hold one cache row per key")
    if cache_rows > 0:
        need_c = (cache_rows - 1) * int(cache_row_stride) + 128
        need_s = ((cache_rows - 1) * int(cache_scale_stride) + 1) * 4
        if cache.numel() * cache.element_size() < need_c or \
                cache_scale.numel() * cache_scale.element_size() < need_s:
            raise ValueError("cache or cache_scale smaller than cache_rows entries")
    pos, cs, rope_rows = _rope_args(positions, cos_sin, n)
    st = lib.dsa_index_k_cache_write(n, _dt(k), _dev(k, "k", contiguous=False), _row_stride_bytes(k, "k"),
                                     pos, cs, rope_rows, int(rope_off), _dev(slots, "slots", torch.int64),
                                     _dev(cache, "cache", (torch.uint8, torch.float8_e4m3fn), contiguous=False),
                                     int(cache_row_stride),
                                     _dev(cache_scale, "cache_scale", (torch.float32, torch.uint8), contiguous=False),
                                     int(cache_scale_stride), int(cache_rows), _stream(stream))
    _check(lib, st)


def dsa_index_q_quant(q: torch.Tensor, positions: Optional[torch.Tensor] = None,
                      cos_sin: Optional[torch.Tensor] = None, rope_off: int = 0,
                      q_fp8: Optional[torch.Tensor] = None, q_scale: Optional[torch.Tensor] = None,
                      stream=None):
    """Rope (optional) + fp8 quantise index queries q [T, H_I, 128] per (row, head).
    Returns (codes uint8 [T, H_I, 128], scales fp32 [T, H_I])."""
    lib = load_library()
    T, H_I, D = q.shape
    if D != 128:
        raise ValueError("index heads are 128 wide")
    if q_fp8 is None:
        q_fp8 = torch.empty((T, H_I, D), dtype=torch.uint8, device=q.device)
    if q_scale is None:
        q_scale = torch.empty((T, H_I), dtype=torch.float32, device=q.device)
    if tuple(q_fp8.shape) != (T, H_I, D) or tuple(q_scale.shape) != (T, H_I):
        raise ValueError("q_fp8 must be [T, H_I, 128] and q_scale [T, H_I]")
    pos, cs, rope_rows = _rope_args(positions, cos_sin, T)
    st = lib.dsa_index_q_quant(T, H_I, _dt(q), _dev(q, "q", contiguous=False), _row_stride_bytes(q, "q"),
                               pos, cs, rope_rows, int(rope_off),
                               _dev(q_fp8, "q_fp8", (torch.uint8, torch.float8_e4m3fn)),
                               _dev(q_scale, "q_scale", torch.float32), _stream(stream))
    _check(lib, st)
    return q_fp8, q_scale


def dsa_index_front_end(q: torch.Tensor, k: torch.Tensor, slots: torch.Tensor, cache: torch.Tensor,
                        cache_scale: torch.Tensor, positions: Optional[torch.Tensor] = None,
                        cos_sin: Optional[torch.Tensor] = None, rope_off: int = 0,
                        q_fp8: Optional[torch.Tensor] = None, q_scale: Optional[torch.Tensor] = None,
                        cache_row_stride: Optional[int] = None, cache_scale_stride: int = 1,
                        cache_rows: Optional[int] = None, stream=None):
    """One launch of both writer calls for T new tokens: q [T, H_I, 128] -> (codes, scales) as
    dsa_index_q_quant returns them; k [T, 128] -> cache rows slots[t], as
    dsa_index_k_cache_write."""
    lib = load_library()
    T, H_I, D = q.shape
    if D != 128 or tuple(k.shape) != (T, 128):
        raise ValueError("q must be [T, H_I, 128] and k [T, 128]")
    if q.dtype != k.dtype:
        raise TypeError("q and k must share a dtype")
    if q_fp8 is None:
        q_fp8 = torch.empty((T, H_I, D), dtype=torch.uint8, device=q.device)
    if q_scale is None:
        q_scale = torch.empty((T, H_I), dtype=torch.float32, device=q.device)
    if tuple(q_fp8.shape) != (T, H_I, D) or tuple(q_scale.shape) != (T, H_I):
        raise ValueError("q_fp8 must be [T, H_I, 128] and q_scale [T, H_I]")
    if cache_row_stride is None:
        cache_row_stride = cache.stride(0) * cache.element_size()
    if cache_rows is None:
        cache_rows = cache.shape[0]
    if slots.numel() != T:
        raise ValueError("slots must hold one cache row per key")
    if cache_rows > 0:
        need_c = (cache_rows - 1) * int(cache_row_stride) + 128
        need_s = ((cache_rows - 1) * int(cache_scale_stride) + 1) * 4
        if cache.numel() * cache.element_size() < need_c or \
                cache_scale.numel() * cache_scale.element_size() < need_s:
            raise ValueError("cache or cache_scale smaller than cache_rows entries")
    pos, cs, rope_rows = _rope_args(positions, cos_sin, T)
    st = lib.dsa_index_front_end(T, H_I, _dt(q), _dev(q, "q", contiguous=False), _row_stride_bytes(q, "q"),
                                 _dev(k, "k", contiguous=False), _row_stride_bytes(k, "k"), pos, cs,
                                 rope_rows, int(rope_off), _dev(slots, "slots", torch.int64),
                                 _dev(cache, "cache", (torch.uint8, torch.float8_e4m3fn), contiguous=False),
                                 int(cache_row_stride),
                                 _dev(cache_scale, "cache_scale", (torch.float32, torch.uint8), contiguous=False),
                                 int(cache_scale_stride), int(cache_rows),
                                 _dev(q_fp8, "q_fp8", (torch.uint8, torch.float8_e4m3fn)),
                                 _dev(q_scale, "q_scale", torch.float32), _stream(stream))
    _check(lib, st)
    return q_fp8, q_scale


def score_pitch(max_ctx: int) -> int:
    """Default row pitch of a score array: max_ctx rounded up to 32 floats (every row starts
    on a 128-byte line)."""
    return (int(max_ctx) + 31) & ~31


def dsa_index_scores(layout: Layout, q: torch.Tensor, w: torch.Tensor, k: torch.Tensor,
                     k_scale: Optional[torch.Tensor] = None, q_scale: Optional[torch.Tensor] = None,
                     scores: Optional[torch.Tensor] = None, ld: Optional[int] = None,
                     k_row_stride: Optional[int] = None, k_scale_stride: int = 1,
                     k_dtype: Optional[int] = None, stream=None) -> torch.Tensor:
    """Indexer scores [T, ld] fp32 (ld defaults to score_pitch(max_ctx)).  q: [T, H_I, D_I];
    k: [rows, D_I] (or a raw uint8 byte buffer with k_row_stride bytes per row and k_dtype
    given)."""
    lib = load_library()
    T, H_I, D_I = q.shape
    kd = _dt(k) if k_dtype is None else k_dtype
    if k_row_stride is None:
        k_row_stride = k.shape[-1] * k.element_size()
    if ld is None:
        ld = scores.shape[1] if scores is not None else score_pitch(layout.max_ctx)
    if scores is None:
        scores = torch.empty((T, ld), dtype=torch.float32, device=q.device)
    _dev(scores, "scores", torch.float32)
    st = lib.dsa_index_scores(ctypes.byref(layout.c), H_I, D_I, _dt(q), _dev(q, "q"),
                              _dev(q_scale, "q_scale", torch.float32), _dev(w, "w", torch.float32),
                              kd, _dev(k, "k", contiguous=False), int(k_row_stride),
                              _dev(k_scale, "k_scale", torch.float32, contiguous=False),
                              int(k_scale_stride), scores.data_ptr(), int(ld), _stream(stream))
    _check(lib, st)
    return scores


def dsa_topk_workspace_size(layout: Layout, ld: int, k: int) -> int:
    return int(load_library().dsa_topk_workspace_size(ctypes.byref(layout.c), int(ld), int(k)))


def topk_workspace(layout: Layout, ld: int, k: int, device="cuda") -> Optional[torch.Tensor]:
    """A zero-filled top-k workspace of the size the library asks for (None if none)."""
    n = dsa_topk_workspace_size(layout, ld, k)
    return torch.zeros(n, dtype=torch.uint8, device=device) if n else None


def dsa_topk(layout: Layout, scores: torch.Tensor, k: int, indices: Optional[torch.Tensor] = None,
             workspace: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Top-k positions int32 [T, k]: the first min(k, n) positions under (score desc, position
    asc), listed in ascending position order, then -1 padding."""
    lib = load_library()
    T, ld = scores.shape
    if indices is None:
        indices = torch.empty((T, k), dtype=torch.int32, device=scores.device)
    if workspace is None:
        workspace = topk_workspace(layout, ld, k, scores.device)
    st = lib.dsa_topk(ctypes.byref(layout.c), _dev(scores, "scores", torch.float32), int(ld), int(k),
                      _dev(indices, "indices", torch.int32), _dev(workspace, "workspace"),
                      workspace.numel() if workspace is not None else 0, _stream(stream))
    _check(lib, st)
    return indices


def dsa_index_topk(layout: Layout, q: torch.Tensor, w: torch.Tensor, k: torch.Tensor, k_top: int,
                   k_scale: Optional[torch.Tensor] = None, q_scale: Optional[torch.Tensor] = None,
                   scores: Optional[torch.Tensor] = None, indices: Optional[torch.Tensor] = None,
                   workspace: Optional[torch.Tensor] = None, ld: Optional[int] = None,
                   k_row_stride: Optional[int] = None, k_scale_stride: int = 1,
                   k_dtype: Optional[int] = None, stream=None):
    """Indexer scores and top-k in one call (the top-k's histogram built by the indexer where
    the kernels allow): returns (scores [T, ld] fp32, indices [T, k_top] int32)."""
    lib = load_library()
    T, H_I, D_I = q.shape
    kd = _dt(k) if k_dtype is None else k_dtype
    if k_row_stride is None:
        k_row_stride = k.shape[-1] * k.element_size()
    if ld is None:
        ld = scores.shape[1] if scores is not None else score_pitch(layout.max_ctx)
    if scores is None:
        scores = torch.empty((T, ld), dtype=torch.float32, device=q.device)
    if indices is None:
        indices = torch.empty((T, k_top), dtype=torch.int32, device=q.device)
    if workspace is None:
        workspace = topk_workspace(layout, ld, k_top, q.device)
    st = lib.dsa_index_topk(ctypes.byref(layout.c), H_I, D_I, _dt(q), _dev(q, "q"),
                            _dev(q_scale, "q_scale", torch.float32), _dev(w, "w", torch.float32),
                            kd, _dev(k, "k", contiguous=False), int(k_row_stride),
                            _dev(k_scale, "k_scale", torch.float32, contiguous=False), int(k_scale_stride),
                            _dev(scores, "scores", torch.float32), int(ld), int(k_top),
                            _dev(indices, "indices", torch.int32), _dev(workspace, "workspace"),
                            workspace.numel() if workspace is not None else 0, _stream(stream))
    _check(lib, st)
    return scores, indices


def dsa_index_scores_hist(layout: Layout, q: torch.Tensor, w: torch.Tensor, k: torch.Tensor, k_top: int,
                          workspace: Optional[torch.Tensor], k_scale: Optional[torch.Tensor] = None,
                          q_scale: Optional[torch.Tensor] = None, scores: Optional[torch.Tensor] = None,
                          ld: Optional[int] = None, k_row_stride: Optional[int] = None, k_scale_stride: int = 1,
                          k_dtype: Optional[int] = None, stream=None):
    """The first half of dsa_index_topk: scores, plus the top-k histogram in `workspace` where
    the kernels fold it in.  Returns (scores [T, ld] fp32, hist_built) for dsa_topk_after_hist."""
    lib = load_library()
    T, H_I, D_I = q.shape
    kd = _dt(k) if k_dtype is None else k_dtype
    if k_row_stride is None:
        k_row_stride = k.shape[-1] * k.element_size()
    if ld is None:
        ld = scores.shape[1] if scores is not None else score_pitch(layout.max_ctx)
    if scores is None:
        scores = torch.empty((T, ld), dtype=torch.float32, device=q.device)
    built = ctypes.c_int(0)
    st = lib.dsa_index_scores_hist(ctypes.byref(layout.c), H_I, D_I, _dt(q), _dev(q, "q"),
                                   _dev(q_scale, "q_scale", torch.float32), _dev(w, "w", torch.float32),
                                   kd, _dev(k, "k", contiguous=False), int(k_row_stride),
                                   _dev(k_scale, "k_scale", torch.float32, contiguous=False), int(k_scale_stride),
                                   _dev(scores, "scores", torch.float32), int(ld), int(k_top),
                                   _dev(workspace, "workspace"), workspace.numel() if workspace is not None else 0,
                                   ctypes.byref(built), _stream(stream))
    _check(lib, st)
    return scores, int(built.value)


def dsa_topk_after_hist(layout: Layout, scores: torch.Tensor, k: int, hist_built: int,
                        indices: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                        stream=None) -> torch.Tensor:
    """The second half of dsa_index_topk: the selection, on the histogram that
    dsa_index_scores_hist left in `workspace` when it returned hist_built = 1."""
    lib = load_library()
    T, ld = scores.shape
    if indices is None:
        indices = torch.empty((T, k), dtype=torch.int32, device=scores.device)
    st = lib.dsa_topk_after_hist(ctypes.byref(layout.c), _dev(scores, "scores", torch.float32), int(ld), int(k),
                                 _dev(indices, "indices", torch.int32), _dev(workspace, "workspace"),
                                 workspace.numel() if workspace is not None else 0, int(hist_built),
                                 _stream(stream))
    _check(lib, st)
    return indices


def sparse_mla_workspace_size(layout: Layout, H: int, D_c: int, D_r: int, k: int, n_layers: int = 1) -> int:
    return int(load_library().sparse_mla_workspace_size(ctypes.byref(layout.c), H, D_c, D_r, k, n_layers))


def mla_workspace(layout: Layout, H: int, D_c: int, D_r: int, k: int, n_layers: int = 1,
                  device="cuda") -> Optional[torch.Tensor]:
    """A zero-filled workspace of the size the library asks for (None if it needs none)."""
    n = sparse_mla_workspace_size(layout, H, D_c, D_r, k, n_layers)
    return torch.zeros(n, dtype=torch.uint8, device=device) if n else None


def _mla(fn_name, layout: Layout, q, kv, indices, sm_scale, D_c, kv_scale=1.0, out=None, lse=None,
         out_dtype=None, workspace=None, kv_dtype=None, stream=None):
    lib = load_library()
    T, H, Dqk = q.shape
    k = indices.shape[1]
    if out_dtype is None:
        out_dtype = torch.float32 if q.dtype == torch.float32 else torch.bfloat16
    if out is None:
        out = torch.empty((T, H, D_c), dtype=out_dtype, device=q.device)
    if workspace is None:
        workspace = mla_workspace(layout, H, D_c, Dqk - D_c, k, 1, q.device)
    kd = _dt(kv) if kv_dtype is None else kv_dtype
    st = getattr(lib, fn_name)(ctypes.byref(layout.c), H, D_c, Dqk - D_c, float(sm_scale), _dt(q),
                               _dev(q, "q"), kd, _dev(kv, "kv"), float(kv_scale),
                               _dev(indices, "indices", torch.int32), k, _dt(out), _dev(out, "out"),
                               _dev(lse, "lse", torch.float32), _dev(workspace, "workspace"),
                               workspace.numel() if workspace is not None else 0, _stream(stream))
    _check(lib, st)
    return out


def sparse_mla_decode(layout: Layout, q, kv, indices, sm_scale, D_c, kv_scale=1.0, out=None, lse=None,
                      out_dtype=None, workspace=None, stream=None) -> torch.Tensor:
    """Sparse MLA output [T, H, D_c]; q [T, H, D_c+D_r]; kv [rows, D_c+D_r]."""
    return _mla("sparse_mla_decode", layout, q, kv, indices, sm_scale, D_c, kv_scale, out, lse,
                out_dtype, workspace, stream=stream)


def sparse_mla_decode_no_alloc(layout: Layout, q, kv, indices, sm_scale, D_c, kv_scale=1.0, out=None, lse=None,
                               out_dtype=None, stream=None) -> torch.Tensor:
    """sparse_mla_decode with the split partials in the library's static scratch (no workspace);
    with `out` given, the call allocates nothing."""
    lib = load_library()
    T, H, Dqk = q.shape
    k = indices.shape[1]
    if out_dtype is None:
        out_dtype = torch.float32 if q.dtype == torch.float32 else torch.bfloat16
    if out is None:
        out = torch.empty((T, H, D_c), dtype=out_dtype, device=q.device)
    st = lib.sparse_mla_decode_no_alloc(ctypes.byref(layout.c), H, D_c, Dqk - D_c, float(sm_scale), _dt(q),
                                        _dev(q, "q"), _dt(kv), _dev(kv, "kv"), float(kv_scale),
                                        _dev(indices, "indices", torch.int32), k, _dt(out), _dev(out, "out"),
                                        _dev(lse, "lse", torch.float32), _stream(stream))
    _check(lib, st)
    return out


def dsa_gather_ceiling(rows: torch.Tensor, indices: torch.Tensor, sink: torch.Tensor, stream=None) -> None:
    """Measurement aid: gather the rows of `rows` ([n, 576] fp8 bytes or [n, 576] bf16) that
    `indices` ([T, k] int32, absolute rows, -1 = none) select, with no arithmetic."""
    lib = load_library()
    n = rows.shape[0]
    rb = rows.shape[1] * rows.element_size()
    T, k = indices.shape
    st = lib.dsa_gather_ceiling(_dev(rows, "rows"), n, rb, _dev(indices, "indices", torch.int32), T, k,
                                _dev(sink, "sink"), _stream(stream))
    _check(lib, st)


def dsa_read_ceiling(k: torch.Tensor, k_scale: torch.Tensor, sink: torch.Tensor, n_tokens: Optional[int] = None,
                     pattern: int = 0, blocks: int = 512, k_row_stride: Optional[int] = None,
                     k_scale_stride: int = 1, stream=None) -> None:
    """Measurement aid: stream the index cache's first n_tokens rows (keys and scales) the way
    the decode indexer does, with no arithmetic; sink (>= blocks int32 words) receives one xor of
    the words read per block."""
    if sink.numel() * sink.element_size() < 4 * int(blocks):
        raise ValueError("sink must hold one 32-bit word per block")
    lib = load_library()
    n = k.shape[0] if n_tokens is None else int(n_tokens)
    if k_row_stride is None:
        k_row_stride = k.shape[-1] * k.element_size()
    st = lib.dsa_read_ceiling(_dev(k, "k", contiguous=False), int(k_row_stride), _dev(k_scale, "k_scale"),
                              int(k_scale_stride), n, int(pattern), int(blocks), _dev(sink, "sink"), _stream(stream))
    _check(lib, st)


def sparse_mla_prefill(layout: Layout, q, kv, indices, sm_scale, D_c, kv_scale=1.0, out=None, lse=None,
                       out_dtype=None, workspace=None, stream=None) -> torch.Tensor:
    return _mla("sparse_mla_prefill", layout, q, kv, indices, sm_scale, D_c, kv_scale, out, lse,
                out_dtype, workspace, stream=stream)


def sparse_mla_decode_shared(layout: Layout, qs: Sequence[torch.Tensor], kvs: Sequence[torch.Tensor],
                             kv_scales: Sequence[float], indices: torch.Tensor, sm_scale: float, D_c: int,
                             outs: Optional[List[torch.Tensor]] = None,
                             lses: Optional[List[Optional[torch.Tensor]]] = None, out_dtype=None,
                             workspace=None, stream=None) -> List[torch.Tensor]:
    """Several layers' sparse MLA over one index set, one launch."""
    lib = load_library()
    nl = len(qs)
    if not (len(kvs) == nl == len(kv_scales)):
        raise ValueError("qs, kvs and kv_scales must have one entry per layer")
    T, H, Dqk = qs[0].shape
    k = indices.shape[1]
    if out_dtype is None:
        out_dtype = torch.float32 if qs[0].dtype == torch.float32 else torch.bfloat16
    if outs is None:
        outs = [torch.empty((T, H, D_c), dtype=out_dtype, device=qs[0].device) for _ in range(nl)]
    if lses is None:
        lses = [None] * nl
    arr = (dsa_mla_layer * max(nl, 1))()
    for l in range(nl):
        if qs[l].shape != qs[0].shape or kvs[l].dtype != kvs[0].dtype or qs[l].dtype != qs[0].dtype:
            raise ValueError("every layer must have the same shapes and dtypes")
        arr[l] = dsa_mla_layer(_dev(qs[l], "q"), _dev(kvs[l], "kv"), float(kv_scales[l]),
                               _dev(outs[l], "out"), _dev(lses[l], "lse", torch.float32))
    if workspace is None:
        workspace = mla_workspace(layout, H, D_c, Dqk - D_c, k, nl, qs[0].device)
    st = lib.sparse_mla_decode_shared(ctypes.byref(layout.c), H, D_c, Dqk - D_c, float(sm_scale),
                                      _dt(qs[0]), _dt(kvs[0]), _dt(outs[0]), nl, arr,
                                      _dev(indices, "indices", torch.int32), k,
                                      _dev(workspace, "workspace"),
                                      workspace.numel() if workspace is not None else 0, _stream(stream))
    _check(lib, st)
    return outs


def dsa_abi_version() -> int:
    return int(load_library().dsa_abi_version())
