"""fp64 CPU oracle for the DSA sparse-attention path (test infrastructure).

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product library never does, and
this package imports nothing from it: the two share no code.

The arithmetic lives in ``dsa_oracle.c`` (plain C, fp64, OpenMP over query
rows); this module only builds it with gcc, marshals numpy arrays and composes
the per-stage functions into the shared-index path.

Citations (reference pages, by title and section):
  * "GLM-5.2 架构解剖" (GLM-5.2 anatomy), 结构全图 (full structure diagram),
    Indexer and sparse-MLA boxes -- shapes, index-cache format, top-2048.
  * same page, 核心机制·层调度 (layer scheduling) -- shared layers reuse the
    indices of the last full layer unchanged (``index_share``).
  * same page, ATOM 侧 (ATOM-side optimisations), stable_topk -- ties are
    resolved deterministically (here: lower position first).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "dsa_oracle.c")
_LIB = os.path.join(_HERE, "_liboracle.so")
_lock = threading.Lock()
_lib = None

F32, BF16, FP8 = 0, 1, 2  # oracle-local dtype codes (see dsa_oracle.c)


def build(force: bool = False) -> str:
    """Compile dsa_oracle.c into _liboracle.so with gcc (OpenMP, -O2, IEEE, no contraction)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-std=c99", "-ffp-contract=off", "-fopenmp", "-fPIC", "-shared", _SRC,
               "-o", tmp, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    with _lock:
        if _lib is None:
            build()
            lib = ctypes.CDLL(_LIB)
            P, I, L, D = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_double
            lib.orc_decode_bf16.argtypes = [ctypes.c_uint16]
            lib.orc_decode_bf16.restype = D
            lib.orc_decode_fp8_e4m3fn.argtypes = [ctypes.c_uint8]
            lib.orc_decode_fp8_e4m3fn.restype = D
            lib.orc_visible_counts.argtypes = [I, P, P, L, P]
            lib.orc_index_scores.argtypes = [I, P, P, L, I, I, I, P, P, P, I, P, L, P, L, P, L, P, P, L, L]
            lib.orc_topk.argtypes = [L, P, P, L, I, P]
            lib.orc_sparse_mla.argtypes = [I, P, P, L, I, I, I, D, I, P, I, P, D, P, I, P, P, L]
            lib.orc_num_threads.argtypes = []
            lib.orc_encode_fp8_e4m3fn.argtypes = [D]
            lib.orc_encode_fp8_e4m3fn.restype = ctypes.c_uint8
            lib.orc_pow2_scale.argtypes = [D]
            lib.orc_pow2_scale.restype = D
            F = ctypes.c_float
            lib.orc_rope_pair_f32.argtypes = [F, F, F, F, P, P]
            lib.orc_rope_pair_f32.restype = None
            lib.orc_index_quant.argtypes = [L, I, I, I, P, P, P, L, I, I, P, P, L, P, L]
            lib.orc_index_quant.restype = I
            for f in (lib.orc_visible_counts, lib.orc_index_scores, lib.orc_topk,
                      lib.orc_sparse_mla, lib.orc_num_threads):
                f.restype = I
            _lib = lib
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return None if a is None else np.ascontiguousarray(a, dtype=dtype)


def _dt_code(a) -> int:
    """Map the storage of an input array to an oracle dtype code.

    float32 -> F32; uint16 (raw bf16 bits) -> BF16; uint8 (raw E4M3FN codes) -> FP8.
    """
    if a.dtype == np.float32:
        return F32
    if a.dtype == np.uint16:
        return BF16
    if a.dtype == np.uint8:
        return FP8
    raise TypeError("oracle inputs are float32, uint16 (bf16 bits) or uint8 (fp8 codes), got %s" % a.dtype)


def _check(rc: int, what: str):
    if rc != 0:
        raise ValueError("oracle %s failed with code %d" % (what, rc))


def decode_bf16(bits) -> np.ndarray:
    """Decode raw bf16 bit patterns (uint16) to float64, one by one."""
    lib = _load()
    flat = np.asarray(bits, dtype=np.uint16).ravel()
    return np.array([lib.orc_decode_bf16(int(b)) for b in flat], dtype=np.float64).reshape(np.shape(bits))


def decode_fp8(codes) -> np.ndarray:
    """Decode raw OCP E4M3FN codes (uint8) to float64, one by one."""
    lib = _load()
    flat = np.asarray(codes, dtype=np.uint8).ravel()
    return np.array([lib.orc_decode_fp8_e4m3fn(int(b)) for b in flat], dtype=np.float64).reshape(np.shape(codes))


def visible_counts(kv_indptr, q_indptr, T) -> np.ndarray:
    """n_i for every query row under the causal ragged layout."""
    lib = _load()
    kv = _c(kv_indptr, np.int64)
    qi = _c(q_indptr, np.int32)
    out = np.zeros(T, dtype=np.int64)
    _check(lib.orc_visible_counts(len(kv) - 1, _ptr(kv), _ptr(qi), T, _ptr(out)), "visible_counts")
    return out


def index_scores(kv_indptr, q_indptr, q, w, k, k_scale=None, q_scale=None, ld=None,
                 k_row_stride_bytes=None, k_scale_stride=1, with_magnitude=False,
                 block_table=None, page_size=0):
    """Indexer scores, fp64 [T, ld]; entries s >= n_i are NaN.

    q: [T, H, D] float32 / uint16 (bf16 bits) / uint8 (fp8 codes).
    k: [rows, D] (or a raw uint8 byte buffer with k_row_stride_bytes).
    block_table: int32 [B, pages] of physical page ids (paged caches), with page_size.
    """
    lib = _load()
    kv = _c(kv_indptr, np.int64)
    qi = _c(q_indptr, np.int32)
    q = np.ascontiguousarray(q)
    T, H, D = q.shape
    k = np.ascontiguousarray(k)
    if k_row_stride_bytes is None:
        k_row_stride_bytes = k.shape[1] * k.itemsize
    n = visible_counts(kv, qi, T)
    if ld is None:
        ld = int(n.max()) if T else 1
    scores = np.full((T, ld), np.nan)
    mag = np.full((T, ld), np.nan) if with_magnitude else None
    w = _c(w, np.float32)
    ks = _c(k_scale, np.float32)
    qs = _c(q_scale, np.float32)
    bt = _c(block_table, np.int32)
    rc = lib.orc_index_scores(len(kv) - 1, _ptr(kv), _ptr(qi), T, H, D, _dt_code(q), _ptr(q),
                              _ptr(qs), _ptr(w), _dt_code(k), _ptr(k), int(k_row_stride_bytes),
                              _ptr(ks), int(k_scale_stride), _ptr(scores), ld, _ptr(mag), _ptr(bt),
                              0 if bt is None else bt.shape[1], int(page_size))
    _check(rc, "index_scores")
    return (scores, mag) if with_magnitude else scores


def topk(scores, n, k) -> np.ndarray:
    """Per-row top-k positions (score desc, position asc), padded with -1."""
    lib = _load()
    s = np.ascontiguousarray(scores, dtype=np.float64)
    T, ld = s.shape
    nn = _c(n, np.int64)
    out = np.zeros((T, k), dtype=np.int32)
    _check(lib.orc_topk(T, _ptr(nn), _ptr(s), ld, int(k), _ptr(out)), "topk")
    return out


def sparse_mla(kv_indptr, q_indptr, q, kv, indices, sm_scale, Dc, kv_scale=1.0, physical=False):
    """Sparse MLA output [T, H, Dc] and lse [T, H], both fp64.  physical: the indices are
    rows of kv (paged caches) instead of positions within each sequence."""
    lib = _load()
    kvp = _c(kv_indptr, np.int64)
    qi = _c(q_indptr, np.int32)
    q = np.ascontiguousarray(q)
    T, H, Dqk = q.shape
    kv = np.ascontiguousarray(kv)
    idx = _c(indices, np.int32)
    k = idx.shape[1]
    out = np.zeros((T, H, Dc))
    lse = np.zeros((T, H))
    rc = lib.orc_sparse_mla(len(kvp) - 1, _ptr(kvp), _ptr(qi), T, H, Dc, Dqk - Dc, float(sm_scale),
                            _dt_code(q), _ptr(q), _dt_code(kv), _ptr(kv), float(kv_scale), _ptr(idx),
                            k, _ptr(out), _ptr(lse), kv.shape[0] if physical else 0)
    _check(rc, "sparse_mla")
    return out, lse


def to_physical(kv_indptr, q_indptr, indices, block_table, page_size):
    """Map top-k positions (logical, per sequence) to physical cache rows through a block
    table: row = block_table[b, s // page_size] * page_size + s % page_size; -1 stays -1."""
    kv = np.asarray(kv_indptr, np.int64)
    idx = np.asarray(indices, np.int64)
    bt = np.asarray(block_table, np.int64)
    T = idx.shape[0]
    out = np.full(idx.shape, -1, np.int32)
    qi = None if q_indptr is None else np.asarray(q_indptr, np.int64)
    for i in range(T):
        b = i if qi is None else int(np.searchsorted(qi, i, side="right") - 1)
        for j, s in enumerate(idx[i]):
            if s >= 0:
                out[i, j] = bt[b, s // page_size] * page_size + s % page_size
    return out


def index_share(kv_indptr, q_indptr, idx_inputs: dict, layers: list, k: int, sm_scale: float, Dc: int):
    """One full layer's indexer + top-k, reused unchanged by every layer.

    idx_inputs: keyword arguments of ``index_scores``.  layers: list of dicts
    with q, kv, kv_scale.  Returns (indices, [(out, lse) per layer]).
    """
    s = index_scores(kv_indptr, q_indptr, **idx_inputs)
    T = s.shape[0]
    n = visible_counts(kv_indptr, q_indptr, T)
    ind = topk(s, n, k)
    outs = [sparse_mla(kv_indptr, q_indptr, L["q"], L["kv"], ind, sm_scale, Dc, L.get("kv_scale", 1.0))
            for L in layers]
    return ind, outs


def encode_fp8(values) -> np.ndarray:
    """Nearest OCP E4M3FN codes (ties to even, saturating) of float64 values, one by one."""
    lib = _load()
    flat = np.asarray(values, dtype=np.float64).ravel()
    return np.array([lib.orc_encode_fp8_e4m3fn(float(v)) for v in flat],
                    dtype=np.uint8).reshape(np.shape(values))


def pow2_scale(amax) -> np.ndarray:
    """ue8m0 group scale: smallest 2^e (e >= -126) with amax <= 448 * 2^e; 1 for amax == 0."""
    lib = _load()
    flat = np.asarray(amax, dtype=np.float64).ravel()
    return np.array([lib.orc_pow2_scale(float(a)) for a in flat]).reshape(np.shape(amax))


def rope_pair_f32(x0, x1, c, s):
    """One interleaved rope pair in fp32: (x0 c - x1 s, x0 s + x1 c)."""
    lib = _load()
    y0, y1 = ctypes.c_float(), ctypes.c_float()
    lib.orc_rope_pair_f32(float(x0), float(x1), float(c), float(s), ctypes.byref(y0), ctypes.byref(y1))
    return np.float32(y0.value), np.float32(y1.value)


def index_quant(x, positions=None, cos_sin=None, rope_off=0, dst_rows=None, out_rows=None,
                codes=None, scales=None):
    """Rope (optional) + fp8 per-head quantisation of x [rows, H, D].

    x is float32 or uint16 (bf16 bits).  cos_sin: float32 [rope_rows, D_r]
    (cos of the D_r/2 frequencies, then their sin), positions: int64 [rows].
    Group (r, h) goes to row dst_rows[r] (r when None; negative = skipped) of
    codes [out_rows, H, D] uint8 and scales [out_rows, H] float32, which start
    as the given arrays (zeros when None).  Returns (codes, scales).
    """
    lib = _load()
    x = np.ascontiguousarray(x)
    rows, H, D = x.shape
    if out_rows is None:
        out_rows = rows if codes is None else codes.shape[0]
    codes = np.zeros((out_rows, H, D), np.uint8) if codes is None else np.array(codes, np.uint8)
    scales = np.zeros((out_rows, H), np.float32) if scales is None else np.array(scales, np.float32)
    dst = _c(dst_rows, np.int64)
    if dst is not None and (dst >= out_rows).any():
        raise ValueError("dst_rows past the output")
    pos = _c(positions, np.int64)
    cs = _c(cos_sin, np.float32)
    rope_rows, D_r = (0, 0) if cs is None else cs.shape
    rc = lib.orc_index_quant(rows, H, D, _dt_code(x), _ptr(x), _ptr(pos), _ptr(cs), rope_rows, D_r,
                             int(rope_off), _ptr(dst), _ptr(codes), H * D, _ptr(scales), H)
    _check(rc, "index_quant")
    return codes, scales


def num_threads() -> int:
    return int(_load().orc_num_threads())
