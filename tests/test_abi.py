"""CPU checks of the C ABI: the library loads, exports every declared entry point, and
rejects bad arguments on the host with the documented status before any HIP call."""
import ctypes
import os
import re

import pytest

import deepseek_sparse_mla_amd as dsa
from deepseek_sparse_mla_amd import _binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dsa.h")

FAKE = 0x10000  # a 64 KiB-aligned address that validation never dereferences


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][\w ]*?[\s\*]+([a-z_][a-z0-9_]*)\s*\(", text, flags=re.M)
    return sorted(set(n for n in names if n not in ("if", "while", "defined")))


@pytest.fixture(scope="module")
def lib():
    return dsa.load_library()


def test_every_declared_symbol_is_exported(lib):
    names = declared_functions()
    assert set(names) == set(B.EXPORTS), names
    for n in names:
        assert hasattr(lib, n), n


def test_abi_version(lib):
    assert lib.dsa_abi_version() == 1


def _layout(batch=2, total_q=2, max_ctx=4096, kv=FAKE, qi=None):
    return B.dsa_layout(batch, total_q, max_ctx, kv, qi)


def _idx(lib, layout, **kw):
    a = dict(H=32, D=128, q_dt=B.DSA_BF16, q=FAKE, qs=None, w=FAKE, k_dt=B.DSA_FP8_E4M3FN, k=FAKE,
             kstride=128, ks=FAKE, ks_stride=1, scores=FAKE, ld=4096)
    a.update(kw)
    L = ctypes.byref(layout) if layout is not None else None
    return lib.dsa_index_scores(L, a["H"], a["D"], a["q_dt"], a["q"], a["qs"], a["w"], a["k_dt"], a["k"],
                                a["kstride"], a["ks"], a["ks_stride"], a["scores"], a["ld"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(H=0), B.DSA_ERR_INVALID_ARG),
    (dict(q_dt=7), B.DSA_ERR_UNSUPPORTED),
    (dict(q=None), B.DSA_ERR_INVALID_ARG),
    (dict(q_dt=B.DSA_FP8_E4M3FN), B.DSA_ERR_INVALID_ARG),      # fp8 q needs q_scale
    (dict(qs=FAKE), B.DSA_ERR_INVALID_ARG),                    # bf16 q takes no q_scale
    (dict(ks=None), B.DSA_ERR_INVALID_ARG),                    # fp8 keys need a scale
    (dict(kstride=100), B.DSA_ERR_INVALID_ARG),                # shorter than a row
    (dict(ld=100), B.DSA_ERR_INVALID_ARG),                     # ld < max_ctx
    (dict(w=FAKE + 2), B.DSA_ERR_INVALID_ARG),                 # misaligned
    (dict(H=128, D=128), B.DSA_ERR_UNSUPPORTED),               # beyond the generic kernel
])
def test_index_scores_rejects(lib, kw, status):
    assert _idx(lib, _layout(), **kw) == status
    assert lib.dsa_last_error()


def test_layout_rejects(lib):
    assert _idx(lib, None) == B.DSA_ERR_INVALID_ARG
    assert _idx(lib, _layout(batch=0)) == B.DSA_ERR_INVALID_ARG
    assert _idx(lib, _layout(kv=None)) == B.DSA_ERR_INVALID_ARG
    assert _idx(lib, _layout(max_ctx=0)) == B.DSA_ERR_INVALID_ARG
    assert _idx(lib, _layout(batch=2, total_q=3)) == B.DSA_ERR_INVALID_ARG  # decode needs T == B
    assert b"total_q" in lib.dsa_last_error()


def test_topk_rejects(lib):
    L = ctypes.byref(_layout())
    assert lib.dsa_topk(L, FAKE, 4096, 0, FAKE, None, 0, None) == B.DSA_ERR_INVALID_ARG
    assert lib.dsa_topk(L, FAKE, 4096, 2049, FAKE, None, 0, None) == B.DSA_ERR_INVALID_ARG
    assert lib.dsa_topk(L, None, 4096, 16, FAKE, None, 0, None) == B.DSA_ERR_INVALID_ARG
    assert lib.dsa_topk(L, FAKE, 10, 16, FAKE, None, 0, None) == B.DSA_ERR_INVALID_ARG
    assert lib.dsa_topk_workspace_size(L, 4096, 2048) == 0


def test_topk_workspace_only_for_rows_past_32768(lib):
    """Rows up to 32768 scores are selected by one block each (no workspace); longer rows
    need the histogram (and, for few rows, bitmap and member) workspace."""
    for max_ctx in (8192, 16384, 32768):
        assert lib.dsa_topk_workspace_size(ctypes.byref(_layout(max_ctx=max_ctx)), max_ctx, 2048) == 0
    for max_ctx in (32769, 131072, 300000):
        assert lib.dsa_topk_workspace_size(ctypes.byref(_layout(max_ctx=max_ctx)), max_ctx, 2048) > 0


def _mla(lib, layout, ws=None, ws_bytes=0, **kw):
    a = dict(H=64, Dc=512, Dr=64, sm=0.0625, q_dt=B.DSA_BF16, q=FAKE, kv_dt=B.DSA_BF16, kv=FAKE,
             kv_scale=1.0, idx=FAKE, k=2048, out_dt=B.DSA_BF16, out=FAKE, lse=None)
    a.update(kw)
    return lib.sparse_mla_decode(ctypes.byref(layout), a["H"], a["Dc"], a["Dr"], a["sm"], a["q_dt"], a["q"],
                                 a["kv_dt"], a["kv"], a["kv_scale"], a["idx"], a["k"], a["out_dt"], a["out"],
                                 a["lse"], ws, ws_bytes, None)


@pytest.mark.parametrize("kw,status", [
    (dict(k=0), B.DSA_ERR_INVALID_ARG),
    (dict(k=4096), B.DSA_ERR_INVALID_ARG),
    (dict(q_dt=B.DSA_FP8_E4M3FN), B.DSA_ERR_UNSUPPORTED),
    (dict(out_dt=B.DSA_FP8_E4M3FN), B.DSA_ERR_UNSUPPORTED),
    (dict(kv_scale=0.0), B.DSA_ERR_INVALID_ARG),
    (dict(sm=float("nan")), B.DSA_ERR_INVALID_ARG),
    (dict(idx=None), B.DSA_ERR_INVALID_ARG),
    (dict(q=FAKE + 8), B.DSA_ERR_INVALID_ARG),                 # tuned path needs 16-byte alignment
    (dict(H=256), B.DSA_ERR_UNSUPPORTED),
])
def test_mla_rejects(lib, kw, status):
    assert _mla(lib, _layout(), FAKE, 1 << 40, **kw) == status


def test_mla_workspace_required(lib):
    L = _layout(batch=8, total_q=8)
    need = lib.sparse_mla_workspace_size(ctypes.byref(L), 64, 512, 64, 2048, 1)
    assert need > 0
    assert _mla(lib, L, None, 0) == B.DSA_ERR_WORKSPACE
    assert _mla(lib, L, FAKE, need - 1) == B.DSA_ERR_WORKSPACE
    # the split count falls as the number of (row, layer) pairs grows; the space never shrinks
    four = lib.sparse_mla_workspace_size(ctypes.byref(L), 64, 512, 64, 2048, 4)
    assert four >= need
    # enough (row, layer) pairs to fill the chip: one split, no workspace
    big = _layout(batch=256, total_q=256)
    assert lib.sparse_mla_workspace_size(ctypes.byref(big), 64, 512, 64, 2048, 1) == 0


def test_shared_rejects_too_many_layers(lib):
    L = _layout()
    arr = (B.dsa_mla_layer * 9)()
    for l in range(9):
        arr[l] = B.dsa_mla_layer(FAKE, FAKE, 1.0, FAKE, None)
    st = lib.sparse_mla_decode_shared(ctypes.byref(L), 64, 512, 64, 0.0625, B.DSA_BF16, B.DSA_FP8_E4M3FN,
                                      B.DSA_BF16, 9, arr, FAKE, 2048, FAKE, 1 << 40, None)
    assert st == B.DSA_ERR_INVALID_ARG
    arr[1] = B.dsa_mla_layer(FAKE, None, 1.0, FAKE, None)
    st = lib.sparse_mla_decode_shared(ctypes.byref(L), 64, 512, 64, 0.0625, B.DSA_BF16, B.DSA_FP8_E4M3FN,
                                      B.DSA_BF16, 2, arr, FAKE, 2048, FAKE, 1 << 40, None)
    assert st == B.DSA_ERR_INVALID_ARG and b"layer 1" in lib.dsa_last_error()


def test_binding_needs_device_tensors():
    import torch
    L = B.Layout.__new__(B.Layout)
    with pytest.raises(ValueError):
        B._dev(torch.zeros(4), "x")
    del L
