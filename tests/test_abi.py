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
    assert lib.dsa_abi_version() == 2


def _layout(batch=2, total_q=2, max_ctx=4096, kv=FAKE, qi=None, bt=None, bt_stride=0, page=0, rows=0):
    return B.dsa_layout(batch, total_q, max_ctx, kv, qi, bt, bt_stride, page, rows)


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


def _kw(lib, **kw):
    a = dict(n=4, k_dt=B.DSA_BF16, k=FAKE, kstride=256, pos=None, cs=None, rope_rows=0, rope_off=0,
             slots=FAKE, cache=FAKE, cstride=132, cscale=FAKE + 128, csstride=33, crows=100)
    a.update(kw)
    return lib.dsa_index_k_cache_write(a["n"], a["k_dt"], a["k"], a["kstride"], a["pos"], a["cs"],
                                       a["rope_rows"], a["rope_off"], a["slots"], a["cache"],
                                       a["cstride"], a["cscale"], a["csstride"], a["crows"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(n=-1), B.DSA_ERR_INVALID_ARG),
    (dict(k_dt=B.DSA_FP8_E4M3FN), B.DSA_ERR_UNSUPPORTED),      # input is already fp8
    (dict(k=None), B.DSA_ERR_INVALID_ARG),
    (dict(k=FAKE + 8), B.DSA_ERR_INVALID_ARG),                 # 16-byte alignment
    (dict(kstride=200), B.DSA_ERR_INVALID_ARG),                # shorter than a row
    (dict(kstride=264), B.DSA_ERR_INVALID_ARG),                # not a multiple of 16
    (dict(slots=None), B.DSA_ERR_INVALID_ARG),
    (dict(cstride=130), B.DSA_ERR_INVALID_ARG),                # not a multiple of 4
    (dict(cache=FAKE + 2), B.DSA_ERR_INVALID_ARG),
    (dict(csstride=0), B.DSA_ERR_INVALID_ARG),
    (dict(cs=FAKE, rope_rows=10), B.DSA_ERR_INVALID_ARG),      # rope without positions
    (dict(cs=FAKE, pos=FAKE, rope_rows=0), B.DSA_ERR_INVALID_ARG),
    (dict(cs=FAKE, pos=FAKE, rope_rows=10, rope_off=32), B.DSA_ERR_INVALID_ARG),
    (dict(crows=-1), B.DSA_ERR_INVALID_ARG),
])
def test_index_k_cache_write_rejects(lib, kw, status):
    assert _kw(lib, **kw) == status
    assert lib.dsa_last_error()


def test_index_k_cache_write_accepts_empty_batch(lib):
    """n = 0 passes every check and launches nothing (no device needed)."""
    assert _kw(lib, n=0) == B.DSA_OK


def test_index_q_quant_rejects(lib):
    q = lambda **kw: lib.dsa_index_q_quant(kw.get("T", 8), kw.get("H", 32), kw.get("dt", B.DSA_BF16),
                                           kw.get("q", FAKE), kw.get("stride", 8192), None, None, 0, 0,
                                           kw.get("out", FAKE), kw.get("scale", FAKE), None)
    assert q(H=0) == B.DSA_ERR_INVALID_ARG
    assert q(stride=4096) == B.DSA_ERR_INVALID_ARG             # shorter than 32 heads of bf16
    assert q(dt=B.DSA_FP8_E4M3FN) == B.DSA_ERR_UNSUPPORTED
    assert q(scale=FAKE + 1) == B.DSA_ERR_INVALID_ARG
    assert q(T=0) == B.DSA_OK


def test_writer_empty_calls_accept_null_pointers(lib):
    """An empty batch is a no-op; empty device tensors carry NULL data pointers."""
    assert _kw(lib, n=0, k=None, slots=None, cache=None, cscale=None) == B.DSA_OK
    assert lib.dsa_index_q_quant(0, 32, B.DSA_BF16, None, 8192, None, None, 0, 0, None, None, None) == B.DSA_OK


def test_index_front_end_rejects(lib):
    def fe(**kw):
        a = dict(T=8, H=32, dt=B.DSA_BF16, q=FAKE, qs=8192, k=FAKE, ks=256, pos=None, cs=None, rr=0, ro=0,
                 slots=FAKE, cache=FAKE, cstride=128, cscale=FAKE, csstride=1, crows=100, q8=FAKE, qsc=FAKE)
        a.update(kw)
        return lib.dsa_index_front_end(a["T"], a["H"], a["dt"], a["q"], a["qs"], a["k"], a["ks"], a["pos"],
                                       a["cs"], a["rr"], a["ro"], a["slots"], a["cache"], a["cstride"],
                                       a["cscale"], a["csstride"], a["crows"], a["q8"], a["qsc"], None)
    assert fe(ks=100) == B.DSA_ERR_INVALID_ARG                   # key row shorter than 128 values
    assert fe(qs=4096) == B.DSA_ERR_INVALID_ARG                  # query row shorter than 32 heads
    assert fe(slots=None) == B.DSA_ERR_INVALID_ARG
    assert fe(dt=B.DSA_FP8_E4M3FN) == B.DSA_ERR_UNSUPPORTED
    assert fe(cs=FAKE, rr=4) == B.DSA_ERR_INVALID_ARG             # rope without positions
    assert fe(crows=-1) == B.DSA_ERR_INVALID_ARG
    assert fe(T=0, q=None, k=None, slots=None, cache=None, cscale=None, q8=None, qsc=None) == B.DSA_OK


def test_paged_layout_rejects(lib):
    """A block table needs a page size, enough pages per row for max_ctx and a cache size."""
    ok = dict(bt=FAKE, bt_stride=64, page=64, rows=1 << 20)  # never passed whole: it would launch
    for bad in (dict(page=0), dict(bt_stride=63), dict(rows=0), dict(bt=FAKE + 2)):
        kw = dict(ok)
        kw.update(bad)
        assert _idx(lib, _layout(**kw)) == B.DSA_ERR_INVALID_ARG, bad
        assert lib.dsa_last_error()
    L = ctypes.byref(_layout(**ok))
    assert lib.dsa_topk(L, FAKE, 4096, 0, FAKE, None, 0, None) == B.DSA_ERR_INVALID_ARG  # k still checked


# ------------------------------------------------------------------ allocation-free entry point

NO_ALLOC_MAX = 64 << 20  # DSA_NO_ALLOC_SCRATCH_BYTES


def test_no_alloc_scratch_holds_every_single_layer_call(lib):
    """The static scratch covers the split partials of every single-layer call with k <= 2048
    (only calls with fewer than 256 rows split their keys)."""
    worst = 0
    for T in list(range(1, 300)) + [511, 512, 4096]:
        for k in (1, 63, 64, 65, 128, 500, 1024, 2047, 2048):
            lay = _layout(batch=T, total_q=T)
            worst = max(worst, lib.sparse_mla_workspace_size(ctypes.byref(lay), 64, 512, 64, k, 1))
    assert 0 < worst <= NO_ALLOC_MAX, worst


def _mla_na(lib, layout, k=2048):
    return lib.sparse_mla_decode_no_alloc(ctypes.byref(layout), 64, 512, 64, 0.0625, B.DSA_BF16, FAKE,
                                          B.DSA_FP8_E4M3FN, FAKE, 1.0, FAKE, k, B.DSA_BF16, FAKE, None, None)


def test_no_alloc_rejects_partials_beyond_the_scratch(lib, monkeypatch):
    """A split count forced past the policy (tuning override) needs more partials than the
    static scratch holds: the call is refused on the host, before any HIP call."""
    monkeypatch.setenv("DSA_MLA_SPLITS", "32")
    st = _mla_na(lib, _layout(batch=255, total_q=255))
    assert st == B.DSA_ERR_WORKSPACE
    assert b"static scratch" in lib.dsa_last_error()


def test_no_alloc_checks_arguments_like_the_workspace_entry(lib):
    assert _mla_na(lib, _layout(), k=0) == B.DSA_ERR_INVALID_ARG
    assert lib.sparse_mla_decode_no_alloc(None, 64, 512, 64, 0.0625, B.DSA_BF16, FAKE, B.DSA_FP8_E4M3FN, FAKE,
                                          1.0, FAKE, 2048, B.DSA_BF16, FAKE, None, None) == B.DSA_ERR_INVALID_ARG


def _it(lib, layout, **kw):
    a = dict(H=32, D=128, q_dt=B.DSA_BF16, q=FAKE, qs=None, w=FAKE, k_dt=B.DSA_FP8_E4M3FN, k=FAKE,
             kstride=128, ks=FAKE, ks_stride=1, scores=FAKE, ld=4096, k_top=2048, idx=FAKE, ws=None, wsb=0)
    a.update(kw)
    return lib.dsa_index_topk(ctypes.byref(layout), a["H"], a["D"], a["q_dt"], a["q"], a["qs"], a["w"], a["k_dt"],
                              a["k"], a["kstride"], a["ks"], a["ks_stride"], a["scores"], a["ld"], a["k_top"],
                              a["idx"], a["ws"], a["wsb"], None)


def _ish(lib, layout, built, **kw):
    a = dict(H=32, D=128, q_dt=B.DSA_BF16, q=FAKE, qs=None, w=FAKE, k_dt=B.DSA_FP8_E4M3FN, k=FAKE,
             kstride=128, ks=FAKE, ks_stride=1, scores=FAKE, ld=4096, k_top=2048, ws=None, wsb=0)
    a.update(kw)
    return lib.dsa_index_scores_hist(ctypes.byref(layout), a["H"], a["D"], a["q_dt"], a["q"], a["qs"], a["w"],
                                     a["k_dt"], a["k"], a["kstride"], a["ks"], a["ks_stride"], a["scores"], a["ld"],
                                     a["k_top"], a["ws"], a["wsb"], built, None)


def test_two_call_form_checks_before_launching(lib):
    """dsa_index_scores_hist refuses what dsa_index_topk refuses (bar indices) and a NULL
    hist_built, and reports hist_built = 0 on failure; dsa_topk_after_hist refuses what dsa_topk
    refuses."""
    built = ctypes.c_int(7)
    assert _ish(lib, _layout(), None) == B.DSA_ERR_INVALID_ARG               # no hist_built
    assert _ish(lib, _layout(), ctypes.byref(built), k_top=0) == B.DSA_ERR_INVALID_ARG
    assert built.value == 0
    assert _ish(lib, _layout(), ctypes.byref(built), H=0) == B.DSA_ERR_INVALID_ARG
    assert _ish(lib, _layout(), ctypes.byref(built), ld=100) == B.DSA_ERR_INVALID_ARG
    long_rows = _layout(batch=4, total_q=4, max_ctx=70000)
    assert _ish(lib, long_rows, ctypes.byref(built), ld=70000) == B.DSA_ERR_WORKSPACE
    L = ctypes.byref(_layout())
    assert lib.dsa_topk_after_hist(L, FAKE, 4096, 0, FAKE, None, 0, 1, None) == B.DSA_ERR_INVALID_ARG
    assert lib.dsa_topk_after_hist(L, FAKE, 4096, 16, None, None, 0, 1, None) == B.DSA_ERR_INVALID_ARG
    assert lib.dsa_topk_after_hist(L, FAKE, 10, 16, FAKE, None, 0, 0, None) == B.DSA_ERR_INVALID_ARG
    assert lib.dsa_topk_after_hist(ctypes.byref(long_rows), FAKE, 70000, 16, FAKE, None, 0, 1,
                                   None) == B.DSA_ERR_WORKSPACE


def test_gather_ceiling_rejects(lib):
    """The gather measurement entry checks its arguments on the host (nothing is launched)."""
    g = lib.dsa_gather_ceiling
    assert g(None, 100, 576, FAKE, 1, 16, FAKE, None) == B.DSA_ERR_INVALID_ARG        # no rows
    assert g(FAKE, 100, 576, None, 1, 16, FAKE, None) == B.DSA_ERR_INVALID_ARG        # no indices
    assert g(FAKE, 100, 576, FAKE, 1, 16, None, None) == B.DSA_ERR_INVALID_ARG        # no sink
    assert g(FAKE, 100, 600, FAKE, 1, 16, FAKE, None) == B.DSA_ERR_INVALID_ARG        # row size
    assert g(FAKE, 100, 1152, FAKE, 0, 16, FAKE, None) == B.DSA_ERR_INVALID_ARG       # no rows of indices
    assert g(FAKE, 100, 1152, FAKE, 1, 0, FAKE, None) == B.DSA_ERR_INVALID_ARG        # k out of range
    assert g(FAKE, 100, 1152, FAKE, 1, 2049, FAKE, None) == B.DSA_ERR_INVALID_ARG
    assert g(FAKE, 0, 1152, FAKE, 1, 16, FAKE, None) == B.DSA_ERR_INVALID_ARG         # empty table
    assert g(FAKE, 1 << 23, 576, FAKE, 1, 16, FAKE, None) == B.DSA_ERR_INVALID_ARG    # table past 4 GiB


def test_read_ceiling_rejects(lib):
    """The read measurement entry checks its arguments on the host (nothing is launched)."""
    r = lib.dsa_read_ceiling
    assert r(None, 128, FAKE, 1, 100, 0, 512, FAKE, None) == B.DSA_ERR_INVALID_ARG     # no keys
    assert r(FAKE, 128, None, 1, 100, 0, 512, FAKE, None) == B.DSA_ERR_INVALID_ARG     # no scales
    assert r(FAKE, 128, FAKE, 1, 100, 0, 512, None, None) == B.DSA_ERR_INVALID_ARG     # no sink
    assert r(FAKE, 128, FAKE, 1, 0, 0, 512, FAKE, None) == B.DSA_ERR_INVALID_ARG       # no tokens
    assert r(FAKE, 128, FAKE, 1, 100, 0, 0, FAKE, None) == B.DSA_ERR_INVALID_ARG       # no blocks
    assert r(FAKE, 128, FAKE, 1, 100, 3, 512, FAKE, None) == B.DSA_ERR_INVALID_ARG     # unknown pattern
    assert r(FAKE, 128, FAKE, 1, 100, -1, 512, FAKE, None) == B.DSA_ERR_INVALID_ARG
    assert r(FAKE, 126, FAKE, 1, 100, 0, 512, FAKE, None) == B.DSA_ERR_INVALID_ARG     # short / unaligned rows
    assert r(FAKE, 130, FAKE, 1, 100, 0, 512, FAKE, None) == B.DSA_ERR_INVALID_ARG
    assert r(FAKE, 128, FAKE, 0, 100, 0, 512, FAKE, None) == B.DSA_ERR_INVALID_ARG     # scale stride
    assert r(FAKE, 132, FAKE, 33, 100, 1, 512, FAKE, None) == B.DSA_ERR_INVALID_ARG    # patterns 1, 2: 128-byte rows
    assert r(FAKE, 132, FAKE, 33, 100, 2, 512, FAKE, None) == B.DSA_ERR_INVALID_ARG


def test_index_topk_checks_both_calls_before_launching(lib):
    """The fused entry refuses, on the host, whatever either separate call would refuse."""
    assert _it(lib, _layout(), k_top=0) == B.DSA_ERR_INVALID_ARG            # top-k: k out of range
    assert _it(lib, _layout(), idx=None) == B.DSA_ERR_INVALID_ARG           # top-k: no indices
    assert _it(lib, _layout(), H=0) == B.DSA_ERR_INVALID_ARG                # indexer: bad shape
    assert _it(lib, _layout(), ks=None) == B.DSA_ERR_INVALID_ARG            # indexer: fp8 keys need a scale
    assert _it(lib, _layout(), ld=100) == B.DSA_ERR_INVALID_ARG             # ld < max_ctx
    long_rows = _layout(batch=4, total_q=4, max_ctx=70000)
    assert _it(lib, long_rows, ld=70000) == B.DSA_ERR_WORKSPACE             # long rows need the workspace
    need = lib.dsa_topk_workspace_size(ctypes.byref(long_rows), 70000, 2048)
    assert _it(lib, long_rows, ld=70000, ws=FAKE, wsb=need - 1) == B.DSA_ERR_WORKSPACE
    assert _it(lib, _layout(batch=0, total_q=0)) == B.DSA_ERR_INVALID_ARG   # a layout needs a sequence
