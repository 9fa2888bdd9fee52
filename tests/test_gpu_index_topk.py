"""The fused indexer + top-k entry (dsa_index_topk) and its two-call form
(dsa_index_scores_hist, then dsa_topk_after_hist) on the GPU, through the C ABI.

Where the decode indexer builds the top-k's histogram itself, both must give the same scores
and indices, bit for bit, as dsa_index_scores followed by dsa_topk, and leave the top-k
workspace all zero.  Shapes: rows past 32768 scores in the decode stream grid (one query
per sequence), in the per-(chunk, row) grid (several bf16 queries per sequence), on paged
caches, more than 512 long rows (the selection's ROW mode), and the shapes that fall back to
the two separate launches (rows of at most 32768 scores; fp8 index queries).  The fused
result is also checked against the oracle on sampled rows.
"""
import numpy as np
import pytest
import torch

import dsa_testlib as tl
import deepseek_sparse_mla_amd as dsa
from deepseek_sparse_mla_amd import synth

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _compare(case, layout=None, ik=None, ik_scale=None, check_rows=()):
    lay = layout or dsa.Layout.of_case(case)
    ik = case.ik if ik is None else ik
    ik_scale = case.ik_scale if ik_scale is None else ik_scale
    ld = case.max_ctx
    s_sep = torch.full((case.T, ld), 3.0, dtype=torch.float32, device=DEV)
    dsa.dsa_index_scores(lay, case.iq, case.iw, ik, k_scale=ik_scale, q_scale=case.iq_scale, scores=s_sep)
    i_sep = dsa.dsa_topk(lay, s_sep, case.topk)
    ws = dsa.topk_workspace(lay, ld, case.topk, DEV)
    s_fus = torch.full((case.T, ld), 3.0, dtype=torch.float32, device=DEV)
    s_fus, i_fus = dsa.dsa_index_topk(lay, case.iq, case.iw, ik, case.topk, k_scale=ik_scale, q_scale=case.iq_scale,
                                      scores=s_fus, workspace=ws)
    torch.cuda.synchronize()
    n = tl.visible(case)
    a, b = s_sep.cpu().numpy(), s_fus.cpu().numpy()
    for r in range(case.T):
        assert np.array_equal(a[r, :n[r]], b[r, :n[r]]), "scores row %d" % r
    assert torch.equal(i_sep, i_fus), "indices differ from the two separate calls"
    if ws is not None:
        assert int(torch.count_nonzero(ws)) == 0, "workspace not left zero"
    # the two-call form of the fused entry
    s_two = torch.full((case.T, ld), 5.0, dtype=torch.float32, device=DEV)
    s_two, built = dsa.dsa_index_scores_hist(lay, case.iq, case.iw, ik, case.topk, ws, k_scale=ik_scale,
                                             q_scale=case.iq_scale, scores=s_two)
    i_two = dsa.dsa_topk_after_hist(lay, s_two, case.topk, built, workspace=ws)
    torch.cuda.synchronize()
    c = s_two.cpu().numpy()
    for r in range(case.T):
        assert np.array_equal(a[r, :n[r]], c[r, :n[r]]), "two-call scores row %d" % r
    assert torch.equal(i_sep, i_two), "two-call indices differ from the two separate calls"
    expect_built = (ws is not None and case.iq_dt == "bf16")
    assert built == int(expect_built), (built, expect_built)
    if ws is not None:
        assert int(torch.count_nonzero(ws)) == 0, "workspace not left zero by the two-call form"
    if check_rows and layout is None:
        o = tl.oracle_scores_rows(case, check_rows)
        ih = i_fus.cpu().numpy()
        for r, osr in zip(check_rows, o):
            tl.check_topk_same_array(ih[r], b[r, :n[r]], case.topk, "fused row %d" % r)
            tl.check_topk_margin(ih[r], osr, case.topk, "fused row %d" % r)
    return i_fus


CASES = {
    "stream_long_rows": dict(ctx=[40000, 70000, 33000, 131072, 50000], iq_dt="bf16"),
    "stream_mixed_rows": dict(ctx=[1000, 40000, 30000, 5000, 65536], iq_dt="bf16"),
    "chunk_grid_bf16_q_len": dict(ctx=[40000, 70000, 36000], q_len=[2, 3, 4], iq_dt="bf16"),
    "direct_rows_fallback": dict(ctx=[9000, 32768, 20000], iq_dt="bf16"),
    "fp8_queries_fallback": dict(ctx=[40000, 34000], q_len=[3, 2], iq_dt="fp8"),
}


@pytest.mark.parametrize("name", sorted(CASES))
def test_fused_equals_separate_calls(name):
    case = synth.make_case(name, 2, sm_scale=1.0 / 16, kv_dt="fp8", device=DEV, **CASES[name])
    _compare(case, check_rows=[0, case.T - 1])


def test_fused_on_paged_caches():
    case = synth.make_case("fused_paged", 2, ctx=[40000, 70000, 3000], sm_scale=1.0 / 16, kv_dt="fp8", device=DEV)
    lay, caches, bt = tl.paged(case, 16, seed=9)
    _compare(case, layout=lay, ik=caches["ik"], ik_scale=caches["ik_scale"])


def test_fused_many_long_rows_row_mode():
    """More than 512 sequences past 32768 tokens: the selection's ROW mode with the indexer's
    histogram."""
    rng = np.random.default_rng(4)
    ctx = [int(c) for c in rng.integers(32769, 40000, 520)]
    case = synth.make_case("fused_row_mode", 2, ctx=ctx, sm_scale=1.0 / 16, kv_dt="fp8", device=DEV)
    _compare(case, check_rows=[0, 519])


def test_fused_indexshare_workload():
    """The IndexShare workload's shape (32 sequences of 131072 tokens)."""
    case = synth.config(5, DEV)
    _compare(case, check_rows=[0, 31])
    del case
    torch.cuda.empty_cache()


def test_long_rows_with_an_unaligned_pitch():
    """Rows of an odd pitch (40001 scores: rows not 16-byte aligned) through the long-row
    selection, plain and with the indexer's histogram: the mark kernel's 4-byte load path."""
    case = synth.make_case("odd_pitch", 2, ctx=[40001, 35003, 33001], sm_scale=1.0 / 16, kv_dt="fp8",
                           iq_dt="bf16", device=DEV)
    lay = dsa.Layout.of_case(case)
    ld = case.max_ctx
    assert ld % 4 != 0
    sc = torch.empty((case.T, ld), dtype=torch.float32, device=DEV)
    dsa.dsa_index_scores(lay, case.iq, case.iw, case.ik, k_scale=case.ik_scale, scores=sc)
    ws = dsa.topk_workspace(lay, ld, case.topk, DEV)
    assert ws is not None
    i_plain = dsa.dsa_topk(lay, sc, case.topk, workspace=ws)
    s2, built = dsa.dsa_index_scores_hist(lay, case.iq, case.iw, case.ik, case.topk, ws, k_scale=case.ik_scale,
                                          scores=torch.empty_like(sc))
    assert built == 1
    i_two = dsa.dsa_topk_after_hist(lay, s2, case.topk, built, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(i_plain, i_two)
    assert int(torch.count_nonzero(ws)) == 0
    n = tl.visible(case)
    s_host, i_host = sc.cpu().numpy(), i_plain.cpu().numpy()
    for r in range(case.T):
        tl.check_topk_same_array(i_host[r], s_host[r, :n[r]], case.topk, "odd pitch row %d" % r)
