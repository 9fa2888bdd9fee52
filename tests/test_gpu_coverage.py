"""Launch paths that the workload tests do not reach, each against the oracle (on the GPU).

* the top-k ROW mode: more than 512 rows longer than 32768 scores (a long-context prefill
  chunk), with tied rows, a threshold bin past the member list, and k < 2048;
* the decode indexer's per-(chunk, query row) grid: bf16 index queries with several queries
  per sequence (the MTP verify shape: q_len = draft tokens + 1), contiguous and paged;
* the fp32-output instantiations of the tuned sparse-MLA kernels (half-head bf16, full-head
  bf16, fp8) and of the split combine.
"""
import numpy as np
import pytest
import torch

import dsa_testlib as tl
import deepseek_sparse_mla_amd as dsa
import oracle
from deepseek_sparse_mla_amd import synth

pytestmark = pytest.mark.gpu

DEV = "cuda"


# ---------------------------------------------------------------------------- top-k ROW mode

def _row_mode_rows(rng):
    """520 rows of 33,000-60,000 scores: random, tied, and rows built to stress the select."""
    f = np.float32
    rows = [rng.standard_normal(int(n)).astype(f) for n in rng.integers(33000, 60001, 520)]
    rows[3] = np.round(rows[3], 1)                                           # heavy ties
    rows[11] = np.full(45000, -2.0, f)                                       # all tied
    rows[17] = np.concatenate([rng.standard_normal(1000) + 10, np.full(20000, 2.0),
                               rng.standard_normal(20000)]).astype(f)       # > 8192 keys in bin d
    rows[29] = rng.integers(-3, 4, 50000).astype(f)                          # 7 distinct values
    rows[41] = np.where(rng.random(40000) < 0.5, -0.0, 0.0).astype(f)        # signed zeros
    rows[519] = rng.standard_normal(60000).astype(f)                         # the longest row last
    for i in (17,):
        rng.shuffle(rows[i])
    return rows


def _run_topk(rows, k, ws=None):
    ctx = [len(r) for r in rows]
    ld = max(ctx)
    sc = np.zeros((len(rows), ld), np.float32)
    for i, r in enumerate(rows):
        sc[i, :len(r)] = r
    kvp = torch.tensor(np.concatenate([[0], np.cumsum(ctx)]), dtype=torch.int64, device=DEV)
    layout = dsa.Layout(kvp, None, len(rows), ld)
    if ws is None:
        n = dsa.dsa_topk_workspace_size(layout, ld, k)
        ws = torch.zeros(n, dtype=torch.uint8, device=DEV)
    idx = dsa.dsa_topk(layout, torch.from_numpy(sc).to(DEV), k, workspace=ws)
    torch.cuda.synchronize()
    return idx.cpu().numpy(), ws, layout, ld


@pytest.mark.parametrize("k", [2048, 500])
def test_topk_row_mode(k):
    """More than 512 rows and rows of 32,769 .. 262,144 scores run the ROW mode (histogram
    blocks, then one block per row reading its row once); the set equals the oracle's on the
    same array and the workspace is all zero again afterwards."""
    rng = np.random.default_rng(40 + k)
    rows = _row_mode_rows(rng)
    ih, ws, layout, ld = _run_topk(rows, k)
    assert dsa.dsa_topk_workspace_size(layout, ld, k) > 0
    for i, r in enumerate(rows):
        tl.check_topk_same_array(ih[i], r, k, "row-mode row %d (n=%d, k=%d)" % (i, len(r), k))
    assert int(torch.count_nonzero(ws)) == 0, "workspace not left zero"
    # the same workspace again, as a caller would reuse it
    ih2, _, _, _ = _run_topk(rows, k, ws)
    assert np.array_equal(ih, ih2)


# ---------------------------------------------------------------- bf16 queries, q_len > 1

MTP = {
    "mtp_verify_contiguous": dict(ctx=[3000, 5000, 2049, 9000], q_len=[2, 3, 4, 2]),
    "mtp_verify_short": dict(ctx=[40, 2100, 700], q_len=[4, 3, 2]),
}


@pytest.mark.parametrize("name", sorted(MTP))
def test_bf16_index_queries_several_per_sequence(name):
    """The MTP verify shape: q_len = 2..4 bf16 index queries per sequence, each at its own
    causal position (the decode indexer's per-(chunk, row) grid)."""
    case = synth.make_case(name, 2, sm_scale=1.0 / 16, kv_dt="fp8", iq_dt="bf16", device=DEV, **MTP[name])
    scores, idx, outs, _ = tl.gpu_path(case)
    n = tl.visible(case)
    s_host, i_host = scores.cpu().numpy(), idx.cpu().numpy()
    o_scores = tl.oracle_scores_rows(case, range(case.T))
    for r in range(case.T):
        tl.check_scores(s_host[r, :n[r]], o_scores[r], "%s row %d" % (name, r))
        tl.check_topk_same_array(i_host[r], s_host[r, :n[r]], case.topk, "%s row %d" % (name, r))
        tl.check_topk_margin(i_host[r], o_scores[r], case.topk, "%s row %d" % (name, r))
    o_or, _ = tl.oracle_mla_rows(case, range(case.T), i_host)
    g = tl.to_f64(outs[0])
    for r in range(case.T):
        tl.check_attention(g[r], o_or[r], tl.ATTN_ATOL_LOWP, "%s row %d" % (name, r))


def test_bf16_index_queries_several_per_sequence_paged():
    """The same MTP verify shape on 16-token pages equals the contiguous run bit for bit."""
    case = synth.make_case("mtp_paged", 2, ctx=[3000, 5000, 2049], q_len=[2, 4, 3], sm_scale=1.0 / 16,
                           kv_dt="fp8", iq_dt="bf16", device=DEV)
    lay_c = dsa.Layout.of_case(case)
    s_c = dsa.dsa_index_scores(lay_c, case.iq, case.iw, case.ik, k_scale=case.ik_scale)
    i_c = dsa.dsa_topk(lay_c, s_c, case.topk)
    lay, caches, bt = tl.paged(case, 16, seed=3)
    s_p = dsa.dsa_index_scores(lay, case.iq, case.iw, caches["ik"], k_scale=caches["ik_scale"])
    i_p = dsa.dsa_topk(lay, s_p, case.topk)
    L = case.layers[0]
    o_c = dsa.sparse_mla_prefill(lay_c, L.q, L.kv, i_c, case.sm_scale, case.Dc, L.kv_scale)
    o_p = dsa.sparse_mla_prefill(lay, L.q, caches["kv"][0], i_p, case.sm_scale, case.Dc, L.kv_scale)
    torch.cuda.synchronize()
    n = tl.visible(case)
    sc, sp = s_c.cpu().numpy(), s_p.cpu().numpy()
    for r in range(case.T):
        assert np.array_equal(sc[r, :n[r]], sp[r, :n[r]]), "scores row %d" % r
    mapped = oracle.to_physical(case.kv_indptr.cpu().numpy(), case.q_indptr.cpu().numpy(),
                                i_c.cpu().numpy(), bt.numpy(), 16)
    assert np.array_equal(i_p.cpu().numpy(), mapped)
    assert torch.equal(o_c, o_p)


# ------------------------------------------------------------------- fp32 outputs, tuned MLA

F32_OUT = {
    # (kv dtype, contexts): the kernel each shape reaches
    "hh_bf16_splits": ("bf16", [3000, 2100, 4096, 9000]),                      # <= 64 rows, splits
    "full_bf16_splits": ("bf16", [2100 + 13 * i for i in range(80)]),          # > 64 rows, splits
    "full_bf16_no_split": ("bf16", [2048 + (7 * i) % 900 for i in range(300)]),  # >= 256 rows: one split
    "fp8_splits": ("fp8", [3000, 2100, 4096, 9000, 2500]),
    "fp8_no_split": ("fp8", [2048 + (11 * i) % 700 for i in range(260)]),
}


@pytest.mark.parametrize("name", sorted(F32_OUT))
def test_tuned_mla_fp32_output(name):
    """fp32 outputs from bf16 or fp8 latent rows: the same kernels with fp32 stores (and fp32
    split partials), at the low-precision attention bar; the bf16 output of the same call is
    the fp32 one rounded once more, so the two agree to one bf16 rounding."""
    kv_dt, ctx = F32_OUT[name]
    case = synth.make_case(name, 2, ctx=ctx, sm_scale=1.0 / 16, kv_dt=kv_dt, out_dt="f32", device=DEV)
    scores, idx, outs, lses = tl.gpu_path(case)
    assert outs[0].dtype == torch.float32
    T = case.T
    rows = sorted({0, 1, T // 2, T - 1})
    i_host = idx.cpu().numpy()
    o_or, l_or = tl.oracle_mla_rows(case, rows, i_host)
    g = tl.to_f64(outs[0])
    for r, oo, lo in zip(rows, o_or, l_or):
        tl.check_attention(g[r], oo, tl.ATTN_ATOL_LOWP, "%s row %d" % (name, r))
        np.testing.assert_allclose(lses[0].cpu().numpy()[r], lo, atol=1e-2, rtol=1e-3)
    layout = dsa.Layout.of_case(case)
    L = case.layers[0]
    o16 = dsa.sparse_mla_decode(layout, L.q, L.kv, idx, case.sm_scale, case.Dc, L.kv_scale,
                                out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    d = (o16.float() - outs[0]).abs()
    bound = outs[0].abs() * 2.0 ** -7 + 1e-3
    assert bool((d <= bound).all()), "bf16 and fp32 outputs differ by more than a bf16 rounding: %.3g" % (
        d.max().item())


def test_fp8_extreme_logit_spread_takes_exact_rerun():
    """fp8 latent rows: a late tile whose logit exceeds the first tile's maximum by far more
    than 2^100 (in exp2 units) makes the fp8 kernel rerun its split with the exact maximum; the
    output must still meet the oracle.  256 one-query sequences give one split per row, so all
    32 tiles of the index list run in one block."""
    B, ctx, H, Dc, Dr = 256, 2048, 64, 512, 64
    g = torch.Generator(device=DEV).manual_seed(321)
    x = torch.randn((B * ctx, Dc + Dr), generator=g, device=DEV)
    codes = x.to(torch.float8_e4m3fn).view(torch.uint8)
    q = torch.randn((B, H, Dc + Dr), generator=g, device=DEV)
    for b in (0, 1):
        codes[b * ctx:(b + 1) * ctx, 0] = 0
        codes[b * ctx + 1500, 0] = 0x7E  # 448
        q[b, :, 0] = 64.0
    q = q.to(torch.bfloat16)
    kvp = torch.arange(0, (B + 1) * ctx, ctx, dtype=torch.int64, device=DEV)
    layout = dsa.Layout(kvp, None, B, ctx)
    idx = torch.arange(ctx, dtype=torch.int32, device=DEV).repeat(B, 1).contiguous()
    lse = torch.empty((B, H), dtype=torch.float32, device=DEV)
    out = dsa.sparse_mla_decode(layout, q, codes, idx, 1.0 / 16, Dc, 1.0, lse=lse)
    torch.cuda.synchronize()
    for b in (0, 1, 2):
        o, l = oracle.sparse_mla([0, ctx], None, synth.host(q[b:b + 1]), synth.host(codes[b * ctx:(b + 1) * ctx]),
                                 idx[b:b + 1].cpu().numpy(), 1.0 / 16, Dc, 1.0)
        tl.check_attention(tl.to_f64(out[b]), o[0], tl.ATTN_ATOL_LOWP, "row %d" % b)
        np.testing.assert_allclose(lse[b].cpu().numpy(), l[0], rtol=1e-4, atol=1e-3)
