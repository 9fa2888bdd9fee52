"""Parity of the HIP path (through the C ABI) against the fp64 oracle, on the GPU.

Small cases cover several tiles, ragged tails, multi-sequence blocks and the degenerate
cases (n < k, n = 1, all-masked tiles, ties); the full-size workloads are checked on
sampled rows.  Tolerances: see dsa_testlib.
"""
import os

import numpy as np
import pytest
import torch

import dsa_testlib as tl
import oracle
import deepseek_sparse_mla_amd as dsa
from deepseek_sparse_mla_amd import synth

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _all_rows_check(case, scores, idx, outs, atol, rows=None):
    n = tl.visible(case)
    rows = range(case.T) if rows is None else rows
    s_host = scores.cpu().numpy()
    i_host = idx.cpu().numpy()
    o_scores = tl.oracle_scores_rows(case, rows)
    for r, osr in zip(rows, o_scores):
        ni = int(n[r])
        tl.check_scores(s_host[r, :ni], osr, "%s row %d" % (case.name, r))
        tl.check_topk_same_array(i_host[r], s_host[r, :ni], case.topk, "%s row %d" % (case.name, r))
        tl.check_topk_margin(i_host[r], osr, case.topk, "%s row %d" % (case.name, r))
    worst = 0.0
    for l, out in enumerate(outs):
        o_or, _ = tl.oracle_mla_rows(case, rows, i_host, layer=l)
        g = tl.to_f64(out)
        for r, oo in zip(rows, o_or):
            worst = max(worst, tl.check_attention(g[r], oo, atol, "%s layer %d row %d" % (case.name, l, r)))
    return worst


def test_tiny_config_full_path():
    case = synth.config(1, DEV)
    scores, idx, outs, lses = tl.gpu_path(case)
    _all_rows_check(case, scores, idx, outs, tl.ATTN_ATOL_F32)
    # lse too
    _, l_or = tl.oracle_mla_rows(case, [0], idx.cpu().numpy())
    np.testing.assert_allclose(lses[0].cpu().numpy()[0], l_or[0], atol=1e-4)


DECODE_CASES = {
    "bf16kv_ragged": dict(ctx=[1000, 2500, 4100, 9000], kv_dt="bf16"),
    "fp8kv_ragged": dict(ctx=[4096, 5000, 2049, 2047, 700], kv_dt="fp8"),
    "short_and_edge": dict(ctx=[1, 2, 64, 2048, 130], kv_dt="bf16"),
}


@pytest.mark.parametrize("name", sorted(DECODE_CASES))
def test_decode_path(name):
    case = synth.make_case(name, 2, sm_scale=1.0 / 16, device=DEV, **DECODE_CASES[name])
    scores, idx, outs, lses = tl.gpu_path(case)
    _all_rows_check(case, scores, idx, outs, tl.ATTN_ATOL_LOWP)
    # lse of every row against the oracle on the same indices
    _, l_or = tl.oracle_mla_rows(case, range(case.T), idx.cpu().numpy())
    np.testing.assert_allclose(lses[0].cpu().numpy(), np.array(l_or), atol=1e-2, rtol=1e-3)


@pytest.mark.parametrize("n_rows", [100, 520])
def test_bf16_decode_many_rows_full_head_blocks(n_rows):
    """More than 64 bf16 rows take the full-head kernel (fewer rows take the half-head one),
    with key splits and the combine at 100 rows, without at 520: sampled rows, including a
    short one and the last."""
    rng = np.random.default_rng(31)
    ctx = [int(c) for c in rng.integers(300, 2600, n_rows)]
    ctx[7] = 40
    case = synth.make_case("many_rows_bf16", 2, ctx=ctx, sm_scale=1.0 / 16, kv_dt="bf16", device=DEV)
    scores, idx, outs, _ = tl.gpu_path(case)
    _all_rows_check(case, scores, idx, outs, tl.ATTN_ATOL_LOWP, rows=[0, 7, n_rows // 2, n_rows - 1])


def test_prefill_single_sequence_sampled_rows():
    case = synth.make_case("prefill_small", 4, ctx=[2600], q_len=[70], iq_dt="fp8", sm_scale=1.0 / 16,
                           kv_dt="bf16", device=DEV)
    scores, idx, outs, _ = tl.gpu_path(case)
    n = tl.visible(case)
    s_host, i_host = scores.cpu().numpy(), idx.cpu().numpy()
    for r, osr in zip(range(case.T), tl.oracle_scores_rows(case, range(case.T))):
        tl.check_scores(s_host[r, :n[r]], osr, "row %d" % r)
        tl.check_topk_same_array(i_host[r], s_host[r, :n[r]], case.topk, "row %d" % r)
        tl.check_topk_margin(i_host[r], osr, case.topk, "row %d" % r)
    rows = [0, 1, 17, 35, 68, 69]
    o_or, _ = tl.oracle_mla_rows(case, rows, i_host)
    g = tl.to_f64(outs[0])
    for r, oo in zip(rows, o_or):
        tl.check_attention(g[r], oo, tl.ATTN_ATOL_LOWP, "row %d" % r)


def test_prefill_ragged_sequences_share_blocks():
    """Query blocks that span two sequences (16 query rows per indexer block)."""
    case = synth.make_case("prefill_ragged", 4, ctx=[1500, 2300, 40], q_len=[20, 37, 5], iq_dt="fp8",
                           sm_scale=1.0 / 16, kv_dt="fp8", topk=512, device=DEV)
    scores, idx, outs, _ = tl.gpu_path(case)
    _all_rows_check(case, scores, idx, outs, tl.ATTN_ATOL_LOWP, rows=[0, 15, 16, 19, 20, 31, 32, 56, 57, 61])


def _single_layer_calls_equal_shared(case, idx, outs, lses, layers=None):
    """Layer l of the shared-index entry equals sparse_mla_decode on layer l alone, bit for
    bit (outputs and lse): both sum each head's keys in the same splits and order."""
    layout = dsa.Layout.of_case(case)
    for l in (range(len(case.layers)) if layers is None else layers):
        L = case.layers[l]
        lse1 = torch.empty_like(lses[l])
        o1 = dsa.sparse_mla_decode(layout, L.q, L.kv, idx, case.sm_scale, case.Dc, L.kv_scale,
                                   out_dtype=outs[l].dtype, lse=lse1)
        torch.cuda.synchronize()
        assert torch.equal(o1, outs[l]), "layer %d: shared and single-layer outputs differ (max %.3g)" % (
            l, (o1.float() - outs[l].float()).abs().max().item())
        assert torch.equal(lse1, lses[l]), "layer %d: shared and single-layer lse differ" % l


@pytest.mark.parametrize("kv_dt,ctx", [
    ("fp8", [3000, 2100, 4096, 2500, 6000, 2048, 3333, 5000]),   # fp8 kernel, key splits
    ("bf16", [3000, 2100, 4096, 2500, 6000, 2048, 3333, 5000]),  # half-head kernel, key splits
    ("bf16", [2100 + 37 * i for i in range(70)]),                # more than 64 rows: full-head kernel
])
def test_shared_layers_match_oracle_and_single_layer_calls(kv_dt, ctx):
    """Every shared layer meets the oracle bar and equals, bit for bit, a single-layer call on
    the same indices ([anatomy], layer scheduling: a shared layer reuses the full layer's
    indices unchanged, so it must compute exactly what the full layer's own attention would)."""
    case = synth.make_case("shared_small", 5, ctx=ctx, sm_scale=1.0 / 16, kv_dt=kv_dt, n_layers=4, device=DEV)
    scores, idx, outs, lses = tl.gpu_path(case)
    rows = None if len(ctx) <= 8 else [0, 1, 35, len(ctx) - 1]
    _all_rows_check(case, scores, idx, outs, tl.ATTN_ATOL_LOWP, rows=rows)
    _single_layer_calls_equal_shared(case, idx, outs, lses)
    again = tl.gpu_path(case)
    for l in range(len(case.layers)):  # the shared call itself is deterministic
        assert torch.equal(again[2][l], outs[l]) and torch.equal(again[3][l], lses[l])


def test_recomputed_indexer_gives_identical_indices_and_outputs():
    case = synth.make_case("determinism", 2, ctx=[5000, 3000, 2048], sm_scale=1.0 / 16, kv_dt="fp8",
                           device=DEV)
    a = tl.gpu_path(case)
    b = tl.gpu_path(case)
    n = tl.visible(case)
    for r in range(case.T):  # only visible positions are written
        assert torch.equal(a[0][r, :n[r]], b[0][r, :n[r]])
    assert torch.equal(a[1], b[1]) and torch.equal(a[2][0], b[2][0]) and torch.equal(a[3][0], b[3][0])


def test_generic_kernels_match_oracle(monkeypatch):
    """The generic kernels (forced) meet the same bar on a GLM-shaped case."""
    monkeypatch.setenv("DSA_KERNEL_VARIANT", "generic")
    case = synth.make_case("generic", 2, ctx=[900, 2100], sm_scale=1.0 / 16, kv_dt="fp8", device=DEV)
    scores, idx, outs, _ = tl.gpu_path(case)
    _all_rows_check(case, scores, idx, outs, tl.ATTN_ATOL_LOWP)


def test_interleaved_132_byte_index_cache():
    """One 132-byte slot per token (128 fp8 codes then the fp32 scale), read in place."""
    case = synth.make_case("aos", 2, ctx=[700, 1300], sm_scale=1.0 / 16, device=DEV)
    N = case.N
    slab = torch.zeros((N, 132), dtype=torch.uint8, device=DEV)
    slab[:, :128] = case.ik
    slab[:, 128:] = case.ik_scale.view(torch.uint8).view(N, 4)
    layout = dsa.Layout.of_case(case)
    scale_slots = slab.view(torch.float32).view(-1)[32:]  # float 32 + 33 r = byte 128 + 132 r
    s_aos = dsa.dsa_index_scores(layout, case.iq, case.iw, slab, k_scale=scale_slots, k_row_stride=132,
                                 k_scale_stride=33, k_dtype=dsa.DSA_FP8_E4M3FN)
    torch.cuda.synchronize()
    n = tl.visible(case)
    o = tl.oracle_scores_rows(case, range(case.T))
    for r in range(case.T):
        tl.check_scores(s_aos[r, :n[r]].cpu().numpy(), o[r], "aos row %d" % r)


@pytest.mark.parametrize("kind", ["decode", "prefill"])
def test_132_byte_entries_match_key_planes_bitwise(kind):
    """132-byte index-cache entries (128 fp8 codes, then the fp32 scale: rows only 4-byte
    aligned) run on the tuned indexer kernels and give the same bits as separate key and scale
    planes, over many tiles with ragged ends; the fused indexer + top-k selects the same
    indices (rows past 32768 scores: the indexer also builds the top-k histogram)."""
    if kind == "decode":  # bf16 index queries, one per sequence: the streamed decode grid
        case = synth.make_case("aos_decode", 2, ctx=[40001, 1300, 70], device=DEV)
    else:  # fp8 index queries, several per sequence: the prefill GEMM kernel
        case = synth.make_case("aos_prefill", 4, ctx=[2600, 700], q_len=[70, 20], iq_dt="fp8", device=DEV)
    N = case.N
    slab = torch.zeros((N, 132), dtype=torch.uint8, device=DEV)
    slab[:, :128] = case.ik
    slab[:, 128:] = case.ik_scale.view(torch.uint8).view(N, 4)
    scale_slots = slab.view(torch.float32).view(-1)[32:]
    layout = dsa.Layout.of_case(case)
    aos = dict(k_scale=scale_slots, k_row_stride=132, k_scale_stride=33, k_dtype=dsa.DSA_FP8_E4M3FN,
               q_scale=case.iq_scale)
    planes = dict(k_scale=case.ik_scale, q_scale=case.iq_scale)
    s_pl = dsa.dsa_index_scores(layout, case.iq, case.iw, case.ik, **planes)
    s_ao = dsa.dsa_index_scores(layout, case.iq, case.iw, slab, **aos)
    _, i_pl = dsa.dsa_index_topk(layout, case.iq, case.iw, case.ik, case.topk, **planes)
    _, i_ao = dsa.dsa_index_topk(layout, case.iq, case.iw, slab, case.topk, **aos)
    torch.cuda.synchronize()
    n = tl.visible(case)
    for r in range(case.T):
        assert torch.equal(s_ao[r, :n[r]], s_pl[r, :n[r]]), "row %d: 132-byte entries and planes differ" % r
    assert torch.equal(i_ao, i_pl)
    o = tl.oracle_scores_rows(case, [0, case.T - 1])
    for r, osr in zip([0, case.T - 1], o):
        tl.check_scores(s_ao[r, :n[r]].cpu().numpy(), osr, "row %d" % r)


# ------------------------------------------------------------------------------ top-k edge cases

def _topk_rows(rows, k=2048, workspace=None):
    """Run dsa_topk on the given fp32 rows (one sequence per row) and compare bit-exactly."""
    ctx = [len(r) for r in rows]
    ld = max(ctx)
    sc = np.zeros((len(rows), ld), np.float32)
    for i, r in enumerate(rows):
        sc[i, :len(r)] = r
    kvp = torch.tensor(np.concatenate([[0], np.cumsum(ctx)]), dtype=torch.int64, device=DEV)
    layout = dsa.Layout(kvp, None, len(rows), ld)
    idx = dsa.dsa_topk(layout, torch.from_numpy(sc).to(DEV), k, workspace=workspace)
    torch.cuda.synchronize()
    ih = idx.cpu().numpy()
    for i, r in enumerate(rows):
        tl.check_topk_same_array(ih[i], np.asarray(r, np.float32), k, "edge row %d (n=%d)" % (i, len(r)))
    return layout


@pytest.mark.parametrize("n", [1, 2, 2047, 2048, 2049, 4096, 4097, 9000, 70000])
def test_topk_sizes_random(n):
    rng = np.random.default_rng(n)
    _topk_rows([rng.standard_normal(n).astype(np.float32) * 8])


def test_topk_ties_and_signed_zeros():
    rng = np.random.default_rng(7)
    rows = [
        np.full(5000, 1.5, np.float32),                                   # all equal: tie path
        np.where(rng.random(6000) < 0.5, -0.0, 0.0).astype(np.float32),   # only signed zeros
        rng.integers(-3, 4, 50000).astype(np.float32),                    # 7 distinct values
        np.round(rng.standard_normal(30000), 1).astype(np.float32),       # heavy ties
        np.sort(rng.standard_normal(10000)).astype(np.float32),           # ascending
        -np.sort(-rng.standard_normal(10000)).astype(np.float32),         # descending
        np.concatenate([np.full(3000, -np.inf), rng.standard_normal(3000)]).astype(np.float32),
    ]
    _topk_rows(rows)


def test_topk_single_block_rows():
    """Rows of at most 8192 scores: one block per row bins by value over the row's range,
    falling back to key bits when the range is zero or not finite; the threshold bin's
    members are ranked by counting (few) or by a radix select (many)."""
    rng = np.random.default_rng(21)
    f = np.float32
    rows = [
        np.full(5000, 1.5, f),                                            # zero range, all tied
        np.where(rng.random(6000) < 0.5, -0.0, 0.0).astype(f),            # only signed zeros
        rng.integers(-3, 4, 8192).astype(f),                              # 7 distinct values
        np.round(rng.standard_normal(8192), 1).astype(f),                 # heavy ties
        np.sort(rng.standard_normal(8191)).astype(f),                     # ascending; ld % 4 != 0
        -np.sort(-rng.standard_normal(7000)).astype(f),                   # descending
        np.concatenate([np.full(3000, -np.inf), rng.standard_normal(3000)]).astype(f),
        np.concatenate([rng.standard_normal(4000), [np.inf, np.inf]]).astype(f),
        (1.0 + (np.arange(6000) % 97) * np.finfo(f).eps).astype(f),       # a range of 96 ulps
        (rng.standard_normal(6000) * 1e-41).astype(f),                    # subnormal range
        (np.clip(rng.standard_normal(6000), -3.3, 3.3) * 1e38).astype(f),  # the range overflows
        np.concatenate([rng.standard_normal(1500) + 10, np.full(3000, 2.0),
                        rng.standard_normal(3000)]).astype(f),            # 3000 tied members
        np.concatenate([rng.standard_normal(1900) + 50, rng.uniform(1.0, 1.0001, 300),
                        rng.standard_normal(5000)]).astype(f),            # > 256 members: radix
        np.concatenate([rng.standard_normal(1900) + 50, rng.uniform(1.0, 1.0001, 150),
                        rng.standard_normal(5000)]).astype(f),            # < 256 members: counting
        rng.standard_normal(2047).astype(f), rng.standard_normal(2048).astype(f), np.zeros(1, f),
    ]
    for r in rows:
        rng.shuffle(r)
    rows[4] = np.sort(rows[4])
    rows[5] = -np.sort(-rows[5])
    _topk_rows(rows)
    for k in (1, 7, 64, 1000):
        _topk_rows(rows, k=k)


def test_topk_threshold_bin_overflow():
    """More keys share the bin of the k-th key than the member list holds: the exact radix
    refinement over the row itself, with the ties taken in position order (rows of one block
    held in LDS, and rows whose histogram and members are spread over many blocks)."""
    rng = np.random.default_rng(11)
    rows = [
        np.full(20000, 1.5, np.float32),
        rng.integers(0, 2, 30000).astype(np.float32),
        np.concatenate([rng.standard_normal(1000) + 10, np.full(15000, 2.0), rng.standard_normal(5000)]).astype(np.float32),
    ]
    _topk_rows(rows)
    rows = [
        np.full(100000, -1.25, np.float32),
        rng.integers(0, 3, 70000).astype(np.float32),
        np.concatenate([rng.standard_normal(1500) + 10, np.full(40000, 2.0), rng.standard_normal(60000)]).astype(np.float32),
    ]
    _topk_rows(rows)


def test_topk_longest_rows_many_blocks():
    """Rows longer than 262144 scores (a bitmap too large for LDS): histogram and marking
    spread over many blocks per row, then one block per row selects among the members."""
    rng = np.random.default_rng(14)
    rows = [rng.standard_normal(300000).astype(np.float32), np.round(rng.standard_normal(270000), 2).astype(np.float32),
            rng.standard_normal(5000).astype(np.float32), np.full(263000, 0.5, np.float32)]
    _topk_rows(rows)


def test_topk_many_long_rows():
    """More than 512 ragged rows longer than 8192 (one block per row, rows in registers)."""
    rng = np.random.default_rng(12)
    rows = [rng.standard_normal(int(n)).astype(np.float32) for n in rng.integers(8193, 12000, 520)]
    rows[5] = np.round(rows[5], 1)
    rows[9] = np.full(9000, -2.0, np.float32)
    _topk_rows(rows)


def test_topk_workspace_reused_across_layouts():
    """One workspace serves calls with different layouts and is all zero after each call."""
    rng = np.random.default_rng(13)
    big = [rng.standard_normal(n).astype(np.float32) for n in (270000, 20000, 9000, 300000)]
    small = [rng.standard_normal(n).astype(np.float32) for n in [280000] * 3]
    lay_b = _topk_rows(big, workspace=None)
    lay_s = _topk_rows(small, workspace=None)
    nb = max(dsa.dsa_topk_workspace_size(lay_b, 300000, 2048), dsa.dsa_topk_workspace_size(lay_s, 280000, 2048))
    assert nb > 0
    ws = torch.zeros(nb, dtype=torch.uint8, device=DEV)
    for rows in (big, small, big):
        _topk_rows(rows, workspace=ws)
        assert int(torch.count_nonzero(ws)) == 0, "workspace not left zero"


def test_topk_small_k_and_wide_ld():
    rng = np.random.default_rng(9)
    rows = [rng.standard_normal(n).astype(np.float32) for n in (100, 5000, 33000)]
    for k in (1, 7, 64, 1000):
        _topk_rows(rows, k=k)


# ------------------------------------------------------------------------ full-size workloads

@pytest.mark.parametrize("cfg,rows", [(2, list(range(8))), (3, [0, 5, 17, 33, 40, 51, 63]),
                                      (4, [0, 1, 511, 1024, 2047, 3001, 4094, 4095]), (5, [0, 9, 18, 31])])
def test_full_size_workload_sampled_rows(cfg, rows):
    case = synth.config(cfg, DEV)
    scores, idx, outs, lses = tl.gpu_path(case)
    _all_rows_check(case, scores, idx, outs, tl.ATTN_ATOL_LOWP, rows=rows)
    if cfg == 5:  # the IndexShare workload: shared layers equal single-layer calls bit for bit
        _single_layer_calls_equal_shared(case, idx, outs, lses, layers=[0, 3])
    del case, scores, idx, outs, lses
    torch.cuda.empty_cache()


def test_extreme_logit_spread_takes_exact_rerun():
    """A late tile whose logit exceeds the first tile's maximum by far more than 2^100 (in
    exp2 units) makes the tuned kernel rerun its split with the exact maximum; the output
    must still match the oracle.  256 one-query sequences give one block per row, so all
    32 tiles of the index list run in the same block."""
    B, ctx, H, Dc, Dr = 256, 2048, 64, 512, 64
    g = torch.Generator(device=DEV).manual_seed(123)
    kv = torch.randn((B * ctx, Dc + Dr), generator=g, device=DEV)
    q = torch.randn((B, H, Dc + Dr), generator=g, device=DEV)
    for b in (0, 1):
        kv[b * ctx:(b + 1) * ctx, 0] = 0.0
        kv[b * ctx + 1500, 0] = 64.0
        q[b, :, 0] = 64.0
    kv = kv.to(torch.bfloat16)
    q = q.to(torch.bfloat16)
    kvp = torch.arange(0, (B + 1) * ctx, ctx, dtype=torch.int64, device=DEV)
    layout = dsa.Layout(kvp, None, B, ctx)
    idx = torch.arange(ctx, dtype=torch.int32, device=DEV).repeat(B, 1).contiguous()
    lse = torch.empty((B, H), dtype=torch.float32, device=DEV)
    out = dsa.sparse_mla_decode(layout, q, kv, idx, 1.0 / 16, Dc, lse=lse)
    torch.cuda.synchronize()
    import oracle
    for b in (0, 1, 2):
        o, l = oracle.sparse_mla([0, ctx], None, synth.host(q[b:b + 1]), synth.host(kv[b * ctx:(b + 1) * ctx]),
                                 idx[b:b + 1].cpu().numpy(), 1.0 / 16, Dc)
        tl.check_attention(tl.to_f64(out[b]), o[0], tl.ATTN_ATOL_LOWP, "row %d" % b)
        np.testing.assert_allclose(lse[b].cpu().numpy(), l[0], rtol=1e-4, atol=1e-3)


def test_draft_steps_reuse_the_first_steps_indices():
    """Speculative draft steps reuse the index set chosen at draft step 0 (the anatomy page's
    MTP note: later draft steps skip the indexer and top-k).  The context grows by one
    token per step; the reused indices (all below the step-0 context) stay valid, and each
    step's attention meets the oracle on them, bitwise equal to the same call made on the
    step-0 layout."""
    c0, D = 5000, 3
    case = synth.make_case("draft", 2, ctx=[c0 + D], kv_dt="bf16", sm_scale=1.0 / 16, device=DEV)
    L = case.layers[0]
    kv_ptr0 = torch.tensor([0, c0], dtype=torch.int64, device=DEV)
    lay0 = dsa.Layout(kv_ptr0, None, 1, c0)
    scores = dsa.dsa_index_scores(lay0, case.iq, case.iw, case.ik, k_scale=case.ik_scale)
    idx = dsa.dsa_topk(lay0, scores, case.topk)
    torch.cuda.synchronize()
    i_host = idx.cpu().numpy()
    assert i_host.max() < c0
    g = torch.Generator(device=DEV).manual_seed(77)
    for d in range(1, D + 1):
        q = torch.randn((1, case.H, case.Dc + case.Dr), generator=g, device=DEV).to(torch.bfloat16)
        lay = dsa.Layout(torch.tensor([0, c0 + d], dtype=torch.int64, device=DEV), None, 1, c0 + d)
        out = dsa.sparse_mla_decode(lay, q, L.kv, idx, case.sm_scale, case.Dc, L.kv_scale)
        out0 = dsa.sparse_mla_decode(lay0, q, L.kv, idx, case.sm_scale, case.Dc, L.kv_scale)
        torch.cuda.synchronize()
        assert torch.equal(out, out0)
        o_or, _ = oracle.sparse_mla([0, c0 + d], None, synth.host(q), synth.host(L.kv[:c0 + d]), i_host,
                                    case.sm_scale, case.Dc, L.kv_scale)
        tl.check_attention(tl.to_f64(out)[0], o_or[0], tl.ATTN_ATOL_LOWP, "draft step %d" % d)
