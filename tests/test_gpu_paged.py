"""Paged caches on the GPU (through the C ABI).

Every per-token cache of a case (index keys, key scales, each layer's latent rows) is
scattered page by page over a larger pool in a shuffled order, the rest of the pool filled
with unrelated values, and the path is run on the paged layout.  Each token's bytes and the
order of every reduction are unchanged, so the results must equal the contiguous run's bit
for bit: the same scores, the top-k's positions mapped through the block table, the same
attention outputs.  A small case is also checked against the oracle's paged layout.
"""
import os

import numpy as np
import pytest
import torch

import dsa_testlib as tl
import deepseek_sparse_mla_amd as dsa
import oracle
from deepseek_sparse_mla_amd import synth

pytestmark = pytest.mark.gpu

DEV = "cuda"


paged = tl.paged


def run_path(case, layout, ik, ik_scale, kvs):
    c = case
    scores = torch.full((c.T, c.max_ctx), 7.0, dtype=torch.float32, device=DEV)
    dsa.dsa_index_scores(layout, c.iq, c.iw, ik, k_scale=ik_scale, q_scale=c.iq_scale, scores=scores)
    idx = dsa.dsa_topk(layout, scores, c.topk)
    if len(c.layers) == 1:
        L = c.layers[0]
        fn = dsa.sparse_mla_prefill if c.q_indptr is not None else dsa.sparse_mla_decode
        lse = torch.empty((c.T, c.H), dtype=torch.float32, device=DEV)
        outs, lses = [fn(layout, L.q, kvs[0], idx, c.sm_scale, c.Dc, L.kv_scale, lse=lse)], [lse]
    else:
        lses = [torch.empty((c.T, c.H), dtype=torch.float32, device=DEV) for _ in c.layers]
        outs = dsa.sparse_mla_decode_shared(layout, [L.q for L in c.layers], kvs, [L.kv_scale for L in c.layers],
                                            idx, c.sm_scale, c.Dc, lses=lses)
    torch.cuda.synchronize()
    return scores, idx, outs, lses


def check_equal(case, page, bt, contig, pg):
    s_c, i_c, o_c, l_c = contig
    s_p, i_p, o_p, l_p = pg
    n = tl.visible(case)
    sc, sp = s_c.cpu().numpy(), s_p.cpu().numpy()
    for r in range(case.T):
        assert np.array_equal(sc[r, :n[r]], sp[r, :n[r]]), "scores row %d" % r
    mapped = oracle.to_physical(case.kv_indptr.cpu().numpy(), None if case.q_indptr is None
                                else case.q_indptr.cpu().numpy(), i_c.cpu().numpy(), bt.numpy(), page)
    assert np.array_equal(i_p.cpu().numpy(), mapped)
    for a, b in zip(o_c + l_c, o_p + l_p):
        assert torch.equal(a, b)


CASES = {
    "decode_bf16_page16": (dict(ctx=[3000, 8192, 5000, 700], kv_dt="bf16"), 16),
    "decode_bf16_page64": (dict(ctx=[3000, 8192, 5000, 700], kv_dt="bf16"), 64),
    "decode_fp8_long_rows_page64": (dict(ctx=[4096, 5000, 2049, 40000], kv_dt="fp8"), 64),
    "shared_fp8_page32": (dict(ctx=[3000, 2100, 6000], kv_dt="fp8", n_layers=2), 32),
    "prefill_page16": (dict(ctx=[5000, 3000], q_len=[300, 200], iq_dt="fp8", kv_dt="bf16"), 16),
    "decode_page1": (dict(ctx=[700, 2500], kv_dt="bf16"), 1),
}


@pytest.mark.parametrize("name", sorted(CASES))
def test_paged_equals_contiguous(name):
    kw, page = CASES[name]
    case = synth.make_case(name, 2, sm_scale=1.0 / 16, device=DEV, **kw)
    contig = run_path(case, dsa.Layout.of_case(case), case.ik, case.ik_scale, [L.kv for L in case.layers])
    lay, caches, bt = paged(case, page, seed=len(name))
    pg = run_path(case, lay, caches["ik"], caches["ik_scale"], caches["kv"])
    check_equal(case, page, bt, contig, pg)


def test_paged_generic_kernels_equal_contiguous():
    """A page size that is not a power of two runs the generic indexer; the generic MLA is
    forced for both runs; results still equal the contiguous ones bit for bit."""
    case = synth.make_case("generic_paged", 2, ctx=[1000, 2300], kv_dt="bf16", sm_scale=1.0 / 16, device=DEV)
    os.environ["DSA_KERNEL_VARIANT"] = "generic"
    try:
        contig = run_path(case, dsa.Layout.of_case(case), case.ik, case.ik_scale, [L.kv for L in case.layers])
        lay, caches, bt = paged(case, 24, seed=5)
        pg = run_path(case, lay, caches["ik"], caches["ik_scale"], caches["kv"])
    finally:
        del os.environ["DSA_KERNEL_VARIANT"]
    check_equal(case, 24, bt, contig, pg)
    # page 24 with the tuned MLA (only the indexer is generic then)
    lay, caches, bt = paged(case, 24, seed=6)
    pg = run_path(case, lay, caches["ik"], caches["ik_scale"], caches["kv"])
    contig = run_path(case, dsa.Layout.of_case(case), case.ik, case.ik_scale, [L.kv for L in case.layers])
    mapped = oracle.to_physical(case.kv_indptr.cpu().numpy(), None, contig[1].cpu().numpy(), bt.numpy(), 24)
    assert np.array_equal(pg[1].cpu().numpy(), mapped)
    assert torch.equal(pg[2][0], contig[2][0])


def test_paged_small_case_against_the_oracle():
    """Scores, selection and attention of a paged decode against the oracle's paged layout."""
    case = synth.make_case("paged_oracle", 2, ctx=[900, 2100, 2049], kv_dt="fp8", sm_scale=1.0 / 16, device=DEV)
    page = 32
    lay, caches, bt = paged(case, page, seed=9)
    s, idx, outs, _ = run_path(case, lay, caches["ik"], caches["ik_scale"], caches["kv"])
    kvp = case.kv_indptr.cpu().numpy()
    o_s = oracle.index_scores(kvp, None, synth.host(case.iq), synth.host(case.iw), synth.host(caches["ik"]),
                              k_scale=synth.host(caches["ik_scale"]), ld=case.max_ctx, block_table=bt.numpy(),
                              page_size=page)
    n = tl.visible(case)
    s_host = s.cpu().numpy()
    i_host = idx.cpu().numpy()
    for r in range(case.T):
        tl.check_scores(s_host[r, :n[r]], o_s[r, :n[r]], "paged row %d" % r)
    # selection: the GPU's positions (mapped) equal the oracle's top-k of the GPU's own scores
    o_idx = oracle.topk(s_host.astype(np.float64), n, case.topk)
    mapped = oracle.to_physical(kvp, None, o_idx, bt.numpy(), page)
    for r in range(case.T):
        assert np.array_equal(np.sort(i_host[r][i_host[r] >= 0]), np.sort(mapped[r][mapped[r] >= 0]))
    L = case.layers[0]
    o_o, _ = oracle.sparse_mla(kvp, None, synth.host(L.q), synth.host(caches["kv"][0]), i_host, case.sm_scale,
                               case.Dc, L.kv_scale, physical=True)
    tl.check_attention(tl.to_f64(outs[0]), o_o, tl.ATTN_ATOL_LOWP, "paged attention")


def test_writer_fills_the_paged_index_cache():
    """Keys written with rope straight into the physical rows the block table gives (slots)
    land byte for byte where the contiguous write puts them, and the paged indexer over that
    pool (other rows junk) equals the contiguous indexer bit for bit, for the plane layout and
    for 132-byte interleaved entries (read in place by the same tuned kernel, so they also equal
    the plane layout's scores)."""
    case = synth.make_case("paged_writer", 2, ctx=[700, 1300, 257], kv_dt="bf16", device=DEV)
    page = 16
    n = int(case.kv_indptr[-1])
    kvp = case.kv_indptr.cpu()
    b_of = torch.repeat_interleave(torch.arange(len(kvp) - 1), kvp[1:] - kvp[:-1])
    pos = (torch.arange(n) - kvp[:-1][b_of]).to(DEV)
    keys = torch.randn((n, 128), generator=torch.Generator(device=DEV).manual_seed(4), device=DEV).to(torch.bfloat16)
    tab = synth.rope_table(case.max_ctx, device=DEV)
    bt, dst, rows = tl.block_table(case, page, seed=3)
    lay_p = tl.paged_layout(case, page, bt, rows)
    vis = tl.visible(case)

    cache_c = torch.zeros((n, 128), dtype=torch.uint8, device=DEV)
    scale_c = torch.zeros(n, dtype=torch.float32, device=DEV)
    dsa.dsa_index_k_cache_write(keys, torch.arange(n, device=DEV), cache_c, scale_c, positions=pos, cos_sin=tab)
    ref = dsa.dsa_index_scores(dsa.Layout.of_case(case), case.iq, case.iw, cache_c, k_scale=scale_c)

    pool = torch.full((rows, 128), 0x3C, dtype=torch.uint8, device=DEV)
    pscale = torch.full((rows,), 3.0, dtype=torch.float32, device=DEV)
    dsa.dsa_index_k_cache_write(keys, dst, pool, pscale, positions=pos, cos_sin=tab)
    got = dsa.dsa_index_scores(lay_p, case.iq, case.iw, pool, k_scale=pscale)
    torch.cuda.synchronize()
    assert torch.equal(pool[dst], cache_c) and torch.equal(pscale[dst], scale_c)
    for r in range(case.T):
        assert torch.equal(got[r, :vis[r]], ref[r, :vis[r]]), "plane layout, row %d" % r

    # 132-byte entries: paged against contiguous entries, both written by the writer, and both
    # against the plane layout (the same kernel and summation order)
    def entries(n_rows, slots, layout):
        ent = torch.full((n_rows, 132), 0x3C, dtype=torch.uint8, device=DEV)
        dsa.dsa_index_k_cache_write(keys, slots, ent, ent.view(-1)[128:], positions=pos, cos_sin=tab,
                                    cache_row_stride=132, cache_scale_stride=33, cache_rows=n_rows)
        return ent, dsa.dsa_index_scores(layout, case.iq, case.iw, ent,
                                         k_scale=ent.view(torch.float32).view(-1)[32:], k_row_stride=132,
                                         k_scale_stride=33, k_dtype=dsa.DSA_FP8_E4M3FN)

    planes = ref
    ent_c, ref = entries(n, torch.arange(n, device=DEV), dsa.Layout.of_case(case))
    ent_p, got = entries(rows, dst, lay_p)
    torch.cuda.synchronize()
    assert torch.equal(ent_p[dst], ent_c) and torch.equal(ent_c[:, :128], cache_c)
    for r in range(case.T):
        assert torch.equal(got[r, :vis[r]], ref[r, :vis[r]]), "132-byte entries, row %d" % r
        assert torch.equal(ref[r, :vis[r]], planes[r, :vis[r]]), "132-byte entries against planes, row %d" % r


def test_paged_latent_pool_past_2gib():
    """A bf16 latent pool of 2.2 GB with a sequence page at its top: the tuned kernels address
    it with unsigned 32-bit offsets past 2^31 and still equal the contiguous run bit for bit."""
    case = synth.make_case("pool_2g", 2, ctx=[3000, 5000], kv_dt="bf16", sm_scale=1.0 / 16, device=DEV)
    page = 64
    rows_needed = (1 << 31) // 1152 + 70000
    used = sum(-(-c // page) for c in (3000, 5000))
    lay, caches, bt = tl.paged(case, page, seed=11, spare=-(-rows_needed // page) - used, top_page=True)
    assert int(bt[-1, 0]) * page * 1152 > (1 << 31)
    contig = run_path(case, dsa.Layout.of_case(case), case.ik, case.ik_scale, [L.kv for L in case.layers])
    pg = run_path(case, lay, caches["ik"], caches["ik_scale"], caches["kv"])
    check_equal(case, page, bt, contig, pg)


def test_paged_latent_pool_past_4gib_runs_the_generic_mla():
    """Past 4 GiB - 1 MiB of latent rows the MLA falls back to the generic kernel (64-bit
    addresses): on the same selected rows it equals the generic kernel on the contiguous cache,
    bit for bit, including a row in the pool's top page."""
    case = synth.make_case("pool_4g", 2, ctx=[2500, 4100], kv_dt="bf16", sm_scale=1.0 / 16, device=DEV)
    page = 64
    rows_needed = (1 << 32) // 1152 + 70000
    used = sum(-(-c // page) for c in (2500, 4100))
    bt, dst, rows = tl.block_table(case, page, seed=12, spare=-(-rows_needed // page) - used)
    last = rows // page - 1
    old = int(bt[-1, 0])
    if old != last:
        bt[bt == last] = old
        bt[-1, 0] = last
    kvp = case.kv_indptr.cpu()
    b_of = torch.repeat_interleave(torch.arange(2), kvp[1:] - kvp[:-1])
    s_of = torch.arange(int(kvp[-1])) - kvp[:-1][b_of]
    dst = (bt[b_of, s_of // page].to(torch.int64) * page + s_of % page).to(DEV)
    L = case.layers[0]
    pool = torch.zeros((rows, 576), dtype=torch.bfloat16, device=DEV)
    pool[dst] = L.kv
    lay = tl.paged_layout(case, page, bt, rows)
    scores = dsa.dsa_index_scores(dsa.Layout.of_case(case), case.iq, case.iw, case.ik, k_scale=case.ik_scale)
    idx = dsa.dsa_topk(dsa.Layout.of_case(case), scores, case.topk)
    idx_p = torch.from_numpy(oracle.to_physical(kvp.numpy(), None, idx.cpu().numpy(), bt.numpy(), page)).to(DEV)
    assert int(idx_p.max()) >= last * page  # the top page is read
    got = dsa.sparse_mla_decode(lay, L.q, pool, idx_p, case.sm_scale, case.Dc, L.kv_scale)
    os.environ["DSA_KERNEL_VARIANT"] = "generic"
    try:
        ref = dsa.sparse_mla_decode(dsa.Layout.of_case(case), L.q, L.kv, idx, case.sm_scale, case.Dc, L.kv_scale)
    finally:
        del os.environ["DSA_KERNEL_VARIANT"]
    torch.cuda.synchronize()
    assert torch.equal(got, ref)

