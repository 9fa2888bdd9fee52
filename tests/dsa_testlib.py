"""Shared helpers of the parity tests: run the HIP path through the C ABI, compute the
oracle on sampled rows, and apply the acceptance rules.

Acceptance rules (fixed by the benchmark's tolerance statement):
  * indexer scores: |g - o| <= 1e-3 * max(|o|, rms of the oracle row);
  * top-k: identical to the oracle's top-k of the SAME fp32 score array (bit-exact), and
    against the oracle's own fp64 scores the two sets may differ only at positions whose
    oracle score lies within 1e-3 * max(|tau|, rms) of the oracle's k-th score tau;
  * sparse MLA: max |g - o| <= 2e-2 for bf16 / fp8 inputs, 1e-4 for fp32 inputs, with the
    oracle run on the GPU's indices.
"""
from __future__ import annotations

import numpy as np
import torch

import oracle
import deepseek_sparse_mla_amd as dsa
from deepseek_sparse_mla_amd import synth

SCORE_RTOL = 1e-3
MARGIN_RTOL = 1e-3
ATTN_ATOL_LOWP = 2e-2
ATTN_ATOL_F32 = 1e-4


def visible(case) -> np.ndarray:
    return oracle.visible_counts(synth.host(case.kv_indptr), synth.host(case.q_indptr), case.T)


def row_bases(case) -> np.ndarray:
    """First cache row of each query row's sequence."""
    kvp = synth.host(case.kv_indptr)
    if case.q_indptr is None:
        return kvp[:-1].copy()
    qi = synth.host(case.q_indptr)
    b = np.searchsorted(qi, np.arange(case.T), side="right") - 1
    return kvp[b]


# ----------------------------------------------------------------------------------- GPU path

def gpu_scores(case, layout=None, ld=None):
    layout = layout or dsa.Layout.of_case(case)
    return dsa.dsa_index_scores(layout, case.iq, case.iw, case.ik, k_scale=case.ik_scale,
                                q_scale=case.iq_scale, ld=ld)


def gpu_path(case, ld=None):
    """indexer -> top-k -> sparse MLA for every layer of the case (one layer: decode entry;
    several: shared entry).  Returns scores, indices, [outs], [lses]."""
    layout = dsa.Layout.of_case(case)
    scores = gpu_scores(case, layout, ld)
    idx = dsa.dsa_topk(layout, scores, case.topk)
    outs, lses = [], []
    odt = torch.float32 if case.out_dt == "f32" else torch.bfloat16
    if len(case.layers) == 1:
        L = case.layers[0]
        lse = torch.empty((case.T, case.H), dtype=torch.float32, device=L.q.device)
        fn = dsa.sparse_mla_prefill if case.q_indptr is not None else dsa.sparse_mla_decode
        o = fn(layout, L.q, L.kv, idx, case.sm_scale, case.Dc, L.kv_scale, lse=lse, out_dtype=odt)
        outs, lses = [o], [lse]
    else:
        lses = [torch.empty((case.T, case.H), dtype=torch.float32, device=case.iq.device)
                for _ in case.layers]
        outs = dsa.sparse_mla_decode_shared(layout, [L.q for L in case.layers], [L.kv for L in case.layers],
                                            [L.kv_scale for L in case.layers], idx, case.sm_scale, case.Dc,
                                            lses=lses, out_dtype=odt)
    torch.cuda.synchronize()
    return scores, idx, outs, lses


# ------------------------------------------------------------------------------ oracle, by row

def oracle_scores_rows(case, rows, with_magnitude=False):
    """Oracle scores of the listed query rows (list of fp64 arrays of length n_i)."""
    n = visible(case)
    base = row_bases(case)
    iq, iw, ik = synth.host(case.iq), synth.host(case.iw), synth.host(case.ik)
    iqs, iks = synth.host(case.iq_scale), synth.host(case.ik_scale)
    res = []
    for i in rows:
        ni, b0 = int(n[i]), int(base[i])
        out = oracle.index_scores([0, ni], None, iq[i:i + 1], iw[i:i + 1], ik[b0:b0 + ni],
                                  k_scale=None if iks is None else iks[b0:b0 + ni],
                                  q_scale=None if iqs is None else iqs[i:i + 1],
                                  with_magnitude=with_magnitude)
        res.append((out[0][0], out[1][0]) if with_magnitude else out[0])
    return res


def oracle_mla_rows(case, rows, indices_host, layer=0):
    """Oracle MLA output/lse of the listed rows on the given indices."""
    n = visible(case)
    base = row_bases(case)
    L = case.layers[layer]
    q = L.q
    outs, lses = [], []
    for i in rows:
        ni, b0 = int(n[i]), int(base[i])
        kv = synth.host(L.kv[b0:b0 + ni])
        o, l = oracle.sparse_mla([0, ni], None, synth.host(q[i:i + 1]), kv, indices_host[i:i + 1],
                                 case.sm_scale, case.Dc, L.kv_scale)
        outs.append(o[0])
        lses.append(l[0])
    return outs, lses


# ---------------------------------------------------------------------------------- acceptance

def check_scores(g_row: np.ndarray, o_row: np.ndarray, what=""):
    o = np.asarray(o_row, np.float64)
    g = np.asarray(g_row, np.float64)
    rms = float(np.sqrt(np.mean(o * o))) if o.size else 0.0
    tol = SCORE_RTOL * np.maximum(np.abs(o), rms)
    err = np.abs(g - o)
    bad = np.nonzero(err > tol)[0]
    assert bad.size == 0, "%s: %d score(s) out of tolerance, worst at %d: gpu %r oracle %r" % (
        what, bad.size, bad[np.argmax(err[bad] - tol[bad])], g[bad[0]], o[bad[0]])


def check_topk_same_array(g_idx_row: np.ndarray, scores_row_f32: np.ndarray, k: int, what=""):
    """Bit-exact check on the same score array: the library lists the selected positions in
    ascending order, the oracle in selection order (score desc, position asc); the selected
    sets must be identical, the listing strictly ascending, and the tail padded with -1."""
    n = scores_row_f32.size
    exp = oracle.topk(scores_row_f32[None].astype(np.float64), [n], k)[0]
    take = min(n, k)
    g = np.asarray(g_idx_row, np.int64)
    assert np.all(g[take:] == -1), "%s: padding slots are not -1" % what
    assert np.all(np.diff(g[:take]) > 0), "%s: selected positions are not strictly ascending" % what
    assert np.array_equal(g[:take], np.sort(np.asarray(exp[:take], np.int64))), \
        "%s: top-k set differs from the oracle on the same scores" % what


def check_topk_margin(g_idx_row: np.ndarray, o_scores_row: np.ndarray, k: int, what=""):
    n = o_scores_row.size
    o_idx = oracle.topk(o_scores_row[None], [n], k)[0]
    take = min(n, k)
    gs = set(int(x) for x in g_idx_row[:take])
    os_ = set(int(x) for x in o_idx[:take])
    assert len(gs) == take and np.all(g_idx_row[take:] == -1), "%s: bad index set size" % what
    diff = gs ^ os_
    if not diff:
        return
    tau = o_scores_row[o_idx[take - 1]]
    rms = float(np.sqrt(np.mean(o_scores_row ** 2)))
    lim = MARGIN_RTOL * max(abs(tau), rms)
    far = [s for s in diff if abs(o_scores_row[s] - tau) >= lim]
    assert not far, "%s: %d selected positions differ beyond the margin" % (what, len(far))


def check_attention(g: np.ndarray, o: np.ndarray, atol: float, what=""):
    err = np.abs(np.asarray(g, np.float64) - o)
    assert np.all(np.isfinite(g)), "%s: non-finite output" % what
    worst = float(err.max()) if err.size else 0.0
    assert worst <= atol, "%s: max |gpu - oracle| = %.3g > %.3g" % (what, worst, atol)
    return worst


def to_f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def block_table(case, page, seed=0, spare=5):
    """A block table that puts each sequence's pages at shuffled pages of a pool with `spare`
    unused pages: (table int32 [B, width] on the CPU, physical row of every contiguous cache
    row (int64, case device), rows of the pool)."""
    kvp = case.kv_indptr.cpu()
    ctx = [int(c) for c in (kvp[1:] - kvp[:-1])]
    npages = [-(-c // page) for c in ctx]
    total = sum(npages) + spare
    perm = torch.randperm(total, generator=torch.Generator().manual_seed(seed))
    width = max(max(npages), -(-case.max_ctx // page))
    bt = torch.zeros((len(ctx), width), dtype=torch.int32)
    k0 = 0
    for b, n in enumerate(npages):
        bt[b, :n] = perm[k0:k0 + n].to(torch.int32)
        k0 += n
    b_of = torch.repeat_interleave(torch.arange(len(ctx)), torch.tensor(ctx))
    s_of = torch.arange(int(kvp[-1])) - kvp[:-1][b_of]
    dst = bt[b_of, s_of // page].to(torch.int64) * page + s_of % page
    return bt, dst.to(case.kv_indptr.device), total * page


def paged_layout(case, page, bt, rows):
    return dsa.Layout(case.kv_indptr, case.q_indptr, case.T, case.max_ctx, block_table=bt.to(case.kv_indptr.device),
                      page_size=page, cache_rows=rows)


def paged(case, page, seed=0, spare=5, top_page=False):
    """(layout, caches, table) of the case's caches scattered over shuffled pages of a pool whose
    other rows hold unrelated values (`spare` unused pages; with top_page the first page of the
    last sequence is moved to the pool's last page)."""
    bt, dst, rows = block_table(case, page, seed, spare)
    if top_page:
        last = rows // page - 1
        old = int(bt[-1, 0])
        if old != last:
            bt[bt == last] = old  # whichever page held the top id takes the old one
            bt[-1, 0] = last
        kvp = case.kv_indptr.cpu()
        ctx = [int(c) for c in (kvp[1:] - kvp[:-1])]
        b_of = torch.repeat_interleave(torch.arange(len(ctx)), torch.tensor(ctx))
        s_of = torch.arange(int(kvp[-1])) - kvp[:-1][b_of]
        dst = (bt[b_of, s_of // page].to(torch.int64) * page + s_of % page).to(case.kv_indptr.device)
    dev = case.kv_indptr.device

    def scatter(x):
        if x.dtype == torch.uint8:
            pool = torch.randint(0, 120, (rows,) + tuple(x.shape[1:]), device=dev, dtype=torch.uint8,
                                 generator=torch.Generator(device=dev).manual_seed(seed + 1))
        else:
            pool = (torch.randn((rows,) + tuple(x.shape[1:]), device=dev,
                                generator=torch.Generator(device=dev).manual_seed(seed + 2)).abs() + 0.5).to(x.dtype)
        pool[dst] = x
        return pool

    caches = dict(ik=scatter(case.ik), ik_scale=scatter(case.ik_scale) if case.ik_scale is not None else None,
                  kv=[scatter(L.kv) for L in case.layers])
    return paged_layout(case, page, bt, rows), caches, bt

