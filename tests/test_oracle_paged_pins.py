"""Pins for the oracle's paged-cache layout (CPU only).

With a block table, token s of sequence b lives in physical row
block_table[b, s // page] * page + s % page of every per-token cache; the top-k's
positions map to physical rows the same way, and sparse MLA then reads those rows.  The
pins: a hand-worked mapping, and the invariant that scattering a contiguous cache's pages
over a pool (any permutation) changes no score and no attention output, bit for bit,
because every value is read from the same bytes in the same order.
"""
import numpy as np
import pytest

import oracle


def test_page_mapping_hand_example():
    """Page 4, sequence 0 on pages [5, 2], sequence 1 on [0]: positions 0, 3, 4, 6 of
    sequence 0 are rows 20, 23, 8, 10; position 1 of sequence 1 is row 1."""
    idx = np.array([[0, 3, 4, 6, -1], [1, -1, -1, -1, -1]], np.int32)
    bt = np.array([[5, 2], [0, 0]], np.int32)
    got = oracle.to_physical([0, 8, 10], None, idx, bt, 4)
    assert got.tolist() == [[20, 23, 8, 10, -1], [1, -1, -1, -1, -1]]


def _scatter(ctx, page, rows_per_tok, seed):
    """A contiguous cache layout and a paged pool holding the same rows at shuffled pages."""
    rng = np.random.default_rng(seed)
    kv_indptr = np.concatenate([[0], np.cumsum(ctx)]).astype(np.int64)
    npages = [-(-c // page) for c in ctx]
    total_pages = sum(npages) + 3  # spare pages nobody uses
    perm = rng.permutation(total_pages)
    bt = np.zeros((len(ctx), max(npages)), np.int32)
    k = 0
    for b, n in enumerate(npages):
        bt[b, :n] = perm[k:k + n]
        k += n
    contig = rng.standard_normal((int(kv_indptr[-1]), rows_per_tok)).astype(np.float32)
    pool = rng.standard_normal((total_pages * page, rows_per_tok)).astype(np.float32)  # junk elsewhere
    for b, c in enumerate(ctx):
        for s in range(c):
            pool[bt[b, s // page] * page + s % page] = contig[kv_indptr[b] + s]
    return kv_indptr, bt, contig, pool


@pytest.mark.parametrize("page", [1, 4, 16])
def test_scattered_pages_give_the_same_scores(page):
    ctx = [37, 16, 50]
    kv_indptr, bt, contig, pool = _scatter(ctx, page, 8, seed=page)
    rng = np.random.default_rng(1)
    T, H = len(ctx), 3
    q = rng.standard_normal((T, H, 8)).astype(np.float32)
    w = rng.standard_normal((T, H)).astype(np.float32)
    ks_c = rng.uniform(0.5, 2, contig.shape[0]).astype(np.float32)
    ks_p = np.ones(pool.shape[0], np.float32)
    for b, c in enumerate(ctx):
        for s in range(c):
            ks_p[bt[b, s // page] * page + s % page] = ks_c[kv_indptr[b] + s]
    s_c = oracle.index_scores(kv_indptr, None, q, w, contig, k_scale=ks_c)
    s_p = oracle.index_scores(kv_indptr, None, q, w, pool, k_scale=ks_p, block_table=bt, page_size=page)
    assert np.array_equal(np.nan_to_num(s_c, nan=7.0), np.nan_to_num(s_p, nan=7.0))


@pytest.mark.parametrize("page", [2, 16])
def test_scattered_pages_give_the_same_attention(page):
    """Top-k positions mapped to physical rows select the same latent rows: outputs and lse
    equal the contiguous layout's bit for bit (a wrong page lookup or offset fails here)."""
    ctx = [40, 23]
    Dc, Dr, H, k = 12, 4, 2, 16
    kv_indptr, bt, contig, pool = _scatter(ctx, page, Dc + Dr, seed=10 + page)
    rng = np.random.default_rng(2)
    q = rng.standard_normal((len(ctx), H, Dc + Dr)).astype(np.float32)
    n = oracle.visible_counts(kv_indptr, None, len(ctx))
    scores = rng.standard_normal((len(ctx), max(ctx)))
    idx = oracle.topk(scores, n, k)
    o_c, l_c = oracle.sparse_mla(kv_indptr, None, q, contig, idx, 0.25, Dc)
    phys = oracle.to_physical(kv_indptr, None, idx, bt, page)
    o_p, l_p = oracle.sparse_mla(kv_indptr, None, q, pool, phys, 0.25, Dc, physical=True)
    assert np.array_equal(o_c, o_p) and np.array_equal(l_c, l_p)


def test_physical_indices_past_the_pool_are_rejected():
    q = np.zeros((1, 1, 8), np.float32)
    kv = np.zeros((10, 8), np.float32)
    with pytest.raises(ValueError):
        oracle.sparse_mla([0, 5], None, q, kv, np.array([[3, 10]], np.int32), 1.0, 4, physical=True)
    o, _ = oracle.sparse_mla([0, 5], None, q, kv, np.array([[3, 9]], np.int32), 1.0, 4, physical=True)
    assert o.shape == (1, 1, 4)
