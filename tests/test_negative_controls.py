"""Negative controls for the acceptance checks (CPU only, no GPU result involved).

Each GPU parity test passes only if its check would have caught a real mistake.  Here every
check is fed arrays that carry one planted mistake of the kind a kernel could make, and
must fail:

* scores: one token's index-cache scale doubled; the four fp8 key bytes of one dword of one
  token swapped (a wrong byte order inside a load);
* top-k on the same array: one selected position shifted by +1; a tie taken by the higher
  position instead of the lower one; a padding slot not -1; a listing out of order;
* top-k against the oracle's scores: a position far below the boundary taken;
* attention: every latent row's bytes swapped within its dwords; the per-tensor latent
  scale doubled; one head's output taken from the next head.

The planted arrays come from the oracle itself on seeded synthetic inputs (the input
generator on the CPU), so each control fails for the planted reason alone.  The same arrays
without the mistake pass, which the first assertion of each test shows.
"""
import numpy as np
import pytest
import torch

import dsa_testlib as tl
import oracle
from deepseek_sparse_mla_amd import synth


@pytest.fixture(scope="module")
def case():
    oracle.build()
    return synth.make_case("negative_controls", 2, ctx=[3000, 2300], sm_scale=1.0 / 16, kv_dt="fp8",
                           device="cpu")


def _scores(case, ik=None, ik_scale=None):
    n = tl.visible(case)
    base = tl.row_bases(case)
    iq, iw = synth.host(case.iq), synth.host(case.iw)
    ik = synth.host(case.ik) if ik is None else ik
    iks = synth.host(case.ik_scale) if ik_scale is None else ik_scale
    out = []
    for i in range(case.T):
        ni, b0 = int(n[i]), int(base[i])
        out.append(oracle.index_scores([0, ni], None, iq[i:i + 1], iw[i:i + 1], ik[b0:b0 + ni],
                                       k_scale=iks[b0:b0 + ni])[0])
    return out


def test_scores_check_catches_a_doubled_token_scale(case):
    ref = _scores(case)
    tl.check_scores(ref[0], ref[0], "unchanged")
    s = int(np.argmax(ref[0]))  # a token with a clearly positive score
    iks = synth.host(case.ik_scale).copy()
    iks[s] *= 2.0
    bad = _scores(case, ik_scale=iks)
    with pytest.raises(AssertionError, match="out of tolerance"):
        tl.check_scores(bad[0], ref[0], "scale x2")


def test_scores_check_catches_bytes_swapped_within_a_dword(case):
    ref = _scores(case)
    ik = synth.host(case.ik).copy()
    s = int(np.argmax(ref[0]))
    d = ik[s].view(np.uint32).copy()
    d[5] = ((d[5] & 0xFF) << 24) | ((d[5] >> 8 & 0xFF) << 16) | ((d[5] >> 16 & 0xFF) << 8) | (d[5] >> 24)
    ik[s] = d.view(np.uint8)
    assert not np.array_equal(ik[s], synth.host(case.ik)[s])
    bad = _scores(case, ik=ik)
    with pytest.raises(AssertionError, match="out of tolerance"):
        tl.check_scores(bad[0], ref[0], "bytes swapped")


def _same_array_selection(scores_row, k):
    """The selection the library must produce: the oracle's set in ascending order, padded."""
    n = scores_row.size
    exp = oracle.topk(scores_row[None].astype(np.float64), [n], k)[0]
    take = min(n, k)
    g = np.full(k, -1, np.int64)
    g[:take] = np.sort(np.asarray(exp[:take], np.int64))
    return g


def test_topk_check_catches_an_index_shifted_by_one(case):
    row = _scores(case)[0].astype(np.float32)
    g = _same_array_selection(row, 2048)
    tl.check_topk_same_array(g, row, 2048, "unchanged")
    # shift the first selected position whose successor is not selected
    sel = set(g.tolist())
    j = next(j for j in range(2048) if g[j] + 1 not in sel and g[j] + 1 < row.size)
    bad = g.copy()
    bad[j] += 1
    with pytest.raises(AssertionError, match="differs"):
        tl.check_topk_same_array(bad, row, 2048, "index +1")


def test_topk_check_catches_a_flipped_tie():
    rng = np.random.default_rng(5)
    row = rng.standard_normal(5000).astype(np.float32)
    k = 100
    order = np.argsort(-row, kind="stable")
    tau = row[order[k - 1]]
    row[4321] = tau  # a tie with the k-th score at a higher position: the lower one is taken
    g = _same_array_selection(row, k)
    tl.check_topk_same_array(g, row, k, "unchanged")
    assert int(order[k - 1]) in g.tolist() and 4321 not in g.tolist()
    bad = np.sort(np.where(g == order[k - 1], 4321, g))
    bad = np.concatenate([bad[bad >= 0], g[g < 0]])
    with pytest.raises(AssertionError, match="differs"):
        tl.check_topk_same_array(bad, row, k, "tie flipped")


def test_topk_check_catches_bad_padding_and_order():
    rng = np.random.default_rng(6)
    row = rng.standard_normal(1500).astype(np.float32)
    g = _same_array_selection(row, 2048)
    tl.check_topk_same_array(g, row, 2048, "unchanged")
    pad = g.copy()
    pad[1600] = 0
    with pytest.raises(AssertionError, match="padding"):
        tl.check_topk_same_array(pad, row, 2048, "padding")
    swapped = g.copy()
    swapped[[10, 11]] = swapped[[11, 10]]
    with pytest.raises(AssertionError, match="ascending"):
        tl.check_topk_same_array(swapped, row, 2048, "order")


def test_topk_margin_check_catches_a_far_position(case):
    ref = _scores(case)[0]
    g = _same_array_selection(ref.astype(np.float32), 2048)
    tl.check_topk_margin(g, ref, 2048, "unchanged")
    worst = int(np.argmin(ref))
    bad = np.sort(np.concatenate([g[1:2048], [worst]]))
    with pytest.raises(AssertionError, match="beyond the margin"):
        tl.check_topk_margin(bad, ref, 2048, "far position")


def _attention(case, kv=None, kv_scale=None, row=0):
    n = tl.visible(case)
    base = tl.row_bases(case)
    L = case.layers[0]
    ni, b0 = int(n[row]), int(base[row])
    kvh = synth.host(L.kv)[b0:b0 + ni] if kv is None else kv[b0:b0 + ni]
    idx = _same_array_selection(_scores(case)[row].astype(np.float32), case.topk)[None].astype(np.int32)
    o, _ = oracle.sparse_mla([0, ni], None, synth.host(L.q[row:row + 1]), kvh, idx, case.sm_scale, case.Dc,
                             L.kv_scale if kv_scale is None else kv_scale)
    return o[0]


def test_attention_check_catches_swapped_latent_bytes(case):
    ref = _attention(case)
    tl.check_attention(ref, ref, tl.ATTN_ATOL_LOWP, "unchanged")
    kv = synth.host(case.layers[0].kv).copy()
    w = kv.view(np.uint32)
    w[:] = ((w & 0xFF) << 8) | ((w >> 8) & 0xFF) | ((w >> 16 & 0xFF) << 24) | ((w >> 24) << 16)
    bad = _attention(case, kv=kv)
    with pytest.raises(AssertionError, match="max"):
        tl.check_attention(bad, ref, tl.ATTN_ATOL_LOWP, "bytes swapped")


def test_attention_check_catches_a_doubled_latent_scale(case):
    ref = _attention(case)
    bad = _attention(case, kv_scale=2.0 * case.layers[0].kv_scale)
    with pytest.raises(AssertionError, match="max"):
        tl.check_attention(bad, ref, tl.ATTN_ATOL_LOWP, "kv_scale x2")


def test_attention_check_catches_a_head_shift(case):
    ref = _attention(case)
    bad = np.roll(ref, 1, axis=0)
    with pytest.raises(AssertionError, match="max"):
        tl.check_attention(bad, ref, tl.ATTN_ATOL_LOWP, "head shift")
