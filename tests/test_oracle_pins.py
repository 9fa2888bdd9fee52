"""Pins for the fp64 oracle (CPU only).

Each test checks the oracle against something other than itself: values fixed
by the fp8 / bf16 format definitions, hand-worked examples (tests/golden),
library routines on special cases (numpy dot and lexsort, torch's scaled-dot-
product attention in float64), closed forms and invariants.  Each test names
the plausible mistake it would catch.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from deepseek_sparse_mla_amd import synth

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _worked():
    with open(os.path.join(GOLD, "worked_examples.json")) as f:
        return json.load(f)


# ------------------------------------------------------------------------------------ decoders

def test_fp8_decoder_spot_values_from_format_definition():
    """Format table values (wrong bias, subnormal or sign handling fails here)."""
    rows = []
    with open(os.path.join(GOLD, "fp8_e4m3fn_values.txt")) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                c, v = line.split()
                rows.append((int(c, 16), float(v)))
    for code, val in rows:
        got = float(oracle.decode_fp8(np.array([code], np.uint8))[0])
        if math.isnan(val):
            assert math.isnan(got), hex(code)
        else:
            assert got == val and math.copysign(1, got) == math.copysign(1, val), hex(code)


def test_fp8_decoder_all_256_codes_match_torch():
    """Exhaustive: all 256 codes against torch's float8_e4m3fn widening (a library routine)."""
    codes = np.arange(256, dtype=np.uint8)
    ours = oracle.decode_fp8(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    finite = np.isfinite(ref)
    assert finite.sum() == 254  # two NaN patterns, no infinities
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    assert np.array_equal(ours[finite], ref[finite])
    assert np.array_equal(np.signbit(ours[finite]), np.signbit(ref[finite]))


def test_fp8_values_are_exact_in_bf16():
    """Every finite E4M3FN value widens to bf16 without rounding (the PR page's premise)."""
    vals = oracle.decode_fp8(np.arange(256, dtype=np.uint8))
    vals = vals[np.isfinite(vals)]
    back = torch.tensor(vals).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(back, vals)


def test_bf16_decoder_matches_torch():
    rng = np.random.default_rng(0)
    bits = np.concatenate([rng.integers(0, 1 << 16, 4000), [0, 0x8000, 0x3F80, 0x7F7F, 0x0001]]).astype(np.uint16)
    bits = bits[((bits >> 7) & 0xFF) != 0xFF]  # skip inf/NaN patterns
    ours = oracle.decode_bf16(bits)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(ours, ref)


# ------------------------------------------------------------------------------------- layout

def test_visible_counts_causal():
    """Query j of a q_len-long chunk at the end of a ctx-long sequence sees ctx - q_len + j + 1."""
    kv = np.array([0, 10, 30], np.int64)
    qi = np.array([0, 3, 4], np.int32)
    assert list(oracle.visible_counts(kv, qi, 4)) == [8, 9, 10, 20]
    assert list(oracle.visible_counts(kv, None, 2)) == [10, 20]


# ------------------------------------------------------------------------------------- indexer

def test_indexer_worked_example():
    """Hand-worked two-token example (catches ReLU after the head sum, a dropped scale,
    a transposed q)."""
    ex = _worked()["indexer"]
    q = np.array(ex["q"], np.float32)[None]
    k = np.array(ex["k"], np.float32)
    s = oracle.index_scores([0, 2], None, q, np.array(ex["w"], np.float32)[None], k,
                            k_scale=np.array(ex["k_scale"], np.float32))
    assert np.array_equal(s[0], np.array(ex["scores"]))


def test_indexer_single_head_is_relu_of_dot():
    """H=1, w=1, scales=1: the score is ReLU(q.k), checked with numpy's dot."""
    rng = np.random.default_rng(1)
    q = rng.standard_normal((1, 1, 37)).astype(np.float32)
    k = rng.standard_normal((50, 37)).astype(np.float32)
    s = oracle.index_scores([0, 50], None, q, np.ones((1, 1), np.float32), k)
    ref = np.maximum(k.astype(np.float64) @ q[0, 0].astype(np.float64), 0)
    np.testing.assert_allclose(s[0], ref, rtol=1e-13, atol=1e-13)


@pytest.mark.parametrize("h", [0, 2, 5])
def test_indexer_one_hot_weights_pick_one_head(h):
    """w = e_h: only head h contributes, with its own q row (catches [H][D] vs [D][H] swaps
    and per-head scale mix-ups)."""
    rng = np.random.default_rng(2 + h)
    H, D, n = 6, 9, 20
    q = rng.standard_normal((1, H, D)).astype(np.float32)
    k = rng.standard_normal((n, D)).astype(np.float32)
    qs = rng.uniform(0.5, 2.0, (1, H)).astype(np.float32)
    ks = rng.uniform(0.5, 2.0, n).astype(np.float32)
    w = np.zeros((1, H), np.float32)
    w[0, h] = 1.5
    s = oracle.index_scores([0, n], None, q, w, k, k_scale=ks, q_scale=qs)
    ref = 1.5 * np.maximum(k.astype(np.float64) @ q[0, h].astype(np.float64), 0) * qs[0, h] * ks
    np.testing.assert_allclose(s[0], ref, rtol=1e-13, atol=1e-13)


def test_indexer_zero_weights_and_linearity():
    rng = np.random.default_rng(3)
    H, D, n = 4, 8, 30
    q = rng.standard_normal((1, H, D)).astype(np.float32)
    k = rng.standard_normal((n, D)).astype(np.float32)
    z = oracle.index_scores([0, n], None, q, np.zeros((1, H), np.float32), k)
    assert np.all(z[0] == 0)
    w1 = rng.standard_normal((1, H)).astype(np.float32)
    w2 = rng.standard_normal((1, H)).astype(np.float32)
    s1 = oracle.index_scores([0, n], None, q, w1, k)
    s2 = oracle.index_scores([0, n], None, q, w2, k)
    s12 = oracle.index_scores([0, n], None, q, (w1.astype(np.float64) + w2).astype(np.float32), k)
    # w1 + w2 is not always exact in fp32; compare against the exactly-summed weights' effect
    np.testing.assert_allclose(s12, s1 + s2, rtol=1e-6, atol=1e-9)


def test_indexer_scale_factors_out_of_relu():
    """Positive scales commute with ReLU: doubling every key scale doubles every score."""
    rng = np.random.default_rng(4)
    H, D, n = 4, 16, 25
    q = rng.standard_normal((1, H, D)).astype(np.float32)
    k = rng.standard_normal((n, D)).astype(np.float32)
    w = rng.standard_normal((1, H)).astype(np.float32)
    ks = rng.uniform(0.1, 3, n).astype(np.float32)
    a = oracle.index_scores([0, n], None, q, w, k, k_scale=ks)
    b = oracle.index_scores([0, n], None, q, w, k, k_scale=2 * ks)
    np.testing.assert_array_equal(b, 2 * a)


def test_indexer_sequences_use_their_own_keys():
    """Row b must read keys kv_indptr[b] .. kv_indptr[b+1]-1 (an offset mistake fails here)."""
    rng = np.random.default_rng(5)
    H, D = 3, 8
    ctx = [7, 11, 5]
    kvp = np.cumsum([0] + ctx)
    q = rng.standard_normal((3, H, D)).astype(np.float32)
    w = np.abs(rng.standard_normal((3, H))).astype(np.float32)
    k = rng.standard_normal((sum(ctx), D)).astype(np.float32)
    s = oracle.index_scores(kvp, None, q, w, k)
    for b in range(3):
        kb = k[kvp[b]:kvp[b + 1]].astype(np.float64)
        ref = (np.maximum(kb @ q[b].astype(np.float64).T, 0) * w[b]).sum(1)
        np.testing.assert_allclose(s[b, :ctx[b]], ref, rtol=1e-12, atol=1e-12)
        assert np.all(np.isnan(s[b, ctx[b]:]))  # invisible positions are never written


def test_indexer_causal_prefill_rows():
    rng = np.random.default_rng(6)
    H, D, ctx, ql = 2, 4, 12, 5
    q = rng.standard_normal((ql, H, D)).astype(np.float32)
    w = np.ones((ql, H), np.float32)
    k = rng.standard_normal((ctx, D)).astype(np.float32)
    s = oracle.index_scores([0, ctx], [0, ql], q, w, k)
    for j in range(ql):
        n = ctx - ql + j + 1
        ref = np.maximum(k[:n].astype(np.float64) @ q[j].astype(np.float64).T, 0).sum(1)
        np.testing.assert_allclose(s[j, :n], ref, rtol=1e-12, atol=1e-12)
        assert np.all(np.isnan(s[j, n:]))


def test_indexer_fp8_interleaved_132_byte_rows_equal_split_planes():
    """One 132-byte slot per token (128 fp8 codes then an fp32 scale) reads like two planes."""
    c = synth.make_case(ctx=[40], H_I=32, D_I=128, iq_dt="bf16", ik_dt="fp8", H=1, Dc=8, Dr=0,
                        topk=16)
    codes = synth.host(c.ik)
    ks = synth.host(c.ik_scale)
    slab = np.zeros((40, 132), np.uint8)
    slab[:, :128] = codes
    slab[:, 128:] = ks.view(np.uint8).reshape(40, 4)
    q, w = synth.host(c.iq), synth.host(c.iw)
    a = oracle.index_scores([0, 40], None, q, w, codes, k_scale=ks)
    flat = slab.reshape(-1)
    b = oracle.index_scores([0, 40], None, q, w, flat.reshape(40, 132)[:, :128].copy(), k_scale=ks)
    # direct AoS read: k pointer over the slab, stride 132, scale at byte 128 with stride 33 floats
    scales_view = np.frombuffer(flat.tobytes(), dtype=np.float32, offset=128)
    d = oracle.index_scores([0, 40], None, q, w, flat.reshape(40, 132), k_scale=scales_view,
                            k_row_stride_bytes=132, k_scale_stride=33)
    np.testing.assert_array_equal(a, b)
    np.testing.assert_array_equal(a, d)


def test_indexer_magnitude_bounds_value():
    c = synth.config(1)
    s, m = oracle.index_scores(synth.host(c.kv_indptr), None, synth.host(c.iq), synth.host(c.iw),
                               synth.host(c.ik), with_magnitude=True)
    assert np.all(np.abs(s[0]) <= m[0] * (1 + 1e-12))


# ---------------------------------------------------------------------------------------- top-k

def test_topk_worked_example():
    ex = _worked()["topk"]
    s = np.array([ex["scores"]])
    assert list(oracle.topk(s, [7], 5)[0]) == ex["k5"]
    assert list(oracle.topk(s, [7], 8)[0]) == ex["k8"]


@pytest.mark.parametrize("n,k", [(1, 1), (10, 3), (100, 16), (257, 64), (2000, 2048), (5000, 2048)])
def test_topk_matches_lexsort(n, k):
    """Against numpy's lexsort on (position asc within score desc), with forced ties."""
    rng = np.random.default_rng(n * 7 + k)
    s = rng.standard_normal((3, n)).round(1)  # rounding creates many ties
    s[1] = 0.0  # an all-equal row
    s[2, ::2] = -0.0
    got = oracle.topk(s, [n] * 3, k)
    for r in range(3):
        order = np.lexsort((np.arange(n), -s[r]))
        take = min(n, k)
        exp = np.full(k, -1, np.int32)
        exp[:take] = order[:take]
        assert np.array_equal(got[r], exp)


def test_topk_respects_visible_count_and_pads():
    s = np.array([[5.0, 4.0, 3.0, 100.0, 200.0]])
    assert list(oracle.topk(s, [3], 4)[0]) == [0, 1, 2, -1]  # entries past n are ignored


def test_topk_all_equal_scores_take_lowest_positions():
    s = np.full((1, 50), 1.25)
    assert list(oracle.topk(s, [50], 8)[0]) == list(range(8))


# ----------------------------------------------------------------------------------- sparse MLA

def test_mla_worked_example():
    ex = _worked()["sparse_mla"]
    q = np.array(ex["q"], np.float32)[None, None]
    kv = np.array(ex["kv"], np.float32)
    o, lse = oracle.sparse_mla([0, 2], None, q, kv, np.array([ex["indices"]], np.int32),
                               ex["sm_scale"], ex["Dc"])
    np.testing.assert_allclose(o[0, 0], ex["out"], rtol=1e-7)
    np.testing.assert_allclose(lse[0, 0], ex["lse"], rtol=1e-7)


def _dense_sdpa(q, kv, Dc, scale):
    """torch's scaled-dot-product attention in float64 over every row (keys = whole rows,
    values = first Dc columns).  q: [H, Dqk]; kv: [S, Dqk]."""
    H = q.shape[0]
    query = torch.from_numpy(q.astype(np.float64))[None, :, None, :]          # [1, H, 1, Dqk]
    kt = torch.from_numpy(kv.astype(np.float64))
    key = kt[None, None].expand(1, H, -1, -1)                                 # [1, H, S, Dqk]
    value = kt[None, None, :, :Dc].expand(1, H, -1, -1)                       # [1, H, S, Dc]
    out = torch.nn.functional.scaled_dot_product_attention(query, key, value, scale=scale)
    return out[0, :, 0].numpy()


def test_mla_take_all_equals_dense_sdpa():
    """k >= context: sparse MLA is dense softmax attention (caveats box of the anatomy page),
    checked against torch's SDPA in float64."""
    c = synth.config(1)
    q = synth.host(c.layers[0].q)
    kv = synth.host(c.layers[0].kv)
    n = c.ctx[0]
    idx = np.arange(n, dtype=np.int32)[None]
    o, _ = oracle.sparse_mla([0, n], None, q, kv, idx, c.sm_scale, c.Dc)
    ref = _dense_sdpa(q[0], kv, c.Dc, c.sm_scale)
    np.testing.assert_allclose(o[0], ref, rtol=1e-12, atol=1e-13)


def test_mla_single_index_returns_that_row():
    rng = np.random.default_rng(8)
    q = rng.standard_normal((1, 3, 10)).astype(np.float32)
    kv = rng.standard_normal((6, 10)).astype(np.float32)
    idx = np.array([[-1, 4, -1]], np.int32)
    o, lse = oracle.sparse_mla([0, 6], None, q, kv, idx, 0.3, 7)
    for h in range(3):
        np.testing.assert_array_equal(o[0, h], kv[4, :7].astype(np.float64))
        np.testing.assert_allclose(lse[0, h], 0.3 * float(q[0, h].astype(np.float64) @ kv[4].astype(np.float64)), rtol=1e-12)


def test_mla_zero_query_is_mean_of_selected_values():
    rng = np.random.default_rng(9)
    kv = rng.standard_normal((9, 6)).astype(np.float32)
    idx = np.array([[2, 7, 0, -1, 5]], np.int32)
    o, lse = oracle.sparse_mla([0, 9], None, np.zeros((1, 2, 6), np.float32), kv, idx, 1.0, 4)
    ref = kv[[2, 7, 0, 5], :4].astype(np.float64).mean(0)
    np.testing.assert_allclose(o[0, 0], ref, rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(lse[0], math.log(4), rtol=1e-13)


def test_mla_index_order_does_not_matter():
    c = synth.config(1)
    q, kv = synth.host(c.layers[0].q), synth.host(c.layers[0].kv)
    rng = np.random.default_rng(10)
    sel = rng.choice(64, 16, replace=False).astype(np.int32)
    o1, l1 = oracle.sparse_mla([0, 64], None, q, kv, sel[None], c.sm_scale, c.Dc)
    o2, l2 = oracle.sparse_mla([0, 64], None, q, kv, rng.permutation(sel)[None], c.sm_scale, c.Dc)
    np.testing.assert_allclose(o1, o2, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(l1, l2, rtol=1e-12)


def test_mla_empty_selection_and_bad_indices():
    q = np.ones((1, 1, 4), np.float32)
    kv = np.ones((5, 4), np.float32)
    o, lse = oracle.sparse_mla([0, 5], None, q, kv, np.full((1, 3), -1, np.int32), 1.0, 2)
    assert np.all(o == 0) and lse[0, 0] == -np.inf
    with pytest.raises(ValueError):
        oracle.sparse_mla([0, 5], None, q, kv, np.array([[1, 5]], np.int32), 1.0, 2)  # >= n
    with pytest.raises(ValueError):
        oracle.sparse_mla([0, 5], None, q, kv, np.array([[1, 1]], np.int32), 1.0, 2)  # repeated
    with pytest.raises(ValueError):  # causal row 0 of a 2-query chunk sees 4 of 5 tokens
        oracle.sparse_mla([0, 5], [0, 2], np.ones((2, 1, 4), np.float32), kv,
                          np.array([[4, -1], [4, -1]], np.int32), 1.0, 2)


def test_mla_fp8_scale_equals_scaled_fp32():
    rng = np.random.default_rng(11)
    codes = rng.integers(0, 256, (12, 8)).astype(np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0x10  # no NaN codes
    vals = oracle.decode_fp8(codes)
    q = rng.standard_normal((1, 2, 8)).astype(np.float32)
    idx = np.array([[0, 3, 11, 7]], np.int32)
    o8, l8 = oracle.sparse_mla([0, 12], None, q, codes, idx, 0.25, 6, kv_scale=0.375)
    of, lf = oracle.sparse_mla([0, 12], None, q, (vals * 0.375).astype(np.float32), idx, 0.25, 6)
    np.testing.assert_allclose(o8, of, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(l8, lf, rtol=1e-12)


# ----------------------------------------------------------------------------------- index share

def test_shared_layer_equals_recomputing_indexer():
    """A shared layer's output is identical to running indexer + top-k again for it."""
    c = synth.make_case(ctx=[90, 130], H_I=4, D_I=16, iq_dt="f32", ik_dt="fp8", topk=32, H=3,
                        Dc=16, Dr=8, mla_q_dt="f32", kv_dt="f32", n_layers=3, seed=3)
    kvp = synth.host(c.kv_indptr)
    idx_in = dict(q=synth.host(c.iq), w=synth.host(c.iw), k=synth.host(c.ik), k_scale=synth.host(c.ik_scale))
    layers = [dict(q=synth.host(L.q), kv=synth.host(L.kv), kv_scale=L.kv_scale) for L in c.layers]
    ind, outs = oracle.index_share(kvp, None, idx_in, layers, c.topk, c.sm_scale, c.Dc)
    for l, L in enumerate(layers):
        ind2, outs2 = oracle.index_share(kvp, None, idx_in, [L], c.topk, c.sm_scale, c.Dc)
        assert np.array_equal(ind, ind2)
        assert np.array_equal(outs[l][0], outs2[0][0]) and np.array_equal(outs[l][1], outs2[0][1])


def test_pipeline_with_k_at_least_context_is_dense_attention():
    """Indexer + top-k (k >= context) + sparse MLA equals dense attention over every token."""
    c = synth.make_case(ctx=[48], H_I=4, D_I=16, iq_dt="f32", ik_dt="f32", topk=64, H=2, Dc=12,
                        Dr=4, mla_q_dt="f32", kv_dt="f32", seed=4)
    kvp = synth.host(c.kv_indptr)
    idx_in = dict(q=synth.host(c.iq), w=synth.host(c.iw), k=synth.host(c.ik))
    q, kv = synth.host(c.layers[0].q), synth.host(c.layers[0].kv)
    ind, outs = oracle.index_share(kvp, None, idx_in, [dict(q=q, kv=kv)], 64, c.sm_scale, c.Dc)
    assert sorted(ind[0][:48]) == list(range(48)) and np.all(ind[0][48:] == -1)
    np.testing.assert_allclose(outs[0][0][0], _dense_sdpa(q[0], kv, c.Dc, c.sm_scale), rtol=1e-12, atol=1e-13)
