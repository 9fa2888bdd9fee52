"""Index-cache writer on the GPU (through the C ABI) against the oracle, bit for bit.

The writer's outputs are integers (fp8 codes) and powers of two (scales), so every
check is an exact byte comparison with the oracle's encoder, which is pinned to
torch's float8 cast and to closed forms on the CPU.  Both sides take the rope in
fp32 with each product and sum rounded on its own, so the codes it decides agree.
"""
import numpy as np
import pytest
import torch

import deepseek_sparse_mla_amd as dsa
import dsa_testlib as tl
import oracle
from deepseek_sparse_mla_amd import synth

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _bf16_bits(x: torch.Tensor) -> np.ndarray:
    return x.to(torch.bfloat16).cpu().view(torch.int16).numpy().view(np.uint16)


def _oracle_in(x: torch.Tensor) -> np.ndarray:
    return _bf16_bits(x) if x.dtype == torch.bfloat16 else x.float().cpu().numpy()


def _randn(shape, seed, spread=3.0):
    g = torch.Generator().manual_seed(seed)
    x = torch.randn(shape, generator=g)
    # per-group magnitudes over many binades, so the scale takes many values
    return x * torch.exp(spread * torch.randn(shape[:-1] + (1,), generator=g))


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("rope_off", [None, 0, 64])
def test_k_cache_write_planes(dtype, rope_off):
    """1000 keys (62.5 blocks of 16) into a 1500-row plane cache through a scattered slot
    list with padding slots; rows no slot names keep their bytes."""
    n, rows = 1000, 1500
    k = _randn((n, 1, 128), 1).to(dtype)
    rng = np.random.default_rng(2)
    slots = rng.permutation(rows)[:n].astype(np.int64)
    slots[rng.choice(n, 37, replace=False)] = -1
    pos = rng.integers(0, 4096, n).astype(np.int64)
    tab = synth.rope_table(4096, device="cpu")
    init_c = rng.integers(0, 256, (rows, 128)).astype(np.uint8)
    init_s = rng.standard_normal(rows).astype(np.float32)

    cache = torch.from_numpy(init_c).to(DEV)
    scale = torch.from_numpy(init_s).to(DEV)
    kw = {}
    if rope_off is not None:
        kw = dict(positions=torch.from_numpy(pos).to(DEV), cos_sin=tab.to(DEV), rope_off=rope_off)
    dsa.dsa_index_k_cache_write(k.reshape(n, 128).to(DEV), torch.from_numpy(slots).to(DEV), cache,
                                scale, **kw)
    torch.cuda.synchronize()

    okw = {}
    if rope_off is not None:
        okw = dict(positions=pos, cos_sin=tab.numpy(), rope_off=rope_off)
    oc, os_ = oracle.index_quant(_oracle_in(k), dst_rows=slots, codes=init_c[:, None, :],
                                 scales=init_s[:, None], **okw)
    assert np.array_equal(cache.cpu().numpy(), oc[:, 0, :])
    assert np.array_equal(scale.cpu().numpy().view(np.uint32), os_[:, 0].view(np.uint32))


def test_k_cache_write_interleaved_132_byte_entries_and_strided_keys():
    """The 132-byte entries (codes then the fp32 scale) from keys that are a column slice
    of a wider projection output (row stride 160 values: 128 key + 32 head weights)."""
    n, rows = 333, 400
    wide = _randn((n, 160), 3).to(torch.bfloat16)
    k = wide[:, :128]
    rng = np.random.default_rng(4)
    slots = rng.permutation(rows)[:n].astype(np.int64)
    pos = rng.integers(0, 1000, n).astype(np.int64)
    tab = synth.rope_table(1000, device="cpu")
    init = rng.integers(0, 256, (rows, 132)).astype(np.uint8)
    init[:, 128:] = np.frombuffer(np.full(rows, 7.0, np.float32).tobytes(), np.uint8).reshape(rows, 4)

    buf = torch.from_numpy(init).to(DEV)
    flat = buf.view(-1)
    scale_view = flat[128:].view(torch.uint8)  # byte view; the library takes a raw pointer
    wide_d = wide.to(DEV)
    dsa.dsa_index_k_cache_write(wide_d[:, :128], torch.from_numpy(slots).to(DEV), buf, scale_view,
                                positions=torch.from_numpy(pos).to(DEV), cos_sin=tab.to(DEV),
                                cache_row_stride=132, cache_scale_stride=33, cache_rows=rows)
    torch.cuda.synchronize()
    got = buf.cpu().numpy()

    oc, os_ = oracle.index_quant(_oracle_in(k.contiguous()).reshape(n, 1, 128), positions=pos,
                                 cos_sin=tab.numpy(), dst_rows=slots,
                                 codes=init[:, None, :128],
                                 scales=init[:, 128:].copy().view(np.float32))
    assert np.array_equal(got[:, :128], oc[:, 0, :])
    assert np.array_equal(got[:, 128:].copy().view(np.float32)[:, 0].view(np.uint32),
                          os_[:, 0].view(np.uint32))


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_q_quant_prefill_rows(dtype):
    """300 index-query rows of 32 heads (a ragged 9600 groups) with rope at each row's
    position."""
    T, H = 300, 32
    q = _randn((T, H, 128), 5).to(dtype)
    pos = np.arange(28672 - 7, 28672 - 7 + T, dtype=np.int64)
    tab = synth.rope_table(32768, device="cpu")
    codes, scales = dsa.dsa_index_q_quant(q.to(DEV), positions=torch.from_numpy(pos).to(DEV),
                                          cos_sin=tab.to(DEV))
    oc, os_ = oracle.index_quant(_oracle_in(q), positions=pos, cos_sin=tab.numpy())
    assert np.array_equal(codes.cpu().numpy(), oc)
    assert np.array_equal(scales.cpu().numpy().view(np.uint32), os_.view(np.uint32))


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_q_quant_four_groups_per_team(dtype):
    """517 rows x 32 heads (16544 groups): the launch shape where each 16-lane team takes
    four heads of one row, with a ragged last block; every row checked."""
    T, H = 517, 32
    q = _randn((T, H, 128), 12).to(dtype)
    pos = np.random.default_rng(13).integers(0, 32768, T).astype(np.int64)
    tab = synth.rope_table(32768, device="cpu")
    codes, scales = dsa.dsa_index_q_quant(q.to(DEV), positions=torch.from_numpy(pos).to(DEV),
                                          cos_sin=tab.to(DEV), rope_off=64)
    oc, os_ = oracle.index_quant(_oracle_in(q), positions=pos, cos_sin=tab.numpy(), rope_off=64)
    assert np.array_equal(codes.cpu().numpy(), oc)
    assert np.array_equal(scales.cpu().numpy().view(np.uint32), os_.view(np.uint32))


@pytest.mark.parametrize("T,H", [(700, 5), (2100, 8)])
def test_q_quant_other_head_counts(T, H):
    """Head counts other than 32: an odd count (one group per team: rows' heads do not split
    into fours) and 8 heads over 16800 groups (four per team); every row checked."""
    q = _randn((T, H, 128), 18).to(torch.bfloat16)
    pos = np.random.default_rng(19).integers(0, 4096, T).astype(np.int64)
    tab = synth.rope_table(4096, device="cpu")
    codes, scales = dsa.dsa_index_q_quant(q.to(DEV), positions=torch.from_numpy(pos).to(DEV),
                                          cos_sin=tab.to(DEV))
    oc, os_ = oracle.index_quant(_oracle_in(q), positions=pos, cos_sin=tab.numpy())
    assert np.array_equal(codes.cpu().numpy(), oc)
    assert np.array_equal(scales.cpu().numpy().view(np.uint32), os_.view(np.uint32))


def test_rounding_on_every_tie_and_its_neighbours():
    """Groups whose largest value is 448 (scale 1) and whose other values are every tie
    between adjacent E4M3FN codes, one fp32 step either side, and the codes themselves."""
    vals = oracle.decode_fp8(np.arange(127, dtype=np.uint8))
    pts = [vals]
    mids = 0.5 * (vals[:-1] + vals[1:])
    pts += [mids, np.nextafter(mids.astype(np.float32), np.float32(0)).astype(np.float64),
            np.nextafter(mids.astype(np.float32), np.float32(1e9)).astype(np.float64)]
    p = np.concatenate(pts)
    p = np.concatenate([p, -p]).astype(np.float32)
    per = 127
    G = (len(p) + per - 1) // per
    x = np.zeros((G, per + 1), np.float32)
    x[:, 0] = 448.0
    x[:, 1:].flat[:len(p)] = p
    x = x[:, None, :]
    codes, scales = dsa.dsa_index_q_quant(torch.from_numpy(x).to(DEV))
    oc, os_ = oracle.index_quant(x)
    assert np.all(os_ == 1.0)
    assert np.array_equal(codes.cpu().numpy(), oc)
    assert np.array_equal(scales.cpu().numpy(), os_)


def test_special_groups():
    """All zero (scale 1), all -0 (codes 0x80), subnormal-only groups (scale 2^-126),
    values near the fp32 maximum, groups mixing 1e30 with 1e-30 (products underflow),
    exact powers 448 * 2^k, and a group just past a power-of-two boundary."""
    G = 12
    x = np.zeros((G, 1, 128), np.float32)
    x[1] = -0.0
    x[2] = np.float32(1e-40)
    x[3, 0, ::2] = -np.float32(3e-41)
    x[4] = np.float32(3.0e38) * np.linspace(-1, 1, 128, dtype=np.float32)
    x[5, 0, 0], x[5, 0, 1:] = 1e30, 1e-30
    x[6, 0, 0] = 448 * 2.0 ** 20
    x[6, 0, 1:] = np.linspace(-3, 3, 127) * 2.0 ** 16
    x[7, 0, 0] = np.nextafter(np.float32(448 * 2.0 ** -3), np.float32(1e9))
    x[7, 0, 1:] = 1.0
    x[8] = np.float32(1.17549435e-38)  # the smallest normal
    x[9, 0, :64], x[9, 0, 64:] = -1.0, 2.0 ** -20
    x[10] = np.float32(2.0 ** -133) * np.arange(128, dtype=np.float32)
    x[11] = np.random.default_rng(6).standard_normal(128).astype(np.float32)
    codes, scales = dsa.dsa_index_q_quant(torch.from_numpy(x).to(DEV))
    oc, os_ = oracle.index_quant(x)
    assert np.array_equal(codes.cpu().numpy(), oc)
    assert np.array_equal(scales.cpu().numpy().view(np.uint32), os_.view(np.uint32))


def test_written_keys_feed_the_indexer():
    """Keys written by the writer (no rope) are byte-identical to the generator's stored
    keys, so the indexer over them returns the same scores bit for bit."""
    case = synth.make_case("writer", 2, ctx=[700, 1300], kv_dt="bf16", device=DEV)
    rows = int(case.kv_indptr[-1])
    g = torch.Generator().manual_seed(8)
    kf = torch.randn(rows, 128, generator=g).to(DEV)
    ref_codes, ref_scale = synth.quant_rows_pow2(kf)
    cache = torch.zeros(rows, 128, dtype=torch.uint8, device=DEV)
    scale = torch.zeros(rows, dtype=torch.float32, device=DEV)
    dsa.dsa_index_k_cache_write(kf, torch.arange(rows, device=DEV), cache, scale)
    assert torch.equal(cache, ref_codes) and torch.equal(scale, ref_scale)
    L = dsa.Layout.of_case(case)
    s1 = dsa.dsa_index_scores(L, case.iq, case.iw, cache, k_scale=scale)
    s2 = dsa.dsa_index_scores(L, case.iq, case.iw, ref_codes.contiguous(), k_scale=ref_scale.contiguous())
    torch.cuda.synchronize()
    for i, n in enumerate(tl.visible(case)):  # entries past a row's visible count are not written
        assert torch.equal(s1[i, :n], s2[i, :n])


def test_decode_step_into_full_size_index_cache():
    """One decode step of 32 sequences of 131072 tokens: 32 new keys with rope at position
    131071 land in the last row of each sequence of a 4M-row, 132-byte-entry index cache
    (553 MB); sampled other rows are untouched."""
    B, ctx = 32, 131072
    rows = B * ctx
    buf = torch.zeros(rows, 132, dtype=torch.uint8, device=DEV)
    k = _randn((B, 128), 9).to(torch.bfloat16)
    slots = torch.arange(1, B + 1, dtype=torch.int64) * ctx - 1
    pos = torch.full((B,), ctx - 1, dtype=torch.int64)
    tab = synth.rope_table(ctx, device="cpu")
    dsa.dsa_index_k_cache_write(k.to(DEV), slots.to(DEV), buf, buf.view(-1)[128:],
                                positions=pos.to(DEV), cos_sin=tab.to(DEV), cache_row_stride=132,
                                cache_scale_stride=33, cache_rows=rows)
    torch.cuda.synchronize()
    got = buf[slots.to(DEV)].cpu().numpy()
    oc, os_ = oracle.index_quant(_oracle_in(k).reshape(B, 1, 128), positions=pos.numpy(),
                                 cos_sin=tab.numpy())
    assert np.array_equal(got[:, :128], oc[:, 0, :])
    assert np.array_equal(got[:, 128:].copy().view(np.float32)[:, 0], os_[:, 0])
    others = torch.randint(0, rows, (4096,), generator=torch.Generator().manual_seed(1))
    others = others[(others + 1) % ctx != 0]
    assert int(buf[others.to(DEV)].count_nonzero()) == 0


def test_prefill_queries_at_full_size_sampled_rows():
    """The prefill shape: 4096 query rows x 32 heads after a 28672-token prefix, rope at
    positions 28672..32767; 64 sampled rows checked against the oracle."""
    T, H = 4096, 32
    g = torch.Generator(device=DEV).manual_seed(10)
    q = torch.randn((T, H, 128), generator=g, device=DEV).to(torch.bfloat16)
    pos = torch.arange(28672, 28672 + T, dtype=torch.int64, device=DEV)
    tab = synth.rope_table(32768, device=DEV)
    codes, scales = dsa.dsa_index_q_quant(q, positions=pos, cos_sin=tab)
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([[0, 1, T - 1], np.random.default_rng(11).integers(0, T, 61)]))
    oc, os_ = oracle.index_quant(_oracle_in(q[rows]), positions=pos.cpu().numpy()[rows],
                                 cos_sin=tab.cpu().numpy())
    assert np.array_equal(codes[rows].cpu().numpy(), oc)
    assert np.array_equal(scales[rows].cpu().numpy(), os_)


@pytest.mark.parametrize("T,dtype", [(300, torch.bfloat16), (517, torch.float32), (4096, torch.bfloat16)])
def test_front_end_equals_the_two_calls(T, dtype):
    """The one-launch front end gives bitwise the separate calls' results (queries and the
    132-byte cache entries), checked against the oracle on every row up to 517 rows and on
    64 sampled rows of the full prefill chunk."""
    H, rows = 32, T + 77
    q = _randn((T, H, 128), 14).to(dtype).to(DEV)
    k = _randn((T, 128), 15).to(dtype).to(DEV)
    pos = torch.arange(28672, 28672 + T, dtype=torch.int64, device=DEV)
    slots = torch.from_numpy(np.random.default_rng(16).permutation(rows)[:T].astype(np.int64)).to(DEV)
    tab = synth.rope_table(32768, device=DEV)
    bufs = [torch.full((rows, 132), 5, dtype=torch.uint8, device=DEV) for _ in range(2)]
    kw = dict(cache_row_stride=132, cache_scale_stride=33, cache_rows=rows)
    c1, s1 = dsa.dsa_index_front_end(q, k, slots, bufs[0], bufs[0].view(-1)[128:], positions=pos,
                                     cos_sin=tab, **kw)
    c2, s2 = dsa.dsa_index_q_quant(q, positions=pos, cos_sin=tab)
    dsa.dsa_index_k_cache_write(k, slots, bufs[1], bufs[1].view(-1)[128:], positions=pos, cos_sin=tab, **kw)
    torch.cuda.synchronize()
    assert torch.equal(c1, c2) and torch.equal(s1.view(torch.int32), s2.view(torch.int32))
    assert torch.equal(bufs[0], bufs[1])
    rows_q = np.arange(T) if T <= 517 else np.unique(
        np.concatenate([[0, T - 1], np.random.default_rng(17).integers(0, T, 62)]))
    oc, os_ = oracle.index_quant(_oracle_in(q[rows_q]), positions=pos.cpu().numpy()[rows_q],
                                 cos_sin=tab.cpu().numpy())
    assert np.array_equal(c1[rows_q].cpu().numpy(), oc)
    assert np.array_equal(s1[rows_q].cpu().numpy().view(np.uint32), os_.view(np.uint32))
    kc, ks = oracle.index_quant(_oracle_in(k[rows_q]).reshape(len(rows_q), 1, 128),
                                positions=pos.cpu().numpy()[rows_q], cos_sin=tab.cpu().numpy())
    got = bufs[0][slots[rows_q]].cpu().numpy()
    assert np.array_equal(got[:, :128], kc[:, 0, :])
    assert np.array_equal(got[:, 128:].copy().view(np.float32)[:, 0].view(np.uint32), ks[:, 0].view(np.uint32))


def test_empty_batch_writes_nothing():
    cache = torch.full((4, 128), 9, dtype=torch.uint8, device=DEV)
    scale = torch.full((4,), 3.0, device=DEV)
    dsa.dsa_index_k_cache_write(torch.empty(0, 128, dtype=torch.bfloat16, device=DEV),
                                torch.empty(0, dtype=torch.int64, device=DEV), cache, scale)
    torch.cuda.synchronize()
    assert int((cache != 9).sum()) == 0 and bool((scale == 3.0).all())
