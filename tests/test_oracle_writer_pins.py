"""Pins for the oracle's index-cache writer (CPU only).

The writer's oracle turns new index keys (and prefill index queries) into the
stored form: optional interleaved rope, then one power-of-two (ue8m0) scale per
head of 128 values and OCP E4M3FN codes.  Each test checks it against something
other than itself: every code of the fp8 format table, torch's float8_e4m3fn
cast (a library routine) on every rounding tie and its fp32 neighbours, closed
forms of the scale rule, complex multiplication for the rotation, the input
generator's independent torch quantiser, and hand-built special groups.  Each
test names the plausible mistake it would catch.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from deepseek_sparse_mla_amd import synth


def _f32_next(x, direction):
    return float(np.nextafter(np.float32(x), np.float32(direction)))


def _torch_fp8(values):
    t = torch.tensor(np.asarray(values, np.float32))
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


# ------------------------------------------------------------------------------------ encoder

def test_encoder_round_trips_every_finite_code():
    """encode(decode(c)) == c for all 254 finite codes, -0 included (a wrong bias or a lost
    sign bit fails here)."""
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], np.uint8)
    assert len(codes) == 254
    assert np.array_equal(oracle.encode_fp8(oracle.decode_fp8(codes)), codes)


def test_encoder_matches_torch_on_every_tie_and_its_neighbours():
    """Ties between adjacent codes go to the even code; one fp32 step either side goes to
    the nearer code.  Checked against torch's float8_e4m3fn cast (ties-away or truncation
    fails here)."""
    vals = oracle.decode_fp8(np.arange(127, dtype=np.uint8))
    pts = []
    for a, b in zip(vals[:-1], vals[1:]):
        m = 0.5 * (a + b)  # exact in fp32: one more mantissa bit than E4M3
        assert float(np.float32(m)) == m
        pts += [m, _f32_next(m, 0.0), _f32_next(m, 1e9)]
    pts = np.array(pts)
    pts = np.concatenate([pts, -pts])
    assert np.array_equal(oracle.encode_fp8(pts), _torch_fp8(pts))


def test_encoder_matches_torch_on_random_values():
    """Random values over the whole range, subnormals and tiny values included."""
    rng = np.random.default_rng(11)
    mags = np.concatenate([rng.uniform(0, 448, 3000), 2.0 ** rng.uniform(-14, 8.8, 3000)])
    v = (mags * rng.choice([-1.0, 1.0], mags.size)).astype(np.float32).astype(np.float64)
    v = v[np.abs(v) <= 448]
    assert np.array_equal(oracle.encode_fp8(v), _torch_fp8(v))


def test_encoder_saturates_and_keeps_sign_of_zero():
    """Past 448 the code saturates to +-448; values that round to zero keep their sign."""
    got = oracle.encode_fp8([449.0, 464.0, 1e6, -500.0, -1e-9, 1e-9, 2.0 ** -10, -(2.0 ** -10)])
    assert list(got) == [0x7E, 0x7E, 0x7E, 0xFE, 0x80, 0x00, 0x00, 0x80]


# -------------------------------------------------------------------------------------- scale

@pytest.mark.parametrize("amax,scale", [
    (0.0, 1.0),
    (448.0, 1.0),
    (448.00000000001, 2.0),
    (224.0, 0.5),
    (1.0, 2.0 ** -8),
    (3.5, 2.0 ** -7),
    (3.5000001, 2.0 ** -6),
    (3.0e38, 2.0 ** 120),
    (2.0 ** -140, 2.0 ** -126),
    (448 * 2.0 ** -126, 2.0 ** -126),
    (448 * 2.0 ** -125, 2.0 ** -125),
])
def test_scale_closed_forms(amax, scale):
    """amax <= 448 * s with s the smallest such power of two (an off-by-one exponent, a
    ceil/floor swap or a missing all-zero rule fails here)."""
    assert oracle.pow2_scale([amax])[0] == scale


def test_scale_is_the_smallest_power_of_two():
    """Property over 250 binades: s = 2^e, amax / s <= 448 < amax / (s / 2), or e = -126."""
    rng = np.random.default_rng(5)
    amax = 2.0 ** rng.uniform(-130, 120, 4000)
    s = oracle.pow2_scale(amax)
    mant, _ = np.frexp(s)
    assert np.all(mant == 0.5)
    assert np.all(amax / s <= 448)
    assert np.all((amax / (s / 2) > 448) | (s == 2.0 ** -126))


def test_scale_matches_generator_quantiser():
    """The input generator's torch formulation (frexp based) agrees on normal fp32 amax."""
    rng = np.random.default_rng(6)
    amax = (2.0 ** rng.uniform(-100, 100, 5000)).astype(np.float32)
    amax[:20] = np.float32(448) * (2.0 ** np.arange(-10, 10)).astype(np.float32)
    ref = synth.pow2_scale(torch.from_numpy(amax)).double().numpy()
    assert np.array_equal(oracle.pow2_scale(amax.astype(np.float64)), ref)


# --------------------------------------------------------------------------------------- rope

def test_rope_pair_is_complex_multiplication():
    """(x0 + i x1) * (c + i s) up to fp32 rounding (a sign flip on sin or swapped outputs
    fails here)."""
    rng = np.random.default_rng(7)
    for _ in range(500):
        x0, x1 = rng.standard_normal(2).astype(np.float32)
        ang = rng.uniform(-10, 10)
        c, s = np.float32(math.cos(ang)), np.float32(math.sin(ang))
        y0, y1 = oracle.rope_pair_f32(x0, x1, c, s)
        z = complex(float(x0), float(x1)) * complex(float(c), float(s))
        bound = 2.0 ** -22 * (abs(float(x0)) + abs(float(x1)))
        assert abs(float(y0) - z.real) <= bound and abs(float(y1) - z.imag) <= bound


def test_rope_pair_identity_and_quarter_turn_are_exact():
    """c = 1, s = 0 leaves the pair unchanged; c = 0, s = 1 maps (x0, x1) to (-x1, x0)."""
    assert oracle.rope_pair_f32(1.5, -2.25, 1.0, 0.0) == (np.float32(1.5), np.float32(-2.25))
    assert oracle.rope_pair_f32(1.5, -2.25, 0.0, 1.0) == (np.float32(2.25), np.float32(1.5))


# -------------------------------------------------------------------------------- whole groups

def _table(rows, Dr=64, seed=8):
    rng = np.random.default_rng(seed)
    ang = rng.uniform(-20, 20, (rows, Dr // 2))
    return np.concatenate([np.cos(ang), np.sin(ang)], axis=1).astype(np.float32)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_groups_without_rope_match_generator_quantiser(dtype):
    """Per-(row, head) codes and scales equal the generator's torch quantiser (a group
    that spans heads, or a per-row scale, fails here)."""
    g = torch.Generator().manual_seed(9)
    x = torch.randn(37, 4, 128, generator=g) * torch.exp(4 * torch.randn(37, 4, 1, generator=g))
    if dtype == "bf16":
        x = x.to(torch.bfloat16).float()
        xin = x.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    else:
        xin = x.numpy()
    codes, scales = oracle.index_quant(xin)
    ref_c, ref_s = synth.quant_rows_pow2(x)
    assert np.array_equal(codes, ref_c.numpy())
    assert np.array_equal(scales, ref_s.numpy())


def test_groups_with_rope_rotate_interleaved_pairs():
    """Rope acts on pairs (2i, 2i+1) of dims [rope_off, rope_off + 64) with table entries i
    and 32 + i: dequantised codes match the complex rotation within half an fp8 step
    (neox-style pairing, a wrong table half or a wrong offset fails here)."""
    rng = np.random.default_rng(10)
    rows, H = 9, 3
    x = rng.standard_normal((rows, H, 128)).astype(np.float32)
    tab = _table(50)
    pos = rng.integers(0, 50, rows)
    for off in (0, 64):
        codes, scales = oracle.index_quant(x, positions=pos, cos_sin=tab, rope_off=off)
        y = x.astype(np.float64).copy()
        for r in range(rows):
            rot = tab[pos[r], :32].astype(np.float64) + 1j * tab[pos[r], 32:].astype(np.float64)
            z = (y[r, :, off:off + 64:2] + 1j * y[r, :, off + 1:off + 64:2]) * rot
            y[r, :, off:off + 64:2], y[r, :, off + 1:off + 64:2] = z.real, z.imag
        deq = oracle.decode_fp8(codes) * scales[..., None]
        s = scales[..., None].astype(np.float64)
        err = np.abs(deq - y)
        assert np.all(err <= np.maximum(np.abs(y) * 2.0 ** -4, s * 2.0 ** -10) * 1.001)
        # the other half is quantised from the untouched values
        keep = slice(64, 128) if off == 0 else slice(0, 64)
        assert np.array_equal(codes[..., keep],
                              oracle.encode_fp8(x[..., keep].astype(np.float64) / s))


def test_position_zero_row_of_identity_is_no_rope():
    """A table row of cos = 1, sin = 0 gives exactly the unrotated result."""
    rng = np.random.default_rng(12)
    x = rng.standard_normal((4, 2, 128)).astype(np.float32)
    tab = np.concatenate([np.ones((1, 32)), np.zeros((1, 32))], axis=1).astype(np.float32)
    a = oracle.index_quant(x, positions=np.zeros(4, np.int64), cos_sin=tab)
    b = oracle.index_quant(x)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_destination_rows_and_skipped_rows():
    """Group r lands in row dst[r]; dst = -1 writes nothing; other rows keep their bytes."""
    rng = np.random.default_rng(13)
    x = rng.standard_normal((5, 1, 128)).astype(np.float32)
    init_c = rng.integers(0, 256, (8, 1, 128)).astype(np.uint8)
    init_s = rng.standard_normal((8, 1)).astype(np.float32)
    dst = np.array([6, -1, 0, 3, 7], np.int64)
    codes, scales = oracle.index_quant(x, dst_rows=dst, codes=init_c, scales=init_s)
    dense_c, dense_s = oracle.index_quant(x)
    for r, d in enumerate(dst):
        if d >= 0:
            assert np.array_equal(codes[d], dense_c[r]) and scales[d, 0] == dense_s[r, 0]
    for d in (1, 2, 4, 5):
        assert np.array_equal(codes[d], init_c[d]) and scales[d, 0] == init_s[d, 0]


def test_special_groups():
    """All-zero group: codes 0, scale 1.  All -0: codes 0x80.  One value 448 * 2^k: code
    0x7E there, scale 2^k.  A subnormal-only group: scale 2^-126, codes 0."""
    x = np.zeros((4, 1, 128), np.float32)
    x[1] = -0.0
    x[2, 0, 5], x[2, 0, 6] = 448 * 2.0 ** 3, 1.0
    x[3, 0, :] = np.float32(2.0 ** -140)
    codes, scales = oracle.index_quant(x)
    assert np.all(codes[0] == 0) and scales[0, 0] == 1.0
    assert np.all(codes[1] == 0x80) and scales[1, 0] == 1.0
    assert codes[2, 0, 5] == 0x7E and scales[2, 0] == 8.0
    assert codes[2, 0, 6] == oracle.encode_fp8([1.0 / 8])[0] and np.all(codes[2, 0, 7:] == 0)
    assert scales[3, 0] == np.float32(2.0 ** -126) and np.all(codes[3] == 0)


def test_bad_positions_are_rejected():
    x = np.zeros((2, 1, 128), np.float32)
    with pytest.raises(ValueError):
        oracle.index_quant(x, positions=np.array([0, 5]), cos_sin=_table(5))


# ------------------------------------------------------------------------- rope table (input)

def test_rope_table_angles_add_and_first_frequency_is_one_radian():
    """The generator's rope table (the writer's caller-supplied input): row p holds cos then sin
    of p * theta^(-2i/64).  Pinned by properties, not by retyping it: the first frequency is 1,
    so row p, column 0 is cos(p rad) (textbook values); angles add, so row p + q is the complex
    product of rows p and q; every pair lies on the unit circle; adjacent frequencies keep the
    ratio theta^(-2/64), seen in the phase of row 1; and row 0 is the identity."""
    import math
    from deepseek_sparse_mla_amd import synth
    tab = synth.rope_table(4096).numpy().astype(np.float64)
    c, s = tab[:, :32], tab[:, 32:]
    assert np.array_equal(tab[0], np.concatenate([np.ones(32), np.zeros(32)]))
    assert abs(c[1, 0] - 0.5403023058681398) < 1e-7 and abs(s[1, 0] - 0.8414709848078965) < 1e-7  # cos 1, sin 1
    assert abs(c[3, 0] - (-0.9899924966004454)) < 1e-7                                              # cos 3
    np.testing.assert_allclose(c * c + s * s, 1.0, atol=2e-7)
    for p, q in ((1, 1), (17, 250), (1000, 3000), (2047, 2048)):
        zp, zq, zpq = c[p] + 1j * s[p], c[q] + 1j * s[q], c[p + q] + 1j * s[p + q]
        np.testing.assert_allclose(zp * zq, zpq, atol=1e-6)
    w = np.angle(c[1] + 1j * s[1])  # the 32 frequencies themselves (all below pi)
    np.testing.assert_allclose(w[1:] / w[:-1], 8e6 ** (-2.0 / 64), rtol=1e-6)
    assert math.isclose(w[0], 1.0, rel_tol=1e-7)
