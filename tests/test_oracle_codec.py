"""Pins for the oracle's norm, codes and byte layouts."""
import bisect
from decimal import Decimal, getcontext
from fractions import Fraction

import numpy as np
import pytest

from oracle import codec
from oracle.hadamard import sylvester
from oracle.lloyd_max import mse_normal
from synth import sign_vector

getcontext().prec = 60
_POS_FP16 = np.arange(0, 0x7C00, dtype=np.uint16).view(np.float16)      # every finite fp16 >= 0, ascending
_POS_DEC = [Decimal(float(v)) for v in _POS_FP16]


def _brute_fp16_round(d: Decimal) -> float:
    """Nearest fp16 to a high-precision decimal, ties to even significand, saturating at 65504."""
    if d >= Decimal(65504):
        return 65504.0
    i = bisect.bisect_left(_POS_DEC, d)
    if _POS_DEC[i] == d:
        return float(_POS_FP16[i])
    lo, hi = i - 1, i
    dl, dh = d - _POS_DEC[lo], _POS_DEC[hi] - d
    if dl < dh:
        return float(_POS_FP16[lo])
    if dh < dl:
        return float(_POS_FP16[hi])
    return float(_POS_FP16[lo] if (_POS_FP16[lo:lo + 1].view(np.uint16)[0] & 1) == 0 else _POS_FP16[hi])


def _brute_norm(x16) -> float:
    s = sum(Fraction(float(v)) ** 2 for v in x16)
    d = (Decimal(s.numerator) / Decimal(s.denominator)).sqrt()
    return _brute_fp16_round(d)


def _group(vals):
    x = np.zeros(128, dtype=np.float16)
    x[:len(vals)] = np.array(vals, dtype=np.float64).astype(np.float16)
    return x


# ----------------------------------------------------------------------------- norm

@pytest.mark.parametrize("vals,want", [
    ([2048, 64, 1], 2048.0),                  # sqrt = 2049 exactly: tie between 2048 and 2050, even wins
    ([2048, 110, 14, 1], 2052.0),             # sqrt = 2051 exactly: tie between 2050 and 2052, even wins
    ([2048, 64, 1, 2.0 ** -24], 2050.0),      # a hair above the tie; an fp64 sum of squares would lose it
    ([3 * 2.0 ** -24, 4 * 2.0 ** -24], 5 * 2.0 ** -24),   # subnormal, exact
    ([-7.5], 7.5),
    ([0.0], 0.0),
])
def test_norm_special_cases(vals, want):
    assert float(codec.group_norm_fp16(_group(vals)[None])[0]) == want


def test_norm_saturates():
    x = np.full((1, 128), 65504.0, dtype=np.float16)
    assert float(codec.group_norm_fp16(x)[0]) == 65504.0


def test_norm_brute_force_random():
    rng = np.random.default_rng(7)
    xs = [rng.standard_normal(128).astype(np.float16) for _ in range(12)]
    xs += [(rng.standard_normal(128) * 1e-3).astype(np.float16) for _ in range(4)]      # subnormal-heavy
    xs += [np.clip(rng.standard_t(3, 128) * 300, -65504, 65504).astype(np.float16) for _ in range(4)]
    got = codec.group_norm_fp16(np.stack(xs))
    for x, g in zip(xs, got):
        assert float(g) == _brute_norm(x)


# ----------------------------------------------------------------------------- codes

def _brute_codes(x16, signs, cb16, n16):
    """argmin_k |y_i - n c_k| in 60-digit decimal, lower index on ties."""
    h = sylvester(128)
    xs = [Fraction(float(v)) * int(s) for v, s in zip(x16, signs)]
    root = Decimal(128).sqrt()
    c = [Decimal(float(v)) for v in cb16]
    n = Decimal(float(n16))
    out = []
    for i in range(128):
        yhat = sum(xs[j] * int(h[i, j]) for j in range(128))
        y = Decimal(yhat.numerator) / Decimal(yhat.denominator) / root
        d = [abs(y - n * ck) for ck in c]
        out.append(min(range(len(c)), key=lambda k: (d[k], k)))
    return np.array(out)


@pytest.mark.parametrize("fmt", ["turbo3", "turbo4"])
def test_codes_equal_brute_force_argmin(fmt, codebooks):
    rng = np.random.default_rng(11)
    s = sign_vector(5, "k")
    x = rng.standard_normal((3, 128)).astype(np.float16)
    x[2] = (x[2] * 40).astype(np.float16)
    codes, n16 = codec.encode(x, s, codebooks[fmt])
    for g in range(3):
        np.testing.assert_array_equal(codes[g], _brute_codes(x[g], s, codebooks[fmt], n16[g]))


@pytest.mark.parametrize("fmt", ["turbo3", "turbo4"])
def test_zero_coordinates_go_to_lower_middle_index(fmt, codebooks):
    s = sign_vector(0, "k")
    x = np.zeros((1, 128), dtype=np.float16)
    x[0, 0] = np.float16(1.0 * s[0])
    x[0, 1] = np.float16(1.0 * s[1])          # y_i = (H_i0 + H_i1)/sqrt(128): zero on every odd i
    codes, n16 = codec.encode(x, s, codebooks[fmt])
    K = len(codebooks[fmt])
    y = codec.rotated_coordinates(x, s)[0]
    assert np.all(y[1::2] == 0.0)
    assert np.all(codes[0, 1::2] == K // 2 - 1)


@pytest.mark.parametrize("fmt", ["turbo3", "turbo4"])
def test_zero_group(fmt, codebooks):
    codes, n16 = codec.encode(np.zeros((1, 128), dtype=np.float16), sign_vector(0, "v"), codebooks[fmt])
    assert float(n16[0]) == 0.0 and np.all(codes == 0)
    assert np.all(codec.dequant(codes, n16, codebooks[fmt], sign_vector(0, "v")) == 0.0)


@pytest.mark.parametrize("fmt", ["turbo3", "turbo4"])
def test_power_of_two_scaling_and_negation(fmt, codebooks):
    rng = np.random.default_rng(3)
    s = sign_vector(2, "k")
    x = rng.standard_normal((64, 128)).astype(np.float16)
    c1, n1 = codec.encode(x, s, codebooks[fmt])
    c2, n2 = codec.encode((x.astype(np.float64) * 4).astype(np.float16), s, codebooks[fmt])
    np.testing.assert_array_equal(c1, c2)
    np.testing.assert_array_equal(n2.astype(np.float64), 4 * n1.astype(np.float64))
    c3, n3 = codec.encode(-x, s, codebooks[fmt])
    np.testing.assert_array_equal(n3, n1)
    np.testing.assert_array_equal(c3.astype(int), len(codebooks[fmt]) - 1 - c1.astype(int))


@pytest.mark.parametrize("fmt,bits", [("turbo3", 3), ("turbo4", 4)])
def test_reconstruction_error_matches_lloyd_max_mse(fmt, bits, codebooks):
    rng = np.random.default_rng(4)
    s = sign_vector(0, "v")
    x = rng.standard_normal((4000, 128)).astype(np.float16)
    codes, n16 = codec.encode(x, s, codebooks[fmt])
    xh = codec.dequant(codes, n16, codebooks[fmt], s)
    xf = x.astype(np.float64)
    rel = np.sum((xf - xh) ** 2, axis=1) / np.sum(xf ** 2, axis=1)
    want = mse_normal(codebooks[fmt].astype(np.float64) * np.sqrt(128))
    assert abs(rel.mean() / want - 1) < 0.03


# Hand-placed coordinates.  A group with x_0 = a and x_1 = c (all else 0) has rotated
# coordinates y_i = (s_0 a + (-1)^i s_1 c) / sqrt(128) (row i of the Sylvester matrix has
# entries +1 and (-1)^i in columns 0 and 1), and the norm RNE_fp16(sqrt(a^2 + c^2)).  The
# pairs below were found by a search over fp16 values; "delta" is where y_0 sits relative
# to n16 * beta_j, checked below with 60-digit arithmetic.  The "+-2e-5" groups lie within
# 1e-5 of the threshold in normalised units (2e-5 / n16 < 1e-5) and the "beta" groups within
# 1e-5 of the unscaled midpoint beta_j itself, so a margin measured in normalised units, or
# against beta_j without the norm, flags them.
_MARGIN_GROUPS = {
    "turbo3": [  # (x_0, x_1, threshold j, where y_0 sits)
        (5.85546875, -0.30078125, 5, "+0.5e-5"),
        (7.73046875, -0.3984375, 5, "-0.5e-5"),
        (5.265625, -0.271484375, 5, "+2e-5"),
        (3.83984375, -0.19775390625, 5, "-2e-5"),
        (0.1256103515625, -0.375, 4, "beta"),
    ],
    "turbo4": [
        (4.2421875, 1.828125, 9, "+0.5e-5"),
        (4.1015625, 0.765625, 10, "-0.5e-5"),
        (4.4765625, 1.9296875, 9, "+2e-5"),
        (7.19921875, -0.7578125, 11, "-2e-5"),
        (0.1251220703125, -0.133056640625, 8, "beta"),
    ],
}


def _exact_coordinates(x16, signs):
    """y = H (s * x) / sqrt(128) per coordinate, as 60-digit decimals (from the matrix
    definition, not the oracle's transform)."""
    H = sylvester()
    sx = [Fraction(float(s)) * Fraction(float(v)) for s, v in zip(signs, x16)]
    root = Decimal(128).sqrt()
    out = []
    for i in range(128):
        acc = sum((sx[j] if H[i, j] > 0 else -sx[j]) for j in range(128) if sx[j] != 0)
        acc = Fraction(acc)
        out.append(Decimal(acc.numerator) / Decimal(acc.denominator) / root)
    return out


def _midpoints(codebook16):
    c = [Fraction(float(v)) for v in codebook16]
    return [(c[j] + c[j + 1]) / 2 for j in range(len(c) - 1)]


@pytest.mark.parametrize("fmt", ["turbo3", "turbo4"])
def test_boundary_margin_hand_placed(fmt, codebooks):
    """Which coordinates lie within 1e-5 (input units) of n16 * beta_j, decided in 60-digit
    arithmetic from the definition, for groups placed just inside and just outside the margin
    of a threshold scaled by a non-unit norm."""
    s = sign_vector(0, "k")
    cb = codebooks[fmt]
    mids = _midpoints(cb)
    eps = Decimal("1e-5")
    rows = []
    for x0, x1, j, where in _MARGIN_GROUPS[fmt]:
        x = _group([x0, x1])
        n16 = _brute_norm(x)
        y = _exact_coordinates(x, s)
        thr = [Decimal(float(n16)) * Decimal(m.numerator) / Decimal(m.denominator) for m in mids]
        beta_j = Decimal(mids[j].numerator) / Decimal(mids[j].denominator)
        d0 = y[0] - thr[j]
        if where == "beta":
            assert abs(y[0] - beta_j) < Decimal("0.5e-5") and abs(float(n16) - 1) > 0.2
            assert min(abs(y[0] - t) for t in thr) > eps
        else:
            target = Decimal(where.replace("e-5", "")) * eps
            assert abs(d0 - target) < Decimal("0.06e-5"), (where, d0)
            if where.endswith("2e-5"):
                assert abs(d0) / Decimal(float(n16)) < eps      # inside a normalised-units margin
        want = np.array([min(abs(yi - t) for t in thr) < eps for yi in y])
        rows.append((x, want, where))
    got = codec.boundary_margin(np.stack([r[0] for r in rows]), s, cb)
    for (x, want, where), g in zip(rows, got):
        np.testing.assert_array_equal(g, want, err_msg=where)
        assert g[0] == (where in ("+0.5e-5", "-0.5e-5")), where


@pytest.mark.parametrize("fmt", ["turbo3", "turbo4"])
def test_boundary_margin_fraction(fmt, codebooks):
    """On N(0,1) rows a rotated coordinate given the norm n is about n times a N(0, 1/128)
    variable, so the fraction within eps of the thresholds n * beta_j is about
    2 eps sum_j phi(sqrt(128) beta_j) E[sqrt(128) / n]; 15.4M coordinates (~500 to ~1000
    events) must land within 20% of it, and under the 1e-4 the parity bars allow."""
    from scipy.stats import norm
    from oracle.lloyd_max import decision_boundaries
    rng = np.random.default_rng(9)
    x = rng.standard_normal((120000, 128)).astype(np.float16)
    s = sign_vector(0, "k")
    frac = np.mean([codec.boundary_margin(x[i:i + 20000], s, codebooks[fmt]).mean()
                    for i in range(0, len(x), 20000)])
    n = codec.group_norm_fp16(x).astype(np.float64)
    b = decision_boundaries(codebooks[fmt]).astype(np.float64) * np.sqrt(128.0)
    predicted = 2e-5 * norm.pdf(b).sum() * np.mean(np.sqrt(128.0) / n)
    assert abs(frac / predicted - 1) < 0.2, (frac, predicted)
    assert frac < 1e-4


# ----------------------------------------------------------------------------- layouts

def _hex(b):
    return bytes(np.asarray(b, dtype=np.uint8)).hex(" ")


def test_sub3_hand_worked_bytes():
    # all 32 codes = 5 (0b101): A,B bytes = 01|101|101 = 0x6D; C bytes = 1|1|101|101 = 0xED
    assert _hex(codec.pack_sub3(np.full(32, 5))) == "6d 6d 6d 6d 6d 6d 6d 6d ed ed ed ed"
    # element 25 = 6 (0b110): j = 1 -> A bits 14..15 = 0b10 (A = 0x8000), C bit 14 = 1 (C = 0x4000)
    c = np.zeros(32, dtype=int)
    c[25] = 6
    assert _hex(codec.pack_sub3(c)) == "00 80 00 00 00 00 00 00 00 40 00 00"
    # element 30 = 7: j = 2 -> B bits 22..23 = 0b11 (0x00C00000), C bit 23 = 1 (0x00800000)
    c = np.zeros(32, dtype=int)
    c[30] = 7
    assert _hex(codec.pack_sub3(c)) == "00 00 00 00 00 00 c0 00 00 00 80 00"
    # element 13 = 3: B bits 11..13 = 0b011 -> B = 0x1800
    c = np.zeros(32, dtype=int)
    c[13] = 3
    assert _hex(codec.pack_sub3(c)) == "00 00 00 00 00 18 00 00 00 00 00 00"


def test_oct4_hand_worked_bytes():
    # ascending indices -> sign-magnitude nibbles: 0->F, 15->7, 7->8, 8->0, 1->E, 14->6, 9->1, 6->9
    # low nibbles of bytes 0..3 = F,7,8,0 ; high nibbles = E,6,1,9
    assert _hex(codec.pack_oct4(np.array([0, 15, 7, 8, 1, 14, 9, 6]))) == "ef 67 18 90"


def test_turbo4_nibble_semantics(codebooks):
    cb = codebooks["turbo4"].astype(np.float64)
    for k in range(16):
        nib = int(codec.turbo4_nibble(k))
        assert bool(nib & 8) == (cb[k] < 0)
        assert codec.turbo4_index(nib) == k
    mags = sorted(range(8), key=lambda m: abs(cb[codec.turbo4_index(m)]))
    assert mags == list(range(8))


def test_v_tile_hand_worked_bytes():
    # turbo4: token slot 21 = (g=1, i=5), dim 42 = (n=5, nb=2) -> chunk 21, word 2, high nibble of
    # byte 1 -> chunk byte 9, in piece 0 -> tile byte 1024*0 + 16*21 + 9 = 345 holds nibble(10) = 2 << 4;
    # all other codes 8 (nibble 0).  Dim 110 = (n=13, nb=6) of slot 30 = (g=3, i=6) -> chunk 61,
    # word 6 = chunk bytes 24..27 (piece 1, bytes 8..11); element 6 is the high nibble of the word's
    # byte 2 -> tile byte 1024 + 16*61 + 10 = 2010 holds nibble(9) = 1 << 4
    c = np.full((32, 128), 8)
    c[21, 42] = 10
    t = codec.pack_v_tiles(c, "turbo4")[0]
    nz = np.nonzero(t)[0]
    assert list(nz) == [345] and t[345] == 0x20
    c = np.full((32, 128), 8)
    c[30, 110] = 9
    t = codec.pack_v_tiles(c, "turbo4")[0]
    nz = np.nonzero(t)[0]
    assert list(nz) == [2010] and t[2010] == 0x10
    # turbo3: slot 2 = (g=0, i=2), dim 127 = (n=15, nb=7) -> chunk 15, element 58 = sub-block 1 element 26
    # -> C word of that sub-block (piece bytes 8..11), bit 22 -> piece byte 10; piece 1 of chunk 15
    # -> tile byte 768*1 + 12*15 + 10 = 958 = 0x40
    c = np.zeros((32, 128), dtype=int)
    c[2, 127] = 4
    t = codec.pack_v_tiles(c, "turbo3")[0]
    nz = np.nonzero(t)[0]
    assert list(nz) == [958] and t[958] == 0x40


def test_v_tile_slot_is_a_bijection():
    slots = sorted(codec.v_tile_slot(g, i) for g in range(4) for i in range(8))
    assert slots == list(range(32))


def test_k_record_byte_positions():
    # turbo3: dim 32q + e lives in sub-block q; turbo4: dim 8w + e lives in word w
    for d in (0, 37, 95, 127):
        c = np.zeros(128, dtype=int)
        c[d] = 7
        nz = np.nonzero(codec.pack_k_record(c, "turbo3"))[0]
        assert all(12 * (d // 32) <= b < 12 * (d // 32) + 12 for b in nz)
        c4 = np.full(128, 8)
        c4[d] = 0
        nz = np.nonzero(codec.pack_k_record(c4, "turbo4"))[0]
        assert list(nz) == [4 * (d // 8) + (d % 8) % 4]


def test_k_memory_order_hand_worked():
    # turbo4: token 37 = block 2, i = 5; dim 100 = word 12, element 4 -> high nibble of record byte 48,
    # piece 3, byte 0 -> memory byte 1024*2 + 256*3 + 16*5 + 0 = 2896 (of the 64 * 64 bytes of 64 tokens)
    c = np.full((64, 128), 8)
    c[37, 100] = 10
    mem = codec.k_records_to_memory(codec.pack_k_record(c, "turbo4"), "turbo4").reshape(-1)
    nz = np.nonzero(mem)[0]
    assert list(nz) == [2896] and mem[2896] == 0x20
    # turbo3: token 37 = block 2, i = 5.  Dim 0 = sub-block 0 element 0 -> bits 0..2 of record byte 0,
    # piece 0 -> memory byte 768*2 + 0 + 0 + 12*5 = 1596 holds 5.  Dim 100 = sub-block 3 element 4
    # -> word A bits 3..5 -> record byte 36 = piece 3 byte 0 -> 768*2 + 384 + 192 + 12*5 = 2172 holds 5 << 3
    c3 = np.zeros((64, 128), dtype=int)
    c3[37, 0] = 5
    mem3 = codec.k_records_to_memory(codec.pack_k_record(c3, "turbo3"), "turbo3").reshape(-1)
    assert list(np.nonzero(mem3)[0]) == [1596] and mem3[1596] == 5
    c3 = np.zeros((64, 128), dtype=int)
    c3[37, 100] = 5
    mem3 = codec.k_records_to_memory(codec.pack_k_record(c3, "turbo3"), "turbo3").reshape(-1)
    assert list(np.nonzero(mem3)[0]) == [2172] and mem3[2172] == 0x28
    # round trip
    rng = np.random.default_rng(2)
    for fmt, nbytes in (("turbo4", 64), ("turbo3", 48)):
        r = rng.integers(0, 256, (3, 48, nbytes), dtype=np.uint8)
        np.testing.assert_array_equal(codec.k_memory_to_records(codec.k_records_to_memory(r, fmt), fmt), r)


@pytest.mark.parametrize("fmt,k", [("turbo3", 8), ("turbo4", 16)])
def test_pack_round_trip_every_value_every_position(fmt, k):
    rng = np.random.default_rng(5)
    rows = []
    for pos in range(128):
        for v in range(k):
            r = rng.integers(0, k, 128)
            r[pos] = v
            rows.append(r)
    codes = np.array(rows)
    np.testing.assert_array_equal(codec.unpack_k_record(codec.pack_k_record(codes, fmt), fmt), codes)
    tiles = codes[:(len(codes) // 32) * 32]
    np.testing.assert_array_equal(codec.unpack_v_tiles(codec.pack_v_tiles(tiles, fmt), fmt), tiles)
    assert codec.pack_k_record(codes[:1], fmt).shape[-1] == codec.K_RECORD_BYTES[fmt]
    assert codec.pack_v_tiles(codes[:32], fmt).shape[-1] == codec.V_TILE_BYTES[fmt]


def test_f16_v_tile_hand_worked_bytes_and_round_trip():
    """The uncompressed comparison layout: token slot 21 = (g=1, i=5), dim 42 = (n=5, nb=2)
    -> chunk 21, element 8*2 + 5 = 21 -> bytes 21*128 + 2*21 = 2730..2731, little-endian fp16.
    Every value at every position round-trips bit for bit (NaN payloads and -0 included)."""
    v = np.zeros((32, 128), dtype=np.float16)
    v[21, 42] = np.float16(-1.5)                     # 0xBE00
    t = codec.pack_v_tiles(v, "f16")[0]
    assert t.shape == (8192,) and codec.V_TILE_BYTES["f16"] == 8192
    nz = np.nonzero(t)[0]
    assert list(nz) == [2731] and t[2731] == 0xBE and t[2730] == 0x00
    rng = np.random.default_rng(9)
    bits = rng.integers(0, 1 << 16, (2, 64, 128), dtype=np.uint16)
    vals = bits.view(np.float16)
    back = codec.unpack_v_tiles(codec.pack_v_tiles(vals, "f16"), "f16")
    np.testing.assert_array_equal(back.view(np.uint16), bits)


def test_reference_f16_cache_dequantises_to_its_values(codebooks):
    """fp16 K and V: the reference keeps both as given, and the bytes unpack to them."""
    from oracle import reference
    rng = np.random.default_rng(4)
    k = rng.standard_normal((2, 40, 128)).astype(np.float16)
    v = rng.standard_normal((2, 40, 128)).astype(np.float16)
    enc = reference.encode_sequence(k, v, "f16", "f16", None, None, codebooks)
    kh, vh = reference.dequant_sequence(enc, "f16", "f16", None, None, codebooks, 40)
    np.testing.assert_array_equal(kh, k.astype(np.float64))
    np.testing.assert_array_equal(vh, v.astype(np.float64))
    _, vv = reference.codes_from_library_layout(None, enc["v_tiles"], "f16", "f16")
    np.testing.assert_array_equal(vv[:, :40], v)
    assert np.all(vv[:, 40:] == 0)
