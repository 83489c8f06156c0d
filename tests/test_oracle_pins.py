"""Pins of the CPU oracle against what the pages and the mathematics fix.

Nothing here compares the oracle with itself: every expected value comes from
the printed tables (tests/golden), a textbook table, a closed form, a library
routine, an exact-arithmetic special case, or brute force on tiny inputs.
"""
import os

import numpy as np
import pytest

import oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def read_signs():
    out = {}
    for ln in open(os.path.join(GOLDEN, "sign_vectors.txt")):
        if ln.startswith("#") or not ln.strip():
            continue
        k, v = ln.split(":")
        out[int(k)] = v.split()
    return out


def read_lloyd_max():
    out = {}
    for ln in open(os.path.join(GOLDEN, "lloyd_max.txt")):
        if ln.startswith("#") or not ln.strip():
            continue
        head, v = ln.split(":")
        b, kind = head.split()
        out.setdefault(int(b), {})[kind] = v.split()
    return out


# ----------------------------------------------------------------- tables

def test_sign_tables_match_printed_text():
    printed = read_signs()
    counts = {64: (35, 29), 128: (69, 59), 256: (124, 132), 512: (262, 250)}
    for d, txt in printed.items():
        want = np.array([float(t) for t in txt], np.float32)
        got = O.signs(d)
        assert got.shape == (d,)
        np.testing.assert_array_equal(got, want)
        assert set(np.unique(got)) == {-1.0, 1.0}
        assert (int((got > 0).sum()), int((got < 0).sum())) == counts[d]


def test_lloyd_max_tables_match_printed_text():
    printed = read_lloyd_max()
    assert sorted(printed) == [2, 3, 4, 5, 8]
    for b, t in printed.items():
        c, bd = O.lloyd_max(b)
        # the page builds Float32Array from the decimal text: double, then binary32
        np.testing.assert_array_equal(c, np.array([np.float32(float(x)) for x in t["centroids"]]))
        np.testing.assert_array_equal(bd, np.array([np.float32(float(x)) for x in t["boundaries"]]))
        assert c.size == 2 ** b and bd.size == 2 ** b - 1
        # each printed decimal is the exact binary32 value (round trip)
        for x in t["centroids"] + t["boundaries"]:
            assert float(np.float32(float(x))) == float(x)


def test_lloyd_max_structure():
    for b in (2, 3, 4, 5, 8):
        c, bd = O.lloyd_max(b)
        assert np.all(np.diff(c) > 0) and np.all(np.diff(bd) > 0)
        assert np.all(c[:-1] < bd) and np.all(bd < c[1:])
        # boundaries are the midpoints of adjacent centroids (Lloyd-Max
        # nearest-neighbour condition): exactly in binary32 for 2/4/5/8 bits,
        # within one ulp for the hard-coded 3-bit table
        mid = ((c[:-1] + c[1:]) / np.float32(2)).astype(np.float32)
        if b == 3:
            assert np.all(np.abs(mid - bd) <= np.spacing(np.abs(bd)) + 1e-30)
        else:
            np.testing.assert_array_equal(mid, bd)


def test_lloyd_max_centroid_condition_on_unit_gaussian():
    """Centroids sit at the conditional mean of N(0,1) over their cell: the
    Lloyd-Max centroid condition for the unit-normal source the tables were
    fitted to (closed form (phi(a) - phi(b)) / (Phi(b) - Phi(a)))."""
    from scipy.stats import norm
    for b, tol_max, tol_med in ((2, 0.005, 0.002), (3, 2e-5, 1e-5), (4, 0.02, 0.002),
                                (5, 0.02, 0.002), (8, 0.5, 0.002)):
        c, bd = O.lloyd_max(b)
        e = np.concatenate([[-np.inf], bd.astype(np.float64), [np.inf]])
        lo, hi = e[:-1], e[1:]
        cm = (norm.pdf(lo) - norm.pdf(hi)) / (norm.cdf(hi) - norm.cdf(lo))
        err = np.abs(c - cm)
        assert err.max() < tol_max and np.median(err) < tol_med, (b, err.max(), np.median(err))


def test_three_bit_table_is_the_textbook_gaussian_quantiser():
    vals = {}
    for ln in open(os.path.join(GOLDEN, "max1960_3bit.txt")):
        if ln.startswith("#") or not ln.strip():
            continue
        k, *v = ln.split()
        vals[k] = np.array([float(x) for x in v])
    c, bd = O.lloyd_max(3)
    np.testing.assert_allclose(c[4:], vals["levels"], atol=6e-4)
    np.testing.assert_allclose(-c[:4][::-1], vals["levels"], atol=6e-4)
    np.testing.assert_allclose(bd[4:], vals["thresholds"], atol=6e-4)
    assert bd[3] == 0.0


def page_tables(text):
    """The printed SIGN_VECTORS and LLOYD_MAX tables of the page "mlx-bun
    0.0.9 -> 0.0.11" (turboquant-tables.ts) as decimal strings, parsed from
    the page's text (diff lines carry a leading '+')."""
    import re
    lines = [ln[1:] if ln.startswith("+") else ln for ln in text.splitlines()]
    body = "\n".join(lines)
    sv = body[body.index("export const SIGN_VECTORS"):]
    sv = sv[:sv.index("\n};")]
    signs = {}
    for m in re.finditer(r"^\s*(\d+): \[(.*?)\]", sv, re.S | re.M):
        signs[int(m.group(1))] = re.findall(r"-?\d+", m.group(2))
    lm = body[body.index("export const LLOYD_MAX"):]
    lm = lm[:lm.index("\n};")]
    tables = {}
    for m in re.finditer(r"^\s*(\d+): \{(.*?)^\s*\},", lm, re.S | re.M):
        t = {}
        for kind in ("centroids", "boundaries"):
            k = re.search(kind + r": \[(.*?)\]", m.group(2), re.S)
            t[kind] = re.findall(r"-?[0-9][0-9.e+-]*", k.group(1))
        tables[int(m.group(1))] = t
    return signs, tables


PAGE_TEXT = os.environ.get("TQ_PAGE_TEXT", "")


@pytest.mark.skipif(not os.path.isfile(PAGE_TEXT),
                    reason="set TQ_PAGE_TEXT to the text of the tables page to compare the golden files with it")
def test_golden_tables_are_the_page_text():
    """Every printed value: each sign of every head_dim and each centroid and
    boundary of every width, as decimal text, equals the golden files."""
    signs, tables = page_tables(open(PAGE_TEXT).read())
    golden_signs = read_signs()
    assert sorted(signs) == sorted(golden_signs) == [64, 128, 256, 512]
    for d in signs:
        assert len(signs[d]) == d
        assert signs[d] == golden_signs[d], d
    golden = read_lloyd_max()
    assert sorted(tables) == sorted(golden) == [2, 3, 4, 5, 8]
    for b in tables:
        for kind in ("centroids", "boundaries"):
            assert tables[b][kind] == golden[b][kind], (b, kind)
            assert len(tables[b][kind]) == 2 ** b - (kind == "boundaries")


def test_page_table_parser_reads_a_printed_block():
    """The parser above on a block laid out as the page prints it (values
    here are placeholders, not the page's), so the page comparison cannot
    pass vacuously."""
    text = "\n".join([
        "+export const SIGN_VECTORS: Record<TurboQuantHeadDim, number[]> = {",
        "+  64: [", "+  1, -1,", "+  -1, 1,", "+  ],", "+};",
        "+export const LLOYD_MAX: Record<TurboQuantValueBits, LloydMaxTable> = {",
        "+  2: {", "+    centroids: [", "+  -1.5, -0.25, 0.25, 1.5,", "+    ],",
        "+    boundaries: [", "+  -0.875, 0, 0.875,", "+    ],", "+  },", "+};",
    ])
    signs, tables = page_tables(text)
    assert signs == {64: ["1", "-1", "-1", "1"]}
    assert tables == {2: {"centroids": ["-1.5", "-0.25", "0.25", "1.5"], "boundaries": ["-0.875", "0", "0.875"]}}


# ------------------------------------------------------------- conversions

def test_f16_conversion_matches_numpy():
    rng = np.random.default_rng(0)
    x = np.concatenate([
        rng.standard_normal(4000).astype(np.float32) * np.float32(3000),
        rng.standard_normal(2000).astype(np.float32) * np.float32(1e-5),
        np.array([0.0, -0.0, 65504, 65519.996, 65520, 65536, 1e30, -1e30, 5e7, 5.96e-8,
                  2.98e-8, 2.9802322e-08, 2.9802326e-08, 6.1035156e-05, np.inf, -np.inf],
                 np.float32),
    ])
    with np.errstate(over="ignore"):
        want = x.astype(np.float16).view(np.uint16)
    np.testing.assert_array_equal(O.f32_to_f16_bits(x), want)
    h = np.arange(0, 65536, 7, dtype=np.uint32).astype(np.uint16)
    f = O.f16_bits_to_f32(h)
    ref = h.view(np.float16).astype(np.float32)
    same = (f == ref) | (np.isnan(f) & np.isnan(ref))
    assert same.all()


def test_bf16_conversion_matches_torch():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(1)
    x = np.concatenate([
        rng.standard_normal(4000).astype(np.float32),
        (rng.standard_normal(2000) * 1e-39).astype(np.float32),
        np.array([0.0, -0.0, 3.3895314e38, 3.39e38, 3.4e38, 1e-45, 1.0039062, 1.0117188,
                  np.inf, -np.inf], np.float32),
    ])
    want = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(O.f32_to_bf16_bits(x), want)


# ---------------------------------------------------------------- rotation

def test_hadamard_scale_is_binary32_of_inverse_sqrt():
    for d in O.HEAD_DIMS:
        assert O.hadamard_scale(d) == np.float32(1.0 / np.sqrt(np.float64(d)))
    assert O.hadamard_scale(64) == 0.125 and O.hadamard_scale(256) == 0.0625


@pytest.mark.parametrize("d", [64, 128, 256, 512])
def test_hadamard_equals_dense_sylvester_product(d):
    from scipy.linalg import hadamard as sylvester
    H = sylvester(d).astype(np.float64)
    rng = np.random.default_rng(d)
    x = rng.standard_normal((4, d)).astype(np.float32)
    for row in x:
        got = O.hadamard(row).astype(np.float64)
        want = (H @ row.astype(np.float64)) / np.sqrt(d)
        np.testing.assert_allclose(got, want, rtol=0, atol=2e-6 * np.abs(want).max() + 1e-7)


@pytest.mark.parametrize("d", [64, 128, 256, 512])
def test_hadamard_exact_on_integer_rows(d):
    """Integer inputs keep every butterfly exact, so the result must equal the
    exact integer product H x rounded once by the final 1/sqrt(d) multiply."""
    from scipy.linalg import hadamard as sylvester
    H = sylvester(d).astype(np.int64)
    rng = np.random.default_rng(10 + d)
    x = rng.integers(-64, 65, size=(3, d))
    r = O.hadamard_scale(d)
    for row in x:
        got = O.hadamard(row.astype(np.float32))
        want = (H @ row).astype(np.float32) * r
        np.testing.assert_array_equal(got, want)


@pytest.mark.parametrize("d", [64, 128, 256, 512])
def test_fwht_sign_order_and_self_inverse(d):
    s = O.signs(d).astype(np.float64)
    e0 = np.zeros(d, np.float32)
    e0[0] = 1.0
    r = float(O.hadamard_scale(d))
    # encode: signs first, then transform -> s_0 * r in every position
    np.testing.assert_array_equal(O.fwht(e0, True), np.full(d, s[0] * r, np.float32))
    # decode: transform first, then signs -> s * r
    np.testing.assert_array_equal(O.fwht(e0, False), (s * r).astype(np.float32))
    rng = np.random.default_rng(d)
    x = rng.standard_normal(d).astype(np.float32)
    y = O.fwht(x, True)
    np.testing.assert_allclose(O.fwht(y, False), x, atol=3e-6)
    # Parseval: the normalised transform is orthogonal
    assert abs(np.linalg.norm(y.astype(np.float64)) - np.linalg.norm(x.astype(np.float64))) < 1e-5 * np.sqrt(d)


# -------------------------------------------------------------- bin count

@pytest.mark.parametrize("bits", [2, 3, 4, 5, 8])
def test_bin_index_is_nearest_centroid_away_from_boundaries(bits):
    c, bd = O.lloyd_max(bits)
    z = np.linspace(-6, 6, 6001, dtype=np.float32)
    z = np.concatenate([z, bd, np.nextafter(bd, np.float32(np.inf)), np.nextafter(bd, np.float32(-np.inf))])
    idx = O.bin_index(z, bits)
    near = np.argmin(np.abs(z.astype(np.float64)[:, None] - c.astype(np.float64)[None, :]), axis=1)
    dist = np.min(np.abs(z.astype(np.float64)[:, None] - bd.astype(np.float64)[None, :]), axis=1)
    far = dist > 2.4e-7
    np.testing.assert_array_equal(idx[far], near[far])
    # ties go to the lower bin (strict comparison); the next float up is above
    np.testing.assert_array_equal(O.bin_index(bd, bits), np.arange(bd.size))
    np.testing.assert_array_equal(O.bin_index(np.nextafter(bd, np.float32(np.inf)), bits), np.arange(1, bd.size + 1))
    assert O.bin_index(np.array([-1e30, 1e30], np.float32), bits).tolist() == [0, 2 ** bits - 1]


# ---------------------------------------------------------------- packing

def test_packed_dim_rule():
    for d in (64, 128, 256, 512):
        for b in (2, 3, 4, 5, 8):
            assert O.packed_dim(d, b) == d * b // 8
    assert O.packed_dim(3, 8) == 3
    for d, b in ((3, 3), (5, 2), (1, 4), (7, 5)):
        with pytest.raises(ValueError):
            O.packed_dim(d, b)


def test_pack_two_and_four_bit_formulas():
    rng = np.random.default_rng(3)
    v = rng.integers(0, 4, 64).astype(np.uint8)
    want = np.array([v[i] | v[i + 1] << 2 | v[i + 2] << 4 | v[i + 3] << 6 for i in range(0, 64, 4)], np.uint8)
    np.testing.assert_array_equal(O.pack_bits(v, 2), want)
    v = rng.integers(0, 16, 64).astype(np.uint8)
    want = np.array([v[i] | v[i + 1] << 4 for i in range(0, 64, 2)], np.uint8)
    np.testing.assert_array_equal(O.pack_bits(v, 4), want)


def test_pack_three_bit_byte_equations():
    """The page's explicit equations for 8 values in 3 bytes:
    b0 = v0 | v1<<3 | v2<<6; b1 = v2>>2 | v3<<1 | v4<<4 | v5<<7;
    b2 = v5>>1 | v6<<2 | v7<<5 (each masked to 8 bits)."""
    rng = np.random.default_rng(4)
    v = rng.integers(0, 8, 8 * 32).astype(np.int64)
    want = []
    for i in range(0, v.size, 8):
        w = v[i:i + 8]
        want += [(w[0] | w[1] << 3 | w[2] << 6) & 0xFF,
                 (w[2] >> 2 | w[3] << 1 | w[4] << 4 | w[5] << 7) & 0xFF,
                 (w[5] >> 1 | w[6] << 2 | w[7] << 5) & 0xFF]
    np.testing.assert_array_equal(O.pack_bits(v.astype(np.uint8), 3), np.array(want, np.uint8))


def test_pack_five_bit_contribution_table():
    """The page's 5-bit packer: for each output byte, every lane whose 5-bit
    range overlaps the byte contributes (lane >> laneBitLo) & mask(width) at
    outBitLo. Rebuilt here from that description."""
    table = []
    for byte in range(5):
        lo, hi = byte * 8, byte * 8 + 8
        row = []
        for lane in range(8):
            a, b = lane * 5, lane * 5 + 5
            ov_lo, ov_hi = max(a, lo), min(b, hi)
            if ov_lo < ov_hi:
                row.append((lane, ov_lo - a, ov_hi - ov_lo, ov_lo - lo))
        table.append(row)
    rng = np.random.default_rng(5)
    v = rng.integers(0, 32, 8 * 32).astype(np.int64)
    want = []
    for i in range(0, v.size, 8):
        w = v[i:i + 8]
        for row in table:
            byte = 0
            for lane, lbl, width, obl in row:
                byte |= ((w[lane] >> lbl) & ((1 << width) - 1)) << obl
            want.append(byte)
    np.testing.assert_array_equal(O.pack_bits(v.astype(np.uint8), 5), np.array(want, np.uint8))


@pytest.mark.parametrize("bits", [2, 3, 4, 5, 8])
def test_unpack_inverts_pack(bits):
    rng = np.random.default_rng(bits)
    v = rng.integers(0, 2 ** bits, 512).astype(np.uint8)
    p = O.pack_bits(v, bits)
    assert p.size == 512 * bits // 8
    np.testing.assert_array_equal(O.unpack_bits(p, 512, bits), v)
    if bits == 8:
        np.testing.assert_array_equal(p, v)


# ----------------------------------------------------------------- key path

def golden_constant_block():
    out = {}
    for ln in open(os.path.join(GOLDEN, "constant_block.txt")):
        if ln.startswith("#") or not ln.strip():
            continue
        k, v = ln.split()
        out[k] = v
    return out


@pytest.mark.parametrize("bits,signed", [(8, True), (8, False), (4, False), (2, False)])
def test_constant_block_zero_point_overflows_fp16(bits, signed):
    g = golden_constant_block()
    x = np.full(128, float(g["block_value"]), np.float32)
    q, sc, zp = O.key_encode_row(x, bits, signed)
    assert (sc == int(g["scale_f16_bits"], 16)).all()
    assert (zp == int(g["zero_f16_bits"], 16)).all()
    assert (q == 0).all()
    out = O.key_decode_row(q, sc, zp, signed)
    assert np.isnan(out).all()          # (0 + inf) * 0
    # the binary32 zero point is "about 5e7": 0.5 / (0 + binary32(1e-8))
    assert abs(np.float32(0.5) / np.float32(1e-8) / float(g["zero_point_f32_order"]) - 1) < 1e-6


def test_zero_block_keys():
    q, sc, zp = O.key_encode_row(np.zeros(64, np.float32), 4, False)
    assert (q == 0).all() and (sc == 0).all() and (zp == 0).all()
    np.testing.assert_array_equal(O.key_decode_row(q, sc, zp, False), np.zeros(64, np.float32))


def test_key_ramps_with_exact_scale():
    """Blocks whose range equals max_val give scale 1 (and scale + 1e-8 rounds
    to 1 in binary32), so the codes are the values minus the zero point."""
    rng = np.random.default_rng(6)
    # unsigned 4-bit: integer values spanning exactly 0..15 (+ an offset)
    base = np.concatenate([rng.permutation(np.arange(16)), rng.integers(0, 16, 16)]).astype(np.float32)
    for off in (0.0, 100.0, -37.0):
        x = np.tile(base + off, 2)
        q, sc, zp = O.key_encode_row(x, 4, False)
        assert (O.f16_bits_to_f32(sc) == 1.0).all()
        assert (O.f16_bits_to_f32(zp) == off).all()
        np.testing.assert_array_equal(q, (x - off).astype(np.uint8))
        np.testing.assert_array_equal(O.key_decode_row(q, sc, zp, False), x)
    # signed 8-bit: integer values spanning exactly -127..127 -> zero point 0
    v = np.concatenate([[-127, 127], rng.integers(-127, 128, 30)]).astype(np.float32)
    x = np.tile(v, 4)
    q, sc, zp = O.key_encode_row(x, 8, True)
    assert (O.f16_bits_to_f32(sc) == 1.0).all() and (O.f16_bits_to_f32(zp) == 0.0).all()
    np.testing.assert_array_equal(q.view(np.int8), x.astype(np.int8))
    np.testing.assert_array_equal(O.key_decode_row(q, sc, zp, True), x)


@pytest.mark.parametrize("bits,signed", [(2, False), (3, False), (4, False), (5, False), (8, False), (8, True)])
def test_key_roundtrip_error_bound(bits, signed):
    """Affine quantisation error is at most half a step plus the fp16
    rounding of scale and zero point (zero points stay small here)."""
    rng = np.random.default_rng(7 + bits)
    x = rng.standard_normal((50, 128)).astype(np.float32)
    for row in x:
        q, sc, zp = O.key_encode_row(row, bits, signed)
        out = O.key_decode_row(q, sc, zp, signed)
        s = np.repeat(O.f16_bits_to_f32(sc), 32).astype(np.float64)
        z = np.repeat(O.f16_bits_to_f32(zp), 32).astype(np.float64)
        assert np.all(np.abs(z) <= 2048)
        qv = q.view(np.int8) if signed else q
        lo, hi = ((-127, 127) if signed else (0, 2 ** bits - 1))
        assert qv.min() >= lo and qv.max() <= hi
        err = np.abs(out.astype(np.float64) - row)
        assert np.all(err <= 0.5 * s * 1.01 + 2e-3 * (np.abs(z) + 2 ** bits) * s + 1e-6)


# --------------------------------------------------------------- value path

@pytest.mark.parametrize("bits,expect", [(2, 2), (3, 3), (4, 8), (5, 16), (8, 130)])
def test_zero_value_row(bits, expect):
    idx, sc, z = O.value_encode_row(np.zeros(128, np.float32), bits)
    assert (idx == expect).all() and (sc == 0).all()
    _, bd = O.lloyd_max(bits)
    assert expect == int((bd < 0).sum())
    out = O.value_decode_row(idx, sc, bits)
    assert (out == 0).all()


@pytest.mark.parametrize("bits", [2, 3, 4, 5, 8])
def test_value_encode_is_invariant_to_power_of_two_scaling(bits):
    rng = np.random.default_rng(20 + bits)
    x = rng.standard_normal(256).astype(np.float32)
    i1, s1, _ = O.value_encode_row(x, bits)
    i2, s2, _ = O.value_encode_row(x * np.float32(4.0), bits)
    np.testing.assert_array_equal(i1, i2)
    np.testing.assert_array_equal(O.f16_bits_to_f32(s2), O.f16_bits_to_f32(s1) * 4)


@pytest.mark.parametrize("d", [64, 128, 256, 512])
def test_value_decode_of_a_constant_code(d):
    """All codes equal and scale 1: the rotated vector is constant, so the
    inverse transform is c * d * (1/sqrt d) at position 0 and exactly 0
    elsewhere, and the sign is applied after the transform."""
    bits = 4
    c, _ = O.lloyd_max(bits)
    k = 11
    idx = np.full(d, k, np.uint8)
    one = np.full(d // 32, 0x3C00, np.uint16)          # fp16 1.0
    out = O.value_decode_row(idx, one, bits)
    want = np.zeros(d, np.float32)
    want[0] = O.signs(d)[0] * (np.float32(c[k] * d) * O.hadamard_scale(d))
    np.testing.assert_array_equal(out, want)
    np.testing.assert_array_equal(O.value_decode_row(idx, one, bits, rotated=True), np.full(d, c[k], np.float32))


def test_value_encode_rms_normalisation():
    """z is the rotated value divided by (RMS of its 32-group + 1e-8): each
    group of z has RMS close to 1, and the fp16 scale is that RMS."""
    rng = np.random.default_rng(8)
    x = (rng.standard_normal(128) * 3).astype(np.float32)
    idx, sc, z = O.value_encode_row(x, 4)
    y = O.fwht(x, True).astype(np.float64).reshape(4, 32)
    rms = np.sqrt((y ** 2).mean(axis=1))
    np.testing.assert_allclose(O.f16_bits_to_f32(sc), rms, rtol=1e-3)
    np.testing.assert_allclose(np.sqrt((z.astype(np.float64).reshape(4, 32) ** 2).mean(axis=1)), 1.0, rtol=1e-6)
    np.testing.assert_array_equal(idx, O.bin_index(z, 4))


@pytest.mark.parametrize("bits,band", [(2, (0.80, 1.02)), (3, (0.80, 1.02)), (4, (0.80, 1.05)),
                                       (5, (0.80, 1.05)), (8, (0.5, 1.5))])
def test_value_roundtrip_distortion_matches_table_distortion(bits, band):
    """Round-trip relative MSE on Gaussian rows against the table's own
    distortion E[(X - Q(X))^2] for X ~ N(0,1), integrated numerically."""
    from scipy import integrate
    from scipy.stats import norm
    c, bd = O.lloyd_max(bits)
    e = np.concatenate([[-np.inf], bd.astype(np.float64), [np.inf]])
    D = sum(integrate.quad(lambda t, ci=float(ci): (t - ci) ** 2 * norm.pdf(t), a, b)[0]
            for ci, a, b in zip(c, e[:-1], e[1:]))
    rng = np.random.default_rng(30 + bits)
    x = rng.standard_normal((64, 128)).astype(np.float32)
    err = 0.0
    for row in x:
        idx, sc, _ = O.value_encode_row(row, bits)
        out = O.value_decode_row(idx, sc, bits)
        err += np.sum((out.astype(np.float64) - row) ** 2)
    rel = err / np.sum(x.astype(np.float64) ** 2)
    assert band[0] * D <= rel <= band[1] * D, (rel, D)


# -------------------------------------------------------- whole-tensor API

def test_encode_decode_kv_tiny_workload_shapes_and_constant_row():
    rng = np.random.default_rng(0)
    k = rng.standard_normal((256, 1, 128), dtype=np.float32)
    v = rng.standard_normal((256, 1, 128), dtype=np.float32)
    k[7, 0, :] = 0.5
    p = O.encode_kv(k, v, head_dim=128, k_bits=8, v_bits=3, k_signed=True)
    assert p["k_codes"].shape == (256, 128) and p["v_codes"].shape == (256, 48)
    assert p["k_scale"].shape == (256, 4) and p["v_scale"].shape == (256, 4)
    assert (p["k_zero"][7] == 0x7C00).all()
    ko, vo = O.decode_kv(p, rows=256, head_dim=128, k_bits=8, v_bits=3, k_signed=True, out_dtype="f32")
    assert np.isnan(ko[7]).all() and not np.isnan(np.delete(ko, 7, axis=0)).any()
    # the whole-tensor path is the row path applied to each row
    for r in (0, 7, 255):
        q, sc, zp = O.key_encode_row(k[r, 0], 8, True)
        np.testing.assert_array_equal(p["k_codes"][r], q)
        idx, vs, _ = O.value_encode_row(v[r, 0], 3)
        np.testing.assert_array_equal(p["v_codes"][r], O.pack_bits(idx, 3))
    # bf16 output is the RNE rounding of the binary32 output
    kb, vb = O.decode_kv(p, rows=256, head_dim=128, k_bits=8, v_bits=3, k_signed=True, out_dtype="bf16")
    np.testing.assert_array_equal(vb.ravel(), O.f32_to_bf16_bits(vo.ravel()))


def test_bf16_input_is_upcast_exactly():
    rng = np.random.default_rng(9)
    x = rng.standard_normal((4, 128)).astype(np.float32)
    xb = O.f32_to_bf16_bits(x).reshape(4, 128)
    xf = (xb.astype(np.uint32) << 16).view(np.float32)
    a = O.encode_kv(xb, xb, head_dim=128, k_bits=4, v_bits=4)
    b = O.encode_kv(xf, xf, head_dim=128, k_bits=4, v_bits=4)
    for n in a:
        np.testing.assert_array_equal(a[n], b[n])


def test_unrotate_is_the_decode_rotation():
    rng = np.random.default_rng(11)
    x = rng.standard_normal((3, 256)).astype(np.float32)
    out = O.unrotate(x, 256)
    for r in range(3):
        np.testing.assert_array_equal(out[r], O.fwht(x[r], False))


def test_key_rounding_ties_go_to_even():
    """ops.round rounds half to even: with scale exactly 1, codes of x.5
    values land on the even neighbour (2.5 -> 2, 3.5 -> 4)."""
    x = np.concatenate([[0.0, 15.0], np.full(15, 2.5), np.full(15, 3.5)]).astype(np.float32)
    q, sc, zp = O.key_encode_row(x, 4, False)
    assert O.f16_bits_to_f32(sc)[0] == 1.0 and O.f16_bits_to_f32(zp)[0] == 0.0
    assert q[2:17].tolist() == [2] * 15 and q[17:].tolist() == [4] * 15
