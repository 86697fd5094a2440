"""Pins for oracle.quant (CPU only): the quantiser, the byte layouts, dequantisation."""
import json
import os

import numpy as np
import pytest

from oracle import quant

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_q4_word_layout_golden():
    g = json.load(open(os.path.join(GOLDEN, "q4_word_layout.json")))
    for c in g["cases"]:
        # the codes go to row 0, inputs 0..7: word 0 of the tiled array
        q = np.zeros((64, 64), dtype=np.uint8)
        q[0, :8] = c["codes"]
        words = quant.pack_q4(q)
        assert int(words[0]) == int(c["word"], 16), c
        assert (words[1:] == 0).all()
        assert (quant.unpack_q4(words, 64, 64) == q).all()
    for t in g["tiled_positions"]:
        q = np.zeros((t["rows"], t["cols"]), dtype=np.uint8)
        q[t["row"], t["col"]] = 0xB
        words = quant.pack_q4(q)
        nz = np.nonzero(words)[0]
        assert list(nz) == [t["word"]], t
        assert int(words[t["word"]]) == 0xB << t["shift"], t


def test_q4_pack_unpack_roundtrip():
    rng = np.random.default_rng(5)
    q = rng.integers(0, 16, size=(128, 192), dtype=np.uint8)
    assert (quant.unpack_q4(quant.pack_q4(q), 128, 192) == q).all()


def test_scale_bias_layouts():
    # q4: pairs in (block of 64 rows, group, row-in-strip, strip) order; q8: row-major pairs
    rows, cols = 128, 128
    s = (np.arange(rows * 2).reshape(rows, 2) + 1).astype(np.float16)
    b = -s
    sb4 = quant.pack_scale_bias(s, b, "q4")
    # row 77 = 64*1 + 16*0 + 13 (block 1, strip 0, n 13), group 1:
    # pair index ((1*2+1)*16+13)*4+0 = 244
    assert sb4[2 * 244] == s[77, 1].view(np.uint16) and sb4[2 * 244 + 1] == b[77, 1].view(np.uint16)
    # row 35 = 16*2 + 3 (block 0, strip 2, n 3), group 0: pair index (0*16+3)*4+2 = 14
    assert sb4[2 * 14] == s[35, 0].view(np.uint16) and sb4[2 * 14 + 1] == b[35, 0].view(np.uint16)
    sb8 = quant.pack_scale_bias(s, b, "q8")
    assert sb8[2 * (77 * 2 + 1)] == s[77, 1].view(np.uint16)
    for fmt, sb in (("q4", sb4), ("q8", sb8)):
        s2, b2 = quant.unpack_scale_bias(sb, rows, cols, fmt)
        assert (s2 == s).all() and (b2 == b).all()


def test_worked_example_linear_ramp():
    # Row w_i = -1 + i/32, i = 0..63 (all exact in float32).
    # min = -1, max = 63/32; (max-min)/15 = 63/480 = 0.13125 -> fp16: 0.13125 = 1.05 * 2^-3,
    # mantissa 0.05*1024 = 51.2 -> 51, so scale = 1075/8192 (bits 0x3033); bias = -1 (0xBC00).
    # Code i = rint((i/32) / (1075/8192)) = rint(256 i / 1075); 512 i - 1075 (2n+1) is odd, so
    # no quotient is within 1/2150 of a tie and float32 rounding cannot move it:
    # q_i = floor((512 i + 1075) / 2150) in integer arithmetic.
    i = np.arange(64)
    w = (-1.0 + i / 32.0).astype(np.float32)[None, :]
    q, s, b = quant.quantize_affine(w, 4)
    assert s.view(np.uint16)[0, 0] == 0x3033
    assert b.view(np.uint16)[0, 0] == 0xBC00
    expect = np.array([(512 * int(k) + 1075) // 2150 for k in i], dtype=np.uint8)
    assert (q[0] == expect).all()
    assert q[0, 0] == 0 and q[0, 63] == 15


@pytest.mark.parametrize("bits,group", [(4, 64), (8, 64), (6, 32)])
def test_grid_values_roundtrip_exactly(bits, group):
    # Groups whose values lie exactly on a grid b + s*q that hits both 0 and qmax:
    # s = m * 2^-14 (m in [1024, 2047]), b = n * 2^-10 (|n| < 1024) are fp16-exact and every
    # b + s*q is an integer times 2^-14 below 2^17 in magnitude, so exact in float32.
    rng = np.random.default_rng(7)
    qmax = 2 ** bits - 1
    rows, groups = 16, 5
    m = rng.integers(1024, 2048, size=(rows, groups))
    n = rng.integers(-1023, 1024, size=(rows, groups))
    q = rng.integers(0, qmax + 1, size=(rows, groups, group))
    q[:, :, 0] = 0
    q[:, :, 1] = qmax
    w = (m[:, :, None] * q * 2.0 ** -14 + n[:, :, None] * 2.0 ** -10)
    w32 = w.astype(np.float32)
    assert (w32.astype(np.float64) == w).all()
    qq, s, b = quant.quantize_affine(w32.reshape(rows, groups * group), bits, group)
    assert (s.astype(np.float64) == m * 2.0 ** -14).all()
    assert (b.astype(np.float64) == n * 2.0 ** -10).all()
    assert (qq.reshape(rows, groups, group) == q).all()
    assert (quant.dequantize(qq, s, b) == w.reshape(rows, -1)).all()


@pytest.mark.parametrize("bits,group", [(4, 64), (8, 64), (6, 32)])
def test_codes_are_nearest_grid_points(bits, group):
    # Brute force: each code must be (one of) the nearest of all 2^bits grid points
    # b + s*q, up to float32 rounding of the quotient (slack 1e-4 * s).
    rng = np.random.default_rng(11)
    w = (rng.standard_normal((24, 256)) * 0.05).astype(np.float32)
    q, s, b = quant.quantize_affine(w, bits, group)
    sv = np.repeat(s.astype(np.float64), group, axis=1)
    bv = np.repeat(b.astype(np.float64), group, axis=1)
    cand = np.arange(2 ** bits, dtype=np.float64)
    dist = np.abs(bv[..., None] + sv[..., None] * cand - w.astype(np.float64)[..., None])
    best = dist.min(axis=-1)
    got = np.take_along_axis(dist, q[..., None].astype(np.int64), axis=-1)[..., 0]
    assert (got <= best + 1e-4 * sv).all()
    assert q.max() <= 2 ** bits - 1


def test_constant_group_has_zero_scale():
    w = np.full((2, 128), 0.3, dtype=np.float32)
    w[1, 64:] = -2.5
    q, s, b = quant.quantize_affine(w, 4)
    assert (s == 0).all()
    assert (q == 0).all()
    v = quant.dequantize(q, s, b)
    assert (v[0] == np.float64(np.float16(0.3))).all()
    assert (v[1, 64:] == -2.5).all()


def test_q8_layout_is_bytes_in_order():
    rng = np.random.default_rng(3)
    w = rng.standard_normal((5, 128)).astype(np.float32)
    codes, sb = quant.pack(w, "q8")
    q, _, _ = quant.quantize_affine(w, 8)
    assert codes.dtype == np.uint8 and codes.shape == (5, 128)
    assert (codes == q).all()
    assert (quant.codes_of(codes, "q8", 5, 128) == q).all()


@pytest.mark.parametrize("fmt", ["q4", "q8", "q6"])
def test_dequantize_matches_grouped_quantised_product(fmt):
    # "dequantise-then-dense equals the quantised reference": v @ W_deq^T against the
    # per-group factored sum s_g * sum(v q) + b_g * sum(v), which never forms W_deq.
    rng = np.random.default_rng(13)
    w = (rng.standard_normal((64, 320)) * 0.04).astype(np.float32)
    codes, sb = quant.pack(w, fmt)
    q = quant.codes_of(codes, fmt, 64, 320)
    s, b = quant.unpack_scale_bias(sb, 64, 320, fmt)
    v = rng.standard_normal((7, 320))
    dense = v @ quant.unpack(codes, sb, fmt, 64, 320).T
    fact = quant.qlinear_grouped(v, q, s, b)
    assert np.allclose(dense, fact, rtol=1e-12, atol=1e-12)
    # a wrong group pairing must be visible to this check
    s_bad = np.roll(s, 1, axis=1)
    assert not np.allclose(dense, quant.qlinear_grouped(v, q, s_bad, b), rtol=1e-6, atol=1e-6)


def test_quantisation_error_bound():
    # |w - w_deq| <= s/2 (+ rounding slack) wherever w lies inside [min, max] of its group.
    rng = np.random.default_rng(17)
    w = (rng.standard_normal((64, 512)) * 0.02).astype(np.float32)
    for fmt in ("q4", "q8"):
        codes, sb = quant.pack(w, fmt)
        s, b = quant.unpack_scale_bias(sb, 64, 512, fmt)
        v = quant.unpack(codes, sb, fmt, 64, 512)
        sv = np.repeat(s.astype(np.float64), 64, axis=1)
        bv = np.repeat(b.astype(np.float64), 64, axis=1)
        top = bv + sv * (15 if fmt == "q4" else 255)
        inside = (w >= bv) & (w <= top)
        err = np.abs(v - w)
        assert (err[inside] <= 0.5 * sv[inside] * (1 + 1e-4) + 1e-9).all()
        # fp16 rounding of scale and bias moves the ends by at most ~2^-11 relative
        assert (err <= 0.5 * sv + 2.0 ** -10 * (np.abs(w) + sv * 16) + 1e-7).all()


# ------------------------------------------------------------------ q4 group 32
def test_q4g32_scale_bias_layout_worked_by_hand():
    # rows 128, cols 128: G = 2 groups of 64, four 32-input halves per row.
    # Pair of row r = 64b + 16s + n, inputs 64q + 32h..: uint16 index
    # ((((b*G + q)*16 + n)*4 + s)*2 + h)*2 + {0, 1}, worked out by hand below.
    rows, cols = 128, 128
    s = (np.arange(rows * 4).reshape(rows, 4) + 1).astype(np.float16)  # [rows, 32-groups]
    b = -s
    sb = quant.pack_scale_bias(s, b, "q4g32")
    cases = [
        # (row, 32-group, pair index)
        (0, 0, 0),
        (0, 1, 1),        # h = 1 of group q = 0
        (16, 0, 2),       # strip 1: s*2 = 2
        (1, 0, 8),        # n = 1: 1*4*2
        (17, 3, 139),     # b 0, s 1, n 1, q 1, h 1: ((0*2+1)*16+1)*8 + 2 + 1
        (70, 2, 432),     # b 1, s 0, n 6, q 1, h 0: ((1*2+1)*16+6)*8
        (127, 3, 511),    # the last pair: b 1, s 3, n 15, q 1, h 1
    ]
    for r, g32, idx in cases:
        assert sb[2 * idx] == s[r, g32].view(np.uint16), (r, g32, idx)
        assert sb[2 * idx + 1] == b[r, g32].view(np.uint16), (r, g32, idx)
    s2, b2 = quant.unpack_scale_bias(sb, rows, cols, "q4g32")
    assert (s2 == s).all() and (b2 == b).all()


def test_q4g32_groups_are_32_inputs():
    # two halves of each 64-input group with very different ranges get their own
    # scales: the narrow half is quantised to its own fine grid (grid values of
    # each 32-group round-trip exactly, as for group 64)
    rng = np.random.default_rng(23)
    rows = 8
    m = rng.integers(1024, 2048, size=(rows, 4))
    n = rng.integers(-1023, 1024, size=(rows, 4))
    q = rng.integers(0, 16, size=(rows, 4, 32))
    q[:, :, 0] = 0
    q[:, :, 1] = 15
    m[:, 1] = 1024          # the second half of group 0: a scale 8x finer than the first's max
    m[:, 0] = 2047
    w = (m[:, :, None] * q * 2.0 ** -14 + n[:, :, None] * 2.0 ** -10)
    w32 = w.astype(np.float32)
    assert (w32.astype(np.float64) == w).all()
    qq, s, b = quant.quantize_affine(w32.reshape(rows, 128), 4, 32)
    assert s.shape == (rows, 4)
    assert (s.astype(np.float64) == m * 2.0 ** -14).all()
    assert (b.astype(np.float64) == n * 2.0 ** -10).all()
    assert (qq.reshape(rows, 4, 32) == q).all()
    # the packed matrix (64 rows: eight copies of the 8 rows) carries the same
    # per-32 scales and codes
    w64 = np.tile(w32.reshape(rows, 128), (8, 1))
    codes, sb = quant.pack(w64, "q4g32")
    s64p, b64p = quant.unpack_scale_bias(sb, 64, 128, "q4g32")
    assert (s64p == np.tile(s, (8, 1))).all() and (b64p == np.tile(b, (8, 1))).all()
    assert (quant.codes_of(codes, "q4g32", 64, 128) == np.tile(qq, (8, 1))).all()
    # with group 64 the same data needs the coarser scale of the wider range
    _, s64, _ = quant.quantize_affine(w32.reshape(rows, 128), 4, 64)
    assert (s64.astype(np.float64) >= np.maximum(s[:, 0::2], s[:, 1::2]).astype(np.float64)).all()


def test_q4g32_codes_nearest_and_error_bound():
    rng = np.random.default_rng(29)
    w = (rng.standard_normal((64, 256)) * 0.05).astype(np.float32)
    codes, sb = quant.pack(w, "q4g32")
    q = quant.codes_of(codes, "q4g32", 64, 256)
    s, b = quant.unpack_scale_bias(sb, 64, 256, "q4g32")
    assert s.shape == (64, 8)
    sv = np.repeat(s.astype(np.float64), 32, axis=1)
    bv = np.repeat(b.astype(np.float64), 32, axis=1)
    cand = np.arange(16, dtype=np.float64)
    dist = np.abs(bv[..., None] + sv[..., None] * cand - w.astype(np.float64)[..., None])
    got = np.take_along_axis(dist, q[..., None].astype(np.int64), axis=-1)[..., 0]
    assert (got <= dist.min(axis=-1) + 1e-4 * sv).all()
    v = quant.unpack(codes, sb, "q4g32", 64, 256)
    assert (np.abs(v - w) <= 0.5 * sv * (1 + 1e-3) + 1e-7).all()
    # the codes use the same nibble layout as Q4G64
    assert (quant.unpack_q4(codes, 64, 256) == q).all()


def test_q4g32_dequantize_matches_grouped_product():
    rng = np.random.default_rng(31)
    w = (rng.standard_normal((64, 320)) * 0.04).astype(np.float32)
    codes, sb = quant.pack(w, "q4g32")
    q = quant.codes_of(codes, "q4g32", 64, 320)
    s, b = quant.unpack_scale_bias(sb, 64, 320, "q4g32")
    v = rng.standard_normal((5, 320))
    dense = v @ quant.unpack(codes, sb, "q4g32", 64, 320).T
    assert np.allclose(dense, quant.qlinear_grouped(v, q, s, b), rtol=1e-12, atol=1e-12)
    # swapping the two halves' pairs of every group must be visible
    s_bad = s.reshape(64, -1, 2)[:, :, ::-1].reshape(64, -1)
    assert not np.allclose(dense, quant.qlinear_grouped(v, q, s_bad, b), rtol=1e-6, atol=1e-6)


# ------------------------------------------------------------------ q6 group 32
def test_q6_planes_worked_by_hand():
    # rows 64, cols 128 (G = 2).  Row 37 = 16*2 + 5 (b 0, s 2, n 5); input
    # 125 = 64*1 + 32*1 + 8*3 + 5 (q 1, h 1, g 3, j 5 = 2p + t: p 2, t 1).
    # Low plane: word ((((0*2 + 1)*4 + 3)*16 + 5)*8 + 2*2 + 1 = 117*8 + 5 = 941,
    # bits 4p + 16t = 24.  High plane: word (((0*2 + 1)*4 + 3)*16 + 5)*4 + 2 =
    # 117*4 + 2 = 470, bits 2(4h + p) + 16t = 12 + 16 = 28.
    q = np.zeros((64, 128), np.uint8)
    q[37, 125] = 45                      # 0b10_1101: low 13, high 2
    lo = quant.pack_q4(q & 15)
    hi = quant.pack_q6_high(q)
    assert lo.size == 64 * 128 // 8 and hi.size == 64 * 128 // 16
    assert list(np.nonzero(lo)[0]) == [941] and lo[941] == 13 << 24
    assert list(np.nonzero(hi)[0]) == [470] and hi[470] == 2 << 28
    rng = np.random.default_rng(9)
    q = rng.integers(0, 64, size=(128, 192)).astype(np.uint8)
    words = np.concatenate([quant.pack_q4(q & 15), quant.pack_q6_high(q)])
    assert np.array_equal(quant.codes_of(words, "q6", 128, 192), q)


def test_q6_pack_uses_q4g32_pairs_and_six_bit_codes():
    rng = np.random.default_rng(10)
    w = (rng.standard_normal((64, 256)) * 0.05).astype(np.float32)
    codes, sb = quant.pack(w, "q6")
    q, s, b = quant.quantize_affine(w, 6, 32)
    assert codes.dtype == np.uint32 and codes.size == 64 * 256 * 6 // 32
    assert q.max() == 63 and np.array_equal(quant.codes_of(codes, "q6", 64, 256), q)
    assert np.array_equal(sb, quant.pack_scale_bias(s, b, "q4g32"))
    v = quant.unpack(codes, sb, "q6", 64, 256)
    sv = np.repeat(s.astype(np.float64), 32, axis=1)
    assert (np.abs(v - w) <= 0.5 * sv * (1 + 1e-3) + 1e-7).all()
    # finer than q4 group 32 on the same data
    c4, sb4 = quant.pack(w, "q4g32")
    e4 = np.abs(quant.unpack(c4, sb4, "q4g32", 64, 256) - w).mean()
    assert np.abs(v - w).mean() < e4 / 3
