"""Pins for oracle.fp4 (CPU only): the E2M1 and E4M3 codecs, the nvfp4
quantiser, its byte layout and exact dequantisation."""
import numpy as np
import pytest

from oracle import fp4, quant


# ------------------------------------------------------------------ E2M1
def test_e2m1_table_is_the_format():
    # sign | exponent (2 bits, bias 1) | mantissa (1 bit); exponent 0 is the
    # subnormal 0.m: the sixteen values of the format, written out
    want = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0,
            -0.0, -0.5, -1.0, -1.5, -2.0, -3.0, -4.0, -6.0]
    got = fp4.e2m1_decode(np.arange(16))
    assert list(got) == want
    assert list(np.signbit(got)) == [False] * 8 + [True] * 8


def test_e2m1_encode_grid_ties_and_saturation():
    grid = fp4.e2m1_decode(np.arange(8))
    assert list(fp4.e2m1_encode(grid.astype(np.float32))) == list(range(8))
    assert list(fp4.e2m1_encode(-grid.astype(np.float32))) == list(range(8, 16))
    # midpoints go to the even code (the one whose mantissa bit is 0)
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0], np.float32)
    assert list(fp4.e2m1_encode(mids)) == [0, 2, 2, 4, 4, 6, 6]
    # above the largest magnitude: 6
    assert list(fp4.e2m1_encode(np.array([6.5, 7.0, 1e30, np.inf], np.float32))) == [7, 7, 7, 7]


def test_e2m1_encode_is_nearest_by_brute_force():
    rng = np.random.default_rng(3)
    x = (rng.standard_normal(20000) * 3).astype(np.float32)
    code = fp4.e2m1_encode(x)
    grid = fp4.e2m1_decode(np.arange(16))
    d = np.abs(x.astype(np.float64)[:, None] - grid[None, :])
    best = d.min(axis=1)
    got = np.abs(x.astype(np.float64) - fp4.e2m1_decode(code))
    assert np.array_equal(got, best)
    assert np.array_equal(np.signbit(fp4.e2m1_decode(code)), np.signbit(x))


# ------------------------------------------------------------------ E4M3
def test_e4m3_known_values():
    # values of the E4M3 (fn) format: bias 7, 3 mantissa bits, subnormals m*2^-9, max 448
    known = {0x00: 0.0, 0x01: 2.0 ** -9, 0x07: 7 * 2.0 ** -9, 0x08: 2.0 ** -6, 0x30: 0.5,
             0x38: 1.0, 0x3F: 1.875, 0x40: 2.0, 0x7E: 448.0, 0x78: 256.0, 0x77: 240.0}
    for c, v in known.items():
        assert fp4.e4m3_decode(c) == v, hex(c)
    assert np.isnan(fp4.e4m3_decode(0x7F))


def test_e4m3_encode_roundtrip_ties_saturation():
    codes = np.arange(0x7F)
    vals = fp4.e4m3_decode(codes)
    assert np.all(np.diff(vals) > 0)                     # positive codes are ordered
    assert np.array_equal(fp4.e4m3_encode(vals.astype(np.float32)), codes)
    # midpoints between neighbours go to the even code
    mid = ((vals[:-1] + vals[1:]) / 2).astype(np.float32)
    assert np.all(mid.astype(np.float64) == (vals[:-1] + vals[1:]) / 2)  # exact in float32
    enc = fp4.e4m3_encode(mid).astype(np.int64)
    lo = codes[:-1]
    assert np.array_equal(enc, np.where(lo % 2 == 0, lo, lo + 1))
    assert list(fp4.e4m3_encode(np.array([449.0, 470.0, 1e6, np.inf], np.float32))) == [0x7E] * 4
    # nearest by brute force on random scales
    rng = np.random.default_rng(4)
    t = np.exp(rng.uniform(np.log(1e-4), np.log(500), 5000)).astype(np.float32)
    enc = fp4.e4m3_encode(t)
    d = np.abs(t.astype(np.float64)[:, None] - vals[None, :])
    assert np.array_equal(np.abs(t - fp4.e4m3_decode(enc)), d.min(axis=1))


# ------------------------------------------------------------------ quantiser
def _grid_matrix(rows, cols, seed):
    """Values e2m1 * e4m3 * 2^-12 with one +-6 code per block and the matrix
    maximum 6 * 448 * 2^-12, so the quantiser must return exactly these codes,
    bytes and gs = 2^-12."""
    rng = np.random.default_rng(seed)
    codes = rng.integers(0, 16, size=(rows, cols)).astype(np.uint8)
    sbyte = rng.integers(0x08, 0x7F, size=(rows, cols // 16)).astype(np.uint8)  # normal scales
    codes.reshape(rows, cols // 16, 16)[:, :, 3] = np.where(rng.random((rows, cols // 16)) < 0.5, 7, 15)
    sbyte[0, 0] = 0x7E
    w = fp4.dequantize_nvfp4(codes, sbyte, 2.0 ** -12)
    assert np.all(w.astype(np.float32).astype(np.float64) == w)
    return w.astype(np.float32), codes, sbyte


def test_quantiser_recovers_grid_values_exactly():
    w, codes, sbyte = _grid_matrix(64, 128, 5)
    q, sb, gs, amax = fp4.quantize_nvfp4(w)
    assert gs == np.float32(2.0 ** -12) and amax == np.float32(6 * 448 * 2.0 ** -12)
    assert np.array_equal(sb, sbyte)
    # the sign of a zero magnitude is the input's sign bit, as in the codes drawn
    assert np.array_equal(q, codes)
    assert np.array_equal(fp4.dequantize_nvfp4(q, sb, gs), w.astype(np.float64))


def test_quantiser_error_bound_and_zero_blocks():
    rng = np.random.default_rng(6)
    w = (rng.standard_normal((64, 256)) * 0.03).astype(np.float32)
    w[1, :16] = 0.0                           # a zero block: scale byte 0, codes 0
    w[2, 16:32] = -0.0                        # (negative zeros too: es == 0 gives code 0)
    w[3, 5] = -0.0                            # in a live block a negative zero keeps its sign
    w[3, 6] = -1e-9                           # and so does a tiny negative that rounds to 0
    q, sb, gs, amax = fp4.quantize_nvfp4(w)
    assert sb[1, 0] == 0 and np.all(q[1, :16] == 0)
    assert sb[2, 1] == 0 and np.all(q[2, 16:32] == 0)
    assert sb[3, 0] > 0 and q[3, 5] == 8 and q[3, 6] == 8
    deq = fp4.dequantize_nvfp4(q, sb, gs)
    blk = np.abs(w).reshape(64, 16, 16).max(axis=2).astype(np.float64)
    es = fp4.e4m3_decode(sb) * float(gs)
    normal = sb >= 0x08
    err = np.abs(deq - w).reshape(64, 16, 16).max(axis=2)
    # half the widest E2M1 step (1, between 4 and 6) times the block scale,
    # which is within 2^-4 of bmax/6 for a normal E4M3 byte
    assert np.all(err[normal] <= es[normal] * (1 + 1e-6))
    assert np.all(es[normal] <= blk[normal] / 6 * (1 + 2.0 ** -4) * (1 + 1e-6))
    # the largest block keeps its maximum on the grid's top (6 * es)
    i = np.unravel_index(np.argmax(blk), blk.shape)
    assert sb[i] == 0x7E


def test_all_zero_matrix():
    q, sb, gs, amax = fp4.quantize_nvfp4(np.zeros((64, 64), np.float32))
    assert gs == 0 and amax == 0 and not q.any() and not sb.any()


def test_dequantize_matches_blockwise_product():
    rng = np.random.default_rng(7)
    w = (rng.standard_normal((64, 192)) * 0.05).astype(np.float32)
    q, sb, gs, _ = fp4.quantize_nvfp4(w)
    v = rng.standard_normal((4, 192))
    dense = v @ fp4.dequantize_nvfp4(q, sb, gs).T
    assert np.allclose(dense, fp4.qlinear_blocks(v, q, sb, gs), rtol=1e-12, atol=1e-12)
    bad = sb.copy()
    bad[:, 0], bad[:, 1] = sb[:, 1], sb[:, 0]  # two blocks' scales swapped
    assert not np.allclose(dense, fp4.qlinear_blocks(v, q, bad, gs), rtol=1e-6, atol=1e-6)


# ------------------------------------------------------------------ layout
def test_scale_layout_worked_by_hand():
    rows, cols = 128, 128  # G = 2; eight 16-input blocks per row
    sbyte = np.zeros((rows, cols // 16), np.uint8)
    # row 81 = 64*1 + 16*1 + 1 (b 1, s 1, n 1); inputs 112..127: q 1, j 3
    # byte (((1*2 + 1)*16 + 1)*4 + 1)*4 + 3 = (49*4 + 1)*4 + 3 = 791
    sbyte[81, 7] = 0x3A
    # row 14 (b 0, s 0, n 14); inputs 16..31: q 0, j 1 -> byte ((0*16 + 14)*4 + 0)*4 + 1 = 225
    sbyte[14, 1] = 0x41
    buf = fp4.pack_scales(sbyte, np.float32(0.125), np.float32(336.0))
    assert buf.size == rows * cols // 16 + 64
    assert buf[791] == 0x3A and buf[225] == 0x41
    assert np.count_nonzero(buf[:rows * cols // 16]) == 2
    assert buf[1024:1028].view(np.float32)[0] == 0.125 and buf[1028:1032].view(np.float32)[0] == 336.0
    assert not buf[1032:].any()
    s2, gs = fp4.unpack_scales(buf, rows, cols)
    assert np.array_equal(s2, sbyte) and gs == np.float32(0.125)


def test_pack_unpack_roundtrip():
    rng = np.random.default_rng(8)
    w = (rng.standard_normal((128, 192)) * 0.02).astype(np.float32)
    words, sbuf = fp4.pack(w)
    q, sb, gs, _ = fp4.quantize_nvfp4(w)
    assert np.array_equal(quant.unpack_q4(words, 128, 192), q)
    assert np.array_equal(fp4.unpack(words, sbuf, 128, 192), fp4.dequantize_nvfp4(q, sb, gs))
