"""Oracle: the nvfp4 expert format -- E2M1 codes, E4M3 block scales, a tensor scale.

TEST INFRASTRUCTURE ONLY (see the package docstring).

What the pages fix: nvfp4 is one of the expert formats of the diffgemma pack
([ARCH] Part II section 8 "Quantization (.dgq)": the nvfp4 profile, and
section 8.2 "Custom quantization classes": experts take q4, q6 or nvfp4, and
nvfp4 needs K a multiple of 16); its decode sits beside the q4/q6/q8 decodes
of the GEMM family ([ARCH] section 10, the dgemm crate: "bf16/fp4 codecs").
The pages do not spell the format out; the reading taken here is NVIDIA's
published NVFP4:
  * elements: FP4 E2M1 -- a sign bit, two exponent bits (bias 1), one mantissa
    bit; magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6 for codes 0..7, bit 3 the sign;
  * one FP8 E4M3 scale per block of 16 consecutive inputs of a row -- a sign
    bit, four exponent bits (bias 7), three mantissa bits, largest finite
    value 448, subnormals m * 2^-9, no infinities (code 0x7F is NaN);
  * one float32 scale per tensor (per expert matrix of a stacked tensor);
  * value = e2m1(code) * e4m3(block scale) * tensor scale.

The quantiser (the pages give none; this is the plain amax reading, and each
step that decides a code or a scale byte is a float32 IEEE operation, which the
GPU packer performs in the same order, so the two agree bit for bit):
  amax = max |w| over the matrix;         gs = amax / 2688   (2688 = 6 * 448)
  per block of 16:  bmax = max |w|;       t = bmax / (6 * gs)   (float32; 0 if gs == 0)
                    scale byte = e4m3_encode(t)   (round to nearest even, values
                                                   above 448 saturate to 448)
                    es = e4m3(scale byte) * gs     (float32)
  per input:        code = e2m1_encode(w / es)     (float32 divide; round to the
                                                    nearest E2M1 value, ties to the
                                                    even code, |x| > 6 saturates;
                                                    the sign bit is w's sign bit);
                    code 0 (positive zero) where es == 0.
  w_deq = e2m1(code) * e4m3(byte) * gs, exact in float64.

Byte layout (a format of this project, declared in include/dgmoe.h as
DGMOE_NVFP4):
  codes: uint32 words exactly as Q4G64 (oracle.quant.pack_q4), the 4-bit
         code of input c of row r in the same word and bit position;
  scales (the matrix's `scale_bias` bytes): rows in blocks of 64, G = cols/64;
         the E4M3 byte of row r = 64 b + 16 s + n and inputs 64 q + 16 j .. +15
         (j < 4) at byte (((b*G + q)*16 + n)*4 + s)*4 + j, then a 64-byte
         trailer: the float32 tensor scale gs, the float32 amax, 56 zero bytes.
         Each expert of a stacked tensor has its own rows*cols/16 + 64 bytes.
"""
import numpy as np

from . import quant

# E2M1 magnitudes of codes 0..7 (the format's definition: 0 and 0.5 are the
# exponent-0 codes, then 1, 1.5, 2, 3, 4, 6 at exponents 1..3)
E2M1 = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
E4M3_MAX = 448.0
TRAILER = 64


def e2m1_decode(codes):
    """4-bit codes (bit 3 the sign) -> float64 values."""
    c = np.asarray(codes).astype(np.int64)
    v = E2M1[c & 7]
    return np.where(c & 8, -v, v)


def e2m1_encode(x):
    """float32 values -> 4-bit codes: nearest E2M1 magnitude, ties to the even
    code, |x| above 6 saturating to 6; the sign bit is x's sign bit."""
    x = np.asarray(x, np.float32)
    a = np.abs(x)
    # thresholds between codes i and i+1; at a tie the even code wins, so a
    # magnitude exactly on the threshold moves up only when i is odd
    thr = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0], np.float32)
    code = np.zeros(a.shape, np.int64)
    for i, t in enumerate(thr):
        code += (a >= t) if i % 2 else (a > t)
    return (code | np.where(np.signbit(x), 8, 0)).astype(np.uint8)


def e4m3_decode(codes):
    """E4M3 bytes (non-negative scales: the sign bit is 0) -> float64."""
    c = np.asarray(codes).astype(np.int64)
    e, m = (c >> 3) & 15, c & 7
    normal = np.ldexp(1.0 + m / 8.0, (e - 7).astype(np.int64))
    sub = m * 2.0 ** -9
    v = np.where(e == 0, sub, normal)
    v = np.where((c & 0x7F) == 0x7F, np.nan, v)
    return np.where(c & 0x80, -v, v)


def e4m3_encode(t):
    """float32 values t >= 0 -> E4M3 bytes: round to nearest even, values above
    448 (and +inf) saturate to 448 (0x7E)."""
    t = np.asarray(t, np.float32).astype(np.float64)  # exact
    t = np.minimum(t, 2 * E4M3_MAX)                   # saturated below; keeps inf out of the casts
    out = np.zeros(t.shape, np.int64)
    sub = t < 2.0 ** -6
    # subnormal range: steps of 2^-9; m = 8 is the smallest normal, code 0x08
    out = np.where(sub, np.rint(np.where(sub, t, 0.0) * 2.0 ** 9).astype(np.int64), out)
    mant, ex = np.frexp(np.where(sub, 1.0, t))        # t = mant * 2^ex, mant in [0.5, 1)
    e = ex - 1                                        # t = (2 mant) * 2^e
    m = np.rint((2.0 * mant - 1.0) * 8.0).astype(np.int64)  # exact scaling, then RNE
    e = np.where(m == 8, e + 1, e)
    m = np.where(m == 8, 0, m)
    normal = ((e + 7) << 3) | m
    out = np.where(sub, out, normal)
    out = np.where(t > E4M3_MAX, 0x7E, out)
    return np.clip(out, 0, 0x7E).astype(np.uint8)


def quantize_nvfp4(w):
    """float32 [rows, cols] -> (codes uint8 [rows, cols], scale bytes uint8
    [rows, cols/16], gs float32, amax float32), per the module docstring."""
    w = np.ascontiguousarray(w, np.float32)
    rows, cols = w.shape
    if cols % 16:
        raise ValueError("nvfp4 needs cols a multiple of 16")
    amax = np.float32(np.max(np.abs(w))) if w.size else np.float32(0)
    gs = np.float32(amax / np.float32(2688.0))
    blk = w.reshape(rows, cols // 16, 16)
    bmax = np.max(np.abs(blk), axis=2)
    if gs > 0:
        t = bmax / np.float32(np.float32(6.0) * gs)
    else:
        t = np.zeros_like(bmax)
    sbyte = e4m3_encode(t)
    es = (e4m3_decode(sbyte).astype(np.float32) * gs).astype(np.float32)  # float32 product
    with np.errstate(divide="ignore", invalid="ignore"):
        x = blk / es[:, :, None]
    codes = np.where(es[:, :, None] > 0, e2m1_encode(x), 0).astype(np.uint8)
    return codes.reshape(rows, cols), sbyte, gs, np.float32(amax)


def dequantize_nvfp4(codes, sbyte, gs):
    """Exact float64 values of a matrix: e2m1(code) * e4m3(byte) * gs."""
    codes = np.asarray(codes)
    rows, cols = codes.shape
    s = np.repeat(e4m3_decode(sbyte), 16, axis=1)
    return e2m1_decode(codes) * s * float(gs)


def pack_scales(sbyte, gs, amax):
    """E4M3 bytes [rows, cols/16] + tensor scale -> the tiled scale bytes and trailer."""
    sbyte = np.asarray(sbyte, np.uint8)
    rows, nb16 = sbyte.shape
    if rows % 64 or nb16 % 4:
        raise ValueError("nvfp4 tiles need rows % 64 == 0 and cols % 64 == 0")
    nb, G = rows // 64, nb16 // 4
    # (b, s, n, q, j) -> (b, q, n, s, j)
    body = sbyte.reshape(nb, 4, 16, G, 4).transpose(0, 3, 2, 1, 4).reshape(-1)
    trailer = np.zeros(TRAILER, np.uint8)
    trailer[0:4] = np.frombuffer(np.float32(gs).tobytes(), np.uint8)
    trailer[4:8] = np.frombuffer(np.float32(amax).tobytes(), np.uint8)
    return np.concatenate([body, trailer])


def unpack_scales(buf, rows, cols):
    """The tiled scale bytes of one matrix -> (E4M3 bytes [rows, cols/16], gs)."""
    buf = np.asarray(buf, np.uint8).reshape(-1)
    nb, G = rows // 64, cols // 64
    n = rows * cols // 16
    sbyte = buf[:n].reshape(nb, G, 16, 4, 4).transpose(0, 3, 2, 1, 4).reshape(rows, cols // 16)
    gs = np.frombuffer(buf[n:n + 4].tobytes(), np.float32)[0]
    return sbyte.copy(), gs


def pack(w):
    """Quantise and lay out one float32 matrix: (code words uint32, scale bytes uint8)."""
    codes, sbyte, gs, amax = quantize_nvfp4(w)
    return quant.pack_q4(codes), pack_scales(sbyte, gs, amax)


def unpack(words, sbuf, rows, cols):
    """Packed matrix -> float64 values (the value every consumer must use)."""
    codes = quant.unpack_q4(words, rows, cols)
    sbyte, gs = unpack_scales(sbuf, rows, cols)
    return dequantize_nvfp4(codes, sbyte, gs)


def qlinear_blocks(v, codes, sbyte, gs):
    """v [n, cols] times the matrix's transpose, factored per 16-input block:
    gs * sum_blocks e4m3(byte) * sum_{c in block} v_c * e2m1(code_c).  Used only
    to pin dequantize_nvfp4."""
    v = np.asarray(v, np.float64)
    rows, cols = np.asarray(codes).shape
    vb = v.reshape(v.shape[0], cols // 16, 16)
    eb = e2m1_decode(codes).reshape(rows, cols // 16, 16)
    part = np.einsum("nbc,rbc->nrb", vb, eb)
    return float(gs) * np.einsum("nrb,rb->nr", part, e4m3_decode(sbyte))
