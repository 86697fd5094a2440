"""Oracle: affine group-64 quantisation, byte layouts and exact dequantisation.

TEST INFRASTRUCTURE ONLY (see the package docstring).

What the pages fix: weights are stored affine-quantised in groups of 64 along
the input dimension, each group with a scale and a bias, as 4-bit (experts and
dense MLP) or 8-bit (router) codes ([PORT] D0 section 1 "Weight schema & quant
map": OptiQ affine quant, group_size 64, the quant predicate; the
``quantized_matmul(..., scales, biases, group_size, bits)`` call in section 3).
The expert-format variant q4 group-32 affine is [ARCH] section 8
"Quantization (.dgq)" (classify_tensor: MoE experts -> q4 group-32 affine;
section 8.2: q4 needs K a multiple of 32).
Weights keep the checkpoint orientation, row-major [out, in] ([ARCH] Part III
"Standing design decisions").  Scale and bias are fp16.

What the pages leave open, and the reading taken here (min/max affine):
  scale = fp16( (max - min) / (2^bits - 1) )      float32 subtract and divide
  bias  = fp16( min )
  q     = clamp( rint( (w - float(bias)) / float(scale) ), 0, 2^bits - 1 )
          in float32 (subtract, divide, round-half-even), q = 0 if scale == 0
  w_deq = float(scale) * q + float(bias)           exact in float64
The codes are an integer decision made in floating point, so they are taken in
float32, the precision the GPU packer uses; both sides then agree bit for bit.

Byte layouts (a format of this project, declared in include/dgmoe.h):
  Q4G64 (MFMA-tiled): rows in blocks of 64 (rows % 64 == 0), G = cols/64.
         For row r = 64*b + 16*s + n (s < 4, n < 16) and input
         c = 64*q + 32*h + 8*g + j (h < 2, g < 4, j < 8), the code sits in uint32
         word ((((b*G + q)*4 + g)*16 + n)*8 + 2*s + h, at bits [4p+16t, 4p+16t+4)
         where j = 2p + t.  scale_bias holds the fp16 pair (scale, bias) of
         (r, q) at uint16 index (((b*G + q)*16 + n)*4 + s)*2 + {0, 1}.
  Q8G64 (row-major): one byte per input, row-major; scale_bias fp16 pairs
         (scale, bias) at uint16 index (r * (cols/64) + q) * 2 + {0, 1}.
  Q4G32 (MFMA-tiled): the codes exactly as Q4G64; one (scale, bias) pair per
         32 inputs: the pair of row r = 64*b + 16*s + n and inputs
         64*q + 32*h .. +31 at uint16 index
         ((((b*G + q)*16 + n)*4 + s)*2 + h)*2 + {0, 1}
         (G = cols/64 as for the codes), so a row's eight pairs of a 64-input
         group (four strips x two halves) are contiguous.
  Q6G32 (MFMA-tiled; the contract's q6 expert format, read as 6-bit affine
         with groups of 32 like its q4 -- both need K a multiple of 32): the
         (scale, bias) pairs exactly as Q4G32; the codes as two planes, the low
         4 bits of every code in the words of Q4G64 (rows*cols/8 words), then
         the high 2 bits (rows*cols/16 words): the high bits of the code in
         low-plane word ((((b*G + q)*4 + g)*16 + n)*8 + 2*s + h, input
         j = 2p + t of its eight, sit in high-plane word
         (((b*G + q)*4 + g)*16 + n)*4 + s at bits [2(4h + p) + 16t, +2).
"""
import numpy as np

GROUP = 64
GROUP_SIZE = {"q4": 64, "q8": 64, "q4g32": 32, "q6": 32}
BITS = {"q4": 4, "q8": 8, "q4g32": 4, "q6": 6}


def quantize_affine(w, bits, group=GROUP):
    """Quantise a float32 matrix [rows, cols] into (q uint8, scale fp16, bias fp16).

    Pinned by tests/test_oracle_quant.py: grid values round-trip exactly; every
    code is a nearest grid point (brute force over all 2^bits candidates);
    constant groups give scale 0, codes 0; a hand-worked ramp example.
    """
    w = np.ascontiguousarray(w, dtype=np.float32)
    if w.ndim != 2 or w.shape[1] % group:
        raise ValueError(f"quantize_affine wants [rows, cols] with cols a multiple of {group}")
    rows, cols = w.shape
    g = w.reshape(rows, cols // group, group)
    lo = g.min(axis=2)
    hi = g.max(axis=2)
    qmax = np.float32(2 ** bits - 1)
    scale16 = ((hi - lo) / qmax).astype(np.float16)
    bias16 = lo.astype(np.float16)
    s = scale16.astype(np.float32)[:, :, None]
    b = bias16.astype(np.float32)[:, :, None]
    with np.errstate(divide="ignore", invalid="ignore"):
        t = (g - b) / s
        q = np.clip(np.rint(t), np.float32(0), qmax)
    q = np.where(s == 0, np.float32(0), q)
    return q.astype(np.uint8).reshape(rows, cols), scale16, bias16


def _nibble_words(q):
    """uint8 codes [rows, cols] -> uint32 words [rows, cols/8], input 8w+2p+h at bits 4p+16h."""
    q = np.asarray(q, dtype=np.uint8)
    rows, cols = q.shape
    e = q.reshape(rows, cols // 8, 4, 2).astype(np.uint32)  # [.., p, h] = input 8w+2p+h
    words = np.zeros((rows, cols // 8), dtype=np.uint32)
    for p in range(4):
        for h in range(2):
            words |= (e[:, :, p, h] & np.uint32(0xF)) << np.uint32(4 * p + 16 * h)
    return words


def _words_nibbles(words, cols):
    rows = words.shape[0]
    q = np.zeros((rows, cols // 8, 4, 2), dtype=np.uint8)
    for p in range(4):
        for h in range(2):
            q[:, :, p, h] = (words >> np.uint32(4 * p + 16 * h)) & np.uint32(0xF)
    return q.reshape(rows, cols)


def _blocks(rows, cols):
    if rows % 64 or cols % 64:
        raise ValueError("Q4G64 needs rows % 64 == 0 and cols % 64 == 0")
    return rows // 64, cols // 64


def pack_q4(q):
    """uint8 codes [rows, cols] (values < 16) -> tiled uint32 words (flat)."""
    q = np.asarray(q, dtype=np.uint8)
    rows, cols = q.shape
    nb, ng = _blocks(rows, cols)
    w = _nibble_words(q)  # [rows, cols/8]: row word 8q + 4h + g holds inputs 64q + 32h + 8g + (0..7)
    # (b, s, n, q, h, g) -> (b, q, g, n, s, h)
    return w.reshape(nb, 4, 16, ng, 2, 4).transpose(0, 3, 5, 2, 1, 4).reshape(-1).copy()


def unpack_q4(words, rows, cols):
    """Tiled uint32 words (flat) -> uint8 codes [rows, cols]."""
    nb, ng = _blocks(rows, cols)
    w = np.asarray(words, dtype=np.uint32).reshape(nb, ng, 4, 16, 4, 2)
    # (b, q, g, n, s, h) -> (b, s, n, q, h, g)
    w = w.transpose(0, 4, 3, 1, 5, 2).reshape(rows, cols // 8)
    return _words_nibbles(w, cols)


def pack_q6_high(q):
    """uint8 codes [rows, cols] (values < 64) -> the high-plane words (flat):
    two bits per code, at the position the module docstring gives."""
    q = np.asarray(q, dtype=np.uint8)
    rows, cols = q.shape
    nb, ng = _blocks(rows, cols)
    hi = (q >> 4).astype(np.uint32).reshape(nb, 4, 16, ng, 2, 4, 4, 2)  # b, s, n, q, h, g, p, t
    w = np.zeros((nb, 4, 16, ng, 4), np.uint32)                          # b, s, n, q, g
    for h in range(2):
        for p in range(4):
            for t in range(2):
                w |= hi[:, :, :, :, h, :, p, t] << np.uint32(2 * (4 * h + p) + 16 * t)
    # (b, s, n, q, g) -> (b, q, g, n, s)
    return w.transpose(0, 3, 4, 2, 1).reshape(-1).copy()


def unpack_q6_high(words, rows, cols):
    """High-plane words (flat) -> the high two bits [rows, cols] (uint8)."""
    nb, ng = _blocks(rows, cols)
    w = np.asarray(words, np.uint32).reshape(nb, ng, 4, 16, 4).transpose(0, 4, 3, 1, 2)  # b,s,n,q,g
    hi = np.zeros((nb, 4, 16, ng, 2, 4, 4, 2), np.uint8)
    for h in range(2):
        for p in range(4):
            for t in range(2):
                hi[:, :, :, :, h, :, p, t] = (w >> np.uint32(2 * (4 * h + p) + 16 * t)) & 3
    return hi.reshape(rows, cols)


def pack_scale_bias(scale16, bias16, fmt):
    """fp16 [rows, groups] scale and bias -> interleaved uint16 pairs in the fmt's order."""
    sb = np.stack([np.asarray(scale16, np.float16).view(np.uint16),
                   np.asarray(bias16, np.float16).view(np.uint16)], axis=-1)  # [rows, g, 2]
    rows, g = sb.shape[:2]
    if fmt == "q4":
        nb = rows // 64
        # (b, s, n, q, pair) -> (b, q, n, s, pair)
        return sb.reshape(nb, 4, 16, g, 2).transpose(0, 3, 2, 1, 4).reshape(-1).copy()
    if fmt in ("q4g32", "q6"):
        nb, g64 = rows // 64, g // 2
        # (b, s, n, q, h, pair) -> (b, q, n, s, h, pair)
        return sb.reshape(nb, 4, 16, g64, 2, 2).transpose(0, 3, 2, 1, 4, 5).reshape(-1).copy()
    return sb.reshape(-1).copy()


def unpack_scale_bias(sb, rows, cols, fmt):
    g = cols // GROUP_SIZE[fmt]
    sb = np.asarray(sb, np.uint16).reshape(-1)
    if fmt == "q4":
        nb = rows // 64
        a = sb.reshape(nb, g, 16, 4, 2).transpose(0, 3, 2, 1, 4).reshape(rows, g, 2)
    elif fmt in ("q4g32", "q6"):
        nb, g64 = rows // 64, g // 2
        a = sb.reshape(nb, g64, 16, 4, 2, 2).transpose(0, 3, 2, 1, 4, 5).reshape(rows, g, 2)
    else:
        a = sb.reshape(rows, g, 2)
    return a[:, :, 0].copy().view(np.float16), a[:, :, 1].copy().view(np.float16)


def pack(w, fmt):
    """Quantise and lay out one float32 matrix. fmt is 'q4', 'q4g32', 'q6' or 'q8'.

    Returns (codes, scale_bias): codes are uint32 words (q4 / q4g32, tiled,
    flat) or uint8 [rows, cols] (q8); scale_bias is the flat uint16 array of
    (scale, bias) fp16 pairs in the format's order.
    """
    q, s, b = quantize_affine(w, BITS[fmt], GROUP_SIZE[fmt])
    if fmt == "q6":  # the low plane, then the high plane
        codes = np.concatenate([pack_q4(q & 15), pack_q6_high(q)])
    else:
        codes = pack_q4(q) if fmt in ("q4", "q4g32") else q.copy()
    return codes, pack_scale_bias(s, b, fmt)


def codes_of(codes, fmt, rows, cols):
    """Packed codes -> uint8 codes [rows, cols]."""
    if fmt in ("q4", "q4g32"):
        return unpack_q4(codes, rows, cols)
    if fmt == "q6":
        codes = np.asarray(codes, np.uint32).reshape(-1)
        n = rows * cols // 8
        return unpack_q4(codes[:n], rows, cols) | (unpack_q6_high(codes[n:], rows, cols) << 4)
    return np.asarray(codes, dtype=np.uint8).reshape(rows, cols)


def dequantize(q, scale16, bias16):
    """Exact affine dequantisation in float64: w = scale*q + bias per group
    (the group size is cols / scale16.shape[1])."""
    q = np.asarray(q)
    rows, cols = q.shape
    gs = cols // np.asarray(scale16).shape[1]
    s = np.repeat(np.asarray(scale16, np.float16).astype(np.float64), gs, axis=1)
    b = np.repeat(np.asarray(bias16, np.float16).astype(np.float64), gs, axis=1)
    return s * q.astype(np.float64) + b


def unpack(codes, scale_bias, fmt, rows, cols):
    """Packed matrix -> float64 [rows, cols] (the value every consumer must use)."""
    s, b = unpack_scale_bias(scale_bias, rows, cols, fmt)
    return dequantize(codes_of(codes, fmt, rows, cols), s, b)


def qlinear_grouped(v, q, scale16, bias16):
    """v [n, cols] times the quantised matrix's transpose, factored per group.

    Computes sum_g ( s_g * sum_{c in g} v_c q_c  +  b_g * sum_{c in g} v_c )
    straight from the integer codes, without forming the dequantised matrix.
    Used only to pin ``dequantize`` (the two must agree to float64 rounding).
    """
    v = np.asarray(v, np.float64)
    q = np.asarray(q, np.float64)
    rows, cols = q.shape
    ng = np.asarray(scale16).shape[1]
    gs = cols // ng
    vg = v.reshape(v.shape[0], ng, gs)
    qg = q.reshape(rows, ng, gs)
    s = np.asarray(scale16, np.float16).astype(np.float64)  # [rows, ng]
    b = np.asarray(bias16, np.float16).astype(np.float64)
    vq = np.einsum("ngc,rgc->nrg", vg, qg)  # per-group integer-weighted sums
    vsum = vg.sum(axis=2)  # [n, ng]
    return np.einsum("nrg,rg->nr", vq, s) + np.einsum("ng,rg->nr", vsum, b)
