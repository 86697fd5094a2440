"""Oracle: affine group-64 quantisation, byte layouts and exact dequantisation.

TEST INFRASTRUCTURE ONLY (see the package docstring).

What the pages fix: weights are stored affine-quantised in groups of 64 along
the input dimension, each group with a scale and a bias, as 4-bit (experts and
dense MLP) or 8-bit (router) codes ([PORT] D0 section 1 "Weight schema & quant
map": OptiQ affine quant, group_size 64, the quant predicate; the
``quantized_matmul(..., scales, biases, group_size, bits)`` call in section 3).
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
  Q4G64: one little-endian uint32 word per 8 consecutive inputs of a row;
         input 8*w + 2*p + h of the row sits in word w at bits [4p+16h, 4p+16h+4).
         Rows are contiguous: row stride = cols/2 bytes.
  Q8G64: one byte per input, row-major.
  scales, biases: fp16, row-major [rows, cols/64].
"""
import numpy as np

GROUP = 64


def quantize_affine(w, bits):
    """Quantise a float32 matrix [rows, cols] into (q uint8, scale fp16, bias fp16).

    Pinned by tests/test_oracle_quant.py: grid values round-trip exactly; every
    code is a nearest grid point (brute force over all 2^bits candidates);
    constant groups give scale 0, codes 0; hand-worked example in
    tests/golden/quant_worked_example.json.
    """
    w = np.ascontiguousarray(w, dtype=np.float32)
    if w.ndim != 2 or w.shape[1] % GROUP:
        raise ValueError("quantize_affine wants [rows, cols] with cols a multiple of 64")
    rows, cols = w.shape
    g = w.reshape(rows, cols // GROUP, GROUP)
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


def pack_q4(q):
    """uint8 codes [rows, cols] (values < 16) -> uint32 words [rows, cols/8]."""
    q = np.asarray(q, dtype=np.uint8)
    rows, cols = q.shape
    if cols % 8:
        raise ValueError("cols must be a multiple of 8")
    e = q.reshape(rows, cols // 8, 4, 2).astype(np.uint32)  # [.., p, h] = input 8w+2p+h
    words = np.zeros((rows, cols // 8), dtype=np.uint32)
    for p in range(4):
        for h in range(2):
            words |= (e[:, :, p, h] & np.uint32(0xF)) << np.uint32(4 * p + 16 * h)
    return words


def unpack_q4(words, cols):
    """uint32 words [rows, cols/8] -> uint8 codes [rows, cols]."""
    words = np.asarray(words, dtype=np.uint32)
    rows = words.shape[0]
    q = np.zeros((rows, cols // 8, 4, 2), dtype=np.uint8)
    for p in range(4):
        for h in range(2):
            q[:, :, p, h] = (words >> np.uint32(4 * p + 16 * h)) & np.uint32(0xF)
    return q.reshape(rows, cols)


def pack(w, fmt):
    """Quantise and lay out one float32 matrix. fmt is 'q4' or 'q8'.

    Returns (codes, scales fp16 [rows, cols/64], biases fp16 [rows, cols/64]);
    codes are uint32 [rows, cols/8] for q4 and uint8 [rows, cols] for q8.
    """
    bits = {"q4": 4, "q8": 8}[fmt]
    q, s, b = quantize_affine(w, bits)
    codes = pack_q4(q) if fmt == "q4" else q.copy()
    return codes, s, b


def codes_of(codes, fmt, cols):
    """Packed codes -> uint8 codes [rows, cols]."""
    if fmt == "q4":
        return unpack_q4(codes, cols)
    return np.asarray(codes, dtype=np.uint8).reshape(-1, cols)


def dequantize(q, scale16, bias16):
    """Exact affine dequantisation in float64: w = scale*q + bias per group of 64."""
    q = np.asarray(q)
    rows, cols = q.shape
    s = np.repeat(np.asarray(scale16, np.float16).astype(np.float64), GROUP, axis=1)
    b = np.repeat(np.asarray(bias16, np.float16).astype(np.float64), GROUP, axis=1)
    return s * q.astype(np.float64) + b


def unpack(codes, scale16, bias16, fmt, cols):
    """Packed matrix -> float64 [rows, cols] (the value every consumer must use)."""
    return dequantize(codes_of(codes, fmt, cols), scale16, bias16)


def qlinear_grouped(v, q, scale16, bias16):
    """v [n, cols] times the quantised matrix's transpose, factored per group.

    Computes sum_g ( s_g * sum_{c in g} v_c q_c  +  b_g * sum_{c in g} v_c )
    straight from the integer codes, without forming the dequantised matrix.
    Used only to pin ``dequantize`` (the two must agree to float64 rounding).
    """
    v = np.asarray(v, np.float64)
    q = np.asarray(q, np.float64)
    rows, cols = q.shape
    ng = cols // GROUP
    vg = v.reshape(v.shape[0], ng, GROUP)
    qg = q.reshape(rows, ng, GROUP)
    s = np.asarray(scale16, np.float16).astype(np.float64)  # [rows, ng]
    b = np.asarray(bias16, np.float16).astype(np.float64)
    vq = np.einsum("ngc,rgc->nrg", vg, qg)  # per-group integer-weighted sums
    vsum = vg.sum(axis=2)  # [n, ng]
    return np.einsum("nrg,rg->nr", vq, s) + np.einsum("ng,rg->nr", vsum, b)
