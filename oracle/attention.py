"""Oracle: the denoise attention of one decoder layer, float64.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The canvas pass of a layer ([ARCH] Part II section 2 "Two attention phases",
the Denoise bullet, and section 2.1 "Forward-pass details": Norms, RoPE, the
unit attention scale, full layers without v_proj; [BLOG] "DiffusionGemma
Explained", the attention section: rotate(), AttentionBlock.forward and the
numbered list of differences from standard attention; [PORT] dossier section 2
"Decoder architecture": Attention.__call__ and _make_decoder_masks; [GGUF]
section 4, facts 2-5).  For canvas rows t = 0..L-1, at absolute positions
p_t = kv_len + t (the canvas follows the kv_len committed positions):

  q_th = rope(rms(qraw_th) * w_q, p_t)      per-head RMSNorm with a learned
  k_tn = rope(rms(kraw_tn) * w_k, p_t)      [head_dim] weight (QK-norm), then
                                            RoPE; h = query head, n = KV head
  v_tn = rms(vraw_tn)                       weightless, no RoPE; full layers
                                            have no v_proj: vraw = kraw (the
                                            raw projection, before k_norm)
  keys of every canvas row: the committed positions j in [s, kv_len) from the
  cache (s = max(0, kv_len - window) on sliding layers, 0 on full ones), then
  all L canvas rows (bidirectional: no causal mask on the canvas)
  score_thj = q_th . K_{n(h) j}             unit scale (no 1/sqrt(head_dim))
  o_th = softmax_j(score_th) @ V_{n(h)}     n(h) = h // (H / H_kv)
  out_t = [o_t0 | o_t1 | ... | o_t,H-1]     heads concatenated, [L, H*head_dim]

The cache holds, at index j = position j, the committed key after k_norm and
RoPE at position j, and the committed value after its weightless norm (the
encode pass writes them so: [BLOG] AttentionBlock.forward, the encode branch;
[ARCH] section 3, the main f16 cache).  Its fp16 values are taken as given.

RoPE, split-half ([ARCH] section 2.1, RoPE bullet; [BLOG] rotate()): for
d < n_rot, with angle a = p * theta^(-2 d / den),
  (x_d, x_{d+S}) -> (x_d cos a - x_{d+S} sin a,  x_{d+S} cos a + x_d sin a)
and every other dimension unchanged.  Sliding layers: theta 1e4, every pair
rotated (n_rot = S = head_dim/2, den = head_dim).  Full layers: theta 1e6,
partial factor 0.25 (n_rot = head_dim/8 pairs), den = head_dim (the
"proportional" type: the exponent's denominator is the whole head_dim).

Readings where the pages disagree or are silent:
  * The partner stride S on full layers.  [ARCH] (and [PORT]'s rotated
    subset of 25% of head_dim) pair d with d + rotary_dim/2, i.e.
    S = n_rot = 64 at head_dim 512; [BLOG]'s rotate() rotates the whole
    head_dim split in half with the frequencies past the first quarter set to
    zero, i.e. S = head_dim/2 = 256.  Both are parameters here (rope_stride);
    the default is [ARCH]'s.
  * The window: a canvas row sees the last window = 1023 committed positions
    on sliding layers ([ARCH] section 2: window-1 encoder positions; [PORT]
    _make_decoder_masks: window_prefix = sliding_window - 1 = 1023).
  * Angles are taken in float64 here (the pages compute them in float32).
"""
import numpy as np


def rms(x, w=None, eps=1e-6):
    """x / sqrt(mean(x^2) + eps) over the last axis, times w if given
    ([ARCH] Part II section 2.1, Norms: classic RMSNorm, weight multiplied
    directly; weightless for V)."""
    x = np.asarray(x, np.float64)
    y = x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)
    return y if w is None else y * np.asarray(w, np.float64)


def rope_freqs(head_dim, theta, n_rot, den):
    """theta^(-2 d / den) for the n_rot rotated pairs d = 0 .. n_rot-1."""
    d = np.arange(n_rot, dtype=np.float64)
    return np.power(float(theta), -2.0 * d / float(den))


def rope(x, pos, theta, n_rot, stride, den):
    """Split-half rotation of x [..., rows, head_dim] at positions pos [rows]:
    pair (d, d + stride) for d < n_rot turned by pos * theta^(-2d/den)."""
    x = np.array(x, np.float64, copy=True)
    f = rope_freqs(x.shape[-1], theta, n_rot, den)
    a = np.asarray(pos, np.float64)[:, None] * f[None, :]      # [rows, n_rot]
    c, s = np.cos(a), np.sin(a)
    lo = x[..., :n_rot].copy()
    hi = x[..., stride:stride + n_rot].copy()
    x[..., :n_rot] = lo * c - hi * s
    x[..., stride:stride + n_rot] = hi * c + lo * s
    return x


def layer_params(kind, head_dim, rope_reading="arch"):
    """(theta, n_rot, stride, den, window) of a sliding or full layer."""
    if kind == "sliding":
        return 1e4, head_dim // 2, head_dim // 2, head_dim, 1023
    n_rot = head_dim // 8                     # 25% of head_dim rotated = head_dim/8 pairs
    stride = n_rot if rope_reading == "arch" else head_dim // 2
    return 1e6, n_rot, stride, head_dim, 0


def canvas_qkv(qraw, kraw, vraw, w_q, w_k, kv_len, H, Hkv, hd, theta, n_rot, stride, den,
               eps=1e-6):
    """The canvas's q [H, L, hd], k [Hkv, L, hd], v [Hkv, L, hd] after the
    norms and RoPE (vraw None: full layer, v from the raw k projection)."""
    L = qraw.shape[0]
    q = rms(np.asarray(qraw, np.float64).reshape(L, H, hd), w_q, eps).transpose(1, 0, 2)
    kr = np.asarray(kraw, np.float64).reshape(L, Hkv, hd)
    k = rms(kr, w_k, eps).transpose(1, 0, 2)
    vsrc = kr if vraw is None else np.asarray(vraw, np.float64).reshape(L, Hkv, hd)
    v = rms(vsrc, None, eps).transpose(1, 0, 2)
    pos = kv_len + np.arange(L)
    q = rope(q, pos, theta, n_rot, stride, den)
    k = rope(k, pos, theta, n_rot, stride, den)
    return q, k, v


def encoder_cache(kraw_enc, vraw_enc, w_k, Hkv, hd, theta, n_rot, stride, den, eps=1e-6):
    """What the encode pass writes for committed positions 0..n-1: k after
    k_norm and RoPE at its position, v after its weightless norm (vraw_enc
    None: full layer, v from the raw k projection).  [Hkv, n, hd] each."""
    n = kraw_enc.shape[0]
    kr = np.asarray(kraw_enc, np.float64).reshape(n, Hkv, hd)
    k = rope(rms(kr, w_k, eps).transpose(1, 0, 2), np.arange(n), theta, n_rot, stride, den)
    vsrc = kr if vraw_enc is None else np.asarray(vraw_enc, np.float64).reshape(n, Hkv, hd)
    return k, rms(vsrc, None, eps).transpose(1, 0, 2)


def attend(q, k_can, v_can, k_cache, v_cache, kv_len, window):
    """Softmax attention of the canvas queries q [H, L, hd] over the visible
    committed keys of the cache ([Hkv, >= kv_len, hd]) and all canvas keys;
    returns [L, H*hd]."""
    H, L, hd = q.shape
    Hkv = k_can.shape[0]
    G = H // Hkv
    s0 = max(0, kv_len - window) if window > 0 else 0
    out = np.empty((L, H * hd))
    for h in range(H):
        n = h // G
        K = np.concatenate([np.asarray(k_cache[n, s0:kv_len], np.float64), k_can[n]], axis=0)
        V = np.concatenate([np.asarray(v_cache[n, s0:kv_len], np.float64), v_can[n]], axis=0)
        sc = q[h] @ K.T                                   # unit scale
        sc = sc - sc.max(axis=1, keepdims=True)
        p = np.exp(sc)
        p /= p.sum(axis=1, keepdims=True)
        out[:, h * hd:(h + 1) * hd] = p @ V
    return out


def denoise_attention(qraw, kraw, vraw, w_q, w_k, k_cache, v_cache, kv_len, H, Hkv, hd, kind,
                      rope_reading="arch", window=None, eps=1e-6):
    """One layer's canvas attention output [L, H*hd] (see the module
    docstring); k_cache / v_cache [Hkv, >= kv_len, hd] as the encode pass left
    them.  window None: the layer type's (1023 sliding, all on full layers)."""
    theta, n_rot, stride, den, win = layer_params(kind, hd, rope_reading)
    window = win if window is None else window
    q, k, v = canvas_qkv(qraw, kraw, vraw, w_q, w_k, kv_len, H, Hkv, hd, theta, n_rot, stride,
                         den, eps)
    return attend(q, k, v, k_cache, v_cache, kv_len, window)
