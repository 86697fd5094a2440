"""Oracle: the two ends of a denoising forward around the FFN blocks, float64.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Both ends read the tied embedding table E [V, D] (the token embeddings are
also the output head: [BLOG] "Complete DiffusionGemma model", W_embed used for
the lookup, the self-conditioning mix and the final logits; [ARCH] Part II
section 1 "Model constants", vocab row: tied embeddings).

Self-conditioned canvas input, per position t ([ARCH] Part II section 5
"Self-conditioning (SC)" and section 2.1, the SC-injection bullet; [PORT]
dossier section 3 "Self-conditioning": SelfConditioning.__call__ and
DecoderModel._embed_canvas; [BLOG] "Complete DiffusionGemma model", _forward):
  e_t    = E[id_t] * sqrt(D)                  hard token embedding
  P_t    = softmax(sc_logits_t)               the previous step's logits, which
                                              arrive already divided by the
                                              schedule temperature
  soft_t = (P_t @ E) * sqrt(D)                expected embedding under P_t (the
                                              soft mix takes the same scale)
  n_t    = rms(soft_t) * w_pre                pre_norm, weighted
  s_t    = down( gelu_tanh(gate n_t) * (up n_t) )
  out_t  = rms(e_t + s_t)                     post_norm, no weight
With no previous prediction the signal is zero: rms(0) = 0 (eps inside the
root), the MLP maps 0 to 0, and out_t = rms(e_t) ([BLOG]: the first decode
step's zero signal is the same as skipping self-conditioning).

Forward tail, per position t ([BLOG] "Complete DiffusionGemma model": the final
norm, x @ W_embed^T in float32, tanh softcap; [BLOG] "Logit Softcapping";
[ARCH] Part II section 1, final softcap 30; section 4 item 3 "Finish"; section
6 item 2, row statistics of the logits divided by T):
  xn_t = rms(x_t) * w_final
  z_t  = xn_t @ E^T                           [V] logits of the tied head
  c_t  = 30 tanh(z_t / 30)                    final softcap
  y_t  = c_t / T                              schedule temperature T
  p_t  = softmax(y_t)
  H_t  = -sum_v p_tv ln p_tv                  entropy in nats
  a_t  = argmax_v y_tv                        lowest index among equal maxima
  m_t  = max_v y_tv,  l_t = sum_v exp(y_tv - m_t)   the softmax normalisers
y_t is also what the next step's self-conditioning reads ([ARCH] section 4
item 3: the logits are divided by T before the soft embedding).

Readings where the pages are silent:
  * sqrt(D) is taken in full precision, not rounded to the activation type.
  * The embedding table is the same quantised table (Q4G64) at both ends; its
    dequantised values are exact (oracle.quant.unpack).
  * The entropy uses ln p = y - m - ln l, so rows whose far tail underflows
    to p = 0 still sum exactly over every vocabulary entry.
  * argmax ties go to the lower vocabulary index, as the router's ties do.

Memory: E can be large (262144 x 2816), so the table is read in chunks of
rows; each chunk is dequantised on its own.  The chunked sums are the plain
matrix products written as sums over row blocks (pinned against the one-shot
products in tests/test_oracle_head.py).
"""
from concurrent.futures import ThreadPoolExecutor

import numpy as np

from . import quant
from .block import gelu_tanh, rms_norm

SOFTCAP = 30.0


class EmbedTable:
    """The tied table E [V, D] as float64 row blocks.

    Either packed Q4G64 bytes of the oracle's own packer (codes, scale_bias) or
    a dense float array.  rows(lo, hi) returns the float64 values of rows
    [lo, hi); for Q4G64, lo and hi must be multiples of 64 (a 64-row block is
    a contiguous slice of both arrays in that layout; V itself is a multiple
    of 64 in that format).
    """

    def __init__(self, V, D, codes=None, scale_bias=None, dense=None):
        self.V, self.D = int(V), int(D)
        self.codes, self.sb, self.dense = codes, scale_bias, dense
        if dense is None and (codes is None or scale_bias is None):
            raise ValueError("EmbedTable needs packed bytes or dense values")

    @classmethod
    def pack_q4(cls, w32, chunk=8192, workers=8):
        """Quantise and pack a float32 table [V, D] with the oracle's packer, in
        row blocks (blocks of whole 64-row groups pack independently)."""
        V, D = w32.shape
        los = list(range(0, V, chunk))
        with ThreadPoolExecutor(max_workers=workers) as ex:
            parts = list(ex.map(lambda lo: quant.pack(w32[lo:lo + chunk], "q4"), los))
        return cls(V, D, np.concatenate([c for c, _ in parts]), np.concatenate([sb for _, sb in parts]))

    def densified(self, chunk=8192, workers=8):
        """The same table with every row dequantised once (float64 [V, D])."""
        if self.dense is not None:
            return self
        out = np.empty((self.V, self.D))
        los = list(range(0, self.V, chunk))

        def fill(lo):
            hi = min(self.V, lo + chunk)
            out[lo:hi] = self.rows(lo, hi)

        with ThreadPoolExecutor(max_workers=workers) as ex:
            list(ex.map(fill, los))
        return EmbedTable(self.V, self.D, dense=out)

    def rows(self, lo, hi):
        if self.dense is not None:
            return np.asarray(self.dense[lo:hi], np.float64)
        G = self.D // 64
        if lo % 64 or hi % 64:
            raise ValueError("Q4G64 row blocks start and end on multiples of 64")
        w0, w1 = lo * G * 8, hi * G * 8      # 8 code words per (row, group)
        s0, s1 = lo * G * 2, hi * G * 2      # one (scale, bias) pair per (row, group)
        return quant.unpack(self.codes[w0:w1], self.sb[s0:s1], "q4", hi - lo, self.D)

    def chunks(self, chunk=8192):
        for lo in range(0, self.V, chunk):
            hi = min(self.V, lo + chunk)
            yield lo, hi, self.rows(lo, hi)


def softmax_rows(y):
    """softmax over the last axis, float64 (max subtracted first)."""
    y = np.asarray(y, np.float64)
    e = np.exp(y - y.max(axis=-1, keepdims=True))
    return e / e.sum(axis=-1, keepdims=True)


def hard_embed(table, ids):
    """E[id] * sqrt(D) for each canvas id."""
    ids = np.asarray(ids, np.int64)
    out = np.empty((ids.shape[0], table.D))
    for i, v in enumerate(ids):
        lo = (int(v) // 64) * 64
        out[i] = table.rows(lo, min(lo + 64, table.V))[int(v) - lo]
    return out * np.sqrt(table.D)


def soft_embed(sc_logits, table, chunk=8192):
    """(softmax(sc_logits) @ E) * sqrt(D), E read in row blocks.

    The probabilities are exp(y - m) / l per row; the sum over the vocabulary
    is taken block by block and divided by l at the end.  Pinned: equals the
    one-shot product softmax(y) @ E; a one-hot row gives the hard embedding;
    uniform logits give the mean embedding; brute force on tiny inputs.
    """
    y = np.asarray(sc_logits, np.float64)
    e = np.exp(y - y.max(axis=1, keepdims=True))
    acc = np.zeros((y.shape[0], table.D))
    for lo, hi, rows in table.chunks(chunk):
        acc += e[:, lo:hi] @ rows
    return acc / e.sum(axis=1, keepdims=True) * np.sqrt(table.D)


def sc_mlp(signal, w_pre, gate_up, down, eps=1e-6):
    """down( gelu_tanh(gate n) * (up n) ) with n = rms(signal) * w_pre.

    gate_up is the stacked [2 I_sc, D] matrix (gate rows first), down is
    [D, I_sc] -- the dense MLP's shapes ([PORT] dossier section 3).  Pinned:
    the diagonal-gate closed form and the zero signal (tests/test_oracle_head.py).
    """
    n = rms_norm(signal, w_pre, eps)
    gate_up = np.asarray(gate_up, np.float64)
    inter = gate_up.shape[0] // 2
    g = n @ gate_up[:inter].T
    u = n @ gate_up[inter:].T
    return (gelu_tanh(g) * u) @ np.asarray(down, np.float64).T


def sc_input(ids, sc_logits, table, w_pre, gate_up, down, eps=1e-6, chunk=8192):
    """The self-conditioned canvas input [L, D]; sc_logits None = no previous step.

    Returns dict(out, embeds, soft, s).
    """
    embeds = hard_embed(table, ids)
    if sc_logits is None:
        soft = np.zeros_like(embeds)
    else:
        soft = soft_embed(sc_logits, table, chunk)
    s = sc_mlp(soft, w_pre, gate_up, down, eps)
    return {"out": rms_norm(embeds + s, None, eps), "embeds": embeds, "soft": soft, "s": s}


def softcap(z, cap=SOFTCAP):
    """cap * tanh(z / cap).  Pinned: closed-form points, oddness, the bound."""
    z = np.asarray(z, np.float64)
    return cap * np.tanh(z / cap)


def tied_logits(xn, table, chunk=8192):
    """xn @ E^T [L, V], E read in row blocks (pinned against the one-shot product)."""
    xn = np.asarray(xn, np.float64)
    z = np.empty((xn.shape[0], table.V))
    for lo, hi, rows in table.chunks(chunk):
        z[:, lo:hi] = xn @ rows.T
    return z


def row_stats(y):
    """Entropy (nats), argmax (lowest index on ties), max m and l = sum exp(y - m).

    Also returns margin = (largest y) - (second largest y), the gap below which
    a float32 GPU may pick another argmax.  Pinned: uniform rows give ln V, a
    dominant entry gives ~0, two equal maxima give ln 2 and the lower index,
    brute force on tiny rows.
    """
    y = np.asarray(y, np.float64)
    m = y.max(axis=1)
    d = y - m[:, None]
    e = np.exp(d)
    l = e.sum(axis=1)
    logp = d - np.log(l)[:, None]
    H = -(e / l[:, None] * logp).sum(axis=1)
    a = np.argmax(y, axis=1).astype(np.int32)
    if y.shape[1] > 1:
        top2 = -np.partition(-y, 1, axis=1)[:, :2]
        margin = top2[:, 0] - top2[:, 1]
    else:
        margin = np.full(y.shape[0], np.inf)
    return {"H": H, "argmax": a, "m": m, "l": l, "margin": margin}


def tail(x, w_final, table, T, eps=1e-6, chunk=8192):
    """The forward tail on the last block's output x [L, D].

    Returns dict(y [L, V], z, H, argmax, m, l, margin) with y = softcap(z) / T.
    """
    xn = rms_norm(x, w_final, eps)
    z = tied_logits(xn, table, chunk)
    y = softcap(z) / float(T)
    out = row_stats(y)
    out.update(y=y, z=z)
    return out
