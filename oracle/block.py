"""Oracle: the parallel dense-MLP + routed-MoE FFN block, in float64.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The block, per canvas position t, with rms(v) = v / sqrt(mean(v^2) + eps):
  1. xh = rms(x_t)                                   (one normalisation of x)
  2. router: u = xh * router_scale * D^-1/2; z = u W_r^T (+ bias);
     the k largest z (ties -> lower expert index); p = softmax over those k;
     w_j = p_j * per_expert_scale[e_j]
  3. dense branch:  h1 = MLP_dense(xh * pre_ff_norm)
  4. experts:       moe = sum_j w_j * MLP_{e_j}(xh * pre_ff_norm_2)
  5. h = rms(h1) * post_ff_norm_1 + rms(moe) * post_ff_norm_2
  6. y_t = layer_scalar * (x_t + rms(h) * post_ff_norm)
with MLP(v) = W_down (gelu_tanh(W_gate v) * (W_up v)), W_gate = the first half
of the stacked gate_up rows.

Sources: [ARCH] Part II section 2.1 "Forward-pass details" (the Norms bullet:
weight used directly, eps 1e-6, seven norms; the MoE-order bullet: no-scale
norm, router_scale * hidden^-0.5, softmax, top-8, renormalise, per_expert_scale,
tie-break, fused [gate||up], gelu_pytorch_tanh, dense MLP always on);
[BLOG] "MLP and mixture-of-experts block" (MLP and MOEBlock: the loop over
experts with a token mask, post_norm_1 / post_norm_2 / post_norm, residual)
and "Complete DiffusionGemma model" (x * layer_scalar after the block);
[PORT] D0 section 2 (DecoderLayer parallel FFN; Router normalising before the
projection and taking the softmax over the selected scores; Experts;
geglu = gelu_approx(gate) * up); [GGUF] section 4 facts 7 and 9.

Readings where the pages differ or are silent:
  * eps sits inside the square root, as [ARCH] writes it ([BLOG] adds eps to
    the norm instead; the difference is of order eps except on near-zero rows).
  * GELU is the tanh approximation (gelu_pytorch_tanh per [ARCH] section 1 and
    [PORT] section 1; [BLOG]'s code calls the erf form).
  * Softmax over all experts then top-k then renormalise ([ARCH], [BLOG]) equals
    top-k on the logits then softmax over the k ([PORT]); selection is done on
    the logits, ties to the lower expert index.
  * Routing weights are kept in full precision (not rounded to bf16).
  * The router reads the block input x (through the weightless norm); the
    experts read pre_ff_norm_2(x) and the dense MLP reads pre_ff_norm(x).
"""
import numpy as np


def rms_norm(x, w=None, eps=1e-6):
    """x / sqrt(mean(x^2) + eps) [* w], over the last axis, float64.

    Pinned: constant-row closed form, zero row, scale invariance
    (tests/test_oracle_block.py).
    """
    x = np.asarray(x, np.float64)
    r = 1.0 / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)
    y = x * r
    if w is not None:
        y = y * np.asarray(w, np.float64)
    return y


def gelu_tanh(g):
    """0.5 g (1 + tanh( sqrt(2/pi) (g + 0.044715 g^3) )), the tanh form of GELU.

    Pinned: the formula's values at seven points (tests/test_oracle_block.py,
    GELU_TANH_POINTS), torch.nn.functional.gelu(approximate="tanh") in float64
    on a dense grid, the odd-part identity gelu(x) - gelu(-x) = x, and its
    distance from the erf form.
    """
    g = np.asarray(g, np.float64)
    c = np.sqrt(2.0 / np.pi)
    return 0.5 * g * (1.0 + np.tanh(c * (g + 0.044715 * g ** 3)))


def router_logits(x, router_w, router_scale, eps=1e-6, router_bias=None):
    """z[t, e] = ((rms(x_t) * router_scale) * D^-1/2) . W_r[e] (+ bias_e).

    The two-step scale (norm, then scale * hidden^-0.5) follows [PORT] D0
    section 2 "Router" and its D1 finding that folding the two is wrong.
    Pinned: the cosine form x / sqrt(|x|^2 + D eps) * D^-1/2 ... identity.
    """
    x = np.asarray(x, np.float64)
    d = x.shape[-1]
    u = rms_norm(x, None, eps) * np.asarray(router_scale, np.float64) * (d ** -0.5)
    z = u @ np.asarray(router_w, np.float64).T
    if router_bias is not None:
        z = z + np.asarray(router_bias, np.float64)[None, :]
    return z


def select_topk(z, k):
    """Indices of the k largest logits per row, ordered by (logit desc, index asc).

    Repeated selection of the maximum; np.argmax returns the first maximal
    position, i.e. the lowest expert index among equal maxima.  Logits must be
    finite.  Pinned against a full sort on tiny inputs with forced ties.
    """
    zz = np.array(z, dtype=np.float64, copy=True)
    n = zz.shape[0]
    rows = np.arange(n)
    idx = np.zeros((n, k), dtype=np.int32)
    for j in range(k):
        best = np.argmax(zz, axis=1)
        idx[:, j] = best
        zz[rows, best] = -np.inf
    return idx


def route(x, router_w, router_scale, per_expert_scale, top_k, eps=1e-6, router_bias=None):
    """Router: returns dict(idx [L,k] int32, w [L,k], p [L,k], z [L,E], margin [L]).

    p is the softmax over the k selected logits (sums to 1); w = p *
    per_expert_scale[idx]; margin = z_(k) - z_(k+1), the gap that decides
    whether a float32 GPU may legitimately pick a different set (inf if k == E).
    """
    z = router_logits(x, router_w, router_scale, eps, router_bias)
    idx = select_topk(z, top_k)
    zs = np.take_along_axis(z, idx.astype(np.int64), axis=1)
    ex = np.exp(zs - zs[:, :1])
    p = ex / ex.sum(axis=1, keepdims=True)
    w = p * np.asarray(per_expert_scale, np.float64)[idx]
    e = z.shape[1]
    if top_k < e:
        srt = -np.sort(-z, axis=1)
        margin = srt[:, top_k - 1] - srt[:, top_k]
    else:
        margin = np.full(z.shape[0], np.inf)
    return {"idx": idx, "w": w, "p": p, "z": z, "margin": margin}


def route_weights_full_softmax(z, idx):
    """The other published order: softmax over all experts, take the selected
    probabilities, renormalise them to sum 1 ([ARCH] MoE order; [BLOG] MOEBlock).
    Used only to pin ``route`` (the two orders agree in exact arithmetic)."""
    z = np.asarray(z, np.float64)
    pf = np.exp(z - z.max(axis=1, keepdims=True))
    pf = pf / pf.sum(axis=1, keepdims=True)
    sel = np.take_along_axis(pf, np.asarray(idx, np.int64), axis=1)
    return sel / sel.sum(axis=1, keepdims=True)


def geglu_mlp(v, gate_up, down):
    """down( gelu_tanh(gate v) * (up v) ) for rows v [n, D].

    gate_up is the stacked [2I, D] matrix, gate = rows [0, I), up = rows [I, 2I)
    ([ARCH] fused [gate||up]; [BLOG] rearrange '(z intermed) D'); down is [D, I].
    Pinned: diagonal-gate / identity-up / permutation-down closed form.
    """
    gate_up = np.asarray(gate_up, np.float64)
    inter = gate_up.shape[0] // 2
    g = v @ gate_up[:inter].T
    u = v @ gate_up[inter:].T
    return (gelu_tanh(g) * u) @ np.asarray(down, np.float64).T


def moe_combine(b, idx, w, expert_gate_up, expert_down, n_experts):
    """moe[t] = sum_j w[t,j] * MLP_{idx[t,j]}(b[t]).

    Written as [BLOG]'s loop: for each expert, gather the positions routed to
    it, run its MLP once on them, add the weighted result back.
    expert_gate_up / expert_down may be arrays [E, ...] or mappings holding
    only the experts that are used.  Pinned: all-experts-identical reduces to
    one MLP; k = 1 gives per_expert_scale * MLP_e.
    """
    b = np.asarray(b, np.float64)
    idx = np.asarray(idx)
    w = np.asarray(w, np.float64)
    out = np.zeros_like(b)
    for e in range(n_experts):
        hit = idx == e  # [L, k]
        rows = np.nonzero(hit.any(axis=1))[0]
        if rows.size == 0:
            continue
        mult = (w * hit)[rows].sum(axis=1)  # each row names an expert at most once
        out[rows] += mult[:, None] * geglu_mlp(b[rows], expert_gate_up[e], expert_down[e])
    return out


def block_forward(x, wt, top_k, eps=1e-6, force_idx=None, force_w=None):
    """The whole block on canvas rows x [L, D]; wt holds float64 weights:

      router [E, D], router_scale [D], per_expert_scale [E], router_bias [E] | None,
      expert_gate_up [E, 2I, D] (or mapping e -> [2I, D]), expert_down [E, D, I],
      dense_gate_up [2I_d, D], dense_down [D, I_d],
      pre_ff_norm, pre_ff_norm_2, post_ff_norm_1, post_ff_norm_2, post_ff_norm [D],
      layer_scalar (float), n_experts (int).

    Returns dict(y, moe, h1, idx, w, margin, z).  force_idx / force_w replace
    the router's choice (tests inject a routing this way).
    Pinned: per-position permutation equivariance, layer_scalar linearity,
    zero rows, the single-expert closed form (tests/test_oracle_block.py).
    """
    x = np.asarray(x, np.float64)
    xh = rms_norm(x, None, eps)
    r = route(x, wt["router"], wt["router_scale"], wt["per_expert_scale"], top_k,
              eps, wt.get("router_bias"))
    idx, w = r["idx"], r["w"]
    if force_idx is not None:
        idx = np.asarray(force_idx)
        w = np.asarray(force_w, np.float64)
    a = xh * np.asarray(wt["pre_ff_norm"], np.float64)
    b = xh * np.asarray(wt["pre_ff_norm_2"], np.float64)
    h1 = geglu_mlp(a, wt["dense_gate_up"], wt["dense_down"])
    moe = moe_combine(b, idx, w, wt["expert_gate_up"], wt["expert_down"], wt["n_experts"])
    h = rms_norm(h1, wt["post_ff_norm_1"], eps) + rms_norm(moe, wt["post_ff_norm_2"], eps)
    y = float(wt["layer_scalar"]) * (x + rms_norm(h, wt["post_ff_norm"], eps))
    return {"y": y, "moe": moe, "h1": h1, "idx": idx, "w": w,
            "margin": r["margin"], "z": r["z"]}
