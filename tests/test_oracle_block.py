"""Pins for oracle.block (CPU only): norms, router, GELU, MLP, the combine, the block."""
import itertools

import numpy as np
import pytest
import scipy.special

from oracle import block, prepare
from moe_denoise_forward_amd import synth

EPS = 1e-6


# ---------------------------------------------------------------- RMSNorm
def test_rms_norm_constant_row_closed_form():
    for c in (3.0, -0.25, 1e-4):
        x = np.full((1, 96), c)
        w = np.linspace(0.5, 1.5, 96)
        got = block.rms_norm(x, w, EPS)
        assert np.allclose(got, c / np.sqrt(c * c + EPS) * w, rtol=1e-15, atol=0)


def test_rms_norm_zero_row_and_scale_invariance():
    assert (block.rms_norm(np.zeros((2, 64)), None, EPS) == 0).all()
    rng = np.random.default_rng(1)
    x = rng.standard_normal((4, 128))
    assert np.allclose(block.rms_norm(1000.0 * x, None, EPS), block.rms_norm(x, None, EPS),
                       rtol=1e-6, atol=0)
    # unit mean square after normalisation (up to eps)
    ms = np.mean(block.rms_norm(x, None, EPS) ** 2, axis=1)
    assert np.allclose(ms, 1.0, rtol=1e-5)


def test_router_input_is_cosine_normalised():
    # rms(x) * D^-1/2 == x / sqrt(|x|^2 + D eps): the L2-normalised router input.
    rng = np.random.default_rng(2)
    d, e = 192, 10
    x = rng.standard_normal((6, d))
    wr = rng.standard_normal((e, d))
    rs = 1 + 0.1 * rng.standard_normal(d)
    z = block.router_logits(x, wr, rs, EPS)
    u = x / np.sqrt((x * x).sum(axis=1, keepdims=True) + d * EPS) * rs
    assert np.allclose(z, u @ wr.T, rtol=1e-12, atol=1e-14)


# ---------------------------------------------------------------- top-k
def test_topk_matches_full_sort_with_ties():
    # Integer-valued logits force many exact ties; the selection must equal the first k of
    # a full sort by (logit desc, index asc).
    rng = np.random.default_rng(3)
    for e, k in ((6, 3), (8, 2), (5, 5), (7, 1)):
        z = rng.integers(-2, 3, size=(300, e)).astype(np.float64)
        idx = block.select_topk(z, k)
        for t in range(z.shape[0]):
            ref = sorted(range(e), key=lambda c: (-z[t, c], c))[:k]
            assert list(idx[t]) == ref


def test_topk_brute_force_subsets():
    # Exhaustive on tiny inputs: the chosen set has the largest logit sum among all k-subsets,
    # and among equal sums the lexicographically smallest index set.
    rng = np.random.default_rng(4)
    e, k = 6, 3
    for _ in range(200):
        z = rng.integers(-3, 4, size=e).astype(np.float64)
        got = tuple(sorted(block.select_topk(z[None, :], k)[0]))
        best = min(itertools.combinations(range(e), k), key=lambda s: (-z[list(s)].sum(), s))
        assert got == best


def test_route_weights_sum_to_one_and_orders_agree():
    rng = np.random.default_rng(5)
    d, e, k = 128, 16, 4
    x = rng.standard_normal((50, d))
    wr = rng.standard_normal((e, d)) * d ** -0.5
    rs = 1 + 0.1 * rng.standard_normal(d)
    pes = 1 + 0.1 * rng.standard_normal(e)
    r = block.route(x, wr, rs, pes, k, EPS)
    assert np.allclose(r["p"].sum(axis=1), 1.0, rtol=0, atol=1e-12)
    assert np.allclose(r["w"], r["p"] * pes[r["idx"]], rtol=1e-15)
    # softmax over all, take top-k, renormalise == softmax over the top-k logits
    assert np.allclose(block.route_weights_full_softmax(r["z"], r["idx"]), r["p"],
                       rtol=1e-12, atol=1e-15)
    # descending order of the selected logits
    zs = np.take_along_axis(r["z"], r["idx"].astype(np.int64), axis=1)
    assert (np.diff(zs, axis=1) <= 0).all()
    # margin is the k-th minus (k+1)-th largest logit
    srt = np.sort(r["z"], axis=1)[:, ::-1]
    assert np.allclose(r["margin"], srt[:, k - 1] - srt[:, k])


def test_route_k_equals_e_is_full_softmax():
    rng = np.random.default_rng(6)
    d, e = 64, 8
    x = rng.standard_normal((9, d))
    wr = rng.standard_normal((e, d))
    rs = np.ones(d)
    pes = 1 + 0.1 * rng.standard_normal(e)
    r = block.route(x, wr, rs, pes, e, EPS)
    sm = scipy.special.softmax(r["z"], axis=1)
    p_by_expert = np.zeros_like(sm)
    np.put_along_axis(p_by_expert, r["idx"].astype(np.int64), r["p"], axis=1)
    assert np.allclose(p_by_expert, sm, rtol=1e-12, atol=1e-15)
    assert np.isinf(r["margin"]).all()


def test_zero_row_routes_to_lowest_indices():
    d, e, k = 64, 8, 3
    rng = np.random.default_rng(7)
    wr = rng.standard_normal((e, d))
    pes = 1 + 0.1 * rng.standard_normal(e)
    r = block.route(np.zeros((2, d)), wr, np.ones(d), pes, k, EPS)
    assert (r["idx"] == np.arange(k)).all()
    assert np.allclose(r["w"], pes[:k] / k)


# ---------------------------------------------------------------- GELU
def test_gelu_tanh_identities():
    x = np.linspace(-8, 8, 2001)
    g = block.gelu_tanh(x)
    # g(x) - g(-x) = x exactly for the form x * (1 + tanh(odd(x))) / 2
    assert np.allclose(g - block.gelu_tanh(-x), x, rtol=0, atol=1e-14)
    assert block.gelu_tanh(np.array([0.0]))[0] == 0.0
    erf_form = 0.5 * x * (1 + scipy.special.erf(x / np.sqrt(2)))
    assert np.max(np.abs(g - erf_form)) < 1e-3
    # and it is the tanh form, not the erf form: they differ by ~4e-4 at x = -3
    assert abs(block.gelu_tanh(np.array([-3.0]))[0] - erf_form[np.argmin(np.abs(x + 3))]) > 3e-4
    # large |x|: identity / zero
    assert abs(block.gelu_tanh(np.array([10.0]))[0] - 10.0) < 1e-12
    assert abs(block.gelu_tanh(np.array([-10.0]))[0]) < 1e-12


# GELU's tanh approximation (Hendrycks & Gimpel 2016), the activation the
# diffgemma contract names as gelu_pytorch_tanh (Part II section 1 "Model
# constants" and the MoE-order bullet of section 2.1), evaluated from its
# formula in double precision at seven points; rounded to 9 decimals.
GELU_TANH_POINTS = {
    -3.0: -0.003637392, -1.0: -0.158808009, -0.5: -0.154285990, 0.0: 0.0,
    0.5: 0.345714010, 1.0: 0.841191991, 3.0: 2.996362608,
}


def test_gelu_tanh_published_values():
    # A change of either constant (0.044715 -> 0.0447, sqrt(2/pi) -> 0.80)
    # moves every nonzero point by more than 1e-6.
    g = np.array(list(GELU_TANH_POINTS))
    want = np.array(list(GELU_TANH_POINTS.values()))
    assert np.max(np.abs(block.gelu_tanh(g) - want)) < 1e-9


def test_gelu_tanh_matches_torch_tanh_gelu():
    # torch's own implementation of the same approximation (what the pages'
    # "gelu_pytorch_tanh" names), in float64 on a dense grid
    import torch
    x = np.linspace(-12.0, 12.0, 48001)
    ref = torch.nn.functional.gelu(torch.from_numpy(x), approximate="tanh").numpy()
    assert np.max(np.abs(block.gelu_tanh(x) - ref)) < 1e-12
    # and it is not torch's erf form anywhere the two differ by more than rounding
    erf = torch.nn.functional.gelu(torch.from_numpy(x)).numpy()
    far = np.abs(erf - ref) > 1e-6
    assert far.sum() > 1000
    assert np.all(np.abs(block.gelu_tanh(x[far]) - erf[far]) > 5e-7)


# ---------------------------------------------------------------- MLP and combine
def _probe_mlp(d, shift, c):
    """gate = diag(c), up = identity, down = cyclic permutation out[n] = in[(n+shift) % d]."""
    gate_up = np.concatenate([np.diag(c), np.eye(d)], axis=0)
    down = np.zeros((d, d))
    down[np.arange(d), (np.arange(d) + shift) % d] = 1.0
    return gate_up, down


def test_mlp_closed_form_catches_transposes_and_gate_up_order():
    rng = np.random.default_rng(8)
    d = 64
    c = rng.uniform(0.5, 2.0, d)
    gu, dn = _probe_mlp(d, 5, c)
    v = rng.standard_normal((11, d)) * 2
    got = block.geglu_mlp(v, gu, dn)
    src = (np.arange(d) + 5) % d
    expect = np.array([[block.gelu_tanh(c[s] * row[s]) * row[s] for s in src] for row in v])
    assert np.allclose(got, expect, rtol=1e-13, atol=1e-14)
    # a transposed down (shift -5) or swapped gate/up would not match
    gu_sw = np.concatenate([gu[d:], gu[:d]], axis=0)
    assert not np.allclose(block.geglu_mlp(v, gu_sw, dn), expect, atol=1e-3)
    assert not np.allclose(block.geglu_mlp(v, gu, dn.T), expect, atol=1e-3)


def _rand_experts(rng, e, d, inter):
    gu = rng.standard_normal((e, 2 * inter, d)) * d ** -0.5
    dn = rng.standard_normal((e, d, inter)) * inter ** -0.5
    return gu, dn


def test_all_experts_identical_reduces_to_one_mlp():
    rng = np.random.default_rng(9)
    d, inter, e, k, n = 64, 32, 6, 3, 40
    gu1, dn1 = _rand_experts(rng, 1, d, inter)
    gu = np.repeat(gu1, e, axis=0)
    dn = np.repeat(dn1, e, axis=0)
    b = rng.standard_normal((n, d))
    # any routing with weights summing to 1
    idx = np.stack([rng.permutation(e)[:k] for _ in range(n)])
    p = rng.uniform(0.1, 1.0, (n, k))
    p /= p.sum(axis=1, keepdims=True)
    moe = block.moe_combine(b, idx, p, gu, dn, e)
    assert np.allclose(moe, block.geglu_mlp(b, gu1[0], dn1[0]), rtol=1e-12, atol=1e-13)


def test_top1_gives_scaled_single_expert():
    rng = np.random.default_rng(10)
    d, inter, e, n = 64, 32, 5, 30
    gu, dn = _rand_experts(rng, e, d, inter)
    b = rng.standard_normal((n, d))
    idx = rng.integers(0, e, size=(n, 1))
    pes = 1 + 0.1 * rng.standard_normal(e)
    moe = block.moe_combine(b, idx, pes[idx], gu, dn, e)
    for t in range(n):
        ex = idx[t, 0]
        assert np.allclose(moe[t], pes[ex] * block.geglu_mlp(b[t:t + 1], gu[ex], dn[ex])[0],
                           rtol=1e-12, atol=1e-13)


def test_combine_is_token_major_sum():
    # the expert-major loop equals the plain per-position sum over the k slots
    rng = np.random.default_rng(11)
    d, inter, e, k, n = 64, 32, 7, 3, 25
    gu, dn = _rand_experts(rng, e, d, inter)
    b = rng.standard_normal((n, d))
    idx = np.stack([rng.permutation(e)[:k] for _ in range(n)])
    w = rng.uniform(0.1, 1.0, (n, k))
    moe = block.moe_combine(b, idx, w, gu, dn, e)
    for t in range(n):
        ref = sum(w[t, j] * block.geglu_mlp(b[t:t + 1], gu[idx[t, j]], dn[idx[t, j]])[0]
                  for j in range(k))
        assert np.allclose(moe[t], ref, rtol=1e-12, atol=1e-13)


# ---------------------------------------------------------------- block
def _small_weights(cfg_name="mid"):
    cfg = synth.config(cfg_name)
    w32 = synth.draw_weights(cfg)
    return cfg, synth.draw_x(cfg), prepare.block_weights(w32, cfg)


def test_block_permutation_equivariance():
    cfg, x, wt = _small_weights()
    perm = np.random.default_rng(12).permutation(x.shape[0])
    y = block.block_forward(x, wt, cfg["k"], EPS)["y"]
    yp = block.block_forward(x[perm], wt, cfg["k"], EPS)["y"]
    assert np.allclose(yp, y[perm], rtol=1e-12, atol=1e-12)


def test_block_layer_scalar_is_final_multiply():
    cfg, x, wt = _small_weights()
    wt1 = dict(wt, layer_scalar=1.0)
    y1 = block.block_forward(x, wt1, cfg["k"], EPS)["y"]
    y = block.block_forward(x, wt, cfg["k"], EPS)["y"]
    assert np.allclose(y, wt["layer_scalar"] * y1, rtol=1e-15, atol=0)


def test_block_zero_rows_give_zero():
    cfg, x, wt = _small_weights()
    x = x.copy()
    x[[0, 7, 33]] = 0
    out = block.block_forward(x, wt, cfg["k"], EPS)
    assert (out["y"][[0, 7, 33]] == 0).all()
    assert (out["idx"][[0, 7, 33]] == np.arange(cfg["k"])).all()


def test_block_single_expert_closed_form():
    # D = I = I_d = 64, one expert, top-1.  Dense: gate diag(cd), up I, down shift 3;
    # expert: gate diag(ce), up I, down shift 1.  Everything is then elementwise:
    #   xh = x / sqrt(mean(x^2)+eps); a = xh*w_pre; b = xh*w_pre2
    #   h1[n] = gelu(cd[s]a[s]) a[s], s = (n+3)%64;  moe[n] = pes0 * gelu(ce[s]b[s]) b[s], s=(n+1)%64
    #   y = ls * (x + rms(rms(h1)*wp1 + rms(moe)*wp2) * wp)
    rng = np.random.default_rng(13)
    d = 64
    cd, ce = rng.uniform(0.5, 2, d), rng.uniform(0.5, 2, d)
    dgu, ddn = _probe_mlp(d, 3, cd)
    egu, edn = _probe_mlp(d, 1, ce)
    norms = {n: 1 + 0.1 * rng.standard_normal(d) for n in synth.NORM_NAMES}
    pes0 = 0.8
    wt = dict(router=rng.standard_normal((1, d)), router_scale=np.ones(d),
              per_expert_scale=np.array([pes0]), router_bias=None,
              expert_gate_up=egu[None], expert_down=edn[None],
              dense_gate_up=dgu, dense_down=ddn, layer_scalar=0.375, n_experts=1, **norms)
    x = rng.standard_normal((9, d)) * 1.7
    y = block.block_forward(x, wt, 1, EPS)["y"]

    def rms(v):
        return v / np.sqrt(np.mean(v * v, axis=1, keepdims=True) + EPS)

    xh = rms(x)
    a, b = xh * norms["pre_ff_norm"], xh * norms["pre_ff_norm_2"]
    sd, se = (np.arange(d) + 3) % d, (np.arange(d) + 1) % d
    h1 = block.gelu_tanh(cd[sd] * a[:, sd]) * a[:, sd]
    moe = pes0 * block.gelu_tanh(ce[se] * b[:, se]) * b[:, se]
    h = rms(h1) * norms["post_ff_norm_1"] + rms(moe) * norms["post_ff_norm_2"]
    expect = 0.375 * (x + rms(h) * norms["post_ff_norm"])
    assert np.allclose(y, expect, rtol=1e-12, atol=1e-13)
    # swapping the two pre-norm weights must break it
    wt_sw = dict(wt, pre_ff_norm=norms["pre_ff_norm_2"], pre_ff_norm_2=norms["pre_ff_norm"])
    assert not np.allclose(block.block_forward(x, wt_sw, 1, EPS)["y"], expect, atol=1e-4)


def test_forced_routing_is_used():
    cfg, x, wt = _small_weights()
    out = block.block_forward(x, wt, cfg["k"], EPS)
    idx = np.roll(out["idx"], 1, axis=0)
    w = np.roll(out["w"], 1, axis=0)
    forced = block.block_forward(x, wt, cfg["k"], EPS, force_idx=idx, force_w=w)
    assert (forced["idx"] == idx).all()
    ref = block.moe_combine(block.rms_norm(x, wt["pre_ff_norm_2"], EPS), idx, w,
                            wt["expert_gate_up"], wt["expert_down"], cfg["E"])
    assert np.allclose(forced["moe"], ref, rtol=1e-13, atol=1e-14)


@pytest.mark.parametrize("name", ["tiny", "mid", "mid_bf16"])
def test_block_runs_on_small_workloads(name):
    cfg, x, wt = _small_weights(name)
    out = block.block_forward(x, wt, cfg["k"], EPS)
    assert out["y"].shape == x.shape and np.isfinite(out["y"]).all()
    idx = out["idx"]
    assert ((idx >= 0) & (idx < cfg["E"])).all()
    assert all(len(set(row)) == cfg["k"] for row in idx.tolist())
