"""Pins of the head oracle (oracle/head.py) against what the pages and the
mathematics fix: closed forms, special cases, brute force on tiny inputs and
the one-shot matrix products the chunked sums stand for."""
import math

import numpy as np
import pytest

from moe_denoise_forward_amd import synth
from oracle import head, quant
from oracle.block import rms_norm

# gelu_tanh at +-1 and +-3: the formula's values (pinned for the block oracle
# in tests/test_oracle_block.py), written out again here as literals
GELU_1, GELU_M1, GELU_3, GELU_M3 = 0.841191991, -0.158808009, 2.996362608, -0.003637392


def _dense_table(V, D, seed=0):
    r = np.random.default_rng(seed)
    return head.EmbedTable(V, D, dense=r.standard_normal((V, D)) * 0.1)


# ---------------------------------------------------------------- the table
def test_q4_row_blocks_are_the_whole_unpack():
    r = np.random.default_rng(1)
    w = r.standard_normal((320, 128)).astype(np.float32)
    t = head.EmbedTable.pack_q4(w, chunk=128)     # packed in three row blocks
    codes, sb = quant.pack(w, "q4")               # and in one
    full = quant.unpack(codes, sb, "q4", 320, 128)
    assert np.array_equal(np.concatenate([r_ for _, _, r_ in t.chunks(64)]), full)
    assert np.array_equal(t.rows(128, 256), full[128:256])
    with pytest.raises(ValueError):
        t.rows(10, 64)


def test_hard_embed_is_the_scaled_row():
    t = _dense_table(256, 64)
    ids = np.array([0, 63, 64, 255, 7])
    e = head.hard_embed(t, ids)
    assert np.array_equal(e, t.dense[ids] * 8.0)   # sqrt(64) = 8


# ---------------------------------------------------------------- soft embedding
def test_chunked_soft_embed_equals_the_one_shot_product():
    t = _dense_table(512, 128)
    y = np.random.default_rng(2).standard_normal((7, 512)) * 3
    one = head.softmax_rows(y) @ t.dense * math.sqrt(128)
    for chunk in (64, 192, 512):
        assert np.allclose(head.soft_embed(y, t, chunk), one, rtol=0, atol=1e-13)


def test_soft_embed_brute_force():
    V, D = 128, 64
    t = _dense_table(V, D, seed=3)
    y = np.random.default_rng(4).standard_normal((3, V)) * 2
    got = head.soft_embed(y, t, chunk=64)
    for i in range(3):
        ex = [math.exp(v) for v in y[i]]
        s = sum(ex)
        for d in range(0, D, 7):
            want = sum(ex[v] / s * t.dense[v, d] for v in range(V)) * math.sqrt(D)
            assert abs(got[i, d] - want) < 1e-12


def test_one_hot_soft_embed_is_the_hard_embed():
    # the soft mix takes the same sqrt(hidden) scale as the token embedding
    t = _dense_table(256, 64)
    ids = np.array([5, 200, 64])
    y = np.zeros((3, 256))
    y[np.arange(3), ids] = 1000.0
    assert np.allclose(head.soft_embed(y, t, 64), head.hard_embed(t, ids), rtol=0, atol=1e-12)


def test_uniform_soft_embed_is_the_mean_row():
    t = _dense_table(192, 64)
    y = np.full((2, 192), -4.25)
    assert np.allclose(head.soft_embed(y, t, 64), t.dense.mean(axis=0) * 8.0, rtol=0, atol=1e-13)


# ---------------------------------------------------------------- self-conditioning
def _sc_weights(D, I, seed=5):
    r = np.random.default_rng(seed)
    return (1 + 0.1 * r.standard_normal(D), r.standard_normal((2 * I, D)) / math.sqrt(D),
            r.standard_normal((D, I)) / math.sqrt(I))


def test_zero_signal_gives_the_post_norm_of_the_embedding():
    t = _dense_table(256, 64)
    w_pre, gu, dn = _sc_weights(64, 32)
    ids = np.array([1, 2, 250])
    r = head.sc_input(ids, None, t, w_pre, gu, dn)
    assert np.array_equal(r["s"], np.zeros((3, 64)))
    assert np.array_equal(r["out"], rms_norm(head.hard_embed(t, ids), None, 1e-6))
    assert np.array_equal(head.sc_mlp(np.zeros((2, 64)), w_pre, gu, dn), np.zeros((2, 64)))
    # the post-norm has no weight: unit mean square per row
    assert np.allclose((r["out"] ** 2).mean(axis=1), 1.0, atol=1e-6)


@pytest.mark.parametrize("c,wp", [(1.0, 1.0), (3.0, 1.0), (2.0, 0.5)])
def test_diagonal_mlp_closed_form(c, wp):
    # D = I_sc = 64, gate = c * identity, up = identity, down = identity,
    # pre-norm weight wp, eps 0, table rows of +-1: a one-hot previous step at
    # token v gives soft = E[v] * 8, n = wp E[v], s = gelu(c n) * n, and
    # out = (E[id] * 8 + s) / rms(E[id] * 8 + s); c * wp is 1 or 3, where the
    # GELU values are known
    D = 64
    r = np.random.default_rng(6)
    table = np.where(r.random((128, D)) < 0.5, -1.0, 1.0)
    t = head.EmbedTable(128, D, dense=table)
    eye = np.eye(D)
    gu = np.concatenate([c * eye, eye])
    ids = np.array([3, 77])
    picks = np.array([10, 100])
    y = np.zeros((2, 128))
    y[np.arange(2), picks] = 800.0
    got = head.sc_input(ids, y, t, np.full(D, wp), gu, eye, eps=0.0)
    gl = {(1.0, 1): GELU_1, (1.0, -1): GELU_M1, (3.0, 1): GELU_3, (3.0, -1): GELU_M3}
    for i in range(2):
        n = table[picks[i]]
        s = np.array([gl[(c * wp, int(v))] * v * wp for v in n])
        v = table[ids[i]] * 8.0 + s
        want = v / math.sqrt((v * v).mean())
        assert np.allclose(got["s"][i], s, rtol=0, atol=2e-9)
        assert np.allclose(got["out"][i], want, rtol=0, atol=2e-9)


# ---------------------------------------------------------------- softcap
def test_softcap_closed_forms():
    assert head.softcap(30.0 * math.atanh(0.5)) == pytest.approx(15.0, abs=1e-12)
    assert head.softcap(30.0 * math.atanh(-0.9)) == pytest.approx(-27.0, abs=1e-12)
    z = np.linspace(-500, 500, 2001)
    c = head.softcap(z)
    assert np.all(np.abs(c) < 30.0 + 1e-12) and np.array_equal(c, -head.softcap(-z))
    assert np.all(np.diff(c) >= 0)
    # small logits pass almost unchanged: 30 tanh(z/30) = z - z^3/2700 + 2 z^5/(15 30^4) - ...
    assert head.softcap(0.3) == pytest.approx(0.3 - 0.3 ** 3 / 2700 + 2 * 0.3 ** 5 / 12150000,
                                              abs=1e-13)


# ---------------------------------------------------------------- row statistics
def test_row_stats_uniform_row_is_ln_V():
    s = head.row_stats(np.full((2, 4096), 1.5))
    assert np.allclose(s["H"], math.log(4096), rtol=0, atol=1e-12)   # nats, not bits
    assert np.array_equal(s["argmax"], [0, 0])
    assert np.allclose(s["l"], 4096) and np.allclose(s["m"], 1.5)


def test_row_stats_ties_and_peaks():
    y = np.full((3, 100), -1e4)
    y[0, [17, 42]] = 3.0            # two equal maxima: ln 2, the lower index
    y[1, 60] = 50.0                  # one dominant entry: entropy ~ 0
    y[2] = np.arange(100) * 0.0
    s = head.row_stats(y)
    assert s["H"][0] == pytest.approx(math.log(2), abs=1e-12) and s["argmax"][0] == 17
    assert s["margin"][0] == 0.0
    assert s["H"][1] < 1e-12 and s["argmax"][1] == 60
    assert s["H"][2] == pytest.approx(math.log(100), abs=1e-12)


def test_row_stats_brute_force():
    y = np.random.default_rng(7).standard_normal((4, 50)) * 4
    s = head.row_stats(y)
    for i in range(4):
        ex = [math.exp(v) for v in y[i]]
        z = sum(ex)
        H = -sum(e / z * math.log(e / z) for e in ex)
        assert abs(s["H"][i] - H) < 1e-12
        best = max(range(50), key=lambda v: (y[i, v], -v))
        assert s["argmax"][i] == best
        assert abs(s["l"][i] - sum(math.exp(v - max(y[i])) for v in y[i])) < 1e-12


# ---------------------------------------------------------------- tail
def test_chunked_tied_logits_equal_the_one_shot_product():
    t = _dense_table(320, 64, seed=8)
    xn = np.random.default_rng(9).standard_normal((5, 64))
    for chunk in (64, 128, 320):
        assert np.allclose(head.tied_logits(xn, t, chunk), xn @ t.dense.T, rtol=0, atol=1e-13)


def test_tail_brute_force():
    V, D, T = 128, 64, 0.7
    t = _dense_table(V, D, seed=10)
    r = np.random.default_rng(11)
    x = r.standard_normal((2, D)) * 3
    w = 1 + 0.1 * r.standard_normal(D)
    got = head.tail(x, w, t, T, eps=1e-6, chunk=64)
    for i in range(2):
        ms = sum(v * v for v in x[i]) / D
        xn = [x[i, d] / math.sqrt(ms + 1e-6) * w[d] for d in range(D)]
        z = [sum(xn[d] * t.dense[v, d] for d in range(D)) for v in range(V)]
        y = [30.0 * math.tanh(zz / 30.0) / T for zz in z]
        m = max(y)
        ex = [math.exp(v - m) for v in y]
        l = sum(ex)
        H = -sum(e / l * math.log(e / l) for e in ex)
        assert np.allclose(got["y"][i], y, rtol=0, atol=1e-12)
        assert abs(got["H"][i] - H) < 1e-12
        assert got["argmax"][i] == y.index(m)


def test_tail_temperature_sharpens():
    t = _dense_table(256, 64, seed=12)
    x = np.random.default_rng(13).standard_normal((3, 64))
    w = np.ones(64)
    hs = [head.tail(x, w, t, T, chunk=64)["H"] for T in (0.8, 0.6, 0.4, 0.05)]
    for a, b in zip(hs, hs[1:]):
        assert np.all(b < a)
    # the argmax does not depend on T
    a = {tuple(head.tail(x, w, t, T, chunk=64)["argmax"]) for T in (0.8, 0.4)}
    assert len(a) == 1


def test_synthetic_tail_rows_span_flat_to_peaked():
    # the drawn workload covers the range of entropies the sampler sees
    cfg = synth.head_config("head_tiny")
    e32 = synth.draw_embed(cfg)
    t = head.EmbedTable.pack_q4(e32)
    hw = synth.draw_head_weights(cfg)
    r = head.tail(synth.draw_tail_x(cfg, e32), hw["final_norm"], t, cfg["T"])
    H = r["H"]
    assert H.max() > 0.8 * math.log(cfg["V"]) and H.min() < 0.05 and np.ptp(r["z"]) < 60


def test_densified_table_is_the_same_table():
    w = np.random.default_rng(14).standard_normal((192, 64)).astype(np.float32)
    t = head.EmbedTable.pack_q4(w, chunk=64)
    d = t.densified(chunk=128)
    assert np.array_equal(d.rows(0, 192), t.rows(0, 192))
