"""Pins of oracle/attention.py against what the pages and the mathematics fix
(closed forms, group properties of the rotation, special cases of the softmax,
and an independent loop-by-loop brute force on tiny shapes)."""
import math

import numpy as np
import pytest

from oracle import attention as oa


def test_rms_unit_and_weight():
    rng = np.random.default_rng(0)
    x = rng.normal(size=(5, 64)) * 3.0
    y = oa.rms(x, eps=0.0)
    assert np.allclose(np.mean(y * y, axis=1), 1.0, atol=1e-12)
    w = rng.normal(size=64)
    assert np.allclose(oa.rms(x, w, eps=0.0), y * w, atol=1e-12)
    # eps inside the root: a zero row stays zero
    assert np.all(oa.rms(np.zeros((1, 8))) == 0.0)


def test_rope_identity_at_position_zero_and_norm_preserving():
    rng = np.random.default_rng(1)
    x = rng.normal(size=(3, 7, 64))
    for n_rot, stride in [(32, 32), (8, 8), (8, 32)]:
        assert np.allclose(oa.rope(x, np.zeros(7), 1e4, n_rot, stride, 64), x, atol=0)
        y = oa.rope(x, np.arange(7) * 13, 1e4, n_rot, stride, 64)
        # each rotated pair keeps its length; unrotated dims are untouched
        for d in range(n_rot):
            assert np.allclose(y[..., d] ** 2 + y[..., d + stride] ** 2,
                               x[..., d] ** 2 + x[..., d + stride] ** 2, atol=1e-12)
        moved = set(range(n_rot)) | set(range(stride, stride + n_rot))
        for d in set(range(64)) - moved:
            assert np.array_equal(y[..., d], x[..., d])


def test_rope_closed_form_pair_zero_and_a_later_pair():
    # pair 0 has frequency 1: e_0 at position p -> cos p at 0, sin p at the partner
    for n_rot, stride in [(32, 32), (8, 8), (8, 32)]:
        e0 = np.zeros((1, 64))
        e0[0, 0] = 1.0
        y = oa.rope(e0, np.array([1.0]), 1e4, n_rot, stride, 64)
        assert abs(y[0, 0] - math.cos(1.0)) < 1e-15 and abs(y[0, stride] - math.sin(1.0)) < 1e-15
        # the partner's own image: (0, 1) -> (-sin, cos)
        e1 = np.zeros((1, 64))
        e1[0, stride] = 1.0
        y = oa.rope(e1, np.array([1.0]), 1e4, n_rot, stride, 64)
        assert abs(y[0, 0] + math.sin(1.0)) < 1e-15 and abs(y[0, stride] - math.cos(1.0)) < 1e-15
    # pair d = den/4 has frequency theta^(-1/2) = 0.01 for theta 1e4: at position 100 the angle is 1
    x = np.zeros((1, 64))
    x[0, 16] = 1.0
    y = oa.rope(x, np.array([100.0]), 1e4, 32, 32, 64)
    assert abs(y[0, 16] - math.cos(1.0)) < 1e-13 and abs(y[0, 48] - math.sin(1.0)) < 1e-13


def test_full_layer_partner_stride_readings():
    # head_dim 512: 64 rotated pairs; [ARCH] pairs d with d + 64, [BLOG] with d + 256
    th, n_rot, s_arch, den, win = oa.layer_params("full", 512, "arch")
    assert (th, n_rot, s_arch, den, win) == (1e6, 64, 64, 512, 0)
    _, _, s_blog, _, _ = oa.layer_params("full", 512, "blog")
    assert s_blog == 256
    assert oa.layer_params("sliding", 256) == (1e4, 128, 128, 256, 1023)
    e0 = np.zeros((1, 512))
    e0[0, 0] = 1.0
    ya = oa.rope(e0, np.array([1.0]), th, n_rot, s_arch, den)
    yb = oa.rope(e0, np.array([1.0]), th, n_rot, s_blog, den)
    assert abs(ya[0, 64] - math.sin(1.0)) < 1e-15 and ya[0, 256] == 0.0
    assert abs(yb[0, 256] - math.sin(1.0)) < 1e-15 and yb[0, 64] == 0.0
    # the last rotated pair's frequency uses the whole head_dim in the exponent
    f = oa.rope_freqs(512, 1e6, 64, 512)
    assert abs(f[63] - 1e6 ** (-126.0 / 512.0)) < 1e-18


def test_rope_relative_position_and_composition():
    rng = np.random.default_rng(2)
    q = rng.normal(size=(1, 64))
    k = rng.normal(size=(1, 64))
    for n_rot, stride in [(32, 32), (8, 8), (8, 32)]:
        def dot(p, r):
            return float(oa.rope(q, np.array([p]), 1e4, n_rot, stride, 64)[0]
                         @ oa.rope(k, np.array([r]), 1e4, n_rot, stride, 64)[0])
        # the score depends on the positions only through their difference
        assert abs(dot(5, 12) - dot(1005, 1012)) < 1e-9
        assert abs(dot(0, 7) - dot(300, 307)) < 1e-9
        # rotations compose: R(a) R(b) = R(a + b)
        x = rng.normal(size=(1, 64))
        two = oa.rope(oa.rope(x, np.array([17.0]), 1e4, n_rot, stride, 64), np.array([25.0]),
                      1e4, n_rot, stride, 64)
        assert np.allclose(two, oa.rope(x, np.array([42.0]), 1e4, n_rot, stride, 64), atol=1e-12)


def _cache(Hkv, n, hd, seed):
    rng = np.random.default_rng(seed)
    return rng.normal(size=(Hkv, n, hd)), rng.normal(size=(Hkv, n, hd))


def test_attend_single_key_returns_its_value():
    rng = np.random.default_rng(3)
    q = rng.normal(size=(2, 1, 16))
    k = rng.normal(size=(1, 1, 16))
    v = rng.normal(size=(1, 1, 16))
    kc, vc = np.zeros((1, 0, 16)), np.zeros((1, 0, 16))
    out = oa.attend(q, k, v, kc, vc, 0, 0)
    assert np.allclose(out[0, :16], v[0, 0]) and np.allclose(out[0, 16:], v[0, 0])


def test_attend_zero_query_averages_exactly_the_visible_keys():
    H, Hkv, L, hd, kv_len, window = 4, 2, 3, 8, 50, 20
    kc, vc = _cache(Hkv, 64, hd, 4)
    rng = np.random.default_rng(5)
    k, v = rng.normal(size=(Hkv, L, hd)), rng.normal(size=(Hkv, L, hd))
    q = np.zeros((H, L, hd))
    for win, s0 in [(window, kv_len - window), (0, 0), (1000, 0)]:
        out = oa.attend(q, k, v, kc, vc, kv_len, win)
        for h in range(H):
            n = h // 2
            mean = np.concatenate([vc[n, s0:kv_len], v[n]]).mean(axis=0)
            for t in range(L):
                assert np.allclose(out[t, h * hd:(h + 1) * hd], mean, atol=1e-12)


def test_attend_masked_keys_have_no_effect_and_visible_ones_do():
    H, Hkv, L, hd, kv_len, window = 2, 1, 2, 8, 30, 10
    kc, vc = _cache(Hkv, 40, hd, 6)
    rng = np.random.default_rng(7)
    q = rng.normal(size=(H, L, hd))
    k, v = rng.normal(size=(Hkv, L, hd)), rng.normal(size=(Hkv, L, hd))
    base = oa.attend(q, k, v, kc, vc, kv_len, window)
    kc2, vc2 = kc.copy(), vc.copy()
    kc2[0, :kv_len - window] = 50.0 * q[0, 0]     # would dominate if it were visible
    vc2[0, :kv_len - window] = 1e6
    kc2[0, kv_len:] = 50.0 * q[0, 0]              # past kv_len: not committed, never read
    vc2[0, kv_len:] = 1e6
    assert np.array_equal(oa.attend(q, k, v, kc2, vc2, kv_len, window), base)
    kc3 = kc.copy()
    kc3[0, kv_len - window] = 50.0 * q[0, 0]      # the first visible position
    assert not np.allclose(oa.attend(q, k, v, kc3, vc, kv_len, window), base)


def test_attend_two_keys_closed_form_and_gqa_mapping():
    # one committed key and one canvas key: weight of the first = 1 / (1 + e^(s2 - s1))
    hd = 4
    q = np.array([[[1.0, 0.0, 0.0, 0.0]]] * 4)            # 4 heads, 1 row
    kc = np.array([[[2.0, 0, 0, 0]], [[-1.0, 0, 0, 0]]])  # kv heads 0, 1
    vc = np.array([[[1.0, 0, 0, 0]], [[0, 1.0, 0, 0]]])
    k = np.array([[[0.5, 0, 0, 0]], [[0.5, 0, 0, 0]]])
    v = np.array([[[0, 0, 1.0, 0]], [[0, 0, 0, 1.0]]])
    out = oa.attend(q, k, v, kc, vc, 1, 0)
    w0 = 1.0 / (1.0 + math.exp(0.5 - 2.0))
    w1 = 1.0 / (1.0 + math.exp(0.5 - (-1.0)))
    # heads 0, 1 read kv head 0; heads 2, 3 kv head 1 (h // (H / Hkv))
    for h in range(4):
        o = out[0, h * hd:(h + 1) * hd]
        if h < 2:
            assert np.allclose(o, [w0, 0, 1 - w0, 0], atol=1e-15)
        else:
            assert np.allclose(o, [0, w1, 0, 1 - w1], atol=1e-15)


def _brute(qraw, kraw, vraw, w_q, w_k, kc, vc, kv_len, H, Hkv, hd, theta, n_rot, stride, den,
           window, eps):
    """Element by element, with Python loops and the math module."""
    L = len(qraw)
    G = H // Hkv

    def norm(vec, w):
        ms = sum(x * x for x in vec) / len(vec)
        r = 1.0 / math.sqrt(ms + eps)
        return [x * r * (1.0 if w is None else w[i]) for i, x in enumerate(vec)]

    def rot(vec, p):
        out = list(vec)
        for d in range(n_rot):
            a = p * theta ** (-2.0 * d / den)
            x0, x1 = vec[d], vec[d + stride]
            out[d] = x0 * math.cos(a) - x1 * math.sin(a)
            out[d + stride] = x1 * math.cos(a) + x0 * math.sin(a)
        return out

    s0 = max(0, kv_len - window) if window > 0 else 0
    res = [[0.0] * (H * hd) for _ in range(L)]
    for h in range(H):
        n = h // G
        keys, vals = [], []
        for j in range(s0, kv_len):
            keys.append(list(kc[n][j]))
            vals.append(list(vc[n][j]))
        for t in range(L):
            kr = list(kraw[t][n * hd:(n + 1) * hd])
            keys.append(rot(norm(kr, w_k), kv_len + t))
            src = kr if vraw is None else list(vraw[t][n * hd:(n + 1) * hd])
            vals.append(norm(src, None))
        for t in range(L):
            qv = rot(norm(list(qraw[t][h * hd:(h + 1) * hd]), w_q), kv_len + t)
            sc = [sum(qv[d] * key[d] for d in range(hd)) for key in keys]
            m = max(sc)
            e = [math.exp(s - m) for s in sc]
            z = sum(e)
            for d in range(hd):
                res[t][h * hd + d] = sum(e[j] * vals[j][d] for j in range(len(keys))) / z
    return np.array(res)


@pytest.mark.parametrize("kind,reading,window", [("sliding", "arch", 6), ("full", "arch", 0),
                                                 ("full", "blog", 0)])
def test_denoise_attention_equals_brute_force(kind, reading, window):
    rng = np.random.default_rng(8)
    H, Hkv, L, hd, kv_len = 4, 2, 5, 16, 9
    qraw = rng.normal(size=(L, H * hd))
    kraw = rng.normal(size=(L, Hkv * hd))
    vraw = None if kind == "full" else rng.normal(size=(L, Hkv * hd))
    w_q, w_k = rng.normal(size=hd) * 0.6, rng.normal(size=hd) * 0.6
    kc, vc = _cache(Hkv, 12, hd, 9)
    theta, n_rot, stride, den, _ = oa.layer_params(kind, hd, reading)
    if kind == "sliding":
        # the page's window is 1023; a small one here so that it cuts the tiny cache
        q, k, v = oa.canvas_qkv(qraw, kraw, vraw, w_q, w_k, kv_len, H, Hkv, hd, theta, n_rot,
                                stride, den)
        got = oa.attend(q, k, v, kc, vc, kv_len, window)
    else:
        got = oa.denoise_attention(qraw, kraw, vraw, w_q, w_k, kc, vc, kv_len, H, Hkv, hd, kind,
                                   reading)
    ref = _brute(qraw.tolist(), kraw.tolist(), None if vraw is None else vraw.tolist(), w_q, w_k,
                 kc.tolist(), vc.tolist(), kv_len, H, Hkv, hd, theta, n_rot, stride, den, window,
                 1e-6)
    assert np.allclose(got, ref, atol=1e-11, rtol=1e-11)


def test_full_layer_value_is_the_normalised_raw_key_projection():
    rng = np.random.default_rng(10)
    H, Hkv, L, hd = 2, 1, 3, 16
    qraw, kraw = rng.normal(size=(L, H * hd)), rng.normal(size=(L, Hkv * hd))
    w = rng.normal(size=hd)
    th, n_rot, stride, den, _ = oa.layer_params("full", hd)
    q, k, v = oa.canvas_qkv(qraw, kraw, None, w, w, 4, H, Hkv, hd, th, n_rot, stride, den)
    _, _, v2 = oa.canvas_qkv(qraw, kraw, kraw, w, w, 4, H, Hkv, hd, th, n_rot, stride, den)
    assert np.array_equal(v, v2)
    assert np.allclose(np.mean(v * v, axis=-1), 1.0, atol=1e-5)   # unit rms, no weight, no RoPE
    kc, vc = oa.encoder_cache(kraw, None, w, Hkv, hd, th, n_rot, stride, den)
    assert np.array_equal(vc, v)                                   # positions do not touch v
    assert np.allclose(kc[:, 0], oa.rms(kraw[0].reshape(Hkv, hd), w))  # position 0: no turn
