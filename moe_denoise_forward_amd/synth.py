"""Seeded synthetic inputs for the MoE FFN block (no part of the block's arithmetic).

Both the GPU path and the CPU oracle consume what this module draws; it only
draws random numbers and rounds activations/weights to the storage type the
workload names (bf16).  Quantisation is NOT done here: each side packs the
float32 weights with its own packer.

Shapes are one decoder layer of DiffusionGemma-26B-A4B (hidden 2816, 128
experts, top-8, expert FF 704, dense FF 2112, canvas 256, eps 1e-6; diffgemma
"architecture & implemented contract" Part II section 1 "Model constants", and
the mlx-bun port's dossier section 1 config table).  There is no checkpoint in
reach, so every tensor is drawn:
  x                   N(0, 1)                        [L, D]   (bf16-rounded for bf16 workloads)
  router              N(0, 1/sqrt(D))                [E, D]
  router_scale        1 + N(0, 0.1)                  [D]
  per_expert_scale    1 + N(0, 0.1)                  [E]
  expert_gate_up      N(0, 1/sqrt(D))                [E, 2I, D]
  expert_down         N(0, 1/sqrt(I))                [E, D, I]
  dense_gate_up       N(0, 1/sqrt(D))                [2I_d, D]
  dense_down          N(0, 1/sqrt(I_d))              [D, I_d]
  five norm weights   1 + N(0, 0.1)                  [D]
  layer_scalar        0.5
  router_bias         zipf only: -s * ln(rank_e), rank a seeded permutation of 1..E
The second argument of N is the standard deviation.  Every tensor has its own
stream keyed by (seed, layer, tensor id), and each expert's two matrices by
(seed, layer, tensor id, expert), so a layer, a tensor or one expert can be
redrawn alone.
"""
from concurrent.futures import ThreadPoolExecutor

import numpy as np

# name -> workload description
CONFIGS = {
    # tiny block, fp32 activations, q4 experts + dense, fp32 router
    "tiny": dict(L=32, D=128, E=8, k=2, I=64, Id=128, x_dtype="f32", weight_fmt="q4",
                 router_fmt="f32", layers=1, zipf=None, seed=0),
    # one full-size block, unquantised bf16 weights, fp32 router
    "canvas256_bf16": dict(L=256, D=2816, E=128, k=8, I=704, Id=2112, x_dtype="bf16",
                           weight_fmt="bf16", router_fmt="f32", layers=1, zipf=None, seed=1),
    # the same block with q4 group-64 experts + dense MLP and a q8 group-64 router
    "canvas256_q4": dict(L=256, D=2816, E=128, k=8, I=704, Id=2112, x_dtype="bf16",
                         weight_fmt="q4", router_fmt="q8", layers=1, zipf=None, seed=2),
    # 8 canvases x 256 positions through the q4 block
    "batch2048_q4": dict(L=2048, D=2816, E=128, k=8, I=704, Id=2112, x_dtype="bf16",
                         weight_fmt="q4", router_fmt="q8", layers=1, zipf=None, seed=3),
    # 30 independent q4 blocks applied in sequence, Zipf(1.1)-skewed router
    "stack30_zipf_q4": dict(L=256, D=2816, E=128, k=8, I=704, Id=2112, x_dtype="bf16",
                            weight_fmt="q4", router_fmt="q8", layers=30, zipf=1.1, seed=4),
    # test shapes: several tiles plus ragged tails, oracle finishes in seconds
    "mid": dict(L=100, D=256, E=16, k=4, I=128, Id=192, x_dtype="bf16", weight_fmt="q4",
                router_fmt="q8", layers=1, zipf=None, seed=11),
    "mid_bf16": dict(L=77, D=192, E=12, k=3, I=64, Id=128, x_dtype="bf16", weight_fmt="bf16",
                     router_fmt="f32", layers=1, zipf=None, seed=12),
    # many pairs per expert (tall-tile GEMMs): ~150 rows per expert over 64-row
    # tiles, odd block counts in every matrix (half column tiles), K of 5 groups
    "tall": dict(L=300, D=320, E=4, k=2, I=192, Id=320, x_dtype="bf16", weight_fmt="q4",
                 router_fmt="q8", layers=1, zipf=None, seed=13),
    # tall tiles with fp32 activations, an expert count that is not a multiple
    # of the router's 16-expert tiles, odd k
    "tall_f32": dict(L=260, D=384, E=6, k=3, I=128, Id=192, x_dtype="f32", weight_fmt="q4",
                     router_fmt="f32", layers=1, zipf=None, seed=15),
    # the largest expert count and top-k the library takes (four router keys per
    # lane, choices in 32 lanes), a ragged number of positions
    "max_experts": dict(L=70, D=512, E=256, k=32, I=64, Id=64, x_dtype="bf16", weight_fmt="q4",
                        router_fmt="q8", layers=1, zipf=None, seed=16),
    # the largest hidden size (the router scale fills the front kernel's LDS,
    # 1024 combine threads per row)
    "max_hidden": dict(L=20, D=8192, E=4, k=2, I=64, Id=64, x_dtype="bf16", weight_fmt="q4",
                       router_fmt="q8", layers=1, zipf=None, seed=17),
    # short q4 tiles past two rounds of the persistent grid (~1160 gate_up
    # tiles, K of 16 groups), tiles of 16 rows and fewer among them
    "short_many": dict(L=128, D=1024, E=64, k=8, I=1024, Id=512, x_dtype="bf16", weight_fmt="q4",
                       router_fmt="q8", layers=1, zipf=None, seed=18),
    # tall tiles, several per workgroup: 16384 positions through four experts,
    # down K of three groups (tiles of four stream positions)
    "tall_many": dict(L=16384, D=512, E=4, k=2, I=192, Id=320, x_dtype="bf16", weight_fmt="q4",
                      router_fmt="q8", layers=1, zipf=None, seed=14),
    # the diffgemma contract's own pack (section 8 "Quantization (.dgq)"): q4
    # group-32 experts, the dense MLP and the router unquantised bf16
    "canvas256_q4g32": dict(L=256, D=2816, E=128, k=8, I=704, Id=2112, x_dtype="bf16",
                            weight_fmt="q4g32", dense_fmt="bf16", router_fmt="bf16", layers=1,
                            zipf=None, seed=5),
    # q4 group-32 at test sizes: experts and dense MLP in it; then the contract's
    # split (dense bf16), and a q4 group-64 dense MLP beside q4 group-32 experts
    "tiny_g32": dict(L=32, D=128, E=8, k=2, I=64, Id=128, x_dtype="f32", weight_fmt="q4g32",
                     router_fmt="f32", layers=1, zipf=None, seed=20),
    "mid_g32": dict(L=100, D=256, E=16, k=4, I=128, Id=192, x_dtype="bf16", weight_fmt="q4g32",
                    dense_fmt="bf16", router_fmt="bf16", layers=1, zipf=None, seed=21),
    "mid_g32_q4dense": dict(L=90, D=320, E=12, k=3, I=192, Id=256, x_dtype="bf16",
                            weight_fmt="q4g32", dense_fmt="q4", router_fmt="q8", layers=1,
                            zipf=None, seed=22),
    # the OptiQ checkpoint's mix (the mlx-bun dossier, section 1 weight schema):
    # q4 group-64 experts, 8-bit group-64 dense MLP and router
    "canvas256_optiq": dict(L=256, D=2816, E=128, k=8, I=704, Id=2112, x_dtype="bf16",
                            weight_fmt="q4", dense_fmt="q8", router_fmt="q8", layers=1,
                            zipf=None, seed=6),
    "mid_q8dense": dict(L=100, D=256, E=16, k=4, I=128, Id=192, x_dtype="bf16", weight_fmt="q4",
                        dense_fmt="q8", router_fmt="q8", layers=1, zipf=None, seed=24),
    "tiny_g32_q8dense": dict(L=32, D=128, E=8, k=2, I=64, Id=128, x_dtype="f32",
                             weight_fmt="q4g32", dense_fmt="q8", router_fmt="f32", layers=1,
                             zipf=None, seed=25),
    # nvfp4 experts (the contract's nvfp4x profile: experts nvfp4 beside its
    # unquantised bf16 dense MLP and router)
    "canvas256_nvfp4": dict(L=256, D=2816, E=128, k=8, I=704, Id=2112, x_dtype="bf16",
                            weight_fmt="nvfp4", dense_fmt="bf16", router_fmt="bf16", layers=1,
                            zipf=None, seed=7),
    "tiny_nvfp4": dict(L=32, D=128, E=8, k=2, I=64, Id=128, x_dtype="f32", weight_fmt="nvfp4",
                       router_fmt="f32", layers=1, zipf=None, seed=26),
    "mid_nvfp4": dict(L=100, D=256, E=16, k=4, I=128, Id=192, x_dtype="bf16", weight_fmt="nvfp4",
                      dense_fmt="bf16", router_fmt="bf16", layers=1, zipf=None, seed=27),
    # q6 experts (the contract's q6 profile: 6-bit group-32 experts beside its
    # unquantised bf16 dense MLP and router)
    "canvas256_q6": dict(L=256, D=2816, E=128, k=8, I=704, Id=2112, x_dtype="bf16",
                         weight_fmt="q6", dense_fmt="bf16", router_fmt="bf16", layers=1,
                         zipf=None, seed=8),
    "tiny_q6": dict(L=32, D=128, E=8, k=2, I=64, Id=128, x_dtype="f32", weight_fmt="q6",
                    router_fmt="f32", layers=1, zipf=None, seed=28),
    "mid_q6": dict(L=100, D=256, E=16, k=4, I=128, Id=192, x_dtype="bf16", weight_fmt="q6",
                   dense_fmt="bf16", router_fmt="bf16", layers=1, zipf=None, seed=29),
    # q4 group-64 experts beside a bf16 dense MLP (the other way round)
    "mid_q4_bf16dense": dict(L=64, D=256, E=8, k=2, I=128, Id=320, x_dtype="f32",
                             weight_fmt="q4", dense_fmt="bf16", router_fmt="f32", layers=1,
                             zipf=None, seed=23),
}


def dense_fmt(cfg):
    """The dense MLP's weight format: its own if the workload names one, else
    the experts' (weight_fmt)."""
    return cfg.get("dense_fmt") or cfg["weight_fmt"]

_TENSOR_IDS = {
    "x": 0, "router": 1, "router_scale": 2, "per_expert_scale": 3,
    "expert_gate_up": 4, "expert_down": 5, "dense_gate_up": 6, "dense_down": 7,
    "pre_ff_norm": 8, "pre_ff_norm_2": 9, "post_ff_norm_1": 10, "post_ff_norm_2": 11,
    "post_ff_norm": 12, "router_bias": 13,
}
NORM_NAMES = ("pre_ff_norm", "pre_ff_norm_2", "post_ff_norm_1", "post_ff_norm_2", "post_ff_norm")


def round_bf16(a):
    """Round float32 values to the nearest bfloat16 (ties to even), kept as float32."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32).reshape(a.shape)


def _rng(seed, layer, name, sub=None):
    key = [int(seed), int(layer), _TENSOR_IDS[name]]
    if sub is not None:
        key.append(int(sub))
    return np.random.default_rng(key)


def _normal(seed, layer, name, shape, std, sub=None):
    r = _rng(seed, layer, name, sub)
    out = r.standard_normal(shape, dtype=np.float32)
    out *= np.float32(std)
    return out


def _one_plus(seed, layer, name, n):
    return np.float32(1.0) + _normal(seed, layer, name, (n,), 0.1)


def config(name, **override):
    c = dict(CONFIGS[name])
    c.update(override)
    c["name"] = name
    return c


def draw_x(cfg, layer=0):
    x = _normal(cfg["seed"], layer, "x", (cfg["L"], cfg["D"]), 1.0)
    return round_bf16(x) if cfg["x_dtype"] == "bf16" else x


def draw_expert(cfg, e, layer=0):
    """float32 (gate_up [2I, D], down [D, I]) of expert e; each expert has its own stream."""
    D, I = cfg["D"], cfg["I"]
    gu = _normal(cfg["seed"], layer, "expert_gate_up", (2 * I, D), D ** -0.5, sub=e)
    dn = _normal(cfg["seed"], layer, "expert_down", (D, I), I ** -0.5, sub=e)
    if cfg["weight_fmt"] == "bf16":
        gu, dn = round_bf16(gu), round_bf16(dn)
    return gu, dn


def draw_weights(cfg, layer=0, experts=True):
    """float32 weights of one block.  experts=False skips the two big expert
    tensors (callers that draw them expert by expert use draw_expert)."""
    s, L, D, E, I, Id = cfg["seed"], layer, cfg["D"], cfg["E"], cfg["I"], cfg["Id"]
    w = {}
    w["router"] = _normal(s, L, "router", (E, D), D ** -0.5)
    w["router_scale"] = _one_plus(s, L, "router_scale", D)
    w["per_expert_scale"] = _one_plus(s, L, "per_expert_scale", E)
    if experts:
        w["expert_gate_up"] = np.empty((E, 2 * I, D), np.float32)
        w["expert_down"] = np.empty((E, D, I), np.float32)

        def fill(e):
            w["expert_gate_up"][e], w["expert_down"][e] = draw_expert(cfg, e, layer)

        with ThreadPoolExecutor(max_workers=8) as ex:
            list(ex.map(fill, range(E)))
    w["dense_gate_up"] = _normal(s, L, "dense_gate_up", (2 * Id, D), D ** -0.5)
    w["dense_down"] = _normal(s, L, "dense_down", (D, Id), Id ** -0.5)
    for n in NORM_NAMES:
        w[n] = _one_plus(s, L, n, D)
    w["layer_scalar"] = 0.5
    w["router_bias"] = None
    if cfg.get("zipf"):
        rank = _rng(s, L, "router_bias").permutation(E).astype(np.float64) + 1.0
        w["router_bias"] = (-float(cfg["zipf"]) * np.log(rank)).astype(np.float32)
    if dense_fmt(cfg) == "bf16":
        for n in ("dense_gate_up", "dense_down"):
            w[n] = round_bf16(w[n])
    if cfg["router_fmt"] == "bf16":
        w["router"] = round_bf16(w["router"])
    return w


# ---------------------------------------------------------------- canvas head
# The two ends of a denoising forward that read the tied embedding table:
# the self-conditioned canvas input and the forward tail.  Shapes: hidden
# 2816, vocabulary 262144, the self-conditioning MLP of the dense MLP's shape
# (intermediate 2112), canvas 256 (the diffgemma contract, Part II section 1;
# the mlx-bun dossier section 3 "Self-conditioning"); the sampler's
# temperature schedule runs from 0.8 down to 0.4 (Part II section 1, sampler
# config), so the tail is drawn at T = 0.6 (full size) and at the two ends.
#   embed         N(0, 1/sqrt(D))                      [V, D]  drawn in row blocks of 8192
#   final_norm    1 + N(0, 0.1)                         [D]
#   sc_pre_norm   1 + N(0, 0.1)                         [D]
#   sc_gate_up    N(0, 1/sqrt(D))                       [2 I_sc, D]
#   sc_down       N(0, 1/sqrt(I_sc))                    [D, I_sc]
#   canvas_ids    uniform over [0, V)                   [L]
#   tail_x        N(0, 1) + beta_t * embed[v_t] / std   [L, D]  beta_t cycles through
#                 0, .02, .05, .1, .2, .5, 1, 3 so the rows span flat to one-hot
#                 predictions; v_t uniform (bf16-rounded for bf16 workloads)
#   sc_logits     N(0, sigma_t) + spike_t at v_t         [L, V]  (sigma, spike) cycles
#                 through (1,0) (3,0) (8,0) (.3,0) (1,5) (2,20) (3,60) (.5,10)
HEAD_CONFIGS = {
    "head_tiny": dict(L=32, D=128, V=4096, Isc=128, T=0.6, x_dtype="f32", seed=20),
    # ragged: 100 rows, 65 blocks of 64 vocabulary rows, K of 4 groups
    "head_mid": dict(L=100, D=256, V=4160, Isc=192, T=0.4, x_dtype="bf16", seed=21),
    # more than one 256-row canvas, odd vocabulary blocks, K of 5 groups
    "head_rows": dict(L=300, D=320, V=8256, Isc=320, T=0.8, x_dtype="f32", seed=23),
    "head_full": dict(L=256, D=2816, V=262144, Isc=2112, T=0.6, x_dtype="bf16", seed=22),
}
EMBED_CHUNK = 8192
_TENSOR_IDS.update({"embed": 14, "final_norm": 15, "sc_pre_norm": 16, "sc_gate_up": 17,
                    "sc_down": 18, "canvas_ids": 19, "tail_x": 20, "tail_pick": 21,
                    "sc_logits": 22, "sc_pick": 23})
TAIL_BETA = (0.0, 0.02, 0.05, 0.1, 0.2, 0.5, 1.0, 3.0)
SC_SHAPE = ((1.0, 0.0), (3.0, 0.0), (8.0, 0.0), (0.3, 0.0), (1.0, 5.0), (2.0, 20.0),
            (3.0, 60.0), (0.5, 10.0))


def head_config(name, **override):
    c = dict(HEAD_CONFIGS[name])
    c.update(override)
    c["name"] = name
    return c


def embed_std(cfg):
    return 1.0 / cfg["D"] ** 0.5


def draw_embed(cfg):
    """float32 table [V, D], one stream per block of EMBED_CHUNK rows."""
    V, D = cfg["V"], cfg["D"]
    out = np.empty((V, D), np.float32)
    starts = list(range(0, V, EMBED_CHUNK))

    def fill(i):
        lo = starts[i]
        hi = min(V, lo + EMBED_CHUNK)
        out[lo:hi] = _normal(cfg["seed"], 0, "embed", (hi - lo, D), embed_std(cfg), sub=i)

    with ThreadPoolExecutor(max_workers=8) as ex:
        list(ex.map(fill, range(len(starts))))
    return out


def draw_head_weights(cfg):
    s, D, I = cfg["seed"], cfg["D"], cfg["Isc"]
    return {
        "final_norm": _one_plus(s, 0, "final_norm", D),
        "sc_pre_norm": _one_plus(s, 0, "sc_pre_norm", D),
        "sc_gate_up": _normal(s, 0, "sc_gate_up", (2 * I, D), D ** -0.5),
        "sc_down": _normal(s, 0, "sc_down", (D, I), I ** -0.5),
    }


def draw_canvas_ids(cfg):
    return _rng(cfg["seed"], 0, "canvas_ids").integers(0, cfg["V"], cfg["L"]).astype(np.int32)


def draw_tail_x(cfg, embed):
    """The last block's output: noise plus a per-row share of one table row."""
    L, D, V = cfg["L"], cfg["D"], cfg["V"]
    x = _normal(cfg["seed"], 0, "tail_x", (L, D), 1.0)
    pick = _rng(cfg["seed"], 0, "tail_pick").integers(0, V, L)
    beta = np.array([TAIL_BETA[t % len(TAIL_BETA)] for t in range(L)], np.float32)
    x += beta[:, None] * embed[pick] * np.float32(1.0 / embed_std(cfg))
    return round_bf16(x) if cfg["x_dtype"] == "bf16" else x


def draw_sc_logits(cfg):
    """The previous step's logits (already divided by the temperature)."""
    L, V = cfg["L"], cfg["V"]
    y = _normal(cfg["seed"], 0, "sc_logits", (L, V), 1.0)
    pick = _rng(cfg["seed"], 0, "sc_pick").integers(0, V, L)
    for t in range(L):
        sigma, spike = SC_SHAPE[t % len(SC_SHAPE)]
        y[t] *= np.float32(sigma)
        y[t, pick[t]] += np.float32(spike)
    return y


# ---------------------------------------------------------------- denoise attention
# One layer's canvas attention at the pages' two layer shapes (16 query heads;
# sliding layers 8 KV heads of 256 with a window of 1023 committed positions,
# full layers 2 KV heads of 512), a 256-row canvas after a committed prompt of
# kv_len positions, plus small ragged shapes whose window cuts the cache.
ATTN_CONFIGS = {
    "attn_tiny_sliding": dict(L=16, kv_len=40, H=4, Hkv=2, hd=64, kind="sliding", window=24,
                              x_dtype="f32", seed=30),
    "attn_tiny_full": dict(L=16, kv_len=40, H=4, Hkv=1, hd=128, kind="full", window=0,
                           x_dtype="f32", seed=31),
    "attn_mid_sliding": dict(L=100, kv_len=300, H=16, Hkv=8, hd=256, kind="sliding", window=200,
                             x_dtype="bf16", seed=32),
    "attn_mid_full": dict(L=100, kv_len=300, H=16, Hkv=2, hd=512, kind="full", window=0,
                          x_dtype="bf16", seed=33),
    "attn_sliding": dict(L=256, kv_len=4096, H=16, Hkv=8, hd=256, kind="sliding", window=1023,
                         x_dtype="bf16", seed=34),
    "attn_full": dict(L=256, kv_len=4096, H=16, Hkv=2, hd=512, kind="full", window=0,
                      x_dtype="bf16", seed=35),
}
_TENSOR_IDS.update({"attn_q": 24, "attn_k": 25, "attn_v": 26, "attn_qn": 27, "attn_kn": 28,
                    "attn_kc": 29, "attn_vc": 30, "attn_shared": 31})
ATTN_CACHE_SLACK = 8   # cache rows past kv_len, filled with values no row may read


def attn_config(name, **override):
    c = dict(ATTN_CONFIGS[name])
    c.update(override)
    c["name"] = name
    return c


def draw_attn(cfg):
    """Inputs of one layer's canvas attention.

    qraw [L, H*hd], kraw / vraw [L, Hkv*hd] (vraw None on full layers): the
    raw projections, N(0, 1) per element plus one shared N(0, 0.5) vector per
    canvas row added to every head of q and k (rows then lean toward each
    other); bf16-rounded when x_dtype is bf16.  w_q, w_k [hd]: the QK-norm
    weights, a * (1 + N(0, 0.1)) with a = sqrt(2) * hd^-1/4, so that a score
    q . k of independent rows has a standard deviation of about 2.  The
    committed cache, fp16 [Hkv, kv_len + ATTN_CACHE_SLACK, hd]: keys N(0, a),
    values N(0, 1); rows at and past kv_len hold 1e4 (never read)."""
    s, L, H, Hkv, hd, kv = cfg["seed"], cfg["L"], cfg["H"], cfg["Hkv"], cfg["hd"], cfg["kv_len"]
    shared = _normal(s, 0, "attn_shared", (L, 1, hd), 0.5)
    q = (_normal(s, 0, "attn_q", (L, H, hd), 1.0) + shared).reshape(L, H * hd)
    k = (_normal(s, 0, "attn_k", (L, Hkv, hd), 1.0) + shared).reshape(L, Hkv * hd)
    v = None if cfg["kind"] == "full" else _normal(s, 0, "attn_v", (L, Hkv * hd), 1.0)
    if cfg["x_dtype"] == "bf16":
        q, k = round_bf16(q), round_bf16(k)
        v = None if v is None else round_bf16(v)
    a = np.float32(np.sqrt(2.0) * hd ** -0.25)
    w_q = a * (np.float32(1.0) + _normal(s, 0, "attn_qn", (hd,), 0.1))
    w_k = a * (np.float32(1.0) + _normal(s, 0, "attn_kn", (hd,), 0.1))
    cap = kv + ATTN_CACHE_SLACK
    kc = _normal(s, 0, "attn_kc", (Hkv, cap, hd), float(a)).astype(np.float16)
    vc = _normal(s, 0, "attn_vc", (Hkv, cap, hd), 1.0).astype(np.float16)
    kc[:, kv:] = np.float16(1e4)
    vc[:, kv:] = np.float16(1e4)
    return dict(qraw=q, kraw=k, vraw=v, w_q=w_q.astype(np.float32), w_k=w_k.astype(np.float32),
                k_cache=kc, v_cache=vc)
