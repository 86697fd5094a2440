"""GPU parity: the HIP library (through its C ABI) against the oracle.

Bars (per the block's contract):
  * packing and unpacking: bit-exact;
  * router: top-k indices bit-exact except at positions whose k-th/(k+1)-th
    logit margin (oracle, float64) is below 1e-4; weights within 1e-5 relative;
  * block / experts output: max|diff| <= 1e-2 * rms(ref) (fp16 MFMA operands,
    fp32 accumulation; the tolerance derivation is in the design notes), with a
    position skipped only where its routing legitimately differs.
"""
import numpy as np
import pytest

from oracle import block as oblock
from oracle import fp4, prepare, quant
from moe_denoise_forward_amd import synth

from gpu_util import (MARGIN, TOL, block_case, gpu_block, gpu_moe_ffn, gpu_route, rel_err,
                      routing_agrees, say, torch_dev)

pytestmark = pytest.mark.gpu


def _dg():
    from moe_denoise_forward_amd import dgmoe
    return dgmoe


# ------------------------------------------------------------------ pack / unpack
def _edge_matrix(rows, cols, seed):
    rng = np.random.default_rng(seed)
    w = (rng.standard_normal((rows, cols)) * 0.05).astype(np.float32)
    w[0, :64] = 0.3                      # constant group -> scale 0
    w[1, :64] = 0.0
    w[1, 64:128] = -0.0                  # signed zeros
    w[2, :64] = np.linspace(-1000, 1000, 64)   # wide range
    w[3, :64] = np.linspace(0, 64 * 2.0 ** -30, 64)  # subnormal fp16 scale
    w[4, -64:] = rng.standard_normal(64).astype(np.float32) * 100
    w[5, :64] = np.float32(1e-7) * np.arange(64)
    return w


@pytest.mark.parametrize("fmt,shape", [("q4", (64, 64)), ("q4", (192, 320)), ("q4", (320, 2816)),
                                       ("q4g32", (64, 64)), ("q4g32", (192, 448)),
                                       ("q4g32", (1408, 2816)),
                                       ("nvfp4", (64, 64)), ("nvfp4", (192, 448)),
                                       ("nvfp4", (1408, 2816)),
                                       ("q6", (64, 64)), ("q6", (192, 448)), ("q6", (1408, 2816)),
                                       ("q8", (7, 64)), ("q8", (33, 320)), ("q8", (300, 2816))])
def test_pack_is_bit_exact(fmt, shape):
    torch = torch_dev()
    dg = _dg()
    w = _edge_matrix(*shape, seed=shape[0])
    say("pack", fmt, shape)
    m = dg.device_matrix(w, fmt)
    torch.cuda.synchronize()
    if fmt == "nvfp4":
        codes, sbuf = fp4.pack(w)
        assert (m.data.cpu().numpy() == codes.view(np.uint8).reshape(-1)).all()
        got = m.scale_bias.cpu().numpy().view(np.uint8)
        assert got.size == sbuf.size
        bad = np.nonzero(got != sbuf)[0]
        assert bad.size == 0, (bad[:8], got[bad[:8]], sbuf[bad[:8]])
        return
    codes, sb = quant.pack(w, fmt)
    assert (m.data.cpu().numpy() == codes.view(np.uint8).reshape(-1)).all()
    assert (m.scale_bias.cpu().numpy().view(np.uint16) == sb.reshape(-1)).all()


@pytest.mark.parametrize("fmt", ["q4", "q8", "q4g32", "nvfp4", "q6"])
def test_unpack_is_bit_exact(fmt):
    torch = torch_dev()
    dg = _dg()
    rows, cols = (65 if fmt == "q8" else 128), 448
    w = _edge_matrix(rows, cols, seed=3)
    m = dg.device_matrix(w, fmt)
    out32 = torch.empty((rows, cols), dtype=torch.float32, device="cuda")
    out16 = torch.empty((rows, cols), dtype=torch.float16, device="cuda")
    dg.dgmoe_unpack(m.data, m.scale_bias, rows, cols, dg.FMT[fmt], dg.DGMOE_F32, out32)
    dg.dgmoe_unpack(m.data, m.scale_bias, rows, cols, dg.FMT[fmt], dg.DGMOE_F16, out16)
    torch.cuda.synchronize()
    if fmt == "nvfp4":
        codes, sbuf = fp4.pack(w)
        exact = fp4.unpack(codes, sbuf, rows, cols)  # float64, exact
        r16 = exact.astype(np.float32).astype(np.float16).view(np.uint16)  # via fp32, as documented
    else:
        codes, sb = quant.pack(w, fmt)
        exact = quant.unpack(codes, sb, fmt, rows, cols)  # float64, exact
        r16 = exact.astype(np.float16).view(np.uint16)
    assert (out32.cpu().numpy() == exact.astype(np.float32)).all()
    g16 = out16.cpu().numpy().view(np.uint16)
    assert (g16 == r16).all(), np.argwhere(g16 != r16)[:5]


# ------------------------------------------------------------------ router
@pytest.mark.parametrize("name", ["tiny", "mid", "mid_bf16"])
def test_route_parity(name):
    dg = _dg()
    cfg, w32, x = block_case(name)
    say("route", name)
    pb = dg.PackedBlock(w32, cfg)
    idx, w, lg = gpu_route(pb, x, cfg)
    wt = prepare.block_weights(w32, cfg)
    ref = oblock.route(x, wt["router"], wt["router_scale"], wt["per_expert_scale"], cfg["k"],
                       1e-6, wt["router_bias"])
    assert np.max(np.abs(lg - ref["z"])) <= 1e-5 * max(1.0, np.max(np.abs(ref["z"])))
    same = routing_agrees(idx, ref["idx"], ref["margin"])
    assert np.allclose(w[same], ref["w"][same], rtol=1e-5, atol=1e-7)


def test_route_ragged_experts_and_k_equals_e():
    # E = 12 (not a multiple of the 16-expert router tile), k = E, L ragged.
    dg = _dg()
    cfg, w32, x = block_case("mid_bf16", E=12, k=12, L=45)
    pb = dg.PackedBlock(w32, cfg)
    idx, w, lg = gpu_route(pb, x, cfg)
    wt = prepare.block_weights(w32, cfg)
    ref = oblock.route(x, wt["router"], wt["router_scale"], wt["per_expert_scale"], cfg["k"])
    # with k = E every expert is chosen; the order is by logit
    assert (np.sort(idx, axis=1) == np.arange(12)).all()
    routing_agrees(idx, ref["idx"], np.ones(45))
    assert np.allclose(w, ref["w"], rtol=1e-5, atol=1e-7)


@pytest.mark.parametrize("E,k,L,ties", [(200, 20, 50, False), (128, 24, 40, False), (40, 17, 33, False),
                                        (256, 32, 20, False), (64, 8, 48, True), (200, 32, 24, True)])
def test_route_selection_is_the_exact_topk_of_its_logits(E, k, L, ties):
    """The selection is index work on the kernel's own fp32 logits: it must be
    exactly the oracle's top-k rule (repeated maximum, the lowest expert among
    equal logits) applied to the logits the call returns, on every row.  Covers
    the lane layouts of the selection (8 or 16 logits per lane, lanes past E,
    choices past 16) and exact ties (pairs of identical router rows give
    bit-identical logits).  The weights are then held to the oracle's."""
    dg = _dg()
    cfg, w32, x = block_case("mid_bf16", E=E, k=k, L=L)
    if ties:
        w32 = dict(w32)
        r = np.array(w32["router"], copy=True)
        r[1::2] = r[0::2]
        w32["router"] = r
    say("route selection", E, k, L, "ties" if ties else "")
    pb = dg.PackedBlock(w32, cfg)
    idx, w, lg = gpu_route(pb, x, cfg)
    assert (idx == oblock.select_topk(lg.astype(np.float32).astype(np.float64), k)).all()
    if ties:
        # every row chose both members of some tied pair, lower index first
        pairs = [(a, b) for row in idx for a, b in zip(row[:-1], row[1:]) if a // 2 == b // 2]
        assert pairs and all(a < b for a, b in pairs)
    wt = prepare.block_weights(w32, cfg)
    ref = oblock.route(x, wt["router"], wt["router_scale"], wt["per_expert_scale"], cfg["k"],
                       1e-6, wt["router_bias"])
    same = routing_agrees(idx, ref["idx"], ref["margin"])
    assert np.allclose(w[same], ref["w"][same], rtol=1e-5, atol=1e-7)


# ------------------------------------------------------------------ experts with given routing
@pytest.mark.parametrize("name", ["tiny", "mid", "mid_bf16", "tall", "tall_f32", "short_many",
                                  "tiny_g32", "mid_g32", "mid_g32_q4dense", "tiny_nvfp4",
                                  "mid_nvfp4", "tiny_q6", "mid_q6"])
def test_moe_ffn_parity_with_injected_routing(name):
    dg = _dg()
    cfg, w32, x = block_case(name)
    say("moe_ffn", name)
    pb = dg.PackedBlock(w32, cfg)
    wt = prepare.block_weights(w32, cfg)
    rng = np.random.default_rng(1)
    L, E, k = cfg["L"], cfg["E"], cfg["k"]
    idx = np.stack([rng.permutation(E)[:k] for _ in range(L)]).astype(np.int32)
    w = rng.uniform(0.05, 1.0, (L, k))
    got = gpu_moe_ffn(pb, x, cfg, idx, w)
    b = oblock.rms_norm(x, wt["pre_ff_norm_2"], 1e-6)
    ref = oblock.moe_combine(b, idx, w.astype(np.float32).astype(np.float64),
                             wt["expert_gate_up"], wt["expert_down"], E)
    err = rel_err(got, ref)
    say("  moe rel err", err)
    assert err <= TOL


def test_moe_ffn_tall_tiles_skewed_experts():
    """Tall tiles with one expert holding every position (five row tiles, the
    last ragged), one expert with no rows, the rest split unevenly."""
    dg = _dg()
    cfg, w32, x = block_case("tall")
    say("moe_ffn tall skewed")
    pb = dg.PackedBlock(w32, cfg)
    wt = prepare.block_weights(w32, cfg)
    rng = np.random.default_rng(5)
    L, E = cfg["L"], cfg["E"]
    idx = np.stack([np.zeros(L, np.int32), np.where(rng.random(L) < 0.8, 2, 3)], axis=1).astype(np.int32)
    w = rng.uniform(0.05, 1.0, (L, 2))
    got = gpu_moe_ffn(pb, x, cfg, idx, w)
    b = oblock.rms_norm(x, wt["pre_ff_norm_2"], 1e-6)
    ref = oblock.moe_combine(b, idx, w.astype(np.float32).astype(np.float64),
                             wt["expert_gate_up"], wt["expert_down"], E)
    err = rel_err(got, ref)
    say("  moe rel err", err)
    assert err <= TOL


def _skewed_routing(L, E, k, seed):
    """Every position routes to expert 0 (L rows), about 70% to expert 1, the
    first 48 to expert 2 and the next 47 to expert 3 (either side of 48
    pairs); the other choices spread over experts 4.. at random."""
    rng = np.random.default_rng(seed)
    idx = np.empty((L, k), np.int32)
    for t in range(L):
        ch = [0]
        if rng.random() < 0.7:
            ch.append(1)
        if t < 48:
            ch.append(2)
        elif t < 95:
            ch.append(3)
        ch += list(rng.permutation(np.arange(4, E))[:k - len(ch)])
        idx[t] = rng.permutation(ch)
    return idx, rng.uniform(0.05, 1.0, (L, k))


@pytest.mark.parametrize("tall_min", [48, 1, 16, 0])
def test_moe_ffn_mixed_tiles_skewed_experts(tall_min):
    """Fewer than 32 pairs per expert on average (32-row tiles), with a few
    experts far above that: the experts with at least tall_min pairs take
    64-row tiles in the same launch (48: experts 0-2 only, expert 3 with 47
    pairs not; 1: every expert with rows; 0: none, the default).  Ragged tall
    and short tiles and experts without rows in one launch."""
    dg = _dg()
    cfg, w32, x = block_case("short_many")
    say("moe_ffn mixed tiles, tall_min", tall_min)
    pb = dg.PackedBlock(w32, cfg)
    wt = prepare.block_weights(w32, cfg)
    L, E, k = cfg["L"], cfg["E"], cfg["k"]
    idx, w = _skewed_routing(L, E, k, 6)
    counts = np.bincount(idx.ravel(), minlength=E)
    assert counts[0] == L and counts[2] == 48 and counts[3] == 47 and L * k < 32 * E
    prev = dg.dgmoe_debug_set_tall_min(tall_min)
    try:
        got = gpu_moe_ffn(pb, x, cfg, idx, w)
    finally:
        dg.dgmoe_debug_set_tall_min(prev)
    b = oblock.rms_norm(x, wt["pre_ff_norm_2"], 1e-6)
    ref = oblock.moe_combine(b, idx, w.astype(np.float32).astype(np.float64),
                             wt["expert_gate_up"], wt["expert_down"], E)
    err = rel_err(got, ref)
    say("  moe rel err", err)
    assert err <= TOL


@pytest.mark.parametrize("name", ["tiny", "mid", "max_experts"])
def test_block_parity_every_expert_tall_in_short_launch(name):
    """Short-tile batches with every expert that has rows on 64-row tiles (the
    dense MLP stays on 32-row tiles, its down K in chunks)."""
    dg = _dg()
    cfg, w32, x = block_case(name)
    prev = dg.dgmoe_debug_set_tall_min(1)
    try:
        _check_block(cfg, w32, x)
    finally:
        dg.dgmoe_debug_set_tall_min(prev)


@pytest.mark.parametrize("name", ["mid", "max_experts"])
def test_moe_ffn_out_of_range_index_contributes_nothing(name):
    # max_experts (k = 32) puts skipped slots in every eight-slot chunk of the sum
    dg = _dg()
    cfg, w32, x = block_case(name)
    pb = dg.PackedBlock(w32, cfg)
    wt = prepare.block_weights(w32, cfg)
    L, E, k = cfg["L"], cfg["E"], cfg["k"]
    rng = np.random.default_rng(2)
    idx = np.stack([rng.permutation(E)[:k] for _ in range(L)]).astype(np.int32)
    w = rng.uniform(0.05, 1.0, (L, k))
    idx[::3, 1] = -1
    idx[1::5, 0] = E + 7
    if k > 8:
        idx[::2, 9] = -3
        idx[1::4, k - 1] = E
        idx[3, :] = -1  # a row with no expert at all
    got = gpu_moe_ffn(pb, x, cfg, idx, w)
    keep = (idx >= 0) & (idx < E)
    b = oblock.rms_norm(x, wt["pre_ff_norm_2"], 1e-6)
    ref = oblock.moe_combine(b, np.where(keep, idx, 0), np.where(keep, w, 0.0).astype(np.float32),
                             wt["expert_gate_up"], wt["expert_down"], E)
    assert rel_err(got, ref) <= TOL


# ------------------------------------------------------------------ whole block
def _check_block(cfg, w32, x, y_dtype="f32"):
    dg = _dg()
    pb = dg.PackedBlock(w32, cfg)
    got = gpu_block(pb, x, cfg, y_dtype=y_dtype)
    wt = prepare.block_weights(w32, cfg)
    ref = oblock.block_forward(x, wt, cfg["k"])
    same = routing_agrees(got["idx"], ref["idx"], ref["margin"])
    err = rel_err(got["y"][same], ref["y"][same])
    say(f"  block {cfg['name']} L={x.shape[0]} rel err {err:.3e}, rerouted {int((~same).sum())}")
    assert err <= TOL
    assert np.allclose(got["w"][same], ref["w"][same], rtol=1e-5, atol=1e-7)
    return pb, got, ref


@pytest.mark.parametrize("name", ["tiny", "mid", "mid_bf16", "tall", "tall_f32", "max_experts",
                                  "max_hidden", "short_many", "tiny_g32", "mid_g32",
                                  "mid_g32_q4dense", "mid_q4_bf16dense", "mid_q8dense",
                                  "tiny_g32_q8dense", "tiny_nvfp4", "mid_nvfp4", "tiny_q6",
                                  "mid_q6"])
def test_block_parity(name):
    cfg, w32, x = block_case(name)
    say("block", name)
    _check_block(cfg, w32, x)


@pytest.mark.parametrize("D", [192, 320, 448])
def test_block_parity_short_tiles_ragged_columns(D):
    # short q4 tiles (16 x 4 pairs over 16 experts stays below the tall-tile
    # threshold) with a hidden size that ends inside a 256-column down tile:
    # some waves of the last tile own no weight block
    cfg, w32, x = block_case("mid", D=D)
    assert cfg["L"] * cfg["k"] < 32 * cfg["E"]
    _check_block(cfg, w32, x)


@pytest.mark.parametrize("L", [1, 17, 33, 64])
def test_block_parity_ragged_lengths(L):
    cfg, w32, x = block_case("mid", L=L)
    _check_block(cfg, w32, x)


def test_block_zero_rows_and_top1():
    cfg, w32, x = block_case("mid", k=1)
    x = x.copy()
    x[[0, 5, 6]] = 0.0
    _, got, ref = _check_block(cfg, w32, x)
    assert (got["y"][[0, 5, 6]] == 0).all()


@pytest.mark.parametrize("x_dtype,router_fmt", [("f32", "q8"), ("f32", "bf16"), ("bf16", "bf16")])
def test_block_activation_and_router_formats(x_dtype, router_fmt):
    # the front kernel's remaining (activation type, router format) pairs
    cfg, w32, x = block_case("mid", x_dtype=x_dtype, router_fmt=router_fmt)
    _check_block(cfg, w32, x)


@pytest.mark.parametrize("x_dtype", ["bf16", "f32"])
def test_block_single_expert(x_dtype):
    # E = k = 1: every position routes to expert 0 with weight pes[0]; one
    # expert tile, one router tile with fifteen padding experts
    cfg, w32, x = block_case("tiny", E=1, k=1, L=45, x_dtype=x_dtype)
    _, got, ref = _check_block(cfg, w32, x)
    assert (got["idx"] == 0).all()


def test_block_forced_routing():
    dg = _dg()
    cfg, w32, x = block_case("mid")
    pb = dg.PackedBlock(w32, cfg)
    wt = prepare.block_weights(w32, cfg)
    rng = np.random.default_rng(4)
    L, E, k = cfg["L"], cfg["E"], cfg["k"]
    idx = np.stack([rng.permutation(E)[:k] for _ in range(L)]).astype(np.int32)
    w = rng.uniform(0.05, 1.0, (L, k)).astype(np.float32)
    got = gpu_block(pb, x, cfg, force=(idx, w))
    ref = oblock.block_forward(x, wt, k, force_idx=idx, force_w=w.astype(np.float64))
    assert (got["idx"] == idx).all() and (got["w"] == w).all()
    assert rel_err(got["y"], ref["y"]) <= TOL


def test_block_bf16_output_is_rne_of_f32_and_runs_are_identical():
    dg = _dg()
    cfg, w32, x = block_case("mid")
    pb = dg.PackedBlock(w32, cfg)
    a = gpu_block(pb, x, cfg)
    b = gpu_block(pb, x, cfg)
    assert (a["y"] == b["y"]).all() and (a["idx"] == b["idx"]).all() and (a["w"] == b["w"]).all()
    c = gpu_block(pb, x, cfg, y_dtype="bf16")
    ref_bits = synth.round_bf16(a["y"].astype(np.float32)).view(np.uint32) >> 16
    assert (c["y_bits"].astype(np.uint32) == ref_bits).all()


def test_block_l_zero_is_noop():
    dg = _dg()
    torch = torch_dev()
    cfg, w32, x = block_case("tiny")
    pb = dg.PackedBlock(w32, cfg)
    dg.dgmoe_block_forward(pb.dims, pb.struct, None, dg.DGMOE_F32, 0, None, None, None,
                           dg.DGMOE_F32, None, None, None, 0)
    torch.cuda.synchronize()


# ------------------------------------------------------------------ full size, every position
def _full_size(name, positions=None):
    """GPU on the whole canvas; the oracle on every position (or on `positions`
    where given).  Positions whose routing legitimately differs (k-th/(k+1)-th
    oracle logit margin below 1e-4) are excluded from the output comparison."""
    dg = _dg()
    cfg = synth.config(name)
    say("full-size", name, "draw")
    w32 = synth.draw_weights(cfg)
    x = synth.draw_x(cfg)
    pb = dg.PackedBlock(w32, cfg)
    say("  gpu block")
    got = gpu_block(pb, x, cfg)
    wt = prepare.block_weights(w32, cfg)
    rows = np.arange(x.shape[0]) if positions is None else np.asarray(positions)
    say(f"  oracle on {rows.size} of {x.shape[0]} positions")
    ref = oblock.block_forward(x[rows], wt, cfg["k"])
    same = routing_agrees(got["idx"][rows], ref["idx"], ref["margin"])
    err = rel_err(got["y"][rows][same], ref["y"][same])
    say(f"  {name}: compared {int(same.sum())} of {x.shape[0]} positions "
        f"({int((~same).sum())} excusably rerouted), rel err {err:.3e}")
    assert err <= TOL
    assert np.allclose(got["w"][rows][same], ref["w"][same], rtol=1e-5, atol=1e-7)
    assert same.sum() >= 0.9 * rows.size
    return cfg, got


def test_full_canvas256_q4_every_position():
    _full_size("canvas256_q4")


def test_full_canvas256_bf16_every_position():
    _full_size("canvas256_bf16")


def test_full_canvas256_optiq_every_position():
    """The OptiQ checkpoint's formats: q4 group-64 experts, 8-bit group-64 dense
    MLP and router."""
    _full_size("canvas256_optiq")


def test_full_canvas256_nvfp4_every_position():
    """nvfp4 experts beside the bf16 dense MLP and router (one launch per phase)."""
    _full_size("canvas256_nvfp4")


def test_full_canvas256_q6_every_position():
    """q6 experts beside the bf16 dense MLP and router (one launch per phase)."""
    _full_size("canvas256_q6")


def test_full_canvas256_q4g32_every_position():
    """The diffgemma contract's own pack: q4 group-32 experts, bf16 dense MLP
    and router (four GEMM launches: the dense MLP in its own format)."""
    _full_size("canvas256_q4g32")


@pytest.mark.parametrize("name,override", [
    ("short_many", dict(weight_fmt="q4g32")),                     # past two rounds of the grid
    ("tall", dict(weight_fmt="q4g32")),                           # 150 rows per expert: short tiles only
    ("max_experts", dict(weight_fmt="q4g32", dense_fmt="bf16")),  # 256 experts, top-32
    ("tall", dict(weight_fmt="q4", dense_fmt="q4g32")),           # tall q4 experts, q4g32 dense alone
    ("tall", dict(weight_fmt="q4", dense_fmt="bf16")),            # tall q4 experts, bf16 dense alone
    ("mid", dict(weight_fmt="bf16", dense_fmt="q4g32")),          # bf16 experts, q4g32 dense alone
    ("short_many", dict(weight_fmt="q4", dense_fmt="bf16")),      # one launch per phase, both bodies
    ("short_many", dict(weight_fmt="q4g32", dense_fmt="q8")),     # the same with an 8-bit dense MLP
    ("tall", dict(weight_fmt="q4", dense_fmt="q8")),              # tall q4 experts, q8 dense alone
    ("max_hidden", dict(dense_fmt="q8")),                         # 8-bit dense rows of 8192 inputs
    ("short_many", dict(weight_fmt="nvfp4", dense_fmt="q4g32")),  # nvfp4 experts, q4g32 dense alone
    ("tall", dict(weight_fmt="nvfp4", dense_fmt="q8")),           # 150 rows per expert, short tiles
    ("max_experts", dict(weight_fmt="nvfp4")),                    # 256 experts, nvfp4 dense too
    ("short_many", dict(weight_fmt="q6", dense_fmt="q8")),        # q6 experts past two grid rounds
    ("mid", dict(weight_fmt="q4", dense_fmt="q6")),               # q6 dense alone
])
def test_block_parity_format_variants(name, override):
    cfg, w32, x = block_case(name, **override)
    say("block", name, override)
    _check_block(cfg, w32, x)


def test_full_batch2048_q4_every_position():
    _full_size("batch2048_q4")


def test_tall_tiles_several_per_workgroup_every_position():
    """More tall tiles than resident workgroups, so each workgroup's streams
    run across several tile boundaries, with tiles as short as four groups."""
    _full_size("tall_many")
