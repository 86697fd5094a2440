"""GPU tests of the library's failure handling.  Every condition here is
forced from the host; every kernel still runs to its normal end.

  * The front kernel's bounded wait for the call stamp: with the diagnostics
    hook the stamp is never published and the wait limited to a few polls, so
    every router workgroup gives up.  The call must end normally with
    DGMOE_FLAG_SYNC_TIMEOUT, and the next normal call on the same workspace
    must be clean and correct.  (The counts the GEMMs then read are clamped;
    tests/test_plan_clamp.py checks that logic on the CPU.)
  * fp16 intermediates: operands near the fp16 limit give correct results and
    no flag; operands or GeGLU outputs past it raise DGMOE_FLAG_FP16_RANGE.
  * A caller routing that names one expert more than L times raises
    DGMOE_FLAG_ROUTE_OVERFLOW.
"""
import numpy as np
import pytest

from oracle import block as oblock
from oracle import prepare

from gpu_util import (TOL, block_case, gpu_block, gpu_moe_ffn, rel_err, routing_agrees, say,
                      torch_dev, x_tensor)

pytestmark = pytest.mark.gpu


def _dg():
    from moe_denoise_forward_amd import dgmoe
    return dgmoe


def _block_raw(pb, x, cfg, ws, n):
    torch = torch_dev()
    dg = _dg()
    L, D, k = x.shape[0], cfg["D"], cfg["k"]
    xt, xd = x_tensor(x, cfg)
    y = torch.empty((L, D), dtype=torch.float32, device="cuda")
    idx = torch.empty((L, k), dtype=torch.int32, device="cuda")
    w = torch.empty((L, k), dtype=torch.float32, device="cuda")
    dg.dgmoe_block_forward(pb.dims, pb.struct, xt, xd, L, None, None, y, dg.DGMOE_F32, idx, w,
                           ws, n)
    torch.cuda.synchronize()
    return y.cpu().numpy().astype(np.float64), idx.cpu().numpy(), dg.dgmoe_check_workspace(pb.dims, L, ws)


def test_stamp_timeout_is_flagged_and_the_next_call_is_clean():
    dg = _dg()
    cfg, w32, x = block_case("mid")
    pb = dg.PackedBlock(w32, cfg)
    ws, n = dg.workspace(pb.dims, cfg["L"])
    say("forced stamp timeout (16 polls, stamp never published)")
    dg.dgmoe_debug_force_stamp_timeout(16)
    try:
        _, _, flags = _block_raw(pb, x, cfg, ws, n)
    finally:
        dg.dgmoe_debug_force_stamp_timeout(0)
    say(f"  flags {flags}")
    assert flags & dg.DGMOE_FLAG_SYNC_TIMEOUT
    # the same workspace, a normal call: clean flags, correct output
    y, idx, flags = _block_raw(pb, x, cfg, ws, n)
    assert flags == 0
    wt = prepare.block_weights(w32, cfg)
    ref = oblock.block_forward(x, wt, cfg["k"])
    same = routing_agrees(idx, ref["idx"], ref["margin"])
    err = rel_err(y[same], ref["y"][same])
    say(f"  next call rel err {err:.3e}")
    assert err <= TOL


# ---------------------------------------------------------------- fp16 range
I0, I1 = 5, 7          # the two spiked input columns
SPIKE_ROW, ACT_ROW = 0, 1


def _spiked(norm_b, norm_a, act_scale):
    """mid_bf16 with: row 0 a spike at column I0 (|xh| ~ sqrt(D)) and pre-norm
    weights norm_b / norm_a there (b / a near or past the fp16 limit), the
    weights reading column I0 shrunk by 2^-12 so the GEMM outputs stay small;
    row 1 a spike at column I1 and pre_ff_norm_2[I1] = act_scale, which drives
    its experts' GeGLU outputs up."""
    cfg, w32, x = block_case("mid_bf16")
    w32 = dict(w32)
    x = x.copy()
    x[SPIKE_ROW] *= 0.01
    x[SPIKE_ROW, I0] = 50.0
    x[ACT_ROW] *= 0.01
    x[ACT_ROW, I1] = 50.0
    for n in ("expert_gate_up",):
        w = w32[n].copy()
        w[:, :, I0] *= 2.0 ** -12
        w32[n] = w
    w = w32["dense_gate_up"].copy()
    w[:, I0] *= 2.0 ** -12
    w32["dense_gate_up"] = w
    w2 = w32["pre_ff_norm_2"].copy()
    w2[I0], w2[I1] = norm_b, act_scale
    w32["pre_ff_norm_2"] = w2
    w1 = w32["pre_ff_norm"].copy()
    w1[I0] = norm_a
    w32["pre_ff_norm"] = w1
    return cfg, w32, x


def _intermediates(cfg, w32, x):
    """Largest |a|, |b|, |act| and |expert output row| the block forms (float64)."""
    wt = prepare.block_weights(w32, cfg)
    xh = oblock.rms_norm(x, None, 1e-6)
    a = xh * wt["pre_ff_norm"]
    b = xh * wt["pre_ff_norm_2"]
    r = oblock.route(x, wt["router"], wt["router_scale"], wt["per_expert_scale"], cfg["k"])
    I = cfg["I"]
    act_max = slot_max = 0.0
    for e in np.unique(r["idx"]):
        rows = np.nonzero((r["idx"] == e).any(axis=1))[0]
        gu = wt["expert_gate_up"][e]
        act = oblock.gelu_tanh(b[rows] @ gu[:I].T) * (b[rows] @ gu[I:].T)
        act_max = max(act_max, np.abs(act).max())
        slot_max = max(slot_max, np.abs(act @ wt["expert_down"][e].T).max())
    Id = cfg["Id"]
    gd = wt["dense_gate_up"]
    act_d = oblock.gelu_tanh(a @ gd[:Id].T) * (a @ gd[Id:].T)
    return dict(a=np.abs(a).max(), b=np.abs(b).max(), act=max(act_max, np.abs(act_d).max()),
                slot=slot_max)


def _act_scale_for(target):
    """pre_ff_norm_2[I1] that puts the largest GeGLU output at `target`."""
    lo, hi = 1.0, 4096.0
    for _ in range(40):
        mid = (lo * hi) ** 0.5
        cfg, w32, x = _spiked(1.0, 1.0, mid)
        if _intermediates(cfg, w32, x)["act"] < target:
            lo = mid
        else:
            hi = mid
    return lo


def test_fp16_intermediates_near_the_limit_are_exact_enough():
    dg = _dg()
    s = _act_scale_for(50000.0)
    cfg, w32, x = _spiked(3400.0, 3400.0, s)
    m = _intermediates(cfg, w32, x)
    say(f"near-limit intermediates: |a| {m['a']:.0f}, |b| {m['b']:.0f}, |act| {m['act']:.0f}, "
        f"|slot| {m['slot']:.0f} (fp16 max 65504)")
    assert 40000 < m["a"] < 60000 and 40000 < m["b"] < 60000 and 40000 < m["act"] < 60000
    assert m["slot"] < 60000
    pb = dg.PackedBlock(w32, cfg)
    got = gpu_block(pb, x, cfg)          # asserts no flag
    wt = prepare.block_weights(w32, cfg)
    ref = oblock.block_forward(x, wt, cfg["k"])
    same = routing_agrees(got["idx"], ref["idx"], ref["margin"])
    assert same[SPIKE_ROW] and same[ACT_ROW]
    err = rel_err(got["y"][same], ref["y"][same])
    say(f"  rel err {err:.3e}")
    assert np.isfinite(got["y"]).all()
    assert err <= TOL


@pytest.mark.parametrize("what", ["operand", "act"])
def test_fp16_overflow_is_flagged(what):
    dg = _dg()
    if what == "operand":   # b and a past the limit, GeGLU outputs small
        cfg, w32, x = _spiked(6000.0, 6000.0, 1.0)
    else:                   # operands in range, GeGLU outputs past it
        cfg, w32, x = _spiked(1.0, 1.0, 2.0 * _act_scale_for(50000.0))
    m = _intermediates(cfg, w32, x)
    say(f"overflow ({what}): |a| {m['a']:.0f}, |b| {m['b']:.0f}, |act| {m['act']:.0f}")
    if what == "operand":
        assert m["b"] > 65520 and m["act"] < 60000
    else:
        assert m["b"] < 60000 and m["act"] > 65520
    pb = dg.PackedBlock(w32, cfg)
    ws, n = dg.workspace(pb.dims, cfg["L"])
    _, _, flags = _block_raw(pb, x, cfg, ws, n)
    say(f"  flags {flags}")
    assert flags == dg.DGMOE_FLAG_FP16_RANGE


def test_route_overflow_is_flagged():
    # every slot of every position names expert 2: L*k pairs for a list of L
    dg = _dg()
    cfg, w32, x = block_case("mid")
    pb = dg.PackedBlock(w32, cfg)
    L, k = cfg["L"], cfg["k"]
    idx = np.full((L, k), 2, np.int32)
    w = np.full((L, k), 0.25)
    flags = []
    gpu_moe_ffn(pb, x, cfg, idx, w, flags_out=flags)
    assert flags[0] == dg.DGMOE_FLAG_ROUTE_OVERFLOW
    # distinct experts per position: clean
    idx = np.stack([np.random.default_rng(t).permutation(cfg["E"])[:k] for t in range(L)])
    flags = []
    gpu_moe_ffn(pb, x, cfg, idx.astype(np.int32), w, flags_out=flags)
    assert flags[0] == 0
