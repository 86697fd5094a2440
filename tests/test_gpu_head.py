"""GPU parity of the canvas head (dgmoe_tail, dgmoe_soft_embed, dgmoe_sc_input)
against the oracle (oracle/head.py) on the same seeded inputs, through the C ABI.

Bars, all derived from the block's bar on what the kernels round (fp16 MFMA
operands, fp32 accumulation), row by row:
  * logits y and soft embeddings: max|diff| <= 1e-2 * rms(ref row);
  * entropy: |diff| <= delta_t * sum_v p_v |ln p_v + H_t| + 1e-4, the first-order
    change of H_t when every logit of the row moves by at most
    delta_t = 1e-2 * rms(y_t) (dH/dy_v = -p_v (ln p_v + H));
  * argmax: equal, or the oracle's top-2 gap is below 2 delta_t and the chosen
    column's oracle logit is within 2 delta_t of the row's max;
  * row max within delta_t; row sum l within (2 delta_t + 1e-5) l;
  * canvas input (unit rms rows): max|diff| <= 1e-2.
The shapes: a tiny head, ragged row and vocabulary tiles (100 rows, 65
vocabulary blocks, K of 4 groups; 300 rows = two row tiles, odd block counts),
and the full DiffusionGemma head (256 x 2816, vocabulary 262144, SC MLP 2112)
on every row.
"""
import math

import numpy as np
import pytest

from moe_denoise_forward_amd import synth
from oracle import head as ohead
from oracle import prepare

from gpu_util import say, torch_dev

pytestmark = pytest.mark.gpu

REL = 1e-2


def _dg():
    from moe_denoise_forward_amd import dgmoe
    return dgmoe


class Case:
    """Draws, the oracle's table and the library's packed head for one config."""

    def __init__(self, name):
        say(f"head case {name}: drawing")
        self.cfg = cfg = synth.head_config(name)
        self.e32 = synth.draw_embed(cfg)
        self.hw = synth.draw_head_weights(cfg)
        self.ids = synth.draw_canvas_ids(cfg)
        self.x = synth.draw_tail_x(cfg, self.e32)
        self.sc_logits = synth.draw_sc_logits(cfg)
        say(f"head case {name}: oracle packing")
        self.table = ohead.EmbedTable.pack_q4(self.e32).densified()
        # the self-conditioning MLP as the library stores it: Q4G64, through the oracle's packer
        self.sc_gate_up = prepare.matrix_values(self.hw["sc_gate_up"], "q4")
        self.sc_down = prepare.matrix_values(self.hw["sc_down"], "q4")
        say(f"head case {name}: device packing")
        w32 = dict(self.hw, embed=self.e32)
        self.ph = _dg().PackedHead(w32, cfg)
        torch_dev().cuda.synchronize()
        self._tail, self._soft, self._sc = {}, None, {}

    def tail_ref(self, T):
        if T not in self._tail:
            say(f"  oracle tail T={T}")
            self._tail[T] = ohead.tail(self.x, self.hw["final_norm"], self.table, T)
        return self._tail[T]

    def soft_ref(self):
        if self._soft is None:
            say("  oracle soft embedding")
            self._soft = ohead.soft_embed(self.sc_logits, self.table)
        return self._soft

    def sc_ref(self, with_signal):
        if with_signal not in self._sc:
            say(f"  oracle canvas input (signal {with_signal})")
            y = self.sc_logits if with_signal else None
            self._sc[with_signal] = ohead.sc_input(self.ids, y, self.table, self.hw["sc_pre_norm"],
                                                   self.sc_gate_up, self.sc_down)
        return self._sc[with_signal]


_CASES = {}


def _case(name):
    if name not in _CASES:
        _CASES[name] = Case(name)
    return _CASES[name]


CASES = ["head_tiny", "head_mid", "head_rows"]


def _x_tensor(c):
    torch = torch_dev()
    dg = _dg()
    t = torch.from_numpy(np.ascontiguousarray(c.x, np.float32)).cuda()
    if c.cfg["x_dtype"] == "bf16":
        return t.to(torch.bfloat16), dg.DGMOE_BF16
    return t, dg.DGMOE_F32


def gpu_tail(c, T, want_logits=True):
    torch = torch_dev()
    dg = _dg()
    L, V = c.cfg["L"], c.cfg["V"]
    xt, xd = _x_tensor(c)
    H = torch.empty(L, dtype=torch.float32, device="cuda")
    am = torch.empty(L, dtype=torch.int32, device="cuda")
    mx = torch.empty(L, dtype=torch.float32, device="cuda")
    sm = torch.empty(L, dtype=torch.float32, device="cuda")
    lg = torch.empty((L, V), dtype=torch.float32, device="cuda") if want_logits else None
    ws, n = dg.head_workspace(c.ph.dims, L)
    dg.dgmoe_tail(c.ph.dims, c.ph.struct, xt, xd, L, T, H, am, mx, sm, lg, ws, n)
    torch.cuda.synchronize()
    assert dg.dgmoe_head_check_workspace(c.ph.dims, L, ws) == 0
    out = {"H": H.cpu().numpy().astype(np.float64), "argmax": am.cpu().numpy(),
           "m": mx.cpu().numpy().astype(np.float64), "l": sm.cpu().numpy().astype(np.float64)}
    if want_logits:
        out["y"] = lg.cpu().numpy()
    return out


def check_tail(got, ref, name):
    y = ref["y"]
    rms_row = np.sqrt(np.mean(y * y, axis=1))
    delta = REL * rms_row
    # entropy: first-order propagation of a logit error bounded by delta
    m = y.max(axis=1, keepdims=True)
    e = np.exp(y - m)
    l = e.sum(axis=1, keepdims=True)
    p = e / l
    logp = (y - m) - np.log(l)
    A = (p * np.abs(logp + ref["H"][:, None])).sum(axis=1)
    tol_H = delta * A + 1e-4
    dH = np.abs(got["H"] - ref["H"])
    say(f"  {name}: entropy max|diff| {dH.max():.2e} (worst ratio to bar {np.max(dH / tol_H):.3f}), "
        f"H in [{ref['H'].min():.3f}, {ref['H'].max():.3f}]")
    assert np.all(dH <= tol_H), np.nonzero(dH > tol_H)[0][:10]
    # argmax
    diff = got["argmax"] != ref["argmax"]
    if diff.any():
        rows = np.nonzero(diff)[0]
        ok = (ref["margin"][rows] < 2 * delta[rows]) & \
             (ref["m"][rows] - y[rows, got["argmax"][rows]] < 2 * delta[rows])
        say(f"  {name}: argmax differs at {rows.size} rows, all near ties: {bool(ok.all())}")
        assert ok.all(), rows[~ok][:10]
    assert np.all(np.abs(got["m"] - ref["m"]) <= delta)
    assert np.all(np.abs(got["l"] - ref["l"]) <= (2 * delta + 1e-5) * ref["l"])
    if "y" in got:
        dy = np.max(np.abs(got["y"] - y), axis=1)
        say(f"  {name}: logits worst row max|diff| / rms {np.max(dy / rms_row):.2e}")
        assert np.all(dy <= delta)


@pytest.mark.parametrize("name", CASES)
def test_tail_parity(name):
    c = _case(name)
    T = c.cfg["T"]
    say(f"tail {name} L={c.cfg['L']} V={c.cfg['V']} T={T}")
    check_tail(gpu_tail(c, T), c.tail_ref(T), name)


@pytest.mark.parametrize("T", [0.4, 0.8])
def test_tail_temperatures_without_logits(T):
    c = _case("head_rows")
    say(f"tail head_rows T={T}, statistics only")
    got = gpu_tail(c, T, want_logits=False)
    check_tail(got, c.tail_ref(T), f"head_rows T={T}")


def _rowwise_ok(got, ref, what):
    rms_row = np.sqrt(np.mean(ref * ref, axis=1))
    d = np.max(np.abs(got - ref), axis=1)
    say(f"  {what}: worst row max|diff| / rms {np.max(d / rms_row):.2e}")
    assert np.all(d <= REL * rms_row)


@pytest.mark.parametrize("name", CASES)
def test_soft_embed_parity(name):
    torch = torch_dev()
    dg = _dg()
    c = _case(name)
    L, D = c.cfg["L"], c.cfg["D"]
    say(f"soft embedding {name} L={L} V={c.cfg['V']}")
    yl = torch.from_numpy(c.sc_logits).cuda()
    soft = torch.empty((L, D), dtype=torch.float32, device="cuda")
    ws, n = dg.head_workspace(c.ph.dims, L)
    dg.dgmoe_soft_embed(c.ph.dims, c.ph.struct, yl, L, soft, ws, n)
    torch.cuda.synchronize()
    assert dg.dgmoe_head_check_workspace(c.ph.dims, L, ws) == 0
    _rowwise_ok(soft.cpu().numpy().astype(np.float64), c.soft_ref(), f"soft {name}")


def gpu_sc(c, with_signal, ids=None, expect_flags=0):
    torch = torch_dev()
    dg = _dg()
    L, D = c.cfg["L"], c.cfg["D"]
    it = torch.from_numpy(np.ascontiguousarray(c.ids if ids is None else ids, np.int32)).cuda()
    yl = torch.from_numpy(c.sc_logits).cuda() if with_signal else None
    out = torch.empty((L, D), dtype=torch.float32, device="cuda")
    ws, n = dg.head_workspace(c.ph.dims, L)
    dg.dgmoe_sc_input(c.ph.dims, c.ph.struct, it, yl, L, out, ws, n)
    torch.cuda.synchronize()
    assert dg.dgmoe_head_check_workspace(c.ph.dims, L, ws) == expect_flags
    return out.cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("name", CASES)
@pytest.mark.parametrize("with_signal", [True, False])
def test_sc_input_parity(name, with_signal):
    c = _case(name)
    say(f"canvas input {name} signal={with_signal}")
    got = gpu_sc(c, with_signal)
    ref = c.sc_ref(with_signal)["out"]
    err = np.max(np.abs(got - ref))
    say(f"  max|diff| {err:.2e} (rows have unit rms)")
    assert err <= REL


def test_sc_input_flags_bad_ids():
    dg = _dg()
    c = _case("head_tiny")
    ids = c.ids.copy()
    ids[3] = c.cfg["V"]
    ids[5] = -1
    got = gpu_sc(c, False, ids=ids, expect_flags=dg.DGMOE_FLAG_INDEX)
    ref_ids = ids.copy()
    ref_ids[[3, 5]] = 0  # an id outside the vocabulary reads row 0
    ref = ohead.sc_input(ref_ids, None, c.table, c.hw["sc_pre_norm"], c.sc_gate_up,
                         c.sc_down)["out"]
    assert np.max(np.abs(got - ref)) <= REL


def test_full_head_parity():
    """The full head (256 x 2816, vocabulary 262144): tail with logits, soft
    embedding, canvas input with and without signal, every row."""
    torch = torch_dev()
    dg = _dg()
    c = Case("head_full")
    try:
        T = c.cfg["T"]
        say(f"full tail T={T}")
        check_tail(gpu_tail(c, T), c.tail_ref(T), "head_full")
        c._tail.clear()
        L, D = c.cfg["L"], c.cfg["D"]
        say("full soft embedding")
        yl = torch.from_numpy(c.sc_logits).cuda()
        soft = torch.empty((L, D), dtype=torch.float32, device="cuda")
        ws, n = dg.head_workspace(c.ph.dims, L)
        dg.dgmoe_soft_embed(c.ph.dims, c.ph.struct, yl, L, soft, ws, n)
        torch.cuda.synchronize()
        assert dg.dgmoe_head_check_workspace(c.ph.dims, L, ws) == 0
        _rowwise_ok(soft.cpu().numpy().astype(np.float64), c.soft_ref(), "soft head_full")
        del yl, ws
        for with_signal in (True, False):
            say(f"full canvas input signal={with_signal}")
            err = np.max(np.abs(gpu_sc(c, with_signal) - c.sc_ref(with_signal)["out"]))
            say(f"  max|diff| {err:.2e}")
            assert err <= REL
    finally:
        del c
        torch.cuda.empty_cache()
