"""GPU parity of the denoise attention (dgmoe_attn_denoise) against the oracle
(oracle/attention.py) on the same seeded inputs, through the C ABI.

Bar: every output row within max|diff| <= 1e-2 * rms(ref row), the block's bar
on the same kind of rounding (q, k, v and the softmax weights rounded to fp16
as MFMA operands, fp32 accumulation; the derivation is in the design notes).
A bf16 output is the RNE of the fp32 output, bit for bit.  Shapes: tiny
sliding / full layers whose window cuts the cache, ragged 100-row canvases of
the model's head shapes (head_dim 256 and 512, both readings of the partial
rotation's partner stride), the full 256-row canvas after a 4096-position
prompt on every row, and edge cases (no committed rows, one canvas row, a
window wider than the cache, a window of exactly the cache).
"""
import numpy as np
import pytest

from moe_denoise_forward_amd import synth
from oracle import attention as oa

from gpu_util import say, torch_dev

pytestmark = pytest.mark.gpu

REL = 1e-2


def _dg():
    from moe_denoise_forward_amd import dgmoe
    return dgmoe


def oracle_out(cfg, d, reading="arch"):
    return oa.denoise_attention(d["qraw"], d["kraw"], d["vraw"], d["w_q"], d["w_k"],
                                d["k_cache"].astype(np.float64), d["v_cache"].astype(np.float64),
                                cfg["kv_len"], cfg["H"], cfg["Hkv"], cfg["hd"], cfg["kind"],
                                reading, window=cfg["window"])


def gpu_out(cfg, d, reading="arch", out_dtype="f32"):
    torch = torch_dev()
    dg = _dg()
    L, H, hd = cfg["L"], cfg["H"], cfg["hd"]
    dims = dg.attn_dims_for(cfg, reading)

    def dev(x):
        if x is None:
            return None
        t = torch.from_numpy(np.ascontiguousarray(x, np.float32)).cuda()
        return t.to(torch.bfloat16) if cfg["x_dtype"] == "bf16" else t

    q, k, v = dev(d["qraw"]), dev(d["kraw"]), dev(d["vraw"])
    ind = dg.DGMOE_BF16 if cfg["x_dtype"] == "bf16" else dg.DGMOE_F32
    wq = torch.from_numpy(d["w_q"]).cuda()
    wk = torch.from_numpy(d["w_k"]).cuda()
    kc = torch.from_numpy(d["k_cache"].view(np.uint16).astype(np.int16)).cuda()
    vc = torch.from_numpy(d["v_cache"].view(np.uint16).astype(np.int16)).cuda()
    rows = d["k_cache"].shape[1]
    od = dg.DGMOE_F32 if out_dtype == "f32" else dg.DGMOE_BF16
    out = torch.empty((L, H * hd), dtype=torch.float32 if out_dtype == "f32" else torch.bfloat16,
                      device="cuda")
    ws, n = dg.attn_workspace(dims, L, cfg["kv_len"])
    dg.dgmoe_attn_denoise(dims, q, k, v, ind, L, wq, wk, kc, vc, rows, cfg["kv_len"], out, od, ws, n)
    torch.cuda.synchronize()
    if out_dtype == "f32":
        return out.cpu().numpy().astype(np.float64)
    return out.view(torch.int16).cpu().numpy().view(np.uint16)


def check(cfg, reading="arch"):
    d = synth.draw_attn(cfg)
    say(f"attention {cfg['name']} {cfg['kind']} L={cfg['L']} kv_len={cfg['kv_len']} "
        f"H={cfg['H']} Hkv={cfg['Hkv']} hd={cfg['hd']} window={cfg['window']} rope={reading}")
    ref = oracle_out(cfg, d, reading)
    got = gpu_out(cfg, d, reading)
    rms = np.sqrt(np.mean(ref * ref, axis=1))
    err = np.max(np.abs(got - ref), axis=1)
    say(f"  worst row max|diff| / rms {np.max(err / rms):.2e}, output rms {np.sqrt(np.mean(ref * ref)):.3f}")
    assert np.all(err <= REL * rms), np.nonzero(err > REL * rms)[0][:10]
    return d, got


@pytest.mark.parametrize("name,reading", [("attn_tiny_sliding", "arch"), ("attn_tiny_full", "arch"),
                                          ("attn_tiny_full", "blog"),
                                          ("attn_mid_sliding", "arch"), ("attn_mid_full", "arch"),
                                          ("attn_mid_full", "blog")])
def test_attention_parity(name, reading):
    check(synth.attn_config(name), reading)


@pytest.mark.parametrize("name,override", [
    ("attn_tiny_sliding", dict(kv_len=0)),              # no committed rows: the canvas alone
    ("attn_tiny_full", dict(L=1)),                      # one canvas row
    ("attn_tiny_sliding", dict(kv_len=10)),             # the window is wider than the cache
    ("attn_tiny_sliding", dict(kv_len=24)),             # the window is exactly the cache
    ("attn_mid_sliding", dict(L=33, kv_len=1)),         # ragged rows, one committed row
    ("attn_mid_full", dict(L=17, kv_len=64, x_dtype="f32")),
])
def test_attention_edge_cases(name, override):
    check(synth.attn_config(name, **override))


def test_attention_bf16_output_is_rne_of_f32_and_runs_are_identical():
    cfg = synth.attn_config("attn_mid_full")
    d = synth.draw_attn(cfg)
    a = gpu_out(cfg, d)
    b = gpu_out(cfg, d)
    assert np.array_equal(a, b)
    c = gpu_out(cfg, d, out_dtype="bf16")
    ref_bits = synth.round_bf16(a.astype(np.float32)).view(np.uint32) >> 16
    assert np.array_equal(c.astype(np.uint32), ref_bits)


@pytest.mark.parametrize("name", ["attn_sliding", "attn_full"])
def test_attention_full_size_every_row(name):
    """The model's layer shapes: 256 canvas rows after a 4096-position prompt
    (sliding: 1023 committed keys of 8 KV heads of 256; full: all 4096 of 2
    KV heads of 512), every row of every head against the oracle."""
    check(synth.attn_config(name))
