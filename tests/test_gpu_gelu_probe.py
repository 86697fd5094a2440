"""GPU probe of the GELU flavour in the GEMM epilogues.

The activation is GELU's tanh approximation (gelu_pytorch_tanh: diffgemma
"architecture & implemented contract", Part II section 1 "Model constants" and
the MoE-order bullet of section 2.1); the ML@Berkeley post's code calls the
erf form instead ("MLP and mixture-of-experts block").  The two differ by at
most ~5e-4, far below the block's 1e-2 * rms gate, so no ordinary parity case
can tell them apart.  This probe makes the difference dominate:

  D = I = 64, one expert, top-1; gate = diag(c), up = v * I, down = v * P
  (P a cyclic permutation), so every output element is one GELU value:
      moe[t, n] = w * v * gelu(c_s * xh[t, s]) * v * xh[t, s],   s = (n + 3) % 64
  with xh[t, i] = +-1 exactly (x entries +-1, eps 0, so the norm is exactly 1)
  and c_s = 15 k / 64 (k = 11..17), values that the q4 quantiser and bf16 both
  store exactly.  Where xh = -1 the GELU argument is in [-3.98, -2.58], where
  the tanh and erf forms are 3% to 35% apart; every other rounding in the path
  (fp16 act and slot rows) is below 1e-3 relative.

Both the q4 short-tile and tall-tile epilogues and the bf16 epilogue are run.
"""
import numpy as np
import pytest
import scipy.special

from oracle import block as oblock

from gpu_util import say, torch_dev

pytestmark = pytest.mark.gpu

D = 64
V = 0.9375                      # 15/16: the q4 quantiser stores it exactly (scale 1/16, code 15)
SHIFT = 3
C = np.array([15 * (11 + i % 7) / 64 for i in range(D)])   # 2.578125 .. 3.984375


def _probe_weights(rng):
    gate = np.diag(C)
    up = V * np.eye(D)
    down = np.zeros((D, D))
    down[np.arange(D), (np.arange(D) + SHIFT) % D] = V
    w32 = {
        "router": rng.standard_normal((1, D)).astype(np.float32),
        "router_scale": np.ones(D, np.float32),
        "per_expert_scale": np.ones(1, np.float32),
        "expert_gate_up": np.concatenate([gate, up])[None].astype(np.float32),
        "expert_down": down[None].astype(np.float32),
        "dense_gate_up": (rng.standard_normal((2 * D, D)) * 0.1).astype(np.float32),
        "dense_down": (rng.standard_normal((D, D)) * 0.1).astype(np.float32),
        "layer_scalar": 0.5,
        "router_bias": None,
    }
    for n in ("pre_ff_norm", "pre_ff_norm_2", "post_ff_norm_1", "post_ff_norm_2", "post_ff_norm"):
        w32[n] = np.ones(D, np.float32)
    return w32


def _gelu_erf(g):
    return 0.5 * g * (1.0 + scipy.special.erf(g / np.sqrt(2.0)))


@pytest.mark.parametrize("fmt,L", [("q4", 16), ("q4", 64), ("bf16", 16), ("bf16", 64)])
def test_gelu_is_the_tanh_form(fmt, L):
    torch = torch_dev()
    from moe_denoise_forward_amd import dgmoe as dg
    rng = np.random.default_rng(21)
    cfg = dict(name="gelu_probe", L=L, D=D, E=1, k=1, I=D, Id=D, x_dtype="bf16",
               weight_fmt=fmt, router_fmt="f32", eps=0.0)
    w32 = _probe_weights(rng)
    x = np.where(rng.random((L, D)) < 0.5, -1.0, 1.0).astype(np.float32)
    w = 0.875
    pb = dg.PackedBlock(w32, cfg)
    xt = torch.from_numpy(x).cuda().to(torch.bfloat16)
    idx = torch.zeros((L, 1), dtype=torch.int32, device="cuda")
    wt = torch.full((L, 1), w, dtype=torch.float32, device="cuda")
    out = torch.empty((L, D), dtype=torch.float32, device="cuda")
    ws, n = dg.workspace(pb.dims, L)
    say(f"gelu probe {fmt} L={L} ({'tall' if fmt == 'q4' and L >= 32 else 'short'} tiles)")
    dg.dgmoe_moe_ffn(pb.dims, pb.struct, xt, dg.DGMOE_BF16, L, idx, wt, out, ws, n)
    torch.cuda.synchronize()
    got = out.cpu().numpy().astype(np.float64)

    # the oracle (tanh form) on the same inputs, through its own expert MLP
    b = oblock.rms_norm(x, None, 0.0)
    assert np.array_equal(b, x)                 # the norm is exactly 1
    gu = np.concatenate([np.diag(C), V * np.eye(D)])
    down = w32["expert_down"][0].astype(np.float64)
    ref = oblock.moe_combine(b, np.zeros((L, 1), np.int64), np.full((L, 1), w), gu[None],
                             down[None], 1)
    src = (np.arange(D) + SHIFT) % D
    g = C[src][None, :] * x[:, src]
    erf_ref = w * V * V * _gelu_erf(g) * x[:, src]
    rel = np.abs(got - ref) / np.abs(ref)
    probed = g < 0
    gap = np.abs(erf_ref - ref) / np.abs(ref)
    say(f"  max rel err vs tanh form {rel.max():.2e}; probed elements {int(probed.sum())}, "
        f"tanh/erf gap there {gap[probed].min():.2e}..{gap[probed].max():.2e}; "
        f"min rel distance of GPU from the erf form {(np.abs(got - erf_ref) / np.abs(erf_ref))[probed].min():.2e}")
    assert probed.sum() >= L * D // 4
    assert rel.max() <= 5e-3
    assert gap[probed].min() >= 4 * 5e-3       # the bar is well inside the gap
    assert np.all(np.abs(got - erf_ref)[probed] > 2e-2 * np.abs(erf_ref)[probed])
