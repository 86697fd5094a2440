"""Helpers of the GPU parity tests: run the library through its C ABI on seeded
inputs and compare with the oracle on the same inputs."""
import sys

import numpy as np

from moe_denoise_forward_amd import synth

TOL = 1e-2          # max|diff| <= TOL * rms(ref), the block's parity bar
MARGIN = 1e-4       # positions whose k-th/(k+1)-th logit gap is below this may route differently


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def torch_dev():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return torch


def x_tensor(x, cfg):
    """Device tensor of x in the workload's activation dtype and the matching enum."""
    torch = torch_dev()
    from moe_denoise_forward_amd import dgmoe as dg
    t = torch.from_numpy(np.ascontiguousarray(x, np.float32)).cuda()
    if cfg["x_dtype"] == "bf16":
        return t.to(torch.bfloat16), dg.DGMOE_BF16
    return t, dg.DGMOE_F32


def gpu_block(pb, x, cfg, force=None, y_dtype="f32", want_route=True):
    """Run dgmoe_block_forward; returns dict(y (float64 numpy), idx, w)."""
    torch = torch_dev()
    from moe_denoise_forward_amd import dgmoe as dg
    L, D, k = x.shape[0], cfg["D"], cfg["k"]
    xt, xd = x_tensor(x, cfg)
    ydt = torch.float32 if y_dtype == "f32" else torch.bfloat16
    y = torch.empty((L, D), dtype=ydt, device="cuda")
    idx = torch.empty((L, k), dtype=torch.int32, device="cuda") if want_route else None
    w = torch.empty((L, k), dtype=torch.float32, device="cuda") if want_route else None
    fi = fw = None
    if force is not None:
        fi = torch.from_numpy(np.ascontiguousarray(force[0], np.int32)).cuda()
        fw = torch.from_numpy(np.ascontiguousarray(force[1], np.float32)).cuda()
    ws, n = dg.workspace(pb.dims, L)
    dg.dgmoe_block_forward(pb.dims, pb.struct, xt, xd, L, fi, fw, y,
                           dg.DGMOE_F32 if y_dtype == "f32" else dg.DGMOE_BF16, idx, w, ws, n)
    torch.cuda.synchronize()
    assert dg.dgmoe_check_workspace(pb.dims, L, ws) == 0, "the call flagged a device-side error"
    out = {"y": y.float().cpu().numpy().astype(np.float64)}
    if y_dtype == "bf16":
        out["y_bits"] = y.view(torch.int16).cpu().numpy().view(np.uint16)
    if want_route:
        out["idx"] = idx.cpu().numpy()
        out["w"] = w.cpu().numpy().astype(np.float64)
    return out


def gpu_route(pb, x, cfg):
    torch = torch_dev()
    from moe_denoise_forward_amd import dgmoe as dg
    L, k, E = x.shape[0], cfg["k"], cfg["E"]
    xt, xd = x_tensor(x, cfg)
    idx = torch.empty((L, k), dtype=torch.int32, device="cuda")
    w = torch.empty((L, k), dtype=torch.float32, device="cuda")
    lg = torch.empty((L, E), dtype=torch.float32, device="cuda")
    ws, n = dg.workspace(pb.dims, L)
    dg.dgmoe_route(pb.dims, pb.struct, xt, xd, L, idx, w, lg, ws, n)
    torch.cuda.synchronize()
    assert dg.dgmoe_check_workspace(pb.dims, L, ws) == 0, "the call flagged a device-side error"
    return idx.cpu().numpy(), w.cpu().numpy().astype(np.float64), lg.cpu().numpy().astype(np.float64)


def gpu_moe_ffn(pb, x, cfg, idx, w, flags_out=None):
    """dgmoe_moe_ffn; asserts the call flagged nothing unless flags_out (a list)
    is given, which then receives the flags."""
    torch = torch_dev()
    from moe_denoise_forward_amd import dgmoe as dg
    L, D = x.shape[0], cfg["D"]
    xt, xd = x_tensor(x, cfg)
    it = torch.from_numpy(np.ascontiguousarray(idx, np.int32)).cuda()
    wt = torch.from_numpy(np.ascontiguousarray(w, np.float32)).cuda()
    out = torch.empty((L, D), dtype=torch.float32, device="cuda")
    ws, n = dg.workspace(pb.dims, L)
    dg.dgmoe_moe_ffn(pb.dims, pb.struct, xt, xd, L, it, wt, out, ws, n)
    torch.cuda.synchronize()
    flags = dg.dgmoe_check_workspace(pb.dims, L, ws)
    if flags_out is None:
        assert flags == 0, "the call flagged a device-side error"
    else:
        flags_out.append(flags)
    return out.cpu().numpy().astype(np.float64)


def rel_err(got, ref):
    """max|got - ref| / rms(ref)."""
    rms = np.sqrt(np.mean(ref * ref))
    return float(np.max(np.abs(got - ref)) / rms)


def routing_agrees(gpu_idx, ref_idx, margin):
    """Rows where the selected sets are equal; asserts every differing row is excusable."""
    same = np.array([list(a) == list(b) for a, b in zip(gpu_idx.tolist(), ref_idx.tolist())])
    bad = np.nonzero(~same & (margin >= MARGIN))[0]
    assert bad.size == 0, f"routing differs at non-excusable rows {bad[:10]} (margins {margin[bad[:10]]})"
    return same


def block_case(name, **override):
    cfg = synth.config(name, **override)
    w32 = synth.draw_weights(cfg)
    x = synth.draw_x(cfg)
    return cfg, w32, x
