"""dgmoe_block_forward_noalloc (static device workspace) against
dgmoe_block_forward (caller workspace): the same kernels on the same inputs,
so the outputs and the routing must agree bit for bit.  Two calls in a row, the
second on fewer positions (the static array keeps the first call's contents),
then the forced-routing path, and a size past the static workspace, which must
be refused before anything is enqueued."""
import numpy as np
import pytest

from moe_denoise_forward_amd import synth

from gpu_util import say, torch_dev, x_tensor

pytestmark = pytest.mark.gpu


def _dg():
    from moe_denoise_forward_amd import dgmoe
    return dgmoe


def _outputs(pb, cfg, x, noalloc, force=None):
    torch = torch_dev()
    dg = _dg()
    L, D, k = x.shape[0], cfg["D"], cfg["k"]
    xt, xd = x_tensor(x, cfg)
    y = torch.full((L, D), float("nan"), dtype=torch.float32, device="cuda")
    idx = torch.full((L, k), -7, dtype=torch.int32, device="cuda")
    w = torch.full((L, k), float("nan"), dtype=torch.float32, device="cuda")
    fi = fw = None
    if force is not None:
        fi = torch.from_numpy(np.ascontiguousarray(force[0], np.int32)).cuda()
        fw = torch.from_numpy(np.ascontiguousarray(force[1], np.float32)).cuda()
    if noalloc:
        dg.dgmoe_block_forward_noalloc(pb.dims, pb.struct, xt, xd, L, fi, fw, y, dg.DGMOE_F32, idx,
                                       w)
    else:
        ws, n = dg.workspace(pb.dims, L)
        dg.dgmoe_block_forward(pb.dims, pb.struct, xt, xd, L, fi, fw, y, dg.DGMOE_F32, idx, w, ws, n)
    torch.cuda.synchronize()
    return y.cpu().numpy(), idx.cpu().numpy(), w.cpu().numpy()


def _same(a, b):
    return all(np.array_equal(u, v, equal_nan=False) for u, v in zip(a, b))


def test_noalloc_matches_the_workspace_entry_point():
    dg = _dg()
    cfg = synth.config("canvas256_q4")
    w32 = synth.draw_weights(cfg)
    x = synth.draw_x(cfg)
    pb = dg.PackedBlock(w32, cfg)
    assert dg.dgmoe_workspace_size(pb.dims, cfg["L"]) <= dg.dgmoe_noalloc_max_bytes()
    for L in (256, 100):
        say(f"noalloc vs workspace: canvas256_q4 shape, L={L}")
        ref = _outputs(pb, cfg, x[:L], noalloc=False)
        got = _outputs(pb, cfg, x[:L], noalloc=True)
        assert np.isfinite(got[0]).all()
        assert _same(got, ref)
    # the forced-routing path through the static workspace
    rng = np.random.default_rng(3)
    L, E, k = 64, cfg["E"], cfg["k"]
    force = (np.stack([rng.permutation(E)[:k] for _ in range(L)]), rng.uniform(0.05, 1.0, (L, k)))
    assert _same(_outputs(pb, cfg, x[:L], True, force), _outputs(pb, cfg, x[:L], False, force))


def test_noalloc_refuses_sizes_past_its_workspace():
    dg = _dg()
    torch = torch_dev()
    cfg = synth.config("canvas256_q4")
    dims = dg.make_dims(cfg["D"], cfg["E"], cfg["k"], cfg["I"], cfg["Id"])
    L = 1
    while dg.dgmoe_workspace_size(dims, L) <= dg.dgmoe_noalloc_max_bytes():
        L *= 2
    y = torch.empty(16, device="cuda")
    with pytest.raises(dg.DgmoeError) as e:
        # pointers are never touched: the size check comes first
        dg.dgmoe_block_forward_noalloc(dims, dg.dgmoe_block_weights(), y, dg.DGMOE_BF16, L, None,
                                       None, y, dg.DGMOE_F32, None, None)
    assert e.value.status == dg.DGMOE_ERR_WORKSPACE
