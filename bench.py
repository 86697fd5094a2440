#!/usr/bin/env python3
"""Throughput of the libdgmoe block forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config canvas256_q4]

A step is one dgmoe_block_forward over one canvas: RMSNorm, router, top-k,
expert plan, grouped gate_up+GeGLU, grouped down+scatter, combine + post-norms
+ layer_scalar.  Inputs and packed weights are resident in HBM before timing;
two copies of the weights alternate between steps so that the 256 MB
last-level cache cannot hold the 442 MB stream.  Prints one JSON line.

After the block, the canvas head at full size (vocabulary 262144) is timed on
its own and reported under "head": dgmoe_tail (final norm, tied head, softcap,
entropy / argmax, statistics only), dgmoe_soft_embed and dgmoe_sc_input, each
with its roofline and, for the tail, the oracle's time on a few positions.
"""
import argparse
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
MFMA_F16_PEAK_TFLOPS = 2500.0  # MI355X dense fp16 MFMA
METRIC = "canvas-tokens/s per MoE block at canvas 256; % of HBM/MFMA roofline"
COUNTERS = os.path.join(ROOT, "profiles", "counters_gemm_canvas256_q4.txt")


def packed_bytes(rows, cols, fmt):
    if fmt == "q4":
        return rows * cols // 2 + rows * (cols // 64) * 4
    if fmt == "q4g32":
        return rows * cols // 2 + rows * (cols // 32) * 4
    if fmt == "nvfp4":
        return rows * cols // 2 + rows * cols // 16 + 64
    if fmt == "q6":
        return rows * cols * 3 // 4 + rows * (cols // 32) * 4
    if fmt == "q8":
        return rows * cols + rows * (cols // 64) * 4
    if fmt == "bf16":
        return rows * cols * 2
    return rows * cols * 4


def algorithmic(cfg, touched):
    """Bytes and flops the block must move / do (one step), and the gate_up kernel's share."""
    L, D, E, k, I, Id = cfg["L"], cfg["D"], cfg["E"], cfg["k"], cfg["I"], cfg["Id"]
    f, rf = cfg["weight_fmt"], cfg["router_fmt"]
    fd = cfg.get("dense_fmt") or f
    xb = 2 if cfg["x_dtype"] == "bf16" else 4
    gu_e = packed_bytes(2 * I, D, f)
    dn_e = packed_bytes(D, I, f)
    gu_d = packed_bytes(2 * Id, D, fd)
    dn_d = packed_bytes(D, Id, fd)
    small = packed_bytes(E, D, rf) + 4 * (6 * D + E)
    block_bytes = touched * (gu_e + dn_e) + gu_d + dn_d + small + L * D * xb + L * D * 2
    block_flops = L * (2 * k * 3 * D * I + 2 * 3 * D * Id + 2 * D * E)
    gate_up_bytes = touched * gu_e + gu_d + 2 * L * D * 2 + (L * k * I + L * Id) * 2
    gate_up_flops = 2 * (L * k * 2 * I * D + L * 2 * Id * D)
    return dict(block_bytes=block_bytes, block_flops=block_flops, gate_up_bytes=gate_up_bytes,
                gate_up_flops=gate_up_flops, gate_up_per_expert=gu_e, down_per_expert=dn_e)


def fmt_label(f):
    return {"q4": "q4g64", "q8": "q8g64"}.get(f, f)


def gate_up_kernel(cfg):
    """The gate_up launch(es) of a workload.  The library takes tall tiles from
    32 pairs per expert on average (q4 group-64 weights); a bf16 or 8-bit dense
    MLP beside 4-bit experts on short tiles shares their launch (k_split_q4);
    any other pair of different formats takes a launch each."""
    L, k, E = cfg["L"], cfg["k"], cfg["E"]
    f = cfg["weight_fmt"]
    fd = cfg.get("dense_fmt") or f
    tall = f == "q4" and L * k >= 32 * E

    def name(fmt):
        if fmt == "q4":
            return "k_tall_q4<gate_up>" if tall else "k_grouped_q4<gate_up, q4g64>"
        return f"k_grouped_q4<gate_up, {fmt_label(fmt)}>"

    if fd == f:
        return name(f) + f" (grouped {fmt_label(f)} gate_up GEMM + GeGLU)"
    if fd in ("bf16", "q8") and f in ("q4", "q4g32", "nvfp4", "q6") and not tall:
        return (f"k_split_q4<gate_up, {fmt_label(f)}, {fmt_label(fd)}> (dense MLP's "
                f"{fmt_label(fd)} tiles, then the experts' {fmt_label(f)} tiles: grouped gate_up "
                f"GEMM + GeGLU)")
    return (name(f) + f" (experts, {fmt_label(f)}) then " + name(fd) +
            f" (dense MLP, {fmt_label(fd)}): grouped gate_up GEMMs + GeGLU")


def roofline(bytes_, flops, seconds):
    t_hbm = bytes_ / (HBM_PEAK_GBS * 1e9)
    t_mfma = flops / (MFMA_F16_PEAK_TFLOPS * 1e12)
    if t_hbm >= t_mfma:
        a = bytes_ / seconds / 1e9
        return {"bound": "hbm", "achieved": round(a, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(a / HBM_PEAK_GBS, 4)}
    a = flops / seconds / 1e12
    return {"bound": "mfma", "achieved": round(a, 2), "peak": MFMA_F16_PEAK_TFLOPS,
            "unit": "TFLOP/s", "frac": round(a / MFMA_F16_PEAK_TFLOPS, 4)}


def kernel_source_hash():
    h = hashlib.sha256()
    for f in ("gemm.hip", "common.h", "kernels.h"):
        h.update(open(os.path.join(ROOT, "moe_denoise_forward_amd", "csrc", f), "rb").read())
    return h.hexdigest()[:16]


def counter_traffic(workload):
    """HBM bytes per gate_up launch from the committed rocprofv3 counter summary, if
    it was taken on the current kernel source and this workload; else None."""
    try:
        text = open(COUNTERS).read()
    except OSError:
        return None
    kv = dict(re.findall(r"^(workload|kernel_source_hash|traffic_bytes_per_launch): (\S+)$", text,
                         re.M))
    if kv.get("kernel_source_hash") != kernel_source_hash() or kv.get("workload") != workload:
        return None
    return int(kv["traffic_bytes_per_launch"])


def cpu_baseline(cfg, w32, x, n_pos):
    """The oracle, as it stands, on the first n_pos positions of the same workload."""
    from oracle import block, prepare
    try:
        from threadpoolctl import threadpool_info
        cores = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    except Exception:
        cores = 1
    t0 = time.perf_counter()
    wt = prepare.block_weights(w32, cfg)
    block.block_forward(x[:n_pos], wt, cfg["k"])
    dt = time.perf_counter() - t0
    return {"value": round(n_pos / dt, 2), "unit": "tokens/s", "cores": int(cores),
            "kind": "oracle",
            "sample": f"full float64 oracle block (own q4/q8 packing + dequant of every touched "
                      f"expert, router, dense MLP, combine) on {n_pos} of {cfg['L']} positions of "
                      f"{cfg['name']}: {dt:.1f} s"}


def run_stack(args, cfg, dg, synth, torch):
    """A stack of independent blocks applied in sequence (the bf16 output of block l
    is the input of block l + 1), one canvas.  Each layer's router offset sends every
    position to the same k experts (the k largest offsets, far ahead of the logits'
    spread), so only those k experts are drawn and packed; the others are zero codes
    and scales that a correct routing never reads, which the routing check below
    confirms.  A pass is all layers; warm-up and timed counts are in passes."""
    L, D, E, k, nl = cfg["L"], cfg["D"], cfg["E"], cfg["k"], cfg["layers"]
    blocks, hot = [], []
    for layer in range(nl):
        w = synth.draw_weights(cfg, layer, experts=False)
        h = [int(e) for e in np.argsort(-w["router_bias"], kind="stable")[:k]]
        blocks.append(dg.PackedBlock(w, cfg, hot_experts={e: synth.draw_expert(cfg, e, layer)
                                                          for e in h}))
        hot.append(sorted(h))
        print(f"bench: layer {layer + 1}/{nl} packed", file=sys.stderr, flush=True)
    x0 = torch.from_numpy(synth.draw_x(cfg)).cuda().to(torch.bfloat16)
    buf = [x0.clone(), torch.empty_like(x0)]
    idx = torch.empty((nl, L, k), dtype=torch.int32, device="cuda")
    rw = torch.empty((nl, L, k), dtype=torch.float32, device="cuda")
    ws, nws = dg.workspace(blocks[0].dims, L)
    st = torch.cuda.current_stream()

    def run_pass(route_out=False, events=None):
        buf[0].copy_(x0)
        for layer, pb in enumerate(blocks):
            src, dst = buf[layer % 2], buf[(layer + 1) % 2]
            if events is not None:
                dg.dgmoe_block_forward_profiled(pb.dims, pb.struct, src, dg.DGMOE_BF16, L, dst,
                                                dg.DGMOE_BF16, ws, nws, st, events[layer])
            else:
                dg.dgmoe_block_forward(pb.dims, pb.struct, src, dg.DGMOE_BF16, L, None, None, dst,
                                       dg.DGMOE_BF16, idx[layer] if route_out else None,
                                       rw[layer] if route_out else None, ws, nws, st)

    run_pass(route_out=True)
    torch.cuda.synchronize()
    got = idx.cpu().numpy()
    routed_ok = all((np.sort(got[layer], axis=1) == np.array(hot[layer])).all() for layer in range(nl))
    hist = [np.bincount(got[layer].ravel(), minlength=E) for layer in range(nl)]
    for _ in range(args.warmup):
        run_pass()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(st)
    for _ in range(args.steps):
        run_pass()
    e1.record(st)
    torch.cuda.synchronize()
    ms_block = e0.elapsed_time(e1) / (args.steps * nl)
    # one more pass with an event before each kernel of each block
    ev = [dg.HipEvents(dg.PROFILE_EVENTS) for _ in range(nl)]
    run_pass(events=ev)
    torch.cuda.synchronize()
    per_kernel = {n: 0.0 for n in dg.PROFILE_KERNELS}
    for e in ev:
        for j, n in enumerate(dg.PROFILE_KERNELS):
            per_kernel[n] += e.elapsed_ms(j, j + 1) / nl
        e.close()
    alg = algorithmic(cfg, k)
    roof = roofline(alg["gate_up_bytes"], alg["gate_up_flops"], per_kernel["gate_up"] * 1e-3)
    roof["kernel"] = "k_grouped_q4<gate_up> (grouped q4 gate_up GEMM + GeGLU)"
    roof["traffic"] = None
    block_roof = roofline(alg["block_bytes"], alg["block_flops"], ms_block * 1e-3)
    out = {
        "metric": METRIC,
        "value": round(L / (ms_block * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_block * nl, 4),
        "ms_per_block": round(ms_block, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": cfg["name"], "layers": nl, "canvas_tokens": L, "hidden": D,
                   "experts": E, "top_k": k, "expert_inter": cfg["I"], "dense_inter": cfg["Id"],
                   "weights": fmt_label(cfg["weight_fmt"]), "router": fmt_label(cfg["router_fmt"]),
                   "activations": "bf16 (each block's output feeds the next)",
                   "step": "one pass over all layers; value is per block",
                   "parallelism": "none (1 GPU)"},
        "roofline": roof,
        "block_roofline": dict(block_roof, bytes=alg["block_bytes"], flops=alg["block_flops"]),
        "tflops": round(alg["block_flops"] / (ms_block * 1e-3) / 1e12, 2),
        "per_kernel_us": {n: round(v * 1e3, 2) for n, v in per_kernel.items()},
        "routing": {"every_position_to_its_layers_hot_experts": bool(routed_ok),
                    "experts_touched_per_layer": sorted({int((h > 0).sum()) for h in hist}),
                    "positions_per_touched_expert": sorted({int(h.max()) for h in hist})},
        "cpu_baseline": None,
    }
    print(json.dumps(out), flush=True)


def head_algorithmic(cfg):
    """Bytes and flops of the two head calls on the full canvas (the tied table
    read once, its activations and outputs)."""
    L, D, V, I = cfg["L"], cfg["D"], cfg["V"], cfg["Isc"]
    table = packed_bytes(V, D, "q4")
    mlp = packed_bytes(2 * I, D, "q4") + packed_bytes(D, I, "q4")
    return {
        "tail": dict(bytes=table + L * D * 2 + 4 * D + L * 16, flops=2 * L * D * V),
        "soft_embed": dict(bytes=table + L * V * 4 + L * D * 4, flops=2 * L * V * D),
        "sc_input": dict(bytes=table + mlp + L * V * 4 + 4 * D + L * 4 + L * D * 4,
                         flops=2 * L * V * D + 2 * L * 3 * D * I),
    }


def head_cpu_baseline(cfg, e32, hw, x, T, n_rows):
    """The oracle's tail, as it stands, on the first n_rows positions (its own
    packing of the table is done before the clock starts)."""
    from oracle import head
    try:
        from threadpoolctl import threadpool_info
        cores = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    except Exception:
        cores = 1
    table = head.EmbedTable.pack_q4(e32)
    t0 = time.perf_counter()
    head.tail(x[:n_rows], hw["final_norm"], table, T)
    dt = time.perf_counter() - t0
    return {"value": round(n_rows / dt, 3), "unit": "positions/s", "cores": int(cores),
            "kind": "oracle",
            "sample": f"float64 oracle tail (dequantise the whole 262144 x 2816 table in row "
                      f"blocks, tied logits, softcap, entropy / argmax) on {n_rows} of "
                      f"{cfg['L']} positions: {dt:.1f} s"}


def run_head(args, dg, synth, torch):
    """The canvas head at full size: the forward tail (statistics only) and the
    self-conditioned canvas input, each timed alone; returns the JSON object."""
    cfg = synth.head_config("head_full")
    L, D, V = cfg["L"], cfg["D"], cfg["V"]
    print("bench: head weights", file=sys.stderr, flush=True)
    e32 = synth.draw_embed(cfg)
    hw = synth.draw_head_weights(cfg)
    ph = dg.PackedHead(dict(hw, embed=e32), cfg)
    x = synth.draw_tail_x(cfg, e32)
    xt = torch.from_numpy(x).cuda().to(torch.bfloat16)
    yl = torch.from_numpy(synth.draw_sc_logits(cfg)).cuda()
    ids = torch.from_numpy(synth.draw_canvas_ids(cfg)).cuda()
    H = torch.empty(L, device="cuda")
    am = torch.empty(L, dtype=torch.int32, device="cuda")
    soft = torch.empty((L, D), device="cuda")
    out = torch.empty((L, D), device="cuda")
    ws, nws = dg.head_workspace(ph.dims, L)
    st = torch.cuda.current_stream()
    T = cfg["T"]
    calls = {
        "tail": lambda: dg.dgmoe_tail(ph.dims, ph.struct, xt, dg.DGMOE_BF16, L, T, H, am, None,
                                      None, None, ws, nws, st),
        "soft_embed": lambda: dg.dgmoe_soft_embed(ph.dims, ph.struct, yl, L, soft, ws, nws, st),
        "sc_input": lambda: dg.dgmoe_sc_input(ph.dims, ph.struct, ids, yl, L, out, ws, nws, st),
    }
    alg = head_algorithmic(cfg)
    res = {"workload": cfg["name"], "canvas_tokens": L, "hidden": D, "vocab": V,
           "sc_inter": cfg["Isc"], "table": "q4g64", "temperature": T}
    n = max(3, args.head_steps)
    for name, fn in calls.items():
        for _ in range(3):
            fn()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(st)
        for _ in range(n):
            fn()
        e1.record(st)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / n
        r = roofline(alg[name]["bytes"], alg[name]["flops"], ms * 1e-3)
        res[name] = {"ms": round(ms, 4), "positions_per_s": round(L / (ms * 1e-3), 1),
                     "tflops": round(alg[name]["flops"] / (ms * 1e-3) / 1e12, 2),
                     "roofline": dict(r, bytes=alg[name]["bytes"], flops=alg[name]["flops"])}
    flags = dg.dgmoe_head_check_workspace(ph.dims, L, ws)
    res["flags"] = flags
    res["steps"] = n
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = head_cpu_baseline(cfg, e32, hw, x, T, args.head_cpu_rows)
    return res


def attn_counts(cfg):
    """Keys per canvas row, flops (QK^T and PV) and the algorithmic bytes of one
    layer's canvas attention: the raw projections in, the visible committed
    K / V rows (fp16) read once, the output written once (bf16)."""
    L, H, Hkv, hd, kv = cfg["L"], cfg["H"], cfg["Hkv"], cfg["hd"], cfg["kv_len"]
    s0 = max(0, kv - cfg["window"]) if cfg["window"] > 0 else 0
    n_keys = kv - s0 + L
    flops = 4 * H * L * n_keys * hd
    proj = L * (H + Hkv + (0 if cfg["kind"] == "full" else Hkv)) * hd * 2
    nbytes = proj + 2 * Hkv * (kv - s0) * hd * 2 + L * H * hd * 2
    return n_keys, flops, nbytes


def attn_cpu_baseline(cfg, d, rows):
    """The oracle's attention, as it stands, on the first `rows` canvas rows
    (every key of the layer, every head)."""
    from oracle import attention as oa
    try:
        from threadpoolctl import threadpool_info
        cores = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    except Exception:
        cores = 1
    kc, vc = d["k_cache"].astype(np.float64), d["v_cache"].astype(np.float64)
    kv = cfg["kv_len"]
    theta, n_rot, stride, den, _ = oa.layer_params(cfg["kind"], cfg["hd"])
    t0 = time.perf_counter()
    # the canvas keys are every row's keys: norm and rotate all of them, then
    # attend with the first `rows` queries
    q, k, v = oa.canvas_qkv(d["qraw"], d["kraw"], d["vraw"], d["w_q"], d["w_k"], kv, cfg["H"],
                            cfg["Hkv"], cfg["hd"], theta, n_rot, stride, den)
    oa.attend(q[:, :rows], k, v, kc, vc, kv, cfg["window"])
    dt = time.perf_counter() - t0
    return {"value": round(rows / dt, 2), "unit": "canvas rows/s", "cores": int(cores),
            "kind": "oracle",
            "sample": f"float64 oracle attention of {rows} of {cfg['L']} canvas rows "
                      f"({cfg['name']}): {dt:.2f} s"}


def run_attention(args, dg, synth, torch):
    """One layer's denoise attention at the model's two layer shapes, a 256-row
    canvas after a 4096-position prompt; each timed alone (HIP events on the
    library's stream around `steps` calls)."""
    res = {}
    st = torch.cuda.current_stream()
    for name in ("attn_sliding", "attn_full"):
        cfg = synth.attn_config(name)
        d = synth.draw_attn(cfg)
        L, H, hd, kv = cfg["L"], cfg["H"], cfg["hd"], cfg["kv_len"]
        dims = dg.attn_dims_for(cfg)

        def dev(x):
            return None if x is None else torch.from_numpy(x).cuda().to(torch.bfloat16)

        q, k, v = dev(d["qraw"]), dev(d["kraw"]), dev(d["vraw"])
        wq, wk = torch.from_numpy(d["w_q"]).cuda(), torch.from_numpy(d["w_k"]).cuda()
        kc = torch.from_numpy(d["k_cache"].view(np.int16)).cuda()
        vc = torch.from_numpy(d["v_cache"].view(np.int16)).cuda()
        out = torch.empty((L, H * hd), dtype=torch.bfloat16, device="cuda")
        ws, nws = dg.attn_workspace(dims, L, kv)
        rows = d["k_cache"].shape[1]

        def call():
            dg.dgmoe_attn_denoise(dims, q, k, v, dg.DGMOE_BF16, L, wq, wk, kc, vc, rows, kv, out,
                                  dg.DGMOE_BF16, ws, nws, st)

        for _ in range(3):
            call()
        n = max(3, args.attn_steps)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(st)
        for _ in range(n):
            call()
        e1.record(st)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / n
        n_keys, flops, nbytes = attn_counts(cfg)
        r = roofline(nbytes, flops, ms * 1e-3)
        res[name] = {"kind": cfg["kind"], "canvas_tokens": L, "committed": kv, "keys": n_keys,
                     "heads": H, "kv_heads": cfg["Hkv"], "head_dim": hd, "window": cfg["window"],
                     "ms": round(ms, 4), "tflops": round(flops / (ms * 1e-3) / 1e12, 2),
                     "roofline": dict(r, bytes=nbytes, flops=flops), "steps": n}
        if not args.no_cpu_baseline:
            res[name]["cpu_baseline"] = attn_cpu_baseline(cfg, d, args.attn_cpu_rows)
        del q, k, v, kc, vc, out, ws
        torch.cuda.empty_cache()
    return res


def profiled_region(args, dg, torch, step):
    """Run the steps again with an event before each kernel of the block
    (dgmoe_block_forward_profiled).  Returns (per-kernel average times in ms,
    average step time in ms)."""
    n = args.steps
    ev = [dg.HipEvents(dg.PROFILE_EVENTS) for _ in range(n)]
    torch.cuda.synchronize()
    for i in range(n):
        step(i, ev[i])
    torch.cuda.synchronize()
    per_kernel = {k: 0.0 for k in dg.PROFILE_KERNELS}
    step_ms = 0.0
    for e in ev:
        for j, k in enumerate(dg.PROFILE_KERNELS):
            per_kernel[k] += e.elapsed_ms(j, j + 1) / n
        step_ms += e.elapsed_ms(0, len(dg.PROFILE_KERNELS)) / n
        e.close()
    return per_kernel, step_ms


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", default="canvas256_q4")
    ap.add_argument("--cpu-positions", type=int, default=None,
                    help="positions the CPU oracle baseline runs on (default: the whole canvas)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-rotate", action="store_true")
    ap.add_argument("--settle-ms", type=float, default=50.0,
                    help="untimed steps run for this long before the warm-up steps, so the GPU's "
                         "clocks have left their idle state when the timed region starts")
    ap.add_argument("--no-head", action="store_true",
                    help="skip the canvas head (forward tail, self-conditioned input)")
    ap.add_argument("--head-steps", type=int, default=20)
    ap.add_argument("--no-attn", action="store_true",
                    help="skip the denoise attention measurement")
    ap.add_argument("--attn-steps", type=int, default=50)
    ap.add_argument("--attn-cpu-rows", type=int, default=64,
                    help="canvas rows of the oracle attention timed for its cpu_baseline")
    ap.add_argument("--head-cpu-rows", type=int, default=64,
                    help="positions the oracle's tail is timed on for the head's CPU baseline")
    ap.add_argument("--copy-mb", type=int, default=0,
                    help="only run a plain device copy of this many MB --steps times (the "
                         "reference kernel that scales the HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); this library has no "
              "multi-GPU path.", file=sys.stderr)
        sys.exit(2)

    import torch
    from moe_denoise_forward_amd import dgmoe as dg
    from moe_denoise_forward_amd import synth

    torch.cuda.set_device(0)
    if args.copy_mb:
        n = args.copy_mb * 1000 * 1000 // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(args.steps):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_per_launch": n * 4, "launches": args.steps}), flush=True)
        return
    cfg = synth.config(args.config)
    if cfg["layers"] > 1:
        run_stack(args, cfg, dg, synth, torch)
        return
    L, D, k = cfg["L"], cfg["D"], cfg["k"]
    w32 = synth.draw_weights(cfg)
    x = synth.draw_x(cfg)
    sets = [dg.PackedBlock(w32, cfg)]
    if not args.no_rotate:
        sets.append(sets[0].clone())
    xt = torch.from_numpy(x).cuda()
    xdt = dg.DGMOE_F32
    if cfg["x_dtype"] == "bf16":
        xt, xdt = xt.to(torch.bfloat16), dg.DGMOE_BF16
    y = torch.empty((L, D), dtype=torch.bfloat16, device="cuda")
    idx = torch.empty((L, k), dtype=torch.int32, device="cuda")
    rw = torch.empty((L, k), dtype=torch.float32, device="cuda")
    ws, nws = dg.workspace(sets[0].dims, L)
    st = torch.cuda.current_stream()

    def step(i, events=None):
        pb = sets[i % len(sets)]
        if events is None:
            dg.dgmoe_block_forward(pb.dims, pb.struct, xt, xdt, L, None, None, y, dg.DGMOE_BF16,
                                   None, None, ws, nws, st)
        else:
            dg.dgmoe_block_forward_profiled(pb.dims, pb.struct, xt, xdt, L, y, dg.DGMOE_BF16, ws,
                                            nws, st, events)

    # routing of this canvas (for the touched-expert count)
    dg.dgmoe_block_forward(sets[0].dims, sets[0].struct, xt, xdt, L, None, None, y, dg.DGMOE_BF16,
                           idx, rw, ws, nws, st)
    torch.cuda.synchronize()
    hist = np.bincount(idx.cpu().numpy().ravel(), minlength=cfg["E"])
    touched = int((hist > 0).sum())

    t_settle = time.perf_counter()
    while (time.perf_counter() - t_settle) * 1e3 < args.settle_ms:
        for i in range(20):
            step(i)
        torch.cuda.synchronize()
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    # timed region: K whole steps; an event after each step gives the per-step
    # times (an event record adds no work to the stream)
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    torch.cuda.synchronize()
    evs[0].record(st)
    for i in range(args.steps):
        step(i)
        evs[i + 1].record(st)
    torch.cuda.synchronize()
    ms = evs[0].elapsed_time(evs[-1]) / args.steps
    step_ms = [evs[i].elapsed_time(evs[i + 1]) for i in range(args.steps)]
    p10, p50, p90 = (float(v) for v in np.percentile(step_ms, [10, 50, 90]))

    # second timed region, same steps, with an event before each kernel
    per_kernel, ms_prof = profiled_region(args, dg, torch, step)

    alg = algorithmic(cfg, touched)
    roof = roofline(alg["gate_up_bytes"], alg["gate_up_flops"], per_kernel["gate_up"] * 1e-3)
    roof["kernel"] = gate_up_kernel(cfg)
    roof["bytes_per_launch"] = alg["gate_up_bytes"]
    roof["launch_us"] = round(per_kernel["gate_up"] * 1e3, 2)
    roof["traffic"] = counter_traffic(cfg["name"])
    block_roof = roofline(alg["block_bytes"], alg["block_flops"], ms * 1e-3)

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(cfg, w32, x, args.cpu_positions or L)
    n_sets = len(sets)
    head = None
    if not args.no_head and cfg["name"] == "canvas256_q4":
        del sets, w32
        torch.cuda.empty_cache()
        head = run_head(args, dg, synth, torch)

    out = {
        "metric": METRIC,
        "value": round(L / (ms * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "settle_ms": args.settle_ms,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": cfg["name"], "canvas_tokens": L, "hidden": D,
                   "experts": cfg["E"], "top_k": k, "expert_inter": cfg["I"],
                   "dense_inter": cfg["Id"],
                   "weights": fmt_label(cfg["weight_fmt"]),
                   "dense_weights": fmt_label(cfg.get("dense_fmt") or cfg["weight_fmt"]),
                   "router": fmt_label(cfg["router_fmt"]), "activations": cfg["x_dtype"],
                   "touched_experts": touched, "weight_sets_rotated": n_sets,
                   "parallelism": "none (1 GPU)"},
        "roofline": roof,
        "block_roofline": dict(block_roof, bytes=alg["block_bytes"], flops=alg["block_flops"]),
        "tflops": round(alg["block_flops"] / (ms * 1e-3) / 1e12, 2),
        "gbs": round(alg["block_bytes"] / (ms * 1e-3) / 1e9, 1),
        "per_kernel_us": {n: round(v * 1e3, 2) for n, v in per_kernel.items()},
        "step_ms_p10_median_p90": [round(p10, 4), round(p50, 4), round(p90, 4)],
        "profiled_step_ms": round(ms_prof, 4),
        "expert_load": {"min": int(hist.min()), "mean": round(float(hist.mean()), 2),
                        "max": int(hist.max())},
        "cpu_baseline": cpu,
    }
    if head is not None:
        out["head"] = head
    if not args.no_attn and cfg["name"] == "canvas256_q4":
        out["attention"] = run_attention(args, dg, synth, torch)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
