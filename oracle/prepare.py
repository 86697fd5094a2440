"""Oracle: turn drawn float32 weights into the float64 values the block uses.

TEST INFRASTRUCTURE ONLY (see the package docstring).

For quantised formats each matrix goes through the oracle's own packer and
back (oracle.quant.pack -> oracle.quant.unpack), so the values are exactly
scale*q + bias of the oracle's bytes.  bf16 / f32 matrices are used as drawn.
Expert matrices can be prepared lazily, one expert at a time, so that a test on
a few sampled positions only pays for the experts those positions use.
"""
import numpy as np

from . import fp4, quant


def matrix_values(w32, fmt):
    """float64 values of one [rows, cols] matrix stored in format fmt."""
    if fmt in ("q4", "q8", "q4g32", "q6"):
        rows, cols = w32.shape
        codes, sb = quant.pack(w32, fmt)
        return quant.unpack(codes, sb, fmt, rows, cols)
    if fmt == "nvfp4":
        codes, sbyte, gs, _ = fp4.quantize_nvfp4(w32)
        return fp4.dequantize_nvfp4(codes, sbyte, gs)
    if fmt in ("bf16", "f32"):
        return np.asarray(w32, np.float64)
    raise ValueError(fmt)


class LazyExperts:
    """Mapping e -> float64 matrix, computed on first use from a draw function."""

    def __init__(self, draw, fmt):
        self._draw, self._fmt, self._cache = draw, fmt, {}

    def __getitem__(self, e):
        e = int(e)
        if e not in self._cache:
            self._cache[e] = matrix_values(self._draw(e), self._fmt)
        return self._cache[e]


def block_weights(w32, cfg, expert_source=None):
    """float64 weight dict for oracle.block.block_forward.

    w32: dict of float32 arrays as drawn; cfg: workload dict with keys E,
    weight_fmt (the experts' format), router_fmt and optionally dense_fmt (the
    dense MLP's, default weight_fmt).  If expert_source is given (a function e ->
    (gate_up, down) float32), experts are prepared lazily from it instead of
    from w32["expert_gate_up"] / w32["expert_down"].
    """
    fmt, rfmt = cfg["weight_fmt"], cfg["router_fmt"]
    dfmt = cfg.get("dense_fmt") or fmt  # the dense MLP's own format, else the experts'
    out = {
        "router": matrix_values(w32["router"], rfmt),
        "router_scale": np.asarray(w32["router_scale"], np.float64),
        "per_expert_scale": np.asarray(w32["per_expert_scale"], np.float64),
        "router_bias": None if w32.get("router_bias") is None
        else np.asarray(w32["router_bias"], np.float64),
        "dense_gate_up": matrix_values(w32["dense_gate_up"], dfmt),
        "dense_down": matrix_values(w32["dense_down"], dfmt),
        "layer_scalar": float(w32["layer_scalar"]),
        "n_experts": int(cfg["E"]),
    }
    for n in ("pre_ff_norm", "pre_ff_norm_2", "post_ff_norm_1", "post_ff_norm_2", "post_ff_norm"):
        out[n] = np.asarray(w32[n], np.float64)
    if expert_source is None:
        gu, dn = w32["expert_gate_up"], w32["expert_down"]
        out["expert_gate_up"] = LazyExperts(lambda e: gu[e], fmt)
        out["expert_down"] = LazyExperts(lambda e: dn[e], fmt)
    else:
        out["expert_gate_up"] = LazyExperts(lambda e: expert_source(e)[0], fmt)
        out["expert_down"] = LazyExperts(lambda e: expert_source(e)[1], fmt)
    return out
