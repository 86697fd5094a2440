"""Python binding of libdgmoe (ctypes).  Argument marshalling only.

Every function here has the name and the argument order of the C entry point
declared in include/dgmoe.h.  Tensor arguments may be torch tensors (their
data_ptr() is passed), plain integers (device addresses) or None (NULL).
`stream` defaults to torch's current stream on the current device.  A status
other than DGMOE_OK raises DgmoeError.  There is no fallback: if the HIP
library is not built, importing this module raises.

`PackedBlock` keeps one block's weights in device memory, packed by the
library's own GPU packer (dgmoe_pack), and fills the weight struct.
"""
import ctypes
import os

import numpy as np

# PyTorch's HIP runtime must be in the process before the library is loaded,
# so that libdgmoe.so binds to that same runtime (see build._runtime_link).
import torch  # noqa: F401,E402

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libdgmoe.so")
if not os.path.exists(LIB_PATH):
    raise ImportError(f"libdgmoe.so is not built ({LIB_PATH}); run python -m moe_denoise_forward_amd.build")
_lib = ctypes.CDLL(LIB_PATH)

DGMOE_OK, DGMOE_ERR_NULL_ARG, DGMOE_ERR_BAD_DIMS, DGMOE_ERR_BAD_DTYPE = 0, 1, 2, 3
DGMOE_ERR_MISALIGNED, DGMOE_ERR_WORKSPACE, DGMOE_ERR_HIP, DGMOE_ERR_DEVICE = 4, 5, 6, 7
DGMOE_FLAG_SYNC_TIMEOUT, DGMOE_FLAG_FP16_RANGE, DGMOE_FLAG_ROUTE_OVERFLOW = 1, 2, 4
DGMOE_FLAG_INDEX = 8
DGMOE_F32, DGMOE_BF16, DGMOE_F16, DGMOE_Q4G64, DGMOE_Q8G64, DGMOE_Q4G32 = 0, 1, 2, 3, 4, 5
DGMOE_NVFP4, DGMOE_Q6G32 = 6, 7
FMT = {"f32": DGMOE_F32, "bf16": DGMOE_BF16, "f16": DGMOE_F16, "q4": DGMOE_Q4G64, "q8": DGMOE_Q8G64,
       "q4g32": DGMOE_Q4G32, "nvfp4": DGMOE_NVFP4, "q6": DGMOE_Q6G32}
PACKED = ("q4", "q8", "q4g32", "nvfp4", "q6")
# formats whose stacked expert tensors hold each expert's matrix in one piece
# that differs from packing the stacked rows as one matrix (a per-matrix tensor
# scale; the two code planes)
PER_EXPERT = ("nvfp4", "q6")


def scale_bytes(rows, cols, fmt):
    """Bytes of the scale_bias array of one [rows, cols] matrix in a packed
    format: fp16 (scale, bias) pairs, or nvfp4's E4M3 bytes and 64-byte trailer."""
    if fmt == "nvfp4":
        return rows * cols // 16 + 64
    return 4 * (rows * cols // (32 if fmt in ("q4g32", "q6") else 64))

# every symbol the header declares
EXPORTS = ("dgmoe_workspace_size", "dgmoe_route", "dgmoe_moe_ffn", "dgmoe_block_forward",
           "dgmoe_packed_bytes", "dgmoe_pack", "dgmoe_unpack", "dgmoe_status_str",
           "dgmoe_abi_version", "dgmoe_last_hip_error", "dgmoe_block_forward_profiled",
           "dgmoe_check_workspace", "dgmoe_debug_force_stamp_timeout", "dgmoe_debug_set_tall_min",
           "dgmoe_block_forward_noalloc", "dgmoe_noalloc_max_bytes",
           "dgmoe_head_workspace_size", "dgmoe_tail", "dgmoe_soft_embed", "dgmoe_sc_input",
           "dgmoe_head_check_workspace", "dgmoe_attn_workspace_size", "dgmoe_attn_denoise")
ABI_VERSION = 9
PROFILE_EVENTS = 5
PROFILE_KERNELS = ("front", "gate_up", "down", "combine")


class dgmoe_dims(ctypes.Structure):
    _fields_ = [("hidden", ctypes.c_int32), ("n_experts", ctypes.c_int32),
                ("top_k", ctypes.c_int32), ("expert_inter", ctypes.c_int32),
                ("dense_inter", ctypes.c_int32), ("rms_eps", ctypes.c_float)]


class dgmoe_matrix(ctypes.Structure):
    _fields_ = [("dtype", ctypes.c_int32), ("data", ctypes.c_void_p),
                ("scale_bias", ctypes.c_void_p)]


class dgmoe_block_weights(ctypes.Structure):
    _fields_ = [("router", dgmoe_matrix), ("router_scale", ctypes.c_void_p),
                ("per_expert_scale", ctypes.c_void_p), ("router_bias", ctypes.c_void_p),
                ("expert_gate_up", dgmoe_matrix), ("expert_down", dgmoe_matrix),
                ("dense_gate_up", dgmoe_matrix), ("dense_down", dgmoe_matrix),
                ("pre_ff_norm", ctypes.c_void_p), ("pre_ff_norm_2", ctypes.c_void_p),
                ("post_ff_norm_1", ctypes.c_void_p), ("post_ff_norm_2", ctypes.c_void_p),
                ("post_ff_norm", ctypes.c_void_p), ("layer_scalar", ctypes.c_float)]


class dgmoe_head_dims(ctypes.Structure):
    _fields_ = [("hidden", ctypes.c_int32), ("vocab", ctypes.c_int32),
                ("sc_inter", ctypes.c_int32), ("rms_eps", ctypes.c_float)]


class dgmoe_attn_dims(ctypes.Structure):
    _fields_ = [("n_heads", ctypes.c_int32), ("n_kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("window", ctypes.c_int32),
                ("rope_pairs", ctypes.c_int32), ("rope_stride", ctypes.c_int32),
                ("rope_theta", ctypes.c_float), ("rope_den", ctypes.c_float),
                ("rms_eps", ctypes.c_float)]


class dgmoe_head_weights(ctypes.Structure):
    _fields_ = [("embed", dgmoe_matrix), ("final_norm", ctypes.c_void_p),
                ("sc_gate_up", dgmoe_matrix), ("sc_down", dgmoe_matrix),
                ("sc_pre_norm", ctypes.c_void_p)]


_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_I32 = ctypes.c_int32
_SZ = ctypes.c_size_t
_DIMS = ctypes.POINTER(dgmoe_dims)
_W = ctypes.POINTER(dgmoe_block_weights)
_sig = {
    "dgmoe_workspace_size": (_SZ, [_DIMS, _I64]),
    "dgmoe_route": (_I32, [_DIMS, _W, _P, _I32, _I64, _P, _P, _P, _P, _SZ, _P]),
    "dgmoe_moe_ffn": (_I32, [_DIMS, _W, _P, _I32, _I64, _P, _P, _P, _P, _SZ, _P]),
    "dgmoe_block_forward": (_I32, [_DIMS, _W, _P, _I32, _I64, _P, _P, _P, _I32, _P, _P, _P, _SZ, _P]),
    "dgmoe_packed_bytes": (_SZ, [_I64, _I64, _I32]),
    "dgmoe_pack": (_I32, [_P, _I64, _I64, _I32, _P, _P, _P]),
    "dgmoe_unpack": (_I32, [_P, _P, _I64, _I64, _I32, _I32, _P, _P]),
    "dgmoe_status_str": (ctypes.c_char_p, [_I32]),
    "dgmoe_abi_version": (ctypes.c_int, []),
    "dgmoe_last_hip_error": (ctypes.c_char_p, []),
    "dgmoe_block_forward_profiled": (_I32, [_DIMS, _W, _P, _I32, _I64, _P, _I32, _P, _SZ, _P,
                                            ctypes.POINTER(ctypes.c_void_p), _I32]),
    "dgmoe_check_workspace": (_I32, [_DIMS, _I64, _P, ctypes.POINTER(ctypes.c_uint32), _P]),
    "dgmoe_debug_force_stamp_timeout": (None, [_I32]),
    "dgmoe_debug_set_tall_min": (_I32, [_I32]),
    "dgmoe_block_forward_noalloc": (_I32, [_DIMS, _W, _P, _I32, _I64, _P, _P, _P, _I32, _P, _P, _P]),
    "dgmoe_noalloc_max_bytes": (_SZ, []),
    "dgmoe_head_workspace_size": (_SZ, [ctypes.POINTER(dgmoe_head_dims), _I64]),
    "dgmoe_tail": (_I32, [ctypes.POINTER(dgmoe_head_dims), ctypes.POINTER(dgmoe_head_weights), _P,
                          _I32, _I64, ctypes.c_float, _P, _P, _P, _P, _P, _P, _SZ, _P]),
    "dgmoe_soft_embed": (_I32, [ctypes.POINTER(dgmoe_head_dims), ctypes.POINTER(dgmoe_head_weights),
                                _P, _I64, _P, _P, _SZ, _P]),
    "dgmoe_sc_input": (_I32, [ctypes.POINTER(dgmoe_head_dims), ctypes.POINTER(dgmoe_head_weights),
                              _P, _P, _I64, _P, _P, _SZ, _P]),
    "dgmoe_head_check_workspace": (_I32, [ctypes.POINTER(dgmoe_head_dims), _I64, _P,
                                          ctypes.POINTER(ctypes.c_uint32), _P]),
    "dgmoe_attn_workspace_size": (_SZ, [ctypes.POINTER(dgmoe_attn_dims), _I64, _I64]),
    "dgmoe_attn_denoise": (_I32, [ctypes.POINTER(dgmoe_attn_dims), _P, _P, _P, _I32, _I64, _P, _P,
                                  _P, _P, _I64, _I64, _P, _I32, _P, _SZ, _P]),
}
for _n, (_r, _a) in _sig.items():
    _f = getattr(_lib, _n)
    _f.restype, _f.argtypes = _r, _a


class DgmoeError(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        extra = f" [{dgmoe_last_hip_error()}]" if status == DGMOE_ERR_HIP else ""
        super().__init__(f"{where}: {dgmoe_status_str(status)} (status {status}){extra}")


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(s):
    if s is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(s, int):
        return s
    return s.cuda_stream


def _check(status, where):
    if status != DGMOE_OK:
        raise DgmoeError(status, where)


def make_dims(D, E, k, I, Id, eps=1e-6):
    return dgmoe_dims(D, E, k, I, Id, eps)


def dgmoe_abi_version():
    return _lib.dgmoe_abi_version()


def dgmoe_last_hip_error():
    return _lib.dgmoe_last_hip_error().decode()


def dgmoe_status_str(s):
    return _lib.dgmoe_status_str(int(s)).decode()


def dgmoe_workspace_size(dims, L):
    return _lib.dgmoe_workspace_size(ctypes.byref(dims), int(L))


def dgmoe_packed_bytes(rows, cols, fmt):
    return _lib.dgmoe_packed_bytes(int(rows), int(cols), int(fmt))


def dgmoe_route(dims, w, x, x_dtype, L, topk_idx, topk_w, logits, ws, ws_bytes, stream=None):
    _check(_lib.dgmoe_route(ctypes.byref(dims), ctypes.byref(w), _ptr(x), int(x_dtype), int(L),
                            _ptr(topk_idx), _ptr(topk_w), _ptr(logits), _ptr(ws), int(ws_bytes),
                            _stream(stream)), "dgmoe_route")


def dgmoe_moe_ffn(dims, w, x, x_dtype, L, topk_idx, topk_w, moe_out, ws, ws_bytes, stream=None):
    _check(_lib.dgmoe_moe_ffn(ctypes.byref(dims), ctypes.byref(w), _ptr(x), int(x_dtype), int(L),
                              _ptr(topk_idx), _ptr(topk_w), _ptr(moe_out), _ptr(ws), int(ws_bytes),
                              _stream(stream)), "dgmoe_moe_ffn")


def dgmoe_block_forward(dims, w, x, x_dtype, L, force_idx, force_w, y, y_dtype, topk_idx_out,
                        topk_w_out, ws, ws_bytes, stream=None):
    _check(_lib.dgmoe_block_forward(ctypes.byref(dims), ctypes.byref(w), _ptr(x), int(x_dtype),
                                    int(L), _ptr(force_idx), _ptr(force_w), _ptr(y), int(y_dtype),
                                    _ptr(topk_idx_out), _ptr(topk_w_out), _ptr(ws), int(ws_bytes),
                                    _stream(stream)), "dgmoe_block_forward")


def dgmoe_block_forward_noalloc(dims, w, x, x_dtype, L, force_idx, force_w, y, y_dtype,
                                topk_idx_out, topk_w_out, stream=None):
    _check(_lib.dgmoe_block_forward_noalloc(ctypes.byref(dims), ctypes.byref(w), _ptr(x),
                                            int(x_dtype), int(L), _ptr(force_idx), _ptr(force_w),
                                            _ptr(y), int(y_dtype), _ptr(topk_idx_out),
                                            _ptr(topk_w_out), _stream(stream)),
           "dgmoe_block_forward_noalloc")


def dgmoe_noalloc_max_bytes():
    return _lib.dgmoe_noalloc_max_bytes()


def dgmoe_check_workspace(dims, L, ws, stream=None):
    """Flags of the last call on ws (0 if none); raises only on argument / HIP errors."""
    flags = ctypes.c_uint32(0)
    st = _lib.dgmoe_check_workspace(ctypes.byref(dims), int(L), _ptr(ws), ctypes.byref(flags),
                                    _stream(stream))
    if st not in (DGMOE_OK, DGMOE_ERR_DEVICE):
        raise DgmoeError(st, "dgmoe_check_workspace")
    return flags.value


def dgmoe_debug_force_stamp_timeout(spin_limit):
    _lib.dgmoe_debug_force_stamp_timeout(int(spin_limit))


def dgmoe_debug_set_tall_min(rows):
    """Pairs from which an expert takes 64-row tiles in a 32-row-tile launch
    (0: none, the default; negative: the default).  Returns the previous value."""
    return int(_lib.dgmoe_debug_set_tall_min(int(rows)))


def dgmoe_block_forward_profiled(dims, w, x, x_dtype, L, y, y_dtype, ws, ws_bytes, stream,
                                 events):
    """events: a HipEvents holding PROFILE_EVENTS raw hipEvent_t handles."""
    _check(_lib.dgmoe_block_forward_profiled(ctypes.byref(dims), ctypes.byref(w), _ptr(x),
                                             int(x_dtype), int(L), _ptr(y), int(y_dtype), _ptr(ws),
                                             int(ws_bytes), _stream(stream), events.array,
                                             len(events)), "dgmoe_block_forward_profiled")


class HipEvents:
    """Raw hipEvent_t handles from the process's HIP runtime (the one torch loaded)."""

    def __init__(self, n):
        self._hip = ctypes.CDLL("libamdhip64.so.7")
        self._hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self._hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                  ctypes.c_void_p]
        self._hip.hipEventSynchronize.argtypes = [ctypes.c_void_p]
        self._hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.array = (ctypes.c_void_p * n)()
        for i in range(n):
            h = ctypes.c_void_p()
            if self._hip.hipEventCreate(ctypes.byref(h)) != 0:
                raise RuntimeError("hipEventCreate failed")
            self.array[i] = h
        self.n = n

    def __len__(self):
        return self.n

    def elapsed_ms(self, i, j):
        self._hip.hipEventSynchronize(self.array[j])
        ms = ctypes.c_float()
        if self._hip.hipEventElapsedTime(ctypes.byref(ms), self.array[i], self.array[j]) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return ms.value

    def close(self):
        for i in range(self.n):
            if self.array[i]:
                self._hip.hipEventDestroy(self.array[i])
                self.array[i] = None


def dgmoe_pack(w, rows, cols, fmt, codes, scale_bias, stream=None):
    _check(_lib.dgmoe_pack(_ptr(w), int(rows), int(cols), int(fmt), _ptr(codes),
                           _ptr(scale_bias), _stream(stream)), "dgmoe_pack")


def dgmoe_unpack(codes, scale_bias, rows, cols, fmt, out_dtype, out, stream=None):
    _check(_lib.dgmoe_unpack(_ptr(codes), _ptr(scale_bias), int(rows), int(cols), int(fmt),
                             int(out_dtype), _ptr(out), _stream(stream)), "dgmoe_unpack")


# ------------------------------------------------------------------ device weights
class DeviceMatrix:
    """One matrix (or E stacked matrices) in device memory in a library format."""

    def __init__(self, fmt, data, scale_bias=None, rows=0, cols=0):
        self.fmt, self.data, self.scale_bias = fmt, data, scale_bias
        self.rows, self.cols = rows, cols

    def struct(self):
        return dgmoe_matrix(FMT[self.fmt], _ptr(self.data), _ptr(self.scale_bias))

    def nbytes(self):
        n = self.data.numel() * self.data.element_size()
        if self.scale_bias is not None:
            n += self.scale_bias.numel() * self.scale_bias.element_size()
        return n


def _empty_aligned(nbytes, device):
    """uint8 device tensor whose data pointer is 256-byte aligned."""
    import torch
    t = torch.empty(int(nbytes) + 256, dtype=torch.uint8, device=device)
    off = (-t.data_ptr()) % 256
    return t[off:off + int(nbytes)]


def device_matrix(w32, fmt, device="cuda", stream=None):
    """Upload a float32 [rows, cols] (or [E, rows, cols]) array and store it in fmt.
    q4 / q4g32 / q8 are packed on the GPU by dgmoe_pack (each expert's matrix on
    its own, which for these layouts is the same as packing the stacked rows);
    bf16 / f32 are converted by torch."""
    import torch
    w32 = np.ascontiguousarray(w32, dtype=np.float32)
    cols = w32.shape[-1]
    rows = int(np.prod(w32.shape[:-1]))
    src = torch.from_numpy(w32).to(device)
    if fmt in PER_EXPERT:
        # each expert of a stacked tensor on its own
        n = w32.shape[0] if w32.ndim == 3 else 1
        r = rows // n
        cb, sbb = dgmoe_packed_bytes(r, cols, FMT[fmt]), scale_bytes(r, cols, fmt)
        codes = _empty_aligned(n * cb, device)
        sb = _empty_aligned(n * sbb, device)
        flat = src.reshape(n, r, cols)
        for e in range(n):
            dgmoe_pack(flat[e], r, cols, FMT[fmt], codes[e * cb:(e + 1) * cb],
                       sb[e * sbb:(e + 1) * sbb], stream)
        del src, flat
        return DeviceMatrix(fmt, codes, sb, rows, cols)
    if fmt in PACKED:
        code_bytes = dgmoe_packed_bytes(rows, cols, FMT[fmt])
        codes = _empty_aligned(code_bytes, device)
        sb = _empty_aligned(scale_bytes(rows, cols, fmt), device).view(torch.int16)
        dgmoe_pack(src, rows, cols, FMT[fmt], codes, sb, stream)
        del src
        return DeviceMatrix(fmt, codes, sb, rows, cols)
    if fmt == "bf16":
        data = _empty_aligned(2 * rows * cols, device).view(torch.bfloat16)
        data.copy_(src.reshape(-1).to(torch.bfloat16))
        return DeviceMatrix(fmt, data, None, rows, cols)
    if fmt == "f32":
        data = _empty_aligned(4 * rows * cols, device).view(torch.float32)
        data.copy_(src.reshape(-1))
        return DeviceMatrix(fmt, data, None, rows, cols)
    raise ValueError(fmt)


def device_sparse_experts(experts, E, rows, cols, fmt, device="cuda", stream=None):
    """[E, rows, cols] in a packed format with only the experts in `experts` (index ->
    float32 [rows, cols]) stored; every other expert is zero codes with zero
    scales and biases, which dequantise to 0.  (Expert e's codes and
    (scale, bias) pairs are the e-th equal slice of the stacked arrays.)"""
    import torch
    if fmt not in PACKED:
        raise ValueError(fmt)
    cb = dgmoe_packed_bytes(rows, cols, FMT[fmt])
    sbb = scale_bytes(rows, cols, fmt)
    codes = _empty_aligned(E * cb, device)
    codes.zero_()
    sb = _empty_aligned(E * sbb, device)
    sb.zero_()
    for e, w in experts.items():
        m = device_matrix(w, fmt, device, stream)
        torch.cuda.synchronize()
        codes[e * cb:(e + 1) * cb].copy_(m.data)
        sb[e * sbb:(e + 1) * sbb].copy_(m.scale_bias.view(torch.uint8))
    torch.cuda.synchronize()
    return DeviceMatrix(fmt, codes, sb, E * rows, cols)


class PackedBlock:
    """One block's weights on the device plus the C struct that points at them.
    With hot_experts (index -> (gate_up, down) float32), only those experts are
    stored and w32 needs no expert tensors."""

    MATS = ("router", "expert_gate_up", "expert_down", "dense_gate_up", "dense_down")
    VECS = ("router_scale", "per_expert_scale", "pre_ff_norm", "pre_ff_norm_2",
            "post_ff_norm_1", "post_ff_norm_2", "post_ff_norm")

    def __init__(self, w32, cfg, device="cuda", stream=None, hot_experts=None):
        import torch
        self.cfg = cfg
        fmt, rfmt = cfg["weight_fmt"], cfg["router_fmt"]
        dfmt = cfg.get("dense_fmt") or fmt  # the dense MLP's own format, else the experts'
        if hot_experts is None:
            gu = device_matrix(w32["expert_gate_up"], fmt, device, stream)
            dn = device_matrix(w32["expert_down"], fmt, device, stream)
        else:
            E, D, I = cfg["E"], cfg["D"], cfg["I"]
            gu = device_sparse_experts({e: v[0] for e, v in hot_experts.items()}, E, 2 * I, D, fmt,
                                       device, stream)
            dn = device_sparse_experts({e: v[1] for e, v in hot_experts.items()}, E, D, I, fmt,
                                       device, stream)
        self.mats = {
            "router": device_matrix(w32["router"], rfmt, device, stream),
            "expert_gate_up": gu,
            "expert_down": dn,
            "dense_gate_up": device_matrix(w32["dense_gate_up"], dfmt, device, stream),
            "dense_down": device_matrix(w32["dense_down"], dfmt, device, stream),
        }
        self.vecs = {n: torch.from_numpy(np.asarray(w32[n], np.float32)).to(device)
                     for n in self.VECS}
        rb = w32.get("router_bias")
        self.router_bias = None if rb is None else torch.from_numpy(np.asarray(rb, np.float32)).to(device)
        self.layer_scalar = float(w32["layer_scalar"])
        self.dims = make_dims(cfg["D"], cfg["E"], cfg["k"], cfg["I"], cfg["Id"], cfg.get("eps", 1e-6))
        self.struct = self._make_struct()

    def _make_struct(self):
        m, v = self.mats, self.vecs
        return dgmoe_block_weights(
            m["router"].struct(), _ptr(v["router_scale"]), _ptr(v["per_expert_scale"]),
            _ptr(self.router_bias), m["expert_gate_up"].struct(), m["expert_down"].struct(),
            m["dense_gate_up"].struct(), m["dense_down"].struct(), _ptr(v["pre_ff_norm"]),
            _ptr(v["pre_ff_norm_2"]), _ptr(v["post_ff_norm_1"]), _ptr(v["post_ff_norm_2"]),
            _ptr(v["post_ff_norm"]), self.layer_scalar)

    def nbytes(self):
        return sum(m.nbytes() for m in self.mats.values())

    def clone(self):
        """A second copy of the packed weights in fresh (256-byte aligned) device memory."""
        import copy

        def dup(t):
            if t is None:
                return None
            n = t.numel() * t.element_size()
            d = _empty_aligned(n, t.device).view(t.dtype)
            d.copy_(t.reshape(-1))
            return d

        other = copy.copy(self)
        other.mats = {n: DeviceMatrix(m.fmt, dup(m.data), dup(m.scale_bias), m.rows, m.cols)
                      for n, m in self.mats.items()}
        other.vecs = {n: v.clone() for n, v in self.vecs.items()}
        other.router_bias = None if self.router_bias is None else self.router_bias.clone()
        other.struct = other._make_struct()
        return other


def workspace(dims, L, device="cuda"):
    """A device workspace of dgmoe_workspace_size bytes, 256-byte aligned."""
    n = dgmoe_workspace_size(dims, L)
    return _empty_aligned(max(n, 256), device), n


# ------------------------------------------------------------------ head
def make_head_dims(D, V, Isc, eps=1e-6):
    return dgmoe_head_dims(D, V, Isc, eps)


def dgmoe_head_workspace_size(hdims, L):
    return _lib.dgmoe_head_workspace_size(ctypes.byref(hdims), int(L))


def dgmoe_tail(hdims, w, x, x_dtype, L, temperature, entropy, argmax, row_max, row_sum, logits,
               ws, ws_bytes, stream=None):
    _check(_lib.dgmoe_tail(ctypes.byref(hdims), ctypes.byref(w), _ptr(x), int(x_dtype), int(L),
                           float(temperature), _ptr(entropy), _ptr(argmax), _ptr(row_max),
                           _ptr(row_sum), _ptr(logits), _ptr(ws), int(ws_bytes), _stream(stream)),
           "dgmoe_tail")


def dgmoe_soft_embed(hdims, w, sc_logits, L, soft, ws, ws_bytes, stream=None):
    _check(_lib.dgmoe_soft_embed(ctypes.byref(hdims), ctypes.byref(w), _ptr(sc_logits), int(L),
                                 _ptr(soft), _ptr(ws), int(ws_bytes), _stream(stream)),
           "dgmoe_soft_embed")


def dgmoe_sc_input(hdims, w, canvas_ids, sc_logits, L, out, ws, ws_bytes, stream=None):
    _check(_lib.dgmoe_sc_input(ctypes.byref(hdims), ctypes.byref(w), _ptr(canvas_ids),
                               _ptr(sc_logits), int(L), _ptr(out), _ptr(ws), int(ws_bytes),
                               _stream(stream)), "dgmoe_sc_input")


def dgmoe_head_check_workspace(hdims, L, ws, stream=None):
    """Flags of the last head call on ws (host, synchronous); 0 if clean."""
    flags = ctypes.c_uint32(0)
    st = _lib.dgmoe_head_check_workspace(ctypes.byref(hdims), int(L), _ptr(ws), ctypes.byref(flags),
                                         _stream(stream))
    if st not in (DGMOE_OK, DGMOE_ERR_DEVICE):
        _check(st, "dgmoe_head_check_workspace")
    return int(flags.value)


def head_workspace(hdims, L, device="cuda"):
    """A device workspace of dgmoe_head_workspace_size bytes, 256-byte aligned."""
    n = dgmoe_head_workspace_size(hdims, L)
    return _empty_aligned(max(n, 256), device), n


class PackedHead:
    """The head's weights on the device (the table and the self-conditioning
    MLP packed Q4G64 by dgmoe_pack) plus the C struct that points at them.
    w32: dict with embed [V, D], final_norm [D], sc_gate_up [2 I_sc, D],
    sc_down [D, I_sc], sc_pre_norm [D] (float32)."""

    def __init__(self, w32, cfg, device="cuda", stream=None):
        import torch
        self.cfg = cfg
        self.mats = {n: device_matrix(w32[n], "q4", device, stream)
                     for n in ("embed", "sc_gate_up", "sc_down")}
        self.vecs = {n: torch.from_numpy(np.asarray(w32[n], np.float32)).to(device)
                     for n in ("final_norm", "sc_pre_norm")}
        self.dims = make_head_dims(cfg["D"], cfg["V"], cfg["Isc"], cfg.get("eps", 1e-6))
        m, v = self.mats, self.vecs
        self.struct = dgmoe_head_weights(m["embed"].struct(), _ptr(v["final_norm"]),
                                         m["sc_gate_up"].struct(), m["sc_down"].struct(),
                                         _ptr(v["sc_pre_norm"]))


# ------------------------------------------------------------------ denoise attention
def make_attn_dims(H, Hkv, hd, window, rope_pairs, rope_stride, theta, den, eps=1e-6):
    return dgmoe_attn_dims(H, Hkv, hd, window, rope_pairs, rope_stride, theta, den, eps)


def attn_dims_for(cfg, rope_reading="arch"):
    """The dims of a sliding or full layer of the given shape: sliding layers
    rotate every pair (theta 1e4); full layers a quarter of head_dim with
    theta 1e6, partner stride rope_pairs ("arch") or head_dim/2 ("blog")."""
    hd = cfg["hd"]
    if cfg["kind"] == "sliding":
        return make_attn_dims(cfg["H"], cfg["Hkv"], hd, cfg["window"], hd // 2, hd // 2, 1e4, hd)
    pairs = hd // 8
    stride = pairs if rope_reading == "arch" else hd // 2
    return make_attn_dims(cfg["H"], cfg["Hkv"], hd, cfg["window"], pairs, stride, 1e6, hd)


def dgmoe_attn_workspace_size(adims, L, kv_len):
    return _lib.dgmoe_attn_workspace_size(ctypes.byref(adims), int(L), int(kv_len))


def dgmoe_attn_denoise(adims, q, k, v, in_dtype, L, q_norm, k_norm, k_cache, v_cache, cache_rows,
                       kv_len, out, out_dtype, ws, ws_bytes, stream=None):
    _check(_lib.dgmoe_attn_denoise(ctypes.byref(adims), _ptr(q), _ptr(k), _ptr(v), int(in_dtype),
                                   int(L), _ptr(q_norm), _ptr(k_norm), _ptr(k_cache),
                                   _ptr(v_cache), int(cache_rows), int(kv_len), _ptr(out),
                                   int(out_dtype), _ptr(ws), int(ws_bytes), _stream(stream)),
           "dgmoe_attn_denoise")


def attn_workspace(adims, L, kv_len, device="cuda"):
    """A device workspace of dgmoe_attn_workspace_size bytes, 256-byte aligned."""
    n = dgmoe_attn_workspace_size(adims, L, kv_len)
    return _empty_aligned(max(n, 256), device), n
