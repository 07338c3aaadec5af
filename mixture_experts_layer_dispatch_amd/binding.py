"""ctypes binding of the MoE layer's C ABI (include/moe.h).

Argument marshalling only: every step of the layer runs in the HIP library
``libmoe_mi355x.so``.  PyTorch supplies device memory (``tensor.data_ptr()``)
and the stream (``torch.cuda.current_stream().cuda_stream``).  If the library
is missing, every entry point raises: there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe_mi355x.so")

MOE_OK = 0
MOE_ERR_INVALID_ARG = 1
MOE_ERR_UNSUPPORTED_DEVICE = 2
MOE_ERR_CAPACITY = 3
MOE_ERR_WORKSPACE = 4
MOE_ERR_HIP = 5
MOE_ERR_UNSUPPORTED = 6

PREC_BF16 = 0
PREC_MXFP8 = 1
PREC_MXFP4 = 2          # forward only: MXFP4 weights, MXFP8 activations

EXPORTED = [
    "moe_status_string", "moe_validate_config", "moe_ring_rows", "moe_workspace_size",
    "moe_device_supported", "moe_schedule", "moe_forward", "moe_backward",
    "moe_check_device_error", "moe_quantize_weights_mxfp8", "moe_profile_enable", "moe_profile_collect", "moe_profile_query",
    "moe_profile_names", "moe_profile_reset", "moe_workspace_region", "moe_schedule_noalloc",
    "moe_router_forward", "moe_router_backward", "moe_quantize_weights_mxfp4",
]

FLAG_RECOMPUTE = 1


class MoEError(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__(f"{where}: {status_string(status)} (status {status})")
        self.status = status


class moe_config(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int32), ("H", ctypes.c_int32), ("I", ctypes.c_int32),
                ("E", ctypes.c_int32), ("k", ctypes.c_int32), ("n_shared", ctypes.c_int32),
                ("macrobatch", ctypes.c_int32), ("minibatch", ctypes.c_int32),
                ("capacity_rows", ctypes.c_int64), ("precision", ctypes.c_int32),
                ("flags", ctypes.c_int32), ("acc_experts", ctypes.c_int32)]


class moe_sched(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in
                ("topk_idx", "topk_w", "counts", "offsets", "mini_counts", "row_of_slot",
                 "slot_of_row")]


MX_FIELDS = ("w_gate_q", "w_gate_s", "w_up_q", "w_up_s", "w_down_q", "w_down_s",
             "w_gate_tq", "w_gate_ts", "w_up_tq", "w_up_ts", "w_down_tq", "w_down_ts",
             "s_gate_q", "s_gate_s", "s_up_q", "s_up_s", "s_down_q", "s_down_s",
             "s_gate_tq", "s_gate_ts", "s_up_tq", "s_up_ts", "s_down_tq", "s_down_ts")


class moe_weights_mx(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in MX_FIELDS]


MX4_FIELDS = ("w_gate_q", "w_gate_s", "w_up_q", "w_up_s", "w_down_q", "w_down_s",
              "s_gate_q", "s_gate_s", "s_up_q", "s_up_s", "s_down_q", "s_down_s")


class moe_weights_mx4(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in MX4_FIELDS]


class moe_weights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in
                ("w_gate", "w_up", "w_down", "s_gate", "s_up", "s_down")] + [
                ("mx", ctypes.POINTER(moe_weights_mx)), ("mx4", ctypes.POINTER(moe_weights_mx4))]


class moe_saved(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in ("g", "u", "sg", "su")]


class moe_grads(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in
                ("d_w_gate", "d_w_up", "d_w_down", "d_s_gate", "d_s_up", "d_s_down")]


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: run `python -m "
                               "mixture_experts_layer_dispatch_amd.build` first")
        L = ctypes.CDLL(LIB_PATH)
        vp, cfgp = ctypes.c_void_p, ctypes.POINTER(moe_config)
        L.moe_status_string.restype = ctypes.c_char_p
        L.moe_status_string.argtypes = [ctypes.c_int]
        L.moe_validate_config.argtypes = [cfgp]
        L.moe_ring_rows.argtypes = [cfgp, ctypes.POINTER(ctypes.c_int64)]
        L.moe_workspace_size.argtypes = [cfgp, ctypes.POINTER(ctypes.c_size_t)]
        L.moe_device_supported.argtypes = []
        L.moe_schedule.argtypes = [cfgp, vp, ctypes.POINTER(moe_sched), vp, ctypes.c_size_t, vp]
        L.moe_schedule_noalloc.argtypes = [cfgp, vp, ctypes.POINTER(moe_sched), vp]
        L.moe_router_forward.argtypes = [cfgp, vp, vp, vp, vp]
        L.moe_router_backward.argtypes = [cfgp, vp, vp, vp, vp, vp, vp, ctypes.c_size_t, vp]
        L.moe_forward.argtypes = [cfgp, ctypes.POINTER(moe_sched), vp, ctypes.POINTER(moe_weights),
                                  vp, ctypes.POINTER(moe_saved), vp, ctypes.c_size_t, vp]
        L.moe_backward.argtypes = [cfgp, ctypes.POINTER(moe_sched), ctypes.POINTER(moe_saved), vp,
                                   ctypes.POINTER(moe_weights), vp, vp, ctypes.POINTER(moe_grads),
                                   vp, vp, vp, ctypes.c_size_t, vp]
        L.moe_check_device_error.argtypes = [vp, ctypes.c_size_t, vp, ctypes.POINTER(ctypes.c_int32)]
        L.moe_quantize_weights_mxfp8.argtypes = [cfgp, ctypes.POINTER(moe_weights),
                                                 ctypes.POINTER(moe_weights_mx), vp]
        L.moe_quantize_weights_mxfp4.argtypes = [cfgp, ctypes.POINTER(moe_weights),
                                                 ctypes.POINTER(moe_weights_mx4), vp]
        L.moe_profile_enable.argtypes = [ctypes.c_int]
        L.moe_profile_collect.argtypes = []
        L.moe_profile_query.argtypes = [ctypes.c_char_p, ctypes.POINTER(ctypes.c_int64),
                                        ctypes.POINTER(ctypes.c_double)]
        L.moe_profile_names.argtypes = [ctypes.c_char_p, ctypes.c_size_t]
        L.moe_profile_reset.argtypes = []
        L.moe_workspace_region.argtypes = [cfgp, ctypes.c_char_p, ctypes.POINTER(ctypes.c_size_t),
                                           ctypes.POINTER(ctypes.c_size_t)]
        for name in EXPORTED:
            if name != "moe_status_string":
                getattr(L, name).restype = ctypes.c_int
        _lib = L
    return _lib


def status_string(status: int) -> str:
    return lib().moe_status_string(int(status)).decode()


def _check(status: int, where: str):
    if status != MOE_OK:
        raise MoEError(status, where)


def _p(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


@dataclass
class Config:
    T: int
    H: int
    I: int
    E: int
    k: int
    n_shared: int = 0
    macrobatch: int = 0
    minibatch: int = 0
    capacity_rows: int = 0
    precision: int = PREC_BF16
    recompute: bool = False
    acc_experts: int = 0

    def c(self) -> moe_config:
        return moe_config(self.T, self.H, self.I, self.E, self.k, self.n_shared, self.macrobatch,
                          self.minibatch, self.capacity_rows, self.precision,
                          FLAG_RECOMPUTE if self.recompute else 0, self.acc_experts)

    @property
    def M(self) -> int:
        return self.macrobatch or self.T

    @property
    def mb(self) -> int:
        return self.minibatch or self.M

    @property
    def n_macro(self) -> int:
        return self.T // self.M

    @property
    def n_mini(self) -> int:
        return self.M // self.mb

    @property
    def S(self) -> int:
        return self.T * self.k


def validate_config(cfg: Config) -> int:
    return lib().moe_validate_config(ctypes.byref(cfg.c()))


def ring_rows(cfg: Config) -> int:
    v = ctypes.c_int64()
    _check(lib().moe_ring_rows(ctypes.byref(cfg.c()), ctypes.byref(v)), "moe_ring_rows")
    return v.value


def workspace_size(cfg: Config) -> int:
    v = ctypes.c_size_t()
    _check(lib().moe_workspace_size(ctypes.byref(cfg.c()), ctypes.byref(v)), "moe_workspace_size")
    return v.value


def device_supported() -> bool:
    return bool(lib().moe_device_supported())


# ------------------------------------------------------------------ buffers
def alloc_workspace(cfg: Config, device="cuda") -> torch.Tensor:
    return torch.empty(workspace_size(cfg), dtype=torch.uint8, device=device)


def alloc_schedule(cfg: Config, device="cuda") -> dict:
    i32 = dict(dtype=torch.int32, device=device)
    return {
        "topk_idx": torch.empty(cfg.T, cfg.k, **i32),
        "topk_w": torch.empty(cfg.T, cfg.k, dtype=torch.float32, device=device),
        "counts": torch.empty(cfg.n_macro, cfg.E, **i32),
        "offsets": torch.empty(cfg.n_macro, cfg.E + 1, **i32),
        "mini_counts": torch.empty(cfg.n_macro, cfg.E, cfg.n_mini, **i32),
        "row_of_slot": torch.empty(cfg.S, **i32),
        "slot_of_row": torch.empty(cfg.S, **i32),
    }


def workspace_region(cfg: Config, name: str) -> tuple:
    """(byte offset, bytes) of a named array inside the workspace (MXFP8:
    "x_codes", "x_scales", "dy_codes", "dy_scales")."""
    off, n = ctypes.c_size_t(), ctypes.c_size_t()
    _check(lib().moe_workspace_region(ctypes.byref(cfg.c()), name.encode(), ctypes.byref(off),
                                      ctypes.byref(n)), "moe_workspace_region")
    return off.value, n.value


def alloc_saved(cfg: Config, device="cuda") -> dict:
    """g, u (and the shared expert's): bf16 in BF16 mode, fp32 in the MX modes;
    nothing in recompute mode."""
    if cfg.recompute:
        return {}
    dt = torch.float32 if cfg.precision in (PREC_MXFP8, PREC_MXFP4) else torch.bfloat16
    bf = dict(dtype=dt, device=device)
    out = {"g": torch.empty(cfg.S, cfg.I, **bf), "u": torch.empty(cfg.S, cfg.I, **bf)}
    if cfg.n_shared:
        out["sg"] = torch.empty(cfg.T, cfg.I, **bf)
        out["su"] = torch.empty(cfg.T, cfg.I, **bf)
    return out


def alloc_grads(cfg: Config, device="cuda") -> dict:
    bf = dict(dtype=torch.bfloat16, device=device)
    out = {"d_w_gate": torch.empty(cfg.E, cfg.I, cfg.H, **bf),
           "d_w_up": torch.empty(cfg.E, cfg.I, cfg.H, **bf),
           "d_w_down": torch.empty(cfg.E, cfg.H, cfg.I, **bf)}
    if cfg.n_shared:
        out["d_s_gate"] = torch.empty(cfg.I, cfg.H, **bf)
        out["d_s_up"] = torch.empty(cfg.I, cfg.H, **bf)
        out["d_s_down"] = torch.empty(cfg.H, cfg.I, **bf)
    return out


def _sched(s: dict) -> moe_sched:
    return moe_sched(*[s[n].data_ptr() for n, _ in moe_sched._fields_])


def _weights_mx(q: dict) -> moe_weights_mx:
    return moe_weights_mx(*[(q[n].data_ptr() if q.get(n) is not None else None) for n in MX_FIELDS])


def _weights_mx4(q: dict) -> moe_weights_mx4:
    return moe_weights_mx4(*[(q[n].data_ptr() if q.get(n) is not None else None) for n in MX4_FIELDS])


def _weights(w: dict):
    """(moe_weights, keep-alive); w may hold an "mx" dict (MXFP8) and an "mx4"
    dict (MXFP4) of quantised arrays."""
    mx = _weights_mx(w["mx"]) if w.get("mx") is not None else None
    mx4 = _weights_mx4(w["mx4"]) if w.get("mx4") is not None else None
    st = moe_weights(*[(w[n].data_ptr() if w.get(n) is not None else None)
                       for n in ("w_gate", "w_up", "w_down", "s_gate", "s_up", "s_down")])
    if mx is not None:
        st.mx = ctypes.pointer(mx)
    if mx4 is not None:
        st.mx4 = ctypes.pointer(mx4)
    return st, (mx, mx4)


def _saved(s) -> moe_saved:
    s = s or {}
    return moe_saved(*[(s[n].data_ptr() if s.get(n) is not None else None)
                       for n, _ in moe_saved._fields_])


def _grads(g: dict) -> moe_grads:
    return moe_grads(*[(g[n].data_ptr() if g.get(n) is not None else None)
                       for n, _ in moe_grads._fields_])


# ------------------------------------------------------------------ argument checks
# The C side can only check pointers for null and alignment; a buffer of the
# wrong size would be written out of bounds on the device.  Every tensor is
# therefore checked against the Config here, before anything reaches the
# library: shape, dtype and contiguity of all of them first, then that each
# lives on a GPU.  The _spec_* helpers list (name, tensor, shape, dtype).
def _validate(specs):
    for name, t, shape, dtype in specs:
        if t is None:
            raise ValueError(f"{name}: missing")
        if not isinstance(t, torch.Tensor):
            raise ValueError(f"{name}: expected a torch.Tensor, got {type(t).__name__}")
        if tuple(t.shape) != tuple(shape):
            raise ValueError(f"{name}: shape {tuple(t.shape)}, expected {tuple(shape)}")
        if t.dtype != dtype:
            raise ValueError(f"{name}: dtype {t.dtype}, expected {dtype}")
        if not t.is_contiguous():
            raise ValueError(f"{name}: must be contiguous")
    for name, t, _, _ in specs:
        if t.device.type != "cuda":
            raise ValueError(f"{name}: must be on the GPU, found on {t.device}")


def _spec_ws(cfg: Config, ws):
    n = ws.numel() if isinstance(ws, torch.Tensor) else -1
    need = workspace_size(cfg)
    if isinstance(ws, torch.Tensor) and ws.dtype == torch.uint8 and n < need:
        raise ValueError(f"workspace: {n} bytes, the config needs {need}")
    return [("workspace", ws, (n,), torch.uint8)]


def _spec_sched(cfg: Config, s: dict):
    i32, f32_ = torch.int32, torch.float32
    want = {"topk_idx": ((cfg.T, cfg.k), i32), "topk_w": ((cfg.T, cfg.k), f32_),
            "counts": ((cfg.n_macro, cfg.E), i32), "offsets": ((cfg.n_macro, cfg.E + 1), i32),
            "mini_counts": ((cfg.n_macro, cfg.E, cfg.n_mini), i32),
            "row_of_slot": ((cfg.S,), i32), "slot_of_row": ((cfg.S,), i32)}
    return [(f"sched[{n!r}]", s.get(n), shape, dt) for n, (shape, dt) in want.items()]


def _spec_weights(cfg: Config, w: dict):
    E, H, I, bf = cfg.E, cfg.H, cfg.I, torch.bfloat16
    out = [("w_gate", w.get("w_gate"), (E, I, H), bf), ("w_up", w.get("w_up"), (E, I, H), bf),
           ("w_down", w.get("w_down"), (E, H, I), bf)]
    if cfg.n_shared:
        out += [("s_gate", w.get("s_gate"), (I, H), bf), ("s_up", w.get("s_up"), (I, H), bf),
                ("s_down", w.get("s_down"), (H, I), bf)]
    return out


def _mx_shapes(cfg: Config):
    """{field: shape} of every quantised weight array (uint8)."""
    E, H, I = cfg.E, cfg.H, cfg.I
    mats = (("gate_", I, H), ("up_", I, H), ("down_", H, I),
            ("gate_t", H, I), ("up_t", H, I), ("down_t", I, H))
    out = {}
    for prefix, lead in (("w_", (E,)), ("s_", ())):
        if prefix == "s_" and not cfg.n_shared:
            continue
        for name, rows, K in mats:
            out[prefix + name + "q"] = (*lead, rows, K)
            out[prefix + name + "s"] = (*lead, K // 128, rows, 4)
    return out


def _spec_weights_mx(cfg: Config, q, forward: bool = True, transposed: bool = True):
    """The quantised arrays a call reads: the forward orientation, the
    transposed one (backward), or both (the quantiser writes both)."""
    if q is None:
        raise ValueError("weights['mx']: the MXFP8 path needs the quantised weights")
    out = []
    for n, shape in _mx_shapes(cfg).items():
        is_t = n.endswith(("_tq", "_ts"))
        if (is_t and transposed) or (not is_t and forward):
            out.append((f"mx[{n!r}]", q.get(n), shape, torch.uint8))
    return out


def _mx4_shapes(cfg: Config):
    """{field: shape} of every MXFP4 weight array (uint8): codes two per byte."""
    E, H, I = cfg.E, cfg.H, cfg.I
    out = {}
    for prefix, lead in (("w_", (E,)), ("s_", ())):
        if prefix == "s_" and not cfg.n_shared:
            continue
        for name, rows, K in (("gate_", I, H), ("up_", I, H), ("down_", H, I)):
            out[prefix + name + "q"] = (*lead, rows, K // 2)
            out[prefix + name + "s"] = (*lead, K // 128, rows, 4)
    return out


def _spec_weights_mx4(cfg: Config, q):
    if q is None:
        raise ValueError("weights['mx4']: the MXFP4 path needs the quantised weights")
    return [(f"mx4[{n!r}]", q.get(n), shape, torch.uint8) for n, shape in _mx4_shapes(cfg).items()]


def alloc_weights_mx4(cfg: Config, device="cuda") -> dict:
    """Buffers of every MXFP4 weight array (uint8): E2M1 codes two per byte
    [.., rows, K/2], scales K-step-major [.., K/128, rows, 4]."""
    return {n: torch.empty(*shape, dtype=torch.uint8, device=device) for n, shape in _mx4_shapes(cfg).items()}


def moe_quantize_weights_mxfp4(cfg: Config, weights: dict, out: dict, stream=None):
    _validate(_spec_weights(cfg, weights) + _spec_weights_mx4(cfg, out))
    wst, _keep = _weights(weights)
    mx4 = _weights_mx4(out)
    _check(lib().moe_quantize_weights_mxfp4(ctypes.byref(cfg.c()), ctypes.byref(wst),
                                            ctypes.byref(mx4), _stream(stream)),
           "moe_quantize_weights_mxfp4")


def _spec_saved(cfg: Config, s: dict):
    if cfg.recompute:
        return []                  # nothing is saved: the backward recomputes g, u
    if s is None:
        raise ValueError("saved: missing (only recompute mode saves nothing)")
    dt = torch.float32 if cfg.precision in (PREC_MXFP8, PREC_MXFP4) else torch.bfloat16
    out = [("saved['g']", s.get("g"), (cfg.S, cfg.I), dt),
           ("saved['u']", s.get("u"), (cfg.S, cfg.I), dt)]
    if cfg.n_shared:
        out += [("saved['sg']", s.get("sg"), (cfg.T, cfg.I), dt),
                ("saved['su']", s.get("su"), (cfg.T, cfg.I), dt)]
    return out


def _spec_grads(cfg: Config, g: dict):
    E, H, I, bf = cfg.E, cfg.H, cfg.I, torch.bfloat16
    out = [("grads['d_w_gate']", g.get("d_w_gate"), (E, I, H), bf),
           ("grads['d_w_up']", g.get("d_w_up"), (E, I, H), bf),
           ("grads['d_w_down']", g.get("d_w_down"), (E, H, I), bf)]
    if cfg.n_shared:
        out += [("grads['d_s_gate']", g.get("d_s_gate"), (I, H), bf),
                ("grads['d_s_up']", g.get("d_s_up"), (I, H), bf),
                ("grads['d_s_down']", g.get("d_s_down"), (H, I), bf)]
    return out


# ------------------------------------------------------------------ entry points
def moe_schedule(cfg: Config, logits: torch.Tensor, sched: dict, ws: torch.Tensor, stream=None):
    _validate([("logits", logits, (cfg.T, cfg.E), torch.float32)] + _spec_sched(cfg, sched)
              + _spec_ws(cfg, ws))
    _check(lib().moe_schedule(ctypes.byref(cfg.c()), _p(logits), ctypes.byref(_sched(sched)),
                              _p(ws), ws.numel(), _stream(stream)), "moe_schedule")


def moe_schedule_noalloc(cfg: Config, logits: torch.Tensor, sched: dict, stream=None):
    """moe_schedule without a workspace: the library's fixed scratch array is
    used instead (overlapping calls on one GPU race)."""
    _validate([("logits", logits, (cfg.T, cfg.E), torch.float32)] + _spec_sched(cfg, sched))
    _check(lib().moe_schedule_noalloc(ctypes.byref(cfg.c()), _p(logits), ctypes.byref(_sched(sched)),
                                      _stream(stream)), "moe_schedule_noalloc")


def moe_router_forward(cfg: Config, x: torch.Tensor, w_router: torch.Tensor, logits: torch.Tensor,
                       stream=None):
    """logits [T, E] fp32 = x [T, H] @ w_router [E, H]^T."""
    _validate([("x", x, (cfg.T, cfg.H), torch.bfloat16),
               ("w_router", w_router, (cfg.E, cfg.H), torch.bfloat16),
               ("logits", logits, (cfg.T, cfg.E), torch.float32)])
    _check(lib().moe_router_forward(ctypes.byref(cfg.c()), _p(x), _p(w_router), _p(logits),
                                    _stream(stream)), "moe_router_forward")


def moe_router_backward(cfg: Config, x: torch.Tensor, w_router: torch.Tensor, d_logits: torch.Tensor,
                        dx: torch.Tensor, dw_router: torch.Tensor, ws: torch.Tensor, stream=None):
    """dx += d_logits @ w_router (in place); dw_router = d_logits^T @ x."""
    bf = torch.bfloat16
    _validate([("x", x, (cfg.T, cfg.H), bf), ("w_router", w_router, (cfg.E, cfg.H), bf),
               ("d_logits", d_logits, (cfg.T, cfg.E), torch.float32), ("dx", dx, (cfg.T, cfg.H), bf),
               ("dw_router", dw_router, (cfg.E, cfg.H), bf)] + _spec_ws(cfg, ws))
    _check(lib().moe_router_backward(ctypes.byref(cfg.c()), _p(x), _p(w_router), _p(d_logits), _p(dx),
                                     _p(dw_router), _p(ws), ws.numel(), _stream(stream)),
           "moe_router_backward")


def moe_forward(cfg: Config, sched: dict, x: torch.Tensor, weights: dict, y: torch.Tensor,
                saved: dict, ws: torch.Tensor, stream=None):
    bf = torch.bfloat16
    specs = _spec_sched(cfg, sched) + [("x", x, (cfg.T, cfg.H), bf), ("y", y, (cfg.T, cfg.H), bf)]
    specs += _spec_weights(cfg, weights)
    if cfg.precision == PREC_MXFP8:
        specs += _spec_weights_mx(cfg, weights.get("mx"), forward=True, transposed=False)
    if cfg.precision == PREC_MXFP4:
        specs += _spec_weights_mx4(cfg, weights.get("mx4"))
    _validate(specs + _spec_saved(cfg, saved) + _spec_ws(cfg, ws))
    wst, _keep = _weights(weights)
    _check(lib().moe_forward(ctypes.byref(cfg.c()), ctypes.byref(_sched(sched)), _p(x),
                             ctypes.byref(wst), _p(y), ctypes.byref(_saved(saved)),
                             _p(ws), ws.numel(), _stream(stream)), "moe_forward")


def moe_backward(cfg: Config, sched: dict, saved: dict, x: torch.Tensor, weights: dict,
                 dy: torch.Tensor, dx: torch.Tensor, grads: dict, dw: torch.Tensor,
                 d_logits, ws: torch.Tensor, stream=None):
    bf = torch.bfloat16
    specs = _spec_sched(cfg, sched) + _spec_saved(cfg, saved)
    specs += [("x", x, (cfg.T, cfg.H), bf), ("dy", dy, (cfg.T, cfg.H), bf),
              ("dx", dx, (cfg.T, cfg.H), bf)]
    specs += _spec_weights(cfg, weights)
    if cfg.precision == PREC_MXFP8:
        specs += _spec_weights_mx(cfg, weights.get("mx"), forward=False, transposed=True)
    specs += _spec_grads(cfg, grads) + [("dw", dw, (cfg.T, cfg.k), torch.float32)]
    if d_logits is not None:
        specs.append(("d_logits", d_logits, (cfg.T, cfg.E), torch.float32))
    _validate(specs + _spec_ws(cfg, ws))
    wst, _keep = _weights(weights)
    _check(lib().moe_backward(ctypes.byref(cfg.c()), ctypes.byref(_sched(sched)),
                              ctypes.byref(_saved(saved)), _p(x), ctypes.byref(wst),
                              _p(dy), _p(dx), ctypes.byref(_grads(grads)), _p(dw), _p(d_logits),
                              _p(ws), ws.numel(), _stream(stream)), "moe_backward")


def alloc_weights_mx(cfg: Config, device="cuda") -> dict:
    """Buffers of every quantised weight array (uint8): codes [.., rows, K],
    scales K-step-major [.., K/128, rows, 4]."""
    u8 = dict(dtype=torch.uint8, device=device)
    return {n: torch.empty(*shape, **u8) for n, shape in _mx_shapes(cfg).items()}


def moe_quantize_weights_mxfp8(cfg: Config, weights: dict, out: dict, stream=None):
    _validate(_spec_weights(cfg, weights) + _spec_weights_mx(cfg, out))
    wst, _keep = _weights(weights)
    mx = _weights_mx(out)
    _check(lib().moe_quantize_weights_mxfp8(ctypes.byref(cfg.c()), ctypes.byref(wst),
                                            ctypes.byref(mx), _stream(stream)),
           "moe_quantize_weights_mxfp8")


# device error bits (moe_check_device_error)
DEVERR_BAD_EXPERT, DEVERR_BAD_SLOT, DEVERR_BAD_ROW, DEVERR_BAD_OFFSETS, DEVERR_ACC_CAPACITY = 1, 2, 4, 8, 16


def moe_check_device_error(ws: torch.Tensor, stream=None) -> int:
    _validate([("workspace", ws, (ws.numel() if isinstance(ws, torch.Tensor) else -1,), torch.uint8)])
    v = ctypes.c_int32()
    _check(lib().moe_check_device_error(_p(ws), ws.numel(), _stream(stream), ctypes.byref(v)),
           "moe_check_device_error")
    return v.value


# ------------------------------------------------------------------ kernel timing
def profile_enable(on: bool = True):
    _check(lib().moe_profile_enable(int(on)), "moe_profile_enable")


def profile_collect():
    _check(lib().moe_profile_collect(), "moe_profile_collect")


def profile_reset():
    _check(lib().moe_profile_reset(), "moe_profile_reset")


def profile_stats() -> dict:
    """{kernel name: (launches, total milliseconds)} of the collected events."""
    buf = ctypes.create_string_buffer(1 << 14)
    _check(lib().moe_profile_names(buf, len(buf)), "moe_profile_names")
    out = {}
    for name in buf.value.decode().split():
        n, ms = ctypes.c_int64(), ctypes.c_double()
        _check(lib().moe_profile_query(name.encode(), ctypes.byref(n), ctypes.byref(ms)),
               "moe_profile_query")
        out[name] = (n.value, ms.value)
    return out
