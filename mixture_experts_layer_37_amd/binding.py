"""ctypes binding of libmoe (include/moe.h): argument marshalling only.

Every function here checks shapes, dtypes, devices and contiguity on the host,
turns tensors into device pointers and calls the C entry point of the same
name on torch's current HIP stream.  All computation happens in the library's
HIP kernels; there is no fallback: if libmoe.so is missing, loading fails.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

from . import debug as _debug

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmoe.so")

MOE_OK, MOE_ERR_INVALID_ARG, MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE, MOE_ERR_HIP = range(5)
MOE_F32, MOE_BF16 = 0, 1
MOE_SCORE_SOFTMAX, MOE_SCORE_SIGMOID = 0, 1
MOE_GATE_RAW, MOE_GATE_RENORM = 0, 1
MOE_FILL_RANK_MAJOR, MOE_FILL_TOKEN_MAJOR = 0, 1
MOE_CAP_ASSIGNMENTS, MOE_CAP_TOKENS = 0, 1
(MOE_WS_ROUTE, MOE_WS_DISPATCH, MOE_WS_EXPERT_FFN, MOE_WS_LAYER, MOE_WS_SHARED_FFN,
 MOE_WS_BACKWARD, MOE_WS_EXPERT_FFN_BACKWARD, MOE_WS_ROUTER_BACKWARD) = range(8)
MOE_NUM_STAGES = 6
STAGE_NAMES = ["route", "dispatch", "gate_up", "down", "combine", "stats"]


class MoeError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_string(status)}")


class moe_config(ctypes.Structure):
    _fields_ = [
        ("T", ctypes.c_int64), ("h", ctypes.c_int64), ("f", ctypes.c_int64),
        ("E", ctypes.c_int64), ("k", ctypes.c_int64),
        ("dtype", ctypes.c_int32), ("score", ctypes.c_int32), ("gate", ctypes.c_int32),
        ("cap_mode", ctypes.c_int32), ("fill", ctypes.c_int32), ("noisy", ctypes.c_int32),
        ("capacity_factor", ctypes.c_double), ("min_capacity", ctypes.c_int64),
        ("n_groups", ctypes.c_int64), ("topk_groups", ctypes.c_int64),
        ("n_shared", ctypes.c_int64), ("f_shared", ctypes.c_int64),
        ("seed", ctypes.c_uint64), ("rng_offset", ctypes.c_uint64),
    ]


class moe_aux_outputs(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in (
        "topk_idx", "topk_gate", "logits", "slot", "row_token", "count", "kept", "offset",
        "prob_sum", "f", "P", "aux_loss", "maxvio", "n_dropped", "X", "Y", "Y_shared",
        "z_loss", "GU", "A", "noise")]


AUX_FIELDS = [n for n, _ in moe_aux_outputs._fields_]


class moe_backward_extras(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in (
        "W_noise", "dW_noise", "Ws_gate", "Ws_up", "Ws_down", "dWs_gate", "dWs_up",
        "dWs_down", "W_downT8", "s_downT")]

_lib = None


def lib() -> ctypes.CDLL:
    """Load libmoe.so; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m mixture_experts_layer_37_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        P, I32, I64, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
        cfgp = ctypes.POINTER(moe_config)
        sig = {
            "moe_status_string": (ctypes.c_char_p, [I32]),
            "moe_capacity": (I32, [cfgp, ctypes.POINTER(I64)]),
            "moe_max_rows": (I32, [cfgp, ctypes.POINTER(I64)]),
            "moe_workspace_size": (I32, [cfgp, I32, ctypes.POINTER(SZ)]),
            "moe_route": (I32, [cfgp] + [P] * 10 + [P, SZ, P]),
            "moe_dispatch": (I32, [cfgp] + [P] * 8 + [P, SZ, P]),
            "moe_dispatch_noalloc": (I32, [cfgp] + [P] * 8 + [P]),
            "moe_stream_read": (I32, [P, SZ, P, I32, P]),
            "moe_expert_ffn": (I32, [cfgp] + [P] * 6 + [P, SZ, P]),
            "moe_combine": (I32, [cfgp] + [P] * 6 + [P]),
            "moe_shared_ffn": (I32, [cfgp] + [P] * 5 + [P, SZ, P]),
            "moe_update_bias": (I32, [cfgp, P, P, ctypes.c_float, P]),
            "moe_stats": (I32, [cfgp] + [P] * 8 + [P]),
            "moe_router_z_loss": (I32, [cfgp, P, P, P]),
            "moe_layer_forward": (I32, [cfgp] + [P] * 12 + [ctypes.POINTER(moe_aux_outputs), P,
                                                          P, SZ, P]),
            "moe_layer_forward_fp8": (I32, [cfgp] + [P] * 14 + [ctypes.POINTER(moe_aux_outputs),
                                                              P, P, SZ, P]),
            "moe_quantize_rows_fp8": (I32, [P, I64, I64, P, P, P]),
            "moe_combine_backward": (I32, [cfgp] + [P] * 6 + [P]),
            "moe_expert_ffn_backward": (I32, [cfgp] + [P] * 12 + [P, SZ, P]),
            "moe_expert_ffn_backward_fp8": (I32, [cfgp] + [P] * 14 + [P, SZ, P]),
            "moe_router_backward": (I32, [cfgp] + [P] * 10 + [ctypes.c_float, ctypes.c_float]
                                    + [P] * 4 + [P, SZ, P]),
            "moe_layer_backward": (I32, [cfgp] + [P] * 12 + [ctypes.c_float, ctypes.c_float]
                                   + [P] * 8 + [P, SZ, P]),
            "moe_dispatch_fp8": (I32, [cfgp] + [P] * 9 + [P, SZ, P]),
            "moe_expert_ffn_fp8": (I32, [cfgp] + [P] * 9 + [P, SZ, P]),
        }
        for name, (res, args) in sig.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def status_string(status: int) -> str:
    return lib().moe_status_string(status).decode()


def _check(status: int, where: str):
    if status != MOE_OK:
        raise MoeError(status, where)


# --------------------------------------------------------------------------- config
_DT = {"f32": MOE_F32, "bf16": MOE_BF16}
_SC = {"softmax": MOE_SCORE_SOFTMAX, "sigmoid": MOE_SCORE_SIGMOID}
_GT = {"raw": MOE_GATE_RAW, "renorm": MOE_GATE_RENORM}
_FL = {"rank_major": MOE_FILL_RANK_MAJOR, "token_major": MOE_FILL_TOKEN_MAJOR}
_CP = {"assignments": MOE_CAP_ASSIGNMENTS, "tokens": MOE_CAP_TOKENS}


def make_config(w, T: Optional[int] = None) -> moe_config:
    """moe_config from a Workload (mixture_experts_layer_37_amd.inputs); the
    noisy router's draws use the workload's rng_seed and rng_offset."""
    return moe_config(T=w.T if T is None else T, h=w.h, f=w.f, E=w.E, k=w.k,
                      dtype=_DT[w.dtype], score=_SC[w.score], gate=_GT[w.gate],
                      cap_mode=_CP[w.cap_mode], fill=_FL[w.fill], noisy=int(w.noisy),
                      capacity_factor=float(w.capacity_factor),
                      min_capacity=int(w.min_capacity),
                      n_groups=int(getattr(w, "n_groups", 0)),
                      topk_groups=int(getattr(w, "topk_groups", 0)),
                      n_shared=int(getattr(w, "n_shared", 0)),
                      f_shared=int(getattr(w, "f_shared", 0)),
                      seed=int(getattr(w, "rng_seed", 0)),
                      rng_offset=int(getattr(w, "rng_offset", 0)))


def capacity(cfg: moe_config) -> int:
    v = ctypes.c_int64()
    _check(lib().moe_capacity(ctypes.byref(cfg), ctypes.byref(v)), "moe_capacity")
    return v.value


def max_rows(cfg: moe_config) -> int:
    v = ctypes.c_int64()
    _check(lib().moe_max_rows(ctypes.byref(cfg), ctypes.byref(v)), "moe_max_rows")
    return v.value


def workspace_size(cfg: moe_config, entry: int) -> int:
    v = ctypes.c_size_t()
    _check(lib().moe_workspace_size(ctypes.byref(cfg), entry, ctypes.byref(v)),
           "moe_workspace_size")
    return v.value


# --------------------------------------------------------------------------- marshalling
def _elem_dtype(cfg) -> torch.dtype:
    return torch.bfloat16 if cfg.dtype == MOE_BF16 else torch.float32


def _ptr(t: Optional[torch.Tensor], name: str, shape=None, dtype=None, min_numel=None):
    """Device pointer of t after checking it; None gives NULL."""
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name}: expected a tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name}: must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name}: dtype {t.dtype}, expected {dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: shape {tuple(t.shape)}, expected {tuple(shape)}")
    if min_numel is not None and t.numel() < min_numel:
        raise ValueError(f"{name}: needs at least {min_numel} elements")
    return t.data_ptr()


def _stream(stream) -> int:
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


def _ws(ws: torch.Tensor, need: int):
    p = _ptr(ws, "ws", dtype=torch.uint8)
    if ws.numel() < need:
        raise ValueError(f"ws: {ws.numel()} bytes, needs {need}")
    return p, ws.numel()


def new_workspace(cfg: moe_config, entry: int, device="cuda") -> torch.Tensor:
    return torch.empty(max(1, workspace_size(cfg, entry)), dtype=torch.uint8, device=device)


# --------------------------------------------------------------------------- entry points
def moe_route(cfg, U, W_r, b_r, W_noise, topk_idx, topk_gate, logits=None,
              prob_sum=None, ws=None, stream=None, b_sel=None, noise_out=None):
    """Router outputs; noise_out [T, E] float32 (noisy layers, optional): the
    standard-normal draws the library made from cfg.seed and cfg.rng_offset."""
    T, h, E, k = cfg.T, cfg.h, cfg.E, cfg.k
    dt = _elem_dtype(cfg)
    need = workspace_size(cfg, MOE_WS_ROUTE)
    ws = new_workspace(cfg, MOE_WS_ROUTE, U.device) if ws is None else ws
    wp, wn = _ws(ws, need)
    args = [
        _ptr(U, "U", (T, h), dt), _ptr(W_r, "W_r", (h, E), dt),
        _ptr(b_r, "b_r", (E,), torch.float32), _ptr(b_sel, "b_sel", (E,), torch.float32),
        _ptr(W_noise, "W_noise", (h, E), dt) if cfg.noisy else None,
        _ptr(noise_out, "noise_out", (T, E), torch.float32) if cfg.noisy else None,
        _ptr(topk_idx, "topk_idx", (T, k), torch.int32),
        _ptr(topk_gate, "topk_gate", (T, k), torch.float32),
        _ptr(logits, "logits", (T, E), torch.float32),
        _ptr(prob_sum, "prob_sum", (E,), torch.float32),
    ]
    _check(lib().moe_route(ctypes.byref(cfg), *args, wp, wn, _stream(stream)), "moe_route")


def moe_dispatch(cfg, U, topk_idx, X, row_token, slot, count, kept, offset, ws=None,
                 stream=None):
    T, h, E, k = cfg.T, cfg.h, cfg.E, cfg.k
    rows = max_rows(cfg)
    dt = _elem_dtype(cfg)
    need = workspace_size(cfg, MOE_WS_DISPATCH)
    ws = new_workspace(cfg, MOE_WS_DISPATCH, U.device) if ws is None else ws
    wp, wn = _ws(ws, need)
    args = [
        _ptr(U, "U", (T, h), dt), _ptr(topk_idx, "topk_idx", (T, k), torch.int32),
        _ptr(X, "X", (rows, h), dt), _ptr(row_token, "row_token", (rows,), torch.int32),
        _ptr(slot, "slot", (T, k), torch.int32), _ptr(count, "count", (E,), torch.int32),
        _ptr(kept, "kept", (E,), torch.int32), _ptr(offset, "offset", (E + 1,), torch.int32),
    ]
    _check(lib().moe_dispatch(ctypes.byref(cfg), *args, wp, wn, _stream(stream)), "moe_dispatch")
    if _debug.enabled():
        _debug_check(cfg, topk_idx, slot, row_token, count, kept, offset, stream)


def _debug_check(cfg, topk_idx, slot, row_token, count, kept, offset, stream):
    """MOE_DEBUG=1: wait for the stream, download the maps and validate them."""
    (torch.cuda.current_stream() if stream is None else stream).synchronize()
    _debug.check_dispatch_maps(*(t.cpu().numpy() for t in (topk_idx, slot, row_token, count,
                                                            kept, offset)), capacity(cfg))


def moe_stream_read(src, sink, blocks: int, stream=None):
    """One read pass over the bytes of src (a uint8 GPU tensor, size a
    multiple of 16); sink: int32 GPU tensor of at least `blocks` words."""
    _check(lib().moe_stream_read(_ptr(src, "src", dtype=torch.uint8), src.numel(),
                                 _ptr(sink, "sink", dtype=torch.int32, min_numel=blocks),
                                 int(blocks), _stream(stream)), "moe_stream_read")


def moe_dispatch_noalloc(cfg, U, topk_idx, X, row_token, slot, count, kept, offset,
                         stream=None):
    """moe_dispatch without a workspace: its scratch is the library's fixed
    device array (calls overlapping on one GPU race)."""
    T, h, E, k = cfg.T, cfg.h, cfg.E, cfg.k
    rows = max_rows(cfg)
    dt = _elem_dtype(cfg)
    args = [
        _ptr(U, "U", (T, h), dt), _ptr(topk_idx, "topk_idx", (T, k), torch.int32),
        _ptr(X, "X", (rows, h), dt), _ptr(row_token, "row_token", (rows,), torch.int32),
        _ptr(slot, "slot", (T, k), torch.int32), _ptr(count, "count", (E,), torch.int32),
        _ptr(kept, "kept", (E,), torch.int32), _ptr(offset, "offset", (E + 1,), torch.int32),
    ]
    _check(lib().moe_dispatch_noalloc(ctypes.byref(cfg), *args, _stream(stream)),
           "moe_dispatch_noalloc")


def moe_expert_ffn(cfg, X, offset, W_gate, W_up, W_down, Y, ws=None, stream=None):
    h, f, E = cfg.h, cfg.f, cfg.E
    rows = max_rows(cfg)
    dt = _elem_dtype(cfg)
    need = workspace_size(cfg, MOE_WS_EXPERT_FFN)
    ws = new_workspace(cfg, MOE_WS_EXPERT_FFN, X.device) if ws is None else ws
    wp, wn = _ws(ws, need)
    args = [
        _ptr(X, "X", (rows, h), dt), _ptr(offset, "offset", (E + 1,), torch.int32),
        _ptr(W_gate, "W_gate", (E, f, h), dt), _ptr(W_up, "W_up", (E, f, h), dt),
        _ptr(W_down, "W_down", (E, h, f), dt), _ptr(Y, "Y", (rows, h), dt),
    ]
    _check(lib().moe_expert_ffn(ctypes.byref(cfg), *args, wp, wn, _stream(stream)),
           "moe_expert_ffn")


def moe_combine(cfg, U, Y, slot, topk_gate, out, stream=None, Y_shared=None):
    T, h, k = cfg.T, cfg.h, cfg.k
    rows = max_rows(cfg)
    dt = _elem_dtype(cfg)
    args = [
        _ptr(U, "U", (T, h), dt), _ptr(Y, "Y", (rows, h), dt),
        _ptr(slot, "slot", (T, k), torch.int32),
        _ptr(topk_gate, "topk_gate", (T, k), torch.float32),
        _ptr(Y_shared, "Y_shared", (cfg.n_shared, T, h), dt), _ptr(out, "out", (T, h), dt),
    ]
    _check(lib().moe_combine(ctypes.byref(cfg), *args, _stream(stream)), "moe_combine")


def moe_shared_ffn(cfg, U, Ws_gate, Ws_up, Ws_down, Y_shared, ws=None, stream=None):
    T, h, ns, fs = cfg.T, cfg.h, cfg.n_shared, cfg.f_shared
    dt = _elem_dtype(cfg)
    need = workspace_size(cfg, MOE_WS_SHARED_FFN)
    ws = new_workspace(cfg, MOE_WS_SHARED_FFN, U.device) if ws is None else ws
    wp, wn = _ws(ws, need)
    args = [
        _ptr(U, "U", (T, h), dt), _ptr(Ws_gate, "Ws_gate", (ns, fs, h), dt),
        _ptr(Ws_up, "Ws_up", (ns, fs, h), dt), _ptr(Ws_down, "Ws_down", (ns, h, fs), dt),
        _ptr(Y_shared, "Y_shared", (ns, T, h), dt),
    ]
    _check(lib().moe_shared_ffn(ctypes.byref(cfg), *args, wp, wn, _stream(stream)),
           "moe_shared_ffn")


def moe_update_bias(cfg, count, b_sel, gamma: float, stream=None):
    E = cfg.E
    _check(lib().moe_update_bias(ctypes.byref(cfg), _ptr(count, "count", (E,), torch.int32),
                                 _ptr(b_sel, "b_sel", (E,), torch.float32), float(gamma),
                                 _stream(stream)), "moe_update_bias")


def moe_stats(cfg, count, kept, prob_sum, f=None, P=None, aux_loss=None, maxvio=None,
              n_dropped=None, stream=None):
    E = cfg.E
    args = [
        _ptr(count, "count", (E,), torch.int32), _ptr(kept, "kept", (E,), torch.int32),
        _ptr(prob_sum, "prob_sum", (E,), torch.float32), _ptr(f, "f", (E,), torch.float32),
        _ptr(P, "P", (E,), torch.float32), _ptr(aux_loss, "aux_loss", (1,), torch.float32),
        _ptr(maxvio, "maxvio", (1,), torch.float32),
        _ptr(n_dropped, "n_dropped", (1,), torch.int32),
    ]
    _check(lib().moe_stats(ctypes.byref(cfg), *args, _stream(stream)), "moe_stats")


def moe_router_z_loss(cfg, logits, z_loss, stream=None):
    """z_loss[0] = mean over tokens of the squared log-sum-exp of logits [T, E]."""
    _check(lib().moe_router_z_loss(ctypes.byref(cfg),
                                   _ptr(logits, "logits", (cfg.T, cfg.E), torch.float32),
                                   _ptr(z_loss, "z_loss", (1,), torch.float32),
                                   _stream(stream)), "moe_router_z_loss")


_AUX_SPEC = {
    "topk_idx": (lambda c, r: (c.T, c.k), torch.int32),
    "topk_gate": (lambda c, r: (c.T, c.k), torch.float32),
    "logits": (lambda c, r: (c.T, c.E), torch.float32),
    "slot": (lambda c, r: (c.T, c.k), torch.int32),
    "row_token": (lambda c, r: (r,), torch.int32),
    "count": (lambda c, r: (c.E,), torch.int32),
    "kept": (lambda c, r: (c.E,), torch.int32),
    "offset": (lambda c, r: (c.E + 1,), torch.int32),
    "prob_sum": (lambda c, r: (c.E,), torch.float32),
    "f": (lambda c, r: (c.E,), torch.float32),
    "P": (lambda c, r: (c.E,), torch.float32),
    "aux_loss": (lambda c, r: (1,), torch.float32),
    "maxvio": (lambda c, r: (1,), torch.float32),
    "n_dropped": (lambda c, r: (1,), torch.int32),
    "X": (lambda c, r: (r, c.h), None),
    "Y": (lambda c, r: (r, c.h), None),
    "Y_shared": (lambda c, r: (c.n_shared, c.T, c.h), None),
    "z_loss": (lambda c, r: (1,), torch.float32),
    "GU": (lambda c, r: (r, 2 * c.f), None),
    "A": (lambda c, r: (r, c.f), None),
    "noise": (lambda c, r: (c.T, c.E), torch.float32),
}

# the forward's outputs that moe_layer_backward can take instead of recomputing
SAVED_FIELDS = ("X", "GU", "A", "Y")


def alloc_aux(cfg, device="cuda", fields=None) -> dict:
    """Allocate device tensors for the optional outputs named in `fields` (all by default)."""
    rows = max_rows(cfg)
    out = {}
    for name in (AUX_FIELDS if fields is None else fields):
        shape_fn, dt = _AUX_SPEC[name]
        out[name] = torch.empty(shape_fn(cfg, rows), dtype=dt or _elem_dtype(cfg), device=device)
    return out


def _layer_call(fn_name, cfg, U, W_r, b_r, W_noise, weights, W_down, out, aux,
                stage_events, ws, stream, b_sel, Ws_gate, Ws_up, Ws_down):
    """Argument marshalling shared by moe_layer_forward and moe_layer_forward_fp8;
    weights: the already checked pointers that stand between W_noise and W_down."""
    T, h, f, E = cfg.T, cfg.h, cfg.f, cfg.E
    ns, fs = cfg.n_shared, cfg.f_shared
    rows = max_rows(cfg)
    dt = _elem_dtype(cfg)
    need = workspace_size(cfg, MOE_WS_LAYER)
    ws = new_workspace(cfg, MOE_WS_LAYER, W_r.device) if ws is None else ws
    wp, wn = _ws(ws, need)
    a = moe_aux_outputs()
    for name, t in (aux or {}).items():
        if name not in _AUX_SPEC:
            raise KeyError(name)
        shape_fn, adt = _AUX_SPEC[name]
        setattr(a, name, _ptr(t, name, shape_fn(cfg, rows), adt or dt))
    ev = None
    if stage_events is not None:
        if len(stage_events) != MOE_NUM_STAGES + 1:
            raise ValueError("stage_events needs MOE_NUM_STAGES + 1 events")
        handles = []
        for e in stage_events:
            if e is None:  # that boundary is not recorded
                handles.append(None)
                continue
            if e.cuda_event == 0:  # torch creates the HIP event lazily
                e.record()
            handles.append(e.cuda_event)
        ev = (ctypes.c_void_p * len(handles))(*handles)
    args = [
        _ptr(U, "U", (T, h), dt), _ptr(W_r, "W_r", (h, E), dt),
        _ptr(b_r, "b_r", (E,), torch.float32), _ptr(b_sel, "b_sel", (E,), torch.float32),
        _ptr(W_noise, "W_noise", (h, E), dt) if cfg.noisy else None,
        *weights,
        _ptr(W_down, "W_down", (E, h, f), dt),
        _ptr(Ws_gate, "Ws_gate", (ns, fs, h), dt) if ns else None,
        _ptr(Ws_up, "Ws_up", (ns, fs, h), dt) if ns else None,
        _ptr(Ws_down, "Ws_down", (ns, h, fs), dt) if ns else None,
        _ptr(out, "out", (T, h), dt),
    ]
    _check(getattr(lib(), fn_name)(ctypes.byref(cfg), *args, ctypes.byref(a),
                                   ctypes.cast(ev, ctypes.c_void_p) if ev is not None else None,
                                   wp, wn, _stream(stream)), fn_name)
    maps = ("topk_idx", "slot", "row_token", "count", "kept", "offset")
    if _debug.enabled() and aux and all(aux.get(n) is not None for n in maps):
        _debug_check(cfg, *(aux[n] for n in maps), stream)


def moe_layer_forward(cfg, U, W_r, b_r, W_noise, W_gate, W_up, W_down, out, aux=None,
                      stage_events=None, ws=None, stream=None, b_sel=None, Ws_gate=None,
                      Ws_up=None, Ws_down=None):
    """The whole layer.  aux: dict of optional output tensors (see alloc_aux).
    stage_events: list of MOE_NUM_STAGES + 1 torch.cuda.Event(enable_timing=True) or None,
    recorded inside the library on the same stream.  b_sel, Ws_*: the
    selection bias and the shared-expert weights (cfg.n_shared > 0)."""
    E, f, h, dt = cfg.E, cfg.f, cfg.h, _elem_dtype(cfg)
    weights = [_ptr(W_gate, "W_gate", (E, f, h), dt), _ptr(W_up, "W_up", (E, f, h), dt)]
    _layer_call("moe_layer_forward", cfg, U, W_r, b_r, W_noise, weights, W_down, out, aux,
                stage_events, ws, stream, b_sel, Ws_gate, Ws_up, Ws_down)


def moe_layer_forward_fp8(cfg, U, W_r, b_r, W_noise, W8_gate, s_gate, W8_up, s_up,
                          W_down, out, aux=None, stage_events=None, ws=None, stream=None,
                          b_sel=None, Ws_gate=None, Ws_up=None, Ws_down=None):
    """The layer with the FP8 dispatch and up-projection: W8_* are E4M3 codes
    (uint8 [E, f, h]) with row scales s_* (float32 [E, f]) from
    moe_quantize_rows_fp8; everything else as in moe_layer_forward."""
    E, f, h = cfg.E, cfg.f, cfg.h
    weights = [_ptr(W8_gate, "W8_gate", (E, f, h), torch.uint8),
               _ptr(s_gate, "s_gate", (E, f), torch.float32),
               _ptr(W8_up, "W8_up", (E, f, h), torch.uint8),
               _ptr(s_up, "s_up", (E, f), torch.float32)]
    _layer_call("moe_layer_forward_fp8", cfg, U, W_r, b_r, W_noise, weights, W_down, out,
                aux, stage_events, ws, stream, b_sel, Ws_gate, Ws_up, Ws_down)


def moe_layer_backward(cfg, U, W_r, W_gate, W_up, W_down, logits, topk_idx, topk_gate, slot,
                       count, offset, dOut, dU, dW_r, dW_gate, dW_up, dW_down, db_r=None,
                       alpha=0.0, c_z=0.0, saved=None, W_noise=None, dW_noise=None,
                       Ws_gate=None, Ws_up=None, Ws_down=None, dWs_gate=None, dWs_up=None,
                       dWs_down=None, W_downT8=None, s_downT=None, ws=None, stream=None):
    """Gradients of <dOut, out> + alpha aux_loss + c_z z_loss for the routing of a
    forward (logits ... offset from its aux outputs).  dU, dW_gate, dW_up,
    dW_down bf16; dW_r [h, E] and db_r [E] float32.  saved: None (the experts
    are recomputed) or a dict with the forward's aux outputs X, GU, A and Y.
    Noisy layers: W_noise as in the forward (the draws come again from cfg's seed
    and rng_offset), dW_noise [h, E] float32.
    Shared experts: Ws_* as in the forward, dWs_* of the same shapes (bf16).
    FP8 output gradients: W_downT8 [E, f, h] uint8 and s_downT [E, f], the
    row-wise E4M3 quantisation of W_down transposed."""
    T, h, f, E, k = cfg.T, cfg.h, cfg.f, cfg.E, cfg.k
    bf = torch.bfloat16
    need = workspace_size(cfg, MOE_WS_BACKWARD)
    ws = new_workspace(cfg, MOE_WS_BACKWARD, W_r.device) if ws is None else ws
    wp, wn = _ws(ws, need)
    args = [
        _ptr(U, "U", (T, h), bf), _ptr(W_r, "W_r", (h, E), bf),
        _ptr(W_gate, "W_gate", (E, f, h), bf), _ptr(W_up, "W_up", (E, f, h), bf),
        _ptr(W_down, "W_down", (E, h, f), bf), _ptr(logits, "logits", (T, E), torch.float32),
        _ptr(topk_idx, "topk_idx", (T, k), torch.int32),
        _ptr(topk_gate, "topk_gate", (T, k), torch.float32),
        _ptr(slot, "slot", (T, k), torch.int32), _ptr(count, "count", (E,), torch.int32),
        _ptr(offset, "offset", (E + 1,), torch.int32), _ptr(dOut, "dOut", (T, h), bf),
        ctypes.c_float(alpha), ctypes.c_float(c_z),
        _ptr(dU, "dU", (T, h), bf), _ptr(dW_r, "dW_r", (h, E), torch.float32),
        _ptr(db_r, "db_r", (E,), torch.float32), _ptr(dW_gate, "dW_gate", (E, f, h), bf),
        _ptr(dW_up, "dW_up", (E, f, h), bf), _ptr(dW_down, "dW_down", (E, h, f), bf),
    ]
    sv = None
    if saved is not None:
        sv = moe_aux_outputs()
        rows = max_rows(cfg)
        for name in SAVED_FIELDS:
            shape_fn, _ = _AUX_SPEC[name]
            setattr(sv, name, _ptr(saved[name], name, shape_fn(cfg, rows), bf))
    ex = None
    if cfg.noisy or cfg.n_shared or W_downT8 is not None:
        ex = moe_backward_extras()
        if W_downT8 is not None:
            ex.W_downT8 = _ptr(W_downT8, "W_downT8", (E, f, h), torch.uint8)
            ex.s_downT = _ptr(s_downT, "s_downT", (E, f), torch.float32)
        ns, fs = cfg.n_shared, cfg.f_shared
        if cfg.noisy:
            ex.W_noise = _ptr(W_noise, "W_noise", (h, E), bf)
            ex.dW_noise = _ptr(dW_noise, "dW_noise", (h, E), torch.float32)
        if ns:
            ex.Ws_gate = _ptr(Ws_gate, "Ws_gate", (ns, fs, h), bf)
            ex.Ws_up = _ptr(Ws_up, "Ws_up", (ns, fs, h), bf)
            ex.Ws_down = _ptr(Ws_down, "Ws_down", (ns, h, fs), bf)
            ex.dWs_gate = _ptr(dWs_gate, "dWs_gate", (ns, fs, h), bf)
            ex.dWs_up = _ptr(dWs_up, "dWs_up", (ns, fs, h), bf)
            ex.dWs_down = _ptr(dWs_down, "dWs_down", (ns, h, fs), bf)
    _check(lib().moe_layer_backward(ctypes.byref(cfg), *args,
                                    ctypes.byref(sv) if sv is not None else None,
                                    ctypes.byref(ex) if ex is not None else None, wp, wn,
                                    _stream(stream)), "moe_layer_backward")


def moe_combine_backward(cfg, dOut, Y, slot, topk_gate, dY, dgate, stream=None):
    """dY[slot] = gate * dOut for every kept rank, dgate = dOut . Y[slot]."""
    T, h, k = cfg.T, cfg.h, cfg.k
    rows, bf = max_rows(cfg), torch.bfloat16
    _check(lib().moe_combine_backward(
        ctypes.byref(cfg), _ptr(dOut, "dOut", (T, h), bf), _ptr(Y, "Y", (rows, h), bf),
        _ptr(slot, "slot", (T, k), torch.int32),
        _ptr(topk_gate, "topk_gate", (T, k), torch.float32), _ptr(dY, "dY", (rows, h), bf),
        _ptr(dgate, "dgate", (T, k), torch.float32), _stream(stream)), "moe_combine_backward")


def moe_expert_ffn_backward(cfg, X, offset, W_gate, W_up, W_down, dY, dX, dW_gate, dW_up,
                            dW_down, GU=None, A=None, ws=None, stream=None):
    """The experts' products backward for rows X and output gradients dY: dX rows and
    the weight gradients.  GU, A: the forward's kept g | u and a, or None to
    recompute them."""
    h, f, E = cfg.h, cfg.f, cfg.E
    rows, bf = max_rows(cfg), torch.bfloat16
    need = workspace_size(cfg, MOE_WS_EXPERT_FFN_BACKWARD)
    ws = new_workspace(cfg, MOE_WS_EXPERT_FFN_BACKWARD, W_gate.device) if ws is None else ws
    wp, wn = _ws(ws, need)
    _check(lib().moe_expert_ffn_backward(
        ctypes.byref(cfg), _ptr(X, "X", (rows, h), bf),
        _ptr(offset, "offset", (E + 1,), torch.int32), _ptr(W_gate, "W_gate", (E, f, h), bf),
        _ptr(W_up, "W_up", (E, f, h), bf), _ptr(W_down, "W_down", (E, h, f), bf),
        _ptr(dY, "dY", (rows, h), bf), _ptr(GU, "GU", (rows, 2 * f), bf),
        _ptr(A, "A", (rows, f), bf), _ptr(dX, "dX", (rows, h), bf),
        _ptr(dW_gate, "dW_gate", (E, f, h), bf), _ptr(dW_up, "dW_up", (E, f, h), bf),
        _ptr(dW_down, "dW_down", (E, h, f), bf), wp, wn, _stream(stream)),
        "moe_expert_ffn_backward")


def moe_expert_ffn_backward_fp8(cfg, X, offset, W_gate, W_up, W_downT8, s_downT, dY8, dY_scale,
                                dX, dW_gate, dW_up, dW_down, GU=None, A=None, ws=None,
                                stream=None):
    """moe_expert_ffn_backward with the output gradients as FP8 rows (dY8 uint8
    [rows_max, h], dY_scale [rows_max]) and W_down^T quantised row-wise
    (W_downT8 [E, f, h], s_downT [E, f])."""
    h, f, E = cfg.h, cfg.f, cfg.E
    rows, bf = max_rows(cfg), torch.bfloat16
    need = workspace_size(cfg, MOE_WS_EXPERT_FFN_BACKWARD)
    ws = new_workspace(cfg, MOE_WS_EXPERT_FFN_BACKWARD, W_gate.device) if ws is None else ws
    wp, wn = _ws(ws, need)
    _check(lib().moe_expert_ffn_backward_fp8(
        ctypes.byref(cfg), _ptr(X, "X", (rows, h), bf),
        _ptr(offset, "offset", (E + 1,), torch.int32), _ptr(W_gate, "W_gate", (E, f, h), bf),
        _ptr(W_up, "W_up", (E, f, h), bf), _ptr(W_downT8, "W_downT8", (E, f, h), torch.uint8),
        _ptr(s_downT, "s_downT", (E, f), torch.float32),
        _ptr(dY8, "dY8", (rows, h), torch.uint8),
        _ptr(dY_scale, "dY_scale", (rows,), torch.float32), _ptr(GU, "GU", (rows, 2 * f), bf),
        _ptr(A, "A", (rows, f), bf), _ptr(dX, "dX", (rows, h), bf),
        _ptr(dW_gate, "dW_gate", (E, f, h), bf), _ptr(dW_up, "dW_up", (E, f, h), bf),
        _ptr(dW_down, "dW_down", (E, h, f), bf), wp, wn, _stream(stream)),
        "moe_expert_ffn_backward_fp8")


def moe_router_backward(cfg, U, W_r, logits, topk_idx, topk_gate, slot, count, dgate, dOut, dX,
                        dU, dW_r, db_r=None, alpha=0.0, c_z=0.0, W_noise=None,
                        dW_noise=None, ws=None, stream=None):
    """dH from the gates' gradient (and the aux and z terms), then
    dU = dOut + sum dX[slot] + dH W_r^T, dW_r, db_r (dW_noise for noisy layers)."""
    T, h, E, k = cfg.T, cfg.h, cfg.E, cfg.k
    rows, bf = max_rows(cfg), torch.bfloat16
    need = workspace_size(cfg, MOE_WS_ROUTER_BACKWARD)
    ws = new_workspace(cfg, MOE_WS_ROUTER_BACKWARD, W_r.device) if ws is None else ws
    wp, wn = _ws(ws, need)
    ex = None
    if cfg.noisy:
        ex = moe_backward_extras()
        ex.W_noise = _ptr(W_noise, "W_noise", (h, E), bf)
        ex.dW_noise = _ptr(dW_noise, "dW_noise", (h, E), torch.float32)
    _check(lib().moe_router_backward(
        ctypes.byref(cfg), _ptr(U, "U", (T, h), bf), _ptr(W_r, "W_r", (h, E), bf),
        _ptr(logits, "logits", (T, E), torch.float32),
        _ptr(topk_idx, "topk_idx", (T, k), torch.int32),
        _ptr(topk_gate, "topk_gate", (T, k), torch.float32),
        _ptr(slot, "slot", (T, k), torch.int32), _ptr(count, "count", (E,), torch.int32),
        _ptr(dgate, "dgate", (T, k), torch.float32), _ptr(dOut, "dOut", (T, h), bf),
        _ptr(dX, "dX", (rows, h), bf), ctypes.c_float(alpha), ctypes.c_float(c_z),
        ctypes.byref(ex) if ex is not None else None, _ptr(dU, "dU", (T, h), bf),
        _ptr(dW_r, "dW_r", (h, E), torch.float32), _ptr(db_r, "db_r", (E,), torch.float32),
        wp, wn, _stream(stream)), "moe_router_backward")


def moe_quantize_rows_fp8(src, dst=None, scale=None, stream=None):
    """Row-wise E4M3 codes (uint8, shape of src) and power-of-two scales
    (float32, src.shape[:-1]) of a bf16 tensor src [..., cols]."""
    if src.dtype != torch.bfloat16:
        raise ValueError("src: expected bfloat16")
    cols = src.shape[-1]
    rows = src.numel() // cols if cols else 0
    dst = torch.empty(src.shape, dtype=torch.uint8, device=src.device) if dst is None else dst
    scale = (torch.empty(src.shape[:-1], dtype=torch.float32, device=src.device)
             if scale is None else scale)
    _check(lib().moe_quantize_rows_fp8(_ptr(src, "src", tuple(src.shape), torch.bfloat16), rows,
                                       cols, _ptr(dst, "dst", tuple(src.shape), torch.uint8),
                                       _ptr(scale, "scale", tuple(src.shape[:-1]), torch.float32),
                                       _stream(stream)), "moe_quantize_rows_fp8")
    return dst, scale


def moe_dispatch_fp8(cfg, U, topk_idx, X8, x_scale, row_token, slot, count, kept, offset,
                     ws=None, stream=None):
    T, h, E, k = cfg.T, cfg.h, cfg.E, cfg.k
    rows = max_rows(cfg)
    need = workspace_size(cfg, MOE_WS_DISPATCH)
    ws = new_workspace(cfg, MOE_WS_DISPATCH, U.device) if ws is None else ws
    wp, wn = _ws(ws, need)
    args = [
        _ptr(U, "U", (T, h), torch.bfloat16), _ptr(topk_idx, "topk_idx", (T, k), torch.int32),
        _ptr(X8, "X8", (rows, h), torch.uint8), _ptr(x_scale, "x_scale", (rows,), torch.float32),
        _ptr(row_token, "row_token", (rows,), torch.int32),
        _ptr(slot, "slot", (T, k), torch.int32), _ptr(count, "count", (E,), torch.int32),
        _ptr(kept, "kept", (E,), torch.int32), _ptr(offset, "offset", (E + 1,), torch.int32),
    ]
    _check(lib().moe_dispatch_fp8(ctypes.byref(cfg), *args, wp, wn, _stream(stream)),
           "moe_dispatch_fp8")
    if _debug.enabled():
        _debug_check(cfg, topk_idx, slot, row_token, count, kept, offset, stream)


def moe_expert_ffn_fp8(cfg, X8, x_scale, offset, W8_gate, s_gate, W8_up, s_up, W_down, Y,
                       ws=None, stream=None):
    h, f, E = cfg.h, cfg.f, cfg.E
    rows = max_rows(cfg)
    need = workspace_size(cfg, MOE_WS_EXPERT_FFN)
    ws = new_workspace(cfg, MOE_WS_EXPERT_FFN, X8.device) if ws is None else ws
    wp, wn = _ws(ws, need)
    args = [
        _ptr(X8, "X8", (rows, h), torch.uint8), _ptr(x_scale, "x_scale", (rows,), torch.float32),
        _ptr(offset, "offset", (E + 1,), torch.int32),
        _ptr(W8_gate, "W8_gate", (E, f, h), torch.uint8),
        _ptr(s_gate, "s_gate", (E, f), torch.float32),
        _ptr(W8_up, "W8_up", (E, f, h), torch.uint8), _ptr(s_up, "s_up", (E, f), torch.float32),
        _ptr(W_down, "W_down", (E, h, f), torch.bfloat16), _ptr(Y, "Y", (rows, h), torch.bfloat16),
    ]
    _check(lib().moe_expert_ffn_fp8(ctypes.byref(cfg), *args, wp, wn, _stream(stream)),
           "moe_expert_ffn_fp8")
