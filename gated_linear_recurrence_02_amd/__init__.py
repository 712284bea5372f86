"""Python binding of librglru.so, the MI355X RG-LRU hot-path library.

Argument marshalling only: each function checks its torch tensors (device,
dtype, contiguity, shape), allocates outputs with torch, and calls the C entry
point of the same name (declared in include/rglru.h) on the current HIP
stream.  Every step of the computation runs in the library's HIP kernels;
there is no fallback: if the library is missing, importing works but every
call raises.

Layouts (row-major, channel fastest): activations [B][T][D], conv history
[B][3][D], state [B][D] fp32, conv_w [D][4] fp32, W_a / W_x [H][K][K] in the
activation dtype with K = 256, b_a / b_x / conv_b / Lambda [D] fp32.
"""
from __future__ import annotations

import ctypes
import dataclasses
import os
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "librglru.so")

F32, BF16 = 0, 1
OP_SCAN_FWD, OP_SCAN_BWD = 0, 1
_IO = {torch.float32: F32, torch.bfloat16: BF16}


class RGLRUError(RuntimeError):
    """A non-zero status from the C library."""


class _Desc(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int64), ("T", ctypes.c_int64), ("D", ctypes.c_int64),
                ("H", ctypes.c_int64), ("io", ctypes.c_int32), ("c", ctypes.c_float)]


class _Weights(ctypes.Structure):
    _fields_ = [("conv_w", ctypes.c_void_p), ("conv_b", ctypes.c_void_p),
                ("W_a", ctypes.c_void_p), ("b_a", ctypes.c_void_p),
                ("W_x", ctypes.c_void_p), ("b_x", ctypes.c_void_p),
                ("Lambda", ctypes.c_void_p)]


class _AttnDesc(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int64), ("T", ctypes.c_int64), ("Hq", ctypes.c_int64),
                ("dh", ctypes.c_int64), ("W", ctypes.c_int64), ("io", ctypes.c_int32),
                ("scale", ctypes.c_float)]


class _Layer(ctypes.Structure):
    _fields_ = [("tnorm_w", ctypes.c_void_p), ("cnorm_w", ctypes.c_void_p), ("gate_w", ctypes.c_void_p),
                ("up_w", ctypes.c_void_p), ("down_w", ctypes.c_void_p), ("d_ff", ctypes.c_int64),
                ("eps", ctypes.c_float)]


class _AttnProj(ctypes.Structure):
    _fields_ = [("wq", ctypes.c_void_p), ("wk", ctypes.c_void_p), ("wv", ctypes.c_void_p), ("wo", ctypes.c_void_p)]


class _Block(ctypes.Structure):
    _fields_ = [("proj_in_1", ctypes.c_void_p), ("proj_in_2", ctypes.c_void_p),
                ("proj_out", ctypes.c_void_p)]


# size of the scratch behind rglru_scan_fwd_noalloc (RGLRU_NOALLOC_SCRATCH_BYTES)
NOALLOC_SCRATCH_BYTES = 64 << 20

_lib = None
SYMBOLS = ("rglru_workspace_size", "rglru_workspace_status", "rglru_conv1d", "rglru_gates", "rglru_scan_fwd",
           "rglru_scan_fwd_noalloc",
           "rglru_step", "rglru_scan_bwd", "rglru_block_workspace_size", "rglru_block_fwd",
           "rglru_attn_fwd", "rglru_attn_workspace_size", "rglru_attn_step", "rglru_layer_workspace_size",
           "rglru_layer_fwd", "rglru_attn_layer_workspace_size", "rglru_attn_layer_fwd",
           "rglru_status_string")


def lib():
    """Load librglru.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RGLRUError(f"{LIB_PATH} is not built; run gated_linear_recurrence_02_amd/build.py")
        L = ctypes.CDLL(LIB_PATH)
        vp, sz = ctypes.c_void_p, ctypes.c_size_t
        D, W = ctypes.POINTER(_Desc), ctypes.POINTER(_Weights)
        L.rglru_status_string.restype = ctypes.c_char_p
        L.rglru_status_string.argtypes = [ctypes.c_int]
        L.rglru_workspace_size.argtypes = [D, ctypes.c_int, ctypes.POINTER(sz)]
        L.rglru_workspace_status.argtypes = [vp, sz, vp]
        L.rglru_conv1d.argtypes = [D, vp, vp, vp, vp, vp, vp, vp]
        L.rglru_gates.argtypes = [D, W, vp, vp, vp, vp]
        L.rglru_scan_fwd.argtypes = [D, W, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
        L.rglru_scan_fwd_noalloc.argtypes = [D, W, vp, vp, vp, vp, vp, vp, vp, vp, vp]
        L.rglru_step.argtypes = [D, W, vp, vp, vp, vp, vp, vp]
        L.rglru_scan_bwd.argtypes = [D, W, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
        A = ctypes.POINTER(_AttnDesc)
        L.rglru_attn_fwd.argtypes = [A, vp, vp, vp, vp, vp, vp, vp]
        L.rglru_attn_workspace_size.argtypes = [A, ctypes.POINTER(sz)]
        L.rglru_attn_step.argtypes = [A, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
        LY = ctypes.POINTER(_Layer)
        L.rglru_layer_workspace_size.argtypes = [D, ctypes.c_int64, LY, ctypes.POINTER(sz)]
        L.rglru_layer_fwd.argtypes = [D, ctypes.c_int64, W, ctypes.POINTER(_Block), LY, vp, vp, vp, vp, vp, vp, vp,
                                      sz, vp]
        L.rglru_attn_layer_workspace_size.argtypes = [A, ctypes.c_int64, LY, ctypes.POINTER(sz)]
        L.rglru_attn_layer_fwd.argtypes = [A, ctypes.c_int64, ctypes.c_int32, ctypes.c_float, ctypes.c_int64,
                                           ctypes.POINTER(_AttnProj), LY, vp, vp, vp, vp, vp, sz, vp]
        L.rglru_block_workspace_size.argtypes = [D, ctypes.c_int64, ctypes.POINTER(sz)]
        L.rglru_block_fwd.argtypes = [D, ctypes.c_int64, W, ctypes.POINTER(_Block), vp, vp, vp, vp, vp, vp,
                                      vp, sz, vp]
        for s in SYMBOLS:
            if s != "rglru_status_string":
                getattr(L, s).restype = ctypes.c_int
        _lib = L
    return _lib


def _check(rc: int, what: str) -> None:
    if rc != 0:
        msg = lib().rglru_status_string(rc).decode()
        raise RGLRUError(f"{what} failed with status {rc}: {msg}")


@dataclasses.dataclass
class Weights:
    """Device tensors of one RG-LRU layer's parameters (conv_b, b_a, b_x optional)."""
    conv_w: torch.Tensor
    W_a: torch.Tensor
    W_x: torch.Tensor
    Lambda: torch.Tensor
    conv_b: Optional[torch.Tensor] = None
    b_a: Optional[torch.Tensor] = None
    b_x: Optional[torch.Tensor] = None
    c: float = 8.0

    @property
    def H(self) -> int:
        return int(self.W_a.shape[0])


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else t.data_ptr()


def _need(t, name, device, dtype=None, shape=None):
    if t is None:
        return
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name} must be a torch.Tensor")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


def _io(t: torch.Tensor) -> int:
    if t.dtype not in _IO:
        raise ValueError(f"activations must be float32 or bfloat16, got {t.dtype}")
    return _IO[t.dtype]


def _stream(device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _weights_struct(w: Weights, D: int, dtype, device, conv: bool, gates: bool):
    if gates:
        H = w.H
        _need(w.W_a, "W_a", device, dtype, (H, D // H, D // H))
        _need(w.W_x, "W_x", device, dtype, (H, D // H, D // H))
        _need(w.b_a, "b_a", device, torch.float32, (D,))
        _need(w.b_x, "b_x", device, torch.float32, (D,))
    if conv:
        _need(w.conv_w, "conv_w", device, torch.float32, (D, 4))
        _need(w.conv_b, "conv_b", device, torch.float32, (D,))
    _need(w.Lambda, "Lambda", device, torch.float32, (D,))
    return _Weights(_ptr(w.conv_w) if conv else None, _ptr(w.conv_b) if conv else None,
                    _ptr(w.W_a) if gates else None, _ptr(w.b_a) if gates else None,
                    _ptr(w.W_x) if gates else None, _ptr(w.b_x) if gates else None,
                    _ptr(w.Lambda))


# ------------------------------------------------------------------ workspace
_ws_cache = {}   # (device, kind) -> [buffer, layout key]


def workspace_size(B, T, D, H, io=BF16, op=OP_SCAN_FWD, c=8.0) -> int:
    n = ctypes.c_size_t(0)
    _check(lib().rglru_workspace_size(ctypes.byref(_Desc(B, T, D, H, io, c)), op, ctypes.byref(n)),
           "rglru_workspace_size")
    return int(n.value)


def block_workspace_size(B, T, D, H, d_model, io=BF16, c=8.0) -> int:
    n = ctypes.c_size_t(0)
    _check(lib().rglru_block_workspace_size(ctypes.byref(_Desc(B, T, D, H, io, c)), d_model,
                                            ctypes.byref(n)), "rglru_block_workspace_size")
    return int(n.value)


def workspace(nbytes: int, device, kind: str = "fwd", key=None) -> torch.Tensor:
    """A zero-filled workspace of at least nbytes, one cached buffer per device
    and kind ("fwd", "bwd", "block", ...).

    The library restores the workspace header at the end of every call, so the
    cached buffer can be reused by calls that run one after another (one
    stream).  A forward-scan workspace holds only counters (at fixed offsets)
    and tagged carry words, so it serves forward calls of any shape.  The
    backward's and the block's also keep plain data, which must not sit where
    a later call of another layout expects carry words: when `key` (the
    layout: shape and dtype) differs from the previous call's, the buffer is
    zero-filled again, on the current stream, before it is handed out.  Calls
    that may overlap need workspaces of their own."""
    device = torch.device(device)
    ent = _ws_cache.get((device, kind))
    if ent is None or ent[0].numel() < nbytes:
        ent = [torch.zeros(max(nbytes, 256), dtype=torch.uint8, device=device), key]
        _ws_cache[(device, kind)] = ent
    elif key != ent[1]:
        ent[0].zero_()
        ent[1] = key
    return ent[0]


def workspace_status(device, kind: str = "fwd") -> None:
    """Wait for the current stream and raise RGLRUError if a chunk-carry wait
    of a call that used the cached workspace of this kind gave up (its
    outputs hold NaN); the report is cleared (rglru_workspace_status)."""
    device = torch.device(device)
    ent = _ws_cache.get((device, kind))
    if ent is None:
        return
    _check(lib().rglru_workspace_status(_ptr(ent[0]), ent[0].numel(), _stream(device)),
           "rglru_workspace_status")


# ----------------------------------------------------------------- entry points
def conv1d(u: torch.Tensor, conv_w: torch.Tensor, conv_b=None, hist_in=None, H: int = 1,
           out=None, hist_out_buf=None):
    """x = causal depthwise conv of u (width 4).  Returns (x, hist_out).

    out / hist_out_buf: optional preallocated outputs."""
    dev = u.device
    _need(u, "u", dev)
    B, T, D = u.shape
    _need(conv_w, "conv_w", dev, torch.float32, (D, 4))
    _need(conv_b, "conv_b", dev, torch.float32, (D,))
    _need(hist_in, "hist_in", dev, u.dtype, (B, 3, D))
    x = torch.empty_like(u) if out is None else out
    hist_out = torch.empty((B, 3, D), dtype=u.dtype, device=dev) if hist_out_buf is None else hist_out_buf
    _need(x, "out", dev, u.dtype, (B, T, D))
    _need(hist_out, "hist_out_buf", dev, u.dtype, (B, 3, D))
    d = _Desc(B, T, D, H, _io(u), 8.0)
    _check(lib().rglru_conv1d(ctypes.byref(d), _ptr(conv_w), _ptr(conv_b), _ptr(u), _ptr(hist_in),
                              _ptr(x), _ptr(hist_out), _stream(dev)), "rglru_conv1d")
    return x, hist_out


def gates(x: torch.Tensor, w: Weights, r_out=None, i_out=None):
    """(r, i) = (sigmoid(W_a x + b_a), sigmoid(W_x x + b_x)), block-diagonal.

    r_out / i_out: optional preallocated outputs."""
    dev = x.device
    _need(x, "x", dev)
    B, T, D = x.shape
    ws = _weights_struct(w, D, x.dtype, dev, conv=False, gates=True)
    r = torch.empty_like(x) if r_out is None else r_out
    i = torch.empty_like(x) if i_out is None else i_out
    _need(r, "r_out", dev, x.dtype, (B, T, D))
    _need(i, "i_out", dev, x.dtype, (B, T, D))
    d = _Desc(B, T, D, w.H, _io(x), w.c)
    _check(lib().rglru_gates(ctypes.byref(d), ctypes.byref(ws), _ptr(x), _ptr(r), _ptr(i),
                             _stream(dev)), "rglru_gates")
    return r, i


def scan_fwd(inp: torch.Tensor, w: Weights, *, r=None, i=None, h0=None, hist_in=None,
             conv: bool = True, want_hist: bool = True, out=None, h_last_out=None,
             hist_out_buf=None):
    """Forward scan.  Mode A (conv=True, no r/i): inp is pre-conv u.  Mode B
    (conv=False, no r/i): inp is x.  Mode C (r and i given): inp is x, scan only.
    Returns (y, h_last, hist_out or None)."""
    return _scan_fwd(inp, w, r, i, h0, hist_in, conv, want_hist, out, h_last_out, hist_out_buf, False)


def scan_fwd_noalloc(inp: torch.Tensor, w: Weights, *, r=None, i=None, h0=None, hist_in=None,
                     conv: bool = True, want_hist: bool = True, out=None, h_last_out=None,
                     hist_out_buf=None):
    """scan_fwd through rglru_scan_fwd_noalloc: the chunk carries live in the
    library's fixed per-device scratch instead of a workspace (calls on one
    device must not overlap).  Outputs not passed in are allocated here, by
    the binding; the library call allocates nothing."""
    return _scan_fwd(inp, w, r, i, h0, hist_in, conv, want_hist, out, h_last_out, hist_out_buf, True)


def _scan_fwd(inp, w, r, i, h0, hist_in, conv, want_hist, out, h_last_out, hist_out_buf, noalloc):
    dev = inp.device
    _need(inp, "in", dev)
    B, T, D = inp.shape
    mode_c = r is not None or i is not None
    if mode_c and (r is None or i is None):
        raise ValueError("r and i go together")
    use_conv = conv and not mode_c
    _need(r, "r", dev, inp.dtype, (B, T, D))
    _need(i, "i", dev, inp.dtype, (B, T, D))
    _need(h0, "h0", dev, torch.float32, (B, D))
    _need(hist_in, "hist_in", dev, inp.dtype, (B, 3, D))
    H = 1 if mode_c else w.H
    ws_ = _weights_struct(w, D, inp.dtype, dev, conv=use_conv, gates=not mode_c)
    y = torch.empty_like(inp) if out is None else out
    h_last = torch.empty((B, D), dtype=torch.float32, device=dev) if h_last_out is None else h_last_out
    hist_out = None
    if use_conv and want_hist:
        hist_out = hist_out_buf if hist_out_buf is not None else torch.empty((B, 3, D), dtype=inp.dtype, device=dev)
    _need(y, "out", dev, inp.dtype, (B, T, D))
    _need(h_last, "h_last_out", dev, torch.float32, (B, D))
    _need(hist_out, "hist_out_buf", dev, inp.dtype, (B, 3, D))
    d = _Desc(B, T, D, H, _io(inp), w.c)
    args = (ctypes.byref(d), ctypes.byref(ws_), _ptr(inp), _ptr(r), _ptr(i),
            _ptr(hist_in) if use_conv else None, _ptr(h0), _ptr(y), _ptr(h_last), _ptr(hist_out))
    if noalloc:
        _check(lib().rglru_scan_fwd_noalloc(*args, _stream(dev)), "rglru_scan_fwd_noalloc")
        return y, h_last, hist_out
    nbytes = workspace_size(B, T, D, H, _io(inp), OP_SCAN_FWD, w.c)
    wsb = workspace(nbytes, dev)
    _check(lib().rglru_scan_fwd(*args, _ptr(wsb), wsb.numel(), _stream(dev)), "rglru_scan_fwd")
    return y, h_last, hist_out


def step(u_t: torch.Tensor, w: Weights, h: torch.Tensor, hist_in=None, hist_out=None, y_out=None):
    """One decode step.  h [B][D] (fp32) is updated in place; the conv history
    goes from hist_in [B][3][D] (None: zeros) to hist_out (allocated if None;
    must not overlap hist_in -- alternate two buffers).  Returns (y_t, hist_out)."""
    dev = u_t.device
    _need(u_t, "u_t", dev)
    B, D = u_t.shape
    _need(hist_in, "hist_in", dev, u_t.dtype, (B, 3, D))
    _need(h, "h", dev, torch.float32, (B, D))
    ws_ = _weights_struct(w, D, u_t.dtype, dev, conv=True, gates=True)
    y_t = torch.empty_like(u_t) if y_out is None else y_out
    if hist_out is None:
        hist_out = torch.empty((B, 3, D), dtype=u_t.dtype, device=dev)
    _need(hist_out, "hist_out", dev, u_t.dtype, (B, 3, D))
    d = _Desc(B, 1, D, w.H, _io(u_t), w.c)
    _check(lib().rglru_step(ctypes.byref(d), ctypes.byref(ws_), _ptr(u_t), _ptr(hist_in), _ptr(hist_out),
                            _ptr(h), _ptr(y_t), _stream(dev)), "rglru_step")
    return y_t, hist_out


def scan_bwd(u: torch.Tensor, w: Weights, dy: torch.Tensor, *, h0=None, hist_in=None,
             dh_last=None, want_dh0: bool = True):
    """Gradients of <dy, y> + <dh_last, h_last> for the mode-A forward.

    Returns a dict: du, dconv_w, dconv_b, dW_a, db_a, dW_x, db_x, dLambda, dh0."""
    dev = u.device
    _need(u, "u", dev)
    B, T, D = u.shape
    _need(dy, "dy", dev, u.dtype, (B, T, D))
    _need(h0, "h0", dev, torch.float32, (B, D))
    _need(hist_in, "hist_in", dev, u.dtype, (B, 3, D))
    _need(dh_last, "dh_last", dev, torch.float32, (B, D))
    ws_ = _weights_struct(w, D, u.dtype, dev, conv=True, gates=True)
    H, K = w.H, D // w.H
    f = dict(dtype=torch.float32, device=dev)
    g = dict(du=torch.empty_like(u), dconv_w=torch.empty((D, 4), **f), dconv_b=torch.empty(D, **f),
             dW_a=torch.empty((H, K, K), **f), db_a=torch.empty(D, **f),
             dW_x=torch.empty((H, K, K), **f), db_x=torch.empty(D, **f),
             dLambda=torch.empty(D, **f),
             dh0=torch.empty((B, D), **f) if want_dh0 else None)
    d = _Desc(B, T, D, H, _io(u), w.c)
    nbytes = workspace_size(B, T, D, H, _io(u), OP_SCAN_BWD, w.c)
    wsb = workspace(nbytes, dev, "bwd", (B, T, D, H, _io(u)))
    _check(lib().rglru_scan_bwd(ctypes.byref(d), ctypes.byref(ws_), _ptr(u), _ptr(hist_in), _ptr(h0),
                                _ptr(dy), _ptr(dh_last), _ptr(g["du"]), _ptr(g["dconv_w"]),
                                _ptr(g["dconv_b"]), _ptr(g["dW_a"]), _ptr(g["db_a"]), _ptr(g["dW_x"]),
                                _ptr(g["db_x"]), _ptr(g["dLambda"]), _ptr(g["dh0"]), _ptr(wsb),
                                wsb.numel(), _stream(dev)), "rglru_scan_bwd")
    return g


@dataclasses.dataclass
class BlockWeights:
    """Device tensors of the recurrent block's projections (activation dtype):
    proj_in_1, proj_in_2 [D][d_model], proj_out [d_model][D]."""
    proj_in_1: torch.Tensor
    proj_in_2: torch.Tensor
    proj_out: torch.Tensor

    @property
    def d_model(self) -> int:
        return int(self.proj_in_1.shape[1])


def block_fwd(x: torch.Tensor, w: Weights, bw: BlockWeights, *, h0=None, hist_in=None,
              want_hist: bool = True, out=None, h_last_out=None, hist_out_buf=None):
    """Recurrent block forward: out = proj_out(RG-LRU(conv(proj_in_1 x)) * GeLU(proj_in_2 x)).

    x [B][T][d_model].  Returns (out, h_last, hist_out or None); the state and
    the conv history are those of branch 1 (width D)."""
    dev = x.device
    _need(x, "x", dev)
    B, T, d_model = x.shape
    D = int(bw.proj_in_1.shape[0])
    _need(bw.proj_in_1, "proj_in_1", dev, x.dtype, (D, d_model))
    _need(bw.proj_in_2, "proj_in_2", dev, x.dtype, (D, d_model))
    _need(bw.proj_out, "proj_out", dev, x.dtype, (d_model, D))
    _need(h0, "h0", dev, torch.float32, (B, D))
    _need(hist_in, "hist_in", dev, x.dtype, (B, 3, D))
    ws_ = _weights_struct(w, D, x.dtype, dev, conv=True, gates=True)
    o = torch.empty_like(x) if out is None else out
    h_last = torch.empty((B, D), dtype=torch.float32, device=dev) if h_last_out is None else h_last_out
    hist_out = None
    if want_hist:
        hist_out = hist_out_buf if hist_out_buf is not None else torch.empty((B, 3, D), dtype=x.dtype, device=dev)
    _need(o, "out", dev, x.dtype, (B, T, d_model))
    _need(h_last, "h_last_out", dev, torch.float32, (B, D))
    _need(hist_out, "hist_out_buf", dev, x.dtype, (B, 3, D))
    d = _Desc(B, T, D, w.H, _io(x), w.c)
    nbytes = block_workspace_size(B, T, D, w.H, d_model, _io(x), w.c)
    wsb = workspace(nbytes, dev, "block", (B, T, D, w.H, d_model, _io(x)))
    blk = _Block(_ptr(bw.proj_in_1), _ptr(bw.proj_in_2), _ptr(bw.proj_out))
    _check(lib().rglru_block_fwd(ctypes.byref(d), d_model, ctypes.byref(ws_), ctypes.byref(blk), _ptr(x),
                                 _ptr(hist_in), _ptr(h0), _ptr(o), _ptr(h_last), _ptr(hist_out), _ptr(wsb),
                                 wsb.numel(), _stream(dev)), "rglru_block_fwd")
    return o, h_last, hist_out


# ------------------------------------------------------------ local attention
def attn_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, window: int, scale: Optional[float] = None,
             *, kcache=None, vcache=None, out=None):
    """Sliding-window MQA prefill: q [B][T][Hq][dh], k, v [B][T][dh]; token t
    attends to t-window+1 .. t.  scale defaults to 1/sqrt(dh).  kcache /
    vcache [B][W][dh] (optional, both or neither) receive the last W positions
    in ring order.  Returns o [B][T][Hq][dh]."""
    dev = q.device
    _need(q, "q", dev)
    B, T, Hq, dh = q.shape
    _need(k, "k", dev, q.dtype, (B, T, dh))
    _need(v, "v", dev, q.dtype, (B, T, dh))
    if (kcache is None) != (vcache is None):
        raise ValueError("kcache and vcache go together")
    _need(kcache, "kcache", dev, q.dtype, (B, window, dh))
    _need(vcache, "vcache", dev, q.dtype, (B, window, dh))
    o = torch.empty_like(q) if out is None else out
    _need(o, "out", dev, q.dtype, (B, T, Hq, dh))
    sc = dh ** -0.5 if scale is None else float(scale)
    d = _AttnDesc(B, T, Hq, dh, window, _io(q), sc)
    _check(lib().rglru_attn_fwd(ctypes.byref(d), _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(kcache),
                                _ptr(vcache), _stream(dev)), "rglru_attn_fwd")
    return o


def attn_workspace_size(B, Hq, dh, W, io=BF16, scale=1.0) -> int:
    n = ctypes.c_size_t(0)
    _check(lib().rglru_attn_workspace_size(ctypes.byref(_AttnDesc(B, 1, Hq, dh, W, io, scale)),
                                           ctypes.byref(n)), "rglru_attn_workspace_size")
    return int(n.value)


def attn_step(q_t: torch.Tensor, k_t: torch.Tensor, v_t: torch.Tensor, kcache: torch.Tensor,
              vcache: torch.Tensor, pos: torch.Tensor, scale: Optional[float] = None, out=None):
    """One decode step: q_t [B][Hq][dh], k_t, v_t [B][dh], ring caches
    [B][W][dh] (updated in place), pos [B] int32 (device; the new token's
    position, not advanced here).  Returns o_t [B][Hq][dh]."""
    dev = q_t.device
    _need(q_t, "q_t", dev)
    B, Hq, dh = q_t.shape
    W = int(kcache.shape[1])
    _need(k_t, "k_t", dev, q_t.dtype, (B, dh))
    _need(v_t, "v_t", dev, q_t.dtype, (B, dh))
    _need(kcache, "kcache", dev, q_t.dtype, (B, W, dh))
    _need(vcache, "vcache", dev, q_t.dtype, (B, W, dh))
    _need(pos, "pos", dev, torch.int32, (B,))
    o = torch.empty_like(q_t) if out is None else out
    _need(o, "out", dev, q_t.dtype, (B, Hq, dh))
    sc = dh ** -0.5 if scale is None else float(scale)
    d = _AttnDesc(B, 1, Hq, dh, W, _io(q_t), sc)
    n = attn_workspace_size(B, Hq, dh, W, _io(q_t), sc)
    wsb = workspace(n, dev, "attn")
    _check(lib().rglru_attn_step(ctypes.byref(d), _ptr(q_t), _ptr(k_t), _ptr(v_t), _ptr(kcache), _ptr(vcache),
                                 _ptr(pos), _ptr(o), _ptr(wsb), wsb.numel(), _stream(dev)), "rglru_attn_step")
    return o


# ------------------------------------------------------------ residual layer
@dataclasses.dataclass
class LayerWeights:
    """Device tensors of the residual layer around the block: the two pre-norm
    weights [d_model] fp32 (applied as 1 + w) and the gated MLP's gate_w,
    up_w [d_ff][d_model], down_w [d_model][d_ff] (activation dtype)."""
    tnorm_w: torch.Tensor
    cnorm_w: torch.Tensor
    gate_w: torch.Tensor
    up_w: torch.Tensor
    down_w: torch.Tensor
    eps: float = 1e-6

    @property
    def d_ff(self) -> int:
        return int(self.gate_w.shape[0])


def _layer_struct(lw: LayerWeights, d_model, dtype, dev):
    F = lw.d_ff
    _need(lw.tnorm_w, "tnorm_w", dev, torch.float32, (d_model,))
    _need(lw.cnorm_w, "cnorm_w", dev, torch.float32, (d_model,))
    _need(lw.gate_w, "gate_w", dev, dtype, (F, d_model))
    _need(lw.up_w, "up_w", dev, dtype, (F, d_model))
    _need(lw.down_w, "down_w", dev, dtype, (d_model, F))
    return _Layer(_ptr(lw.tnorm_w), _ptr(lw.cnorm_w), _ptr(lw.gate_w), _ptr(lw.up_w), _ptr(lw.down_w), F, lw.eps)


def layer_workspace_size(B, T, D, H, d_model, lw: LayerWeights, io=BF16, c=8.0) -> int:
    n = ctypes.c_size_t(0)
    st = _Layer(None, None, None, None, None, lw.d_ff, lw.eps)
    _check(lib().rglru_layer_workspace_size(ctypes.byref(_Desc(B, T, D, H, io, c)), d_model, ctypes.byref(st),
                                            ctypes.byref(n)), "rglru_layer_workspace_size")
    return int(n.value)


def layer_fwd(x: torch.Tensor, w: Weights, bw: BlockWeights, lw: LayerWeights, *, h0=None, hist_in=None,
              want_hist: bool = True, out=None, h_last_out=None, hist_out_buf=None):
    """Residual layer: x~ = x + block(RMSNorm(x)), y = x~ + MLP(RMSNorm(x~)).
    Returns (y, h_last, hist_out or None)."""
    dev = x.device
    _need(x, "x", dev)
    B, T, d_model = x.shape
    D = int(bw.proj_in_1.shape[0])
    _need(bw.proj_in_1, "proj_in_1", dev, x.dtype, (D, d_model))
    _need(bw.proj_in_2, "proj_in_2", dev, x.dtype, (D, d_model))
    _need(bw.proj_out, "proj_out", dev, x.dtype, (d_model, D))
    _need(h0, "h0", dev, torch.float32, (B, D))
    _need(hist_in, "hist_in", dev, x.dtype, (B, 3, D))
    ws_ = _weights_struct(w, D, x.dtype, dev, conv=True, gates=True)
    ls = _layer_struct(lw, d_model, x.dtype, dev)
    y = torch.empty_like(x) if out is None else out
    h_last = torch.empty((B, D), dtype=torch.float32, device=dev) if h_last_out is None else h_last_out
    hist_out = None
    if want_hist:
        hist_out = hist_out_buf if hist_out_buf is not None else torch.empty((B, 3, D), dtype=x.dtype, device=dev)
    _need(y, "out", dev, x.dtype, (B, T, d_model))
    _need(h_last, "h_last_out", dev, torch.float32, (B, D))
    _need(hist_out, "hist_out_buf", dev, x.dtype, (B, 3, D))
    d = _Desc(B, T, D, w.H, _io(x), w.c)
    nbytes = layer_workspace_size(B, T, D, w.H, d_model, lw, _io(x), w.c)
    wsb = workspace(nbytes, dev, "layer", (B, T, D, w.H, d_model, lw.d_ff, _io(x)))
    blk = _Block(_ptr(bw.proj_in_1), _ptr(bw.proj_in_2), _ptr(bw.proj_out))
    _check(lib().rglru_layer_fwd(ctypes.byref(d), d_model, ctypes.byref(ws_), ctypes.byref(blk), ctypes.byref(ls),
                                 _ptr(x), _ptr(hist_in), _ptr(h0), _ptr(y), _ptr(h_last), _ptr(hist_out),
                                 _ptr(wsb), wsb.numel(), _stream(dev)), "rglru_layer_fwd")
    return y, h_last, hist_out


def hawk_stack_fwd(x: torch.Tensor, layers, *, states=None):
    """A Hawk stack: residual layers (each a (Weights, BlockWeights,
    LayerWeights) triple) applied in order, each one rglru_layer_fwd call.
    states: optional per-layer (h0, hist_in) pairs carried in (decode-style
    continuation); returns (y, [(h_last, hist_out) per layer])."""
    out_states = []
    y = x
    for idx, (w, bw, lw) in enumerate(layers):
        h0, hist = (None, None) if states is None else states[idx]
        y, h_last, hist_out = layer_fwd(y, w, bw, lw, h0=h0, hist_in=hist)
        out_states.append((h_last, hist_out))
    return y, out_states


# ------------------------------------------------------------ attention layer
@dataclasses.dataclass
class AttnProjWeights:
    """Attention layer projections (activation dtype, [out][in]): wq
    [Hq*dh][d_model], wk, wv [dh][d_model], wo [d_model][Hq*dh]."""
    wq: torch.Tensor
    wk: torch.Tensor
    wv: torch.Tensor
    wo: torch.Tensor


def attn_layer_fwd(x: torch.Tensor, ap: AttnProjWeights, lw: LayerWeights, Hq: int, window: int, *,
                   scale: Optional[float] = None, rot: Optional[int] = None, rope_base: float = 10000.0,
                   pos0: int = 0, kcache=None, vcache=None, out=None):
    """Attention residual layer: x~ = x + attn(RoPE(q), RoPE(k), v) wo^T,
    y = x~ + MLP(RMSNorm(x~)), with q, k, v projections of RMSNorm(x).
    rot defaults to dh (full rotary); positions are pos0 + t.  Returns y."""
    dev = x.device
    _need(x, "x", dev)
    B, T, d_model = x.shape
    dh = int(ap.wk.shape[0])
    _need(ap.wq, "wq", dev, x.dtype, (Hq * dh, d_model))
    _need(ap.wk, "wk", dev, x.dtype, (dh, d_model))
    _need(ap.wv, "wv", dev, x.dtype, (dh, d_model))
    _need(ap.wo, "wo", dev, x.dtype, (d_model, Hq * dh))
    if (kcache is None) != (vcache is None):
        raise ValueError("kcache and vcache go together")
    _need(kcache, "kcache", dev, x.dtype, (B, window, dh))
    _need(vcache, "vcache", dev, x.dtype, (B, window, dh))
    ls = _layer_struct(lw, d_model, x.dtype, dev)
    y = torch.empty_like(x) if out is None else out
    _need(y, "out", dev, x.dtype, (B, T, d_model))
    sc = dh ** -0.5 if scale is None else float(scale)
    d = _AttnDesc(B, T, Hq, dh, window, _io(x), sc)
    n = ctypes.c_size_t(0)
    _check(lib().rglru_attn_layer_workspace_size(ctypes.byref(d), d_model, ctypes.byref(ls), ctypes.byref(n)),
           "rglru_attn_layer_workspace_size")
    wsb = workspace(int(n.value), dev, "attn_layer")
    pr = _AttnProj(_ptr(ap.wq), _ptr(ap.wk), _ptr(ap.wv), _ptr(ap.wo))
    _check(lib().rglru_attn_layer_fwd(ctypes.byref(d), d_model, dh if rot is None else int(rot), rope_base, pos0,
                                      ctypes.byref(pr), ctypes.byref(ls), _ptr(x), _ptr(y), _ptr(kcache),
                                      _ptr(vcache), _ptr(wsb), wsb.numel(), _stream(dev)), "rglru_attn_layer_fwd")
    return y
