"""ctypes front end of the double-precision CPU oracle (oracle.c).

TEST INFRASTRUCTURE.  Only tests/, the smoke check and the bench's CPU
baseline import this package.  The GPU library never loads it and it never
loads the GPU library.

All array arguments are numpy float64, C-contiguous, in the layouts below
(row-major, channel fastest):
  u, x, r, i, y, dy, du : [B][T][D]
  hist                  : [B][3][D]   (pre-conv inputs t-3, t-2, t-1)
  h0, h_last, dh_last   : [B][D]
  conv_w                : [D][4]      (tap k multiplies u[t-3+k])
  W_a, W_x              : [H][K][K]   (W[h][o][j]: input hK+j -> output hK+o)
  b_a, b_x, conv_b, Lambda : [D]
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liboracle.so")
SRC_PATH = os.path.join(_HERE, "oracle.c")

_lib = None


def build() -> str:
    """Compile oracle.c with gcc (IEEE double, no fast-math, no FMA contraction)."""
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp",
           "-fno-fast-math", "-ffp-contract=off", SRC_PATH, "-o", LIB_PATH + ".tmp", "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(LIB_PATH + ".tmp", LIB_PATH)
    return LIB_PATH


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH) or os.path.getmtime(LIB_PATH) < os.path.getmtime(SRC_PATH):
            build()
        _lib = ctypes.CDLL(LIB_PATH)
        _lib.oracle_num_threads.restype = ctypes.c_int
    return _lib


def _p(a):
    if a is None:
        return None
    assert a.dtype == np.float64 and a.flags["C_CONTIGUOUS"], "oracle wants contiguous float64"
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def _f64(a):
    return None if a is None else np.ascontiguousarray(a, dtype=np.float64)


def num_threads() -> int:
    return int(lib().oracle_num_threads())


def set_threads(n: int) -> None:
    lib().oracle_set_threads(ctypes.c_int(n))


def conv1d(u, conv_w, conv_b=None, hist_in=None):
    u, conv_w, conv_b, hist_in = map(_f64, (u, conv_w, conv_b, hist_in))
    B, T, D = u.shape
    x = np.empty_like(u)
    hist_out = np.empty((B, 3, D))
    lib().oracle_conv1d(B, T, D, _p(u), _p(conv_w), _p(conv_b), _p(hist_in), _p(x), _p(hist_out))
    return x, hist_out


def gates(x, W_a, b_a, W_x, b_x):
    x, W_a, b_a, W_x, b_x = map(_f64, (x, W_a, b_a, W_x, b_x))
    B, T, D = x.shape
    H = W_a.shape[0]
    r = np.empty_like(x)
    i = np.empty_like(x)
    lib().oracle_gates(B, T, D, H, _p(x), _p(W_a), _p(b_a), _p(W_x), _p(b_x), _p(r), _p(i))
    return r, i


def decay(r, Lambda, c=8.0):
    r, Lambda = _f64(r), _f64(Lambda)
    D = r.shape[-1]
    N = r.size // D
    a = np.empty_like(r)
    beta = np.empty_like(r)
    lib().oracle_decay(ctypes.c_long(N), D, ctypes.c_double(c), _p(r), _p(Lambda), _p(a), _p(beta))
    return a, beta


def scan(x, r, i, Lambda, h0=None, c=8.0):
    x, r, i, Lambda, h0 = map(_f64, (x, r, i, Lambda, h0))
    B, T, D = x.shape
    y = np.empty_like(x)
    h_last = np.empty((B, D))
    lib().oracle_scan(B, T, D, ctypes.c_double(c), _p(x), _p(r), _p(i), _p(Lambda), _p(h0),
                      _p(y), _p(h_last))
    return y, h_last


def fwd(u, conv_w, conv_b, W_a, b_a, W_x, b_x, Lambda, h0=None, hist_in=None, c=8.0):
    """Whole forward u -> (y, h_last, hist_out).  conv_w None means no conv (x = u)."""
    u, conv_w, conv_b, W_a, b_a, W_x, b_x, Lambda, h0, hist_in = map(
        _f64, (u, conv_w, conv_b, W_a, b_a, W_x, b_x, Lambda, h0, hist_in))
    B, T, D = u.shape
    H = W_a.shape[0]
    y = np.empty_like(u)
    h_last = np.empty((B, D))
    hist_out = np.empty((B, 3, D))
    lib().oracle_fwd(B, T, D, H, ctypes.c_double(c), _p(u), _p(conv_w), _p(conv_b), _p(hist_in),
                     _p(W_a), _p(b_a), _p(W_x), _p(b_x), _p(Lambda), _p(h0),
                     _p(y), _p(h_last), _p(hist_out))
    if conv_w is None:
        hist_out = None
    return y, h_last, hist_out


def step(u_t, conv_w, conv_b, W_a, b_a, W_x, b_x, Lambda, hist, h, c=8.0):
    """One decode step.  Returns (y_t, hist_new, h_new); inputs are not modified."""
    u_t, conv_w, conv_b, W_a, b_a, W_x, b_x, Lambda = map(
        _f64, (u_t, conv_w, conv_b, W_a, b_a, W_x, b_x, Lambda))
    hist = np.array(hist, dtype=np.float64, order="C", copy=True)
    h = np.array(h, dtype=np.float64, order="C", copy=True)
    B, D = u_t.shape
    H = W_a.shape[0]
    y_t = np.empty((B, D))
    lib().oracle_step(B, D, H, ctypes.c_double(c), _p(u_t), _p(conv_w), _p(conv_b), _p(W_a),
                      _p(b_a), _p(W_x), _p(b_x), _p(Lambda), _p(hist), _p(h), _p(y_t))
    return y_t, hist, h


def bwd(u, conv_w, conv_b, W_a, b_a, W_x, b_x, Lambda, dy, h0=None, hist_in=None,
        dh_last=None, c=8.0):
    """Gradients of L = <dy, y> + <dh_last, h_last> w.r.t. every input.

    Returns a dict: du, dconv_w, dconv_b, dW_a, db_a, dW_x, db_x, dLambda, dh0."""
    u, conv_w, conv_b, W_a, b_a, W_x, b_x, Lambda, dy, h0, hist_in, dh_last = map(
        _f64, (u, conv_w, conv_b, W_a, b_a, W_x, b_x, Lambda, dy, h0, hist_in, dh_last))
    B, T, D = u.shape
    H, K, _ = W_a.shape
    g = dict(du=np.empty_like(u), dconv_w=np.empty((D, 4)), dconv_b=np.empty(D),
             dW_a=np.empty((H, K, K)), db_a=np.empty(D), dW_x=np.empty((H, K, K)),
             db_x=np.empty(D), dLambda=np.empty(D), dh0=np.empty((B, D)))
    lib().oracle_bwd(B, T, D, H, ctypes.c_double(c), _p(u), _p(conv_w), _p(conv_b), _p(hist_in),
                     _p(W_a), _p(b_a), _p(W_x), _p(b_x), _p(Lambda), _p(h0), _p(dy), _p(dh_last),
                     _p(g["du"]), _p(g["dconv_w"]), _p(g["dconv_b"]), _p(g["dW_a"]), _p(g["db_a"]),
                     _p(g["dW_x"]), _p(g["db_x"]), _p(g["dLambda"]), _p(g["dh0"]))
    return g


def linear(x, W):
    """A linear layer without bias: y[..., n] = sum_k x[..., k] W[n][k] (W [N][K])."""
    x, W = _f64(x), _f64(W)
    K = x.shape[-1]
    N = W.shape[0]
    M = x.size // K
    y = np.empty(x.shape[:-1] + (N,))
    lib().oracle_linear(ctypes.c_long(M), K, N, _p(x), _p(W), _p(y))
    return y


def gelu(v):
    """GeLU(v) = 0.5 v (1 + erf(v / sqrt 2)) (the exact form, reading R6)."""
    v = _f64(v)
    out = np.empty_like(v)
    lib().oracle_gelu(ctypes.c_long(v.size), _p(v), _p(out))
    return out


def merge(y, g):
    """z = y * GeLU(g), elementwise."""
    y, g = _f64(y), _f64(g)
    z = np.empty_like(y)
    lib().oracle_merge(ctypes.c_long(y.size), _p(y), _p(g), _p(z))
    return z


def block_fwd(x, proj_in_1, proj_in_2, proj_out, conv_w, conv_b, W_a, b_a, W_x, b_x, Lambda,
              h0=None, hist_in=None, c=8.0):
    """Recurrent block (reading R6): out = proj_out(y * GeLU(proj_in_2 x)) with y the
    RG-LRU of conv(proj_in_1 x).  x [B][T][d_model]; proj_in_* [D][d_model];
    proj_out [d_model][D].  Returns (out, h_last, hist_out) -- the state and the
    conv history are those of branch 1."""
    b1 = linear(x, proj_in_1)
    b2 = linear(x, proj_in_2)
    y, h_last, hist_out = fwd(b1, conv_w, conv_b, W_a, b_a, W_x, b_x, Lambda, h0=h0, hist_in=hist_in, c=c)
    return linear(merge(y, b2), proj_out), h_last, hist_out


def rel_err(got, ref) -> float:
    """max_i |g_i - o_i| / max(|o_i|, RMS(o)): elementwise relative error with
    an RMS floor, so that outputs crossing zero are judged against the
    tensor's scale rather than against a vanishing denominator."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    rms = float(np.sqrt(np.mean(ref * ref))) if ref.size else 0.0
    den = np.maximum(np.abs(ref), rms)
    den = np.where(den == 0.0, 1.0, den)
    return float(np.max(np.abs(got - ref) / den)) if ref.size else 0.0


# ------------------------------------------------------------ local attention
def attn_fwd(q, k, v, window: int, scale: float):
    """Sliding-window MQA (reading R7): q [B][T][Hq][dh], k, v [B][T][dh].
    Token t attends to positions t-window+1 .. t.  Returns o [B][T][Hq][dh]."""
    q, k, v = map(_f64, (q, k, v))
    B, T, Hq, dh = q.shape
    assert k.shape == (B, T, dh) and v.shape == (B, T, dh)
    o = np.empty_like(q)
    lib().oracle_attn_fwd(B, T, Hq, dh, int(window), ctypes.c_double(scale), _p(q), _p(k), _p(v), _p(o))
    return o


def attn_step(q_t, k_t, v_t, kcache, vcache, pos, scale: float):
    """One decode step with ring caches kcache, vcache [B][W][dh] (updated in
    place: the new key/value go to slot pos mod W).  q_t [B][Hq][dh], k_t, v_t
    [B][dh], pos [B] (int, the new token's position).  Returns o_t."""
    q_t, k_t, v_t = map(_f64, (q_t, k_t, v_t))
    assert kcache.dtype == np.float64 and kcache.flags["C_CONTIGUOUS"]
    assert vcache.dtype == np.float64 and vcache.flags["C_CONTIGUOUS"]
    B, Hq, dh = q_t.shape
    W = kcache.shape[1]
    pos = np.ascontiguousarray(pos, dtype=np.int64)
    o = np.empty_like(q_t)
    lib().oracle_attn_step(B, Hq, dh, W, ctypes.c_double(scale), _p(q_t), _p(k_t), _p(v_t),
                           _p(kcache), _p(vcache), pos.ctypes.data_as(ctypes.POINTER(ctypes.c_long)),
                           _p(o))
    return o


# ------------------------------------------------------------ residual layer
def rmsnorm(x, w, eps=1e-6):
    """Reading R8: x / sqrt(mean over the last axis of x^2 + eps) * (1 + w)."""
    x, w = map(_f64, (x, w))
    D = x.shape[-1]
    out = np.empty_like(x)
    lib().oracle_rmsnorm(ctypes.c_long(x.size // D), D, _p(x), _p(w), ctypes.c_double(eps), _p(out))
    return out


def gelu_tanh(v):
    """GELU, tanh form (reading R8)."""
    v = _f64(v)
    out = np.empty_like(v)
    lib().oracle_gelu_tanh(ctypes.c_long(v.size), _p(v), _p(out))
    return out


def mlp(x, gate_w, up_w, down_w):
    """Gated MLP (reading R8): down(GELU_tanh(gate x) * (up x)); weights [out][in]."""
    return linear(gelu_tanh(linear(x, gate_w)) * linear(x, up_w), down_w)


def hawk_layer(x, tnorm_w, cnorm_w, proj_in_1, proj_in_2, proj_out, conv_w, conv_b, W_a, b_a, W_x, b_x,
               Lambda, gate_w, up_w, down_w, h0=None, hist_in=None, c=8.0, eps=1e-6):
    """Residual layer with the recurrent block as temporal mixer ([L] "Residual
    Block View"): x~ = x + block(RMSNorm(x)), y = x~ + MLP(RMSNorm(x~)).
    Returns (y, h_last, hist_out)."""
    t, h_last, hist_out = block_fwd(rmsnorm(x, tnorm_w, eps), proj_in_1, proj_in_2, proj_out, conv_w, conv_b,
                                    W_a, b_a, W_x, b_x, Lambda, h0=h0, hist_in=hist_in, c=c)
    xt = _f64(x) + t
    return xt + mlp(rmsnorm(xt, cnorm_w, eps), gate_w, up_w, down_w), h_last, hist_out


# ------------------------------------------------------------ attention layer
def rope(x, positions, rot, base=10000.0):
    """Rotary embedding (reading R9): x [..][H][dh] with positions [..] (one per
    row); pairs (j, j + rot/2), j < rot/2, turn by pos * base^(-2j/rot)."""
    x = np.array(x, dtype=np.float64, order="C", copy=True)
    H, dh = x.shape[-2], x.shape[-1]
    pos = np.ascontiguousarray(np.broadcast_to(positions, x.shape[:-2]).reshape(-1), dtype=np.int64)
    lib().oracle_rope(ctypes.c_long(pos.size), H, dh, int(rot), ctypes.c_double(base),
                      pos.ctypes.data_as(ctypes.POINTER(ctypes.c_long)), _p(x))
    return x


def attn_layer(x, tnorm_w, cnorm_w, wq, wk, wv, wo, gate_w, up_w, down_w, Hq, window, scale, rot,
               base=10000.0, pos0=0, eps=1e-6):
    """Residual layer with local MQA as temporal mixer (readings R8, R9):
    x~ = x + o_proj(attn(RoPE(q), RoPE(k), v)), y = x~ + MLP(RMSNorm(x~)).
    wq [Hq*dh][d_model], wk, wv [dh][d_model], wo [d_model][Hq*dh]; token t has
    position pos0 + t.  Returns y."""
    x = _f64(x)
    B, T, dm = x.shape
    dh = wk.shape[0]
    xn = rmsnorm(x, tnorm_w, eps)
    pos = pos0 + np.arange(T)[None, :].repeat(B, axis=0)
    q = rope(linear(xn, wq).reshape(B, T, Hq, dh), pos, rot, base)
    k = rope(linear(xn, wk).reshape(B, T, 1, dh), pos, rot, base).reshape(B, T, dh)
    v = linear(xn, wv)
    o = attn_fwd(q, k, v, window, scale).reshape(B, T, Hq * dh)
    xt = x + linear(o, wo)
    return xt + mlp(rmsnorm(xt, cnorm_w, eps), gate_w, up_w, down_w)
