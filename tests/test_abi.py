"""Host-only checks of the C ABI: the library loads, exports every function that
include/rglru.h declares, and rejects bad arguments with the documented status
codes before anything reaches a GPU (validation runs on the host first, so
none of these calls launches work)."""
import ctypes
import os
import re

import pytest

import gated_linear_recurrence_02_amd as glr

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "rglru.h")

OK, ENULL, ESHAPE, EDTYPE, EALIGN, EWS, ELAUNCH, EARG, EBLAS, ETIMEOUT = 0, -1, -2, -3, -4, -5, -6, -7, -8, -9
ESCRATCH = -10
P = 0x7F0000000000          # a 16-byte aligned fake device address (never dereferenced)


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(rglru_\w+)\s*\(", src)))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(glr.LIB_PATH):
        import gated_linear_recurrence_02_amd.build as b
        b.build()
    return glr.lib()


def test_library_exports_every_declared_function(L):
    names = declared_functions()
    assert names == sorted(glr.SYMBOLS)
    for n in names:
        assert hasattr(L, n), n


def desc(B=2, T=64, D=512, H=2, io=glr.BF16, c=8.0):
    return glr._Desc(B, T, D, H, io, c)


def weights(conv=True):
    return glr._Weights(P if conv else None, None, P + 0x10000, None, P + 0x20000, None, P + 0x30000)


def ws_size(d, op=glr.OP_SCAN_FWD):
    n = ctypes.c_size_t()
    rc = glr.lib().rglru_workspace_size(ctypes.byref(d), op, ctypes.byref(n))
    return rc, n.value


def test_status_strings(L):
    for rc in (OK, ENULL, ESHAPE, EDTYPE, EALIGN, EWS, ELAUNCH, EARG, EBLAS, ETIMEOUT, ESCRATCH):
        assert L.rglru_status_string(rc) != b"unknown status"
    assert L.rglru_status_string(123) == b"unknown status"


def test_workspace_status_validation(L):
    # argument checks come before any device call
    assert L.rglru_workspace_status(None, 4096, None) == ENULL
    assert L.rglru_workspace_status(ctypes.c_void_p(0x1008), 4096, None) == EALIGN
    assert L.rglru_workspace_status(ctypes.c_void_p(0x1000), 255, None) == EWS


def test_workspace_size(L):
    rc, n = ws_size(desc())
    assert rc == OK and n >= 256 + 3 * 2 * 2 * 512 * 8
    assert ws_size(desc(T=65))[1] > n                      # one more chunk
    assert ws_size(desc(io=7))[0] == EDTYPE
    assert ws_size(desc(D=500, H=3))[0] == ESHAPE
    assert ws_size(desc(T=0))[0] == ESHAPE
    assert ws_size(desc(), op=9)[0] == EARG
    assert ws_size(desc(D=768, H=2), op=glr.OP_SCAN_BWD)[0] == ESHAPE   # K = 384
    # the chunked scans keep one claim counter per 256-channel group in a
    # region of fixed size: at most 4096 groups (D <= 2^20), for both ops
    for op in (glr.OP_SCAN_FWD, glr.OP_SCAN_BWD):
        assert ws_size(desc(B=1, T=1, D=(1 << 20) + 256, H=(1 << 12) + 1), op=op)[0] == ESHAPE
        assert ws_size(desc(B=1, T=1, D=1 << 20, H=1 << 12), op=op)[0] == OK
    # the forward's workspace: a fixed prefix (header + claim region) then
    # 3 tagged words per (stream, chunk, channel)
    n1, n2 = ws_size(desc(B=1, T=32, D=256, H=1))[1], ws_size(desc(B=1, T=32, D=512, H=2))[1]
    assert n2 - n1 == 3 * 256 * 8
    # the backward's workspace depends on the I/O type (fp16 r and fp32 i for bf16)
    assert ws_size(desc(io=glr.BF16), op=glr.OP_SCAN_BWD)[1] < ws_size(desc(io=glr.F32), op=glr.OP_SCAN_BWD)[1]
    assert L.rglru_workspace_size(None, 0, None) == ENULL


def test_conv1d_validation(L):
    d = desc()
    s = None
    assert L.rglru_conv1d(None, P, None, P, None, P, None, s) == ENULL
    assert L.rglru_conv1d(ctypes.byref(d), None, None, P, None, P + 0x100000, None, s) == ENULL
    assert L.rglru_conv1d(ctypes.byref(d), P + 4, None, P + 0x100000, None, P + 0x200000, None, s) == EALIGN
    bad = desc(io=5)
    assert L.rglru_conv1d(ctypes.byref(bad), P, None, P + 0x100000, None, P + 0x200000, None, s) == EDTYPE
    # x overlapping u
    assert L.rglru_conv1d(ctypes.byref(d), P, None, P + 0x100000, None, P + 0x100010, None, s) == EARG


def test_gates_validation(L):
    w = weights()
    s = None
    d = desc(D=300, H=1)                                  # K != 256
    assert L.rglru_gates(ctypes.byref(d), ctypes.byref(w), P + 0x1000000, P + 0x2000000, P + 0x3000000, s) == ESHAPE
    d = desc()
    assert L.rglru_gates(ctypes.byref(d), None, P, P, P, s) == ENULL
    assert L.rglru_gates(ctypes.byref(d), ctypes.byref(w), P + 0x1000000, P + 0x1000000, P + 0x3000000, s) == EARG


def test_scan_fwd_validation(L):
    d = desc()
    rc, n = ws_size(d)
    w = weights()
    wb = weights(conv=False)
    s = None
    u, y, r, i = P + 0x1000000, P + 0x2000000, P + 0x3000000, P + 0x4000000
    ws = P + 0x10000000
    f = L.rglru_scan_fwd
    assert f(ctypes.byref(d), ctypes.byref(w), u, None, None, None, None, y, None, None, None, n, s) == EWS
    assert f(ctypes.byref(d), ctypes.byref(w), u, None, None, None, None, y, None, None, ws, n - 1, s) == EWS
    assert f(ctypes.byref(d), ctypes.byref(w), u, r, None, None, None, y, None, None, ws, n, s) == EARG
    assert f(ctypes.byref(d), ctypes.byref(w), u, r, i, None, None, y, None, None, ws, n, s) == EARG   # conv + r/i
    assert f(ctypes.byref(d), ctypes.byref(wb), u, None, None, P, None, y, None, None, ws, n, s) == EARG  # hist in mode B
    assert f(ctypes.byref(d), ctypes.byref(w), u, None, None, None, None, None, None, None, ws, n, s) == ENULL
    assert f(ctypes.byref(d), ctypes.byref(w), u + 8, None, None, None, None, y, None, None, ws, n, s) == EALIGN
    assert f(ctypes.byref(d), ctypes.byref(w), u, None, None, None, None, u, None, None, ws, n, s) == EARG
    d300 = desc(D=300, H=1)
    _, n3 = ws_size(d300)
    assert f(ctypes.byref(d300), ctypes.byref(w), u, None, None, None, None, y, None, None, ws, n3, s) == ESHAPE


def test_scan_fwd_noalloc_validation(L):
    # the same checks as rglru_scan_fwd, and a size limit in place of the
    # workspace size: 16640 + 24 B ceil(T/32) D bytes must fit the scratch
    d = desc()
    w = weights()
    s = None
    u, y, r = P + 0x1000000, P + 0x2000000, P + 0x3000000
    f = L.rglru_scan_fwd_noalloc
    assert f(ctypes.byref(d), ctypes.byref(w), u, r, None, None, None, y, None, None, s) == EARG
    assert f(ctypes.byref(d), ctypes.byref(w), u, None, None, None, None, None, None, None, s) == ENULL
    assert f(ctypes.byref(d), ctypes.byref(w), u + 8, None, None, None, None, y, None, None, s) == EALIGN
    assert f(ctypes.byref(d), ctypes.byref(w), u, None, None, None, None, u, None, None, s) == EARG
    assert f(None, ctypes.byref(w), u, None, None, None, None, y, None, None, s) == ENULL
    fits = desc(B=1, T=1091 * 32, D=2560, H=10)
    rc, n = ws_size(fits)
    assert rc == OK and n == 16640 + 24 * 1091 * 2560 <= glr.NOALLOC_SCRATCH_BYTES
    over = desc(B=1, T=1092 * 32, D=2560, H=10)
    rc, n = ws_size(over)
    assert rc == OK and n > glr.NOALLOC_SCRATCH_BYTES
    assert f(ctypes.byref(over), ctypes.byref(w), u, None, None, None, None, y, None, None, s) == ESCRATCH
    big = desc(B=4, T=8192, D=4096, H=16)
    assert f(ctypes.byref(big), ctypes.byref(w), u, None, None, None, None, y, None, None, s) == ESCRATCH


def test_step_validation(L):
    d = desc(T=2)
    w = weights()
    s = None
    u, hi, ho, h, y = P + 0x1000000, P + 0x2000000, P + 0x3000000, P + 0x4000000, P + 0x5000000
    assert L.rglru_step(ctypes.byref(d), ctypes.byref(w), u, hi, ho, h, y, s) == ESHAPE
    d = desc(T=1)
    assert L.rglru_step(ctypes.byref(d), ctypes.byref(weights(conv=False)), u, hi, ho, h, y, s) == ENULL
    assert L.rglru_step(ctypes.byref(d), ctypes.byref(w), u, hi, ho, None, y, s) == ENULL
    assert L.rglru_step(ctypes.byref(d), ctypes.byref(w), u, hi + 8, ho, h, y, s) == EALIGN
    # the new history written over the old one, h over the history, y over h
    assert L.rglru_step(ctypes.byref(d), ctypes.byref(w), u, hi, hi, h, y, s) == EARG
    assert L.rglru_step(ctypes.byref(d), ctypes.byref(w), u, hi, ho, ho, y, s) == EARG
    assert L.rglru_step(ctypes.byref(d), ctypes.byref(w), u, hi, ho, h, h, s) == EARG


def test_scan_bwd_validation(L):
    d = desc()
    rc, n = ws_size(d, glr.OP_SCAN_BWD)
    assert rc == OK
    w = weights()
    s = None
    base = [P + k * 0x1000000 for k in range(1, 20)]
    u, dy, du, dcw, dcb, dWa, dba, dWx, dbx, dL = base[:10]
    ws = P + 0x100000000
    f = L.rglru_scan_bwd
    good = (u, None, None, dy, None, du, dcw, dcb, dWa, dba, dWx, dbx, dL, None)
    assert f(ctypes.byref(d), ctypes.byref(w), *good, ws, n - 16, s) == EWS
    bad = list(good)
    bad[5] = None
    assert f(ctypes.byref(d), ctypes.byref(w), *bad, ws, n, s) == ENULL
    bad = list(good)
    bad[5] = u                                               # du == u
    assert f(ctypes.byref(d), ctypes.byref(w), *bad, ws, n, s) == EARG
    many = desc(B=65536, T=1)                                # one stream past the carry scan's grid
    assert f(ctypes.byref(many), ctypes.byref(w), *good, ws, n, s) == ESHAPE


def block_ws_size(d, d_model):
    n = ctypes.c_size_t()
    rc = glr.lib().rglru_block_workspace_size(ctypes.byref(d), d_model, ctypes.byref(n))
    return rc, n.value


def test_block_workspace_size(L):
    d = desc()
    rc, n = block_ws_size(d, 384)
    _, nf = ws_size(d)
    act = d.B * d.T * d.D * 2
    assert rc == OK and n >= nf + 2 * act                 # scan carries + b1 + b2
    assert block_ws_size(desc(io=glr.F32), 384)[1] >= nf + 2 * 2 * act
    assert block_ws_size(d, 0)[0] == ESHAPE
    assert block_ws_size(desc(D=768, H=2), 384)[0] == ESHAPE   # K = 384
    assert block_ws_size(desc(io=4), 384)[0] == EDTYPE
    assert L.rglru_block_workspace_size(ctypes.byref(d), 384, None) == ENULL


def test_block_fwd_validation(L):
    d = desc()
    dm = 384
    rc, n = block_ws_size(d, dm)
    assert rc == OK
    w = weights()
    s = None
    x, out = P + 0x1000000, P + 0x2000000
    ws = P + 0x10000000
    blk = glr._Block(P + 0x3000000, P + 0x4000000, P + 0x5000000)
    f = L.rglru_block_fwd
    args = lambda **k: [k.get(a, v) for a, v in (("x", x), ("hin", None), ("h0", None), ("out", out),
                                                   ("hl", None), ("hout", None), ("ws", ws), ("n", n))]
    assert f(ctypes.byref(d), dm, ctypes.byref(w), ctypes.byref(blk), *args(n=n - 1), s) == EWS
    assert f(ctypes.byref(d), dm, ctypes.byref(w), ctypes.byref(blk), *args(ws=None), s) == EWS
    assert f(ctypes.byref(d), dm, ctypes.byref(w), None, *args(), s) == ENULL
    assert f(ctypes.byref(d), dm, ctypes.byref(weights(conv=False)), ctypes.byref(blk), *args(), s) == ENULL
    assert f(ctypes.byref(d), 0, ctypes.byref(w), ctypes.byref(blk), *args(), s) == ESHAPE
    assert f(ctypes.byref(d), dm, ctypes.byref(w), ctypes.byref(blk), *args(x=x + 4), s) == EALIGN
    assert f(ctypes.byref(d), dm, ctypes.byref(w), ctypes.byref(blk), *args(out=x + 16), s) == EARG
    # the workspace overlapping a projection weight
    assert f(ctypes.byref(d), dm, ctypes.byref(w), ctypes.byref(blk), *args(ws=P + 0x3000000), s) == EARG
    bad = glr._Block(P + 0x3000000, None, P + 0x5000000)
    assert f(ctypes.byref(d), dm, ctypes.byref(w), ctypes.byref(bad), *args(), s) == ENULL


def adesc(B=2, T=64, Hq=10, dh=256, W=128, io=glr.BF16, scale=0.0625):
    return glr._AttnDesc(B, T, Hq, dh, W, io, scale)


def test_attn_validation(L):
    s = None
    q, k, v, o = P + 0x1000000, P + 0x2000000, P + 0x3000000, P + 0x4000000
    kc, vc = P + 0x5000000, P + 0x6000000
    f = L.rglru_attn_fwd
    assert f(None, q, k, v, o, None, None, s) == ENULL
    assert f(ctypes.byref(adesc(dh=260)), q, k, v, o, None, None, s) == ESHAPE
    assert f(ctypes.byref(adesc(dh=12)), q, k, v, o, None, None, s) == ESHAPE
    assert f(ctypes.byref(adesc(W=0)), q, k, v, o, None, None, s) == ESHAPE
    assert f(ctypes.byref(adesc(T=0)), q, k, v, o, None, None, s) == ESHAPE
    assert f(ctypes.byref(adesc(io=3)), q, k, v, o, None, None, s) == EDTYPE
    assert f(ctypes.byref(adesc()), q, k, v, o, kc, None, s) == EARG            # caches go together
    assert f(ctypes.byref(adesc()), q, k, v, q + 16, None, None, s) == EARG     # o overlaps q
    assert f(ctypes.byref(adesc()), q + 8, k, v, o, None, None, s) == EALIGN
    assert f(ctypes.byref(adesc(scale=float("inf"))), q, k, v, o, None, None, s) == EARG
    n = ctypes.c_size_t()
    assert L.rglru_attn_workspace_size(ctypes.byref(adesc(T=0)), ctypes.byref(n)) == OK   # T ignored
    g = L.rglru_attn_step
    ws, pos = P + 0x10000000, P + 0x7000000
    assert g(ctypes.byref(adesc()), q, k, v, kc, vc, pos, o, ws, n.value - 1, s) == EWS
    assert g(ctypes.byref(adesc()), q, k, v, kc, vc, None, o, ws, n.value, s) == ENULL
    assert g(ctypes.byref(adesc()), q, k, v, kc, vc, pos + 2, o, ws, n.value, s) == EALIGN
    assert g(ctypes.byref(adesc()), q, k, v, kc, kc, pos, o, ws, n.value, s) == EARG   # caches overlap


def test_layer_validation(L):
    d = desc()
    dm = 384
    lw = glr._Layer(P + 0x6000000, P + 0x6100000, P + 0x7000000, P + 0x8000000, P + 0x9000000, 1024, 1e-6)
    n = ctypes.c_size_t()
    assert L.rglru_layer_workspace_size(ctypes.byref(d), dm, ctypes.byref(lw), ctypes.byref(n)) == OK
    nb, _ = block_ws_size(d, dm)[1], None
    assert n.value > nb
    bad = glr._Layer(P, P, P, P, P, 0, 1e-6)
    assert L.rglru_layer_workspace_size(ctypes.byref(d), dm, ctypes.byref(bad), ctypes.byref(n)) == ESHAPE
    bad = glr._Layer(P, P, P, P, P, 64, float("nan"))
    assert L.rglru_layer_workspace_size(ctypes.byref(d), dm, ctypes.byref(bad), ctypes.byref(n)) == EARG
    w = weights()
    blk = glr._Block(P + 0x3000000, P + 0x4000000, P + 0x5000000)
    x, y, ws = P + 0x1000000, P + 0x2000000, P + 0x100000000
    f = L.rglru_layer_fwd
    assert f(ctypes.byref(d), dm, ctypes.byref(w), ctypes.byref(blk), None, x, None, None, y, None, None, ws,
             n.value, None) == ENULL
    assert f(ctypes.byref(d), dm, ctypes.byref(w), ctypes.byref(blk), ctypes.byref(lw), x, None, None, y, None,
             None, ws, n.value - 1, None) == EWS
    assert f(ctypes.byref(d), dm, ctypes.byref(w), ctypes.byref(blk), ctypes.byref(lw), x, None, None, x + 16,
             None, None, ws, n.value, None) == EARG
