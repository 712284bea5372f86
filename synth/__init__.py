"""Seeded synthetic inputs for the RG-LRU hot path.

This module is shared by the CPU oracle's tests, the GPU parity tests, the
bench and the smoke check.  It holds no arithmetic of the method itself: only
random-number generation, the parameter-initialisation recipe, storage
rounding (fp32 -> bf16) and the table of workload shapes.

Generator
---------
SplitMix64 (Steele, Lea & Flood, "Fast splittable pseudorandom number
generators", OOPSLA 2014), used counter-style: the n-th draw (n >= 1) of the
stream with seed s is mix(s + n * 0x9E3779B97F4A7C15), where mix is the
published 64-bit finaliser.  Because every draw is a pure function of its
index, any sub-range of a tensor can be generated on its own (the decode
workload generates one step at a time, the oracle slices one sequence).

Uniforms are (z >> 11) * 2^-53 in [0, 1).  Normals come from the Box-Muller
transform (Box & Muller, 1958): element k uses draws 2k+1 and 2k+2,
u1 = ((z1 >> 11) + 1) * 2^-53 in (0, 1], u2 = (z2 >> 11) * 2^-53,
n = sqrt(-2 ln u1) * cos(2 pi u2).

Streams: seed = 0x52474C5500000000 ^ (config << 16) ^ tensor_id.

Initialisation recipe (RG-LRU page, section "Formulation of the RG-LRU
Gating Mechanism" and the module's Lambda initialiser): the decay base
a = sigmoid(Lambda) is drawn so that a^c is uniform on [0.9, 0.999], i.e.
u ~ U[0.9, 0.999], a = u^(1/c), Lambda = log(a / (1 - a)); c = 8.  Gate
weights are N(0, 1/K) (variance; std 1/sqrt(K)), conv weights N(0, 1/4)
(std 0.5), biases 0, activations N(0, 1).  The recurrent block's
projections (no bias, stored [out][in]) are N(0, 1/fan_in), which keeps
unit-variance activations at unit variance; the pages give no initialiser
for them.

Rounding: values are generated in float64, rounded to float32 (IEEE
round-to-nearest-even) and, for bf16 storage, from float32 to bf16 with
round-to-nearest-even on the bit pattern.
"""
from __future__ import annotations

import dataclasses
import math
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

GOLDEN = np.uint64(0x9E3779B97F4A7C15)
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)
SEED_BASE = 0x52474C5500000000
_BLOCK = 1 << 20
_THREADS = max(1, min(16, os.cpu_count() or 1))

# tensor ids of the per-tensor streams
TID = dict(u=0, conv_w=1, conv_b=2, W_a=3, W_x=4, lam_u=5, dy=6, h0=7,
           b_a=8, b_x=9, hist=10, dh_last=11,
           block_x=12, proj_in_1=13, proj_in_2=14, proj_out=15,
           attn_q=16, attn_k=17, attn_v=18, attn_hk=19, attn_hv=20,
           tnorm_w=21, cnorm_w=22, gate_w=23, up_w=24, down_w=25,
           wq=26, wk=27, wv=28, wo=29)

C_CONST = 8.0


def seed_for(cfg: int, tensor: str) -> int:
    return (SEED_BASE ^ (int(cfg) << 16) ^ TID[tensor]) & 0xFFFFFFFFFFFFFFFF


def _mix(z: np.ndarray) -> np.ndarray:
    z = (z ^ (z >> np.uint64(30))) * _M1
    z = (z ^ (z >> np.uint64(27))) * _M2
    return z ^ (z >> np.uint64(31))


def raw_u64(seed: int, start: int, count: int) -> np.ndarray:
    """Draws number start+1 .. start+count of the SplitMix64 stream `seed`."""
    n = np.arange(start + 1, start + count + 1, dtype=np.uint64)
    with np.errstate(over="ignore"):
        return _mix(np.uint64(seed) + n * GOLDEN)


def _blocks(count: int, fill) -> None:
    """Run fill(b0, n) over [0, count) in blocks; numpy releases the GIL, so
    blocks run on several threads.  Every element is a pure function of its
    index, so the result does not depend on the split."""
    spans = [(b0, min(_BLOCK, count - b0)) for b0 in range(0, count, _BLOCK)]
    if len(spans) <= 1:
        for b0, n in spans:
            fill(b0, n)
        return
    with ThreadPoolExecutor(min(_THREADS, len(spans))) as ex:
        list(ex.map(lambda sp: fill(*sp), spans))


def uniform(seed: int, start: int, count: int) -> np.ndarray:
    """Uniform float64 in [0, 1): element k of the tensor is draw start+k+1."""
    out = np.empty(count, dtype=np.float64)

    def fill(b0, n):
        z = raw_u64(seed, start + b0, n)
        out[b0:b0 + n] = (z >> np.uint64(11)).astype(np.float64) * 2.0 ** -53
    _blocks(count, fill)
    return out


def normal(seed: int, start: int, count: int) -> np.ndarray:
    """Standard normal float64; element k of the tensor uses draws 2k+1, 2k+2."""
    out = np.empty(count, dtype=np.float64)

    def fill(b0, n):
        z = raw_u64(seed, 2 * (start + b0), 2 * n)
        u1 = ((z[0::2] >> np.uint64(11)).astype(np.float64) + 1.0) * 2.0 ** -53
        u2 = (z[1::2] >> np.uint64(11)).astype(np.float64) * 2.0 ** -53
        out[b0:b0 + n] = np.sqrt(-2.0 * np.log(u1)) * np.cos(2.0 * math.pi * u2)
    _blocks(count, fill)
    return out


# ---------------------------------------------------------------- bf16 storage
def f32_to_bf16_bits(x) -> np.ndarray:
    """float32 -> bf16 bit pattern (uint16), round to nearest even."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    nan = (b & 0x7FFFFFFF) > 0x7F800000
    r = ((b + np.uint32(0x7FFF) + ((b >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16))
    r = np.where(nan, (b >> np.uint32(16)) | np.uint32(0x40), r)
    return r.astype(np.uint16)


def bf16_bits_to_f32(bits) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def store(x64: np.ndarray, io: str) -> np.ndarray:
    """Round float64 values to the storage dtype.

    Returns float32 for io='f32' and uint16 bf16 bit patterns for io='bf16'."""
    x64 = np.asarray(x64, dtype=np.float64)
    flat = np.ravel(x64)
    out = np.empty(flat.size, dtype=np.float32 if io == "f32" else np.uint16)

    def fill(b0, n):
        f = flat[b0:b0 + n].astype(np.float32)
        out[b0:b0 + n] = f if io == "f32" else f32_to_bf16_bits(f)
    _blocks(flat.size, fill)
    return out.reshape(x64.shape)


def widen(stored: np.ndarray) -> np.ndarray:
    """Stored values (float32, or uint16 bf16 bits) as exact float64."""
    if stored.dtype == np.uint16:
        return bf16_bits_to_f32(stored).astype(np.float64)
    return np.asarray(stored, dtype=np.float32).astype(np.float64)


# ------------------------------------------------------------- workload table
@dataclasses.dataclass(frozen=True)
class Config:
    idx: int
    name: str
    B: int
    T: int
    D: int
    H: int
    io: str          # storage dtype of activations and gate weights
    steps: int = 0   # decode workload: number of one-token calls

    @property
    def K(self) -> int:
        return self.D // self.H


CONFIGS = [
    Config(0, "tiny fp32 forward", 1, 256, 256, 1, "f32"),
    Config(1, "2B-width prefill", 8, 2048, 2560, 10, "bf16"),
    Config(2, "long-sequence prefill", 1, 32768, 2560, 10, "bf16"),
    Config(3, "decode step", 256, 1, 2560, 10, "bf16", steps=512),
    Config(4, "9B-width forward+backward", 4, 8192, 4096, 16, "bf16"),
]

# the same workloads by name (the index stays the seed component)
TINY, PREFILL_2B, PREFILL_32K, DECODE_256, FWD_BWD_9B = CONFIGS


def lambda_from_uniform(u01: np.ndarray, c: float = C_CONST) -> np.ndarray:
    """Lambda = logit(u^(1/c)) with u = 0.9 + 0.099 * u01 (float64)."""
    u = 0.9 + (0.999 - 0.9) * u01
    a = u ** (1.0 / c)
    return np.log(a / (1.0 - a))


@dataclasses.dataclass
class Params:
    """Stored parameters: float32 arrays, gate weights in the io storage form."""
    conv_w: np.ndarray   # [D][4] f32
    conv_b: np.ndarray   # [D] f32
    W_a: np.ndarray      # [H][K][K] io
    b_a: np.ndarray      # [D] f32
    W_x: np.ndarray      # [H][K][K] io
    b_x: np.ndarray      # [D] f32
    Lambda: np.ndarray   # [D] f32
    lam_u: np.ndarray    # [D] float64: the a^c draw each Lambda came from


def make_params(cfg: int, D: int, H: int, io: str, c: float = C_CONST) -> Params:
    K = D // H
    cw = store(0.5 * normal(seed_for(cfg, "conv_w"), 0, D * 4), "f32").reshape(D, 4)
    wstd = 1.0 / math.sqrt(K)
    Wa = store(wstd * normal(seed_for(cfg, "W_a"), 0, H * K * K), io).reshape(H, K, K)
    Wx = store(wstd * normal(seed_for(cfg, "W_x"), 0, H * K * K), io).reshape(H, K, K)
    u01 = uniform(seed_for(cfg, "lam_u"), 0, D)
    lam = store(lambda_from_uniform(u01, c), "f32")
    zeros = np.zeros(D, dtype=np.float32)
    return Params(cw, zeros.copy(), Wa, zeros.copy(), Wx, zeros.copy(), lam,
                  0.9 + (0.999 - 0.9) * u01)


def make_activation(cfg: int, tensor: str, shape, io: str, start: int = 0,
                    scale: float = 1.0) -> np.ndarray:
    n = int(np.prod(shape))
    return store(scale * normal(seed_for(cfg, tensor), start, n), io).reshape(shape)


def make_u(cfg: Config, B=None, T=None) -> np.ndarray:
    B = cfg.B if B is None else B
    T = cfg.T if T is None else T
    return make_activation(cfg.idx, "u", (B, T, cfg.D), cfg.io)


def make_decode_u(cfg: Config, step: int) -> np.ndarray:
    """Input of decode call `step` ([B][D]); the decode stream is [steps][B][D]."""
    n = cfg.B * cfg.D
    return make_activation(cfg.idx, "u", (cfg.B, cfg.D), cfg.io, start=step * n)


def make_dy(cfg: Config) -> np.ndarray:
    return make_activation(cfg.idx, "dy", (cfg.B, cfg.T, cfg.D), cfg.io)


@dataclasses.dataclass
class BlockParams:
    """Projections of the recurrent block, stored [out][in] in the io form."""
    proj_in_1: np.ndarray   # [D][d_model]
    proj_in_2: np.ndarray   # [D][d_model]
    proj_out: np.ndarray    # [d_model][D]


def make_block_params(cfg: int, d_model: int, D: int, io: str) -> BlockParams:
    s_in, s_out = 1.0 / math.sqrt(d_model), 1.0 / math.sqrt(D)
    p1 = store(s_in * normal(seed_for(cfg, "proj_in_1"), 0, D * d_model), io).reshape(D, d_model)
    p2 = store(s_in * normal(seed_for(cfg, "proj_in_2"), 0, D * d_model), io).reshape(D, d_model)
    po = store(s_out * normal(seed_for(cfg, "proj_out"), 0, d_model * D), io).reshape(d_model, D)
    return BlockParams(p1, p2, po)


@dataclasses.dataclass
class LayerParams:
    """Residual-layer weights around the block: pre-norm weights [d_model] fp32
    (applied as 1 + w), gated MLP gate_w, up_w [d_ff][d_model], down_w
    [d_model][d_ff] in the io form."""
    tnorm_w: np.ndarray
    cnorm_w: np.ndarray
    gate_w: np.ndarray
    up_w: np.ndarray
    down_w: np.ndarray


def make_layer_params(cfg: int, d_model: int, d_ff: int, io: str) -> LayerParams:
    tn = store(0.1 * normal(seed_for(cfg, "tnorm_w"), 0, d_model), "f32")
    cn = store(0.1 * normal(seed_for(cfg, "cnorm_w"), 0, d_model), "f32")
    g = store(normal(seed_for(cfg, "gate_w"), 0, d_ff * d_model) / math.sqrt(d_model), io).reshape(d_ff, d_model)
    u = store(normal(seed_for(cfg, "up_w"), 0, d_ff * d_model) / math.sqrt(d_model), io).reshape(d_ff, d_model)
    dn = store(normal(seed_for(cfg, "down_w"), 0, d_model * d_ff) / math.sqrt(d_ff), io).reshape(d_model, d_ff)
    return LayerParams(tn, cn, g, u, dn)


@dataclasses.dataclass
class AttnProj:
    """Attention layer projections [out][in] in the io form: wq [Hq*dh][d_model],
    wk, wv [dh][d_model], wo [d_model][Hq*dh]."""
    wq: np.ndarray
    wk: np.ndarray
    wv: np.ndarray
    wo: np.ndarray


def make_attn_proj(cfg: int, d_model: int, Hq: int, dh: int, io: str) -> AttnProj:
    s_in, s_o = 1.0 / math.sqrt(d_model), 1.0 / math.sqrt(Hq * dh)
    wq = store(s_in * normal(seed_for(cfg, "wq"), 0, Hq * dh * d_model), io).reshape(Hq * dh, d_model)
    wk = store(s_in * normal(seed_for(cfg, "wk"), 0, dh * d_model), io).reshape(dh, d_model)
    wv = store(s_in * normal(seed_for(cfg, "wv"), 0, dh * d_model), io).reshape(dh, d_model)
    wo = store(s_o * normal(seed_for(cfg, "wo"), 0, d_model * Hq * dh), io).reshape(d_model, Hq * dh)
    return AttnProj(wq, wk, wv, wo)
