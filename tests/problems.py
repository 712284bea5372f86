"""Seeded problems in two forms: torch device tensors for the HIP library and
float64 numpy arrays (the same stored values, widened) for the oracle."""
from __future__ import annotations

import dataclasses

import numpy as np
import torch

import gated_linear_recurrence_02_amd as glr
import synth

TOL = {"f32": 1e-5, "bf16": 2e-2}   # max |g - o| / max(|o|, RMS(o))


def to_dev(stored: np.ndarray, dev) -> torch.Tensor:
    if stored.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(stored).view(np.int16)).view(torch.bfloat16).to(dev)
    return torch.from_numpy(np.ascontiguousarray(stored, dtype=np.float32)).to(dev)


def from_dev(t: torch.Tensor) -> np.ndarray:
    """Device tensor -> float64 numpy (exact widening)."""
    return t.detach().float().cpu().numpy().astype(np.float64)


@dataclasses.dataclass
class Problem:
    cfg: int
    B: int
    T: int
    D: int
    H: int
    io: str
    params: synth.Params
    u: np.ndarray          # stored
    h0: np.ndarray | None  # float32
    hist: np.ndarray | None  # stored

    @property
    def dtype(self):
        return torch.bfloat16 if self.io == "bf16" else torch.float32

    def weights(self, dev) -> glr.Weights:
        p = self.params
        return glr.Weights(conv_w=to_dev(p.conv_w, dev), W_a=to_dev(p.W_a, dev),
                           W_x=to_dev(p.W_x, dev), Lambda=to_dev(p.Lambda, dev),
                           conv_b=to_dev(p.conv_b, dev), b_a=to_dev(p.b_a, dev),
                           b_x=to_dev(p.b_x, dev))

    def oracle_params(self, h=None):
        """Oracle parameter dict, optionally restricted to block h (D = K, H = 1)."""
        p = self.params
        K = self.D // self.H
        sl = slice(None) if h is None else slice(h * K, (h + 1) * K)
        hs = slice(None) if h is None else slice(h, h + 1)
        return dict(conv_w=synth.widen(p.conv_w)[sl], conv_b=synth.widen(p.conv_b)[sl],
                    W_a=synth.widen(p.W_a)[hs], b_a=synth.widen(p.b_a)[sl],
                    W_x=synth.widen(p.W_x)[hs], b_x=synth.widen(p.b_x)[sl],
                    Lambda=synth.widen(p.Lambda)[sl])

    def slice_block(self, arr: np.ndarray, b=None, h=None):
        """arr [B][..][D] -> rows b (all if None), channels of block h."""
        K = self.D // self.H
        out = arr if b is None else arr[b:b + 1]
        if h is not None:
            out = out[..., h * K:(h + 1) * K]
        return np.ascontiguousarray(out)


def make_problem(cfg: int, B=None, T=None, with_state=False, param_cfg=None) -> Problem:
    c = synth.CONFIGS[cfg]
    B = c.B if B is None else B
    T = c.T if T is None else T
    p = synth.make_params(c.idx if param_cfg is None else param_cfg, c.D, c.H, c.io)
    u = synth.make_activation(c.idx, "u", (B, T, c.D), c.io)
    h0 = hist = None
    if with_state:
        h0 = synth.store(synth.normal(synth.seed_for(c.idx, "h0"), 0, B * c.D), "f32").reshape(B, c.D)
        hist = synth.make_activation(c.idx, "hist", (B, 3, c.D), c.io)
    return Problem(c.idx, B, T, c.D, c.H, c.io, p, u, h0, hist)
