"""fp8 (e4m3, OCP encoding) inputs for the fp8 step: quantisation and the error model.

Quantisation (test input preparation, not the method's arithmetic): a tensor x
gets the power-of-two scale s = 2^ceil(log2(max|x| / 448)), so that x / s fits
e4m3's range (448), and codes = RNE(x / s) in e4m3.  The dequantised values
codes * s are exact in fp64; the oracle consumes exactly those.

Error model: the kernel rounds the probabilities to e4m3 before the PV
product and normalises by the fp32 sum of the unrounded ones, then rounds the
output to bf16.  `emulated_error` reproduces that in fp64 for given rows and
returns the max-abs deviation from the exact output; the tolerance of the fp8
parity test is derived from it.  The model takes the probabilities relative
to each row's exact maximum (the largest is then exactly 1).  The kernel takes
them against its lazily kept maximum, which may sit up to 8 binades below the
row's, so its probabilities are the model's times some 2^delta and fall
differently on the e4m3 grid; `phases` > 1 evaluates delta = i/phases of a
binade and keeps the largest deviation (an envelope over that shift).
"""
from __future__ import annotations

import math

import numpy as np
import torch

E4M3_MAX = 448.0


def quantize(x: torch.Tensor):
    """(codes as torch.float8_e4m3fn, scale) for a float tensor x (CPU)."""
    amax = float(x.abs().max())
    s = 2.0 ** math.ceil(math.log2(amax / E4M3_MAX)) if amax > 0 else 1.0
    codes = (x.to(torch.float64) / s).to(torch.float32).to(torch.float8_e4m3fn)
    return codes, s


def dequantize(codes: torch.Tensor, s: float) -> np.ndarray:
    return codes.to(torch.float64).numpy() * s


def round_e4m3(p: np.ndarray) -> np.ndarray:
    return torch.from_numpy(np.asarray(p, np.float32)).to(torch.float8_e4m3fn).to(torch.float64).numpy()


def emulated_error(q: np.ndarray, k: np.ndarray, v: np.ndarray, q_pos: np.ndarray, scale: float,
                   k_pos: np.ndarray | None = None, phases: int = 1, block: int = 512) -> float:
    """Max over rounding phases delta = i/phases (i = 0..phases-1) of max |O_model - O_exact| over the
    rows q [n, D] at positions q_pos that see at least one key (keys k, v [m, D] at positions k_pos, by
    default 0..m-1; causal), where O_model rounds the probabilities exp(s - max) * 2^delta to e4m3,
    multiplies by V and divides by the unrounded sum.  Rows are processed in blocks of `block`."""
    k_pos = np.arange(k.shape[0]) if k_pos is None else np.asarray(k_pos)
    q_pos = np.asarray(q_pos)
    worst = 0.0
    for r0 in range(0, q.shape[0], block):
        qb, pb = q[r0:r0 + block], q_pos[r0:r0 + block]
        s = scale * (qb @ k.T)
        vis = k_pos[None, :] <= pb[:, None]
        has = vis.any(axis=1)
        if not has.any():
            continue
        s, vis = np.where(vis, s, -np.inf)[has], vis[has]
        m = s.max(axis=1, keepdims=True)
        p = np.where(vis, np.exp(s - m), 0.0)
        l = p.sum(axis=1, keepdims=True)
        exact = (p @ v) / l
        for i in range(phases):
            f = 2.0 ** (i / phases)
            model = (round_e4m3(p * f) @ v) / (l * f)
            worst = max(worst, float(np.max(np.abs(model - exact))))
    return worst


# The fp8 output tolerance: MODEL_MARGIN times the model's deviation on the
# same rows (exact maximum), plus the bf16 rounding of the output (at most
# 2^-9 of |out|; 2^-8 of max |out| is allowed).  The margin covers the
# kernel's lazily shifted rounding phase: measured on the GPU over every fp8
# parity case, the kernel's deviation reached up to MEASURED_RATIO times the
# model's.
MEASURED_RATIO = 2.63
MODEL_MARGIN = 3.0


def out_tolerance(model_error: float, max_abs_out: float) -> float:
    return MODEL_MARGIN * model_error + max_abs_out / 256.0
