"""fp8 (e4m3, OCP encoding) inputs for the fp8 step: quantisation and the error model.

Quantisation (test input preparation, not the method's arithmetic): a tensor x
gets the power-of-two scale s = 2^ceil(log2(max|x| / 448)), so that x / s fits
e4m3's range (448), and codes = RNE(x / s) in e4m3.  The dequantised values
codes * s are exact in fp64; the oracle consumes exactly those.

Error model: the kernel rounds the probabilities to e4m3 before the PV
product and normalises by the fp32 sum of the unrounded ones, then rounds the
output to bf16.  `emulated_error` reproduces that in fp64 for given rows
(probabilities relative to the exact row maximum, i.e. in (0, 1]) and returns
the max-abs deviation from the exact output; the tolerance of the fp8 parity
test is derived from it.
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
                   k_pos: np.ndarray | None = None) -> float:
    """Max |O_kernel_model - O_exact| over the rows q [n, D] at positions q_pos
    that see at least one key (keys k, v [m, D] at positions k_pos, by default
    0..m-1; causal)."""
    k_pos = np.arange(k.shape[0]) if k_pos is None else np.asarray(k_pos)
    s = scale * (q @ k.T)
    vis = k_pos[None, :] <= np.asarray(q_pos)[:, None]
    has = vis.any(axis=1)
    s, vis = np.where(vis, s, -np.inf)[has], vis[has]
    if s.shape[0] == 0:
        return 0.0
    m = s.max(axis=1, keepdims=True)
    p = np.where(vis, np.exp(s - m), 0.0)
    l = p.sum(axis=1, keepdims=True)
    exact = (p @ v) / l
    model = (round_e4m3(p) @ v) / l
    return float(np.max(np.abs(model - exact)))


# The fp8 output tolerance is this multiple of the model's deviation: on the
# zigzag workloads the model gives 0.035-0.039 and the bound there is 0.1.
# Rows that see few keys (near a chunk start, or crafted key tables) average
# the rounding over fewer terms, so their bound comes from the model on the
# same inputs with the same margin.
MODEL_MARGIN = 2.5


def out_tolerance(model_error: float, floor: float) -> float:
    return max(floor, MODEL_MARGIN * model_error)
