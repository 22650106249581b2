"""fp8 (e4m3, OCP encoding) inputs for the fp8 step: quantisation and the error model.

Quantisation (test input preparation, not the method's arithmetic): a tensor x
gets the power-of-two scale s = 2^ceil(log2(max|x| / 448)), so that x / s fits
e4m3's range (448), and codes = RNE(x / s) in e4m3.  The dequantised values
codes * s are exact in fp64; the oracle consumes exactly those.

Error model: the kernel rounds the probabilities to e4m3 before the PV
product and normalises by the fp32 sum of the unrounded ones, then rounds the
output to bf16.  The probabilities are taken against a row maximum the
kernel keeps lazily per wave, so where they fall on the e4m3 grid depends on
that maximum; `lazy_model` repeats the kernel's arithmetic (tile order, lazy
maximum, rounding, per-launch merge) in fp64 and `lazy_model_error` returns
its max-abs deviation from the exact output on given rows.  The tolerance of
the fp8 parity test is derived from it.
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


# The fp8 output tolerance: MODEL_MARGIN times the deviation of the
# kernel's rounding model (lazy_model) on the same rows, plus the bf16
# rounding of the output (at most 2^-9 of |out|; 2^-8 of max |out| is
# allowed).  The model repeats the kernel's arithmetic in fp64; what it leaves
# out is the kernel's fp32 exponentials and sums, which can move a
# probability across an e4m3 rounding boundary now and then.
MODEL_MARGIN = 1.25


def out_tolerance(model_error: float, max_abs_out: float) -> float:
    return MODEL_MARGIN * model_error + max_abs_out / 256.0


# ---------------------------------------------------------------- lazy-maximum model
# The fp8 step kernel takes the probabilities of a 64-key tile against the row
# maximum it keeps lazily: on a wave's first tile, and whenever some lane's sum
# of 32 probabilities of a tile (against the maximum as it stands) exceeds 256
# or is not finite, every row of the wave (32 consecutive local rows) raises
# its maximum to its tile maximum; otherwise the maximum stays.  A lane of
# row i holds the tile's keys t with (t // 4) % 2 == g for its half g.  The
# tiles of a launch are its key chunks in table order, 64 keys at a time from
# each chunk's start; a new launch (or ring step) starts afresh and its
# partial result is merged by log-sum-exp.  lazy_model reproduces this in
# fp64: probabilities exp2(s log2(e) - m) against the lazily kept m, rounded
# to e4m3 for the PV product, normalised by the sum of the unrounded ones.
_LANE_G = (np.arange(64) // 4) % 2


def lazy_model(q: np.ndarray, k: np.ndarray, v: np.ndarray, q_pos: np.ndarray, waves: np.ndarray,
               k_pos: np.ndarray, segments, scale: float, rounding: bool = True):
    """(out [n, D], lse [n]) of the kernel's rounding model for rows q [n, D] at positions q_pos, wave ids
    `waves` [n] (rows sharing a wave share its rescaling decisions; pass every row of each wave), keys and
    values k, v [m, D] at positions k_pos; `segments` lists, per launch, the key indices in visit order
    (whole 64-key tiles of each chunk).  rounding=False skips the e4m3 rounding (the exact result)."""
    q_pos = np.asarray(q_pos)
    n, D = q.shape[0], v.shape[1]
    _, wave_ix = np.unique(np.asarray(waves), return_inverse=True)
    n_w = int(wave_ix.max()) + 1 if n else 0
    c = scale / math.log(2.0)
    out_tot = np.zeros((n, D))
    lse_tot = np.full(n, -np.inf)
    for seg in segments:
        seg = np.asarray(seg)
        m = np.full(n, -np.inf)
        l = np.zeros(n)
        o = np.zeros((n, D))
        for t0 in range(0, len(seg), 64):
            idx = seg[t0:t0 + 64]
            s2 = (q @ k[idx].T) * c
            vis = k_pos[idx][None, :] <= q_pos[:, None]
            s2 = np.where(vis, s2, -np.inf)
            g = _LANE_G[:len(idx)]
            with np.errstate(invalid="ignore", over="ignore"):
                p = np.exp2(s2 - m[:, None])
                lane = np.stack([np.where(g == h, p, 0.0).sum(axis=1) for h in (0, 1)], axis=1)
            redo = ~np.all(lane <= 256.0, axis=1)
            fire = np.zeros(n_w, bool)
            np.logical_or.at(fire, wave_ix, redo)
            fire = fire[wave_ix]
            m_new = np.where(fire, np.maximum(m, s2.max(axis=1)), m)
            with np.errstate(invalid="ignore"):
                alpha = np.where(m_new == m, 1.0, np.exp2(m - m_new))
            o *= alpha[:, None]
            l *= alpha
            m = m_new
            p = np.exp2(s2 - np.where(np.isfinite(m), m, 0.0)[:, None])
            l += p.sum(axis=1)
            o += (round_e4m3(p) if rounding else p) @ v[idx]
        has = l > 0
        lse_seg = np.where(has, (np.where(np.isfinite(m), m, 0.0) + np.log2(np.where(has, l, 1.0))) * math.log(2.0),
                           -np.inf)
        o_seg = np.where(has[:, None], o / np.where(has, l, 1.0)[:, None], 0.0)
        # exact log-sum-exp merge with the launches before
        L = np.logaddexp(lse_tot, lse_seg)
        with np.errstate(invalid="ignore"):
            wa = np.where(np.isfinite(lse_tot), np.exp(lse_tot - L), 0.0)
            wb = np.where(np.isfinite(lse_seg), np.exp(lse_seg - L), 0.0)
        out_tot = wa[:, None] * out_tot + wb[:, None] * o_seg
        lse_tot = L
    return out_tot, lse_tot


def ring_segments(kv_tables, grouped: bool):
    """Key positions per launch of a ring share, in visit order: one launch per ring step (`grouped`
    False: the chain of step calls), or step 0 alone and then the rest in the fewest groups of at most
    four steps, smaller groups first (the ring driver's grouping).  kv_tables: per step, a list of
    (chunk start, chunk length)."""
    steps = [np.concatenate([np.arange(s, s + L) for s, L in t]) for t in kv_tables]
    if not grouped:
        return steps
    rest = len(steps) - 1
    segs = [steps[0]]
    if rest > 0:
        groups = (rest + 3) // 4
        j = 1
        for gi in range(groups):
            cnt = rest // groups + (1 if gi >= groups - rest % groups else 0)
            segs.append(np.concatenate(steps[j:j + cnt]))
            j += cnt
    return segs


def lazy_model_error(q_all: np.ndarray, q_pos_all: np.ndarray, local_rows, k: np.ndarray, v: np.ndarray,
                     segments, scale: float):
    """The kernel model's max |out_model - out_exact| over `local_rows` of a rank's local buffer (queries
    q_all [Sq, D] at positions q_pos_all; keys/values k, v [S, D] indexed by absolute position), computing
    every row of the waves (32 local rows) that contain them.  Returns (that error, the oracle's out and
    lse of local_rows)."""
    import oracle
    local_rows = np.asarray(local_rows)
    waves = np.unique(local_rows // 32)
    rows = np.concatenate([np.arange(32 * w, 32 * w + 32) for w in waves])
    rows = rows[rows < len(q_pos_all)]
    kmax = int(max(int(np.max(sg)) for sg in segments)) + 1
    mo, _ = lazy_model(q_all[rows], k[:kmax], v[:kmax], q_pos_all[rows], rows // 32, np.arange(kmax), segments,
                       scale)
    mo = mo[np.searchsorted(rows, local_rows)]
    # the exact result over the keys the launches hold
    keys = np.unique(np.concatenate([np.asarray(sg) for sg in segments]))
    sel = q_pos_all[local_rows]
    ex, ls = oracle.masked_attention(q_all[local_rows], sel, k[keys], v[keys], keys, scale)
    ok = np.isfinite(ls)
    err = float(np.max(np.abs(mo[ok] - ex[ok]))) if ok.any() else 0.0
    return err, ex, ls
