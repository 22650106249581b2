"""fp64 gradients of causal attention (oracle; test infrastructure only).

The backward pass of the context-parallel attention is the mirror image of
its forward: what the forward brings in block by block, the backward sends
back as gradients ([MLM] section 2), inside one autograd function with a
forward and a backward ([MLM] section 5).  The gradients themselves are those
of the definition in ``attention.py``, written out.  For a loss whose
gradient with respect to the output is dO (and which does not depend on the
LSE), with P_ij = exp(s_ij - LSE_i) for visible keys and 0 otherwise:

    dV_j    = sum_i P_ij dO_i
    dP_ij   = <dO_i, v_j>
    Delta_i = <dO_i, out_i>            (= sum_j P_ij dP_ij)
    dS_ij   = P_ij (dP_ij - Delta_i)
    dQ_i    = tau sum_j dS_ij k_j
    dK_j    = tau sum_i dS_ij q_i

Every term for key j uses only that key and the queries' full forward
results (out, LSE), so the gradients split over any blocks of keys: the dQ
parts of the blocks add up, and each block's dK and dV are its own rows of
the full dK and dV.  That is how one ring step's backward is cut: a K/V
block's dK and dV travel with the block, dQ stays on the rank.

Two functions:

* ``masked_attention_grad`` -- what one block of keys (at absolute positions
  ``k_pos``) contributes, given the queries' full ``out`` and ``lse``:
  returns ``(dq_part [n, D], dk [m, D], dv [m, D])``.
* ``causal_attention_grad`` -- full-sequence gradients of the causal
  attention of ``Q, K, V`` [S, D] for upstream ``dO`` [S, D].

Arithmetic is float64: scores by matmul, explicit mask, P from the saved LSE,
then the five products above.
"""
from __future__ import annotations

import numpy as np

from .attention import masked_attention


def masked_attention_grad(q: np.ndarray, q_pos: np.ndarray, k: np.ndarray, v: np.ndarray, k_pos: np.ndarray,
                          d_out: np.ndarray, out: np.ndarray, lse: np.ndarray, scale: float):
    """Gradient contributions of keys ``k``/``v`` [m, D] at ``k_pos`` for queries ``q`` [n, D] at ``q_pos``.

    ``out`` [n, D] and ``lse`` [n] are the queries' results over ALL their
    visible keys (not only this block's); ``d_out`` [n, D] is the upstream
    gradient.  Returns ``(dq_part, dk, dv)`` in float64.
    """
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    d_out = np.asarray(d_out, np.float64)
    out = np.asarray(out, np.float64)
    lse = np.asarray(lse, np.float64)
    q_pos = np.asarray(q_pos, np.int64)
    k_pos = np.asarray(k_pos, np.int64)
    n, m = q.shape[0], k.shape[0]
    dq = np.zeros((n, q.shape[1]), np.float64)
    dk = np.zeros((m, k.shape[1]), np.float64)
    dv = np.zeros((m, v.shape[1]), np.float64)
    if n == 0 or m == 0:
        return dq, dk, dv
    visible = (k_pos[None, :] <= q_pos[:, None]) & np.isfinite(lse)[:, None]
    s = scale * (q @ k.T)
    p = np.where(visible, np.exp(np.where(visible, s - lse[:, None], 0.0)), 0.0)  # [n, m]
    dv = p.T @ d_out
    dp = d_out @ v.T
    delta = np.sum(d_out * out, axis=1)
    ds = p * (dp - delta[:, None])
    dq = scale * (ds @ k)
    dk = scale * (ds.T @ q)
    return dq, dk, dv


def causal_attention_grad(Q: np.ndarray, K: np.ndarray, V: np.ndarray, dO: np.ndarray, scale: float | None = None):
    """Gradients (dQ, dK, dV) [S, D] of full-sequence causal attention for upstream ``dO`` [S, D]."""
    Q = np.asarray(Q, np.float64)
    K = np.asarray(K, np.float64)
    V = np.asarray(V, np.float64)
    S, D = Q.shape
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    pos = np.arange(S, dtype=np.int64)
    out, lse = masked_attention(Q, pos, K, V, pos, scale)
    return masked_attention_grad(Q, pos, K, V, pos, dO, out, lse, scale)
