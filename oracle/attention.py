"""fp64 causal attention from its definition (oracle; test infrastructure only).

Follows the causal self-attention that the pages rely on: each query attends
to every key at or before its own absolute position ([RAF] section 1: a
token's query meets all previous keys and values; [RAF] section 3, note 2:
the mask is built from the blocks' real offsets so no later token leaks in;
[MLM] section 3: causal mask type).  The softmax scale is 1/sqrt(D).

Two functions:

* ``masked_attention`` -- queries at given absolute positions against an
  arbitrary set of keys with their own absolute positions; a key is visible
  iff its position <= the query's.  A query with no visible key gets
  out = 0 and LSE = -inf (the partial result of a ring step that holds
  nothing before that query).
* ``causal_attention_rows`` -- the full-sequence definition evaluated on a
  chosen set of query rows, against keys 0 .. max(row) in blocks of at most
  512 rows.

Arithmetic is float64 throughout: scores by matmul, explicit mask, row
maximum, exponentials, row sum, then P @ V divided by the sum.
"""
from __future__ import annotations

import numpy as np

ROW_BLOCK = 512


def to_f64(t) -> np.ndarray:
    """Exact up-cast of a (bf16 / fp32) torch tensor or array to float64."""
    try:
        import torch
        if isinstance(t, torch.Tensor):
            return t.detach().to("cpu", torch.float64).numpy()
    except ImportError:  # pragma: no cover
        pass
    return np.asarray(t, dtype=np.float64)


def masked_attention(q: np.ndarray, q_pos: np.ndarray, k: np.ndarray, v: np.ndarray,
                     k_pos: np.ndarray, scale: float):
    """Attention of queries ``q`` [n, D] at ``q_pos`` over keys ``k``/``v`` [m, D] at ``k_pos``.

    Returns ``(out [n, D], lse [n])`` in float64, natural-log LSE.
    """
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    q_pos = np.asarray(q_pos, np.int64)
    k_pos = np.asarray(k_pos, np.int64)
    n, d = q.shape
    out = np.zeros((n, v.shape[1]), np.float64)
    lse = np.full(n, -np.inf, np.float64)
    if n == 0 or k.shape[0] == 0:
        return out, lse
    s = scale * (q @ k.T)                                   # [n, m]
    visible = k_pos[None, :] <= q_pos[:, None]
    s = np.where(visible, s, -np.inf)
    has_key = visible.any(axis=1)
    if not has_key.any():
        return out, lse
    sr = s[has_key]
    m = sr.max(axis=1)
    e = np.exp(sr - m[:, None])                             # masked entries -> exp(-inf) = 0
    z = e.sum(axis=1)
    out[has_key] = (e @ v) / z[:, None]
    lse[has_key] = m + np.log(z)
    return out, lse


def causal_attention_rows(Q: np.ndarray, K: np.ndarray, V: np.ndarray,
                          rows, scale: float | None = None):
    """Full-sequence causal attention evaluated at absolute positions ``rows``.

    ``Q, K, V``: float64 [..., S, D] over the whole sequence (any leading
    batch/head dims).  ``rows``: 1-D positions shared by all heads, or an
    integer array shaped like the leading dims plus one trailing axis giving
    per-head rows.  Returns ``(out [..., n, D], lse [..., n])``.
    """
    Q = np.asarray(Q, np.float64)
    K = np.asarray(K, np.float64)
    V = np.asarray(V, np.float64)
    lead = Q.shape[:-2]
    D = Q.shape[-1]
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    rows = np.asarray(rows, np.int64)
    per_head = rows.ndim > 1
    n = rows.shape[-1]
    out = np.empty(lead + (n, V.shape[-1]), np.float64)
    lse = np.empty(lead + (n,), np.float64)
    for idx in np.ndindex(*lead):
        r = rows[idx] if per_head else rows
        q, k, v = Q[idx], K[idx], V[idx]
        for a in range(0, n, ROW_BLOCK):
            blk = r[a:a + ROW_BLOCK]
            kmax = int(blk.max()) + 1
            o, l = masked_attention(q[blk], blk, k[:kmax], v[:kmax],
                                    np.arange(kmax, dtype=np.int64), scale)
            out[idx + (slice(a, a + len(blk)),)] = o
            lse[idx + (slice(a, a + len(blk)),)] = l
    return out, lse
