"""Zigzag sharding and ring order, written out from the pages (oracle's own copy).

* Load balancing for causal attention ([RAF] section 5, item 1; also the
  note after section 3): the sequence is cut into 2N equal chunks and rank r
  of N holds chunks r and 2N-1-r, e.g. for N = 4: GPU0 chunks 0 and 7, GPU1
  1 and 6, GPU2 2 and 5, GPU3 3 and 4.  A rank's local buffer is its two
  chunks concatenated in ascending chunk order.
* Ring order ([RAF] section 3, the RingAttention loop): at step j rank r
  works on the K/V block that rank (r - j) mod N holds; step 0 is its own.
* Contiguous sharding ([MLM] section 1: each GPU handles 1/N of the
  sequence): rank r holds positions [r S/N, (r+1) S/N).
"""
from __future__ import annotations

import numpy as np


def zigzag_chunk_ids(cp: int, rank: int):
    if not 0 <= rank < cp:
        raise ValueError("rank out of range")
    return (rank, 2 * cp - 1 - rank)


def _chunks_positions(chunks, chunk_len: int) -> np.ndarray:
    return np.concatenate([np.arange(c * chunk_len, (c + 1) * chunk_len, dtype=np.int64)
                           for c in sorted(chunks)])


def local_positions(S: int, cp: int, rank: int) -> np.ndarray:
    """Absolute positions of a rank's local rows, in local order (zigzag)."""
    if S % (2 * cp):
        raise ValueError("S must be a multiple of 2*cp")
    return _chunks_positions(zigzag_chunk_ids(cp, rank), S // (2 * cp))


def contiguous_positions(S: int, cp: int, rank: int) -> np.ndarray:
    n = S // cp
    return np.arange(rank * n, (rank + 1) * n, dtype=np.int64)


def ring_source(rank: int, step: int, cp: int) -> int:
    return (rank - step) % cp


def ring_kv_positions(S: int, cp: int, rank: int, step: int) -> np.ndarray:
    """Absolute positions of the K/V block a rank attends to at ring step ``step``."""
    return local_positions(S, cp, ring_source(rank, step, cp))


def visible_pairs(q_pos, k_pos) -> int:
    """Number of (query, key) pairs with key position <= query position (brute force)."""
    q_pos = np.asarray(q_pos, np.int64)
    k_pos = np.sort(np.asarray(k_pos, np.int64))
    return int(np.searchsorted(k_pos, q_pos, side="right").sum())
