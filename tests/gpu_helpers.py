"""Shared plumbing for the GPU parity tests: rank buffers, ring calls, oracle rows.

Zigzag chunk tables are built from the oracle's index maths
(oracle.local_positions, oracle.ring_kv_positions) and checked equal to the
library's cp_zigzag_chunks before use; rank buffers are gathered from the
full sequence with them, and expected values come from the fp64 oracle.  The oracle runs per (batch, head) in a thread
pool (numpy releases the GIL in matmul and exp), at most 16 threads.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import torch

import oracle
import long_sequence_causal_cp_amd as cp

OUT_TOL = 2e-2
LSE_TOL = 1e-3


def threads():
    return max(1, min(16, len(os.sched_getaffinity(0))))


def positions(table):
    return np.concatenate([np.arange(s, s + table.chunk_len) for s in table.starts()])


def gather(x, table, dev):
    idx = torch.from_numpy(positions(table))
    return x.index_select(2, idx).contiguous().to(dev)


def table_from_positions(pos, chunk_len):
    """Chunk table of a local buffer whose rows sit at absolute positions ``pos`` (whole chunks)."""
    pos = np.asarray(pos, np.int64)
    assert len(pos) % chunk_len == 0
    starts = [int(s) for s in pos[::chunk_len]]
    for i, s in enumerate(starts):
        assert np.array_equal(pos[i * chunk_len:(i + 1) * chunk_len], np.arange(s, s + chunk_len))
    return cp.CpChunks.make(starts, chunk_len)


def zigzag_tables(cp_size, rank, L):
    """The rank's query table and the K/V table of every ring step, from the oracle's positions; the
    library's cp_zigzag_chunks must give the same tables."""
    S = 2 * cp_size * L
    q_tab = table_from_positions(oracle.local_positions(S, cp_size, rank), L)
    kv = [table_from_positions(oracle.ring_kv_positions(S, cp_size, rank, j), L) for j in range(cp_size)]
    for j in range(cp_size):
        lq, lkv = cp.cp_zigzag_chunks(cp_size, rank, L, j)
        assert (lq.starts(), lq.chunk_len) == (q_tab.starts(), L), (cp_size, rank, j)
        assert (lkv.starts(), lkv.chunk_len) == (kv[j].starts(), L), (cp_size, rank, j)
    return q_tab, kv


def run_ring(Q, K, V, q_tab, kv_tabs, scale, dev, stream=None, copy_stream=None, kv_cache=None):
    """Gather the rank's Q and each step's K/V, run cp_ring_attn_fwd; returns (out, lse) on device."""
    B, H, _, D = Q.shape
    q = gather(Q, q_tab, dev)
    ks, vs = [], []
    for t in kv_tabs:
        key = tuple(t.starts())
        if kv_cache is not None and key in kv_cache:
            kk, vv = kv_cache[key]
        else:
            kk, vv = gather(K, t, dev), gather(V, t, dev)
            if kv_cache is not None:
                kv_cache[key] = (kk, vv)
        ks.append(kk)
        vs.append(vv)
    Sq, Skv = q.shape[2], ks[0].shape[2]
    out = torch.empty_like(q)
    lse = torch.empty((B, H, Sq), dtype=torch.float32, device=dev)
    ws = torch.empty(cp.cp_ring_attn_workspace_bytes(B, H, Skv, D, Sq), dtype=torch.uint8, device=dev)
    copy_stream = copy_stream or torch.cuda.Stream()
    cp.cp_ring_attn_fwd(q, q_tab, ks, vs, kv_tabs, out, lse, scale, ws, stream=stream, copy_stream=copy_stream)
    return out, lse


def oracle_rows(Q, K, V, pos_per_head, scale):
    """Oracle (out, lse) at absolute positions pos_per_head [B, H, n] (bf16 inputs, fp64 maths)."""
    B, H = Q.shape[:2]
    n = pos_per_head.shape[-1]
    D = V.shape[-1]
    out = np.empty((B, H, n, D))
    lse = np.empty((B, H, n))

    def one(bh):
        b, h = divmod(bh, H)
        rows = pos_per_head[b, h]
        kmax = int(rows.max()) + 1
        q = oracle.to_f64(Q[b, h])
        k = oracle.to_f64(K[b, h, :kmax])
        v = oracle.to_f64(V[b, h, :kmax])
        out[b, h], lse[b, h] = oracle.causal_attention_rows(q, k, v, rows, scale)

    with ThreadPoolExecutor(threads()) as ex:
        list(ex.map(one, range(B * H)))
    return out, lse


# Half an ulp of bf16 is at most 2^-8 of the value: the bf16 output's own rounding.
BF16_HALF_ULP_REL = 2.0 ** -8


def compare(out_gpu, lse_gpu, out_ref, lse_ref, local_rows=None, output_rounding=False):
    """Max-abs errors of GPU results (optionally at local_rows [B,H,n]) against the oracle's.

    With output_rounding, the output error is counted beyond the bf16 output's own rounding,
    max(|out - ref| - 2^-8 |ref|): for stress inputs whose outputs reach magnitudes where half an ulp
    of bf16 alone approaches the bound (|out| >= 2: 2^-7 and more)."""
    o = out_gpu.float().cpu().numpy()
    l = lse_gpu.cpu().numpy()
    if local_rows is not None:
        o = np.take_along_axis(o, local_rows[..., None], axis=2)
        l = np.take_along_axis(l, local_rows, axis=2)
    assert np.isfinite(o).all() and np.isfinite(l).all()
    err = np.abs(o - out_ref)
    if output_rounding:
        err = err - BF16_HALF_ULP_REL * np.abs(out_ref)
    return float(np.max(err)), float(np.max(np.abs(l - lse_ref)))
