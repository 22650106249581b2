"""Stream ordering of the ring drivers on the GPU: injected delays change no bit.

The double-buffered staging of [MLM] section 5 (the transfer for a later step
fills one buffer while the current step computes on the other, on its own
stream) is only correct if every copy waits for the launch that last read its
slot and every launch waits for its copy.  cp_test_set_delays makes the
drivers spin (a bounded device-side wait) before every launch that reads a
slot, on the compute stream, or before every staging copy, on the copy
stream; with either, a missing wait would let a copy overwrite a slot that a
launch has not yet read, or let a launch read a slot before its copy lands.
Rings here are long enough that both slots are reused several times
(forward: 16 and 64 steps in 5 and 17 launches; backward: from step 3 on).
The results must equal, bit for bit, the undelayed run and the run with
every copy in order on the compute stream; the undelayed forward is checked
against the oracle as well.  The CPU test test_ring_plan_sanitized.py checks
the same plans' happens-before order exhaustively.
"""
import math

import numpy as np
import pytest
import torch

import workloads
import long_sequence_causal_cp_amd as cp
from gpu_helpers import LSE_TOL, OUT_TOL, compare, gather, oracle_rows, positions, run_ring, zigzag_tables

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
DELAY_US = 1500   # per launch or copy: far longer than any launch or copy here


@pytest.fixture(scope="module", autouse=True)
def _lib():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    cp.load_library()
    yield
    cp.cp_test_set_delays(0, 0)


def _announce(*a):
    print("[case]", *a, flush=True)


@pytest.mark.parametrize("N,rank,L,D,H", [(16, 5, 64, 64, 2), (64, 17, 64, 128, 2), (8, 0, 128, 128, 4)])
def test_ring_fwd_slot_reuse_under_delays(N, rank, L, D, H):
    S = 2 * N * L
    scale = 1 / math.sqrt(D)
    Q, K, V = workloads.make_qkv_scaled((1, H, S, D), 500 + N)
    q_tab, kv_tabs = zigzag_tables(N, rank, L)
    cache = {}
    _announce("fwd delays", "N", N, "rank", rank, "L", L, "D", D, "H", H, "reference")
    cp.cp_test_set_delays(0, 0)
    ref_out, ref_lse = run_ring(Q, K, V, q_tab, kv_tabs, scale, DEV, kv_cache=cache)
    torch.cuda.synchronize()
    qpos = positions(q_tab)
    local = np.broadcast_to(np.arange(len(qpos)), (1, H, len(qpos))).copy()
    ro, rl = oracle_rows(Q, K, V, qpos[local], scale)
    eo, el = compare(ref_out, ref_lse, ro, rl, local)
    assert eo <= OUT_TOL and el <= LSE_TOL, (eo, el)
    main = torch.cuda.current_stream()
    try:
        for compute_us, copy_us in ((DELAY_US, 0), (0, DELAY_US), (DELAY_US, DELAY_US // 3)):
            _announce("fwd delays", "N", N, "compute_us", compute_us, "copy_us", copy_us)
            cp.cp_test_set_delays(compute_us, copy_us)
            out, lse = run_ring(Q, K, V, q_tab, kv_tabs, scale, DEV, kv_cache=cache)
            torch.cuda.synchronize()
            assert torch.equal(out, ref_out) and torch.equal(lse, ref_lse), (compute_us, copy_us)
        # every copy in order on the compute stream, with the compute-side delays
        cp.cp_test_set_delays(DELAY_US, DELAY_US)
        out, lse = run_ring(Q, K, V, q_tab, kv_tabs, scale, DEV, stream=main, copy_stream=main, kv_cache=cache)
        torch.cuda.synchronize()
        assert torch.equal(out, ref_out) and torch.equal(lse, ref_lse), "in order"
    finally:
        cp.cp_test_set_delays(0, 0)


def test_ring_fwd_fp8_slot_reuse_under_delays():
    """The fp8 ring shares the replay: 16 steps, delays on both sides, bit-identical."""
    N, rank, L, D, H = 16, 3, 128, 128, 2
    S = 2 * N * L
    gen = torch.Generator().manual_seed(808)
    codes = [torch.randn(1, H, S, D, generator=gen).clamp(-8, 8).to(torch.float8_e4m3fn) for _ in range(3)]
    q_tab, kv_tabs = zigzag_tables(N, rank, L)

    def g8(c, t):
        return gather(c.view(torch.uint8), t, DEV)
    q = g8(codes[0], q_tab).view(torch.float8_e4m3fn)
    ks = [g8(codes[1], t).view(torch.float8_e4m3fn) for t in kv_tabs]
    vts = [g8(codes[2], t).transpose(2, 3).contiguous().view(torch.float8_e4m3fn) for t in kv_tabs]
    ws = torch.empty(cp.cp_ring_attn_fwd_fp8_workspace_bytes(1, H, 2 * L, D, 2 * L), dtype=torch.uint8, device=DEV)

    def run():
        out = torch.empty((1, H, 2 * L, D), dtype=torch.bfloat16, device=DEV)
        lse = torch.empty((1, H, 2 * L), dtype=torch.float32, device=DEV)
        cp.cp_ring_attn_fwd_fp8(q, q_tab, ks, vts, kv_tabs, out, lse, 1 / math.sqrt(D), 0.25, 0.25, 0.5, ws,
                                copy_stream=torch.cuda.Stream())
        torch.cuda.synchronize()
        return out, lse

    try:
        _announce("fp8 fwd delays reference")
        cp.cp_test_set_delays(0, 0)
        ref = run()
        assert torch.isfinite(ref[0].float()).all() and torch.isfinite(ref[1]).all()
        for compute_us, copy_us in ((DELAY_US, 0), (0, DELAY_US)):
            _announce("fp8 fwd delays", compute_us, copy_us)
            cp.cp_test_set_delays(compute_us, copy_us)
            out, lse = run()
            assert torch.equal(out, ref[0]) and torch.equal(lse, ref[1]), (compute_us, copy_us)
    finally:
        cp.cp_test_set_delays(0, 0)


@pytest.mark.parametrize("N,rank,L,D,H", [(6, 2, 64, 64, 2), (9, 0, 128, 128, 2)])
def test_ring_bwd_slot_reuse_under_delays(N, rank, L, D, H):
    """cp_ring_attn_bwd with the ring's pattern (step 0 writes, later steps add to incoming partial sums):
    slot (j-1) % 2 is reused from step 3 on; delays on either stream leave dq and every dK/dV buffer
    bit-identical."""
    S = 2 * N * L
    scale = 1 / math.sqrt(D)
    Q, K, V = workloads.make_qkv_scaled((1, H, S, D), 700 + N)
    gen = torch.Generator().manual_seed(701 + N)
    dO = torch.randn(1, H, S, D, generator=gen).to(torch.bfloat16)
    q_tab, kv_tabs = zigzag_tables(N, rank, L)
    q, do = gather(Q, q_tab, DEV), gather(dO, q_tab, DEV)
    ks = [gather(K, t, DEV) for t in kv_tabs]
    vs = [gather(V, t, DEV) for t in kv_tabs]
    Sq, Skv = q.shape[2], ks[0].shape[2]
    cp.cp_test_set_delays(0, 0)
    out = torch.empty_like(q)
    lse = torch.empty(q.shape[:-1], dtype=torch.float32, device=DEV)
    wsf = torch.empty(cp.cp_ring_attn_workspace_bytes(1, H, Skv, D, Sq), dtype=torch.uint8, device=DEV)
    cp.cp_ring_attn_fwd(q, q_tab, ks, vs, kv_tabs, out, lse, scale, wsf, copy_stream=torch.cuda.Stream())
    init = [(torch.randn(ks[0].shape, generator=gen), torch.randn(ks[0].shape, generator=gen)) for _ in kv_tabs]
    ws = torch.empty(cp.cp_ring_attn_bwd_workspace_bytes(1, H, Skv, D, Sq), dtype=torch.uint8, device=DEV)
    main = torch.cuda.current_stream()

    def run(copy_stream):
        dks = [a.to(DEV) for a, _ in init]
        dvs = [b.to(DEV) for _, b in init]
        dq = torch.empty((1, H, Sq, D), dtype=torch.float32, device=DEV)
        cp.cp_ring_attn_bwd(q, q_tab, do, out, lse, ks, vs, kv_tabs, dks, dvs, dq, scale, ws,
                            copy_stream=copy_stream)
        torch.cuda.synchronize()
        return [dq] + dks + dvs

    try:
        _announce("bwd delays", "N", N, "rank", rank, "reference")
        ref = run(torch.cuda.Stream())
        assert all(torch.isfinite(x).all() for x in ref)
        for compute_us, copy_us in ((DELAY_US, 0), (0, DELAY_US), (DELAY_US, DELAY_US // 3)):
            _announce("bwd delays", "N", N, "compute_us", compute_us, "copy_us", copy_us)
            cp.cp_test_set_delays(compute_us, copy_us)
            got = run(torch.cuda.Stream())
            assert all(torch.equal(a, b) for a, b in zip(got, ref)), (compute_us, copy_us)
        cp.cp_test_set_delays(DELAY_US, DELAY_US)
        got = run(main)
        assert all(torch.equal(a, b) for a, b in zip(got, ref)), "in order"
    finally:
        cp.cp_test_set_delays(0, 0)
