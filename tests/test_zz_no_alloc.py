"""cp_ring_attn_fwd_noalloc against cp_ring_attn_fwd, through the C ABI.

The no-allocation entry point runs the same ring from the library's static
per-device scratch array instead of a caller workspace.  Two calls in a row,
the second with a smaller share, must each agree with cp_ring_attn_fwd on the
same inputs within the parity tolerance (2e-2 on the bf16 output, 1e-3 on the
LSE); where the share fits the scratch with the same launch grouping (four
ring steps per launch) they must be bit-identical.  A share too large for the
scratch is refused with CP_ERR_WORKSPACE before anything is enqueued.
"""
import ctypes
import math

import pytest
import torch

import workloads
import long_sequence_causal_cp_amd as cp
from long_sequence_causal_cp_amd import binding as cb
from gpu_helpers import LSE_TOL, OUT_TOL, gather, zigzag_tables

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


@pytest.fixture(scope="module", autouse=True)
def _lib():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    cp.load_library()


def _share(N, rank, L, D, H, B, seed):
    S = 2 * N * L
    Q, K, V = workloads.make_qkv_scaled((B, H, S, D), seed)
    q_tab, kv_tabs = zigzag_tables(N, rank, L)
    q = gather(Q, q_tab, DEV)
    ks = [gather(K, t, DEV) for t in kv_tabs]
    vs = [gather(V, t, DEV) for t in kv_tabs]
    return q, q_tab, ks, vs, kv_tabs, 1 / math.sqrt(D)


def _with_workspace(q, q_tab, ks, vs, kv_tabs, scale):
    B, H, Sq, D = q.shape
    out = torch.empty_like(q)
    lse = torch.empty((B, H, Sq), dtype=torch.float32, device=DEV)
    ws = torch.empty(cp.cp_ring_attn_workspace_bytes(B, H, ks[0].shape[2], D, Sq), dtype=torch.uint8, device=DEV)
    cp.cp_ring_attn_fwd(q, q_tab, ks, vs, kv_tabs, out, lse, scale, ws, copy_stream=torch.cuda.Stream())
    return out, lse


def test_noalloc_matches_workspace_entry_point_twice():
    # first call: 16 heads of 256-token chunks, cp=4 (the four-step grouping fits the scratch);
    # second call, smaller: 2 heads of 64-token chunks, cp=8, D=64
    cases = [(4, 1, 256, 128, 16, 1, 801), (8, 5, 64, 64, 2, 1, 802)]
    for N, rank, L, D, H, B, seed in cases:
        print("[case] no-alloc", "N", N, "rank", rank, "L", L, "D", D, "H", H, flush=True)
        q, q_tab, ks, vs, kv_tabs, scale = _share(N, rank, L, D, H, B, seed)
        ref_out, ref_lse = _with_workspace(q, q_tab, ks, vs, kv_tabs, scale)
        out = torch.full_like(q, float("nan"))
        lse = torch.full(ref_lse.shape, float("nan"), dtype=torch.float32, device=DEV)
        cp.cp_ring_attn_fwd_noalloc(q, q_tab, ks, vs, kv_tabs, out, lse, scale, copy_stream=torch.cuda.Stream())
        torch.cuda.synchronize()
        eo = float((out.float() - ref_out.float()).abs().max())
        el = float((lse - ref_lse).abs().max())
        print(f"  max|dout| = {eo:.3e}  max|dlse| = {el:.3e}", flush=True)
        assert torch.isfinite(out.float()).all() and torch.isfinite(lse).all()
        assert eo <= OUT_TOL and el <= LSE_TOL, (eo, el)
        assert torch.equal(out, ref_out) and torch.equal(lse, ref_lse)


def test_noalloc_refuses_a_share_beyond_its_scratch():
    lib = cb.load_library()
    cap = lib.cp_ring_attn_fwd_noalloc_max_bytes()
    assert cap == 64 << 20
    # 32 heads of 4096 local rows at D = 128: one ring step per launch already needs
    # 4 * 33.5 MB of slots + 67 MB of running output, beyond 64 MiB
    q_tab, kv_tabs = zigzag_tables(8, 0, 2048)
    T = cb.CpChunks * 8
    ptrs = (ctypes.c_void_p * 8)(*[0x7F0000000000 + (i + 4) * (1 << 30) for i in range(8)])
    st = lib.cp_ring_attn_fwd_noalloc(ctypes.c_void_p(0x7F0000000000), ctypes.byref(q_tab), ptrs, ptrs,
                                      T(*kv_tabs), 8, ctypes.c_void_p(0x7F0000000000 + (1 << 30)),
                                      ctypes.c_void_p(0x7F0000000000 + (2 << 30)), 1, 32, 128,
                                      ctypes.c_float(0.088), None, ctypes.c_void_p(0x1234))
    assert st == cb.CP_ERR_WORKSPACE
    assert "scratch" in cb.cp_last_error()
