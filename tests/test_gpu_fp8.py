"""GPU parity of the fp8 ring step (cp_attn_step_fwd_fp8) against the fp64 oracle.

Q, K and V are quantised to e4m3 with power-of-two per-tensor scales
(tests/fp8_helpers.py); the oracle consumes exactly the dequantised values.
A rank's share is computed as the ring's chain of steps: step 0 writes,
later steps merge, the last one also writes the bf16 output.

Tolerance: 1e-3 on the natural-log LSE, and on the output, per case, the
deviation from the exact result of a model of the kernel's own rounding on
the compared rows (fp8_helpers.lazy_model: the probabilities of each 64-key
tile against the maximum the kernel keeps lazily per wave, rounded to e4m3
before the PV product, normalised by the unrounded sum; launches merged by
log-sum-exp) times MODEL_MARGIN, plus 2^-8 of max |out| for the bf16 output.
The LSE is formed from fp32 sums of the unrounded probabilities of exact fp8
products, as in the bf16 path.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
import long_sequence_causal_cp_amd as cp
from fp8_helpers import dequantize, lazy_model_error, out_tolerance, quantize, ring_segments
from gpu_helpers import positions, zigzag_tables

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
LSE_TOL = 1e-3


@pytest.fixture(scope="module", autouse=True)
def _lib():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    cp.load_library()


def _gather(codes, table):
    idx = torch.from_numpy(positions(table))
    return codes.view(torch.uint8).index_select(2, idx).contiguous().view(torch.float8_e4m3fn)


def _ring_fp8(qc, kc, vc, sq, sk, sv, q_tab, kv_tabs, scale):
    q = _gather(qc, q_tab).to(DEV)
    B, H, Sq, D = q.shape
    o = torch.empty((B, H, Sq, D), dtype=torch.float32, device=DEV)
    lse = torch.empty((B, H, Sq), dtype=torch.float32, device=DEV)
    out = torch.empty((B, H, Sq, D), dtype=torch.bfloat16, device=DEV)
    for j, t in enumerate(kv_tabs):
        k = _gather(kc, t).to(DEV)
        vt = _gather(vc, t).view(torch.uint8).transpose(2, 3).contiguous().view(torch.float8_e4m3fn).to(DEV)
        last = j == len(kv_tabs) - 1
        cp.cp_attn_step_fwd_fp8(q, k, vt, o, lse, out if last else None, q_tab, t, scale, sq, sk, sv,
                                cp.CP_STEP_WRITE if j == 0 else cp.CP_STEP_MERGE)
    torch.cuda.synchronize()
    return out, lse


def _tables(kv_tabs):
    return [[(st, t.chunk_len) for st in t.starts()] for t in kv_tabs]


def _compare(out, lse, Qd, Kd, Vd, qpos, local, heads, scale, segments):
    """Max-abs output and LSE errors of the GPU at local rows `local` of the (batch, head) pairs `heads`
    against the oracle on dequantised values, and the output bound from the kernel's rounding model on
    those rows (key visit order `segments`)."""
    eo = el = em = amax = 0.0
    o_h = out.float().cpu().numpy()
    l_h = lse.cpu().numpy()
    for b, h in heads:
        err, ro, rl = lazy_model_error(Qd[b, h][qpos], qpos, local, Kd[b, h], Vd[b, h], segments, scale)
        ok = np.isfinite(rl)
        assert np.array_equal(np.isneginf(l_h[b, h, local]), ~ok), "rows without a visible key"
        assert not np.any(o_h[b, h, local][~ok]), "rows without a visible key must be 0"
        eo = max(eo, float(np.max(np.abs(o_h[b, h, local][ok] - ro[ok]))) if ok.any() else 0.0)
        el = max(el, float(np.max(np.abs(l_h[b, h, local][ok] - rl[ok]))) if ok.any() else 0.0)
        em = max(em, err)
        amax = max(amax, float(np.max(np.abs(ro[ok]))) if ok.any() else 0.0)
    tol = out_tolerance(em, amax)
    print(f"  max|dout| = {eo:.3e} (model {em:.3e}, ratio {eo / max(em, 1e-30):.2f}, bound {tol:.3e})  "
          f"max|dlse| = {el:.3e}", flush=True)
    return eo, el, tol


@pytest.mark.parametrize("name,H,ranks,rows", [("s8k_cp2", 2, (0, 1), None), ("s16k_cp4", 2, (1, 2), 256),
                                               ("s32k_cp8", 2, (0, 7), 128)])
def test_fp8_ring_share_matches_oracle(name, H, ranks, rows):
    w = workloads.get(name)
    Q, K, V = workloads.make_qkv(w, H=H)
    (qc, sq), (kc, sk), (vc, sv) = quantize(Q.float()), quantize(K.float()), quantize(V.float())
    Qd, Kd, Vd = (torch.from_numpy(dequantize(c, s)) for c, s in ((qc, sq), (kc, sk), (vc, sv)))
    for r in ranks:
        print("[case] fp8", w.describe(), "H", H, "rank", r, flush=True)
        q_tab, kv_tabs = zigzag_tables(w.cp, r, w.chunk_len)
        out, lse = _ring_fp8(qc, kc, vc, sq, sk, sv, q_tab, kv_tabs, w.scale)
        qpos = positions(q_tab)
        n = len(qpos)
        local = np.arange(n) if rows is None else np.unique(np.concatenate(
            [np.random.default_rng(r).choice(n, rows, replace=False), [0, 1, w.chunk_len - 1, w.chunk_len, n - 1]]))
        eo, el, tol = _compare(out, lse, Qd.numpy(), Kd.numpy(), Vd.numpy(), qpos, local, [(0, h) for h in range(H)],
                               w.scale, ring_segments(_tables(kv_tabs), grouped=False))
        assert eo <= tol and el <= LSE_TOL, (eo, tol, el)


@pytest.mark.parametrize("name,H,ranks,rows", [("s8k_cp2", 2, (0, 1), None), ("s32k_cp8", 2, (0, 7), 128)])
def test_fp8_ring_driver_matches_oracle(name, H, ranks, rows):
    """cp_ring_attn_fwd_fp8 (grouped launches, e4m3 staging copies on a side stream) against the oracle;
    the copies run in order on the launch stream give identical bits."""
    w = workloads.get(name)
    Q, K, V = workloads.make_qkv(w, H=H)
    (qc, sq), (kc, sk), (vc, sv) = quantize(Q.float()), quantize(K.float()), quantize(V.float())
    Qd, Kd, Vd = (torch.from_numpy(dequantize(c, s)) for c, s in ((qc, sq), (kc, sk), (vc, sv)))
    for r in ranks:
        print("[case] fp8 ring", w.describe(), "H", H, "rank", r, flush=True)
        q_tab, kv_tabs = zigzag_tables(w.cp, r, w.chunk_len)
        q = _gather(qc, q_tab).to(DEV)
        ks = [_gather(kc, t).to(DEV) for t in kv_tabs]
        vts = [_gather(vc, t).view(torch.uint8).transpose(2, 3).contiguous().view(torch.float8_e4m3fn).to(DEV)
               for t in kv_tabs]
        B, _, Sq, D = q.shape
        ws = torch.empty(cp.cp_ring_attn_fwd_fp8_workspace_bytes(B, H, ks[0].shape[2], D, Sq), dtype=torch.uint8,
                         device=DEV)
        res = []
        for in_order in (False, True):
            out = torch.empty((B, H, Sq, D), dtype=torch.bfloat16, device=DEV)
            lse = torch.empty((B, H, Sq), dtype=torch.float32, device=DEV)
            cs = torch.cuda.current_stream() if in_order else torch.cuda.Stream()
            cp.cp_ring_attn_fwd_fp8(q, q_tab, ks, vts, kv_tabs, out, lse, w.scale, sq, sk, sv, ws, copy_stream=cs)
            torch.cuda.synchronize()
            res.append((out, lse))
        assert torch.equal(res[0][0], res[1][0]) and torch.equal(res[0][1], res[1][1])
        out, lse = res[0]
        qpos = positions(q_tab)
        n = len(qpos)
        local = np.arange(n) if rows is None else np.unique(np.concatenate(
            [np.random.default_rng(r).choice(n, rows, replace=False), [0, 1, w.chunk_len - 1, w.chunk_len, n - 1]]))
        eo, el, tol = _compare(out, lse, Qd.numpy(), Kd.numpy(), Vd.numpy(), qpos, local, [(0, h) for h in range(H)],
                               w.scale, ring_segments(_tables(kv_tabs), grouped=True))
        assert eo <= tol and el <= LSE_TOL, (eo, tol, el)


@pytest.mark.parametrize("H", [2, 256])
@pytest.mark.parametrize("T", [1, 2, 3, 4, 5, 6, 7, 8])
def test_fp8_step_few_visible_tiles(T, H):
    """One fp8 step whose first 256 query rows see exactly T key tiles of 64: the kernel's pipeline has its
    own prologue and drain for one, two and three tiles, and an odd or even count of tiles after them.  The
    key chunk starts 8 positions past a tile boundary, so the causal limit crosses tiles mid-way and the
    first rows see no key at all (LSE -inf, output 0).  With 2 heads the grid is small and the launch takes
    128-row workgroups (the 128-row blocks then see 0 or T tiles); with 256 heads it takes 256-row ones."""
    D = 128
    q_start, q_len = 1000, 512
    kv_start = q_start + 256 - 64 * T + 8
    q_tab = cp.CpChunks.make([q_start], q_len)
    kv_tab = cp.CpChunks.make([kv_start], 64 * T)
    _check_fp8_step(q_tab, kv_tab, H, D, seed=500 + T)


def test_fp8_step_chunk_switching():
    """Three key chunks of one tile each: one in the past, one crossing the first row block's diagonal and
    one wholly in the future, so the tile cursor moves across chunks and skips the invisible one."""
    q_tab = cp.CpChunks.make([1000], 512)
    kv_tab = cp.CpChunks.make([0, 1100, 5000], 64)
    _check_fp8_step(q_tab, kv_tab, 2, 128, seed=520)


def _check_fp8_step(q_tab, kv_tab, H, D, seed):
    print("[case] fp8 step", q_tab, kv_tab, "H", H, flush=True)
    qpos, kpos = positions(q_tab), positions(kv_tab)
    S = int(max(qpos.max(), kpos.max())) + 1
    Q, K, V = workloads.make_qkv_scaled((1, H, S, D), seed)
    (qc, sq), (kc, sk), (vc, sv) = quantize(Q.float()), quantize(K.float()), quantize(V.float())
    Qd, Kd, Vd = (dequantize(c, s) for c, s in ((qc, sq), (kc, sk), (vc, sv)))
    q = _gather(qc, q_tab).to(DEV)
    k = _gather(kc, kv_tab).to(DEV)
    vt = _gather(vc, kv_tab).view(torch.uint8).transpose(2, 3).contiguous().view(torch.float8_e4m3fn).to(DEV)
    Sq = len(qpos)
    o = torch.empty((1, H, Sq, D), dtype=torch.float32, device=DEV)
    lse = torch.empty((1, H, Sq), dtype=torch.float32, device=DEV)
    out = torch.empty((1, H, Sq, D), dtype=torch.bfloat16, device=DEV)
    scale = 1.0 / np.sqrt(D)
    cp.cp_attn_step_fwd_fp8(q, k, vt, o, lse, out, q_tab, kv_tab, scale, sq, sk, sv, cp.CP_STEP_WRITE)
    torch.cuda.synchronize()
    segs = [positions(kv_tab)]
    eo, el, tol = _compare(out, lse, Qd, Kd, Vd, qpos, np.arange(Sq), [(0, h) for h in range(H)], scale, segs)
    assert eo <= tol and el <= LSE_TOL, (eo, tol, el)


@pytest.mark.parametrize("L", [512, 384])
@pytest.mark.parametrize("rank", [0, 1])
def test_fp8_ring_batch_heads_xcd_mapping(rank, L):
    """Batch 2 x 4 heads: B*H = 8 is a multiple of the eight XCDs, so the launches use the XCD-aware
    block-to-head mapping.  Chunks of 384 tokens (a multiple of 128, not of 256) take 128-row workgroups
    whatever the grid.  The ring driver against the oracle on every row of every (batch, head)."""
    B, H, D, N = 2, 4, 128, 2
    S = 2 * N * L
    Q, K, V = workloads.make_qkv_scaled((B, H, S, D), 610 + rank + L)
    (qc, sq), (kc, sk), (vc, sv) = quantize(Q.float()), quantize(K.float()), quantize(V.float())
    Qd, Kd, Vd = (dequantize(c, s) for c, s in ((qc, sq), (kc, sk), (vc, sv)))
    scale = 1.0 / np.sqrt(D)
    print("[case] fp8 ring B", B, "H", H, "N", N, "L", L, "rank", rank, flush=True)
    q_tab, kv_tabs = zigzag_tables(N, rank, L)
    q = _gather(qc, q_tab).to(DEV)
    ks = [_gather(kc, t).to(DEV) for t in kv_tabs]
    vts = [_gather(vc, t).view(torch.uint8).transpose(2, 3).contiguous().view(torch.float8_e4m3fn).to(DEV)
           for t in kv_tabs]
    Sq = q.shape[2]
    ws = torch.empty(cp.cp_ring_attn_fwd_fp8_workspace_bytes(B, H, ks[0].shape[2], D, Sq), dtype=torch.uint8,
                     device=DEV)
    out = torch.empty((B, H, Sq, D), dtype=torch.bfloat16, device=DEV)
    lse = torch.empty((B, H, Sq), dtype=torch.float32, device=DEV)
    cp.cp_ring_attn_fwd_fp8(q, q_tab, ks, vts, kv_tabs, out, lse, scale, sq, sk, sv, ws,
                            copy_stream=torch.cuda.Stream())
    torch.cuda.synchronize()
    qpos = positions(q_tab)
    eo, el, tol = _compare(out, lse, Qd, Kd, Vd, qpos, np.arange(Sq), [(b, h) for b in range(B) for h in range(H)],
                           scale, ring_segments(_tables(kv_tabs), grouped=True))
    assert eo <= tol and el <= LSE_TOL, (eo, tol, el)


@pytest.mark.parametrize("rank", [0, 1])
def test_fp8_ring_head_groups(rank):
    """Batch 2 x 32 heads, 2048-token chunks: 8 heads per XCD whose row blocks (8 per chunk) exceed what an
    XCD runs at once, so the launches take the XCD's heads in groups (4 of the 8 in a group launch).
    Sampled rows of (batch, head) pairs from different groups and XCDs against the oracle."""
    B, H, D, N, L = 2, 32, 128, 2, 2048
    S = 2 * N * L
    Q, K, V = workloads.make_qkv_scaled((B, H, S, D), 640 + rank)
    (qc, sq), (kc, sk), (vc, sv) = quantize(Q.float()), quantize(K.float()), quantize(V.float())
    heads = [(0, 0), (0, 13), (1, 7), (1, 30)]
    deq = {}
    for name, (c, s) in zip("QKV", ((qc, sq), (kc, sk), (vc, sv))):
        deq[name] = {bh: dequantize(c[bh[0]:bh[0] + 1, bh[1]:bh[1] + 1], s)[0, 0] for bh in heads}
    scale = 1.0 / np.sqrt(D)
    print("[case] fp8 ring head groups B", B, "H", H, "N", N, "L", L, "rank", rank, flush=True)
    q_tab, kv_tabs = zigzag_tables(N, rank, L)
    q = _gather(qc, q_tab).to(DEV)
    ks = [_gather(kc, t).to(DEV) for t in kv_tabs]
    vts = [_gather(vc, t).view(torch.uint8).transpose(2, 3).contiguous().view(torch.float8_e4m3fn).to(DEV)
           for t in kv_tabs]
    Sq = q.shape[2]
    ws = torch.empty(cp.cp_ring_attn_fwd_fp8_workspace_bytes(B, H, ks[0].shape[2], D, Sq), dtype=torch.uint8,
                     device=DEV)
    out = torch.empty((B, H, Sq, D), dtype=torch.bfloat16, device=DEV)
    lse = torch.empty((B, H, Sq), dtype=torch.float32, device=DEV)
    cp.cp_ring_attn_fwd_fp8(q, q_tab, ks, vts, kv_tabs, out, lse, scale, sq, sk, sv, ws,
                            copy_stream=torch.cuda.Stream())
    torch.cuda.synchronize()
    qpos = positions(q_tab)
    local = np.unique(np.concatenate([np.random.default_rng(rank).choice(Sq, 96, replace=False),
                                      [0, L - 1, L, Sq - 1]]))
    segs = ring_segments(_tables(kv_tabs), grouped=True)
    for bh in heads:
        e_o, e_l, tol = _compare(out[bh[0]:bh[0] + 1, bh[1]:bh[1] + 1], lse[bh[0]:bh[0] + 1, bh[1]:bh[1] + 1],
                                 deq["Q"][bh][None, None], deq["K"][bh][None, None], deq["V"][bh][None, None],
                                 qpos, local, [(0, 0)], scale, segs)
        assert e_o <= tol and e_l <= LSE_TOL, (bh, e_o, tol, e_l)


def test_fp8_ring_full_share_256_row_blocks():
    """The bench's configuration: rank 0 of the 32K cp=8 share with all 32 heads, where every launch's grid
    fills the chip with 256-row workgroups (the small-head cases above run 128-row ones).  Sampled rows of
    three heads against the oracle."""
    w = workloads.get("s32k_cp8")
    Q, K, V = workloads.make_qkv(w)
    (qc, sq), (kc, sk), (vc, sv) = quantize(Q.float()), quantize(K.float()), quantize(V.float())
    print("[case] fp8 ring", w.describe(), "rank 0, all heads", flush=True)
    q_tab, kv_tabs = zigzag_tables(w.cp, 0, w.chunk_len)
    q = _gather(qc, q_tab).to(DEV)
    ks = [_gather(kc, t).to(DEV) for t in kv_tabs]
    vts = [_gather(vc, t).view(torch.uint8).transpose(2, 3).contiguous().view(torch.float8_e4m3fn).to(DEV)
           for t in kv_tabs]
    B, H, Sq, D = q.shape
    ws = torch.empty(cp.cp_ring_attn_fwd_fp8_workspace_bytes(B, H, ks[0].shape[2], D, Sq), dtype=torch.uint8,
                     device=DEV)
    out = torch.empty((B, H, Sq, D), dtype=torch.bfloat16, device=DEV)
    lse = torch.empty((B, H, Sq), dtype=torch.float32, device=DEV)
    cp.cp_ring_attn_fwd_fp8(q, q_tab, ks, vts, kv_tabs, out, lse, w.scale, sq, sk, sv, ws,
                            copy_stream=torch.cuda.Stream())
    torch.cuda.synchronize()
    qpos = positions(q_tab)
    L = w.chunk_len
    local = np.unique(np.concatenate([np.random.default_rng(3).choice(len(qpos), 48, replace=False),
                                      [0, 1, L - 1, L, 2 * L - 1]]))
    heads = [(0, h) for h in (0, 17, 31)]
    Qd, Kd, Vd = ({bh: dequantize(c[bh], sc) for bh in heads} for c, sc in ((qc, sq), (kc, sk), (vc, sv)))
    eo, el, tol = _compare(out, lse, Qd, Kd, Vd, qpos, local, heads, w.scale,
                           ring_segments(_tables(kv_tabs), grouped=True))
    assert eo <= tol and el <= LSE_TOL, (eo, tol, el)
