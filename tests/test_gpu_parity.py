"""GPU parity: the HIP path against the fp64 oracle, through the C ABI.

Tolerances (max-abs over every compared element): bf16 output 2e-2, natural
LSE 1e-3, fp32 partial O 2e-2.  Inputs are the seeded bf16 workloads; the
oracle consumes the same bf16 values.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import workloads
import long_sequence_causal_cp_amd as cp
from gpu_helpers import (LSE_TOL, OUT_TOL, compare, gather, oracle_rows, positions, run_ring,
                         zigzag_tables)

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


@pytest.fixture(scope="module", autouse=True)
def _lib():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    cp.load_library()


def _announce(*a):
    print("[case]", *a, flush=True)


# ---------------------------------------------------------------- step level
@pytest.mark.parametrize("name", ["tiny", "s8k_cp2"])
def test_step_partials_and_merge_chain(name):
    w = workloads.get(name)
    Q, K, V = workloads.make_qkv(w)
    L, N = w.chunk_len, w.cp
    for r in range(N):
        _announce(name, "rank", r)
        q_tab, kv_tabs = zigzag_tables(N, r, L)
        qpos = positions(q_tab)
        q = gather(Q, q_tab, DEV)
        Sq = q.shape[2]
        o_run = torch.empty((w.B, w.H, Sq, w.D), dtype=torch.float32, device=DEV)
        lse_run = torch.empty((w.B, w.H, Sq), dtype=torch.float32, device=DEV)
        for j, t in enumerate(kv_tabs):
            k, v = gather(K, t, DEV), gather(V, t, DEV)
            # partial of this block alone
            o = torch.empty_like(o_run)
            lse = torch.empty_like(lse_run)
            out = torch.empty_like(q)
            cp.cp_attn_step_fwd(q, k, v, o, lse, out, q_tab, t, w.scale, cp.CP_STEP_WRITE)
            # running merge chain
            cp.cp_attn_step_fwd(q, k, v, o_run, lse_run, None, q_tab, t, w.scale,
                                cp.CP_STEP_WRITE if j == 0 else cp.CP_STEP_MERGE)
            torch.cuda.synchronize()
            kpos = positions(t)
            qf, kf, vf = (oracle.to_f64(x) for x in (q.cpu(), k.cpu(), v.cpu()))
            ro = np.empty((w.B, w.H, Sq, w.D))
            rl = np.empty((w.B, w.H, Sq))
            for b in range(w.B):
                for h in range(w.H):
                    ro[b, h], rl[b, h] = oracle.masked_attention(qf[b, h], qpos, kf[b, h], vf[b, h], kpos, w.scale)
            og, lg, outg = o.cpu().numpy(), lse.cpu().numpy(), out.float().cpu().numpy()
            empty = np.isneginf(rl)
            assert np.array_equal(np.isneginf(lg), empty)
            assert np.all(og[empty] == 0) and np.all(outg[empty] == 0)
            full = ~empty
            if full.any():
                assert np.max(np.abs(og[full] - ro[full])) <= OUT_TOL
                assert np.max(np.abs(outg[full] - ro[full])) <= OUT_TOL
                assert np.max(np.abs(lg[full] - rl[full])) <= LSE_TOL
        ro, rl = oracle_rows(Q, K, V, np.broadcast_to(qpos, (w.B, w.H, Sq)), w.scale)
        eo = np.max(np.abs(o_run.cpu().numpy() - ro))
        el = np.max(np.abs(lse_run.cpu().numpy() - rl))
        assert eo <= OUT_TOL and el <= LSE_TOL, (eo, el)


@pytest.mark.parametrize("D,Sq", [(128, 4096), (64, 333), (12, 50), (1028, 7)])
def test_merge_kernel(D, Sq):
    _announce("merge", D, Sq)
    g = torch.Generator().manual_seed(D * 1000 + Sq)
    B, H = 2, 3
    oa = torch.randn(B, H, Sq, D, generator=g)
    ob = torch.randn(B, H, Sq, D, generator=g)
    la = torch.randn(B, H, Sq, generator=g) * 4
    lb = torch.randn(B, H, Sq, generator=g) * 4
    la[0, 0, ::3] = -math.inf
    lb[0, 0, ::5] = -math.inf
    lb[1, 2, ::2] = -math.inf
    oa[la == -math.inf] = 0
    ob[lb == -math.inf] = 0
    ro, rl = oracle.lse_merge(oa.double().numpy(), la.double().numpy(), ob.double().numpy(), lb.double().numpy())
    o_acc, l_acc = oa.to(DEV), la.to(DEV)
    out = torch.empty(B, H, Sq, D, dtype=torch.bfloat16, device=DEV)
    cp.cp_attn_merge(o_acc, l_acc, ob.to(DEV), lb.to(DEV), out)
    torch.cuda.synchronize()
    lg = l_acc.cpu().numpy()
    assert np.array_equal(np.isneginf(lg), np.isneginf(rl))
    fin = ~np.isneginf(rl)
    assert np.max(np.abs(lg[fin] - rl[fin])) <= 1e-5
    assert np.max(np.abs(o_acc.cpu().numpy() - ro)) <= 1e-5
    assert np.max(np.abs(out.float().cpu().numpy() - ro)) <= 2e-2


# ---------------------------------------------------------------- full ring
RING_CASES = [
    ("tiny", r, None) for r in range(2)
] + [
    ("s8k_cp2", r, None) for r in range(2)
] + [
    ("s16k_cp4", 0, None)    # rank 0: every row of every head
] + [
    ("s16k_cp4", r, 256) for r in range(1, 4)
] + [
    ("s32k_cp8", 0, None), ("s32k_cp8", 7, 128),
    ("s64k_cp16", 0, 512),
]

_QKV = {}


def _qkv(name):
    if name not in _QKV:
        _QKV.clear()
        _QKV[name] = workloads.make_qkv(workloads.get(name))
    return _QKV[name]


@pytest.mark.parametrize("name,rank,rows", RING_CASES)
def test_ring_parity(name, rank, rows):
    w = workloads.get(name)
    _announce("ring", w.describe(), "rank", rank, "rows/head", rows or "all")
    Q, K, V = _qkv(name)
    q_tab, kv_tabs = zigzag_tables(w.cp, rank, w.chunk_len)
    out, lse = run_ring(Q, K, V, q_tab, kv_tabs, w.scale, DEV)
    torch.cuda.synchronize()
    qpos = positions(q_tab)
    if rows is None:
        local = np.broadcast_to(np.arange(len(qpos)), (w.B, w.H, len(qpos))).copy()
    else:
        local = workloads.sample_local_rows(w, n_rows=rows)
    ro, rl = oracle_rows(Q, K, V, qpos[local], w.scale)
    eo, el = compare(out, lse, ro, rl, local)
    print(f"  max|dout| = {eo:.3e}  max|dlse| = {el:.3e}", flush=True)
    assert eo <= OUT_TOL and el <= LSE_TOL, (eo, el)


# ---------------------------------------------------------------- invariants
def _small(name="s8k_cp2", H=4, S=None):
    w = workloads.get(name)
    return w, (w.B, H, S or w.S, w.D)


def test_ring_q_zero_closed_form():
    w, shape = _small(H=2)
    _, K, V = workloads.make_qkv(w, H=2)
    Q = torch.zeros(shape, dtype=torch.bfloat16)
    for r in range(w.cp):
        q_tab, kv_tabs = zigzag_tables(w.cp, r, w.chunk_len)
        out, lse = run_ring(Q, K, V, q_tab, kv_tabs, w.scale, DEV)
        torch.cuda.synchronize()
        pos = positions(q_tab)
        lg = lse.cpu().numpy()
        assert np.max(np.abs(lg - np.log(pos + 1.0))) <= LSE_TOL
        mean = np.cumsum(oracle.to_f64(V), axis=2) / np.arange(1, w.S + 1)[:, None]
        assert np.max(np.abs(out.float().cpu().numpy() - mean[:, :, pos])) <= OUT_TOL


def test_ring_constant_v_and_first_token():
    w, shape = _small(H=2)
    Q, K, _ = workloads.make_qkv_scaled(shape, 77, q_scale=3.0, k_scale=3.0)
    c = torch.linspace(-2, 2, w.D).to(torch.bfloat16)
    V = c.expand(shape).contiguous()
    q_tab, kv_tabs = zigzag_tables(w.cp, 0, w.chunk_len)
    out, lse = run_ring(Q, K, V, q_tab, kv_tabs, w.scale, DEV)
    torch.cuda.synchronize()
    assert np.max(np.abs(out.float().cpu().numpy() - c.float().numpy())) <= 1e-2
    # position 0 is local row 0 of rank 0: it sees only itself
    q0, k0 = oracle.to_f64(Q[:, :, 0]), oracle.to_f64(K[:, :, 0])
    assert np.max(np.abs(lse[:, :, 0].cpu().numpy() - (q0 * k0).sum(-1) * w.scale)) <= LSE_TOL


@pytest.mark.parametrize("qs,ks", [(1.0, 1.0), (3.0, 3.0), (0.2, 6.0)])
def test_ring_peaked_and_flat_softmax(qs, ks):
    """Peaked rows return nearly a single value row, whose magnitude reaches about 5 for N(0, 1) values;
    the output is compared beyond its own bf16 rounding (half an ulp, up to 2^-8 of the value)."""
    w, shape = _small(H=4)
    Q, K, V = workloads.make_qkv_scaled(shape, 11, q_scale=qs, k_scale=ks)
    for r in range(w.cp):
        q_tab, kv_tabs = zigzag_tables(w.cp, r, w.chunk_len)
        out, lse = run_ring(Q, K, V, q_tab, kv_tabs, w.scale, DEV)
        torch.cuda.synchronize()
        pos = positions(q_tab)
        ro, rl = oracle_rows(Q, K, V, np.broadcast_to(pos, (w.B, 4, len(pos))), w.scale)
        eo, el = compare(out, lse, ro, rl, output_rounding=True)
        print(f"  rank {r}: max(|dout| - 2^-8 |out|) = {eo:.3e}  max|dlse| = {el:.3e}", flush=True)
        assert eo <= OUT_TOL and el <= LSE_TOL, (qs, ks, r, eo, el)


def test_ring_needle_keys():
    """Keys equal to 4x a later query make single keys dominate their rows (output compared beyond its
    own bf16 rounding, as for peaked rows)."""
    w, shape = _small(H=2)
    Q, K, V = workloads.make_qkv_scaled(shape, 5)
    rng = np.random.default_rng(0)
    for i in rng.choice(w.S - 1, size=64, replace=False):
        j = int(rng.integers(i + 1, w.S))
        K[:, :, i] = (Q[:, :, j].float() * 4).to(torch.bfloat16)
    q_tab, kv_tabs = zigzag_tables(w.cp, 1, w.chunk_len)
    out, lse = run_ring(Q, K, V, q_tab, kv_tabs, w.scale, DEV)
    torch.cuda.synchronize()
    pos = positions(q_tab)
    ro, rl = oracle_rows(Q, K, V, np.broadcast_to(pos, (w.B, 2, len(pos))), w.scale)
    eo, el = compare(out, lse, ro, rl, output_rounding=True)
    assert eo <= OUT_TOL and el <= LSE_TOL


def test_contiguous_and_permuted_tables():
    """The ABI takes any chunk tables: contiguous sharding and a permuted ring order."""
    name = "s16k_cp4"
    w = workloads.get(name)
    H = 2
    Q, K, V = workloads.make_qkv(w, H=H)
    N = w.cp
    n = w.S // N
    # contiguous: rank r holds [r n, (r+1) n) as one chunk; step j gets rank (r-j) mod N
    for r in (0, N - 1):
        q_tab = cp.CpChunks.make([r * n], n)
        kv_tabs = [cp.CpChunks.make([((r - j) % N) * n], n) for j in range(N)]
        out, lse = run_ring(Q, K, V, q_tab, kv_tabs, w.scale, DEV)
        torch.cuda.synchronize()
        pos = positions(q_tab)
        local = np.stack([np.sort(np.random.default_rng(r).choice(n, 256, replace=False))] * H)[None]
        ro, rl = oracle_rows(Q, K, V, pos[local], w.scale)
        eo, el = compare(out, lse, ro, rl, local)
        assert eo <= OUT_TOL and el <= LSE_TOL, ("contiguous", r, eo, el)
    # zigzag with the steps after the first in reverse order: same result
    q_tab, kv_tabs = zigzag_tables(N, 2, w.chunk_len)
    out1, lse1 = run_ring(Q, K, V, q_tab, kv_tabs, w.scale, DEV)
    out2, lse2 = run_ring(Q, K, V, q_tab, [kv_tabs[0]] + kv_tabs[1:][::-1], w.scale, DEV)
    torch.cuda.synchronize()
    assert (out1.float() - out2.float()).abs().max().item() <= 2e-2
    assert (lse1 - lse2).abs().max().item() <= 1e-4


def test_many_chunks_one_step_per_launch():
    """Five interleaved chunks per rank and step: two steps' chunks exceed the
    launch's chunk table, so the ring driver launches one step at a time."""
    N, H, D, L, per_rank = 3, 2, 128, 256, 5
    S = N * per_rank * L
    Q, K, V = workloads.make_qkv_scaled((1, H, S, D), 97)
    tabs = [cp.CpChunks.make([(i * N + r) * L for i in range(per_rank)], L) for r in range(N)]
    for r in range(N):
        q_tab = tabs[r]
        kv_tabs = [tabs[(r - j) % N] for j in range(N)]
        _announce("many chunks", r)
        out, lse = run_ring(Q, K, V, q_tab, kv_tabs, 1 / math.sqrt(D), DEV)
        torch.cuda.synchronize()
        pos = positions(q_tab)
        ro, rl = oracle_rows(Q, K, V, np.broadcast_to(pos, (1, H, len(pos))), 1 / math.sqrt(D))
        eo, el = compare(out, lse, ro, rl)
        assert eo <= OUT_TOL and el <= LSE_TOL, (r, eo, el)


@pytest.mark.parametrize("D,L", [(128, 64), (64, 128), (64, 64), (128, 192)])
def test_kernel_variants(D, L):
    """All four compiled step-kernel variants (D in {64,128}, 64- and 128-row blocks)."""
    _announce("variant", D, L)
    N, H = 3, 2
    S = 2 * N * L
    Q, K, V = workloads.make_qkv_scaled((1, H, S, D), D + L)
    for r in range(N):
        q_tab, kv_tabs = zigzag_tables(N, r, L)
        out, lse = run_ring(Q, K, V, q_tab, kv_tabs, 1 / math.sqrt(D), DEV)
        torch.cuda.synchronize()
        pos = positions(q_tab)
        ro, rl = oracle_rows(Q, K, V, np.broadcast_to(pos, (1, H, len(pos))), 1 / math.sqrt(D))
        eo, el = compare(out, lse, ro, rl)
        assert eo <= OUT_TOL and el <= LSE_TOL, (r, eo, el)


def test_full_sequence_single_step():
    """All-gather variant: the whole sequence as one query block against all keys in one step."""
    w = workloads.get("s8k_cp2")
    H = 2
    Q, K, V = workloads.make_qkv(w, H=H)
    t = cp.CpChunks.make([0], w.S)
    q, k, v = (x.contiguous().to(DEV) for x in (Q, K, V))
    o = torch.empty(q.shape, dtype=torch.float32, device=DEV)
    lse = torch.empty(q.shape[:-1], dtype=torch.float32, device=DEV)
    out = torch.empty_like(q)
    cp.cp_attn_step_fwd(q, k, v, o, lse, out, t, t, w.scale, cp.CP_STEP_WRITE)
    torch.cuda.synchronize()
    rows = np.sort(np.random.default_rng(3).choice(w.S, 512, replace=False))
    ro, rl = oracle_rows(Q, K, V, np.broadcast_to(rows, (1, H, 512)), w.scale)
    eo, el = compare(out, lse, ro, rl, np.broadcast_to(rows, (1, H, 512)).copy())
    assert eo <= OUT_TOL and el <= LSE_TOL


@pytest.mark.parametrize("name,rank,H,rows", [("s16k_cp4", 2, 4, 256), ("s32k_cp8", 0, 2, 128)])
def test_allgather_rank_share(name, rank, H, rows):
    """All-gather form of context parallelism: the rank's zigzag queries against the gathered keys of the
    whole sequence (one K/V chunk in natural order) in a single step; matches the oracle and agrees with the
    ring result within the tolerance."""
    w = workloads.get(name)
    _announce("all-gather", w.describe(), "H", H, "rank", rank)
    Q, K, V = workloads.make_qkv(w, H=H)
    q_tab, kv_tabs = zigzag_tables(w.cp, rank, w.chunk_len)
    q = gather(Q, q_tab, DEV)
    k, v = K.contiguous().to(DEV), V.contiguous().to(DEV)
    full = cp.CpChunks.make([0], w.S)
    o = torch.empty(q.shape, dtype=torch.float32, device=DEV)
    lse = torch.empty(q.shape[:-1], dtype=torch.float32, device=DEV)
    out = torch.empty_like(q)
    cp.cp_attn_step_fwd(q, k, v, o, lse, out, q_tab, full, w.scale, cp.CP_STEP_WRITE)
    ring_out, ring_lse = run_ring(Q, K, V, q_tab, kv_tabs, w.scale, DEV)
    torch.cuda.synchronize()
    qpos = positions(q_tab)
    local = np.sort(np.stack([np.random.default_rng(7 + h).choice(len(qpos), rows, replace=False)
                              for h in range(H)]), axis=1)[None]
    local[..., 0] = 0                      # first row of the early chunk: a single visible key
    ro, rl = oracle_rows(Q, K, V, qpos[local], w.scale)
    eo, el = compare(out, lse, ro, rl, local)
    print(f"  max|dout| = {eo:.3e}  max|dlse| = {el:.3e}", flush=True)
    assert eo <= OUT_TOL and el <= LSE_TOL, (eo, el)
    assert float((out.float() - ring_out.float()).abs().max()) <= 2 * OUT_TOL
    assert float((lse - ring_lse).abs().max()) <= 2 * LSE_TOL


@pytest.mark.parametrize("N,rank", [(64, 0), (64, 63), (1, 0)])
def test_ring_extreme_step_counts(N, rank):
    """The most ring steps the driver takes (64, in 17 launches) and a ring of one rank (its own block, the
    whole sequence), against the oracle on every local row."""
    L, D, H = 64, 64, 2
    S = 2 * N * L
    _announce("ring extremes", "N", N, "rank", rank)
    Q, K, V = workloads.make_qkv_scaled((1, H, S, D), 90 + N)
    q_tab, kv_tabs = zigzag_tables(N, rank, L)
    out, lse = run_ring(Q, K, V, q_tab, kv_tabs, 1 / math.sqrt(D), DEV)
    torch.cuda.synchronize()
    qpos = positions(q_tab)
    local = np.broadcast_to(np.arange(len(qpos)), (1, H, len(qpos))).copy()
    ro, rl = oracle_rows(Q, K, V, qpos[local], 1 / math.sqrt(D))
    eo, el = compare(out, lse, ro, rl, local)
    print(f"  max|dout| = {eo:.3e}  max|dlse| = {el:.3e}", flush=True)
    assert eo <= OUT_TOL and el <= LSE_TOL, (eo, el)


@pytest.mark.parametrize("H,L,D,kernels", [
    (16, 2048, 128, ("step_kernel_128<128>", "step_kernel_256s<128>")),
    (12, 256, 128, ("step_kernel_128s<128>", "step_kernel_256s<128>")),
    (3, 128, 128, ("step_kernel_128s<128>", "step_kernel_128s<128>")),
    (8, 512, 64, ("step_kernel_128s<64>", "step_kernel_256s<64>")),
])
def test_ring_key_split(H, L, D, kernels):
    """Launches that would leave compute units idle split each row block's key tiles over two workgroups
    that merge by log-sum-exp: 256-row blocks when the launch holds no diagonal chunk pair (the 8K cp=2
    share's ring step 1 on rank 0: 16 heads with one query chunk active), 128-row blocks otherwise.
    12 and 3 heads are not multiples of the 8 XCDs (pairs on different XCDs).  Every rank against the
    oracle on every row; rank 0's two launches ran the kernels named, and two more runs of rank 0 give the
    same bits (the merge does not depend on which half arrives last)."""
    N = 2
    S = 2 * N * L
    Q, K, V = workloads.make_qkv_scaled((1, H, S, D), 900 + H)
    for r in range(N):
        _announce("key split", "H", H, "L", L, "D", D, "rank", r)
        q_tab, kv_tabs = zigzag_tables(N, r, L)
        cp.cp_profile_enable(True)
        out, lse = run_ring(Q, K, V, q_tab, kv_tabs, 1 / math.sqrt(D), DEV)
        torch.cuda.synchronize()
        names = [n for _, n in cp.cp_profile_read_named()]
        cp.cp_profile_enable(False)
        if r == 0:
            assert tuple(names[:2]) == kernels, names
            # the halves merge in their own order whichever arrives last: repeated runs give the same bits
            for _ in range(2):
                out2, lse2 = run_ring(Q, K, V, q_tab, kv_tabs, 1 / math.sqrt(D), DEV)
                torch.cuda.synchronize()
                assert torch.equal(out2, out) and torch.equal(lse2, lse)
        qpos = positions(q_tab)
        local = np.broadcast_to(np.arange(len(qpos)), (1, H, len(qpos))).copy()
        ro, rl = oracle_rows(Q, K, V, qpos[local], 1 / math.sqrt(D))
        eo, el = compare(out, lse, ro, rl, local)
        print(f"  {names}  max|dout| = {eo:.3e}  max|dlse| = {el:.3e}", flush=True)
        assert eo <= OUT_TOL and el <= LSE_TOL, (eo, el)
