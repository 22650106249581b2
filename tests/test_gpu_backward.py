"""GPU parity of the backward ring step: the HIP kernels against the fp64 oracle.

The GPU gets what a training step would hand it: the forward's bf16 output
(here the oracle's, rounded to bf16) and its fp32 LSE; Delta comes from the
library's own delta kernel.  The oracle differentiates the exact fp64 forward.

Tolerance (per gradient tensor, max-abs over every element):
    max |g_gpu - g_oracle| <= GRAD_TOL * max |g_oracle|,   GRAD_TOL = 2e-2.
An emulation of the kernels' arithmetic (fp32 accumulation; P and dS rounded
to bf16 before their products; Delta from the bf16 output) against the oracle
gives at most 3.4e-3 on the seeded workloads and 7.5e-3 on peaked scores
(Q, K scaled by 3); the bound leaves a factor of about 3 over the worst.
Rows and keys that no visible pair reaches must be exactly 0 (write mode) or
unchanged (accumulate mode).  Delta itself is checked against an fp64 dot
product of the same bf16 values.
"""
import math
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

import oracle
import workloads
import long_sequence_causal_cp_amd as cp
from gpu_helpers import gather, positions, threads, zigzag_tables

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
GRAD_TOL = 2e-2


@pytest.fixture(scope="module", autouse=True)
def _lib():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    cp.load_library()


def _announce(*a):
    print("[case]", *a, flush=True)


def _per_head(B, H, fn):
    with ThreadPoolExecutor(threads()) as ex:
        return list(ex.map(lambda bh: fn(*divmod(bh, H)), range(B * H)))


def forward_rows(Q, K, V, qpos, scale):
    """Oracle out [B,H,n,D], lse [B,H,n] of full-sequence causal attention at positions qpos."""
    B, H = Q.shape[:2]
    kmax = int(qpos.max()) + 1
    kpos = np.arange(kmax)

    def one(b, h):
        return oracle.masked_attention(oracle.to_f64(Q[b, h])[qpos], qpos, oracle.to_f64(K[b, h, :kmax]),
                                       oracle.to_f64(V[b, h, :kmax]), kpos, scale)
    res = _per_head(B, H, one)
    out = np.stack([r[0] for r in res]).reshape(B, H, len(qpos), -1)
    lse = np.stack([r[1] for r in res]).reshape(B, H, len(qpos))
    return out, lse


def oracle_step_grads(Q, K, V, dO, qpos, kpos, out, lse, scale):
    """Oracle (dq_part [B,H,n,D], dk [B,H,m,D], dv [B,H,m,D]) of the block at kpos for queries at qpos."""
    B, H = Q.shape[:2]

    def one(b, h):
        f = lambda X, p: oracle.to_f64(X[b, h])[p]
        return oracle.masked_attention_grad(f(Q, qpos), qpos, f(K, kpos), f(V, kpos), kpos, f(dO, qpos),
                                            out[b, h], lse[b, h], scale)
    res = _per_head(B, H, one)
    return tuple(np.stack([r[i] for r in res]).reshape(B, H, *res[0][i].shape) for i in range(3))


def device_inputs(out, lse):
    """The forward results as the GPU receives them: bf16 out, fp32 LSE."""
    o = torch.from_numpy(out).to(torch.float32).to(torch.bfloat16).contiguous().to(DEV)
    l = torch.from_numpy(lse).to(torch.float32).contiguous().to(DEV)
    return o, l


def gpu_delta(out_dev, do_dev):
    B, H, Sq, _ = out_dev.shape
    delta = torch.empty((B, H, Sq), dtype=torch.float32, device=DEV)
    cp.cp_attn_bwd_delta(out_dev, do_dev, delta)
    return delta


def assert_grad(name, g, ref):
    g = g.cpu().numpy().astype(np.float64)
    assert np.isfinite(g).all(), name
    scale = float(np.max(np.abs(ref))) if ref.size else 0.0
    err = float(np.max(np.abs(g - ref))) if ref.size else 0.0
    print(f"  {name}: max|ref| = {scale:.3e}  max|err| = {err:.3e}  rel = {err / max(scale, 1e-30):.2e}",
          flush=True)
    assert err <= GRAD_TOL * scale + 1e-6, (name, err, scale)


def no_pair_rows(qpos, kpos):
    """Boolean masks: queries with no visible key in the block, keys with no query seeing them."""
    return qpos < kpos.min(), kpos > qpos.max()


def run_step(q, k, v, do, lse, delta, q_tab, kv_tab, scale, mode=0, dq=None, dk=None, dv=None):
    B, H, Sq, D = q.shape
    Skv = k.shape[2]
    dq = torch.empty((B, H, Sq, D), dtype=torch.float32, device=DEV) if dq is None else dq
    dk = torch.empty((B, H, Skv, D), dtype=torch.float32, device=DEV) if dk is None else dk
    dv = torch.empty((B, H, Skv, D), dtype=torch.float32, device=DEV) if dv is None else dv
    cp.cp_attn_step_bwd(q, k, v, do, lse, delta, dq, dk, dv, q_tab, kv_tab, scale, mode)
    return dq, dk, dv


def check_step(Q, K, V, dO, q_tab, kv_tab, scale, fwd=None):
    """One step's backward on the GPU vs the oracle; returns the GPU results."""
    qpos, kpos = positions(q_tab), positions(kv_tab)
    out, lse = fwd if fwd is not None else forward_rows(Q, K, V, qpos, scale)
    q = gather(Q, q_tab, DEV)
    do = gather(dO, q_tab, DEV)
    k, v = gather(K, kv_tab, DEV), gather(V, kv_tab, DEV)
    out_d, lse_d = device_inputs(out, lse)
    delta = gpu_delta(out_d, do)
    dq, dk, dv = run_step(q, k, v, do, lse_d, delta, q_tab, kv_tab, scale)
    torch.cuda.synchronize()
    rq, rk, rv = oracle_step_grads(Q, K, V, dO, qpos, kpos, out, lse, scale)
    assert_grad("dq", dq, rq)
    assert_grad("dk", dk, rk)
    assert_grad("dv", dv, rv)
    q_none, k_none = no_pair_rows(qpos, kpos)
    assert np.all(dq.cpu().numpy()[:, :, q_none] == 0)
    assert np.all(dk.cpu().numpy()[:, :, k_none] == 0) and np.all(dv.cpu().numpy()[:, :, k_none] == 0)
    return dq, dk, dv


# ---------------------------------------------------------------- delta
@pytest.mark.parametrize("D,B,H,Sq", [(64, 1, 2, 256), (128, 2, 3, 333), (128, 1, 1, 1), (64, 1, 1, 0)])
def test_delta_kernel(D, B, H, Sq):
    _announce("delta", D, B, H, Sq)
    gen = torch.Generator().manual_seed(D + Sq)
    o = torch.randn(B, H, Sq, D, generator=gen).to(torch.bfloat16)
    d = torch.randn(B, H, Sq, D, generator=gen).to(torch.bfloat16)
    delta = gpu_delta(o.to(DEV), d.to(DEV))
    torch.cuda.synchronize()
    of, df = oracle.to_f64(o), oracle.to_f64(d)
    ref = np.sum(of * df, axis=-1)
    bound = 1e-5 * np.sum(np.abs(of * df), axis=-1) + 1e-6
    assert np.all(np.abs(delta.cpu().numpy() - ref) <= bound)


# ---------------------------------------------------------------- ring steps
@pytest.mark.parametrize("name,H,ranks,steps", [
    ("tiny", 2, None, None),
    ("s8k_cp2", 4, None, None),
    ("s32k_cp8", 2, (0, 7), (0, 1, 7)),
])
def test_step_bwd_zigzag(name, H, ranks, steps):
    w = workloads.get(name)
    Q, K, V = workloads.make_qkv(w, H=H)
    dO = workloads.make_grad_out(w, H=H)
    for r in (ranks or range(w.cp)):
        q_tab, kv_tabs = zigzag_tables(w.cp, r, w.chunk_len)
        fwd = forward_rows(Q, K, V, positions(q_tab), w.scale)
        for j in (steps or range(w.cp)):
            _announce("step bwd", w.describe(), "H", H, "rank", r, "step", j)
            check_step(Q, K, V, dO, q_tab, kv_tabs[j], w.scale, fwd=fwd)


@pytest.mark.parametrize("D,L,B,H", [(128, 64, 1, 2), (64, 128, 2, 3), (64, 64, 1, 8), (128, 192, 1, 2),
                                     (128, 256, 2, 4), (64, 256, 1, 2)])
def test_bwd_kernel_variants(D, L, B, H):
    """The dq kernel at 64 and 128 rows and the dk/dv kernel at 64, 128 and 256 keys (256 only off the
    diagonal step), both head-to-XCD mappings.  With B*H*Sq/256 at most the compute-unit count the launch
    takes 128-row dq blocks for every 256-multiple chunk, and 128-key dk/dv blocks on diagonal steps; the
    256-row dq and diagonal 256-key dk/dv blocks are covered by test_bwd_grids_above_cu_count."""
    N = 3
    S = 2 * N * L
    Q, K, V = workloads.make_qkv_scaled((B, H, S, D), 3 * D + L)
    gen = torch.Generator().manual_seed(D * L)
    dO = torch.randn(B, H, S, D, generator=gen).to(torch.bfloat16)
    for r in (0, N - 1):
        q_tab, kv_tabs = zigzag_tables(N, r, L)
        fwd = forward_rows(Q, K, V, positions(q_tab), 1 / math.sqrt(D))
        for j in range(N):
            _announce("variant", D, L, B, H, "rank", r, "step", j)
            check_step(Q, K, V, dO, q_tab, kv_tabs[j], 1 / math.sqrt(D), fwd=fwd)


def test_bwd_grids_above_cu_count():
    """72 heads of 1024 local rows: B*H*Sq/256 = 288 exceeds the 256 compute units, so the launches take
    256-row dq blocks and, on the diagonal step 0, 256-key dk/dv blocks (the forms of the 32K cp=8
    share's backward); every rank and step against the oracle on all heads."""
    N, L, D, H = 2, 512, 128, 72
    S = 2 * N * L
    assert H * 2 * L // 256 > torch.cuda.get_device_properties(DEV).multi_processor_count
    Q, K, V = workloads.make_qkv_scaled((1, H, S, D), 909)
    gen = torch.Generator().manual_seed(910)
    dO = torch.randn(1, H, S, D, generator=gen).to(torch.bfloat16)
    for r in range(N):
        q_tab, kv_tabs = zigzag_tables(N, r, L)
        fwd = forward_rows(Q, K, V, positions(q_tab), 1 / math.sqrt(D))
        for j in range(N):
            _announce("grid above CUs", "H", H, "rank", r, "step", j)
            cp.cp_profile_enable(True)
            check_step(Q, K, V, dO, q_tab, kv_tabs[j], 1 / math.sqrt(D), fwd=fwd)
            names = [n for _, n in cp.cp_profile_read_named()]
            cp.cp_profile_enable(False)
            assert names == ["bwd_dq_kernel<128, 8>", "bwd_dkdv_kernel<128, 8>"], names


@pytest.mark.parametrize("qs,ks", [(3.0, 3.0), (0.2, 6.0)])
def test_bwd_peaked_and_flat(qs, ks):
    w = workloads.get("s8k_cp2")
    H, S = 2, 4096
    Q, K, V = workloads.make_qkv_scaled((1, H, S, w.D), 11, qs, ks, 1.0)
    dO = workloads.make_grad_out(w, H=H, S=S)
    q_tab, kv_tabs = zigzag_tables(2, 0, S // 4)
    fwd = forward_rows(Q, K, V, positions(q_tab), w.scale)
    for j in range(2):
        _announce("peaked", qs, ks, "step", j)
        check_step(Q, K, V, dO, q_tab, kv_tabs[j], w.scale, fwd=fwd)


def test_bwd_general_tables_and_empty_rows():
    """Several chunks in arbitrary order, a K/V chunk after every query, and rows whose LSE is -inf."""
    D, L, H = 128, 128, 2
    S = 16 * L
    Q, K, V = workloads.make_qkv_scaled((1, H, S, D), 5)
    gen = torch.Generator().manual_seed(6)
    dO = torch.randn(1, H, S, D, generator=gen).to(torch.bfloat16)
    q_tab = cp.CpChunks.make([9 * L, 2 * L, 5 * L], L)
    kv_tab = cp.CpChunks.make([4 * L, 12 * L, 0, 8 * L], L)
    qpos = positions(q_tab)
    out, lse = forward_rows(Q, K, V, qpos, 1 / math.sqrt(D))
    _announce("general tables")
    check_step(Q, K, V, dO, q_tab, kv_tab, 1 / math.sqrt(D), fwd=(out, lse))
    lse2 = lse.copy()
    lse2[:, :, 100:140] = -np.inf   # rows treated as having no visible key
    _announce("general tables, empty rows")
    dq, _, _ = check_step(Q, K, V, dO, q_tab, kv_tab, 1 / math.sqrt(D), fwd=(out, lse2))
    assert torch.all(dq[:, :, 100:140] == 0)


def test_bwd_accumulate_and_no_visible_pairs():
    """Accumulate mode adds exactly the write-mode result; a block after every query leaves outputs unchanged."""
    D, L, H = 64, 128, 2
    S = 8 * L
    Q, K, V = workloads.make_qkv_scaled((1, H, S, D), 8)
    gen = torch.Generator().manual_seed(9)
    dO = torch.randn(1, H, S, D, generator=gen).to(torch.bfloat16)
    q_tab = cp.CpChunks.make([L, 6 * L], L)
    kv_tab = cp.CpChunks.make([0, 3 * L], L)
    out, lse = forward_rows(Q, K, V, positions(q_tab), 1 / math.sqrt(D))
    q, do = gather(Q, q_tab, DEV), gather(dO, q_tab, DEV)
    k, v = gather(K, kv_tab, DEV), gather(V, kv_tab, DEV)
    out_d, lse_d = device_inputs(out, lse)
    delta = gpu_delta(out_d, do)
    dq, dk, dv = run_step(q, k, v, do, lse_d, delta, q_tab, kv_tab, 1 / math.sqrt(D))
    base = [torch.randn(x.shape, generator=gen).to(DEV) for x in (dq, dk, dv)]
    acc = [b.clone() for b in base]
    run_step(q, k, v, do, lse_d, delta, q_tab, kv_tab, 1 / math.sqrt(D),
             mode=cp.CP_BWD_DQ_ACCUMULATE | cp.CP_BWD_DKV_ACCUMULATE, dq=acc[0], dk=acc[1], dv=acc[2])
    torch.cuda.synchronize()
    for a, b, x in zip(acc, base, (dq, dk, dv)):
        # the kernel may fuse the scaling into the addition: equal up to one rounding
        assert torch.allclose(a, b + x, rtol=1e-6, atol=1e-6)
    # a K/V block entirely after the queries: write mode gives zeros, accumulate leaves values as they were
    late = cp.CpChunks.make([7 * L], L)
    k2, v2 = gather(K, late, DEV), gather(V, late, DEV)
    z = run_step(q, k2, v2, do, lse_d, delta, q_tab, late, 1 / math.sqrt(D))
    keep = [b.clone() for b in base]
    dk2, dv2 = keep[1][:, :, :L].contiguous(), keep[2][:, :, :L].contiguous()
    dk2_0, dv2_0 = dk2.clone(), dv2.clone()
    run_step(q, k2, v2, do, lse_d, delta, q_tab, late, 1 / math.sqrt(D),
             mode=cp.CP_BWD_DQ_ACCUMULATE | cp.CP_BWD_DKV_ACCUMULATE, dq=keep[0], dk=dk2, dv=dv2)
    torch.cuda.synchronize()
    assert all(torch.all(t == 0) for t in z)
    assert torch.equal(keep[0], base[0]) and torch.equal(dk2, dk2_0) and torch.equal(dv2, dv2_0)


def test_bwd_deterministic():
    w = workloads.get("s8k_cp2")
    H = 2
    Q, K, V = workloads.make_qkv(w, H=H)
    dO = workloads.make_grad_out(w, H=H)
    q_tab, kv_tabs = zigzag_tables(w.cp, 1, w.chunk_len)
    out, lse = forward_rows(Q, K, V, positions(q_tab), w.scale)
    q, do = gather(Q, q_tab, DEV), gather(dO, q_tab, DEV)
    k, v = gather(K, kv_tabs[1], DEV), gather(V, kv_tabs[1], DEV)
    out_d, lse_d = device_inputs(out, lse)
    delta = gpu_delta(out_d, do)
    a = run_step(q, k, v, do, lse_d, delta, q_tab, kv_tabs[1], w.scale)
    b = run_step(q, k, v, do, lse_d, delta, q_tab, kv_tabs[1], w.scale)
    torch.cuda.synchronize()
    assert all(torch.equal(x, y) for x, y in zip(a, b))


# ---------------------------------------------------------------- whole ring
@pytest.mark.parametrize("N,L,D,H", [(2, 64, 64, 2), (4, 128, 128, 2)])
def test_ring_backward_end_to_end(N, L, D, H):
    """GPU forward (cp_ring_attn_fwd) on every rank, then every rank's backward steps: dq accumulates
    on the rank, each K/V block's dk/dv accumulates over the ranks that see it; the assembled
    gradients match the oracle's full-sequence causal attention gradients."""
    S = 2 * N * L
    scale = 1 / math.sqrt(D)
    Q, K, V = workloads.make_qkv_scaled((1, H, S, D), 40 + N)
    gen = torch.Generator().manual_seed(41 + N)
    dO = torch.randn(1, H, S, D, generator=gen).to(torch.bfloat16)
    dk_blocks = {}
    dq_full = np.zeros((1, H, S, D))
    for r in range(N):
        _announce("ring bwd", N, L, D, "rank", r)
        q_tab, kv_tabs = zigzag_tables(N, r, L)
        q = gather(Q, q_tab, DEV)
        do = gather(dO, q_tab, DEV)
        ks = [gather(K, t, DEV) for t in kv_tabs]
        vs = [gather(V, t, DEV) for t in kv_tabs]
        out = torch.empty_like(q)
        lse = torch.empty(q.shape[:-1], dtype=torch.float32, device=DEV)
        ws = torch.empty(cp.cp_ring_attn_workspace_bytes(1, H, ks[0].shape[2], D, q.shape[2]),
                         dtype=torch.uint8, device=DEV)
        cp.cp_ring_attn_fwd(q, q_tab, ks, vs, kv_tabs, out, lse, scale, ws, copy_stream=torch.cuda.Stream())
        delta = gpu_delta(out, do)
        dq = torch.empty(q.shape, dtype=torch.float32, device=DEV)
        for j, t in enumerate(kv_tabs):
            src = (r - j) % N
            if src not in dk_blocks:
                dk_blocks[src] = [torch.empty(ks[j].shape, dtype=torch.float32, device=DEV) for _ in range(2)]
                first = True
            else:
                first = False
            mode = (cp.CP_BWD_DQ_ACCUMULATE if j > 0 else 0) | (0 if first else cp.CP_BWD_DKV_ACCUMULATE)
            run_step(q, ks[j], vs[j], do, lse, delta, q_tab, t, scale, mode=mode,
                     dq=dq, dk=dk_blocks[src][0], dv=dk_blocks[src][1])
        torch.cuda.synchronize()
        dq_full[:, :, positions(q_tab)] = dq.cpu().numpy()
    dk_full = np.zeros((1, H, S, D))
    dv_full = np.zeros((1, H, S, D))
    for src, (dk, dv) in dk_blocks.items():
        p = positions(zigzag_tables(N, src, L)[0])
        dk_full[:, :, p] = dk.cpu().numpy()
        dv_full[:, :, p] = dv.cpu().numpy()
    ref = _per_head(1, H, lambda b, h: oracle.causal_attention_grad(
        oracle.to_f64(Q[b, h]), oracle.to_f64(K[b, h]), oracle.to_f64(V[b, h]), oracle.to_f64(dO[b, h]), scale))
    for i, (name, got) in enumerate((("dq", dq_full), ("dk", dk_full), ("dv", dv_full))):
        r_all = np.stack([x[i] for x in ref])[None]
        assert_grad(name, torch.from_numpy(got), r_all)


# ---------------------------------------------------------------- ring driver
def run_ring_bwd(q, q_tab, do, out, lse, ks, vs, kv_tabs, dks, dvs, scale, acc=None, copy_stream=None):
    B, H, Sq, D = q.shape
    Skv = ks[0].shape[2]
    dq = torch.empty((B, H, Sq, D), dtype=torch.float32, device=DEV)
    ws = torch.empty(cp.cp_ring_attn_bwd_workspace_bytes(B, H, Skv, D, Sq), dtype=torch.uint8, device=DEV)
    cp.cp_ring_attn_bwd(q, q_tab, do, out, lse, ks, vs, kv_tabs, dks, dvs, dq, scale, ws, dkv_accumulate=acc,
                        copy_stream=torch.cuda.Stream() if copy_stream is None else copy_stream)
    return dq


@pytest.mark.parametrize("N,L,D,H,B", [(2, 64, 64, 2, 1), (4, 128, 128, 2, 1), (2, 256, 128, 2, 1),
                                       (3, 192, 64, 3, 2), (2, 256, 128, 4, 2), (1, 128, 128, 2, 1)])
def test_ring_attn_bwd_all_ranks(N, L, D, H, B):
    """cp_ring_attn_bwd on every rank after the GPU forward: each block's dK/dV buffers start at zero and
    every rank adds its contribution (all steps accumulate); the assembled gradients match the oracle's
    full-sequence causal attention gradients."""
    S = 2 * N * L
    scale = 1 / math.sqrt(D)
    Q, K, V = workloads.make_qkv_scaled((B, H, S, D), 60 + N + L)
    gen = torch.Generator().manual_seed(61 + N + L)
    dO = torch.randn(B, H, S, D, generator=gen).to(torch.bfloat16)
    Skv = 2 * L
    blocks = {src: (torch.zeros((B, H, Skv, D), dtype=torch.float32, device=DEV),
                    torch.zeros((B, H, Skv, D), dtype=torch.float32, device=DEV)) for src in range(N)}
    dq_full = np.zeros((B, H, S, D))
    for r in range(N):
        _announce("ring attn bwd", N, L, D, "rank", r)
        q_tab, kv_tabs = zigzag_tables(N, r, L)
        q, do = gather(Q, q_tab, DEV), gather(dO, q_tab, DEV)
        ks = [gather(K, t, DEV) for t in kv_tabs]
        vs = [gather(V, t, DEV) for t in kv_tabs]
        out = torch.empty_like(q)
        lse = torch.empty(q.shape[:-1], dtype=torch.float32, device=DEV)
        ws = torch.empty(cp.cp_ring_attn_workspace_bytes(B, H, Skv, D, q.shape[2]), dtype=torch.uint8, device=DEV)
        cp.cp_ring_attn_fwd(q, q_tab, ks, vs, kv_tabs, out, lse, scale, ws, copy_stream=torch.cuda.Stream())
        dks = [blocks[(r - j) % N][0] for j in range(N)]
        dvs = [blocks[(r - j) % N][1] for j in range(N)]
        dq = run_ring_bwd(q, q_tab, do, out, lse, ks, vs, kv_tabs, dks, dvs, scale, acc=[1] * N)
        torch.cuda.synchronize()
        dq_full[:, :, positions(q_tab)] = dq.cpu().numpy()
    dk_full = np.zeros((B, H, S, D))
    dv_full = np.zeros((B, H, S, D))
    for src, (dk, dv) in blocks.items():
        p = positions(zigzag_tables(N, src, L)[0])
        dk_full[:, :, p] = dk.cpu().numpy()
        dv_full[:, :, p] = dv.cpu().numpy()
    ref = _per_head(B, H, lambda b, h: oracle.causal_attention_grad(
        oracle.to_f64(Q[b, h]), oracle.to_f64(K[b, h]), oracle.to_f64(V[b, h]), oracle.to_f64(dO[b, h]), scale))
    for i, (name, got) in enumerate((("dq", dq_full), ("dk", dk_full), ("dv", dv_full))):
        r_all = np.stack([x[i] for x in ref]).reshape(B, H, S, D)
        assert_grad(name, torch.from_numpy(got), r_all)


@pytest.mark.parametrize("name,H,rank", [("s8k_cp2", 2, 1), ("s32k_cp8", 1, 0)])
def test_ring_attn_bwd_rank_share(name, H, rank):
    """One rank's share with the ring's own pattern (step 0 writes, later steps add to incoming partial
    sums): dq equals the oracle's gradient of the rank's rows, dk_steps[0] this rank's contribution to its
    own block, dk_steps[j] the incoming partial sums plus this rank's contribution.  Running every copy in
    order on the launch stream gives identical bits."""
    w = workloads.get(name)
    Q, K, V = workloads.make_qkv(w, H=H)
    dO = workloads.make_grad_out(w, H=H)
    q_tab, kv_tabs = zigzag_tables(w.cp, rank, w.chunk_len)
    qpos = positions(q_tab)
    _announce("ring attn bwd share", w.describe(), "H", H, "rank", rank)
    fwd_out, fwd_lse = forward_rows(Q, K, V, qpos, w.scale)
    out_d, lse_d = device_inputs(fwd_out, fwd_lse)
    q, do = gather(Q, q_tab, DEV), gather(dO, q_tab, DEV)
    ks = [gather(K, t, DEV) for t in kv_tabs]
    vs = [gather(V, t, DEV) for t in kv_tabs]
    gen = torch.Generator().manual_seed(77)
    init = [(torch.randn(ks[0].shape, generator=gen), torch.randn(ks[0].shape, generator=gen)) for _ in kv_tabs]
    results = []
    for in_order in (False, True):
        dks = [a.to(DEV) for a, _ in init]
        dvs = [b.to(DEV) for _, b in init]
        dq = run_ring_bwd(q, q_tab, do, out_d, lse_d, ks, vs, kv_tabs, dks, dvs, w.scale,
                          copy_stream=torch.cuda.current_stream() if in_order else None)
        torch.cuda.synchronize()
        results.append((dq, dks, dvs))
    dq, dks, dvs = results[0]
    rq_total = 0.0
    for j, t in enumerate(kv_tabs):
        rq, rk, rv = oracle_step_grads(Q, K, V, dO, qpos, positions(t), fwd_out, fwd_lse, w.scale)
        rq_total = rq_total + rq
        for nm, got, ref, x0 in (("dk", dks[j], rk, init[j][0]), ("dv", dvs[j], rv, init[j][1])):
            mine = got.cpu().numpy().astype(np.float64) - (x0.numpy().astype(np.float64) if j > 0 else 0.0)
            assert_grad(f"{nm}[{j}]", torch.from_numpy(mine), ref)
    assert_grad("dq", dq, rq_total)
    dq2, dks2, dvs2 = results[1]
    assert torch.equal(dq, dq2)
    assert all(torch.equal(a, b) for a, b in zip(dks + dvs, dks2 + dvs2))
