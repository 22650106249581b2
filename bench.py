"""Benchmark: one CP rank's share of causal ring attention on one MI355X.

A step is one cp_ring_attn_fwd call: every ring step of the rank's share
(staging copy of the next K/V block on a side stream, attention of the local
queries against the current block, fused log-sum-exp merge, bf16 output).
Default workload: S = 32768, context-parallel size 8, rank 0, B = 1, H = 32,
D = 128 (local queries 4096 tokens in two zigzag chunks of 2048, eight ring
steps of 4096 keys).  Inputs are seeded synthetic bf16 ~ N(0, 1), resident in
HBM (all eight ranks' K/V blocks) before timing starts.

Prints one JSON line.  The metric is causal-effective TFLOP/s: 4*D*B*H times
the number of visible (query, key) pairs of the rank's share, per second.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6   # MI355X dense bf16 MFMA (256 CU x 2.4 GHz x 4096 flop/clk)
PEAK_HBM_GBS = 8000.0


def visible_pairs(q_tab, kv_tabs):
    """Visible (query, key) pairs of one (batch, head), summed over ring steps and chunk pairs.

    For a query chunk starting at qs (length Lq) and a key chunk at ks (length
    Lk), query position p sees min(max(p - ks + 1, 0), Lk) keys.
    """
    def S(n, Lk):   # sum_{x=1..n} min(x, Lk)
        if n <= 0:
            return 0
        return n * (n + 1) // 2 if n <= Lk else Lk * (Lk + 1) // 2 + (n - Lk) * Lk

    total = 0
    Lq = q_tab.chunk_len
    for t in kv_tabs:
        for qs in q_tab.starts():
            for ks in t.starts():
                total += S(qs - ks + Lq, t.chunk_len) - S(qs - ks, t.chunk_len)
    return total


def settle(fn, stream, batch=5, tol=0.01, window=3, max_calls=400):
    """Untimed clock settling: run ``fn`` in batches of ``batch`` calls until the
    mean call time of the last ``window`` batches agrees within ``tol``
    (max/min - 1), at most ``max_calls`` calls.  After host-side setup the GPU
    runs the first few dozen forwards slower while its clocks ramp up; the
    timed region starts only once they have settled.  Returns the number of
    calls and the last batch's mean milliseconds."""
    import torch
    times, n = [], 0
    while n < max_calls:
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(batch):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1) / batch)
        n += batch
        last = times[-window:]
        if len(last) == window and max(last) <= (1.0 + tol) * min(last):
            break
    return n, times[-1]


def cpu_baseline(w, rank, budget_s, Q, K, V, keep=None):
    """Time the fp64 oracle on a bounded sample of the same share.

    The sample is the rank's full set of query rows for as many (batch, head)
    pairs as fit in ``budget_s`` seconds (at least one head), taken in order.
    If ``keep`` is a dict, the oracle's (out, lse) of each computed head is
    stored in it under (b, h), for the bench's parity check.
    """
    import numpy as np
    import oracle
    import workloads
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:  # pragma: no cover
        cores = len(os.sched_getaffinity(0))
    pos = oracle.local_positions(w.S, w.cp, rank)
    heads = [(b, h) for b in range(w.B) for h in range(w.H)]
    # warm up BLAS threads
    oracle.causal_attention_rows(oracle.to_f64(Q[0, 0]), oracle.to_f64(K[0, 0]), oracle.to_f64(V[0, 0]),
                                 pos[:8], w.scale)
    done, pairs, t0 = 0, 0, time.perf_counter()
    for b, h in heads:
        q, k, v = (oracle.to_f64(x[b, h]) for x in (Q, K, V))
        res = oracle.causal_attention_rows(q, k, v, pos, w.scale)
        if keep is not None:
            keep[(b, h)] = res
        pairs += int((pos + 1).sum())
        done += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    dt = time.perf_counter() - t0
    flops = 4.0 * w.D * pairs
    info = workloads.host_info()
    return {
        "value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
        "sample": f"all {len(pos)} query rows of rank {rank} for {done} of {len(heads)} (batch, head) "
                  f"pairs: {pairs} visible pairs in {dt:.1f} s; {info['cpu_model']}",
    }


def cpu_baseline_bwd(w, rank, budget_s, Q, K, V, kv_tabs):
    """Time the fp64 gradient oracle on a bounded sample of the backward share.

    The sample is (head, ring step) blocks taken in order: for each, the
    oracle's forward rows of the rank's queries (needed for LSE and Delta) are
    computed once per head, then the block's gradient contributions.  Only
    the visible pairs of the gradient blocks count towards the rate.
    """
    import numpy as np
    import oracle
    import workloads
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:  # pragma: no cover
        cores = len(os.sched_getaffinity(0))
    pos = oracle.local_positions(w.S, w.cp, rank)
    dO = workloads.make_grad_out(w)
    done, pairs, t0 = 0, 0, time.perf_counter()
    for b in range(w.B):
        for h in range(w.H):
            q, k, v, do = (oracle.to_f64(x[b, h]) for x in (Q, K, V, dO))
            o, l = oracle.causal_attention_rows(q, k, v, pos, w.scale)
            for j, t in enumerate(kv_tabs):
                kpos = oracle.local_positions(w.S, w.cp, (rank - j) % w.cp)
                oracle.masked_attention_grad(q[pos], pos, k[kpos], v[kpos], kpos, do[pos], o, l, w.scale)
                pairs += int((kpos[None, :] <= pos[:, None]).sum())
                done += 1
                if time.perf_counter() - t0 >= budget_s:
                    break
            if time.perf_counter() - t0 >= budget_s:
                break
        if time.perf_counter() - t0 >= budget_s:
            break
    dt = time.perf_counter() - t0
    info = workloads.host_info()
    return {
        "value": 10.0 * w.D * pairs / dt / 1e12, "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
        "sample": f"{done} (head, ring step) gradient blocks of rank {rank}'s {len(pos)} query rows, with "
                  f"the forward rows they need: {pairs} visible pairs in {dt:.1f} s; {info['cpu_model']}",
    }


def kernel_traffic(workload, kernel):
    """Calibrated HBM bytes per launch of a kernel, from its counter
    summary, only if taken on this workload and on the kernel source built now."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_traffic.json")
    try:
        from long_sequence_causal_cp_amd.prof_summary import kernel_source_sha256, sources_for
        with open(path) as f:
            tj = json.load(f)
        if tj.get("workload") == workload and tj.get("kernel_source_sha256") == kernel_source_sha256(sources_for(kernel)):
            return round(tj["bytes_per_launch"])
    except (OSError, ValueError, KeyError):
        pass
    return None


# ---- the rest of the cpu_baseline leg: the oracle's reference values for the
# few rows each pass spot-checks after its timed region (head (0, 0)) ----
def cpu_baseline_rows(w, rank, Q, K, V, rows):
    """The oracle's (out, LSE) of the rank's local query rows ``rows``."""
    import oracle
    pos = oracle.local_positions(w.S, w.cp, rank)
    return oracle.causal_attention_rows(oracle.to_f64(Q[0, 0]), oracle.to_f64(K[0, 0]), oracle.to_f64(V[0, 0]),
                                        pos[rows], w.scale)


def cpu_baseline_rows_fp8(w, rank, qd, kd, vd, rows):
    """The oracle's (out, LSE) of local rows ``rows`` on dequantised fp8 values
    (qd, kd, vd: float64 [S, D] in natural token order)."""
    import numpy as np
    import oracle
    pos = oracle.local_positions(w.S, w.cp, rank)
    kmax = int(pos[rows].max()) + 1
    return oracle.masked_attention(qd[pos[rows]], pos[rows], kd[:kmax], vd[:kmax], np.arange(kmax), w.scale)


def cpu_baseline_grads(w, rank, Q, K, V, dO, rows, keys):
    """The oracle's dQ of local rows ``rows`` (over every visible key) and the
    dK, dV contributions of this rank's queries to keys ``keys`` of its own
    block."""
    import numpy as np
    import oracle
    pos = oracle.local_positions(w.S, w.cp, rank)
    f64 = lambda X: oracle.to_f64(X[0, 0])
    Qh, Kh, Vh, dOh = f64(Q), f64(K), f64(V), f64(dO)
    kmax = int(pos[rows].max()) + 1
    o_r, l_r = oracle.causal_attention_rows(Qh, Kh, Vh, pos[rows], w.scale)
    dq_ref, _, _ = oracle.masked_attention_grad(Qh[pos[rows]], pos[rows], Kh[:kmax], Vh[:kmax], np.arange(kmax),
                                                dOh[pos[rows]], o_r, l_r, w.scale)
    o_all, l_all = oracle.causal_attention_rows(Qh, Kh, Vh, pos, w.scale)
    kpos = pos[keys]
    _, dk_ref, dv_ref = oracle.masked_attention_grad(Qh[pos], pos, Kh[kpos], Vh[kpos], kpos, dOh[pos], o_all, l_all,
                                                     w.scale)
    return dq_ref, dk_ref, dv_ref


def bench_backward(args, w, Q, K, V, q, q_tab, ks, vs, kv_tabs, out, lse, stream, gather):
    """The rank's backward share: one cp_ring_attn_bwd call.

    out and lse come from the GPU ring forward over the same inputs; dO is a
    seeded bf16 N(0, 1) draw.  The call computes Delta, then every ring step:
    step 0 on the rank's own block writes its dK/dV; steps j >= 1 receive the
    block and its travelling dK/dV partial sums into a staging slot, add this
    rank's contribution and send the sums back (copies on a side stream).
    dq accumulates over the steps.  Algorithmic flops: five products per
    visible pair (S, dP, dV, dQ, dK), 10*D flop; the dq kernel's own work is
    S, dP and dQ (6*D per pair), the dk/dv kernel's S, dP, dV and dK (8*D).
    """
    import numpy as np
    import torch
    import workloads
    import long_sequence_causal_cp_amd as cp

    B, H, Sq, D = q.shape
    Skv = ks[0].shape[2]
    N, r = len(kv_tabs), args.rank
    dev = q.device
    do = gather(workloads.make_grad_out(w), q_tab)
    dq = torch.empty((B, H, Sq, D), dtype=torch.float32, device=dev)
    dks = [torch.zeros((B, H, Skv, D), dtype=torch.float32, device=dev) for _ in range(N)]
    dvs = [torch.zeros((B, H, Skv, D), dtype=torch.float32, device=dev) for _ in range(N)]
    ws = torch.empty(cp.cp_ring_attn_bwd_workspace_bytes(B, H, Skv, D, Sq), dtype=torch.uint8, device=dev)
    copy_stream = torch.cuda.Stream()

    def step(cs=copy_stream):
        cp.cp_ring_attn_bwd(q, q_tab, do, out, lse, ks, vs, kv_tabs, dks, dvs, dq, w.scale, ws, stream=stream,
                            copy_stream=cs)

    pairs = visible_pairs(q_tab, kv_tabs)
    flops = 10.0 * D * B * H * pairs
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    settle_n = settle(step, stream)[0] if args.settle else 0
    print(f"[bench bwd] {w.describe()} rank {r}: warmup {args.warmup} done, settled after {settle_n} more",
          file=sys.stderr, flush=True)
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(args.steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = ev0.elapsed_time(ev1) / args.steps
    value = flops / (ms_per_step * 1e-3) / 1e12

    cp.cp_profile_enable(True)
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    kern = cp.cp_profile_read_named(8192)
    cp.cp_profile_enable(False)
    kern_ms = [t for t, _ in kern]
    assert len(kern_ms) == 2 * N * args.steps, (len(kern_ms), N, args.steps)
    dq_names = sorted(set(n for _, n in kern[0::2]))
    dkdv_names = sorted(set(n for _, n in kern[1::2]))
    dq_ms = statistics.fmean(kern_ms[0::2])
    dkdv_ms = statistics.fmean(kern_ms[1::2])
    dq_flop = 6.0 * D * B * H * pairs / N      # per launch, averaged over the ring steps
    dkdv_flop = 8.0 * D * B * H * pairs / N
    kernels = {
        "dq": {"avg_launch_ms": round(dq_ms, 5), "flop_per_launch": dq_flop,
               "achieved": round(dq_flop / (dq_ms * 1e-3) / 1e12, 2)},
        "dkdv": {"avg_launch_ms": round(dkdv_ms, 5), "flop_per_launch": dkdv_flop,
                 "achieved": round(dkdv_flop / (dkdv_ms * 1e-3) / 1e12, 2)},
    }
    dom = "dkdv" if dkdv_ms >= dq_ms else "dq"

    def timed_each(fn, n):
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
        for e0, e1 in evs:
            e0.record(stream)
            fn()
            e1.record(stream)
        torch.cuda.synchronize()
        return [e0.elapsed_time(e1) for e0, e1 in evs]

    median_ms = statistics.median(timed_each(step, args.steps))
    no_overlap_ms = statistics.median(timed_each(lambda: step(stream), args.steps))

    # spot check against the oracle (outside the timed region): dq of four
    # local rows, and dk/dv of four keys of the rank's own block (step 0
    # writes them, so they hold this rank's contribution alone)
    step()
    torch.cuda.synchronize()
    L = w.chunk_len
    rows = np.array([0, L - 1, L, 2 * L - 1])
    keys = np.array([0, L - 1, L, 2 * L - 1])
    dq_ref, dk_ref, dv_ref = cpu_baseline_grads(w, r, Q, K, V, workloads.make_grad_out(w), rows, keys)
    rel = lambda got, ref: float(np.max(np.abs(got - ref)) / max(np.max(np.abs(ref)), 1e-30))
    check = {"dq_rel": rel(dq[0, 0, rows].cpu().numpy(), dq_ref),
             "dk_rel": rel(dks[0][0, 0, keys].cpu().numpy(), dk_ref),
             "dv_rel": rel(dvs[0][0, 0, keys].cpu().numpy(), dv_ref)}
    print(f"[bench bwd] timed {args.steps} steps: {ms_per_step:.4f} ms/step, {value:.1f} TFLOP/s; dq kernel "
          f"{dq_ms:.4f} ms, dk/dv kernel {dkdv_ms:.4f} ms per launch; spot check {check}",
          file=sys.stderr, flush=True)
    res = {
        "metric": "causal-effective attention backward TFLOP/s per CP-rank share; % of bf16 MFMA peak",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "settle_forwards": settle_n,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "pct_of_bf16_peak": round(100.0 * value / PEAK_BF16_TFLOPS, 2),
        "config": {
            "workload": f"{w.name}: backward of causal ring attention, one rank's share (rank {r} of cp={N}), "
                        f"B={B} H={H} D={D} S={w.S}, zigzag chunks of {L}, {N} ring steps of {Skv} keys",
            "seq_len": w.S, "cp": N, "rank": r, "B": B, "H": H, "D": D,
            "visible_pairs_per_head": pairs, "flop_per_step": flops, "wall_s_timed": round(wall, 4),
        },
        "roofline": {
            "kernel": " + ".join(dkdv_names if dom == "dkdv" else dq_names), "bound": "mfma",
            "achieved": kernels[dom]["achieved"], "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
            "frac": round(kernels[dom]["achieved"] / PEAK_BF16_TFLOPS, 4),
            "traffic": kernel_traffic(w.name, f"bwd_{dom}_kernel"),
            "kernels": kernels, "kernel_ms_per_step": round(N * (dq_ms + dkdv_ms), 5),
        },
        "timing": {
            "ms_per_step_median": round(median_ms, 5),
            "ms_per_step_no_overlap_median": round(no_overlap_ms, 5),
            "note": "median over --steps backward calls, each bracketed by HIP events; no_overlap runs every "
                    "staging copy in order on the launch stream",
        },
        "cpu_baseline": cpu_baseline_bwd(w, r, args.cpu_budget, Q, K, V, kv_tabs) if args.cpu_budget > 0 else None,
        "check": check,
    }
    print(json.dumps(res), flush=True)


def bench_allgather(args, w, Q, K, V, q, q_tab, kv_tabs, stream):
    """All-gather form of context parallelism: one cp_attn_step_fwd of the rank's
    queries against the keys of the whole sequence, gathered in natural order
    (one K/V chunk of S tokens).  The visible pairs, and so the flops, are the
    ring's.  The gather itself (the other ranks' blocks, copied in) is not in
    the timed region; its bytes are reported.
    """
    import numpy as np
    import torch
    import long_sequence_causal_cp_amd as cp

    B, H, Sq, D = q.shape
    dev = q.device
    k_full, v_full = K.contiguous().to(dev), V.contiguous().to(dev)
    full = cp.CpChunks.make([0], w.S)
    o = torch.empty((B, H, Sq, D), dtype=torch.float32, device=dev)
    lse = torch.empty((B, H, Sq), dtype=torch.float32, device=dev)
    out = torch.empty_like(q)

    def step():
        cp.cp_attn_step_fwd(q, k_full, v_full, o, lse, out, q_tab, full, w.scale, cp.CP_STEP_WRITE, stream=stream)

    pairs = visible_pairs(q_tab, kv_tabs)
    assert pairs == visible_pairs(q_tab, [full])
    flops = 4.0 * D * B * H * pairs
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    if args.settle:
        settle(step, stream)
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(args.steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = ev0.elapsed_time(ev1) / args.steps
    value = flops / (ms_per_step * 1e-3) / 1e12
    cp.cp_profile_enable(True)
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    kern = cp.cp_profile_read_named(8192)
    cp.cp_profile_enable(False)
    kern_ms = [t for t, _ in kern]
    ag_names = sorted(set(n for _, n in kern))
    avg = statistics.fmean(kern_ms)
    achieved = flops / (avg * 1e-3) / 1e12
    L = w.chunk_len
    rows = np.array([0, L - 1, L, 2 * L - 1])
    ro, rl = cpu_baseline_rows(w, args.rank, Q, K, V, rows)
    eo = float(np.max(np.abs(out[0, 0, rows].float().cpu().numpy() - ro)))
    el = float(np.max(np.abs(lse[0, 0, rows].cpu().numpy() - rl)))
    gather_bytes = 2 * B * H * (w.S - Sq) * D * 2
    print(f"[bench allgather] {w.describe()} rank {args.rank}: {ms_per_step:.4f} ms/step, {value:.1f} TFLOP/s; "
          f"step kernel {avg:.4f} ms; spot check max|dout| {eo:.2e} max|dlse| {el:.2e}", file=sys.stderr, flush=True)
    res = {
        "metric": "causal-effective attention TFLOP/s per CP-rank share, all-gather form (gather not timed); "
                  "% of bf16 MFMA peak",
        "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic", "pct_of_bf16_peak": round(100.0 * value / PEAK_BF16_TFLOPS, 2),
        "config": {
            "workload": f"{w.name}: rank {args.rank} of cp={w.cp}, local queries {Sq} tokens (zigzag chunks of {L}) "
                        f"against the gathered {w.S} keys in one step, B={B} H={H} D={D}",
            "seq_len": w.S, "cp": w.cp, "rank": args.rank, "B": B, "H": H, "D": D,
            "visible_pairs_per_head": pairs, "flop_per_step": flops, "wall_s_timed": round(wall, 4),
            "gather_bytes_not_timed": gather_bytes,
        },
        "roofline": {
            "kernel": " + ".join(ag_names) + " over one K/V chunk of the whole sequence", "bound": "mfma",
            "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
            "frac": round(achieved / PEAK_BF16_TFLOPS, 4), "traffic": None, "launches_per_step": 1,
            "avg_launch_ms": round(avg, 5),
        },
        "cpu_baseline": None,
        "check": {"max_abs_dout": eo, "max_abs_dlse": el},
    }
    print(json.dumps(res), flush=True)


PEAK_FP8_TFLOPS = 5033.2   # MI355X dense fp8 MFMA, twice the bf16 figure


def bench_fp8(args, w, Q, K, V, q_tab, kv_tabs, stream):
    """The rank's share with Q, K, V in e4m3 through cp_ring_attn_fwd_fp8 (the
    ring of the bf16 forward: grouped launches, e4m3 staging copies on a side
    stream) -- the value.  Beside it, on the same GPU: the bf16 ring, and the
    chains of one step launch per ring step in fp8 and bf16 (every step's
    blocks resident, no staging).  Quantisation: power-of-two per-tensor
    scales, codes = RNE(x / scale)."""
    import math as _m
    import numpy as np
    import torch
    import long_sequence_causal_cp_amd as cp

    dev = torch.device("cuda:0")

    def quant(x):
        amax = float(x.abs().max())
        sc = 2.0 ** _m.ceil(_m.log2(amax / 448.0))
        return (x.to(torch.float64) / sc).to(torch.float32).to(torch.float8_e4m3fn), sc

    (qc, sq), (kc, sk), (vc, sv) = quant(Q.float()), quant(K.float()), quant(V.float())

    def g8(codes, t):
        idx = torch.cat([torch.arange(s0, s0 + t.chunk_len) for s0 in t.starts()])
        return codes.view(torch.uint8).index_select(2, idx).contiguous()

    q = g8(qc, q_tab).to(dev).view(torch.float8_e4m3fn)
    ks = [g8(kc, t).to(dev).view(torch.float8_e4m3fn) for t in kv_tabs]
    vts = [g8(vc, t).transpose(2, 3).contiguous().to(dev).view(torch.float8_e4m3fn) for t in kv_tabs]
    B, H, Sq, D = q.shape
    N = len(kv_tabs)
    o = torch.empty((B, H, Sq, D), dtype=torch.float32, device=dev)
    lse = torch.empty((B, H, Sq), dtype=torch.float32, device=dev)
    out = torch.empty((B, H, Sq, D), dtype=torch.bfloat16, device=dev)

    def step():
        for j in range(N):
            cp.cp_attn_step_fwd_fp8(q, ks[j], vts[j], o, lse, out if j == N - 1 else None, q_tab, kv_tabs[j], w.scale,
                                    sq, sk, sv, cp.CP_STEP_WRITE if j == 0 else cp.CP_STEP_MERGE, stream=stream)

    pairs = visible_pairs(q_tab, kv_tabs)
    flops = 4.0 * D * B * H * pairs
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(args.steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = ev0.elapsed_time(ev1) / args.steps
    value = flops / (ms_per_step * 1e-3) / 1e12
    cp.cp_profile_enable(True)
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    kern_ms = cp.cp_profile_read(8192)
    cp.cp_profile_enable(False)
    avg = statistics.fmean(kern_ms)
    achieved = flops / N / (avg * 1e-3) / 1e12
    chain_ms = ms_per_step
    # the ring driver in fp8 (grouped launches, e4m3 staging copies on a side stream): the value
    ws8 = torch.empty(cp.cp_ring_attn_fwd_fp8_workspace_bytes(B, H, ks[0].shape[2], D, Sq), dtype=torch.uint8,
                      device=dev)
    cs = torch.cuda.Stream()

    def ring8():
        cp.cp_ring_attn_fwd_fp8(q, q_tab, ks, vts, kv_tabs, out, lse, w.scale, sq, sk, sv, ws8, stream=stream,
                                copy_stream=cs)

    def timed_loop(fn):
        for _ in range(args.warmup):
            fn()
        torch.cuda.synchronize()
        if args.settle:
            settle(fn, stream)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(args.steps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / args.steps

    t0 = time.perf_counter()
    ms_per_step = timed_loop(ring8)
    wall = time.perf_counter() - t0
    value = flops / (ms_per_step * 1e-3) / 1e12
    cp.cp_profile_enable(True)
    for _ in range(args.steps):
        ring8()
    torch.cuda.synchronize()
    kern_ms = cp.cp_profile_read(8192)
    cp.cp_profile_enable(False)
    avg = statistics.fmean(kern_ms)
    n_launch = len(kern_ms) // args.steps
    achieved = flops / n_launch / (avg * 1e-3) / 1e12

    # the bf16 ring and the bf16 chain of step launches, for comparison (same GPU)
    def g16(x, t):
        idx = torch.cat([torch.arange(s0, s0 + t.chunk_len) for s0 in t.starts()])
        return x.index_select(2, idx).contiguous().to(dev)
    q16 = g16(Q, q_tab)
    k16 = [g16(K, t) for t in kv_tabs]
    v16 = [g16(V, t) for t in kv_tabs]
    out16 = torch.empty_like(out)
    ws16 = torch.empty(cp.cp_ring_attn_workspace_bytes(B, H, k16[0].shape[2], D, Sq), dtype=torch.uint8, device=dev)

    def ring16():
        cp.cp_ring_attn_fwd(q16, q_tab, k16, v16, kv_tabs, out16, lse, w.scale, ws16, stream=stream, copy_stream=cs)

    def chain16():
        for j in range(N):
            cp.cp_attn_step_fwd(q16, k16[j], v16[j], o, lse, out16 if j == N - 1 else None, q_tab, kv_tabs[j],
                                w.scale, cp.CP_STEP_WRITE if j == 0 else cp.CP_STEP_MERGE, stream=stream)

    bf16_ring_ms = timed_loop(ring16)
    bf16_ms = timed_loop(chain16)
    ring8()
    torch.cuda.synchronize()

    L = w.chunk_len
    rows = np.array([0, L - 1, L, 2 * L - 1])
    deq = lambda c, sc: c.to(torch.float64).numpy() * sc
    ro, rl = cpu_baseline_rows_fp8(w, args.rank, deq(qc[0, 0], sq), deq(kc[0, 0], sk), deq(vc[0, 0], sv), rows)
    eo = float(np.max(np.abs(out[0, 0, rows].float().cpu().numpy() - ro)))
    el = float(np.max(np.abs(lse[0, 0, rows].cpu().numpy() - rl)))
    print(f"[bench fp8] {w.describe()} rank {args.rank}: ring {ms_per_step:.4f} ms/step, {value:.1f} TFLOP/s "
          f"(bf16 ring {bf16_ring_ms:.4f}; fp8 step chain {chain_ms:.4f}, bf16 step chain {bf16_ms:.4f}); "
          f"fp8 kernel {avg:.4f} ms per launch; spot check max|dout| {eo:.2e} max|dlse| {el:.2e}",
          file=sys.stderr, flush=True)
    res = {
        "metric": "causal-effective attention TFLOP/s per CP-rank share, fp8 (e4m3) Q/K/V ring; % of fp8 MFMA peak",
        "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "fp8-e4m3", "data": "synthetic", "pct_of_fp8_peak": round(100.0 * value / PEAK_FP8_TFLOPS, 2),
        "config": {
            "workload": f"{w.name}: rank {args.rank} of cp={w.cp}, B={B} H={H} D={D} S={w.S}, zigzag chunks of {L}, "
                        f"{N} ring steps in fp8 (cp_ring_attn_fwd_fp8: grouped launches, e4m3 staging copies)",
            "seq_len": w.S, "cp": w.cp, "rank": args.rank, "B": B, "H": H, "D": D,
            "visible_pairs_per_head": pairs, "flop_per_step": flops, "wall_s_timed": round(wall, 4),
            "scales": {"q": sq, "k": sk, "v": sv},
            "fp8_step_chain_ms_per_step": round(chain_ms, 5),
            "bf16_ring_ms_per_step": round(bf16_ring_ms, 5),
            "bf16_step_chain_ms_per_step": round(bf16_ms, 5),
        },
        "roofline": {
            "kernel": "fp8_step_kernel (e4m3 QK^T and PV, v_mfma_scale_f32_32x32x64_f8f6f4 with unit scales)", "bound": "mfma",
            "achieved": round(achieved, 2), "peak": PEAK_FP8_TFLOPS, "unit": "TFLOP/s",
            "frac": round(achieved / PEAK_FP8_TFLOPS, 4), "traffic": None, "launches_per_step": n_launch,
            "avg_launch_ms": round(avg, 5),
        },
        "cpu_baseline": None,
        "check": {"max_abs_dout": eo, "max_abs_dlse": el},
    }
    print(json.dumps(res), flush=True)


def copy_probe(mib, reps):
    """Plain device copy of ``mib`` MiB (torch copy kernel), for counter calibration.

    Each launch reads and writes exactly mib MiB; FETCH_SIZE / WRITE_SIZE of
    this kernel give the counters' scale against known bytes.
    """
    import torch
    n = mib * (1 << 20) // 4
    x = torch.ones(n, dtype=torch.float32, device="cuda:0")
    y = torch.empty_like(x)
    for _ in range(reps):
        y.copy_(x)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes_read": n * 4, "copy_probe_bytes_written": n * 4, "launches": reps}),
          flush=True)


def bench_merge(args, w, stream):
    """The standalone log-sum-exp merge (cp_attn_merge) at the rank share's
    shape: fp32 (O, LSE) pairs [B,H,2L,D] / [B,H,2L] merged in place, with the
    bf16 finalize.  Inputs are seeded: O ~ N(0, 1), LSE ~ N(0, 4) with one row
    in 16 of each operand -inf (an empty partial).  HBM-bound: per row the
    call reads two (O, LSE) pairs and writes one, plus the bf16 row, so the
    algorithmic bytes are B*H*2L*(3*4*D + 3*4 + 2*D).  Repeated calls merge the
    same partial into the evolving accumulator, which stays finite: each O row
    is a convex combination of finite rows, and after n calls
    exp(LSE) = exp(LSE_0) + n exp(LSE_part)."""
    import torch
    import long_sequence_causal_cp_amd as cp

    dev = torch.device("cuda:0")
    B, H, D, Sq = w.B, w.H, w.D, 2 * w.chunk_len
    g = torch.Generator().manual_seed(7000 + w.seed)

    def pair():
        o = torch.randn((B, H, Sq, D), generator=g)
        l = 2.0 * torch.randn((B, H, Sq), generator=g)
        l[torch.rand((B, H, Sq), generator=g) < 1.0 / 16] = float("-inf")
        return o.to(dev), l.to(dev)

    o_acc, lse_acc = pair()
    o_part, lse_part = pair()
    out = torch.empty((B, H, Sq, D), dtype=torch.bfloat16, device=dev)
    nbytes = B * H * Sq * (3 * 4 * D + 3 * 4 + 2 * D)

    # one call checked by properties: the merged LSE is at least either input's, everything finite
    l_before = torch.maximum(lse_acc, lse_part)
    cp.cp_attn_merge(o_acc, lse_acc, o_part, lse_part, out, stream=stream)
    torch.cuda.synchronize()
    ok = bool(torch.all((lse_acc >= l_before) | torch.isneginf(l_before))) and bool(torch.isfinite(o_acc).all()) \
        and bool(torch.isfinite(out.float()).all())
    both_empty = torch.isneginf(l_before)
    ok = ok and bool(torch.isneginf(lse_acc[both_empty]).all())
    assert ok, "merge property check failed"

    def step():
        cp.cp_attn_merge(o_acc, lse_acc, o_part, lse_part, out, stream=stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(args.steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = ev0.elapsed_time(ev1) / args.steps
    gbs = nbytes / (ms * 1e-3) / 1e9
    print(f"[bench merge] {w.describe()} rank share {B}x{H}x{Sq}x{D}: {ms * 1e3:.2f} us per merge, "
          f"{gbs:.0f} GB/s of {nbytes / 1e6:.1f} MB", file=sys.stderr, flush=True)
    res = {
        "metric": "HBM GB/s of the standalone LSE merge (cp_attn_merge, in place, with bf16 finalize) on one "
                  "CP-rank share; % of 8 TB/s",
        "value": round(gbs, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms, 5), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f32", "data": "synthetic",
        "config": {
            "workload": f"{w.name}: rank share of cp={w.cp}, (O, LSE) fp32 [B={B}, H={H}, {Sq}, D={D}] pairs, "
                        "one row in 16 of each operand empty",
            "seq_len": w.S, "cp": w.cp, "B": B, "H": H, "D": D, "rows": B * H * Sq,
            "bytes_per_merge": nbytes, "wall_s_timed": round(wall, 4),
        },
        "roofline": {
            "kernel": "merge_kernel", "bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS,
            "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4), "traffic": kernel_traffic(w.name, "merge_kernel"),
            "launches_per_step": 1,
            "avg_launch_ms": round(ms, 5),
        },
        "cpu_baseline": None,
    }
    print(json.dumps(res), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=30,
                    help="untimed forwards first; after host-side setup the GPU needs ~30 ms of load to reach steady clocks")
    ap.add_argument("--workload", default="s32k_cp8")
    ap.add_argument("--rank", type=int, default=0)
    ap.add_argument("--cpu-budget", type=float, default=15.0, help="seconds of oracle timing (0 = skip)")
    ap.add_argument("--no-settle", dest="settle", action="store_false",
                    help="skip the untimed clock-settling forwards between warm-up and the timed region")
    ap.add_argument("--traffic-json", default=os.path.join(ROOT, "profiles", "step_kernel_s32k_cp8_traffic.json"))
    ap.add_argument("--pass", dest="pass_", choices=("fwd", "bwd", "allgather", "fp8", "merge"), default="fwd",
                    help="fwd: the ring forward (headline); bwd: the rank's backward ring steps; allgather: "
                         "the rank's queries against the gathered keys of the whole sequence in one step; fp8: "
                         "the share's ring steps in fp8 (cp_attn_step_fwd_fp8 per step); merge: the standalone "
                         "LSE merge (cp_attn_merge) at the share's shape")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="only run a plain copy of this many MiB --steps times (counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU's rank share only; runs on more than one GPU are not "
              "supported (use --gpus 1)", file=sys.stderr)
        sys.exit(2)

    if args.copy_probe_mib > 0:
        copy_probe(args.copy_probe_mib, args.steps)
        return

    import numpy as np
    import torch
    import workloads
    import long_sequence_causal_cp_amd as cp

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    cp.load_library()
    dev = torch.device("cuda:0")
    w = workloads.get(args.workload)
    L, N, r = w.chunk_len, w.cp, args.rank
    if args.pass_ == "merge":
        return bench_merge(args, w, torch.cuda.current_stream())
    Q, K, V = workloads.make_qkv(w)

    def gather(x, t):
        idx = torch.cat([torch.arange(s, s + t.chunk_len) for s in t.starts()])
        return x.index_select(2, idx).contiguous().to(dev)

    q_tab = cp.cp_zigzag_chunks(N, r, L, 0)[0]
    rank_kv = {}
    for src in range(N):       # every rank's K/V block resident in HBM
        t = cp.cp_zigzag_chunks(N, src, L, 0)[0]
        rank_kv[src] = (gather(K, t), gather(V, t), t)
    kv_tabs, ks, vs = [], [], []
    for j in range(N):
        src = (r - j) % N
        kk, vv, t = rank_kv[src]
        ks.append(kk)
        vs.append(vv)
        kv_tabs.append(t)
    q = gather(Q, q_tab)
    B, H, Sq, D = q.shape
    Skv = ks[0].shape[2]
    out = torch.empty_like(q)
    lse = torch.empty((B, H, Sq), dtype=torch.float32, device=dev)
    ws = torch.empty(cp.cp_ring_attn_workspace_bytes(B, H, Skv, D, Sq), dtype=torch.uint8, device=dev)
    copy_stream = torch.cuda.Stream()
    stream = torch.cuda.current_stream()

    def step():
        cp.cp_ring_attn_fwd(q, q_tab, ks, vs, kv_tabs, out, lse, w.scale, ws, stream=stream,
                            copy_stream=copy_stream)

    if args.pass_ == "bwd":
        step()
        return bench_backward(args, w, Q, K, V, q, q_tab, ks, vs, kv_tabs, out, lse, stream, gather)
    if args.pass_ == "allgather":
        return bench_allgather(args, w, Q, K, V, q, q_tab, kv_tabs, stream)
    if args.pass_ == "fp8":
        return bench_fp8(args, w, Q, K, V, q_tab, kv_tabs, stream)

    pairs = visible_pairs(q_tab, kv_tabs)
    flops = 4.0 * D * B * H * pairs

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    settle_n, settle_ms = settle(step, stream) if args.settle else (0, None)
    print(f"[bench] {w.describe()} rank {r}: warmup {args.warmup} done, clocks settled after {settle_n} more "
          f"forwards ({settle_ms} ms each)", file=sys.stderr, flush=True)

    # timed region: exactly K steps between two HIP events on the launch stream
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(args.steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    gpu_ms = ev0.elapsed_time(ev1)
    ms_per_step = gpu_ms / args.steps
    value = flops / (ms_per_step * 1e-3) / 1e12
    out_timed = out.clone()
    lse_timed = lse.clone()

    # kernel-timing region: K more steps in which the library brackets every
    # step-kernel launch with two HIP events on its stream.  Kept apart from
    # the timed region because each bracketing pair adds a few microseconds
    # between launches.
    cp.cp_profile_enable(True)
    ek0, ek1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ek0.record(stream)
    for _ in range(args.steps):
        step()
    ek1.record(stream)
    torch.cuda.synchronize()
    kern = cp.cp_profile_read_named(8192)
    cp.cp_profile_enable(False)
    kern_ms = [t for t, _ in kern]
    ms_per_step_instrumented = ek0.elapsed_time(ek1) / args.steps

    # per-forward times (median), and the forward with every staging copy run
    # in order on the launch stream (no copy/compute overlap)
    def timed_each(fn, n):
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
        for e0, e1 in evs:
            e0.record(stream)
            fn()
            e1.record(stream)
        torch.cuda.synchronize()
        return [e0.elapsed_time(e1) for e0, e1 in evs]

    def step_in_order():
        cp.cp_ring_attn_fwd(q, q_tab, ks, vs, kv_tabs, out, lse, w.scale, ws, stream=stream, copy_stream=stream)

    median_ms = statistics.median(timed_each(step, args.steps))
    step_in_order()
    no_overlap_ms = statistics.median(timed_each(step_in_order, args.steps))
    props = torch.cuda.get_device_properties(dev)

    # the plan the driver ran: launches per forward and the fp32 running-O
    # round trips between them (read when merging, written when not final)
    plan = cp.cp_ring_attn_fwd_plan(q_tab, kv_tabs)
    launches_per_step = len(plan)
    n_launch = len(kern_ms)
    assert n_launch == launches_per_step * args.steps, (n_launch, launches_per_step, args.steps)
    avg_kernel_ms = statistics.fmean(kern_ms)
    kernel_names = sorted(set(n for _, n in kern))
    # a ring forward's algorithmic flops spread over its launches (the launches
    # differ in size: step 0 alone, later steps in groups)
    per_launch_flops = flops / launches_per_step
    achieved = per_launch_flops / (avg_kernel_ms * 1e-3) / 1e12
    # algorithmic bytes of the share: Q once, K and V of every ring step once,
    # out and LSE once; the running-O round trips and the staging copies are
    # artefacts of the per-launch design and of the one-GPU replay, reported apart
    rows = B * H * Sq
    alg_bytes = rows * D * 2 + N * 2 * B * H * Skv * D * 2 + rows * D * 2 + rows * 4
    o_chunk = B * H * L * D * 4
    o_run_bytes = sum(o_chunk * (bool(f & cp.CP_PLAN_MERGE) + bool(f & cp.CP_PLAN_WRITE_O))
                      for _, _, fl in plan for f in fl.values())
    staging_bytes = sum(2 * 2 * B * H * Skv * D * 2 * cnt for first, cnt, _ in plan if first > 0)
    # HBM bytes per launch from the FETCH_SIZE / WRITE_SIZE counters, only if they
    # were taken on this workload and on the kernel source that is built now
    traffic = None
    if os.path.exists(args.traffic_json):
        try:
            from long_sequence_causal_cp_amd.prof_summary import kernel_source_sha256
            with open(args.traffic_json) as f:
                tj = json.load(f)
            if tj.get("workload") == w.name and tj.get("kernel_source_sha256") == kernel_source_sha256():
                traffic = round(tj["bytes_per_launch"])
        except (OSError, ValueError, KeyError):
            traffic = None

    # parity of the timed forwards' result: every row of every (batch, head)
    # the cpu_baseline leg computed with the oracle (all heads on a machine whose
    # host finishes them within the budget), else a few rows of head (0, 0)
    cpu, ref = None, {}
    if args.cpu_budget > 0:
        cpu = cpu_baseline(w, r, args.cpu_budget, Q, K, V, keep=ref)
    o_gpu = out_timed.float().cpu().numpy()
    l_gpu = lse_timed.cpu().numpy()
    if ref:
        eo = max(float(np.max(np.abs(o_gpu[b, h] - ro))) for (b, h), (ro, _) in ref.items())
        el = max(float(np.max(np.abs(l_gpu[b, h] - rl))) for (b, h), (_, rl) in ref.items())
        checked = f"all {Sq} rows of {len(ref)} of {B * H} (batch, head) pairs"
    else:
        sel = np.array([0, L - 1, L, 2 * L - 1])
        ro, rl = cpu_baseline_rows(w, r, Q, K, V, sel)
        eo = float(np.max(np.abs(o_gpu[0, 0, sel] - ro)))
        el = float(np.max(np.abs(l_gpu[0, 0, sel] - rl)))
        checked = "rows 0, L-1, L, 2L-1 of head (0, 0)"
    ok = bool(np.isfinite(o_gpu).all() and np.isfinite(l_gpu).all()) and eo <= 2e-2 and el <= 1e-3
    print(f"[bench] timed {args.steps} steps: {ms_per_step:.4f} ms/step, {value:.1f} TFLOP/s; "
          f"step kernel avg {avg_kernel_ms:.4f} ms over {n_launch} launches ({', '.join(kernel_names)}); "
          f"parity on {checked}: max|dout| {eo:.2e} max|dlse| {el:.2e}", file=sys.stderr, flush=True)
    if not ok:
        print(f"[bench] PARITY FAILURE: max|dout| {eo:.3e} (bound 2e-2), max|dlse| {el:.3e} (bound 1e-3)",
              file=sys.stderr, flush=True)
        sys.exit(3)

    res = {
        "metric": "causal-effective attention TFLOP/s per CP-rank share; % of bf16 MFMA peak",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "settle_forwards": settle_n,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "pct_of_bf16_peak": round(100.0 * value / PEAK_BF16_TFLOPS, 2),
        "config": {
            "workload": f"{w.name}: causal ring attention, one rank's share (rank {r} of cp={N}), "
                        f"B={B} H={H} D={D} S={w.S}, zigzag chunks of {L}, {N} ring steps of {Skv} keys",
            "seq_len": w.S, "cp": N, "rank": r, "B": B, "H": H, "D": D,
            "visible_pairs_per_head": pairs, "flop_per_step": flops,
            "wall_s_timed": round(wall, 4),
        },
        "roofline": {
            "kernel": " + ".join(kernel_names) + " (QK^T, mask, online softmax, PV, fused LSE merge)",
            "bound": "mfma",
            "achieved": round(achieved, 2),
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
            "traffic": traffic,
            "traffic_gb_per_s": (round(traffic / (avg_kernel_ms * 1e-3) / 1e9, 1) if traffic else None),
            "alg_bytes_per_step": alg_bytes,
            "alg_bytes_per_launch": round(alg_bytes / launches_per_step),
            "traffic_over_alg_bytes": (round(traffic / (alg_bytes / launches_per_step), 3) if traffic else None),
            "o_run_bytes_per_step": o_run_bytes,
            "staging_copy_bytes_per_step": staging_bytes,
            "launches": n_launch,
            "launches_per_step": launches_per_step,
            "flop_per_launch": per_launch_flops,
            "avg_launch_ms": round(avg_kernel_ms, 5),
            "launch_ms_first_forward": [round(t, 5) for t in kern_ms[:launches_per_step]],
            "ms_per_step_with_kernel_events": round(ms_per_step_instrumented, 5),
            "kernel_ms_per_step": round(avg_kernel_ms * launches_per_step, 5),
        },
        "timing": {
            "ms_per_step_median": round(median_ms, 5),
            "ms_per_step_no_overlap_median": round(no_overlap_ms, 5),
            "settle_ms_last_batch": round(settle_ms, 5) if settle_ms else None,
            "note": "median over --steps forwards, each bracketed by HIP events; no_overlap runs every "
                    "staging copy in order on the launch stream; the timed region starts after --warmup "
                    "forwards and settle_forwards more, run until three batches of five agree within 1%",
        },
        "device": {"name": props.name, "arch": getattr(props, "gcnArchName", ""),
                   "compute_units": props.multi_processor_count},
        "cpu_baseline": cpu,
        "check": {"max_abs_dout": eo, "max_abs_dlse": el, "rows": checked, "out_tol": 2e-2, "lse_tol": 1e-3},
    }
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
