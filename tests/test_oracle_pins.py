"""Pins for the fp64 oracle against facts other than the oracle itself.

* scalar brute force (pure Python loops) on tiny inputs;
* closed forms: Q = 0 gives LSE_i = ln(i+1) and out_i = mean(v_0..v_i);
  the first token gives out_0 = v_0 and LSE_0 = tau <q_0, k_0>;
* invariants: merge of any blockwise key split (random cuts, random order,
  and the ring's zigzag blocks) equals the full result; V = 1 gives 1;
  constant V is returned; shifting every key by u leaves out unchanged and
  moves LSE_i by tau <q_i, u>;
* library special case: PyTorch's fp64 scaled_dot_product_attention with
  is_causal=True, and torch.logsumexp of the masked scores;
* the zigzag worked example printed on the RingAttention+FlashAttention page
  (section 5, item 1), in tests/golden/zigzag_cp4.txt;
* ring order and work balance: over N steps each rank sees every block once,
  and every rank's visible-pair count is the same, 2 N L^2 + L.
"""
import math
import os

import numpy as np
import pytest
import torch

import oracle
import workloads

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def brute_force(q, k, v, scale):
    """Causal attention with Python scalars only: no numpy arithmetic."""
    S, D = len(q), len(q[0])
    out, lse = [], []
    for i in range(S):
        scores = []
        for j in range(i + 1):
            acc = 0.0
            for t in range(D):
                acc += float(q[i][t]) * float(k[j][t])
            scores.append(scale * acc)
        m = max(scores)
        w = [math.exp(s - m) for s in scores]
        z = math.fsum(w)
        row = []
        for t in range(v.shape[1]):
            row.append(math.fsum(w[j] * float(v[j][t]) for j in range(i + 1)) / z)
        out.append(row)
        lse.append(m + math.log(z))
    return np.array(out), np.array(lse)


def rand_qkv(shape, seed, scale=1.0):
    q, k, v = workloads.make_qkv_scaled(shape, seed, q_scale=scale, k_scale=scale)
    return oracle.to_f64(q), oracle.to_f64(k), oracle.to_f64(v)


@pytest.mark.parametrize("S,D,seed", [(1, 4, 0), (7, 4, 1), (33, 8, 2), (64, 8, 3), (40, 64, 4)])
def test_brute_force_random(S, D, seed):
    q, k, v = rand_qkv((S, D), seed, scale=2.0)
    tau = 1.0 / math.sqrt(D)
    ob, lb = brute_force(q, k, v, tau)
    oo, lo = oracle.causal_attention_rows(q, k, v, np.arange(S))
    assert np.max(np.abs(oo - ob)) <= 1e-12
    assert np.max(np.abs(lo - lb)) <= 1e-12


def test_brute_force_tiny_workload_one_head():
    """The tiny workload's first head, every row, by brute force."""
    w = workloads.get("tiny")
    Q, K, V = workloads.make_qkv(w)
    q, k, v = (oracle.to_f64(t)[0, 0] for t in (Q, K, V))
    ob, lb = brute_force(q, k, v, w.scale)
    oo, lo = oracle.causal_attention_rows(q, k, v, np.arange(w.S), w.scale)
    assert np.max(np.abs(oo - ob)) <= 1e-12
    assert np.max(np.abs(lo - lb)) <= 1e-12


def test_rows_subset_and_order_independent():
    q, k, v = rand_qkv((2, 3, 700, 16), 5)
    full_o, full_l = oracle.causal_attention_rows(q, k, v, np.arange(700))
    rows = np.array([699, 0, 513, 512, 511, 1, 350])
    o, l = oracle.causal_attention_rows(q, k, v, rows)
    # blocking changes only BLAS summation order
    assert np.max(np.abs(o - full_o[..., rows, :])) <= 1e-13
    assert np.max(np.abs(l - full_l[..., rows])) <= 1e-13


def test_closed_form_q_zero():
    S, D = 300, 16
    _, k, v = rand_qkv((S, D), 6)
    q = np.zeros((S, D))
    o, l = oracle.causal_attention_rows(q, k, v, np.arange(S))
    n = np.arange(1, S + 1)
    assert np.max(np.abs(l - np.log(n))) <= 1e-12
    mean = np.cumsum(v, axis=0) / n[:, None]
    assert np.max(np.abs(o - mean)) <= 1e-12


def test_closed_form_first_token():
    q, k, v = rand_qkv((3, 2, 50, 32), 7, scale=3.0)
    o, l = oracle.causal_attention_rows(q, k, v, np.array([0, 10]))
    assert np.max(np.abs(o[..., 0, :] - v[..., 0, :])) <= 1e-14
    dot = (q[..., 0, :] * k[..., 0, :]).sum(-1) / math.sqrt(32)
    assert np.max(np.abs(l[..., 0] - dot)) <= 1e-12


def test_softmax_rows_sum_to_one_and_constant_v():
    q, k, _ = rand_qkv((2, 200, 64), 8, scale=2.0)
    ones = np.ones((2, 200, 64))
    o, _ = oracle.causal_attention_rows(q, k, ones, np.arange(200))
    assert np.max(np.abs(o - 1.0)) <= 1e-12
    c = np.linspace(-3, 3, 64)
    const_v = np.broadcast_to(c, (2, 200, 64)).copy()
    o, _ = oracle.causal_attention_rows(q, k, const_v, np.arange(200))
    assert np.max(np.abs(o - c)) <= 1e-12


def test_key_shift_invariance():
    q, k, v = rand_qkv((150, 32), 9)
    u = np.random.default_rng(0).standard_normal(32)
    o1, l1 = oracle.causal_attention_rows(q, k, v, np.arange(150))
    o2, l2 = oracle.causal_attention_rows(q, k + u, v, np.arange(150))
    assert np.max(np.abs(o2 - o1)) <= 1e-11
    assert np.max(np.abs(l2 - (l1 + q @ u / math.sqrt(32)))) <= 1e-11


def test_later_keys_do_not_leak():
    """Changing keys/values after position p leaves rows <= p unchanged."""
    q, k, v = rand_qkv((120, 16), 10)
    o1, l1 = oracle.causal_attention_rows(q, k, v, np.arange(120))
    k2, v2 = k.copy(), v.copy()
    k2[61:] += 5.0
    v2[61:] *= -7.0
    o2, l2 = oracle.causal_attention_rows(q, k2, v2, np.arange(120))
    assert np.max(np.abs(o1[:61] - o2[:61])) <= 1e-13
    assert np.max(np.abs(l1[:61] - l2[:61])) <= 1e-13
    assert np.max(np.abs(o1[61:] - o2[61:])) > 1e-3


def test_sdpa_library_case():
    S, D = 384, 64
    q, k, v = rand_qkv((2, 2, S, D), 11, scale=1.5)
    o, l = oracle.causal_attention_rows(q, k, v, np.arange(S))
    tq, tk, tv = (torch.from_numpy(x) for x in (q, k, v))
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=True)
    assert np.max(np.abs(o - ref.numpy())) <= 1e-12
    s = (tq @ tk.transpose(-1, -2)) / math.sqrt(D)
    mask = torch.ones(S, S, dtype=torch.bool).triu(1)
    ref_l = torch.logsumexp(s.masked_fill(mask, float("-inf")), dim=-1)
    assert np.max(np.abs(l - ref_l.numpy())) <= 1e-12


def test_masked_attention_partial_matches_brute_force():
    """Partial over an arbitrary key subset at absolute positions, incl. empty rows."""
    rng = np.random.default_rng(12)
    q, k, v = rand_qkv((96, 8), 12)
    k_pos = np.sort(rng.choice(96, size=30, replace=False))
    q_pos = np.sort(rng.choice(96, size=25, replace=False))
    o, l = oracle.masked_attention(q[q_pos], q_pos, k[k_pos], v[k_pos], k_pos, 0.5)
    for a, p in enumerate(q_pos):
        vis = [j for j in k_pos if j <= p]
        if not vis:
            assert l[a] == -np.inf and np.all(o[a] == 0)
            continue
        s = [0.5 * math.fsum(q[p][t] * k[j][t] for t in range(8)) for j in vis]
        m = max(s)
        w = [math.exp(x - m) for x in s]
        z = math.fsum(w)
        assert abs(l[a] - (m + math.log(z))) <= 1e-12
        for t in range(8):
            assert abs(o[a][t] - math.fsum(wi * v[j][t] for wi, j in zip(w, vis)) / z) <= 1e-12


@pytest.mark.parametrize("seed", range(4))
def test_merge_of_random_split_equals_full(seed):
    rng = np.random.default_rng(100 + seed)
    S, D = 257, 16
    q, k, v = rand_qkv((S, D), 200 + seed, scale=2.5)
    tau = 1.0 / math.sqrt(D)
    pos = np.arange(S)
    full_o, full_l = oracle.causal_attention_rows(q, k, v, pos)
    cuts = np.sort(rng.choice(np.arange(1, S), size=rng.integers(1, 8), replace=False))
    blocks = np.split(rng.permutation(S) if seed % 2 else pos, cuts)
    rng.shuffle(blocks)
    acc_o = np.zeros((S, D))
    acc_l = np.full(S, -np.inf)
    for b in blocks:
        b = np.sort(b)
        po, pl = oracle.masked_attention(q, pos, k[b], v[b], b, tau)
        acc_o, acc_l = oracle.lse_merge(acc_o, acc_l, po, pl)
    assert np.max(np.abs(acc_o - full_o)) <= 1e-12
    assert np.max(np.abs(acc_l - full_l)) <= 1e-12


def test_merge_empty_operands():
    o = np.arange(6.0).reshape(2, 3)
    l = np.array([0.5, -1.0])
    z = np.zeros((2, 3))
    ninf = np.full(2, -np.inf)
    mo, ml = oracle.lse_merge(o, l, z, ninf)
    assert np.array_equal(mo, o) and np.array_equal(ml, l)
    mo, ml = oracle.lse_merge(z, ninf, o, l)
    assert np.array_equal(mo, o) and np.array_equal(ml, l)
    mo, ml = oracle.lse_merge(z, ninf, z, ninf)
    assert np.all(mo == 0) and np.all(np.isneginf(ml)) and not np.isnan(mo).any()


def test_zigzag_golden_worked_example():
    rows = []
    with open(os.path.join(GOLDEN, "zigzag_cp4.txt")) as f:
        for line in f:
            if line.strip() and not line.startswith("#"):
                rows.append(tuple(int(x) for x in line.split()))
    assert len(rows) == 4
    for r, a, b in rows:
        assert oracle.zigzag_chunk_ids(4, r) == (a, b)


def test_zigzag_tiny_rank0():
    w = workloads.get("tiny")
    assert oracle.zigzag_chunk_ids(w.cp, 0) == (0, 3)
    pos = oracle.local_positions(w.S, w.cp, 0)
    assert np.array_equal(pos, np.r_[0:64, 192:256])


@pytest.mark.parametrize("cp", [1, 2, 3, 4, 8, 16])
def test_ring_order_visits_every_block_once(cp):
    for r in range(cp):
        srcs = [oracle.ring_source(r, j, cp) for j in range(cp)]
        assert srcs[0] == r
        assert sorted(srcs) == list(range(cp))
        # the block a rank uses at step j+1 is the one its predecessor used at step j
        for j in range(cp - 1):
            assert oracle.ring_source(r, j + 1, cp) == oracle.ring_source((r - 1) % cp, j, cp)


@pytest.mark.parametrize("name", list(workloads.WORKLOADS))
def test_work_balance_every_rank(name):
    """Visible pairs per rank are equal, 2 N L^2 + L, counted step by step over the ring."""
    w = workloads.get(name)
    N, L = w.cp, w.chunk_len
    counts = []
    for r in range(N):
        qp = oracle.local_positions(w.S, N, r)
        seen = []
        total = 0
        for j in range(N):
            kp = oracle.ring_kv_positions(w.S, N, r, j)
            seen.append(kp)
            total += oracle.visible_pairs(qp, kp)
        assert np.array_equal(np.sort(np.concatenate(seen)), np.arange(w.S))
        counts.append(total)
    assert counts == [2 * N * L * L + L] * N


def test_visible_pairs_brute_force_small():
    for S, cp in [(16, 2), (24, 3), (32, 4)]:
        for r in range(cp):
            qp = oracle.local_positions(S, cp, r)
            n = sum(1 for p in qp for j in range(S) if j <= p)
            assert oracle.visible_pairs(qp, np.arange(S)) == n
    # contiguous sharding is unbalanced: the last rank does the most work
    S, cp = 64, 4
    c = [oracle.visible_pairs(oracle.contiguous_positions(S, cp, r), np.arange(S)) for r in range(cp)]
    assert c[0] < c[-1]


def test_zigzag_and_contiguous_shares_reassemble():
    S, cp, D = 128, 4, 16
    q, k, v = rand_qkv((2, S, D), 13)
    full_o, full_l = oracle.causal_attention_rows(q, k, v, np.arange(S))
    zz_o = np.zeros_like(full_o)
    zz_l = np.zeros_like(full_l)
    ct_o = np.zeros_like(full_o)
    for r in range(cp):
        pos = oracle.local_positions(S, cp, r)
        # ring replay in the oracle: merge the rank's partials step by step
        acc_o = np.zeros((2, len(pos), D))
        acc_l = np.full((2, len(pos)), -np.inf)
        for j in range(cp):
            kp = oracle.ring_kv_positions(S, cp, r, j)
            for h in range(2):
                po, pl = oracle.masked_attention(q[h][pos], pos, k[h][kp], v[h][kp], kp, 0.25)
                acc_o[h], acc_l[h] = oracle.lse_merge(acc_o[h], acc_l[h], po, pl)
        zz_o[:, pos] = acc_o
        zz_l[:, pos] = acc_l
        cpos = oracle.contiguous_positions(S, cp, r)
        ct_o[:, cpos], _ = oracle.causal_attention_rows(q, k, v, cpos)
    assert np.max(np.abs(zz_o - full_o)) <= 1e-12
    assert np.max(np.abs(zz_l - full_l)) <= 1e-12
    assert np.max(np.abs(ct_o - full_o)) <= 1e-12
