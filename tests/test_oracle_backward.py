"""Pins for the fp64 backward oracle (gradients of causal attention).

Independent of the oracle's own arithmetic:

* central finite differences of the loss sum <dO, out> through the scalar
  brute-force forward (pure Python loops) on tiny inputs;
* PyTorch fp64 autograd of scaled_dot_product_attention(is_causal=True)
  (a library special case, not the oracle);
* closed forms: Q = 0 (uniform weights: dV_j = sum_{i>=j} dO_i/(i+1),
  dK = 0, dQ_i = tau/(i+1) sum_{j<=i} <dO_i, v_j - mean_i v> k_j); constant
  V (the output does not move: dQ = dK = 0); the first token (one key:
  dQ_0 = 0);
* invariants: sum_j dK_j = 0 (every row of dS sums to zero), sum_j dV_j =
  sum_i dO_i (every row of P sums to one), dO = 0 gives zeros;
* splits: over random key blocks the dQ parts add up to dQ and the blocks'
  dK, dV are the rows of the full ones; over the zigzag ring of N ranks, the
  contributions of every rank's queries to one rank's K/V block add up to
  that block's rows of dK and dV ([MLM] section 2: the backward sends the
  gradients back along the path the blocks came).

Planted mistakes in a copy of the oracle (dropped Delta term, missing scale,
unnormalised P, transposed dS, strict diagonal) each fail at least one pin.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import oracle.backward as obwd
import workloads
from test_oracle_pins import brute_force


def _rand(shape, seed, scale=1.0):
    rng = np.random.default_rng(seed)
    return [scale * rng.standard_normal(shape) for _ in range(4)]  # Q, K, V, dO


def _loss_brute(Q, K, V, dO, tau):
    out, _ = brute_force(Q, K, V, tau)
    return float(np.sum(dO * out))


@pytest.mark.parametrize("S,D,seed", [(1, 3, 0), (5, 4, 1), (7, 3, 2)])
def test_finite_differences(S, D, seed):
    Q, K, V, dO = _rand((S, D), seed)
    tau = 1.0 / math.sqrt(D)
    dq, dk, dv = oracle.causal_attention_grad(Q, K, V, dO, tau)
    h = 1e-5
    for X, dX in ((Q, dq), (K, dk), (V, dv)):
        num = np.zeros_like(X)
        for idx in np.ndindex(*X.shape):
            x0 = X[idx]
            X[idx] = x0 + h
            lp = _loss_brute(Q, K, V, dO, tau)
            X[idx] = x0 - h
            lm = _loss_brute(Q, K, V, dO, tau)
            X[idx] = x0
            num[idx] = (lp - lm) / (2 * h)
        np.testing.assert_allclose(dX, num, rtol=1e-6, atol=1e-8)


@pytest.mark.parametrize("S,D,seed", [(64, 16, 3), (256, 64, 4)])
def test_torch_autograd_library_case(S, D, seed):
    Q, K, V, dO = _rand((S, D), seed)
    tau = 1.0 / math.sqrt(D)
    dq, dk, dv = oracle.causal_attention_grad(Q, K, V, dO, tau)
    q, k, v = (torch.tensor(x[None, None], dtype=torch.float64, requires_grad=True) for x in (Q, K, V))
    out = torch.nn.functional.scaled_dot_product_attention(q, k, v, is_causal=True, scale=tau)
    out.backward(torch.tensor(dO[None, None], dtype=torch.float64))
    for mine, ref in ((dq, q.grad), (dk, k.grad), (dv, v.grad)):
        np.testing.assert_allclose(mine, ref[0, 0].numpy(), rtol=1e-9, atol=1e-11)


def test_closed_form_q_zero():
    S, D = 24, 8
    _, K, V, dO = _rand((S, D), 5)
    Q = np.zeros((S, D))
    tau = 1.0 / math.sqrt(D)
    dq, dk, dv = oracle.causal_attention_grad(Q, K, V, dO, tau)
    dv_ref = np.array([sum(dO[i] / (i + 1) for i in range(j, S)) for j in range(S)])
    dq_ref = np.zeros((S, D))
    for i in range(S):
        vbar = V[:i + 1].mean(axis=0)
        dq_ref[i] = tau / (i + 1) * sum(float(dO[i] @ (V[j] - vbar)) * K[j] for j in range(i + 1))
    np.testing.assert_allclose(dv, dv_ref, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(dk, 0.0, atol=1e-14)
    np.testing.assert_allclose(dq, dq_ref, rtol=1e-11, atol=1e-13)


def test_constant_v_and_first_token():
    S, D = 17, 8
    Q, K, _, dO = _rand((S, D), 6, scale=2.0)
    V = np.tile(np.random.default_rng(7).standard_normal(D), (S, 1))
    dq, dk, _ = oracle.causal_attention_grad(Q, K, V, dO)
    np.testing.assert_allclose(dq, 0.0, atol=1e-12)
    np.testing.assert_allclose(dk, 0.0, atol=1e-12)
    Q, K, V, dO = _rand((S, D), 8)
    dq, _, _ = oracle.causal_attention_grad(Q, K, V, dO)
    np.testing.assert_allclose(dq[0], 0.0, atol=1e-14)   # one visible key: out_0 = v_0 whatever q_0 is


def test_row_sum_invariants():
    S, D = 40, 16
    Q, K, V, dO = _rand((S, D), 9, scale=1.5)
    dq, dk, dv = oracle.causal_attention_grad(Q, K, V, dO)
    np.testing.assert_allclose(dk.sum(axis=0), 0.0, atol=1e-11)
    np.testing.assert_allclose(dv.sum(axis=0), dO.sum(axis=0), rtol=1e-12, atol=1e-12)
    z = oracle.causal_attention_grad(Q, K, V, np.zeros_like(dO))
    for g in z:
        assert not np.any(g)


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_random_key_blocks_add_up(seed):
    S, D = 48, 8
    Q, K, V, dO = _rand((S, D), 10 + seed)
    tau = 1.0 / math.sqrt(D)
    dq, dk, dv = oracle.causal_attention_grad(Q, K, V, dO, tau)
    pos = np.arange(S)
    out, lse = oracle.masked_attention(Q, pos, K, V, pos, tau)
    rng = np.random.default_rng(seed)
    cuts = np.sort(rng.choice(np.arange(1, S), size=4, replace=False))
    blocks = np.split(pos, cuts)
    rng.shuffle(blocks)
    dq_sum = np.zeros_like(dq)
    for b in blocks:
        dq_b, dk_b, dv_b = oracle.masked_attention_grad(Q, pos, K[b], V[b], b, dO, out, lse, tau)
        dq_sum += dq_b
        np.testing.assert_allclose(dk_b, dk[b], rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(dv_b, dv[b], rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(dq_sum, dq, rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("N,L", [(2, 8), (4, 4)])
def test_zigzag_ring_backward_adds_up(N, L):
    S, D = 2 * N * L, 8
    Q, K, V, dO = _rand((S, D), 20 + N)
    tau = 1.0 / math.sqrt(D)
    dq, dk, dv = oracle.causal_attention_grad(Q, K, V, dO, tau)
    pos_all = np.arange(S)
    out, lse = oracle.masked_attention(Q, pos_all, K, V, pos_all, tau)
    dk_ring = np.zeros_like(dk)
    dv_ring = np.zeros_like(dv)
    for r in range(N):
        rows = oracle.local_positions(S, N, r)
        dq_r = np.zeros((len(rows), D))
        for j in range(N):
            src = (r - j) % N
            keys = oracle.local_positions(S, N, src)
            dq_b, dk_b, dv_b = oracle.masked_attention_grad(Q[rows], rows, K[keys], V[keys], keys, dO[rows],
                                                            out[rows], lse[rows], tau)
            dq_r += dq_b
            dk_ring[keys] += dk_b
            dv_ring[keys] += dv_b
        np.testing.assert_allclose(dq_r, dq[rows], rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(dk_ring, dk, rtol=1e-11, atol=1e-13)
    np.testing.assert_allclose(dv_ring, dv, rtol=1e-12, atol=1e-13)


def test_bf16_workload_shapes():
    """The seeded C1 draws (bf16-rounded, up-cast) go through without trouble."""
    w = workloads.get("tiny")
    Q, K, V = (oracle.to_f64(x)[0, 0] for x in workloads.make_qkv(w))
    dO = np.random.default_rng(1).standard_normal(Q.shape)
    dq, dk, dv = oracle.causal_attention_grad(Q, K, V, dO, w.scale)
    assert all(np.isfinite(g).all() for g in (dq, dk, dv))


# ---------------------------------------------------------------- planted mistakes
def _mutant(kind):
    def f(q, q_pos, k, v, k_pos, d_out, out, lse, scale):
        q, k, v, d_out, out, lse = (np.asarray(x, np.float64) for x in (q, k, v, d_out, out, lse))
        q_pos, k_pos = np.asarray(q_pos, np.int64), np.asarray(k_pos, np.int64)
        if kind == "strict_mask":
            vis = k_pos[None, :] < q_pos[:, None]
        else:
            vis = k_pos[None, :] <= q_pos[:, None]
        s = scale * (q @ k.T)
        shift = 0.0 if kind == "unnormalised_p" else lse[:, None]
        p = np.where(vis, np.exp(np.where(vis, s - shift, 0.0)), 0.0)
        dv = p.T @ d_out
        dp = d_out @ v.T
        delta = 0.0 if kind == "no_delta" else np.sum(d_out * out, axis=1)[:, None]
        ds = p * (dp - delta)
        sc = 1.0 if kind == "no_scale" else scale
        dq = sc * (ds @ k)
        dk = scale * ((ds if kind == "transposed_ds" else ds.T) @ q)
        return dq, dk, dv
    return f


PINS = [
    lambda: test_finite_differences(5, 4, 1),
    lambda: test_torch_autograd_library_case(64, 16, 3),
    test_closed_form_q_zero,
    test_constant_v_and_first_token,
    test_row_sum_invariants,
]


@pytest.mark.parametrize("kind", ["no_delta", "no_scale", "unnormalised_p", "transposed_ds", "strict_mask"])
def test_backward_mutant_is_caught(kind, monkeypatch):
    monkeypatch.setattr(obwd, "masked_attention_grad", _mutant(kind))
    failed = 0
    for call in PINS:
        try:
            call()
        except (AssertionError, ValueError, IndexError):
            failed += 1
    assert failed >= 1, f"mutant {kind} passed every pin"

