"""The oracle's pins are strong enough: planted mistakes in the oracle fail them.

Each mutant is a plausible slip in the fp64 definition (dropped scale, strict
instead of inclusive diagonal, transposed operand, missing normalisation,
dropped max term in the LSE, an off-by-one key index, a wrong merge sign).
The mutation is planted in a copy of the oracle function on the CPU and the
pin tests are re-run against it; every mutant must make at least one fail.
"""
import numpy as np
import pytest

import oracle.attention as oatt
import oracle.merge as omerge
import test_oracle_pins as pins


def _mutant(kind):
    def f(q, q_pos, k, v, k_pos, scale):
        q = np.asarray(q, np.float64)
        k = np.asarray(k, np.float64)
        v = np.asarray(v, np.float64)
        q_pos = np.asarray(q_pos, np.int64)
        k_pos = np.asarray(k_pos, np.int64)
        n = q.shape[0]
        out = np.zeros((n, v.shape[1]))
        lse = np.full(n, -np.inf)
        if n == 0 or k.shape[0] == 0:
            return out, lse
        sc = 1.0 if kind == "no_scale" else scale
        s = sc * (q @ k.T)
        if kind == "transposed" and q.shape[0] == k.shape[0]:
            s = s.T
        if kind == "strict_mask":
            vis = k_pos[None, :] < q_pos[:, None]
        elif kind == "no_mask":
            vis = np.ones((n, k.shape[0]), bool)
        else:
            vis = k_pos[None, :] <= q_pos[:, None]
        s = np.where(vis, s, -np.inf)
        has = vis.any(axis=1)
        sr = s[has]
        m = sr.max(axis=1)
        e = np.exp(sr - m[:, None])
        z = e.sum(axis=1)
        vv = np.roll(v, 1, axis=0) if kind == "v_off_by_one" else v
        o = e @ vv
        out[has] = o if kind == "no_normalise" else o / z[:, None]
        lse[has] = np.log(z) if kind == "lse_drops_max" else m + np.log(z)
        return out, lse
    return f


PIN_CALLS = [
    lambda: pins.test_brute_force_random(33, 8, 2),
    lambda: pins.test_brute_force_random(40, 64, 4),
    pins.test_closed_form_q_zero,
    pins.test_closed_form_first_token,
    pins.test_softmax_rows_sum_to_one_and_constant_v,
    pins.test_sdpa_library_case,
    pins.test_later_keys_do_not_leak,
]


@pytest.mark.parametrize("kind", ["no_scale", "transposed", "strict_mask", "no_mask",
                                  "v_off_by_one", "no_normalise", "lse_drops_max"])
def test_attention_mutant_is_caught(kind, monkeypatch):
    monkeypatch.setattr(oatt, "masked_attention", _mutant(kind))
    failed = 0
    for call in PIN_CALLS:
        try:
            call()
        except (AssertionError, ValueError, IndexError):
            failed += 1
    assert failed >= 1, f"mutant {kind} passed every pin"


def _merge_wrong_sign(o1, l1, o2, l2):
    l = np.logaddexp(l1, l2)
    o = np.exp(l - l1)[..., None] * o1 + np.exp(l - l2)[..., None] * o2
    return o, l


def _merge_plain_sum(o1, l1, o2, l2):
    return o1 + o2, np.logaddexp(l1, l2)


@pytest.mark.parametrize("bad", [_merge_wrong_sign, _merge_plain_sum])
def test_merge_mutant_is_caught(bad, monkeypatch):
    monkeypatch.setattr(omerge, "lse_merge", bad)
    monkeypatch.setattr(pins.oracle, "lse_merge", bad)
    with pytest.raises(AssertionError):
        pins.test_merge_of_random_split_equals_full(0)
