"""The error model behind the fp8 step's tolerance (CPU, fp64; no GPU).

Pins the model itself: e4m3 rounding is RNE with 3 mantissa bits; without the
rounding the kernel model is the exact result; its launch grouping is the ring
driver's; and the modelled output error is nonzero but well inside the worst
case of the rounding.
"""
import numpy as np
import torch

import oracle
from fp8_helpers import round_e4m3


def test_e4m3_rounding_is_round_to_nearest_with_three_mantissa_bits():
    # representable neighbours around 1: 1, 1.125; halfway 1.0625 ties to even (1.0)
    got = round_e4m3(np.array([1.0, 1.06, 1.0625, 1.07, 1.125, 448.0, 0.015625]))
    assert np.array_equal(got, [1.0, 1.0, 1.0, 1.125, 1.125, 448.0, 0.015625])


def test_fp8_error_model_on_the_workloads():
    """The fp8 step's output tolerance is derived from the kernel's rounding model (1.25 times its
    deviation on the compared rows); on the workloads the fp8 GPU test uses, the model's deviation is
    nonzero and well below the worst case of the e4m3 rounding, 2^-4 of max |v|."""
    import workloads
    from fp8_helpers import dequantize, lazy_model_error, quantize, ring_segments
    for name, H, rows in (("s8k_cp2", 1, 256), ("s32k_cp8", 1, 128)):
        w = workloads.get(name)
        Q, K, V = workloads.make_qkv(w, H=H)
        Qd, Kd, Vd = (dequantize(*quantize(x.float())) for x in (Q, K, V))
        L = w.chunk_len
        for r in (0, w.cp - 1):
            pos = oracle.local_positions(w.S, w.cp, r)
            local = np.unique(np.concatenate([np.random.default_rng(r).choice(len(pos), rows, replace=False),
                                              np.arange(4)]))
            tabs = [[(c * L, L) for c in sorted([(r - j) % w.cp, 2 * w.cp - 1 - (r - j) % w.cp])]
                    for j in range(w.cp)]
            e, _, _ = lazy_model_error(Qd[0, 0][pos], pos, local, Kd[0, 0], Vd[0, 0], ring_segments(tabs, True),
                                       w.scale)
            assert 1e-4 < e < np.max(np.abs(Vd[0, 0])) / 16 / 2, (name, r, e)


def test_lazy_model_without_rounding_is_the_exact_result():
    """The kernel model's lazy maximum, tile-wise rescaling and per-launch log-sum-exp merge are exact
    arithmetic: without the e4m3 rounding it reproduces the oracle, for peaked scores, several launches
    and chunk tables out of order."""
    from fp8_helpers import lazy_model, ring_segments
    rng = np.random.default_rng(0)
    S, D = 512, 16
    q, k = rng.standard_normal((S, D)) * 3, rng.standard_normal((S, D)) * 3
    v = rng.standard_normal((S, D))
    pos = np.arange(S)
    ro, rl = oracle.causal_attention_rows(q, k, v, pos, 0.25)
    for tables, grouped in (([[(0, 128), (384, 128)], [(128, 128), (256, 128)]], False),
                            ([[(256, 256)], [(0, 128)], [(128, 128)]], True)):
        segs = ring_segments(tables, grouped)
        o, l = lazy_model(q, k, v, pos, pos // 32, pos, segs, 0.25, rounding=False)
        assert np.max(np.abs(o - ro)) < 1e-12 and np.max(np.abs(l - rl)) < 1e-12
        o2, l2 = lazy_model(q, k, v, pos, pos // 32, pos, segs, 0.25)
        assert np.max(np.abs(l2 - rl)) < 1e-12          # the LSE uses the unrounded sums
        assert np.array_equal(o2[0], v[0])               # one key: p = 1 exactly
        assert 1e-3 < np.max(np.abs(o2 - ro)) < 0.5


def test_ring_segments_follow_the_driver_grouping():
    from fp8_helpers import ring_segments
    tabs = [[(j * 64, 64)] for j in range(8)]
    segs = ring_segments(tabs, grouped=True)
    assert [len(s) // 64 for s in segs] == [1, 3, 4]          # step 0, then 1-3 and 4-7
    assert [len(s) // 64 for s in ring_segments(tabs[:6], True)] == [1, 2, 3]
    assert [len(s) // 64 for s in ring_segments(tabs, False)] == [1] * 8
    assert np.array_equal(np.concatenate(segs), np.arange(512))
