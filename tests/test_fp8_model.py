"""The error model behind the fp8 step's tolerance (CPU, fp64; no GPU).

Pins the model itself: e4m3 rounding is RNE with 3 mantissa bits, and the
modelled output error is nonzero but well inside the stated bound.
"""
import numpy as np
import torch

import oracle
from fp8_helpers import round_e4m3


def test_e4m3_rounding_is_round_to_nearest_with_three_mantissa_bits():
    # representable neighbours around 1: 1, 1.125; halfway 1.0625 ties to even (1.0)
    got = round_e4m3(np.array([1.0, 1.06, 1.0625, 1.07, 1.125, 448.0, 0.015625]))
    assert np.array_equal(got, [1.0, 1.0, 1.0, 1.125, 1.125, 448.0, 0.015625])


def test_fp8_error_model_within_tolerance():
    """The fp8 step's output tolerance is derived from the e4m3 rounding of the
    probabilities (1.5 times this model's deviation on the compared rows); the
    model's deviation is nonzero and stays below 0.05 on the workloads the fp8
    GPU test uses."""
    import numpy as np
    import workloads
    from fp8_helpers import dequantize, emulated_error, quantize
    for name, H, rows in (("s8k_cp2", 1, 256), ("s32k_cp8", 1, 128)):
        w = workloads.get(name)
        Q, K, V = workloads.make_qkv(w, H=H)
        Qd, Kd, Vd = (dequantize(*quantize(x.float())) for x in (Q, K, V))
        for r in (0, w.cp - 1):
            pos = oracle.local_positions(w.S, w.cp, r)
            sel = np.unique(np.concatenate([np.random.default_rng(r).choice(pos, rows, replace=False), pos[:4]]))
            kmax = int(sel.max()) + 1
            e = emulated_error(Qd[0, 0][sel], Kd[0, 0, :kmax], Vd[0, 0, :kmax], sel, w.scale)
            assert 1e-3 < e < 0.05, (name, r, e)
