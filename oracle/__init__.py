"""Plain fp64 CPU oracle for causal context-parallel (ring) attention.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
link this package: only the tests, the smoke check and the CPU-baseline leg of
the benchmark use it.  It shares no code with the HIP library (no kernels,
headers, index helpers or tables) and never reads a value that the HIP path
produced.

Sources (web pages; cited by title and section):

* [MLM] "Megatron-LM源码解析：Context Parallel如何革新长序列训练"
  (mieleap.com/news/151524), sections 1-6.
* [RAF] "如何用Context并行加速大模型训练？手把手教你配置RingAttention+FlashAttention"
  (devpress.csdn.net), sections 1-5.

What it computes (the plain definition; the ring method reaches the same
real-valued result, only the order of summation differs):

    s_ij  = tau * <q_i, k_j>           for every key position j <= i
    LSE_i = ln sum_{j <= i} exp(s_ij)
    out_i = sum_{j <= i} exp(s_ij - LSE_i) * v_j

with tau = 1/sqrt(D) and positions absolute in the full sequence.

Gradients (``backward.py``): dQ, dK, dV of the same definition for an
upstream dO, and the part one block of keys contributes to them (how a ring
step's backward splits).

Pins (tests marked "not gpu"): scalar brute force on tiny inputs, the closed
forms for Q = 0 and for the first token, the merge invariant over arbitrary
key splits, softmax normalisation, constant-V and key-shift invariance,
PyTorch's fp64 scaled-dot-product attention as an independent library case,
and the zigzag worked example printed in [RAF] section 5.
"""
from .attention import causal_attention_rows, masked_attention, to_f64
from .backward import causal_attention_grad, masked_attention_grad
from .merge import lse_merge
from .zigzag import (zigzag_chunk_ids, local_positions, contiguous_positions,
                     ring_source, ring_kv_positions, visible_pairs)

__all__ = [
    "causal_attention_rows", "masked_attention", "to_f64", "lse_merge",
    "causal_attention_grad", "masked_attention_grad",
    "zigzag_chunk_ids", "local_positions", "contiguous_positions",
    "ring_source", "ring_kv_positions", "visible_pairs",
]
