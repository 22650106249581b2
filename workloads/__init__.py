"""Seeded synthetic workloads for causal context-parallel attention.

This module is shared by the fp64 oracle's tests and by the HIP path's
tests and benchmark. It holds shapes, seeds and random draws only -- none of
the attention arithmetic, none of the zigzag/ring index maths and no merge
rule -- so that neither side can inherit a mistake from the other through it.

Workload recipe (the pages print no data; every input is synthetic):

* Q, K, V are drawn in that order with ``torch.randn(B, H, S, D)`` in fp32
  from a CPU ``torch.Generator`` seeded with the workload's seed, in natural
  token order over the full sequence of length S.
* They are rounded to bf16 (round-to-nearest-even).  Both the GPU path and the
  oracle consume exactly these bf16 values (the oracle after an exact up-cast
  to fp64), so the comparison measures the kernel's arithmetic only.
* With scale 1/sqrt(D), the scores are close to N(0, 1).

Shapes follow the five workloads of the causal ring attention rank share
(one rank of a simulated context-parallel group of size ``cp``, each rank
holding two zigzag chunks of ``S / (2 cp)`` tokens).
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np
import torch

__all__ = ["Workload", "WORKLOADS", "get", "make_qkv", "make_qkv_scaled", "make_grad_out",
           "sample_local_rows", "host_info"]


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    D: int
    S: int          # total sequence length
    cp: int         # simulated context-parallel group size
    seed: int
    rows_per_head: int | None = None   # sampled rows per (b, h) for parity, None = all

    @property
    def chunk_len(self) -> int:
        return self.S // (2 * self.cp)

    @property
    def local_len(self) -> int:
        return 2 * self.chunk_len

    @property
    def scale(self) -> float:
        return 1.0 / float(np.sqrt(self.D))

    def describe(self) -> str:
        return (f"{self.name}: B={self.B} H={self.H} D={self.D} S={self.S} "
                f"cp={self.cp} chunk={self.chunk_len}")


WORKLOADS = {
    "tiny": Workload("tiny", B=1, H=2, D=64, S=256, cp=2, seed=1),
    "s8k_cp2": Workload("s8k_cp2", B=1, H=16, D=128, S=8192, cp=2, seed=2),
    "s16k_cp4": Workload("s16k_cp4", B=1, H=32, D=128, S=16384, cp=4, seed=3),
    "s32k_cp8": Workload("s32k_cp8", B=1, H=32, D=128, S=32768, cp=8, seed=4),
    "s64k_cp16": Workload("s64k_cp16", B=2, H=64, D=128, S=65536, cp=16, seed=5,
                          rows_per_head=512),
}


def get(name: str) -> Workload:
    return WORKLOADS[name]


def _draw(shape, gen: torch.Generator) -> torch.Tensor:
    x = torch.randn(*shape, generator=gen, dtype=torch.float32)
    return x.to(torch.bfloat16)        # RNE rounding


def make_qkv(w: Workload, seed: int | None = None, B: int | None = None,
             H: int | None = None, S: int | None = None, D: int | None = None):
    """Full-sequence Q, K, V as bf16 CPU tensors of shape [B, H, S, D].

    Draw order is Q, then K, then V from one generator seeded with
    ``w.seed`` (or ``seed``).  Overrides of the shape exist for small
    variants of a workload used by tests.
    """
    gen = torch.Generator(device="cpu")
    gen.manual_seed(w.seed if seed is None else seed)
    shape = (B or w.B, H or w.H, S or w.S, D or w.D)
    q = _draw(shape, gen)
    k = _draw(shape, gen)
    v = _draw(shape, gen)
    return q, k, v


def make_grad_out(w: Workload, seed: int | None = None, B: int | None = None,
                  H: int | None = None, S: int | None = None, D: int | None = None):
    """Upstream gradient dO of the attention output, bf16 CPU [B, H, S, D].

    Drawn like Q, K, V (standard normal in fp32, rounded to bf16) from its own
    generator seeded with ``w.seed + 1000`` (or ``seed``), over the full
    sequence in natural token order.
    """
    gen = torch.Generator(device="cpu")
    gen.manual_seed(w.seed + 1000 if seed is None else seed)
    return _draw((B or w.B, H or w.H, S or w.S, D or w.D), gen)


def make_qkv_scaled(shape, seed: int, q_scale: float = 1.0, k_scale: float = 1.0,
                    v_scale: float = 1.0):
    """Q, K, V ~ N(0, scale^2), drawn in fp32 then rounded to bf16.

    Larger Q/K scales give peaked softmax rows, which exercise the online
    rescaling of the running maximum.
    """
    gen = torch.Generator(device="cpu")
    gen.manual_seed(seed)
    q = (torch.randn(*shape, generator=gen) * q_scale).to(torch.bfloat16)
    k = (torch.randn(*shape, generator=gen) * k_scale).to(torch.bfloat16)
    v = (torch.randn(*shape, generator=gen) * v_scale).to(torch.bfloat16)
    return q, k, v


def sample_local_rows(w: Workload, n_rows: int | None = None, seed: int | None = None):
    """Seeded sample of local query rows (indices into the rank's 2L rows).

    Returns an int64 array of shape [B, H, n] (sorted per head): ``n_rows``
    distinct rows drawn uniformly without replacement with
    ``numpy.random.default_rng(seed)`` (default ``w.seed + 1``), plus the
    first and last row of each of the two local chunks.
    """
    n = n_rows if n_rows is not None else (w.rows_per_head or w.local_len)
    rng = np.random.default_rng(w.seed + 1 if seed is None else seed)
    L = w.chunk_len
    edges = np.array([0, L - 1, L, 2 * L - 1], dtype=np.int64)
    out = []
    for _ in range(w.B * w.H):
        if n >= w.local_len:
            rows = np.arange(w.local_len, dtype=np.int64)
        else:
            rows = rng.choice(w.local_len, size=n, replace=False).astype(np.int64)
            rows = np.unique(np.concatenate([rows, edges]))
        out.append(rows)
    m = max(len(r) for r in out)
    # pad every head to the same count with repeats of its own last row
    arr = np.stack([np.concatenate([r, np.full(m - len(r), r[-1], np.int64)]) for r in out])
    return arr.reshape(w.B, w.H, m)


def host_info() -> dict:
    """Host CPU model and the cores this process may use."""
    import os
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"cpu_model": model, "cores": len(os.sched_getaffinity(0))}
