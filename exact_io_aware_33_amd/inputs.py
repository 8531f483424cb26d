"""Seeded synthetic inputs shared by the tests, the smoke check and the bench.

This module holds no attention arithmetic: it only draws numbers and rounds
them to the storage dtype.  Both the HIP path and the fp64 oracle consume what
it returns (the oracle the exact float64 upcast of the rounded values).

Recipe (one numpy PCG64 generator per call, ``default_rng(seed)``), in this
fixed draw order:
  1. Q, K, V, then dO, each i.i.d. N(0, 1) of shape [B, H, N, d] in float64,
     rounded to the storage dtype with round-to-nearest-even;
  2. key-padding lengths, if requested: integers uniform on [lo, hi], both
     ends inclusive, one per batch element (shared by all heads);
  3. block mask, if requested: [N/mb, N/mb] uint8, off-diagonal blocks
     Bernoulli(density), diagonal blocks forced to 1, shared by all heads.

The workloads below stand in for the pages' benchmarks (GPT-2 at 1K, BERT-large
at 512, long-context 16K, block-sparse): same shapes, synthetic values.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np
import torch

_TORCH_DTYPE = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    N: int
    d: int
    dtype: str
    causal: bool = False
    lens: tuple | None = None        # (lo, hi) inclusive, or None
    mb: int | None = None            # block-mask granularity, or None
    density: float = 0.1
    backward: bool = True
    note: str = ""

    @property
    def scale(self) -> float:
        """1/sqrt(d), as the float32 value handed to the library."""
        return float(np.float32(1.0 / math.sqrt(self.d)))


WORKLOADS = {
    w.name: w for w in [
        Workload("fp32_fwd_n256", 1, 1, 256, 64, "f32", backward=False,
                 note="forward only, non-causal fp32, no mask"),
        Workload("gpt2_causal_n1k", 8, 12, 1024, 64, "bf16", causal=True,
                 note="GPT-2-small-shaped causal self-attention"),
        Workload("bert_padding_n512", 16, 16, 512, 64, "f16", lens=(128, 512),
                 note="BERT-large-shaped encoder attention with key padding"),
        Workload("long_causal_n16k", 1, 16, 16384, 64, "bf16", causal=True,
                 note="long-context causal attention, d=64"),
        Workload("long_causal_n8k_d128", 1, 16, 8192, 128, "bf16", causal=True,
                 note="long-context causal attention, d=128"),
        Workload("blocksparse_n16k", 1, 8, 16384, 64, "f16", mb=128, density=0.1,
                 note="block-sparse attention, 128x128 blocks, diagonal set"),
    ]
}


def torch_dtype(name: str) -> torch.dtype:
    return _TORCH_DTYPE[name]


def make_inputs(B, H, N, d, dtype, *, seed=0, with_do=True, lens=None, mb=None,
                density=0.1):
    """Draw one problem's inputs.  Returns a dict of CPU tensors:

    q, k, v, (do): storage dtype, contiguous [B, H, N, d];
    key_lens: int32 [B] or None;  block_mask: uint8 [N/mb, N/mb] or None.
    """
    rng = np.random.default_rng(seed)
    td = _TORCH_DTYPE[dtype]
    out = {}
    names = ["q", "k", "v"] + (["do"] if with_do else [])
    for n in names:
        x = rng.standard_normal((B, H, N, d))
        out[n] = torch.from_numpy(x).to(td).contiguous()
    out["key_lens"] = None
    if lens is not None:
        lo, hi = lens
        out["key_lens"] = torch.from_numpy(rng.integers(lo, hi + 1, B).astype(np.int32))
    out["block_mask"] = None
    if mb is not None:
        assert N % mb == 0
        nb = N // mb
        m = (rng.random((nb, nb)) < density).astype(np.uint8)
        np.fill_diagonal(m, 1)
        out["block_mask"] = torch.from_numpy(m)
    return out


def make_workload_inputs(w: Workload, *, seed=0, B=None, H=None, N=None):
    """Inputs for a named workload (optionally with smaller B/H/N for tests)."""
    B = w.B if B is None else B
    H = w.H if H is None else H
    N = w.N if N is None else N
    return make_inputs(B, H, N, w.d, w.dtype, seed=seed, with_do=w.backward,
                       lens=w.lens, mb=w.mb, density=w.density)


def as_f64(t) -> np.ndarray | None:
    """Exact float64 upcast of a CPU tensor (no rounding: every storage dtype
    embeds in float64)."""
    if t is None:
        return None
    return t.detach().to("cpu").to(torch.float64).numpy()
