"""Seeded synthetic inputs shared by the tests, the smoke check and the bench.

This module holds no attention arithmetic: it only draws numbers and rounds
them to the storage dtype.  Both the HIP path and the fp64 oracle consume what
it returns (the oracle the exact float64 upcast of the rounded values).

Recipe (one numpy PCG64 generator per call, ``default_rng(seed)``), in this
fixed draw order:
  1. Q, K, V, then dO, each i.i.d. N(0, 1) in float64, Q and dO of shape
     [B, H, N, d], K and V of shape [B, H, N_k, d] (N_k = N unless given),
     rounded to the storage dtype with round-to-nearest-even;
  2. key-padding lengths, if requested: integers uniform on [lo, hi], both
     ends inclusive, one per batch element (shared by all heads);
  3. block mask, if requested: [N/mb, N_k/mb] uint8, blocks Bernoulli(density),
     then the diagonal (block i, i) forced to 1, shared by all heads.

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
    n_keys: int | None = None        # N_k when it differs from N (queries)
    note: str = ""

    @property
    def Nk(self) -> int:
        return self.N if self.n_keys is None else self.n_keys

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
        Workload("chunked_prefill_q4k_k16k", 1, 16, 4096, 64, "bf16", causal=True, n_keys=16384,
                 note="4K new queries against a 16K-key context, causal aligned bottom-right"),
        Workload("blocksparse_n64k", 1, 4, 65536, 64, "f16", mb=128, density=0.05,
                 note="block-sparse attention at the 64K Path-256 length, 128x128 blocks"),
        Workload("decode_q1_k32k", 8, 32, 1, 128, "bf16", causal=True, n_keys=32768, backward=False,
                 note="decoding: one new query per sequence against a 32K-key cache (split-KV)"),
    ]
}


def torch_dtype(name: str) -> torch.dtype:
    return _TORCH_DTYPE[name]


def make_inputs(B, H, N, d, dtype, *, seed=0, with_do=True, lens=None, mb=None,
                density=0.1, n_keys=None):
    """Draw one problem's inputs.  Returns a dict of CPU tensors:

    q, (do): storage dtype, contiguous [B, H, N, d]; k, v: [B, H, N_k, d]
    (N_k = n_keys, default N); key_lens: int32 [B] or None;
    block_mask: uint8 [N/mb, N_k/mb] or None.
    """
    rng = np.random.default_rng(seed)
    td = _TORCH_DTYPE[dtype]
    Nk = N if n_keys is None else n_keys
    out = {}
    names = ["q", "k", "v"] + (["do"] if with_do else [])
    for n in names:
        x = rng.standard_normal((B, H, Nk if n in ("k", "v") else N, d))
        out[n] = torch.from_numpy(x).to(td).contiguous()
    out["key_lens"] = None
    if lens is not None:
        lo, hi = lens
        out["key_lens"] = torch.from_numpy(rng.integers(lo, hi + 1, B).astype(np.int32))
    out["block_mask"] = None
    if mb is not None:
        assert N % mb == 0 and Nk % mb == 0
        m = (rng.random((N // mb, Nk // mb)) < density).astype(np.uint8)
        np.fill_diagonal(m, 1)
        out["block_mask"] = torch.from_numpy(m)
    return out


def make_workload_inputs(w: Workload, *, seed=0, B=None, H=None, N=None):
    """Inputs for a named workload (optionally with smaller B/H/N for tests)."""
    B = w.B if B is None else B
    H = w.H if H is None else H
    N = w.N if N is None else N
    Nk = w.Nk if N is None else N + (w.Nk - w.N)
    return make_inputs(B, H, N, w.d, w.dtype, seed=seed, with_do=w.backward,
                       lens=w.lens, mb=w.mb, density=w.density, n_keys=Nk)


def as_f64(t) -> np.ndarray | None:
    """Exact float64 upcast of a CPU tensor (no rounding: every storage dtype
    embeds in float64)."""
    if t is None:
        return None
    return t.detach().to("cpu").to(torch.float64).numpy()
