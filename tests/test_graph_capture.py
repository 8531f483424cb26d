"""The library's launches can be captured in a HIP graph and replayed.

The C ABI allocates, frees, synchronises and memsets nothing, so a whole
training step (forward, then the backward launch sequence) can be recorded
once into a graph (torch.cuda.CUDAGraph drives hipStreamBeginCapture on its
capture stream, which the binding passes to every call) and replayed.  Each
replay here runs on new inputs copied into the captured buffers, with eager
work and synchronisations between replays, and must equal an eager step on
the same inputs bit for bit (every kernel is deterministic: no atomics);
the last replay is also checked against the oracle.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
from exact_io_aware_33_amd import fa_bwd, fa_bwd_workspace_bytes, fa_fwd, fa_fwd_blocksparse, \
    fa_bwd_blocksparse
from exact_io_aware_33_amd.inputs import as_f64, make_inputs

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True, scope="module")
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def rel(x, ref):
    x = x.detach().cpu().to(torch.float64).numpy()
    return float(np.max(np.abs(x - ref)) / np.max(np.abs(ref)))


@pytest.mark.parametrize("mode", ["causal", "blocksparse_dropout"])
def test_step_replays_in_a_graph(mode):
    B, H, N, d, dt = 2, 3, 384, 64, "bf16"
    scale = float(np.float32(1.0 / np.sqrt(d)))
    sparse = mode == "blocksparse_dropout"
    say(f"case graph replay {mode} B={B} H={H} N={N} d={d} {dt}")
    first = make_inputs(B, H, N, d, dt, seed=0, mb=128 if sparse else None, density=0.4)
    q, k, v, do = (first[n].cuda() for n in ("q", "k", "v", "do"))
    bm = first["block_mask"].cuda() if sparse else None
    o, dq, dk, dv = (torch.empty_like(q) for _ in range(4))
    lse = torch.empty(B, H, N, dtype=torch.float32, device="cuda")
    ws = torch.empty(fa_bwd_workspace_bytes(q, k, scale=scale, causal=not sparse),
                     dtype=torch.uint8, device="cuda")
    drop = dict(dropout_p=0.2, dropout_seed=12345, dropout_offset=7) if sparse else {}

    def step():
        if sparse:
            fa_fwd_blocksparse(q, k, v, bm, mask_block=128, out=o, lse=lse, scale=scale, **drop)
            fa_bwd_blocksparse(q, k, v, o, lse, do, bm, mask_block=128, workspace=ws, dq=dq, dk=dk,
                               dv=dv, scale=scale, **drop)
        else:
            fa_fwd(q, k, v, out=o, lse=lse, scale=scale, causal=True)
            fa_bwd(q, k, v, o, lse, do, workspace=ws, dq=dq, dk=dk, dv=dv, scale=scale, causal=True)

    step()  # load the library and every kernel before capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()

    outs = (o, lse, dq, dk, dv)
    for seed in (1, 2, 3):
        new = make_inputs(B, H, N, d, dt, seed=seed)
        for name, t in (("q", q), ("k", k), ("v", v), ("do", do)):
            t.copy_(new[name].cuda())
        for t in outs:
            t.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        got = [t.clone() for t in outs]
        for t in outs:
            t.fill_(float("nan"))
        step()  # eager, same inputs
        torch.cuda.synchronize()
        for name, a, b in zip(("o", "lse", "dq", "dk", "dv"), got, outs):
            assert torch.equal(a, b), f"replay {seed}: {name} differs from the eager step"
        say(f"  replay on seed {seed}: bitwise equal to the eager step")

    # the last replay against the oracle
    f64 = [as_f64(new[n]) for n in ("q", "k", "v", "do")]
    kw = dict(block_mask=first["block_mask"].numpy(), mb=128,
              dropout=(0.2, 12345, 7)) if sparse else dict(causal=True)
    rdq, rdk, rdv, (ro, rlse, _, _) = oracle.backward(*f64, scale, return_aux=True, **kw)
    errs = {"o": rel(got[0], ro), "dq": rel(got[2], rdq), "dk": rel(got[3], rdk), "dv": rel(got[4], rdv)}
    say("  last replay vs oracle: " + " ".join(f"{n}={e:.2e}" for n, e in errs.items()))
    assert all(e <= 2e-2 for e in errs.values()), errs
