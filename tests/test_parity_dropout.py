"""Parity of the fused-dropout HIP path (through the C ABI) with the oracle.

The keep decisions are integer work, so they are checked bit for bit: with
Q = 0 every visible probability is 1/N, and choosing V, dO or K as the
identity makes the forward's O, the dK/dV kernel's dV and the dQ kernel's dQ
spell out the mask each kernel regenerated; it must equal the oracle's
keep_mask exactly.  The floating-point outputs are compared element by element
with the fp64 oracle (same inputs, same tolerances as without dropout), on
small cases over every mask mode and, at full size, on sampled rows/columns.
"""
import math
import sys

import numpy as np
import pytest
import torch

import oracle
from exact_io_aware_33_amd import fa_bwd, fa_bwd_blocksparse, fa_fwd, fa_fwd_blocksparse
from exact_io_aware_33_amd.inputs import WORKLOADS, as_f64, make_inputs

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-5, "f16": 2e-3, "bf16": 2e-2}


@pytest.fixture(autouse=True, scope="module")
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def rel_err(x, ref):
    x = np.asarray(x, np.float64)
    ref = np.asarray(ref, np.float64)
    assert x.shape == ref.shape
    assert not np.isnan(x).any(), "NaN in GPU output (unwritten or invalid element)"
    fin = np.isfinite(ref)
    assert np.array_equal(np.isfinite(x), fin), "finite/infinite pattern differs"
    assert np.array_equal(x[~fin], ref[~fin]), "non-finite values differ"
    if not fin.any():
        return 0.0
    den = float(np.max(np.abs(ref[fin])))
    num = float(np.max(np.abs(x[fin] - ref[fin])))
    return num if den == 0.0 else num / den


def nan_like(t):
    return torch.full_like(t, float("nan"))


def run(inp, scale, *, causal=False, key_lens=None, mb=None, drop=(0.0, 0, 0), backward=True):
    p, seed, off = drop
    dk = dict(dropout_p=p, dropout_seed=seed, dropout_offset=off)
    q, k, v = (inp[n].cuda() for n in ("q", "k", "v"))
    kl = None if key_lens is None else key_lens.cuda()
    o = nan_like(q)
    lse = torch.full(q.shape[:3], float("nan"), device="cuda", dtype=torch.float32)
    bm = None if mb is None else inp["block_mask"].cuda()
    if mb is None:
        fa_fwd(q, k, v, scale=scale, causal=causal, key_lens=kl, out=o, lse=lse, **dk)
    else:
        fa_fwd_blocksparse(q, k, v, bm, mask_block=mb, scale=scale, causal=causal, key_lens=kl,
                           out=o, lse=lse, **dk)
    if not backward:
        return o, lse, None
    do = inp["do"].cuda()
    g = [nan_like(q) for _ in range(3)]
    if mb is None:
        fa_bwd(q, k, v, o, lse, do, scale=scale, causal=causal, key_lens=kl,
               dq=g[0], dk=g[1], dv=g[2], **dk)
    else:
        fa_bwd_blocksparse(q, k, v, o, lse, do, bm, mask_block=mb, scale=scale, causal=causal,
                           key_lens=kl, dq=g[0], dk=g[1], dv=g[2], **dk)
    return o, lse, g


def check_case(B, H, N, d, dtype, drop, *, causal=False, lens=None, mb=None, density=0.3, seed=0):
    say(f"case B={B} H={H} N={N} d={d} {dtype} causal={causal} lens={lens} mb={mb} dropout={drop}")
    inp = make_inputs(B, H, N, d, dtype, seed=seed, lens=lens, mb=mb, density=density)
    scale = float(np.float32(1.0 / math.sqrt(d)))
    o, lse, (dq, dk, dv) = run(inp, scale, causal=causal, key_lens=inp["key_lens"], mb=mb, drop=drop)
    torch.cuda.synchronize()
    lens_np = None if inp["key_lens"] is None else np.clip(inp["key_lens"].numpy().astype(np.int64), 0, N)
    bm = None if mb is None else inp["block_mask"].numpy()
    kw = dict(causal=causal, key_lens=lens_np, block_mask=bm, mb=mb or 128, dropout=drop)
    rdq, rdk, rdv, (ro, rlse, _, _) = oracle.backward(*(as_f64(inp[n]) for n in ("q", "k", "v", "do")),
                                                      scale, return_aux=True, **kw)
    errs = dict(o=rel_err(as_f64(o), ro), lse=rel_err(lse.cpu().numpy(), rlse),
                dq=rel_err(as_f64(dq), rdq), dk=rel_err(as_f64(dk), rdk), dv=rel_err(as_f64(dv), rdv))
    say("  errors: " + " ".join(f"{n}={e:.2e}" for n, e in errs.items()))
    tol = TOL[dtype]
    bad = {n: e for n, e in errs.items() if not e <= tol}
    assert not bad, f"over tolerance {tol}: {bad}"


MODES = {
    "dense": dict(),
    "causal": dict(causal=True),
    "padding": dict(lens=(1, 300)),
    "causal_padding": dict(causal=True, lens=(1, 300)),
}


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("mode", list(MODES))
@pytest.mark.parametrize("N", [77, 300])
def test_dropout_forward_backward_small(dtype, d, mode, N):
    kw = dict(MODES[mode])
    if "lens" in kw:
        kw["lens"] = (1, N)
    check_case(2, 3, N, d, dtype, (0.2, 0x1234_5678_9ABC, 7), **kw)


@pytest.mark.parametrize("dtype", ["f16", "bf16", "f32"])
@pytest.mark.parametrize("causal", [False, True])
def test_dropout_blocksparse_small(dtype, causal):
    check_case(1, 2, 512, 64, dtype, (0.3, 99, 3), causal=causal, mb=128, density=0.4, seed=2)


@pytest.mark.parametrize("p", [0.05, 0.5, 0.9])
def test_dropout_rates(p):
    check_case(1, 2, 256, 64, "bf16", (p, 5, 0), causal=True, seed=3)


# ------------------------------------------------------ exact keep decisions
def _mask_inputs(B, H, N, which, blk=0):
    """Q = 0 (uniform P); V, dO and K chosen so that one kernel's output reads
    out the keep mask of the key (or query) columns blk*d .. blk*d + d - 1,
    d = min(N, 128): E[j, c] = 1 iff j = blk*d + c selects those columns and
    R[j, c] = 1 iff j = c (mod d) has one 1 in every row."""
    d = min(N, 128)
    z = torch.zeros(B, H, N, d, dtype=torch.float32)
    ones = torch.ones(B, H, N, d, dtype=torch.float32)
    rows = torch.arange(N)[:, None]
    cols = torch.arange(d)[None, :]
    sel = (rows == blk * d + cols).float().expand(B, H, N, d).contiguous()
    rep = (rows % d == cols).float().expand(B, H, N, d).contiguous()
    if which == "fwd":
        return dict(q=z, k=ones, v=sel, do=ones)
    if which == "dv":
        return dict(q=z, k=ones, v=ones, do=sel)
    return dict(q=z, k=sel, v=rep, do=ones)   # dQ: dP = 1, so dS = P (Z - D)


def _oracle_mask(B, H, N, drop):
    p, seed, off = drop
    rows = np.arange(N)
    return np.stack([np.stack([oracle.keep_mask(b * H + h, rows, rows, p, seed, off) for h in range(H)])
                     for b in range(B)])


# N = 512 takes every kernel through its steady (software-pipelined) loop,
# where the keep bytes of the next tile are generated a tile ahead; the
# columns are then read out 128 at a time.
@pytest.mark.parametrize("shape", [(2, 3, 128), (1, 2, 512)])
@pytest.mark.parametrize("drop", [(0.5, 2024, 0), (0.25, (7 << 32) | 11, 123456)])
def test_keep_decisions_bit_exact_in_all_three_kernels(drop, shape):
    B, H, N = shape
    ref = _oracle_mask(B, H, N, drop)
    t = oracle.drop_threshold(drop[0])
    zscale = np.float32(256.0 / (256.0 - t))
    d = min(N, 128)
    for blk in range(N // d):
        cs = slice(blk * d, (blk + 1) * d)
        say(f"case mask readout B={B} H={H} N={N} dropout={drop} columns {blk * d}..{(blk + 1) * d - 1}")
        # forward: O_i[c] = Z_i,(blk d + c) / N
        o, _, _ = run(_mask_inputs(B, H, N, "fwd", blk), 1.0, drop=drop, backward=False)
        o = o.cpu().numpy()
        assert np.array_equal(o != 0, ref[..., cs])
        assert np.all(o[ref[..., cs]] == np.float32(zscale / N))
        # dK/dV kernel: dV_j[c] = Z_(blk d + c),j / N
        _, _, (_, _, dv) = run(_mask_inputs(B, H, N, "dv", blk), 1.0, drop=drop)
        dv = dv.cpu().numpy()
        assert np.array_equal(np.swapaxes(dv, 2, 3) != 0, ref[:, :, cs, :])
        # dQ kernel: dQ_i[c] = (Z_i,(blk d + c) - D_i) / N, two values per row, the larger kept
        _, _, (dq, _, _) = run(_mask_inputs(B, H, N, "dq", blk), 1.0, drop=drop)
        dq = dq.cpu().numpy().astype(np.float64)
        mid = 0.5 * (dq.max(axis=3, keepdims=True) + dq.min(axis=3, keepdims=True))
        assert np.array_equal(dq > mid, ref[..., cs])
    say(f"  kept fraction {ref.mean():.4f} (expected {1 - t / 256:.4f})")


# ------------------------------------------------- reproducibility and p = 0
def test_same_counters_same_bits_other_offset_other_mask():
    inp = make_inputs(1, 2, 500, 64, "bf16", seed=8)
    s = float(np.float32(0.125))
    o1, _, g1 = run(inp, s, causal=True, drop=(0.1, 42, 5))
    o2, _, g2 = run(inp, s, causal=True, drop=(0.1, 42, 5))
    o3, _, _ = run(inp, s, causal=True, drop=(0.1, 42, 6))
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and all(torch.equal(a, b) for a, b in zip(g1, g2))
    assert not torch.equal(o1, o3)


@pytest.mark.parametrize("p", [0.0, 0.001])   # 0.001 rounds to t = 0: nothing dropped
def test_no_drop_threshold_is_the_plain_path(p):
    inp = make_inputs(2, 2, 300, 64, "f16", seed=9)
    s = float(np.float32(0.125))
    o0, l0, g0 = run(inp, s, causal=True)
    o1, l1, g1 = run(inp, s, causal=True, drop=(p, 77, 1))
    torch.cuda.synchronize()
    assert torch.equal(o0, o1) and torch.equal(l0, l1)
    assert all(torch.equal(a, b) for a, b in zip(g0, g1))


# ------------------------------------------------------------ full size
def test_workload_long_causal_n16k_dropout_full():
    """The 16K causal workload with dropout 0.1: full-size launch, every
    element of every head against the oracle (each head's keep mask drawn
    for its own (batch, head) index)."""
    from tests import _oracle_pool as pool

    w = WORKLOADS["long_causal_n16k"]
    drop = (0.1, 0xDEADBEEF, 1)
    say(f"case {w.name} full size with dropout {drop}, every head against the oracle")
    inp = make_inputs(w.B, w.H, w.N, w.d, w.dtype, seed=0)
    o, lse, (dq, dk, dv) = run(inp, w.scale, causal=True, drop=drop)
    torch.cuda.synchronize()
    got = (as_f64(o), lse.cpu().numpy(), as_f64(dq), as_f64(dk), as_f64(dv))
    del o, lse, dq, dk, dv
    rdq, rdk, rdv, ro, rlse = pool.backward_all_heads(
        *(as_f64(inp[n]) for n in ("q", "k", "v", "do")), w.scale, causal=True, dropout=drop)
    errs = {n: rel_err(g, r) for n, g, r in zip(("o", "lse", "dq", "dk", "dv"), got,
                                                 (ro, rlse, rdq, rdk, rdv))}
    say("  errors: " + " ".join(f"{n}={e:.2e}" for n, e in errs.items()))
    bad = {n: e for n, e in errs.items() if not e <= TOL[w.dtype]}
    assert not bad, f"over tolerance: {bad}"
