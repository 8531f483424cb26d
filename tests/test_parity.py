"""Parity of the HIP path (through the C ABI) with the fp64 oracle.

Every comparison is element by element on the same seeded inputs: the oracle
gets the exact float64 upcast of the rounded values the GPU reads, and the
float32 scale the GPU uses.  Error = max|x - ref| / max|ref| per output
tensor (LSE: the same, and -inf entries must match exactly).  Tolerances are
1e-5 for fp32, 2e-3 for fp16 and 2e-2 for bf16 outputs and gradients.
Outputs are pre-filled with NaN so an element the kernels never write fails.
"""
import math
import sys

import numpy as np
import pytest
import torch

import oracle
from exact_io_aware_33_amd import (FA_BWD_DQ, FA_BWD_MAIN, FA_BWD_PRE, FaError, fa_bwd,
                                   fa_bwd_blocksparse, fa_bwd_ex, fa_bwd_workspace_bytes, fa_fwd,
                                   fa_fwd_blocksparse)
from exact_io_aware_33_amd.inputs import WORKLOADS, Workload, as_f64, make_inputs, torch_dtype
from tests import _oracle_pool as pool

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
    if den == 0.0:
        return num
    return num / den


def nan_like(t):
    return torch.full_like(t, float("nan"))


def gpu_forward(inp, dtype, scale, causal, key_lens, mb, out_nan=True, query_tile=0):
    q, k, v = (inp[n].cuda() for n in ("q", "k", "v"))
    kl = None if key_lens is None else key_lens.cuda()
    o = nan_like(q)
    lse = torch.full(q.shape[:3], float("nan"), device="cuda", dtype=torch.float32)
    if mb is None:
        fa_fwd(q, k, v, scale=scale, causal=causal, key_lens=kl, out=o, lse=lse, query_tile=query_tile)
    else:
        fa_fwd_blocksparse(q, k, v, inp["block_mask"].cuda(), mask_block=mb, scale=scale,
                           causal=causal, key_lens=kl, out=o, lse=lse, query_tile=query_tile)
    return (q, k, v, kl), o, lse


def gpu_backward(dev, inp, o, lse, scale, causal, mb):
    q, k, v, kl = dev
    do = inp["do"].cuda()
    dq, dk, dv = nan_like(q), nan_like(q), nan_like(q)
    if mb is None:
        fa_bwd(q, k, v, o, lse, do, scale=scale, causal=causal, key_lens=kl, dq=dq, dk=dk, dv=dv)
    else:
        fa_bwd_blocksparse(q, k, v, o, lse, do, inp["block_mask"].cuda(), mask_block=mb, scale=scale,
                           causal=causal, key_lens=kl, dq=dq, dk=dk, dv=dv)
    return dq, dk, dv


def check_case(B, H, N, d, dtype, *, causal=False, lens=None, key_lens=None, mb=None, density=0.3,
               seed=0, backward=True, scale=None, block_mask=None, tol=None, query_tile=0):
    say(f"case B={B} H={H} N={N} d={d} {dtype} causal={causal} lens={lens} mb={mb} seed={seed}"
        f"{f' query_tile={query_tile}' if query_tile else ''}")
    inp = make_inputs(B, H, N, d, dtype, seed=seed, with_do=backward, lens=lens, mb=mb, density=density)
    if key_lens is not None:
        inp["key_lens"] = torch.tensor(key_lens, dtype=torch.int32)
    if block_mask is not None:
        inp["block_mask"] = torch.as_tensor(block_mask, dtype=torch.uint8)
    scale = float(np.float32(1.0 / math.sqrt(d))) if scale is None else float(np.float32(scale))
    tol = TOL[dtype] if tol is None else tol
    dev, o, lse = gpu_forward(inp, dtype, scale, causal, inp["key_lens"], mb, query_tile=query_tile)
    if backward:
        dq, dk, dv = gpu_backward(dev, inp, o, lse, scale, causal, mb)
    torch.cuda.synchronize()
    q64, k64, v64 = (as_f64(inp[n]) for n in ("q", "k", "v"))
    lens_np = None
    if inp["key_lens"] is not None:
        lens_np = np.clip(inp["key_lens"].numpy().astype(np.int64), 0, N)
    bm = None if mb is None else inp["block_mask"].numpy()
    kw = dict(causal=causal, key_lens=lens_np, block_mask=bm, mb=mb or 128)
    errs = {}
    if backward:
        rdq, rdk, rdv, (ro, rlse, _, _) = oracle.backward(q64, k64, v64, as_f64(inp["do"]), scale,
                                                          return_aux=True, **kw)
        errs.update(dq=rel_err(as_f64(dq), rdq), dk=rel_err(as_f64(dk), rdk), dv=rel_err(as_f64(dv), rdv))
    else:
        ro, rlse = oracle.forward(q64, k64, v64, scale, **kw)
    errs.update(o=rel_err(as_f64(o), ro), lse=rel_err(lse.cpu().numpy(), rlse))
    say("  errors: " + " ".join(f"{n}={e:.2e}" for n, e in errs.items()))
    bad = {n: e for n, e in errs.items() if not e <= tol}
    assert not bad, f"over tolerance {tol}: {bad}"
    return errs


# --------------------------------------------------------------- small sweeps
MODES = {
    "dense": dict(),
    "causal": dict(causal=True),
    "padding": dict(lens=(1, 300)),
    "causal_padding": dict(causal=True, lens=(1, 300)),
}


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("mode", list(MODES))
@pytest.mark.parametrize("N", [1, 77, 128, 192, 256, 300, 320])
def test_forward_backward_small(dtype, d, mode, N):
    """Every mode at lengths below one tile, at whole tiles (2, 3, 4 and 5
    tiles of 64 keys: the pipelined iterations then run up to the last tile)
    and with a ragged tail."""
    kw = dict(MODES[mode])
    if "lens" in kw:
        kw["lens"] = (1, max(1, N))
    check_case(2, 3, N, d, dtype, seed=N + d, **kw)


@pytest.mark.parametrize("query_tile", [64, 256])
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("mode", list(MODES))
@pytest.mark.parametrize("N", [77, 300, 1000])
def test_forward_query_tiles(query_tile, dtype, d, mode, N):
    """The 64- and 256-query forward workgroups (2 and 8 wavefronts) against
    the oracle: every mask mode, lengths that leave ragged last tiles."""
    kw = dict(MODES[mode])
    if "lens" in kw:
        kw["lens"] = (1, N)
    check_case(2, 3, N, d, dtype, seed=N + d + query_tile, backward=False, query_tile=query_tile, **kw)


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("causal", [False, True])
def test_blocksparse_query_tile_64(dtype, causal):
    check_case(2, 2, 1024, 64, dtype, causal=causal, mb=128, density=0.4, seed=17, backward=False,
               query_tile=64)
    check_case(1, 2, 512, 128, dtype, causal=causal, mb=256, density=0.5, seed=18, backward=False,
               query_tile=64)


def test_query_tiles_rank_major_and_bitwise_equal_rows():
    """The query tile only regroups rows: each row's arithmetic is the same,
    so O and LSE are bitwise equal across tiles 64 / 128 / 256 (16 heads, 8K
    causal: rank-major order at 64 and 128, head by head at 256)."""
    inp = make_inputs(1, 16, 8192, 64, "bf16", seed=5, with_do=False)
    q, k, v = (inp[n].cuda() for n in ("q", "k", "v"))
    outs = [fa_fwd(q, k, v, causal=True, query_tile=t) for t in (64, 128, 256)]
    torch.cuda.synchronize()
    for o, l in outs[1:]:
        assert torch.equal(o, outs[0][0]) and torch.equal(l, outs[0][1])


@pytest.mark.parametrize("dtype", ["f16", "bf16", "f32"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("mb", [128, 256])
def test_blocksparse_small(dtype, d, causal, mb):
    check_case(2, 2, 512, d, dtype, causal=causal, mb=mb, density=0.4, seed=mb + d)


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("B,H,N,d,lens", [(2, 4, 1024, 64, None), (1, 8, 2048, 64, None),
                                          (2, 8, 640, 128, (1, 640)), (1, 8, 4096, 64, None),
                                          (2, 12, 1536, 64, None), (1, 24, 2048, 64, (1, 2048)),
                                          (4, 16, 1024, 64, None)])
def test_causal_rank_major_tile_order(dtype, B, H, N, d, lens):
    """Causal launches whose heads split evenly over the 8 XCDs and that have
    at most 64 tiles per head are issued rank-major (longest tiles of every
    head first), the first passes of 32 slots of each XCD dealt in
    alternating direction (36, 48 and 64 slots per XCD here: a partial
    reversed pass, a full one): every (head, tile) must still be computed
    exactly once."""
    check_case(B, H, N, d, dtype, causal=True, lens=lens, seed=3)


def test_blocksparse_with_padding_and_empty_rows():
    nb = 4
    m = np.ones((nb, nb), np.uint8)
    m[1, :] = 0            # query block 1 sees nothing -> O = 0, LSE = -inf
    m[:, 2] = 0            # key block 2 is never seen -> dK = dV = 0
    m[3, 0] = 0
    check_case(2, 3, 512, 64, "f16", mb=128, block_mask=m, key_lens=[400, 130])
    check_case(2, 3, 512, 64, "bf16", mb=128, block_mask=m, causal=True, key_lens=[512, 200])


def test_blocksparse_per_head_mask():
    H, nb = 3, 4
    rng = np.random.default_rng(9)
    m = (rng.random((H, nb, nb)) < 0.5).astype(np.uint8)
    for h in range(H):
        np.fill_diagonal(m[h], 1)
    check_case(1, H, 512, 64, "f16", mb=128, block_mask=m)
    check_case(1, H, 512, 128, "bf16", mb=128, block_mask=m, causal=True)


# ------------------------------------------------------------------ edge cases
def test_single_token():
    for dtype in ("f32", "f16", "bf16"):
        check_case(1, 2, 1, 64, dtype)
        check_case(3, 1, 1, 128, dtype, causal=True)


def test_zero_scale_is_mean_of_visible_values():
    check_case(2, 2, 200, 64, "f32", scale=0.0)
    check_case(2, 2, 200, 64, "bf16", scale=0.0, causal=True)
    check_case(2, 2, 200, 128, "f16", scale=0.0, key_lens=[3, 150])


def test_key_lengths_zero_clamped_and_full():
    # 0 -> every row fully masked; negative clamps to 0; > N clamps to N
    check_case(4, 2, 150, 64, "f16", key_lens=[0, -5, 1000, 150])
    check_case(4, 2, 150, 64, "bf16", causal=True, key_lens=[0, 1, 149, 10 ** 6])
    check_case(2, 2, 150, 128, "f32", key_lens=[0, 77])


def test_large_score_magnitudes():
    """Scores of order +-100 (the max subtraction must keep exp finite).

    fp32 tolerance, derived from the scores: the kernel rounds S (fp32) and
    the exponent S*scale*log2(e) - m (one fp32 FMA) to within a few units of
    the last place of their magnitude, and an absolute error delta in an
    exponent is a relative error ln(2)*delta of that weight of the softmax:
    normalised O error <~ 1e-5 (the workloads' fp32 tolerance, for the
    accumulations) + 4 u max|S| with u = 2^-24.  A float32 rendering of the
    same steps on the CPU errs by 9.4e-6 on these inputs.  The 16-bit
    tolerances (dominated by input rounding) are unchanged."""
    errs = check_case(1, 2, 256, 64, "f32", scale=12.0, tol=1.0)   # measured first
    inp = make_inputs(1, 2, 256, 64, "f32", seed=0)
    q, k = as_f64(inp["q"]), as_f64(inp["k"])
    max_s = float(np.max(np.abs(np.float32(12.0) * (q @ np.swapaxes(k, -1, -2)))))
    tol = 1e-5 + 4 * 2.0 ** -24 * max_s
    say(f"  fp32 stress: max|S| = {max_s:.1f}, tolerance {tol:.2e}, measured "
        + " ".join(f"{n}={e:.2e}" for n, e in errs.items()))
    assert max(errs.values()) <= tol
    check_case(1, 2, 256, 64, "bf16", scale=12.0, causal=True)


def test_strided_bnhd_layout():
    """[B, N, H, d] storage seen as a [B, H, N, d] view."""
    B, H, N, d = 2, 3, 200, 64
    inp = make_inputs(B, H, N, d, "bf16", seed=5)
    say("case strided BNHD bf16")
    dev = {n: inp[n].permute(0, 2, 1, 3).contiguous().cuda().permute(0, 2, 1, 3) for n in ("q", "k", "v", "do")}
    assert dev["q"].stride(2) == H * d
    o, lse = fa_fwd(dev["q"], dev["k"], dev["v"], causal=True)
    dq, dk, dv = fa_bwd(dev["q"], dev["k"], dev["v"], o, lse, dev["do"], causal=True)
    assert o.stride() == dev["q"].stride()
    scale = float(np.float32(1 / math.sqrt(d)))
    rdq, rdk, rdv, (ro, rlse, _, _) = oracle.backward(*(as_f64(inp[n]) for n in ("q", "k", "v", "do")),
                                                      scale, causal=True, return_aux=True)
    for x, r in ((o, ro), (dq, rdq), (dk, rdk), (dv, rdv)):
        assert rel_err(as_f64(x), r) <= TOL["bf16"]
    assert rel_err(lse.cpu().numpy(), rlse) <= TOL["bf16"]


def test_forward_is_bitwise_reproducible():
    inp = make_inputs(2, 4, 1000, 64, "bf16", seed=3)
    q, k, v = (inp[n].cuda() for n in ("q", "k", "v"))
    o1, l1 = fa_fwd(q, k, v, causal=True)
    o2, l2 = fa_fwd(q, k, v, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


@pytest.mark.parametrize("dtype,d", [("bf16", 64), ("f16", 128), ("f32", 64), ("f32", 128)])
def test_backward_is_bitwise_reproducible_and_stage_split_matches(dtype, d):
    """No atomics: the backward is deterministic, and running its stages
    through fa_bwd_ex gives exactly fa_bwd's result: PRE, then DQ, then MAIN
    (MAIN and DQ in either order once PRE is done), and PRE | DQ (the dQ pass
    doing the preprocessing itself, as fa_bwd does) then MAIN.  The workspace
    the fused dQ pass leaves is bitwise the preprocessing kernel's."""
    inp = make_inputs(2, 3, 700, d, dtype, seed=4)
    q, k, v, do = (inp[n].cuda() for n in ("q", "k", "v", "do"))
    o, lse = fa_fwd(q, k, v, causal=True)
    g1 = fa_bwd(q, k, v, o, lse, do, causal=True)
    g2 = fa_bwd(q, k, v, o, lse, do, causal=True)
    nws = fa_bwd_workspace_bytes(q, causal=True)
    results, spaces = [], []
    for order in ([FA_BWD_PRE, FA_BWD_DQ, FA_BWD_MAIN], [FA_BWD_PRE, FA_BWD_MAIN, FA_BWD_DQ],
                  [FA_BWD_PRE | FA_BWD_DQ, FA_BWD_MAIN]):
        ws = torch.full((nws,), 255, dtype=torch.uint8, device="cuda")
        g3 = tuple(torch.full_like(q, float("nan")) for _ in range(3))
        common = dict(causal=True, workspace=ws, dq=g3[0], dk=g3[1], dv=g3[2])
        for st in order:
            fa_bwd_ex(q, k, v, o, lse, do, st, **common)
        results.append(g3)
        spaces.append(ws)
    torch.cuda.synchronize()
    for a, b in zip(g1, g2):
        assert torch.equal(a, b)
    for g3 in results:
        for a, c in zip(g1, g3):
            assert torch.equal(a, c)
    assert torch.equal(spaces[0], spaces[2])


def test_binding_and_library_reject_bad_calls_on_gpu():
    inp = make_inputs(1, 2, 64, 64, "f16", seed=1)
    q, k, v = (inp[n].cuda() for n in ("q", "k", "v"))
    with pytest.raises(ValueError):
        fa_fwd(q, k.float(), v)                            # mixed dtypes
    with pytest.raises(ValueError):
        fa_fwd(q.transpose(2, 3), k.transpose(2, 3), v.transpose(2, 3))   # d not contiguous
    q96 = torch.zeros(1, 2, 64, 96, dtype=torch.float16, device="cuda")
    with pytest.raises(FaError) as e:
        fa_fwd(q96, q96, q96)
    assert e.value.status == 2                             # FA_ERR_UNSUPPORTED
    bm = torch.ones(1, 1, dtype=torch.uint8, device="cuda")
    with pytest.raises(FaError) as e:
        fa_fwd_blocksparse(q, k, v, bm, mask_block=96)     # does not divide N = 64
    assert e.value.status == 1
    o, lse = fa_fwd(q, k, v)
    small = torch.empty(8, dtype=torch.uint8, device="cuda")
    with pytest.raises(FaError):
        fa_bwd(q, k, v, o, lse, q, workspace=small)        # workspace too small
    # caller-supplied per-row statistics: the library writes / reads B*H*N
    # floats through a bare pointer, so the binding checks them first
    for bad in (torch.empty(1, 2, 64, dtype=torch.bfloat16, device="cuda"),   # not float32
                torch.empty(1, 2, 32, dtype=torch.float32, device="cuda"),    # too small
                torch.empty(1, 2, 128, dtype=torch.float32, device="cuda")[:, :, ::2],  # strided
                torch.empty(1, 2, 64, dtype=torch.float32)):                  # host memory
        with pytest.raises(ValueError):
            fa_fwd(q, k, v, lse=bad)
        with pytest.raises(ValueError):
            fa_bwd(q, k, v, o, bad, q)
    with pytest.raises(ValueError):
        fa_bwd(q, k, v, o, None, q)                        # LSE is required


# ---------------------------------------------------- the named workloads
def test_workload_fp32_fwd_n256():
    w = WORKLOADS["fp32_fwd_n256"]
    check_case(w.B, w.H, w.N, w.d, w.dtype, backward=False)


def test_workload_gpt2_causal_n1k():
    w = WORKLOADS["gpt2_causal_n1k"]
    check_case(w.B, w.H, w.N, w.d, w.dtype, causal=True)


def test_workload_bert_padding_n512():
    w = WORKLOADS["bert_padding_n512"]
    check_case(w.B, w.H, w.N, w.d, w.dtype, lens=w.lens)


def _full(w, seed=0):
    """Full-size launch; every output element of every head against the
    oracle (heads evaluated in parallel on the host's cores)."""
    say(f"case {w.name} full size (B={w.B} H={w.H} N={w.N} d={w.d} {w.dtype} causal={w.causal} "
        f"mb={w.mb}), every head against the oracle")
    inp = make_inputs(w.B, w.H, w.N, w.d, w.dtype, seed=seed, lens=w.lens, mb=w.mb, density=w.density)
    dev, o, lse = gpu_forward(inp, w.dtype, w.scale, w.causal, inp["key_lens"], w.mb)
    dq, dk, dv = gpu_backward(dev, inp, o, lse, w.scale, w.causal, w.mb)
    torch.cuda.synchronize()
    got = (as_f64(o), lse.cpu().numpy(), as_f64(dq), as_f64(dk), as_f64(dv))
    del dev, o, lse, dq, dk, dv
    lens = None if inp["key_lens"] is None else inp["key_lens"].numpy()
    bm = None if w.mb is None else inp["block_mask"].numpy()
    rdq, rdk, rdv, ro, rlse = pool.backward_all_heads(
        *(as_f64(inp[n]) for n in ("q", "k", "v", "do")), w.scale, causal=w.causal, key_lens=lens,
        block_mask=bm, mb=w.mb or 128)
    ref = (ro, rlse, rdq, rdk, rdv)
    names = ("o", "lse", "dq", "dk", "dv")
    errs = {n: rel_err(g, r) for n, g, r in zip(names, got, ref)}
    # the worst head of each tensor (normalised by that tensor's overall max)
    worst = {}
    for n, g, r in zip(names, got, ref):
        fin = np.isfinite(r)
        diff = np.where(fin, np.abs(np.where(fin, g, 0.0) - np.where(fin, r, 0.0)), 0.0)
        per_head = diff.reshape(w.B * w.H, -1).max(axis=1) / np.max(np.abs(r[fin]))
        worst[n] = (int(per_head.argmax()), float(per_head.max()))
    say("  errors: " + " ".join(f"{n}={e:.2e}" for n, e in errs.items()))
    say("  worst head (b*H+h, error): " + " ".join(f"{n}={h}:{e:.2e}" for n, (h, e) in worst.items()))
    tol = TOL[w.dtype]
    bad = {n: e for n, e in errs.items() if not e <= tol}
    assert not bad, f"over tolerance {tol}: {bad}"


def _sampled(w, heads, n_rows=192, n_cols=192, seed=0):
    """Full-size launch; oracle on sampled rows/columns of some heads."""
    say(f"case {w.name} full size, sampled heads {heads}")
    inp = make_inputs(w.B, w.H, w.N, w.d, w.dtype, seed=seed, lens=w.lens, mb=w.mb, density=w.density)
    scale = w.scale
    dev, o, lse = gpu_forward(inp, w.dtype, scale, w.causal, inp["key_lens"], w.mb)
    dq, dk, dv = gpu_backward(dev, inp, o, lse, scale, w.causal, w.mb)
    torch.cuda.synchronize()
    for t in (o, lse, dq, dk, dv):
        assert not torch.isnan(t).any().item(), "unwritten element"
    # invariants of the exact gradients, checked on every head at full size:
    # each row of dS sums to 0, so sum_j dK_j = 0; each row of P sums to 1, so
    # sum_j dV_j = sum_i dO_i (every row sees at least its diagonal block/key).
    dk64, dv64, do64 = (x.double() for x in (dk, dv, inp["do"].cuda()))
    skd = dk64.sum(dim=2).abs().max().item() / dk64.abs().max().item()
    svd = (dv64.sum(dim=2) - do64.sum(dim=2)).abs().max().item() / do64.sum(dim=2).abs().max().item()
    say(f"  invariants: |sum_j dK_j|/max|dK| = {skd:.2e}, sum dV vs sum dO rel = {svd:.2e}")
    # bound: 5x the dtype tolerance (measured 1-2e-2 for bf16, 5e-3 for fp16;
    # a dropped D term or a missing scale would give O(1))
    assert skd < 5 * TOL[w.dtype] and svd < 5 * TOL[w.dtype]
    rng = np.random.default_rng(1234)
    N = w.N
    edges = np.array([0, 1, 63, 64, 127, 128, N // 2, N - 129, N - 128, N - 2, N - 1])
    rows = np.unique(np.concatenate([edges, rng.choice(N, n_rows, replace=False)]))
    cols = np.unique(np.concatenate([edges, rng.choice(N, n_cols, replace=False)]))
    bm = None if w.mb is None else inp["block_mask"].numpy()
    tol = TOL[w.dtype]
    for (b, h) in heads:
        ro, rlse, rdq, rdk, rdv = oracle.gradients_sampled(
            *(as_f64(inp[n][b, h]) for n in ("q", "k", "v", "do")), scale, rows, cols,
            causal=w.causal, block_mask=bm, mb=w.mb or 128)
        errs = dict(
            o=rel_err(as_f64(o[b, h])[rows], ro), lse=rel_err(lse[b, h].cpu().numpy()[rows], rlse),
            dq=rel_err(as_f64(dq[b, h])[rows], rdq), dk=rel_err(as_f64(dk[b, h])[cols], rdk),
            dv=rel_err(as_f64(dv[b, h])[cols], rdv))
        say(f"  head ({b},{h}) errors: " + " ".join(f"{n}={e:.2e}" for n, e in errs.items()))
        bad = {n: e for n, e in errs.items() if not e <= tol}
        assert not bad, f"over tolerance {tol}: {bad}"


def test_workload_long_causal_n16k_full():
    _full(WORKLOADS["long_causal_n16k"])


def test_workload_long_causal_n8k_d128_full():
    _full(WORKLOADS["long_causal_n8k_d128"])


def test_workload_blocksparse_n16k_full():
    _full(WORKLOADS["blocksparse_n16k"])


@pytest.mark.parametrize("N", [1024, 16384])
def test_sweep_dense_noncausal_full(N):
    """The metric's sweep shapes (bf16, d = 64, H = 16, B = 16384 / N),
    non-causal, at both ends of N = 1K-16K: every head against the oracle."""
    _full(Workload(f"sweep_n{N}_full", 16384 // N, 16, N, 64, "bf16"))


def test_sweep_causal_n4k_full():
    """A middle point of the sweep, causal (B = 4, H = 16, N = 4096)."""
    _full(Workload("sweep_n4096_causal", 4, 16, 4096, 64, "bf16", causal=True))


def test_workload_long_causal_n16k_sampled_edges():
    """The sampled evaluation kept as a fast cross-check of the full one: the
    edge rows and columns of two heads."""
    _sampled(WORKLOADS["long_causal_n16k"], heads=[(0, 0), (0, 15)], n_rows=32, n_cols=32)
