"""Parity of the row softmax and LayerNorm / GroupNorm kernels with the oracle.

Every launch shape is covered: 8, 64, 256 or 1024 threads per row with the
row held in registers (4, 8 or 16 vectors per thread), and rows streamed
twice (unaligned or ragged rows, and rows too long to hold); row lengths
that leave a ragged last vector; strided rows;
-inf entries and an all -inf row (softmax); a large common offset (the
moment merge must not lose the variance); GroupNorm through the same kernel;
in-place calls.  Inputs are rounded to the storage type first; the oracle
sees the rounded values.  Error = max |x - ref| / max |ref| per output.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
from exact_io_aware_33_amd import fa_group_norm, fa_layernorm_rows, fa_softmax_rows

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-5, "f16": 2e-3, "bf16": 2e-2}
TD = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


@pytest.fixture(autouse=True, scope="module")
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def rel(x, ref):
    x = np.asarray(x, np.float64)
    ref = np.asarray(ref, np.float64)
    assert not np.isnan(x).any(), "NaN in GPU output"
    fin = np.isfinite(ref)
    assert np.array_equal(np.isfinite(x), fin) and np.array_equal(x[~fin], ref[~fin])
    den = float(np.max(np.abs(ref[fin]))) if fin.any() else 0.0
    num = float(np.max(np.abs(x[fin] - ref[fin]))) if fin.any() else 0.0
    return num if den == 0.0 else num / den


def draw(rows, cols, dtype, seed, *, scale=1.0, offset=0.0, ld=None):
    rng = np.random.default_rng(seed)
    ld = cols if ld is None else ld
    full = torch.from_numpy(rng.standard_normal((rows, ld)) * scale + offset).to(TD[dtype])
    x = full.cuda()[:, :cols]
    return x, x.double().cpu().numpy()


# Together these reach every launch shape the library picks (threads per row
# 8 / 64 / 256 / 1024 with 4 / 8 / 16 vectors held per thread, and the rows
# streamed twice) for both 16-bit types and fp32.
SIZES = [(2100, 7), (2100, 1000), (2100, 4100), (2100, 9000), (3, 1), (3, 513), (3, 16384),
         (3, 16390), (2, 70000), (5000, 64), (2500, 512), (1100, 4096), (1100, 8192),
         (500, 8192), (3, 65536)]


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("rows,cols", SIZES)
def test_softmax_rows(dtype, rows, cols):
    say(f"case softmax rows={rows} cols={cols} {dtype}")
    ld = cols + (8 if cols % 8 == 0 else 8 - cols % 8) + 8   # strided rows, 16-byte multiple
    x, x64 = draw(rows, cols, dtype, 1, scale=3.0, ld=ld)
    if cols > 4:
        x[0, 1::3] = float("-inf")
        x64[0, 1::3] = -np.inf
    x[rows - 1] = float("-inf")
    x64[rows - 1] = -np.inf
    y = torch.full((rows, ld), float("nan"), dtype=TD[dtype], device="cuda")[:, :cols]
    y, lse = fa_softmax_rows(x, out=y)
    torch.cuda.synchronize()
    ry, rlse = oracle.softmax_rows(x64)
    ey = rel(y.double().cpu().numpy(), ry)
    fin = np.isfinite(rlse)
    el = float(np.max(np.abs(lse.cpu().numpy()[fin] - rlse[fin]) / np.maximum(1.0, np.abs(rlse[fin]))))
    assert np.all(np.isneginf(lse.cpu().numpy()[~fin]))
    say(f"  errors: y={ey:.2e} lse={el:.2e}")
    assert ey <= TOL[dtype] and el <= 1e-5


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("rows,cols", SIZES)
@pytest.mark.parametrize("affine", [False, True])
def test_layernorm_rows(dtype, rows, cols, affine):
    say(f"case layernorm rows={rows} cols={cols} {dtype} affine={affine}")
    x, x64 = draw(rows, cols, dtype, 2, scale=2.0, offset=30.0)
    g = b = None
    if affine:
        g = torch.from_numpy(np.random.default_rng(3).standard_normal(cols)).to(TD[dtype]).cuda()
        b = torch.from_numpy(np.random.default_rng(4).standard_normal(cols)).to(TD[dtype]).cuda()
    y, mean, rstd = fa_layernorm_rows(x, g, b, eps=1e-5)
    torch.cuda.synchronize()
    ry, rm, rr = oracle.layernorm_rows(x64, None if g is None else g.double().cpu().numpy(),
                                       None if b is None else b.double().cpu().numpy(), eps=1e-5)
    errs = dict(y=rel(y.double().cpu().numpy(), ry), mean=rel(mean.cpu().numpy(), rm),
                rstd=rel(rstd.cpu().numpy(), rr))
    say("  errors: " + " ".join(f"{n}={e:.2e}" for n, e in errs.items()))
    # y: the storage tolerance; mean / rstd are fp32 statistics of exact inputs
    assert errs["y"] <= TOL[dtype] and errs["mean"] <= 1e-5 and errs["rstd"] <= 1e-4


def test_layernorm_large_offset_keeps_the_variance():
    """fp32 rows of mean 1e4 and unit spread: the moment merge keeps rstd."""
    x, x64 = draw(2100, 3000, "f32", 5, scale=1.0, offset=1e4)
    y, mean, rstd = fa_layernorm_rows(x, eps=0.0)
    torch.cuda.synchronize()
    ry, rm, rr = oracle.layernorm_rows(x64, eps=0.0)
    er = rel(rstd.cpu().numpy(), rr)
    ey = rel(y.double().cpu().numpy(), ry)
    say(f"  large offset: rstd={er:.2e} y={ey:.2e}")
    assert er <= 1e-3 and ey <= 1e-3


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("N,C,S,G", [(2, 64, 49, 8), (3, 32, 1000, 4), (4, 16, 3, 16), (2, 12, 8, 3),
                                     (2, 16, 4096, 4)])
def test_group_norm(dtype, N, C, S, G):
    say(f"case groupnorm N={N} C={C} S={S} G={G} {dtype}")
    rng = np.random.default_rng(6)
    x = torch.from_numpy(rng.standard_normal((N, C, S)) * 2 + 1).to(TD[dtype]).cuda()
    g = torch.from_numpy(rng.standard_normal(C)).to(TD[dtype]).cuda()
    b = torch.from_numpy(rng.standard_normal(C)).to(TD[dtype]).cuda()
    y, mean, rstd = fa_group_norm(x, G, g, b, eps=1e-6)
    torch.cuda.synchronize()
    x64 = x.double().cpu().numpy()
    ry, rm, rr = oracle.layernorm_rows(x64.reshape(N * G, C // G * S), g.double().cpu().numpy(),
                                       b.double().cpu().numpy(), eps=1e-6, groups=G, inner=S)
    ey = rel(y.double().cpu().numpy(), ry.reshape(N, C, S))
    say(f"  errors: y={ey:.2e}")
    assert ey <= TOL[dtype] and rel(mean.cpu().numpy().ravel(), rm) <= 1e-5


@pytest.mark.parametrize("cols", [7, 100, 1003])
def test_unaligned_rows(cols):
    """Rows that do not start 16-byte aligned (odd lengths, offset views) take
    element accesses."""
    rng = np.random.default_rng(9)
    base = torch.from_numpy(rng.standard_normal((2200, cols + 1))).to(torch.bfloat16).cuda()
    x = base[:, 1:]                      # every row starts one element in
    x64 = x.double().cpu().numpy()
    y, _ = fa_softmax_rows(x)
    yl, _, _ = fa_layernorm_rows(x)
    torch.cuda.synchronize()
    assert rel(y.double().cpu().numpy(), oracle.softmax_rows(x64)[0]) <= TOL["bf16"]
    assert rel(yl.double().cpu().numpy(), oracle.layernorm_rows(x64)[0]) <= TOL["bf16"]


def test_in_place():
    x, x64 = draw(300, 1000, "bf16", 7, scale=2.0)
    y, _ = fa_softmax_rows(x, out=x)
    torch.cuda.synchronize()
    assert y.data_ptr() == x.data_ptr()
    assert rel(x.double().cpu().numpy(), oracle.softmax_rows(x64)[0]) <= TOL["bf16"]
    x, x64 = draw(2100, 700, "f16", 8, scale=2.0)
    fa_layernorm_rows(x, out=x)
    torch.cuda.synchronize()
    assert rel(x.double().cpu().numpy(), oracle.layernorm_rows(x64)[0]) <= TOL["f16"]
