"""Pins of the oracle's row softmax and LayerNorm / GroupNorm (CPU only).

Library cross-checks (scipy's softmax / logsumexp, torch fp64 layer_norm and
group_norm), 50-digit brute force on tiny rows, closed forms and invariances,
and the streaming states against the two-pass definitions: the softmax
(m, l) merge over random partitions, the Chan-Golub-LeVeque moment merge over
random partitions.
"""
from decimal import Decimal, getcontext

import numpy as np
import pytest
import scipy.special
import torch

import oracle
from oracle import streaming
from tests.test_oracle import rand, rel_err


# ---------------------------------------------------------------- softmax
@pytest.mark.parametrize("shape", [(1, 1), (3, 7), (5, 1000)])
def test_softmax_against_scipy(shape):
    x = rand(shape, 1) * 4.0
    y, lse = oracle.softmax_rows(x)
    assert rel_err(y, scipy.special.softmax(x, axis=1)) < 1e-14
    assert rel_err(lse, scipy.special.logsumexp(x, axis=1)) < 1e-14


def test_softmax_decimal_bruteforce():
    getcontext().prec = 50
    x = rand((3, 6), 2) * 50.0
    y, lse = oracle.softmax_rows(x)
    for i in range(3):
        d = [Decimal(v) for v in x[i]]
        m = max(d)
        e = [(v - m).exp() for v in d]
        s = sum(e)
        for j in range(6):
            assert abs(float(e[j] / s) - y[i, j]) <= 1e-15 * max(1.0, abs(y[i, j]))
        assert abs(float(m + s.ln()) - lse[i]) <= 1e-13


def test_softmax_closed_forms_and_invariances():
    x = rand((4, 9), 3)
    y, lse = oracle.softmax_rows(x)
    y2, lse2 = oracle.softmax_rows(x + 123.0)
    assert rel_err(y, y2) < 1e-13 and np.max(np.abs(lse2 - lse - 123.0)) < 1e-12
    assert np.allclose(y.sum(axis=1), 1.0, atol=1e-14)
    yc, lc = oracle.softmax_rows(np.full((2, 5), 3.0))
    assert np.allclose(yc, 0.2) and np.allclose(lc, 3.0 + np.log(5.0))
    xm = x.copy()
    xm[1] = -np.inf
    xm[2, :4] = -np.inf
    ym, lm = oracle.softmax_rows(xm)
    assert np.all(ym[1] == 0) and np.isneginf(lm[1])
    assert np.all(ym[2, :4] == 0) and abs(ym[2].sum() - 1) < 1e-14


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_softmax_state_merge_over_partitions(seed):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal(300) * 5
    cuts = np.sort(rng.choice(np.arange(1, 300), 7, replace=False))
    m, l = -np.inf, 0.0
    for blk in np.split(np.arange(300), cuts):
        mb = x[blk].max()
        m, l = streaming.merge_stats(m, l, mb, np.exp(x[blk] - mb).sum())
    _, lse = oracle.softmax_rows(x[None])
    assert abs(float(m + np.log(l)) - lse[0]) < 1e-12


# ---------------------------------------------------------------- layernorm
@pytest.mark.parametrize("shape", [(1, 2), (4, 33), (3, 1000)])
@pytest.mark.parametrize("affine", [False, True])
def test_layernorm_against_torch(shape, affine):
    x = rand(shape, 4) * 3 + 1.5
    g = rand((shape[1],), 5) if affine else None
    b = rand((shape[1],), 6) if affine else None
    y, mean, rstd = oracle.layernorm_rows(x, g, b, eps=1e-5)
    ref = torch.nn.functional.layer_norm(torch.from_numpy(x), (shape[1],),
                                         None if g is None else torch.from_numpy(g),
                                         None if b is None else torch.from_numpy(b), eps=1e-5).numpy()
    assert rel_err(y, ref) < 1e-13
    assert rel_err(mean, x.mean(axis=1)) < 1e-14
    assert rel_err(rstd, 1 / np.sqrt(x.var(axis=1) + 1e-5)) < 1e-13


@pytest.mark.parametrize("N,C,S,G", [(2, 6, 5, 3), (3, 8, 1, 2), (1, 4, 7, 4), (2, 6, 4, 1)])
def test_groupnorm_against_torch(N, C, S, G):
    x = rand((N, C, S), 7) * 2 - 0.5
    g, b = rand((C,), 8), rand((C,), 9)
    y, _, _ = oracle.layernorm_rows(x.reshape(N * G, C // G * S), g, b, eps=1e-6, groups=G, inner=S)
    ref = torch.nn.functional.group_norm(torch.from_numpy(x), G, torch.from_numpy(g),
                                         torch.from_numpy(b), eps=1e-6).numpy()
    assert rel_err(y.reshape(N, C, S), ref) < 1e-13


def test_layernorm_decimal_bruteforce():
    getcontext().prec = 50
    x = rand((2, 7), 10) * 1e3 + 5e4       # large offset: a naive one-pass variance loses digits
    y, mean, rstd = oracle.layernorm_rows(x, eps=1e-3)
    for i in range(2):
        d = [Decimal(v) for v in x[i]]
        mu = sum(d) / 7
        var = sum((v - mu) ** 2 for v in d) / 7
        rs = 1 / (var + Decimal(1e-3)).sqrt()
        for j in range(7):
            assert abs(float((d[j] - mu) * rs) - y[i, j]) <= 1e-12
        assert abs(float(mu) - mean[i]) <= 1e-10 and abs(float(rs) - rstd[i]) <= 1e-15


def test_layernorm_closed_forms_and_invariances():
    x = rand((3, 20), 11)
    y, _, _ = oracle.layernorm_rows(x, eps=0.0)
    y2, _, _ = oracle.layernorm_rows(2.5 * x - 7.0, eps=0.0)
    assert rel_err(y, y2) < 1e-13
    assert np.allclose(y.mean(axis=1), 0, atol=1e-14) and np.allclose((y ** 2).mean(axis=1), 1, atol=1e-13)
    b = rand((20,), 12)
    yc, mc, rc = oracle.layernorm_rows(np.full((2, 20), 4.0), np.ones(20), b, eps=1e-5)
    assert np.allclose(yc, b[None]) and np.allclose(mc, 4.0) and np.allclose(rc, 1 / np.sqrt(1e-5))


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_moment_merge_over_partitions(seed):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal(500) * 3 + 1e4
    cuts = np.sort(rng.choice(np.arange(1, 500), 9, replace=False))
    n, mean, m2 = oracle.streaming_moments(x, np.split(np.arange(500), cuts))
    assert n == 500
    assert abs(mean - x.mean()) < 1e-10 and abs(m2 / n - x.var()) < 1e-9 * x.var()
    # one element at a time (Welford's special case) too
    n1, mean1, m21 = oracle.streaming_moments(x, [[i] for i in range(500)])
    assert abs(mean1 - x.mean()) < 1e-10 and abs(m21 / n1 - x.var()) < 1e-9 * x.var()
