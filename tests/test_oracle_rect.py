"""Pins of the oracle for N_q queries against N_k keys (CPU only).

Causal masking with N_q != N_k is aligned at the bottom right (key j visible to
query i iff j <= i + N_k - N_q: the queries are the last N_q positions of the
key sequence).  What pins it, independently of the oracle's own code:

* torch's lower-right causal bias (torch.nn.attention.bias.causal_lower_right),
  a library definition of the same alignment, materialised and handed to
  torch's fp64 SDPA and autograd;
* suffix equivalence: N_q < N_k queries give exactly the last N_q rows of the
  square causal problem, and their gradients those of the square problem
  whose first N_k - N_q rows of dO are zero;
* N_q > N_k: the first N_q - N_k rows see no key (O = 0, LSE = -inf, zero dQ),
  the rest equal the square problem on those rows;
* the element mask against a per-element loop; 50-digit brute force;
  central differences; sampled rows/columns equal to the full backward.
"""
import numpy as np
import pytest
import torch
from torch.nn.attention.bias import causal_lower_right

import oracle
from tests.test_oracle import _decimal_attention, rand, rel_err

SHAPES = [(3, 7), (7, 3), (1, 9), (5, 5), (8, 4)]


def _fwd(q, k, v, scale, **kw):
    o, lse = oracle.forward(q[None, None], k[None, None], v[None, None], scale, **kw)
    return o[0, 0], lse[0, 0]


def _bwd(q, k, v, do, scale, **kw):
    g = oracle.backward(q[None, None], k[None, None], v[None, None], do[None, None], scale, **kw)
    return tuple(x[0, 0] for x in g)


def _rule(nq, nk, causal=False, key_len=None, bm=None, mb=1):
    a = np.ones((nq, nk), bool)
    for i in range(nq):
        for j in range(nk):
            if causal and j > i + nk - nq:
                a[i, j] = False
            if key_len is not None and j >= key_len:
                a[i, j] = False
            if bm is not None and bm[i // mb][j // mb] == 0:
                a[i, j] = False
    return a


def test_allowed_mask_rectangular_bruteforce():
    rng = np.random.default_rng(3)
    for nq, nk in [(4, 10), (10, 4), (6, 6), (2, 8)]:
        mb = 2
        bm = (rng.random(((nq + 1) // mb, (nk + 1) // mb)) < 0.6).astype(np.uint8)
        for causal in (False, True):
            for key_len in (None, 0, 3):
                for blk in (None, bm):
                    a = oracle.allowed_mask(np.arange(nq), nk, causal=causal, key_len=key_len,
                                            block_mask=blk, mb=mb, n_queries=nq)
                    assert np.array_equal(a, _rule(nq, nk, causal, key_len, blk, mb))


@pytest.mark.parametrize("nq,nk", SHAPES)
def test_causal_alignment_is_torch_lower_right(nq, nk):
    want = causal_lower_right(nq, nk)._materialize().numpy()
    got = oracle.allowed_mask(np.arange(nq), nk, causal=True, n_queries=nq)
    assert np.array_equal(got, want)


@pytest.mark.parametrize("nq,nk", SHAPES)
@pytest.mark.parametrize("causal", [False, True])
def test_against_torch_sdpa_and_autograd_fp64(nq, nk, causal):
    B, H, d = 2, 2, 4
    q, k, v = rand((B, H, nq, d), 1), rand((B, H, nk, d), 2), rand((B, H, nk, d), 3)
    do = rand((B, H, nq, d), 4)
    a = causal_lower_right(nq, nk)._materialize().numpy() if causal else np.ones((nq, nk), bool)
    o, lse = oracle.forward(q, k, v, 0.55, causal=causal)
    dq, dk, dv = oracle.backward(q, k, v, do, 0.55, causal=causal)
    rows = a.any(1)
    tq, tk, tv = (torch.from_numpy(x.copy()).requires_grad_() for x in (q, k, v))
    out = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=torch.from_numpy(a),
                                                           scale=0.55)
    # torch gives NaN on rows with no visible key; compare the others and
    # check the oracle's convention (zeros) on those
    ref = out.detach().numpy()
    assert rel_err(o[:, :, rows], ref[:, :, rows]) < 1e-13
    assert np.all(o[:, :, ~rows] == 0) and np.all(np.isneginf(lse[:, :, ~rows]))
    dmask = torch.from_numpy(np.where(rows, 1.0, 0.0))[None, None, :, None]
    (torch.nan_to_num(out) * torch.from_numpy(do) * dmask).sum().backward()
    for g, t in ((dq, tq), (dk, tk), (dv, tv)):
        tg = torch.nan_to_num(t.grad).numpy()
        assert rel_err(g, tg) < 1e-12


@pytest.mark.parametrize("nq", [1, 3, 6])
def test_suffix_of_the_square_causal_problem(nq):
    nk, d = 9, 4
    qf, k, v, dof = rand((nk, d), 1), rand((nk, d), 2), rand((nk, d), 3), rand((nk, d), 4)
    off = nk - nq
    dof[:off] = 0.0
    q, do = qf[off:], dof[off:]
    o, lse = _fwd(q, k, v, 0.7, causal=True)
    of, lsef = _fwd(qf, k, v, 0.7, causal=True)
    assert rel_err(o, of[off:]) < 1e-14 and rel_err(lse, lsef[off:]) < 1e-14
    dq, dk, dv = _bwd(q, k, v, do, 0.7, causal=True)
    dqf, dkf, dvf = _bwd(qf, k, v, dof, 0.7, causal=True)
    assert rel_err(dq, dqf[off:]) < 1e-13
    assert rel_err(dk, dkf) < 1e-13 and rel_err(dv, dvf) < 1e-13


@pytest.mark.parametrize("nq", [10, 13])
def test_more_queries_than_keys(nq):
    nk, d = 6, 3
    q, k, v, do = rand((nq, d), 1), rand((nk, d), 2), rand((nk, d), 3), rand((nq, d), 4)
    off = nq - nk
    o, lse = _fwd(q, k, v, 0.5, causal=True)
    dq, dk, dv = _bwd(q, k, v, do, 0.5, causal=True)
    assert np.all(o[:off] == 0) and np.all(np.isneginf(lse[:off])) and np.all(dq[:off] == 0)
    o2, lse2 = _fwd(q[off:], k, v, 0.5, causal=True)
    dq2, dk2, dv2 = _bwd(q[off:], k, v, do[off:], 0.5, causal=True)
    assert rel_err(o[off:], o2) < 1e-14 and rel_err(lse[off:], lse2) < 1e-14
    assert rel_err(dq[off:], dq2) < 1e-14 and rel_err(dk, dk2) < 1e-14 and rel_err(dv, dv2) < 1e-14


@pytest.mark.parametrize("nq,nk", SHAPES)
@pytest.mark.parametrize("causal", [False, True])
def test_decimal_bruteforce_rectangular(nq, nk, causal):
    d = 3
    q, k, v = rand((nq, d), 5) * 30.0, rand((nk, d), 6), rand((nk, d), 7)
    o, lse = _fwd(q, k, v, 0.37, causal=causal, key_lens=[nk - 1])
    o_ref, lse_ref = _decimal_attention(q, k, v, 0.37, _rule(nq, nk, causal, nk - 1))
    assert rel_err(o, o_ref) < 1e-13
    assert rel_err(lse, lse_ref) < 1e-13


@pytest.mark.parametrize("nq,nk", [(3, 8), (8, 3)])
def test_rectangular_central_differences(nq, nk):
    d = 3
    q, k, v, do = rand((nq, d), 8), rand((nk, d), 9), rand((nk, d), 10), rand((nq, d), 11)
    kw = dict(causal=True, key_lens=[nk - 1], dropout=(0.25, 3, 1))
    dq, dk, dv = _bwd(q, k, v, do, 0.8, **kw)
    h = 1e-6
    for x, g in ((q, dq), (k, dk), (v, dv)):
        num = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            old = x[idx]
            x[idx] = old + h
            fp = float(np.sum(_fwd(q, k, v, 0.8, **kw)[0] * do))
            x[idx] = old - h
            fm = float(np.sum(_fwd(q, k, v, 0.8, **kw)[0] * do))
            x[idx] = old
            num[idx] = (fp - fm) / (2 * h)
        assert np.max(np.abs(num - g)) <= 1e-6 * max(1.0, np.max(np.abs(g)))


@pytest.mark.parametrize("nq,nk", [(40, 100), (100, 40)])
def test_sampled_equals_full_rectangular(nq, nk):
    d = 8
    q, k, v, do = rand((nq, d), 12), rand((nk, d), 13), rand((nk, d), 14), rand((nq, d), 15)
    bm = np.ones((-(-nq // 25), -(-nk // 25)), np.uint8)
    bm[0, -1] = 0
    kw = dict(causal=True, block_mask=bm, mb=25, dropout=(0.3, 9, 2))
    dq, dk, dv = _bwd(q, k, v, do, 0.3, key_lens=[nk - 3], **kw)
    o, lse = _fwd(q, k, v, 0.3, key_lens=[nk - 3], **kw)
    rows, cols = np.array([0, 7, nq - 1]), np.array([2, 19, nk - 1])
    ro, rl, rdq, rdk, rdv = oracle.gradients_sampled(q, k, v, do, 0.3, rows, cols, key_len=nk - 3, **kw)
    np.testing.assert_allclose(ro, o[rows], atol=1e-12)
    np.testing.assert_array_equal(np.isfinite(rl), np.isfinite(lse[rows]))
    np.testing.assert_allclose(rdq, dq[rows], atol=1e-12)
    np.testing.assert_allclose(rdk, dk[cols], atol=1e-12)
    np.testing.assert_allclose(rdv, dv[cols], atol=1e-12)
