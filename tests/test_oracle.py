"""Pins for the fp64 oracle, against things other than itself.

Each test below ties a part of ``oracle`` to something it does not share code
with: hand-derived values of the definition (tests/golden), 50-digit decimal
brute force, the pages' own block recurrence and merge equation, closed forms,
invariants, library routines (torch fp64 SDPA/autograd, scipy logsumexp) and
central finite differences.  A dropped term, a wrong sign, a swapped operand or
a mis-applied mask in the oracle fails at least one of them.
"""
import json
import math
import os
from decimal import Decimal, getcontext
from fractions import Fraction

import numpy as np
import pytest
import scipy.special
import torch

import oracle
from oracle import streaming

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ----------------------------------------------------------------- helpers
def _ev(expr):
    """Evaluate a golden-file entry: a fraction, ln(x), or products of those."""
    return float(eval(expr, {"__builtins__": {}}, {"ln": math.log}))


def _arr(rows):
    return np.array([[_ev(x) for x in r] for r in rows], dtype=np.float64)


def rel_err(x, ref):
    x, ref = np.asarray(x, np.float64), np.asarray(ref, np.float64)
    den = np.max(np.abs(ref[np.isfinite(ref)])) if np.isfinite(ref).any() else 1.0
    fin = np.isfinite(ref)
    assert np.array_equal(np.isfinite(x), fin), "finite patterns differ"
    assert np.array_equal(x[~fin], ref[~fin])
    return float(np.max(np.abs(x[fin] - ref[fin])) / max(den, 1e-300)) if fin.any() else 0.0


def rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def fwd1(q, k, v, scale, **kw):
    """oracle.forward on one (batch, head) given as 2-D arrays."""
    key_len = kw.pop("key_len", None)
    o, lse = oracle.forward(q[None, None], k[None, None], v[None, None], scale,
                            key_lens=None if key_len is None else [key_len], **kw)
    return o[0, 0], lse[0, 0]


def bwd1(q, k, v, do, scale, **kw):
    key_len = kw.pop("key_len", None)
    dq, dk, dv = oracle.backward(q[None, None], k[None, None], v[None, None],
                                 do[None, None], scale,
                                 key_lens=None if key_len is None else [key_len], **kw)
    return dq[0, 0], dk[0, 0], dv[0, 0]


MASKS = [
    dict(),
    dict(causal=True),
    dict(key_len=3),
    dict(causal=True, key_len=4),
    dict(block_mask=np.array([[1, 0, 1], [0, 1, 0], [1, 1, 1]], np.uint8), mb=2),
    dict(causal=True, block_mask=np.array([[1, 0, 0], [1, 1, 0], [0, 1, 1]], np.uint8), mb=2),
]


# ------------------------------------------------- hand-derived golden values
def test_golden_hand_example():
    g = json.load(open(os.path.join(GOLDEN, "hand_example.json")))
    q, k, v, do = (_arr(g[n]) for n in ("q", "k", "v", "dout"))
    scale = _ev(g["scale"])
    o, lse = fwd1(q, k, v, scale)
    assert np.allclose(o, _arr(g["o"]), rtol=0, atol=1e-14)
    assert np.allclose(lse, [_ev(x) for x in g["lse"]], rtol=0, atol=1e-14)
    o, lse = fwd1(q, k, v, scale, causal=True)
    assert np.allclose(o, _arr(g["o_causal"]), rtol=0, atol=1e-14)
    assert np.allclose(lse, [_ev(x) for x in g["lse_causal"]], rtol=0, atol=1e-14)
    dq, dk, dv = bwd1(q, k, v, do, scale)
    assert np.allclose(dq, _arr(g["dq"]), rtol=0, atol=1e-14)
    assert np.allclose(dk, _arr(g["dk"]), rtol=0, atol=1e-14)
    assert np.allclose(dv, _arr(g["dv"]), rtol=0, atol=1e-14)


# ------------------------------------------------ 50-digit decimal brute force
def _decimal_attention(q, k, v, scale, allowed):
    getcontext().prec = 50
    N, d = k.shape
    R = q.shape[0]
    o = np.zeros((R, v.shape[1]))
    lse = np.zeros(R)
    sc = Decimal(scale)
    for i in range(R):
        s = []
        for j in range(N):
            if allowed[i, j]:
                s.append((j, sc * sum(Decimal(q[i, c]) * Decimal(k[j, c]) for c in range(d))))
        if not s:
            lse[i] = -np.inf
            continue
        m = max(x for _, x in s)
        e = [(j, (x - m).exp()) for j, x in s]
        l = sum(x for _, x in e)
        for c in range(v.shape[1]):
            o[i, c] = float(sum(x * Decimal(v[j, c]) for j, x in e) / l)
        lse[i] = float(m + l.ln())
    return o, lse


@pytest.mark.parametrize("mi", range(len(MASKS)))
@pytest.mark.parametrize("gap", [1.0, 1000.0])
def test_decimal_bruteforce_forward(mi, gap):
    kw = dict(MASKS[mi])
    N, d = 6, 3
    q, k, v = rand((N, d), 1) * gap, rand((N, d), 2), rand((N, d), 3)
    scale = 0.37
    o, lse = fwd1(q, k, v, scale, **dict(kw))
    allowed = oracle.allowed_mask(np.arange(N), N, causal=kw.get("causal", False),
                                  key_len=kw.get("key_len"), block_mask=kw.get("block_mask"),
                                  mb=kw.get("mb", 128))
    o_ref, lse_ref = _decimal_attention(q, k, v, scale, allowed)
    assert rel_err(o, o_ref) < 1e-13
    assert rel_err(lse, lse_ref) < 1e-13


def test_allowed_mask_bruteforce():
    """The element mask against a per-element loop over the stated rules."""
    N, mb = 10, 2
    bm = (np.random.default_rng(5).random((5, 5)) < 0.5).astype(np.uint8)
    for causal in (False, True):
        for key_len in (None, 0, 7):
            for blk in (None, bm):
                a = oracle.allowed_mask(np.arange(N), N, causal=causal, key_len=key_len,
                                        block_mask=blk, mb=mb)
                for i in range(N):
                    for j in range(N):
                        ok = True
                        if causal and j > i:
                            ok = False
                        if key_len is not None and j >= key_len:
                            ok = False
                        if blk is not None and blk[i // mb][j // mb] == 0:
                            ok = False
                        assert a[i, j] == ok


# ---------------------------------------- the pages' recurrence and merge rule
@pytest.mark.parametrize("mi", range(len(MASKS)))
@pytest.mark.parametrize("seed", [0, 1, 2])
def test_streaming_recurrence_matches_two_pass(mi, seed):
    kw = dict(MASKS[mi])
    N, d = 6, 4
    rng = np.random.default_rng(100 + seed)
    q, k, v = rng.standard_normal((N, d)) * 3, rng.standard_normal((N, d)), rng.standard_normal((N, d))
    scale = 0.5
    o, lse = fwd1(q, k, v, scale, **dict(kw))
    allowed = oracle.allowed_mask(np.arange(N), N, causal=kw.get("causal", False),
                                  key_len=kw.get("key_len"), block_mask=kw.get("block_mask"),
                                  mb=kw.get("mb", 128))
    # random partition of the key axis into contiguous blocks, in a random order
    cuts = sorted(rng.choice(np.arange(1, N), size=rng.integers(1, N), replace=False))
    blocks = np.split(np.arange(N), cuts)
    rng.shuffle(blocks)
    o_s, m_s, l_s = streaming.streaming_forward(q, k, v, scale, blocks, allowed=allowed)
    lse_s = np.where(l_s > 0, m_s + np.log(np.where(l_s > 0, l_s, 1)), -np.inf)
    assert rel_err(o_s, o) < 1e-12
    assert rel_err(lse_s, lse) < 1e-12


def test_merge_rule_of_two_halves():
    rng = np.random.default_rng(7)
    x = rng.standard_normal((5, 9)) * 10
    a, b = x[:, :4], x[:, 4:]
    m, l = streaming.merge_stats(a.max(1), np.exp(a - a.max(1, keepdims=True)).sum(1),
                                 b.max(1), np.exp(b - b.max(1, keepdims=True)).sum(1))
    assert np.allclose(m, x.max(1), rtol=0, atol=0)
    assert np.allclose(m + np.log(l), scipy.special.logsumexp(x, axis=1), rtol=1e-14, atol=1e-13)
    # an empty part (m = -inf, l = 0) is the identity of the merge
    m2, l2 = streaming.merge_stats(np.full(5, -np.inf), np.zeros(5), m, l)
    assert np.array_equal(m2, m) and np.allclose(l2, l, rtol=1e-15)


# ------------------------------------------------ closed forms, special cases
def test_single_key():
    q, k, v = rand((1, 5), 1), rand((1, 5), 2), rand((1, 5), 3)
    o, lse = fwd1(q, k, v, 0.3)
    assert np.allclose(o, v, rtol=0, atol=1e-15)
    assert np.allclose(lse, 0.3 * (q @ k.T)[0], rtol=1e-15)


def test_causal_first_row_is_first_value():
    q, k, v = rand((7, 4), 1), rand((7, 4), 2), rand((7, 4), 3)
    o, lse = fwd1(q, k, v, 0.5, causal=True)
    assert np.allclose(o[0], v[0], rtol=0, atol=1e-15)
    assert math.isclose(lse[0], 0.5 * float(q[0] @ k[0]), rel_tol=1e-14)


@pytest.mark.parametrize("mi", range(len(MASKS)))
def test_zero_scale_gives_mean_of_visible_values(mi):
    kw = dict(MASKS[mi])
    N = 6
    q, k, v = rand((N, 3), 1), rand((N, 3), 2), rand((N, 3), 3)
    o, lse = fwd1(q, k, v, 0.0, **dict(kw))
    a = oracle.allowed_mask(np.arange(N), N, causal=kw.get("causal", False), key_len=kw.get("key_len"),
                            block_mask=kw.get("block_mask"), mb=kw.get("mb", 128))
    for i in range(N):
        cnt = a[i].sum()
        if cnt == 0:
            assert np.all(o[i] == 0) and lse[i] == -np.inf
        else:
            assert np.allclose(o[i], v[a[i]].mean(0), rtol=0, atol=1e-15)
            assert math.isclose(lse[i], math.log(cnt), rel_tol=1e-15)


def test_constant_values_give_constant_output():
    q, k = rand((9, 4), 1) * 4, rand((9, 4), 2)
    v = np.tile(np.array([[1.5, -2.0, 0.25, 3.0]]), (9, 1))
    for kw in (dict(), dict(causal=True), dict(key_len=5)):
        o, _ = fwd1(q, k, v, 0.7, **kw)
        assert np.allclose(o, v, rtol=0, atol=1e-14)


def test_padding_equals_truncated_dense():
    N, L = 9, 5
    q, k, v = rand((N, 4), 1), rand((N, 4), 2), rand((N, 4), 3)
    o, lse = fwd1(q, k, v, 0.4, key_len=L)
    o2, lse2 = fwd1(q, k[:L].copy(), v[:L].copy(), 0.4)   # N_k = L: same rows, fewer keys
    assert rel_err(o, o2) < 1e-14 and rel_err(lse, lse2) < 1e-14
    o3, lse3 = fwd1(q, k, v, 0.4, key_len=N)
    o4, lse4 = fwd1(q, k, v, 0.4)
    assert np.array_equal(o3, o4) and np.array_equal(lse3, lse4)


def test_block_mask_special_cases():
    N, mb = 8, 2
    q, k, v = rand((N, 3), 1), rand((N, 3), 2), rand((N, 3), 3)
    ones = np.ones((4, 4), np.uint8)
    o, lse = fwd1(q, k, v, 0.6, block_mask=ones, mb=mb)
    o2, lse2 = fwd1(q, k, v, 0.6)
    assert rel_err(o, o2) < 1e-15 and rel_err(lse, lse2) < 1e-15
    eye = np.eye(4, dtype=np.uint8)
    o, lse = fwd1(q, k, v, 0.6, block_mask=eye, mb=mb)
    for c in range(4):
        sl = slice(c * mb, (c + 1) * mb)
        oc, lc = fwd1(q[sl].copy(), k[sl].copy(), v[sl].copy(), 0.6)
        assert rel_err(o[sl], oc) < 1e-14 and rel_err(lse[sl], lc) < 1e-14


def test_fully_masked_row_convention():
    q, k, v, do = (rand((4, 3), s) for s in range(4))
    bm = np.array([[1, 0], [0, 0]], np.uint8)    # rows 2,3 see nothing
    o, lse = fwd1(q, k, v, 0.5, block_mask=bm, mb=2)
    assert np.all(o[2:] == 0) and np.all(lse[2:] == -np.inf) and np.all(np.isfinite(o))
    dq, dk, dv = bwd1(q, k, v, do, 0.5, block_mask=bm, mb=2)
    assert np.all(dq[2:] == 0) and np.all(np.isfinite(dq)) and np.all(np.isfinite(dk))
    o, lse = fwd1(q, k, v, 0.5, key_len=0)
    assert np.all(o == 0) and np.all(lse == -np.inf)


# --------------------------------------------------------------- invariants
@pytest.mark.parametrize("mi", range(len(MASKS)))
def test_probability_rows_sum_to_one(mi):
    """With V = identity, O is P itself."""
    kw = dict(MASKS[mi])
    N = 6
    q, k = rand((N, 5), 1) * 3, rand((N, 5), 2)
    o, _ = fwd1(q, k, np.eye(N), 0.8, **dict(kw))
    p = oracle.probabilities(q, k, 0.8, causal=kw.get("causal", False), key_len=kw.get("key_len"),
                             block_mask=kw.get("block_mask"), mb=kw.get("mb", 128))
    assert np.allclose(o, p, rtol=0, atol=1e-15)
    sums = o.sum(1)
    has = sums > 0
    assert np.all(np.abs(sums[has] - 1) < 1e-14)
    assert np.all(o >= 0)


def test_permutation_equivariance_and_shift_invariance():
    N = 11
    q, k, v = rand((N, 4), 1), rand((N, 4), 2), rand((N, 4), 3)
    o, lse = fwd1(q, k, v, 0.5)
    perm = np.random.default_rng(3).permutation(N)
    o2, lse2 = fwd1(q, k[perm].copy(), v[perm].copy(), 0.5)
    assert rel_err(o2, o) < 1e-14 and rel_err(lse2, lse) < 1e-14
    o3, lse3 = fwd1(q[perm].copy(), k, v, 0.5)
    assert rel_err(o3, o[perm]) < 1e-14 and rel_err(lse3, lse[perm]) < 1e-14
    u = np.array([0.3, -1.2, 2.0, 0.7])
    o4, _ = fwd1(q, k + u[None, :], v, 0.5)       # shifts each score row by a constant
    assert rel_err(o4, o) < 1e-13


# ----------------------------------------------------- library cross-checks
@pytest.mark.parametrize("mi", range(len(MASKS)))
def test_against_torch_sdpa_fp64(mi):
    kw = dict(MASKS[mi])
    B, H, N, d = 2, 3, 6, 5
    q, k, v = rand((B, H, N, d), 1), rand((B, H, N, d), 2), rand((B, H, N, d), 3)
    a = oracle.allowed_mask(np.arange(N), N, causal=kw.get("causal", False), key_len=kw.get("key_len"),
                            block_mask=kw.get("block_mask"), mb=kw.get("mb", 128))
    if not a.any(1).all():
        pytest.skip("torch returns NaN on a fully masked row")
    lens = None if kw.get("key_len") is None else [kw["key_len"]] * B
    o, lse = oracle.forward(q, k, v, 0.45, causal=kw.get("causal", False), key_lens=lens,
                            block_mask=kw.get("block_mask"), mb=kw.get("mb", 128))
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v),
        attn_mask=torch.from_numpy(a), scale=0.45).numpy()
    assert rel_err(o, ref) < 1e-13
    s = 0.45 * np.einsum("bhid,bhjd->bhij", q, k)
    lse_ref = scipy.special.logsumexp(np.where(a, s, -np.inf), axis=-1)
    assert rel_err(lse, lse_ref) < 1e-13


@pytest.mark.parametrize("mi", range(len(MASKS)))
def test_backward_against_torch_autograd(mi):
    kw = dict(MASKS[mi])
    B, H, N, d = 1, 2, 6, 4
    q, k, v, do = (rand((B, H, N, d), s) for s in (1, 2, 3, 4))
    a = oracle.allowed_mask(np.arange(N), N, causal=kw.get("causal", False), key_len=kw.get("key_len"),
                            block_mask=kw.get("block_mask"), mb=kw.get("mb", 128))
    if not a.any(1).all():
        pytest.skip("torch returns NaN on a fully masked row")
    lens = None if kw.get("key_len") is None else [kw["key_len"]] * B
    dq, dk, dv = oracle.backward(q, k, v, do, 0.6, causal=kw.get("causal", False), key_lens=lens,
                                 block_mask=kw.get("block_mask"), mb=kw.get("mb", 128))
    tq, tk, tv = (torch.from_numpy(x.copy()).requires_grad_() for x in (q, k, v))
    out = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=torch.from_numpy(a), scale=0.6)
    out.backward(torch.from_numpy(do))
    assert rel_err(dq, tq.grad.numpy()) < 1e-12
    assert rel_err(dk, tk.grad.numpy()) < 1e-12
    assert rel_err(dv, tv.grad.numpy()) < 1e-12


# -------------------------------------------------- finite-difference gradients
@pytest.mark.parametrize("mi", range(len(MASKS)))
def test_backward_central_differences(mi):
    kw = dict(MASKS[mi])
    N, d = 6, 3
    q, k, v, do = (rand((N, d), s) for s in (11, 12, 13, 14))
    scale = 0.7
    dq, dk, dv = bwd1(q, k, v, do, scale, **dict(kw))

    def loss(q_, k_, v_):
        o, _ = fwd1(q_, k_, v_, scale, **dict(kw))
        return float(np.sum(o * do))

    eps = 1e-6
    for which, g in ((0, dq), (1, dk), (2, dv)):
        num = np.zeros_like(g)
        for i in range(N):
            for c in range(d):
                args_p = [q.copy(), k.copy(), v.copy()]
                args_m = [q.copy(), k.copy(), v.copy()]
                args_p[which][i, c] += eps
                args_m[which][i, c] -= eps
                num[i, c] = (loss(*args_p) - loss(*args_m)) / (2 * eps)
        assert np.max(np.abs(num - g)) <= 1e-6 * max(1.0, np.max(np.abs(g)))


@pytest.mark.parametrize("mi", range(len(MASKS)))
def test_backward_invariants(mi):
    kw = dict(MASKS[mi])
    N, d = 6, 4
    q, k, v, do = (rand((N, d), s) for s in (21, 22, 23, 24))
    lens = None if kw.get("key_len") is None else [kw["key_len"]]
    dq, dk, dv, (o, lse, Dp, Do) = oracle.backward(
        q[None, None], k[None, None], v[None, None], do[None, None], 0.5,
        causal=kw.get("causal", False), key_lens=lens, block_mask=kw.get("block_mask"),
        mb=kw.get("mb", 128), return_aux=True)
    dq, dk, dv = dq[0, 0], dk[0, 0], dv[0, 0]
    a = oracle.allowed_mask(np.arange(N), N, causal=kw.get("causal", False), key_len=kw.get("key_len"),
                            block_mask=kw.get("block_mask"), mb=kw.get("mb", 128))
    # rows of dS sum to zero -> sum over keys of dK is zero
    assert np.allclose(dk.sum(0), 0, atol=1e-13)
    # each row of P sums to 1 -> sum over keys of dV equals sum of dO over rows with a visible key
    assert np.allclose(dv.sum(0), do[a.any(1)].sum(0), atol=1e-13)
    # rowsum(dO * O) == rowsum(P * dP)
    assert np.allclose(Dp, Do, atol=1e-13)
    # keys nobody sees get zero gradient
    unseen = ~a.any(0)
    assert np.all(dk[unseen] == 0) and np.all(dv[unseen] == 0)
    # forward returned by backward equals forward
    o2, lse2 = fwd1(q, k, v, 0.5, **dict(kw))
    assert np.array_equal(o[0, 0], o2) and np.array_equal(lse[0, 0], lse2)


def test_backward_single_key():
    q, k, v, do = (rand((1, 4), s) for s in range(4))
    dq, dk, dv = bwd1(q, k, v, do, 0.9)
    assert np.all(dq == 0) and np.all(dk == 0) and np.allclose(dv, do, rtol=0, atol=1e-15)


def test_chunking_does_not_change_results():
    B, H, N, d = 1, 2, 37, 8
    q, k, v, do = (rand((B, H, N, d), s) for s in range(4))
    o1, l1 = oracle.forward(q, k, v, 0.3, causal=True, chunk=5)
    o2, l2 = oracle.forward(q, k, v, 0.3, causal=True, chunk=1024)
    assert rel_err(o1, o2) < 1e-15 and rel_err(l1, l2) < 1e-15
    g1 = oracle.backward(q, k, v, do, 0.3, causal=True, chunk=5)
    g2 = oracle.backward(q, k, v, do, 0.3, causal=True, chunk=1024)
    for x, y in zip(g1, g2):
        assert rel_err(x, y) < 1e-13


@pytest.mark.parametrize("mi", range(len(MASKS)))
def test_sampled_gradients_equal_full_backward(mi):
    """The sampled-row/column evaluation used at full sizes equals the full
    backward (which the finite-difference and autograd tests pin)."""
    kw = dict(MASKS[mi])
    N, d = 6, 4
    q, k, v, do = (rand((N, d), s) for s in (31, 32, 33, 34))
    dq, dk, dv = bwd1(q, k, v, do, 0.55, **dict(kw))
    o, lse = fwd1(q, k, v, 0.55, **dict(kw))
    rows, cols = np.array([0, 3, 5]), np.array([1, 2, 5])
    o_r, lse_r, dq_r, dk_c, dv_c = oracle.gradients_sampled(
        q, k, v, do, 0.55, rows, cols, causal=kw.get("causal", False), key_len=kw.get("key_len"),
        block_mask=kw.get("block_mask"), mb=kw.get("mb", 128), chunk=4)
    assert rel_err(o_r, o[rows]) < 1e-14 and rel_err(lse_r, lse[rows]) < 1e-14
    assert np.allclose(dq_r, dq[rows], rtol=0, atol=1e-13)
    assert np.allclose(dk_c, dk[cols], rtol=0, atol=1e-13)
    assert np.allclose(dv_c, dv[cols], rtol=0, atol=1e-13)
