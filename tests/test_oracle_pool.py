"""The head-parallel schedule of the oracle (tests/_oracle_pool.py) gives what
one oracle call over all heads gives: the per-(batch, head) slices, with
their key lengths, per-head block masks and dropout head indices, are the
same problem."""
import numpy as np
import pytest

import oracle
from tests import _oracle_pool as pool


def _rel(a, b):
    return float(np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300))


@pytest.mark.parametrize("mode", ["dense", "causal_padding", "blocksparse_per_head", "dropout"])
def test_pool_equals_one_call(mode):
    rng = np.random.default_rng(11)
    B, H, N, d = 2, 3, 256, 16
    q, k, v, do = (rng.standard_normal((B, H, N, d)) for _ in range(4))
    kw = {}
    if mode == "causal_padding":
        kw = dict(causal=True, key_lens=np.array([200, 37]))
    elif mode == "blocksparse_per_head":
        m = (rng.random((H, 2, 2)) < 0.5).astype(np.uint8)
        for h in range(H):
            np.fill_diagonal(m[h], 1)
        m[1, 0, 1] = 1
        m[2, 1, 0] = 0
        kw = dict(block_mask=m, mb=128, key_lens=np.array([256, 130]))
    elif mode == "dropout":
        kw = dict(causal=True, dropout=(0.3, 12345 + (7 << 32), 5))
    ref = oracle.backward(q, k, v, do, 0.25, return_aux=True, **kw)
    got = pool.backward_all_heads(q, k, v, do, 0.25, n_workers=4, **kw)
    for x, r in zip(got[:3], ref[:3]):
        assert _rel(x, r) < 1e-12
    assert _rel(got[3], ref[3][0]) < 1e-12
    fin = np.isfinite(ref[3][1])
    assert np.array_equal(np.isfinite(got[4]), fin)
    assert np.max(np.abs(got[4][fin] - ref[3][1][fin])) < 1e-12
    fo, fl = pool.forward_all_heads(q, k, v, 0.25, n_workers=3, **kw)
    assert _rel(fo, ref[3][0]) < 1e-12
    assert np.array_equal(np.isfinite(fl), fin)


def test_bh_offset_selects_the_dropout_head():
    """One head evaluated alone with bh_offset = b*H + h draws that head's keep
    mask: equal to the head of the full call, and different without it."""
    rng = np.random.default_rng(3)
    B, H, N, d = 2, 2, 64, 8
    q, k, v, do = (rng.standard_normal((B, H, N, d)) for _ in range(4))
    dr = (0.5, 99, 0)
    o_all, _ = oracle.forward(q, k, v, 0.3, dropout=dr)
    b, h = 1, 1
    sl = (slice(b, b + 1), slice(h, h + 1))
    o_one, _ = oracle.forward(q[sl], k[sl], v[sl], 0.3, dropout=dr, bh_offset=b * H + h)
    o_wrong, _ = oracle.forward(q[sl], k[sl], v[sl], 0.3, dropout=dr)
    assert np.array_equal(o_one[0, 0], o_all[b, h])
    assert not np.allclose(o_wrong[0, 0], o_all[b, h])


@pytest.mark.parametrize("causal", [False, True])
def test_row_blocks_equal_one_call(causal):
    """Query-row blocks (causal: each against the keys up to its last row)
    reassemble the whole problem: O, LSE, dQ rows exactly, dK and dV as the
    sum of the blocks' shares."""
    rng = np.random.default_rng(5)
    B, H, N, d = 1, 2, 300, 16
    q, k, v, do = (rng.standard_normal((B, H, N, d)) for _ in range(4))
    ref = oracle.backward(q, k, v, do, 0.3, causal=causal, return_aux=True)
    got = pool.backward_row_blocks(q, k, v, do, 0.3, causal=causal, block_rows=64, chunk=50,
                                   n_workers=4)
    for x, r in zip(got[:4], ref[:3] + (ref[3][0],)):
        assert _rel(x, r) < 1e-12
    assert np.max(np.abs(got[4] - ref[3][1])) < 1e-12


@pytest.mark.parametrize("causal", [False, True])
def test_row_blocks_with_more_keys_than_queries(causal):
    rng = np.random.default_rng(6)
    q, do = (rng.standard_normal((1, 2, 200, 8)) for _ in range(2))
    k, v = (rng.standard_normal((1, 2, 520, 8)) for _ in range(2))
    ref = oracle.backward(q, k, v, do, 0.4, causal=causal, return_aux=True)
    got = pool.backward_row_blocks(q, k, v, do, 0.4, causal=causal, block_rows=48, chunk=30,
                                   n_workers=3)
    for x, r in zip(got[:4], ref[:3] + (ref[3][0],)):
        assert _rel(x, r) < 1e-12


def test_row_blocks_with_block_mask():
    rng = np.random.default_rng(8)
    B, H, N, d = 1, 2, 512, 8
    q, k, v, do = (rng.standard_normal((B, H, N, d)) for _ in range(4))
    m = (rng.random((H, 4, 4)) < 0.4).astype(np.uint8)
    for h in range(H):
        np.fill_diagonal(m[h], 1)
    ref = oracle.backward(q, k, v, do, 0.3, block_mask=m, mb=128, return_aux=True)
    got = pool.backward_row_blocks(q, k, v, do, 0.3, block_mask=m, mb=128, block_rows=256,
                                   chunk=100, n_workers=4)
    for x, r in zip(got[:4], ref[:3] + (ref[3][0],)):
        assert _rel(x, r) < 1e-12
