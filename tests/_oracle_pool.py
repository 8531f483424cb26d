"""Run the fp64 oracle over every (batch, head) of a full-size problem, one
head per worker thread (test infrastructure).

Each (b, h) of exact attention is an independent problem: the oracle is called
on the one-head slice with that batch's key length, that head's block mask
and, for dropout, ``bh_offset = b*H + h`` (the keep mask's head index), and
the slices are put back together.  numpy releases the interpreter lock inside
its matrix products and element-wise kernels, so heads run in parallel; the
BLAS library is held to one thread per worker so that the workers do not
oversubscribe the cores.  The per-head result is exactly what one call over
all heads returns (``tests/test_oracle.py`` pins that), so this is only a
faster schedule of the same computation.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

import oracle


def workers() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _head_args(b, h, H, key_lens, block_mask):
    kl = None if key_lens is None else np.asarray(key_lens).reshape(-1)[b:b + 1]
    bm = None
    if block_mask is not None:
        bm = np.asarray(block_mask)
        if bm.ndim == 3:
            bm = bm[h]
    return kl, bm


def backward_all_heads(q, k, v, do, scale, *, causal=False, key_lens=None, block_mask=None, mb=128,
                       dropout=None, n_workers=None):
    """oracle.backward over every head, heads in parallel.

    q, do: [B, H, N_q, d] float64; k, v: [B, H, N_k, d].  Returns
    (dq, dk, dv, o, lse) as float64 arrays of the same shapes (lse [B, H, N_q]).
    """
    B, H, Nq, d = q.shape
    Nk = k.shape[2]
    dq = np.empty_like(q)
    dk = np.empty_like(k)
    dv = np.empty_like(v)
    o = np.empty((B, H, Nq, v.shape[3]))
    lse = np.empty((B, H, Nq))

    def one(bh):
        b, h = divmod(bh, H)
        kl, bm = _head_args(b, h, H, key_lens, block_mask)
        sl = (slice(b, b + 1), slice(h, h + 1))
        g = oracle.backward(q[sl], k[sl], v[sl], do[sl], scale, causal=causal, key_lens=kl,
                            block_mask=bm, mb=mb, return_aux=True, dropout=dropout,
                            bh_offset=b * H + h)
        dq[b, h], dk[b, h], dv[b, h] = g[0][0, 0], g[1][0, 0], g[2][0, 0]
        o[b, h], lse[b, h] = g[3][0][0, 0], g[3][1][0, 0]

    _run(one, B * H, n_workers)
    return dq, dk, dv, o, lse


def forward_all_heads(q, k, v, scale, *, causal=False, key_lens=None, block_mask=None, mb=128,
                      dropout=None, n_workers=None):
    """oracle.forward over every head, heads in parallel.  Returns (o, lse)."""
    B, H, Nq, d = q.shape
    o = np.empty((B, H, Nq, v.shape[3]))
    lse = np.empty((B, H, Nq))

    def one(bh):
        b, h = divmod(bh, H)
        kl, bm = _head_args(b, h, H, key_lens, block_mask)
        sl = (slice(b, b + 1), slice(h, h + 1))
        ob, lb = oracle.forward(q[sl], k[sl], v[sl], scale, causal=causal, key_lens=kl,
                                block_mask=bm, mb=mb, dropout=dropout, bh_offset=b * H + h)
        o[b, h], lse[b, h] = ob[0, 0], lb[0, 0]

    _run(one, B * H, n_workers)
    return o, lse


def backward_row_blocks(q, k, v, do, scale, *, causal=False, block_mask=None, mb=128,
                        block_rows=1024, chunk=256, n_workers=None):
    """oracle.backward of a problem without key padding, split by blocks of
    query rows as well as by heads.

    Query rows are independent: block [r0, r1) has the O, LSE and dQ rows of
    the whole problem, and contributes its share of dK and dV.  Causal, the
    block is given only the keys [0, r1 + N_k - N_q) (the others are
    invisible to all of its rows), and the oracle's causal rule for
    N_q' = r1 - r0 queries against N_k' = r1 + N_k - N_q keys,
    j <= i' + N_k' - N_q' = (i' + r0) + N_k - N_q, is the rule of the whole
    problem at row i = i' + r0.  With a block mask (non-causal only, blocks of
    rows a multiple of mb) the block gets the mask rows r0/mb .. r1/mb - 1.
    The dK / dV shares are summed in float64 (in completion order; the sums
    differ from a fixed order by rounding in the 16th digit).  ``chunk``
    bounds the oracle's working set per worker.
    """
    import threading

    B, H, N, d = q.shape
    Nk = k.shape[2]
    assert not causal or Nk >= N, "causal with fewer keys than queries is not split here"
    assert block_mask is None or (not causal and block_rows % mb == 0)
    dq = np.empty_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    o = np.empty((B, H, N, v.shape[3]))
    lse = np.empty((B, H, N))
    tasks = [(b, h, r0, min(N, r0 + block_rows)) for b in range(B) for h in range(H)
             for r0 in range(0, N, block_rows)]
    lock = threading.Lock()

    def one(t):
        b, h, r0, r1 = tasks[t]
        kend = r1 + Nk - N if causal else Nk
        sl = (slice(b, b + 1), slice(h, h + 1))
        bm = None
        if block_mask is not None:
            _, bm = _head_args(b, h, H, None, block_mask)
            bm = bm[r0 // mb:(r1 + mb - 1) // mb]
        g = oracle.backward(q[sl][:, :, r0:r1], k[sl][:, :, :kend], v[sl][:, :, :kend],
                            do[sl][:, :, r0:r1], scale, causal=causal, block_mask=bm, mb=mb,
                            chunk=chunk, return_aux=True)
        dq[b, h, r0:r1] = g[0][0, 0]
        o[b, h, r0:r1], lse[b, h, r0:r1] = g[3][0][0, 0], g[3][1][0, 0]
        with lock:
            dk[b, h, :kend] += g[1][0, 0]
            dv[b, h, :kend] += g[2][0, 0]

    _run(one, len(tasks), n_workers)
    return dq, dk, dv, o, lse


def _run(fn, n, n_workers):
    nw = min(n, n_workers or workers())
    try:
        from threadpoolctl import threadpool_limits
    except ImportError:  # BLAS threads then follow the environment
        threadpool_limits = None
    if threadpool_limits is None:
        with ThreadPoolExecutor(nw) as ex:
            list(ex.map(fn, range(n)))
        return
    with threadpool_limits(limits=1 if nw > 1 else None):
        with ThreadPoolExecutor(nw) as ex:
            list(ex.map(fn, range(n)))
