"""fp64 reference for exact scaled-dot-product attention (test infrastructure).

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py``; never by the product path.

What is computed, and where the pages define it
-----------------------------------------------
* FlashAttention summary page (xyznot.com, paper 2205.14135), section
  "Problem and motivation": S = Q K^T, P = softmax(S), O = P V.  The method is
  exact, so the oracle is that definition written out: every score row is
  formed in full, its maximum and exponential sum are taken in a first pass,
  and P and O in a second pass.
* The same page, section "Key ideas" (recomputation bullet): the forward pass
  keeps the softmax statistics (l, m) for the backward pass.  We keep them as
  the natural log-sum-exp of the scaled, masked score row, LSE = m + ln(l);
  P = exp(S - LSE) recovers the probabilities from it.
* Masking is named in the same section's kernel-fusion bullet; the
  block-sparse section of that page defines the block mask M over row and
  column blocks.  The pages leave the details open; this oracle takes: the
  scale applied before masking, causal j <= i, key padding j < len_b, and
  element (i, j) governed by block (i // mb, j // mb).
  With N_q queries and N_k keys (N_q != N_k: cross-attention, decoding) the
  causal rule is aligned at the bottom right, j <= i + (N_k - N_q): the
  queries are the last N_q positions of the key sequence (the pages define
  causal masking only by name).
* The gradients are not printed on the pages; they are the analytic
  derivatives of the definition above for the loss <dO, O>:
      dV = P^T dO,  dP = dO V^T,  D_i = sum_j P_ij dP_ij,
      dS = P * (dP - D 1^T),  dQ = scale dS K,  dK = scale dS^T Q.

* Dropout (named in the kernel-fusion bullet of the same section) is
  optional: ``dropout=(p, seed, offset)`` applies the keep mask Z of
  :mod:`oracle.dropout` (kept entries scaled by 1 / (1 - p)) to P before the
  product with V:  O = (P * Z) V, LSE unchanged (statistics of the undropped
  softmax).  Gradients of <dO, O> with the mask held fixed:
      dV = (P * Z)^T dO,  dP = dO V^T,  D_i = sum_c dO_ic O_ic,
      dS = P * (Z * dP - D 1^T),  dQ = scale dS K,  dK = scale dS^T Q.

Conventions: arrays are float64 numpy arrays shaped [B, H, N, d]; ``scale`` is
applied as a float64 number (callers pass the float32 value the GPU uses); a
query row with no visible key has O = 0, LSE = -inf and zero gradients.
Rows are processed in chunks of ``chunk`` queries only to bound memory; each
chunk still forms its full score rows.
"""
from __future__ import annotations

import numpy as np

from .dropout import keep_mask, keep_scale

__all__ = ["allowed_mask", "forward", "forward_rows", "backward", "probabilities",
           "gradients_sampled"]


def _block_mask_for_head(block_mask, h):
    if block_mask is None:
        return None
    bm = np.asarray(block_mask)
    if bm.ndim == 3:
        return bm[h]
    return bm


def allowed_mask(rows, N, *, causal=False, key_len=None, block_mask=None, mb=128,
                 n_queries=None, cols=None):
    """Boolean [len(rows), N] (or [len(rows), len(cols)]): True where query
    ``rows[r]`` may see key j < N (j = cols[c] when ``cols`` is given).

    The allowed set is the AND of every active mask: causal
    (j <= i + N - n_queries; n_queries defaults to N, giving j <= i), key
    padding (j < key_len) and block (M[i//mb, j//mb] != 0).
    """
    rows = np.asarray(rows, dtype=np.int64)
    cols = np.arange(N, dtype=np.int64) if cols is None else np.asarray(cols, dtype=np.int64)
    a = np.ones((rows.size, cols.size), dtype=bool)
    if causal:
        shift = 0 if n_queries is None else N - int(n_queries)
        a &= cols[None, :] <= rows[:, None] + shift
    if key_len is not None:
        a &= cols[None, :] < int(key_len)
    if block_mask is not None:
        bm = np.asarray(block_mask) != 0
        a &= bm[rows[:, None] // mb, cols[None, :] // mb]
    return a


def _row_softmax_stats(s):
    """Two-pass statistics of masked score rows (-inf marks a masked entry).

    Returns (m, l, valid): row max, sum of exp(s - m), and whether the row has
    any visible key.
    """
    valid = np.isfinite(s).any(axis=1)
    m = np.where(valid, np.max(np.where(np.isfinite(s), s, -np.inf), axis=1), 0.0)
    e = np.exp(s - m[:, None])          # exp(-inf) = 0 for masked entries
    l = e.sum(axis=1)
    return m, l, valid, e


def _z(bh, rows, cols, dropout):
    """Dropout factor Z (0 or 1/(1-p)) for the given rows / columns, or None."""
    if dropout is None:
        return None
    p, seed, offset = dropout
    return keep_mask(bh, rows, cols, p, seed, offset) * keep_scale(p)


def forward_rows(q, k, v, scale, rows, *, causal=False, key_len=None,
                 block_mask=None, mb=128, dropout=None, bh=0):
    """O and LSE of one (batch, head) for the query indices ``rows`` only.

    q: [N_q, d] (only ``rows`` are read), k, v: [N_k, d].  Returns
    (o [R, d], lse [R]).  Used for sampled parity at sizes where every row is
    too many.
    """
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    N = k.shape[0]
    rows = np.asarray(rows, dtype=np.int64)
    s = float(scale) * (q[rows] @ k.T)
    a = allowed_mask(rows, N, causal=causal, key_len=key_len,
                     block_mask=block_mask, mb=mb, n_queries=q.shape[0])
    s = np.where(a, s, -np.inf)
    m, l, valid, e = _row_softmax_stats(s)
    p = np.where(valid[:, None], e / np.where(valid, l, 1.0)[:, None], 0.0)
    z = _z(bh, rows, np.arange(N), dropout)
    o = (p if z is None else p * z) @ v
    lse = np.where(valid, m + np.log(np.where(valid, l, 1.0)), -np.inf)
    return o, lse


def _lens(key_lens, B):
    if key_lens is None:
        return [None] * B
    kl = np.asarray(key_lens).reshape(-1)
    assert kl.size == B
    return [int(x) for x in kl]


def forward(q, k, v, scale, *, causal=False, key_lens=None, block_mask=None,
            mb=128, chunk=1024, dropout=None, bh_offset=0):
    """Exact attention forward.  Returns (O [B,H,N,dv], LSE [B,H,N]) in fp64.

    N is the number of query rows; K and V may hold a different number of
    rows (keys), and V a different width dv.  ``bh_offset`` is added to the
    (batch, head) index b*H + h that the dropout keep mask is drawn for, so
    that one head of a larger problem can be evaluated on its own (it has no
    other effect).
    """
    B, H, N, _ = q.shape
    o = np.zeros((B, H, N, v.shape[-1]), np.float64)
    lse = np.zeros((B, H, N), np.float64)
    lens = _lens(key_lens, B)
    for b in range(B):
        for h in range(H):
            bm = _block_mask_for_head(block_mask, h)
            for r0 in range(0, N, chunk):
                rows = np.arange(r0, min(N, r0 + chunk))
                ob, lb = forward_rows(q[b, h], k[b, h], v[b, h], scale, rows,
                                      causal=causal, key_len=lens[b],
                                      block_mask=bm, mb=mb, dropout=dropout,
                                      bh=bh_offset + b * H + h)
                o[b, h, rows] = ob
                lse[b, h, rows] = lb
    return o, lse


def probabilities(q, k, scale, *, causal=False, key_len=None, block_mask=None, mb=128):
    """P = softmax of the scaled, masked score matrix of one (batch, head): [N_q, N_k].

    A row with no visible key is all zeros.  Only for small N (tests).
    """
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    N = k.shape[0]
    rows = np.arange(q.shape[0])
    s = float(scale) * (q @ k.T)
    s = np.where(allowed_mask(rows, N, causal=causal, key_len=key_len,
                              block_mask=block_mask, mb=mb, n_queries=q.shape[0]), s, -np.inf)
    m, l, valid, e = _row_softmax_stats(s)
    return np.where(valid[:, None], e / np.where(valid, l, 1.0)[:, None], 0.0)


def backward(q, k, v, do, scale, *, causal=False, key_lens=None, block_mask=None,
             mb=128, chunk=1024, return_aux=False, dropout=None, bh_offset=0):
    """Analytic gradients of <dO, O> w.r.t. Q, K, V (fp64).

    Returns (dq, dk, dv); with ``return_aux`` also (o, lse, D_from_p, D_from_o),
    where D_from_p = rowsum(P * dP) and D_from_o = rowsum(dO * O) -- equal in
    exact arithmetic; the GPU computes the latter.  ``bh_offset``: as for
    :func:`forward` (dropout head index only).
    """
    B, H, N, d = q.shape
    Nk = k.shape[2]
    dq = np.zeros_like(q, dtype=np.float64)
    dk = np.zeros_like(k, dtype=np.float64)
    dv = np.zeros_like(v, dtype=np.float64)
    o = np.zeros((B, H, N, v.shape[-1]), np.float64)
    lse = np.zeros((B, H, N), np.float64)
    D_p = np.zeros((B, H, N), np.float64)
    D_o = np.zeros((B, H, N), np.float64)
    lens = _lens(key_lens, B)
    for b in range(B):
        for h in range(H):
            bm = _block_mask_for_head(block_mask, h)
            qb, kb, vb, dob = (np.asarray(x[b, h], np.float64) for x in (q, k, v, do))
            for r0 in range(0, N, chunk):
                rows = np.arange(r0, min(N, r0 + chunk))
                s = float(scale) * (qb[rows] @ kb.T)
                a = allowed_mask(rows, Nk, causal=causal, key_len=lens[b],
                                 block_mask=bm, mb=mb, n_queries=N)
                s = np.where(a, s, -np.inf)
                m, l, valid, e = _row_softmax_stats(s)
                p = np.where(valid[:, None], e / np.where(valid, l, 1.0)[:, None], 0.0)
                z = _z(bh_offset + b * H + h, rows, np.arange(Nk), dropout)
                pz = p if z is None else p * z
                oc = pz @ vb
                dpc = dob[rows] @ vb.T
                zdp = dpc if z is None else z * dpc
                Dp = np.sum(p * zdp, axis=1)
                ds = p * (zdp - Dp[:, None])
                dq[b, h, rows] = float(scale) * (ds @ kb)
                dk[b, h] += float(scale) * (ds.T @ qb[rows])
                dv[b, h] += pz.T @ dob[rows]
                o[b, h, rows] = oc
                lse[b, h, rows] = np.where(valid, m + np.log(np.where(valid, l, 1.0)), -np.inf)
                D_p[b, h, rows] = Dp
                D_o[b, h, rows] = np.sum(dob[rows] * oc, axis=1)
    if return_aux:
        return dq, dk, dv, (o, lse, D_p, D_o)
    return dq, dk, dv


def gradients_sampled(q, k, v, do, scale, rows, cols, *, causal=False, key_len=None,
                      block_mask=None, mb=128, chunk=1024, dropout=None, bh=0):
    """Exact gradients of one (batch, head) at selected rows / columns only.

    Same definition as :func:`backward`; used at sizes where the full N x d
    gradients take too long in fp64.  Returns (o_rows [R,d], lse_rows [R],
    dq_rows [R,d], dk_cols [C,d], dv_cols [C,d]).

    dQ_i needs only row i of P and dP.  dK_j and dV_j need column j of P and
    dS for every query row i that sees key j, hence those rows' LSE and
    D_i = rowsum(P * dP): a first pass over the selected rows and every row
    that sees a selected column (in chunks) computes them, a second forms the
    selected columns from those rows (the others have P_ij = 0 there).
    """
    q, k, v, do = (np.asarray(x, np.float64) for x in (q, k, v, do))
    Nq, N = q.shape[0], k.shape[0]
    mk = dict(causal=causal, key_len=key_len, block_mask=block_mask, mb=mb, n_queries=Nq)
    rows = np.asarray(rows, dtype=np.int64)
    cols = np.asarray(cols, dtype=np.int64)
    sees = allowed_mask(np.arange(Nq), N, cols=cols, **mk).any(axis=1)
    sees[rows] = True
    need = np.nonzero(sees)[0]
    lse_all = np.full(Nq, np.nan)
    D_all = np.full(Nq, np.nan)
    for c0 in range(0, need.size, chunk):
        rr = need[c0:c0 + chunk]
        s = float(scale) * (q[rr] @ k.T)
        a = allowed_mask(rr, N, **mk)
        s = np.where(a, s, -np.inf)
        m, l, valid, e = _row_softmax_stats(s)
        p = np.where(valid[:, None], e / np.where(valid, l, 1.0)[:, None], 0.0)
        dp = do[rr] @ v.T
        z = _z(bh, rr, np.arange(N), dropout)
        if z is not None:
            dp = z * dp
        lse_all[rr] = np.where(valid, m + np.log(np.where(valid, l, 1.0)), -np.inf)
        D_all[rr] = np.sum(p * dp, axis=1)
    # selected rows: O, LSE, dQ
    s = float(scale) * (q[rows] @ k.T)
    a = allowed_mask(rows, N, **mk)
    s = np.where(a, s, -np.inf)
    lr = lse_all[rows]
    fin = np.isfinite(lr)
    p = np.where(fin[:, None], np.exp(s - np.where(fin, lr, 0.0)[:, None]), 0.0)
    z = _z(bh, rows, np.arange(N), dropout)
    o_rows = (p if z is None else p * z) @ v
    dpr = do[rows] @ v.T
    ds = p * ((dpr if z is None else z * dpr) - D_all[rows][:, None])
    dq_rows = float(scale) * (ds @ k)
    # selected columns: dK, dV
    dk_cols = np.zeros((cols.size, q.shape[1]))
    dv_cols = np.zeros((cols.size, v.shape[1]))
    for c0 in range(0, need.size, chunk):
        rr = need[c0:c0 + chunk]
        s = float(scale) * (q[rr] @ k[cols].T)
        a = allowed_mask(rr, N, cols=cols, **mk)
        s = np.where(a, s, -np.inf)
        lc = lse_all[rr]
        fin = np.isfinite(lc)
        p = np.where(fin[:, None], np.exp(s - np.where(fin, lc, 0.0)[:, None]), 0.0)
        z = _z(bh, rr, cols, dropout)
        dpc = do[rr] @ v[cols].T
        ds = p * ((dpc if z is None else z * dpc) - D_all[rr][:, None])
        dk_cols += float(scale) * (ds.T @ q[rr])
        dv_cols += (p if z is None else p * z).T @ do[rr]
    return o_rows, lse_all[rows], dq_rows, dk_cols, dv_cols
