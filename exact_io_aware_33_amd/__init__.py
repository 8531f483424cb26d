"""Exact IO-aware attention for AMD Instinct MI355X (gfx950).

Thin Python binding over the C ABI of ``libfa.so`` (include/fa.h).  Each
function below has the name of the C entry point it calls and only marshals
arguments: torch supplies device memory and the current HIP stream, every step
of the computation runs in the library's HIP kernels.  There is no fallback:
if the library is missing, the call raises.

Tensors are ``[B, H, N, d]`` views with unit stride along d: Q, O, dO and dQ
([B, H, N_q, d]) share one set of strides, K, V, dK and dV ([B, H, N_k, d])
another (N_q != N_k: cross-attention or decoding, causal aligned bottom-right).

Dropout: every entry point takes ``dropout_p`` (0 = none), ``dropout_seed``
(64-bit Philox key) and ``dropout_offset`` (32-bit counter word); the backward
call must repeat the forward's values (the keep mask is regenerated, never
stored).
"""
from __future__ import annotations

import ctypes
import math

import torch

from . import _lib
from ._lib import FaError, FaProblem

__all__ = ["fa_fwd", "fa_fwd_blocksparse", "fa_fwd_splitkv", "fa_fwd_splitkv_num_splits",
           "fa_fwd_splitkv_workspace_bytes", "fa_bwd", "fa_bwd_blocksparse", "fa_bwd_ex",
           "fa_bwd_noalloc", "fa_merge_partials",
           "fa_bwd_workspace_bytes", "fa_softmax_rows", "fa_layernorm_rows", "fa_group_norm",
           "attention", "FaError", "library_path", "load_library",
           "FA_BWD_PRE", "FA_BWD_MAIN", "FA_BWD_DQ", "FA_BWD_ALL"]

FA_BWD_PRE, FA_BWD_MAIN, FA_BWD_DQ, FA_BWD_ALL = (_lib.FA_BWD_PRE, _lib.FA_BWD_MAIN,
                                                  _lib.FA_BWD_DQ, _lib.FA_BWD_ALL)

_DTYPES = {torch.float32: _lib.FA_DTYPE_F32, torch.float16: _lib.FA_DTYPE_F16,
           torch.bfloat16: _lib.FA_DTYPE_BF16}


def load_library():
    """Load libfa.so now (raises if it was not built)."""
    return _lib.load()


def library_path() -> str:
    return _lib.LIB_PATH


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(t):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _problem(q, k, scale, causal, key_lens, dropout_p=0.0, dropout_seed=0, dropout_offset=0,
             query_tile=0):
    if q.dim() != 4 or k.dim() != 4:
        raise ValueError("expected [B, H, N, d] tensors")
    if q.dtype not in _DTYPES:
        raise ValueError(f"unsupported dtype {q.dtype}")
    B, H, N, d = q.shape
    if k.shape[0] != B or k.shape[1] != H or k.shape[3] != d:
        raise ValueError("K/V must be [B, H, N_k, d] with the B, H, d of Q")
    if k.dtype != q.dtype or k.device != q.device:
        raise ValueError("Q and K/V must share dtype and device")
    if q.stride(3) != 1 or k.stride(3) != 1:
        raise ValueError("the head dimension must be contiguous (stride 1)")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if key_lens is not None:
        if key_lens.dtype != torch.int32 or key_lens.device != q.device or key_lens.numel() != B:
            raise ValueError("key_lens must be an int32 [B] tensor on the device of q")
        key_lens = key_lens.contiguous()
    if not 0 <= int(dropout_seed) < 2 ** 64 or not 0 <= int(dropout_offset) < 2 ** 32:
        raise ValueError("dropout_seed must fit 64 bits and dropout_offset 32 bits (unsigned)")
    p = FaProblem(batch=B, heads=H, seqlen=N, head_dim=d,
                  stride_b=q.stride(0), stride_h=q.stride(1), stride_n=q.stride(2),
                  scale=float(scale), causal=1 if causal else 0, dtype=_DTYPES[q.dtype],
                  key_lens=None if key_lens is None else key_lens.data_ptr(),
                  dropout_p=float(dropout_p), dropout_offset=int(dropout_offset),
                  dropout_seed=int(dropout_seed), seqlen_k=k.shape[2],
                  fwd_query_tile=int(query_tile),
                  k_stride_b=k.stride(0), k_stride_h=k.stride(1), k_stride_n=k.stride(2))
    return p, key_lens


def _same_layout(ref, *others):
    for t in others:
        if t.shape != ref.shape or t.stride() != ref.stride() or t.dtype != ref.dtype \
                or t.device != ref.device:
            raise ValueError("Q, O, dO, dQ (and K, V, dK, dV) must share shape, strides, dtype "
                             "and device")


def _stats(t, shape, like, name, required=False):
    """A float32 per-row array (LSE, mean, rstd) of the given shape, new when
    ``t`` is None.  The library reads or writes prod(shape) contiguous floats
    through the bare pointer, so a caller's tensor must hold exactly that, on
    the device of ``like``."""
    if t is None:
        if required:
            raise ValueError(f"{name} is required")
        return torch.empty(shape, dtype=torch.float32, device=like.device)
    n = math.prod(shape)
    if t.dtype != torch.float32 or not t.is_contiguous() or t.numel() != n or t.device != like.device:
        raise ValueError(f"{name} must be a contiguous float32 tensor of {n} elements on {like.device}")
    return t


def _workspace(ws, need, like):
    if ws is None:
        return torch.empty(max(need, 16), dtype=torch.uint8, device=like.device)
    if ws.device != like.device or not ws.is_contiguous():
        raise ValueError(f"workspace must be a contiguous tensor on {like.device}")
    return ws


def _empty_like_layout(q):
    return torch.empty_strided(q.shape, q.stride(), dtype=q.dtype, device=q.device)


def fa_fwd(q, k, v, *, scale=None, causal=False, key_lens=None, out=None, lse=None,
           dropout_p=0.0, dropout_seed=0, dropout_offset=0, query_tile=0):
    """Exact attention forward; returns (O, LSE).  ``query_tile``: queries per
    workgroup (0 = the library's choice, or 64 / 128 / 256).  Calls fa_fwd."""
    _same_layout(k, v)
    p, kl = _problem(q, k, scale, causal, key_lens, dropout_p, dropout_seed, dropout_offset,
                     query_tile)
    o = _empty_like_layout(q) if out is None else out
    lse = _stats(lse, tuple(q.shape[:3]), q, "lse")
    _same_layout(q, o)
    lib = _lib.load()
    _lib.check(lib.fa_fwd(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _stream(q)))
    return o, lse


def fa_fwd_blocksparse(q, k, v, block_mask, *, mask_block=128, scale=None, causal=False,
                       key_lens=None, out=None, lse=None, dropout_p=0.0, dropout_seed=0,
                       dropout_offset=0, query_tile=0):
    """Block-sparse forward; ``block_mask`` is uint8 [N/mb, N/mb] (shared by all heads)
    or [H, N/mb, N/mb].  Returns (O, LSE).  Calls fa_fwd_blocksparse."""
    _same_layout(k, v)
    p, kl = _problem(q, k, scale, causal, key_lens, dropout_p, dropout_seed, dropout_offset,
                     query_tile)
    bm, hstride = _mask(block_mask, q, k, mask_block)
    o = _empty_like_layout(q) if out is None else out
    lse = _stats(lse, tuple(q.shape[:3]), q, "lse")
    _same_layout(q, o)
    lib = _lib.load()
    _lib.check(lib.fa_fwd_blocksparse(ctypes.byref(p), _ptr(bm), int(mask_block), int(hstride),
                                      _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _stream(q)))
    return o, lse


def _mask(block_mask, q, k, mask_block):
    if block_mask.dtype != torch.uint8 or block_mask.device != q.device:
        raise ValueError("block_mask must be a uint8 tensor on the device of q")
    bm = block_mask.contiguous()
    mb = int(mask_block)
    # the library checks mask_block against N_q and N_k (and rejects a block
    # that does not divide them); the mask's extent, which it reads through a
    # bare pointer, is checked here
    nq, nk = q.shape[2], k.shape[2]
    want = (nq // mb, nk // mb) if mb > 0 and nq % mb == 0 and nk % mb == 0 else None
    if bm.dim() == 2 and (want is None or tuple(bm.shape) == want):
        return bm, 0
    if bm.dim() == 3 and bm.shape[0] == q.shape[1] and (want is None or tuple(bm.shape[1:]) == want):
        return bm, bm.stride(0)
    raise ValueError(f"block_mask must be [N_q/mb, N_k/mb] = {want} or [H, N_q/mb, N_k/mb]")


def fa_merge_partials(o_parts, lse_parts, *, out=None, lse=None):
    """Merge partial results (O_s, LSE_s) computed over disjoint key sets into
    (O, LSE): LSE = log sum_s exp(LSE_s), O = sum_s exp(LSE_s - LSE) O_s.
    ``o_parts``: sequence of S [B, H, N_q, d] tensors sharing one layout;
    ``lse_parts``: S float32 [B, H, N_q] tensors.  ``out`` / ``lse`` may be
    one of the parts (in-place).  Calls fa_merge_partials."""
    o_parts, lse_parts = list(o_parts), list(lse_parts)
    S = len(o_parts)
    if S < 1 or S != len(lse_parts) or S > _lib.FA_MERGE_MAX_PARTS:
        raise ValueError(f"need 1..{_lib.FA_MERGE_MAX_PARTS} O parts and as many LSE parts")
    ref = o_parts[0]
    _same_layout(ref, *o_parts[1:])
    shape = tuple(ref.shape[:3])
    for t in lse_parts:
        _stats(t, shape, ref, "each LSE part", required=True)
    o = _empty_like_layout(ref) if out is None else out
    _same_layout(ref, o)
    lse = _stats(lse, shape, ref, "lse")
    p, _ = _problem(ref, ref, 1.0, False, None)
    optr = (ctypes.c_void_p * S)(*[t.data_ptr() for t in o_parts])
    lptr = (ctypes.c_void_p * S)(*[t.data_ptr() for t in lse_parts])
    lib = _lib.load()
    _lib.check(lib.fa_merge_partials(ctypes.byref(p), S, optr, lptr, _ptr(o), _ptr(lse), _stream(ref)))
    return o, lse


def fa_fwd_splitkv_num_splits(q, k, *, scale=None, causal=False, key_lens=None) -> int:
    """The split count the library picks for this problem.  Calls fa_fwd_splitkv_num_splits."""
    p, _ = _problem(q, k, scale, causal, key_lens)
    lib = _lib.load()
    n = lib.fa_fwd_splitkv_num_splits(ctypes.byref(p))
    if n <= 0:
        raise FaError(_lib.FA_ERR_INVALID, lib.fa_last_error().decode())
    return int(n)


def fa_fwd_splitkv_workspace_bytes(q, k, num_splits=0, *, scale=None, causal=False,
                                   key_lens=None) -> int:
    """Workspace bytes fa_fwd_splitkv needs.  Calls fa_fwd_splitkv_workspace_bytes."""
    p, _ = _problem(q, k, scale, causal, key_lens)
    lib = _lib.load()
    n = lib.fa_fwd_splitkv_workspace_bytes(ctypes.byref(p), int(num_splits))
    if n == 0:
        raise FaError(_lib.FA_ERR_INVALID, lib.fa_last_error().decode())
    return int(n)


def fa_fwd_splitkv(q, k, v, *, num_splits=0, block_mask=None, mask_block=128, scale=None,
                   causal=False, key_lens=None, workspace=None, out=None, lse=None):
    """Split-KV forward (decoding shapes); returns (O, LSE).  num_splits <= 0 lets the
    library choose; block_mask None selects the dense path.  Calls fa_fwd_splitkv."""
    _same_layout(k, v)
    p, kl = _problem(q, k, scale, causal, key_lens)
    bm, hstride = (None, 0) if block_mask is None else _mask(block_mask, q, k, mask_block)
    o = _empty_like_layout(q) if out is None else out
    lse = _stats(lse, tuple(q.shape[:3]), q, "lse")
    _same_layout(q, o)
    lib = _lib.load()
    workspace = _workspace(workspace, lib.fa_fwd_splitkv_workspace_bytes(ctypes.byref(p), int(num_splits)), q)
    _lib.check(lib.fa_fwd_splitkv(ctypes.byref(p), _ptr(bm), int(mask_block), int(hstride),
                                  int(num_splits), _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse),
                                  _ptr(workspace), workspace.numel() * workspace.element_size(),
                                  _stream(q)))
    return o, lse


def fa_bwd_workspace_bytes(q, k=None, *, scale=None, causal=False, key_lens=None) -> int:
    """Workspace bytes fa_bwd needs for this problem (K defaults to the
    shape of Q).  Calls fa_bwd_workspace_bytes."""
    p, _ = _problem(q, q if k is None else k, scale, causal, key_lens)
    lib = _lib.load()
    n = lib.fa_bwd_workspace_bytes(ctypes.byref(p))
    if n == 0:
        raise FaError(_lib.FA_ERR_INVALID, lib.fa_last_error().decode())
    return int(n)


def _bwd_outputs(q, k, workspace, p, grads):
    lib = _lib.load()
    workspace = _workspace(workspace, lib.fa_bwd_workspace_bytes(ctypes.byref(p)), q)
    outs = []
    for like, g in zip((q, k, k), grads):
        if g is None:
            g = _empty_like_layout(like)
        else:
            _same_layout(like, g)
        outs.append(g)
    return outs[0], outs[1], outs[2], workspace


def fa_bwd(q, k, v, o, lse, do, *, scale=None, causal=False, key_lens=None, workspace=None,
           dq=None, dk=None, dv=None, dropout_p=0.0, dropout_seed=0, dropout_offset=0):
    """Gradients (dQ, dK, dV) of <dO, O>.  Calls fa_bwd."""
    _same_layout(q, o, do)
    _same_layout(k, v)
    p, kl = _problem(q, k, scale, causal, key_lens, dropout_p, dropout_seed, dropout_offset)
    _stats(lse, tuple(q.shape[:3]), q, "lse", required=True)
    dq, dk, dv, ws = _bwd_outputs(q, k, workspace, p, (dq, dk, dv))
    lib = _lib.load()
    _lib.check(lib.fa_bwd(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(do),
                          _ptr(dq), _ptr(dk), _ptr(dv), _ptr(ws), ws.numel() * ws.element_size(),
                          _stream(q)))
    return dq, dk, dv


def fa_bwd_blocksparse(q, k, v, o, lse, do, block_mask, *, mask_block=128, scale=None,
                       causal=False, key_lens=None, workspace=None, dq=None, dk=None, dv=None,
                       dropout_p=0.0, dropout_seed=0, dropout_offset=0):
    """Block-sparse gradients (dQ, dK, dV).  Calls fa_bwd_blocksparse."""
    _same_layout(q, o, do)
    _same_layout(k, v)
    p, kl = _problem(q, k, scale, causal, key_lens, dropout_p, dropout_seed, dropout_offset)
    _stats(lse, tuple(q.shape[:3]), q, "lse", required=True)
    bm, hstride = _mask(block_mask, q, k, mask_block)
    dq, dk, dv, ws = _bwd_outputs(q, k, workspace, p, (dq, dk, dv))
    lib = _lib.load()
    _lib.check(lib.fa_bwd_blocksparse(ctypes.byref(p), _ptr(bm), int(mask_block), int(hstride),
                                      _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(do),
                                      _ptr(dq), _ptr(dk), _ptr(dv), _ptr(ws),
                                      ws.numel() * ws.element_size(), _stream(q)))
    return dq, dk, dv


def fa_bwd_ex(q, k, v, o, lse, do, stages, *, block_mask=None, mask_block=128, scale=None,
              causal=False, key_lens=None, workspace, dq, dk, dv, dropout_p=0.0, dropout_seed=0,
              dropout_offset=0):
    """One or more stages of the backward launch sequence (FA_BWD_PRE, _MAIN,
    _DQ bits), writing into caller-provided gradients and workspace.  Calls
    fa_bwd_ex; block_mask None selects the dense path."""
    _same_layout(q, o, do, dq)
    _same_layout(k, v, dk, dv)
    p, kl = _problem(q, k, scale, causal, key_lens, dropout_p, dropout_seed, dropout_offset)
    _stats(lse, tuple(q.shape[:3]), q, "lse", required=True)
    bm, hstride = (None, 0) if block_mask is None else _mask(block_mask, q, k, mask_block)
    lib = _lib.load()
    workspace = _workspace(workspace, 0, q)
    _lib.check(lib.fa_bwd_ex(ctypes.byref(p), _ptr(bm), int(mask_block), int(hstride),
                             _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(do),
                             _ptr(dq), _ptr(dk), _ptr(dv), _ptr(workspace),
                             workspace.numel() * workspace.element_size(), int(stages), _stream(q)))


def fa_bwd_noalloc(q, k, v, o, lse, do, *, block_mask=None, mask_block=128, scale=None,
                   causal=False, key_lens=None, dq=None, dk=None, dv=None, dropout_p=0.0,
                   dropout_seed=0, dropout_offset=0):
    """Gradients (dQ, dK, dV) with the library's static workspace instead of a
    caller-supplied one (the entry point for callers that cannot allocate; at
    most FA_BWD_NOALLOC_MAX_WORKSPACE_BYTES of workspace).  Calls
    fa_bwd_noalloc on the device of q; block_mask None selects the dense path.
    Gradient tensors the caller omits are allocated here, by torch, before
    the call."""
    _same_layout(q, o, do)
    _same_layout(k, v)
    p, kl = _problem(q, k, scale, causal, key_lens, dropout_p, dropout_seed, dropout_offset)
    _stats(lse, tuple(q.shape[:3]), q, "lse", required=True)
    bm, hstride = (None, 0) if block_mask is None else _mask(block_mask, q, k, mask_block)
    outs = []
    for like, g in zip((q, k, k), (dq, dk, dv)):
        if g is None:
            g = _empty_like_layout(like)
        else:
            _same_layout(like, g)
        outs.append(g)
    lib = _lib.load()
    with torch.cuda.device(q.device):
        _lib.check(lib.fa_bwd_noalloc(ctypes.byref(p), _ptr(bm), int(mask_block), int(hstride),
                                      _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(do),
                                      _ptr(outs[0]), _ptr(outs[1]), _ptr(outs[2]), _stream(q)))
    return outs[0], outs[1], outs[2]


def _rows_view(x):
    """A 2-D [rows, cols] tensor with unit column stride: (rows, cols, ld)."""
    if x.dim() != 2 or x.stride(1) != 1:
        raise ValueError("expected a 2-D tensor with contiguous rows")
    if x.dtype not in _DTYPES:
        raise ValueError(f"unsupported dtype {x.dtype}")
    return x.shape[0], x.shape[1], x.stride(0)


def fa_softmax_rows(x, *, out=None, lse=None):
    """Row softmax of a 2-D tensor; returns (y, lse [rows] fp32).  Calls fa_softmax_rows."""
    rows, cols, ld = _rows_view(x)
    y = torch.empty_like(x) if out is None else out
    _, _, ldy = _rows_view(y)
    if y.shape != x.shape or y.dtype != x.dtype:
        raise ValueError("out must match x in shape and dtype")
    lse = _stats(lse, (rows,), x, "lse")
    lib = _lib.load()
    _lib.check(lib.fa_softmax_rows(_DTYPES[x.dtype], rows, cols, _ptr(x), ld, _ptr(y), ldy, _ptr(lse),
                                   _stream(x)))
    return y, lse


def fa_layernorm_rows(x, gamma=None, beta=None, *, eps=1e-5, groups=1, inner=1, out=None,
                      mean=None, rstd=None):
    """LayerNorm (groups = inner = 1) or GroupNorm rows of a 2-D tensor; returns
    (y, mean, rstd).  Calls fa_layernorm_rows."""
    rows, cols, ld = _rows_view(x)
    y = torch.empty_like(x) if out is None else out
    _, _, ldy = _rows_view(y)
    if y.shape != x.shape or y.dtype != x.dtype:
        raise ValueError("out must match x in shape and dtype")
    nch = groups * (cols // inner)
    for t in (gamma, beta):
        if t is not None and (t.dtype != x.dtype or t.numel() != nch or not t.is_contiguous()):
            raise ValueError(f"gamma / beta must be contiguous {x.dtype} of {nch} channels")
    mean = _stats(mean, (rows,), x, "mean")
    rstd = _stats(rstd, (rows,), x, "rstd")
    lib = _lib.load()
    _lib.check(lib.fa_layernorm_rows(_DTYPES[x.dtype], rows, cols, _ptr(x), ld, _ptr(gamma), _ptr(beta),
                                     float(eps), int(groups), int(inner), _ptr(y), ldy, _ptr(mean),
                                     _ptr(rstd), _stream(x)))
    return y, mean, rstd


def fa_group_norm(x, groups, gamma=None, beta=None, *, eps=1e-5):
    """GroupNorm of an [N, C, *] tensor through fa_layernorm_rows (rows = N * groups)."""
    N, C = x.shape[0], x.shape[1]
    S = x[0, 0].numel()
    if C % groups:
        raise ValueError("groups must divide C")
    x2 = x.contiguous().view(N * groups, (C // groups) * S)
    y, mean, rstd = fa_layernorm_rows(x2, gamma, beta, eps=eps, groups=groups, inner=S)
    return y.view(x.shape), mean.view(N, groups), rstd.view(N, groups)


class _Attention(torch.autograd.Function):
    """fa_fwd / fa_fwd_blocksparse forward, fa_bwd / fa_bwd_blocksparse
    backward; saves Q, K, V, O and the LSE (O(N) beyond the inputs), nothing
    of size N x N."""

    @staticmethod
    def forward(ctx, q, k, v, scale, causal, key_lens, block_mask, mask_block, dropout_p, dropout_seed,
                dropout_offset):
        dr = dict(dropout_p=dropout_p, dropout_seed=dropout_seed, dropout_offset=dropout_offset)
        if block_mask is None:
            o, lse = fa_fwd(q, k, v, scale=scale, causal=causal, key_lens=key_lens, **dr)
        else:
            o, lse = fa_fwd_blocksparse(q, k, v, block_mask, mask_block=mask_block, scale=scale,
                                        causal=causal, key_lens=key_lens, **dr)
        ctx.save_for_backward(q, k, v, o, lse)
        ctx.args = (scale, causal, key_lens, block_mask, mask_block, dr)
        return o

    @staticmethod
    def backward(ctx, do):
        q, k, v, o, lse = ctx.saved_tensors
        scale, causal, key_lens, block_mask, mask_block, dr = ctx.args
        if do.stride() != o.stride() or do.dtype != o.dtype:  # dO in O's layout
            do = torch.empty_strided(o.shape, o.stride(), dtype=o.dtype, device=o.device).copy_(do)
        if block_mask is None:
            dq, dk, dv = fa_bwd(q, k, v, o, lse, do, scale=scale, causal=causal, key_lens=key_lens, **dr)
        else:
            dq, dk, dv = fa_bwd_blocksparse(q, k, v, o, lse, do, block_mask, mask_block=mask_block,
                                            scale=scale, causal=causal, key_lens=key_lens, **dr)
        return dq, dk, dv, None, None, None, None, None, None, None, None


def attention(q, k, v, *, scale=None, causal=False, key_lens=None, block_mask=None, mask_block=128,
              dropout_p=0.0, dropout_seed=None, dropout_offset=0):
    """O = softmax(scale Q K^T [+ masks]) V as a differentiable torch op:
    the forward calls fa_fwd (fa_fwd_blocksparse with a block mask), the
    backward fa_bwd (fa_bwd_blocksparse) with the saved O and LSE.  With
    dropout and no seed given, a 64-bit seed is drawn from torch's default
    CPU generator (so torch.manual_seed makes it reproducible); the backward
    regenerates the same keep mask.  Tensors as for fa_fwd; dO is copied
    into O's layout if it has another."""
    if dropout_p > 0.0 and dropout_seed is None:
        dropout_seed = int(torch.randint(0, 2 ** 62, (1,)).item())
    return _Attention.apply(q, k, v, scale, causal, key_lens, block_mask, mask_block, dropout_p,
                            dropout_seed or 0, dropout_offset)
