"""attention(): the differentiable wrapper over fa_fwd / fa_bwd (and their
block-sparse forms).  Its gradients must be exactly what fa_bwd returns for
the same inputs (the parity tests compare fa_bwd with the oracle)."""
import pytest
import torch

from exact_io_aware_33_amd import attention, fa_bwd, fa_bwd_blocksparse, fa_fwd, fa_fwd_blocksparse

pytestmark = pytest.mark.gpu


def _inputs(B, H, N, d, dtype, seed):
    g = torch.Generator().manual_seed(seed)
    return [torch.randn(B, H, N, d, generator=g).to(dtype).cuda() for _ in range(4)]


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16])
def test_autograd_matches_fa_bwd(causal, dtype):
    q, k, v, do = _inputs(2, 3, 300, 64, dtype, seed=1)
    qa, ka, va = (t.clone().requires_grad_() for t in (q, k, v))
    o = attention(qa, ka, va, causal=causal)
    o.backward(do)
    o_ref, lse = fa_fwd(q, k, v, causal=causal)
    dq, dk, dv = fa_bwd(q, k, v, o_ref, lse, do, causal=causal)
    torch.cuda.synchronize()
    assert torch.equal(o.detach(), o_ref)
    for a, b in zip((qa.grad, ka.grad, va.grad), (dq, dk, dv)):
        assert torch.equal(a, b)


def test_autograd_dropout_and_block_mask_and_layout():
    """Dropout with a drawn seed (the backward regenerates the forward's
    mask), a block mask, and an upstream gradient in another layout."""
    q, k, v, do = _inputs(1, 2, 512, 64, torch.bfloat16, seed=2)
    bm = (torch.rand(2, 4, 4, generator=torch.Generator().manual_seed(3)) < 0.5).to(torch.uint8)
    bm[:, torch.arange(4), torch.arange(4)] = 1
    bm = bm.cuda()
    qa, ka, va = (t.clone().requires_grad_() for t in (q, k, v))
    torch.manual_seed(11)
    o = attention(qa, ka, va, causal=True, block_mask=bm, dropout_p=0.2)
    torch.manual_seed(11)
    seed = int(torch.randint(0, 2 ** 62, (1,)).item())
    o.backward(do.transpose(2, 3).contiguous().transpose(2, 3))   # same values, other strides
    dr = dict(dropout_p=0.2, dropout_seed=seed, dropout_offset=0)
    o_ref, lse = fa_fwd_blocksparse(q, k, v, bm, causal=True, **dr)
    dq, dk, dv = fa_bwd_blocksparse(q, k, v, o_ref, lse, do, bm, causal=True, **dr)
    torch.cuda.synchronize()
    assert torch.equal(o.detach(), o_ref)
    for a, b in zip((qa.grad, ka.grad, va.grad), (dq, dk, dv)):
        assert torch.equal(a, b)
