"""Context-parallel (ring) attention, the part one GPU can show: the per-hop
kernels at their real shape and the merge of their partial results
(fa_merge_partials), against the fp64 oracle of the whole problem.

In a ring over P devices each device keeps a shard of the queries and the
key / value shards visit it one hop at a time.  A hop is one fa_fwd (or
fa_fwd_blocksparse) call of the local queries against the visiting shard; the
device merges the hops' (O_s, LSE_s) with the merge equation of the summary
page's "Incremental softmax tracking" section.  The backward pass runs fa_bwd
per hop with the MERGED O and LSE: that hop's dK and dV are then exact for
the queries of this device, and the hops' dQ shares sum to dQ.  Here the
devices and hops run one after another on one GPU; the transfers between
devices are not modelled.
"""
import math
import sys

import numpy as np
import pytest
import torch

import oracle
from exact_io_aware_33_amd import (fa_bwd, fa_bwd_blocksparse, fa_fwd, fa_fwd_blocksparse,
                                   fa_merge_partials)
from exact_io_aware_33_amd.inputs import as_f64, make_inputs
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
    assert not np.isnan(x).any(), "NaN in GPU output"
    fin = np.isfinite(ref)
    assert np.array_equal(np.isfinite(x), fin), "finite/infinite pattern differs"
    assert np.array_equal(x[~fin], ref[~fin])
    if not fin.any():
        return 0.0
    return float(np.max(np.abs(x[fin] - ref[fin])) / np.max(np.abs(ref[fin])))


def _scale(d):
    return float(np.float32(1.0 / math.sqrt(d)))


# ------------------------------------------------------------------ merge alone
@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("d", [64, 128])
def test_merge_of_key_shards_matches_oracle(dtype, d):
    """Keys cut into shards of uneven length (one of them with every key
    padded away, so its LSE is -inf and its O, filled with NaN here, must
    weigh nothing); each shard's fa_fwd, then the merge, equals attention over
    all keys.  The merge is done in place into the first part."""
    B, H, Nq, cuts = 2, 3, 200, [0, 77, 77 + 300, 77 + 300 + 5, 77 + 300 + 5 + 130]
    Nk = cuts[-1]
    say(f"case merge {dtype} d={d} N_q={Nq} shards={np.diff(cuts).tolist()}")
    inp = make_inputs(B, H, Nq, d, dtype, seed=d + 7, with_do=False, n_keys=Nk)
    q, k, v = (inp[n].cuda() for n in ("q", "k", "v"))
    o_parts, lse_parts = [], []
    for s in range(len(cuts) - 1):
        ks, vs = k[:, :, cuts[s]:cuts[s + 1]], v[:, :, cuts[s]:cuts[s + 1]]
        o, lse = fa_fwd(q, ks, vs, scale=_scale(d))
        o_parts.append(o)
        lse_parts.append(lse)
    # an empty part: a shard whose keys are all padded away
    kl0 = torch.zeros(B, dtype=torch.int32, device="cuda")
    o_e, lse_e = fa_fwd(q, k[:, :, :64], v[:, :, :64], scale=_scale(d), key_lens=kl0)
    torch.cuda.synchronize()
    assert torch.isinf(lse_e).all().item()
    o_e.fill_(float("nan"))
    o_parts.insert(2, o_e)
    lse_parts.insert(2, lse_e)
    o, lse = fa_merge_partials(o_parts, lse_parts, out=o_parts[0], lse=lse_parts[0])
    torch.cuda.synchronize()
    ro, rlse = oracle.forward(*(as_f64(inp[n]) for n in ("q", "k", "v")), _scale(d))
    errs = dict(o=rel_err(as_f64(o), ro), lse=rel_err(lse.cpu().numpy(), rlse))
    say("  errors: " + " ".join(f"{n}={e:.2e}" for n, e in errs.items()))
    assert max(errs.values()) <= TOL[dtype]


def test_merge_rows_no_part_saw():
    """Key padding split across shards: batch 0 keeps 190 of 300 keys (shard
    0 whole, 40 of shard 1), batch 1 keeps none, so every part of batch 1 is
    empty and its merged rows must be O = 0, LSE = -inf.  Against the oracle
    of the unsplit padded problem."""
    B, H, Nq, Nk, d = 2, 2, 256, 300, 64
    lens = [190, 0]
    inp = make_inputs(B, H, Nq, d, "bf16", seed=3, with_do=False, n_keys=Nk)
    q, k, v = (inp[n].cuda() for n in ("q", "k", "v"))
    parts = []
    for a, n in ((0, 150), (150, 150)):
        kl = torch.tensor([min(max(x - a, 0), n) for x in lens], dtype=torch.int32, device="cuda")
        parts.append(fa_fwd(q, k[:, :, a:a + n], v[:, :, a:a + n], key_lens=kl))
    o, lse = fa_merge_partials([x[0] for x in parts], [x[1] for x in parts])
    torch.cuda.synchronize()
    ro, rlse = oracle.forward(*(as_f64(inp[n]) for n in ("q", "k", "v")), _scale(d),
                              key_lens=np.array(lens))
    assert np.isinf(rlse[1]).all() and np.isfinite(rlse[0]).all()
    assert rel_err(as_f64(o), ro) <= TOL["bf16"]
    assert rel_err(lse.cpu().numpy(), rlse) <= TOL["bf16"]
    assert torch.all(o[1] == 0).item()


# ------------------------------------------------------------- ring schedules
def _compare(tag, got, ref, tol):
    errs = {n: rel_err(g, r) for n, g, r in zip(("o", "lse", "dq", "dk", "dv"), got, ref)}
    say(f"  {tag} errors: " + " ".join(f"{n}={e:.2e}" for n, e in errs.items()))
    bad = {n: e for n, e in errs.items() if not e <= tol}
    assert not bad, f"over tolerance {tol}: {bad}"


def test_ring_per_hop_shape_noncausal():
    """One device of a 4-device ring at the per-hop shape: 16K local queries,
    four visiting K / V shards of 16K keys each (64K keys), bf16, d = 64,
    non-causal.  Forward: four fa_fwd hops merged; backward: fa_bwd per hop
    with the merged O and LSE, dQ shares summed in fp32, the shards' dK / dV
    side by side.  Checked against the oracle of the 16K x 64K problem on
    every element."""
    B, H, Nq, S, d = 1, 2, 16384, 4, 64
    Ns = 16384
    say(f"case ring non-causal: {H} heads, {Nq} queries x {S} shards of {Ns} keys, bf16 d={d}")
    inp = make_inputs(B, H, Nq, d, "bf16", seed=21, n_keys=S * Ns)
    q, k, v, do = (inp[n].cuda() for n in ("q", "k", "v", "do"))
    parts = [fa_fwd(q, k[:, :, s * Ns:(s + 1) * Ns], v[:, :, s * Ns:(s + 1) * Ns]) for s in range(S)]
    o, lse = fa_merge_partials([x[0] for x in parts], [x[1] for x in parts])
    dq = torch.zeros(q.shape, dtype=torch.float32, device="cuda")
    dks, dvs = [], []
    for s in range(S):
        ks, vs = k[:, :, s * Ns:(s + 1) * Ns], v[:, :, s * Ns:(s + 1) * Ns]
        g = fa_bwd(q, ks, vs, o, lse, do)
        dq += g[0].float()
        dks.append(g[1])
        dvs.append(g[2])
    dk, dv = torch.cat(dks, dim=2), torch.cat(dvs, dim=2)
    torch.cuda.synchronize()
    say("  oracle (query-row blocks in parallel)...")
    rdq, rdk, rdv, ro, rlse = pool.backward_row_blocks(
        *(as_f64(inp[n]) for n in ("q", "k", "v", "do")), _scale(d))
    _compare("ring", (as_f64(o), lse.cpu().numpy(), as_f64(dq), as_f64(dk), as_f64(dv)),
             (ro, rlse, rdq, rdk, rdv), TOL["bf16"])


def _zigzag(P, chunk):
    """Global positions of device r's tokens: chunks r and 2P-1-r."""
    return [np.concatenate([np.arange(r * chunk, (r + 1) * chunk),
                            np.arange((2 * P - 1 - r) * chunk, (2 * P - r) * chunk)]) for r in range(P)]


def _hop_mask(pos_q, pos_k, chunk, mb):
    """Block mask of a hop between two devices (r != s): every chunk pair is
    either wholly visible (key chunk earlier) or wholly invisible."""
    nq, nk = pos_q.size // mb, pos_k.size // mb
    gq = pos_q[::mb][:nq] // chunk
    gk = pos_k[::mb][:nk] // chunk
    return (gk[None, :] < gq[:, None]).astype(np.uint8)


def test_ring_zigzag_causal():
    """Causal attention over 32K tokens on a 2-device ring with the zig-zag
    assignment (4 chunks of 8K: device 0 holds chunks 0 and 3, device 1 holds
    chunks 1 and 2, which balances the causal work).  Each device's queries
    meet each device's keys in one hop at the per-hop shape (16K x 16K):
    its own shard is a plain causal call, the other one a block-sparse call
    whose 128 x 128 mask says which chunk pairs see each other.  Forward hops
    merged per device, backward per hop with the merged statistics; dK / dV
    shares summed over devices, dQ shares over hops.  Checked, in global
    order, against the oracle of the whole causal 32K problem."""
    B, H, d, P, chunk, mb = 1, 2, 64, 2, 8192, 128
    N = 2 * P * chunk
    say(f"case ring zig-zag causal: {H} heads, N={N}, {P} devices, chunks of {chunk}, bf16 d={d}")
    inp = make_inputs(B, H, N, d, "bf16", seed=22)
    pos = _zigzag(P, chunk)
    dev = {n: [inp[n][:, :, torch.from_numpy(pos[r])].contiguous().cuda() for r in range(P)]
           for n in ("q", "k", "v", "do")}
    merged = []
    for r in range(P):
        o_parts, l_parts = [], []
        for s in range(P):
            q, k, v = dev["q"][r], dev["k"][s], dev["v"][s]
            if r == s:
                o, l = fa_fwd(q, k, v, causal=True)
            else:
                m = torch.from_numpy(_hop_mask(pos[r], pos[s], chunk, mb)).cuda()
                o, l = fa_fwd_blocksparse(q, k, v, m, mask_block=mb)
            o_parts.append(o)
            l_parts.append(l)
        merged.append(fa_merge_partials(o_parts, l_parts))
    dq = [torch.zeros(x.shape, dtype=torch.float32, device="cuda") for x in dev["q"]]
    dk = [torch.zeros(x.shape, dtype=torch.float32, device="cuda") for x in dev["k"]]
    dv = [torch.zeros(x.shape, dtype=torch.float32, device="cuda") for x in dev["k"]]
    for r in range(P):
        o, l = merged[r]
        for s in range(P):
            q, k, v, do = dev["q"][r], dev["k"][s], dev["v"][s], dev["do"][r]
            if r == s:
                g = fa_bwd(q, k, v, o, l, do, causal=True)
            else:
                m = torch.from_numpy(_hop_mask(pos[r], pos[s], chunk, mb)).cuda()
                g = fa_bwd_blocksparse(q, k, v, o, l, do, m, mask_block=mb)
            dq[r] += g[0].float()
            dk[s] += g[1].float()
            dv[s] += g[2].float()
    torch.cuda.synchronize()
    # back to global order
    def glob(parts, width):
        out = np.empty((B, H, N, width) if width else (B, H, N))
        for r in range(P):
            out[:, :, pos[r]] = parts[r]
        return out
    got = (glob([as_f64(merged[r][0]) for r in range(P)], d),
           glob([merged[r][1].cpu().numpy() for r in range(P)], 0),
           glob([as_f64(x) for x in dq], d), glob([as_f64(x) for x in dk], d),
           glob([as_f64(x) for x in dv], d))
    say("  oracle (query-row blocks in parallel)...")
    rdq, rdk, rdv, ro, rlse = pool.backward_row_blocks(
        *(as_f64(inp[n]) for n in ("q", "k", "v", "do")), _scale(d), causal=True)
    _compare("zig-zag", got, (ro, rlse, rdq, rdk, rdv), TOL["bf16"])
