"""Pins of the oracle's dropout (CPU only).

Dropout is only named by the pages (FlashAttention summary page, "Key ideas",
kernel-fusion bullet); the contract is in oracle/dropout.py.  What pins it:

* the generator against the known-answer vectors that the authors of
  Philox4x32-10 publish with their Random123 library (ten rounds);
* the decision rule against its statistics (kept fraction 1 - t/256, byte
  uniformity, independence across heads, offsets and seeds);
* the 1/(1 - p) scale against the expectation E[O_dropout] = O;
* the gradient formulas against central differences of <dO, O_dropout> with
  the mask held fixed, and against the D identity;
* p = 0 against the plain definition.
"""
import numpy as np
import pytest

import oracle
from oracle import dropout as drop

from tests.test_oracle import MASKS, rand


# Random123 known-answer vectors for philox4x32, 10 rounds:
# (counter words, key words) -> output words.
KAT = [
    ((0x00000000, 0x00000000, 0x00000000, 0x00000000), (0x00000000, 0x00000000),
     (0x6627E8D5, 0xE169C58D, 0xBC57AC4C, 0x9B00DBD8)),
    ((0xFFFFFFFF, 0xFFFFFFFF, 0xFFFFFFFF, 0xFFFFFFFF), (0xFFFFFFFF, 0xFFFFFFFF),
     (0x408F276D, 0x41C83B0E, 0xA20BC7C6, 0x6D5451FD)),
    ((0x243F6A88, 0x85A308D3, 0x13198A2E, 0x03707344), (0xA4093822, 0x299F31D0),
     (0xD16CFE09, 0x94FDCCEB, 0x5001E420, 0x24126EA1)),
]


@pytest.mark.parametrize("ctr,key,out", KAT)
def test_philox_known_answers(ctr, key, out):
    got = drop.philox4x32_10(*ctr, *key)
    assert [int(x) for x in got] == list(out)


def test_philox_vectorised_equals_scalar_calls():
    rng = np.random.default_rng(5)
    c = rng.integers(0, 2 ** 32, size=(4, 37), dtype=np.uint64)
    k0, k1 = 0x12345678, 0x9ABCDEF0
    vec = drop.philox4x32_10(c[0], c[1], c[2], c[3], k0, k1)
    for n in range(37):
        one = drop.philox4x32_10(int(c[0, n]), int(c[1, n]), int(c[2, n]), int(c[3, n]), k0, k1)
        assert [int(w[n]) for w in vec] == [int(x) for x in one]


def _keep_by_definition(bh, i, j, p, seed, offset):
    """One decision from the written contract, scalar Python ints."""
    words = drop.philox4x32_10(i // 4, j // 4, bh, offset, seed & 0xFFFFFFFF, seed >> 32)
    byte = (int(words[i % 4]) >> (8 * (j % 4))) & 0xFF
    return byte >= min(255, max(0, round(p * 256)))


def test_keep_mask_follows_the_written_mapping():
    bh, p, seed, offset = 5, 0.3, (1 << 40) + 17, 3
    rows, cols = np.arange(3, 27), np.arange(1, 21)
    m = drop.keep_mask(bh, rows, cols, p, seed, offset)
    for a, i in enumerate(rows):
        for b, j in enumerate(cols):
            assert bool(m[a, b]) == _keep_by_definition(bh, int(i), int(j), p, seed, offset)


@pytest.mark.parametrize("p", [0.0, 0.1, 0.5, 0.9])
def test_kept_fraction(p):
    m = drop.keep_mask(7, np.arange(1024), np.arange(1024), p, 99, 0)
    q = 1.0 - drop.drop_threshold(p) / 256.0
    n = m.size
    assert abs(m.mean() - q) <= 5.0 * np.sqrt(q * (1 - q) / n) + 1e-12


def test_bytes_are_uniform():
    c = np.arange(1 << 16, dtype=np.uint64)
    words = drop.philox4x32_10(c, 11, 3, 0, 2024, 7)
    b = np.concatenate([((w >> np.uint64(8 * k)) & np.uint64(0xFF)).astype(np.int64)
                        for w in words for k in range(4)])
    counts = np.bincount(b, minlength=256)
    e = b.size / 256.0
    chi2 = float(((counts - e) ** 2 / e).sum())
    # 255 degrees of freedom: mean 255, sd ~22.6; 400 is beyond 6 sd
    assert chi2 < 400.0


def test_masks_independent_across_heads_offsets_and_seeds():
    p = 0.5
    base = drop.keep_mask(0, np.arange(512), np.arange(512), p, 1, 0)
    same = drop.keep_mask(0, np.arange(512), np.arange(512), p, 1, 0)
    assert np.array_equal(base, same)
    for other in (drop.keep_mask(1, np.arange(512), np.arange(512), p, 1, 0),
                  drop.keep_mask(0, np.arange(512), np.arange(512), p, 1, 1),
                  drop.keep_mask(0, np.arange(512), np.arange(512), p, 2, 0),
                  drop.keep_mask(0, np.arange(512), np.arange(512), p, 1 + (1 << 32), 0)):
        agree = (base == other).mean()
        assert abs(agree - 0.5) <= 5.0 * np.sqrt(0.25 / base.size)


def test_threshold_and_scale():
    assert drop.drop_threshold(0.0) == 0 and drop.keep_scale(0.0) == 1.0
    assert drop.drop_threshold(0.25) == 64 and drop.keep_scale(0.25) == 256.0 / 192.0
    assert drop.drop_threshold(0.999) == 255
    with pytest.raises(ValueError):
        drop.drop_threshold(1.0)


def _case(N=24, d=8, B=2, H=2, seed=0):
    q, k, v, do = (rand((B, H, N, d), seed + s) for s in range(4))
    return q, k, v, do


def _kw1(mask, N):
    """A mask case of the single-head pins, its 3 x 3 block mask stretched to
    cover N rows."""
    kw = dict(mask)
    if "block_mask" in kw:
        kw["mb"] = -(-N // 3)
    return kw


def _kw4(mask, B, N):
    """The same case as keywords of the batched oracle."""
    kw = _kw1(mask, N)
    if "key_len" in kw:
        kw["key_lens"] = [kw.pop("key_len")] * B
    return kw


@pytest.mark.parametrize("mi", range(len(MASKS)))
def test_p_zero_is_the_plain_definition(mi):
    q, k, v, do = _case()
    kw = _kw4(MASKS[mi], 2, 24)
    o0, l0 = oracle.forward(q, k, v, 0.4, **kw)
    o1, l1 = oracle.forward(q, k, v, 0.4, dropout=(0.0, 3, 1), **kw)
    assert np.array_equal(o0, o1) and np.array_equal(l0, l1)
    g0 = oracle.backward(q, k, v, do, 0.4, **kw)
    g1 = oracle.backward(q, k, v, do, 0.4, dropout=(0.0, 3, 1), **kw)
    for a, b in zip(g0, g1):
        assert np.array_equal(a, b)


def test_lse_ignores_dropout():
    q, k, v, _ = _case()
    _, l0 = oracle.forward(q, k, v, 0.4, causal=True)
    _, l1 = oracle.forward(q, k, v, 0.4, causal=True, dropout=(0.3, 3, 1))
    assert np.array_equal(l0, l1)


def test_expectation_over_masks_is_the_plain_output():
    q, k, v, _ = _case(N=16, d=4, B=1, H=1, seed=3)
    o, _ = oracle.forward(q, k, v, 0.5)
    samples = np.stack([oracle.forward(q, k, v, 0.5, dropout=(0.3, 77, off))[0] for off in range(600)])
    mean, se = samples.mean(0), samples.std(0) / np.sqrt(samples.shape[0])
    assert np.all(np.abs(mean - o) <= 6.0 * se + 1e-12)
    # without the 1/(1-p) scale the mean would be (1 - p) O: far outside
    assert np.max(np.abs(mean - 0.7 * o) / (6.0 * se + 1e-12)) > 1.0


def _loss(q, k, v, do, scale, kw):
    o, _ = oracle.forward(q, k, v, scale, **kw)
    return float(np.sum(o * do))


@pytest.mark.parametrize("mi", range(len(MASKS)))
def test_gradients_central_differences(mi):
    q, k, v, do = _case(N=12, d=4, B=1, H=2, seed=mi)
    kw = dict(_kw4(MASKS[mi], 1, 12), dropout=(0.35, 1234, 5))
    dq, dk, dv = oracle.backward(q, k, v, do, 0.6, **kw)
    h = 1e-6
    for x, g in ((q, dq), (k, dk), (v, dv)):
        num = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            old = x[idx]
            x[idx] = old + h
            fp = _loss(q, k, v, do, 0.6, kw)
            x[idx] = old - h
            fm = _loss(q, k, v, do, 0.6, kw)
            x[idx] = old
            num[idx] = (fp - fm) / (2 * h)
        assert np.max(np.abs(num - g)) <= 1e-6 * max(1.0, np.max(np.abs(g)))


def test_d_identity_with_dropout():
    q, k, v, do = _case(seed=9)
    _, _, _, (o, lse, D_p, D_o) = oracle.backward(q, k, v, do, 0.5, causal=True,
                                                    dropout=(0.2, 5, 0), return_aux=True)
    assert np.max(np.abs(D_p - D_o)) <= 1e-12 * max(1.0, np.max(np.abs(D_o)))


@pytest.mark.parametrize("mi", range(len(MASKS)))
def test_sampled_gradients_with_dropout_equal_full(mi):
    q, k, v, do = _case(N=40, d=8, B=1, H=1, seed=mi)
    kw, full_kw = _kw1(MASKS[mi], 40), _kw4(MASKS[mi], 1, 40)
    dr = (0.4, 8, 2)
    dq, dk, dv = oracle.backward(q, k, v, do, 0.3, dropout=dr, **full_kw)
    o, lse = oracle.forward(q, k, v, 0.3, dropout=dr, **full_kw)
    rows, cols = np.array([0, 5, 39]), np.array([1, 17, 38])
    orr, lr, dqr, dkc, dvc = oracle.gradients_sampled(q[0, 0], k[0, 0], v[0, 0], do[0, 0], 0.3, rows, cols,
                                                       dropout=dr, bh=0, **kw)
    np.testing.assert_allclose(orr, o[0, 0, rows], atol=1e-12)
    np.testing.assert_allclose(dqr, dq[0, 0, rows], atol=1e-12)
    np.testing.assert_allclose(dkc, dk[0, 0, cols], atol=1e-12)
    np.testing.assert_allclose(dvc, dv[0, 0, cols], atol=1e-12)
