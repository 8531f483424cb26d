"""Mutation test of the oracle's pins (CPU only).

Each mutant is a copy of oracle/attention.py with one plausible mistake
planted in its source text (a dropped scale, a flipped sign, a swapped
operand, an off-by-one mask, a missing max subtraction, ...).  The pins of
tests/test_oracle.py are then run against the mutant; at least one must fail,
otherwise the pins would not have caught that mistake in the real oracle.
The mistakes are planted only in these in-memory copies, never in the oracle.
"""
import importlib.util
import inspect
import itertools
import os
import sys
import types

import pytest

import oracle
import oracle.attention
import oracle.dropout
from tests import test_oracle as pins
from tests import test_oracle_dropout as drop_pins
from tests import test_oracle_rect as rect_pins
from tests import test_oracle_reductions as red_pins

_ORACLE = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle")
SRC = os.path.join(_ORACLE, "attention.py")
DROP_SRC = os.path.join(_ORACLE, "dropout.py")
RED_SRC = os.path.join(_ORACLE, "reductions.py")

MUTANTS = [
    ("dQ without the scale", "dq[b, h, rows] = float(scale) * (ds @ kb)", "dq[b, h, rows] = (ds @ kb)"),
    ("dK without the scale", "dk[b, h] += float(scale) * (ds.T @ qb[rows])", "dk[b, h] += (ds.T @ qb[rows])"),
    ("D enters dS with the wrong sign", "ds = p * (zdp - Dp[:, None])", "ds = p * (zdp + Dp[:, None])"),
    ("dK from K instead of Q", "dk[b, h] += float(scale) * (ds.T @ qb[rows])",
     "dk[b, h] += float(scale) * (ds.T @ kb[rows])"),
    ("dV from V instead of dO", "dv[b, h] += pz.T @ dob[rows]", "dv[b, h] += pz.T @ vb[rows]"),
    ("dP transposed operand", "dpc = dob[rows] @ vb.T", "dpc = vb[rows] @ dob.T"),
    ("dQ from dS^T", "dq[b, h, rows] = float(scale) * (ds @ kb)", "dq[b, h, rows] = float(scale) * (ds.T @ kb[rows])"),
    ("causal mask j < i", "a &= cols[None, :] <= rows[:, None]", "a &= cols[None, :] < rows[:, None]"),
    ("causal mask transposed", "a &= cols[None, :] <= rows[:, None]", "a &= cols[None, :] >= rows[:, None]"),
    ("padding mask off by one", "a &= cols[None, :] < int(key_len)", "a &= cols[None, :] <= int(key_len)"),
    ("block mask transposed", "a &= bm[rows[:, None] // mb, cols[None, :] // mb]",
     "a &= bm[cols[None, :] // mb, rows[:, None] // mb]"),
    ("no max subtraction", "e = np.exp(s - m[:, None])", "e = np.exp(s)"),
    ("LSE without the max", "lse = np.where(valid, m + np.log(np.where(valid, l, 1.0)), -np.inf)",
     "lse = np.where(valid, np.log(np.where(valid, l, 1.0)), -np.inf)"),
    ("scale applied twice", "s = float(scale) * (q[rows] @ k.T)", "s = float(scale) ** 2 * (q[rows] @ k.T)"),
    ("O not normalised", "p = np.where(valid[:, None], e / np.where(valid, l, 1.0)[:, None], 0.0)\n    z = _z(bh, rows",
     "p = np.where(valid[:, None], e, 0.0)\n    z = _z(bh, rows"),
    ("empty row gives NaN-free but nonzero O",
     "p = np.where(valid[:, None], e / np.where(valid, l, 1.0)[:, None], 0.0)\n    z = _z(bh, rows",
     "p = np.where(valid[:, None], e / np.where(valid, l, 1.0)[:, None], 1.0 / s.shape[1])\n    z = _z(bh, rows"),
]

# Mistakes in the dropout path: in attention.py (where Z enters) or in
# dropout.py (the generator and the mapping); caught by the dropout pins.
DROP_MUTANTS = [
    ("O without Z", SRC, "o = (p if z is None else p * z) @ v", "o = p @ v"),
    ("dV without Z", SRC, "dv[b, h] += pz.T @ dob[rows]", "dv[b, h] += p.T @ dob[rows]"),
    ("dP without Z", SRC, "zdp = dpc if z is None else z * dpc", "zdp = dpc"),
    ("D without Z", SRC, "Dp = np.sum(p * zdp, axis=1)", "Dp = np.sum(p * dpc, axis=1)"),
    ("kept entries not rescaled", SRC, "keep_mask(bh, rows, cols, p, seed, offset) * keep_scale(p)",
     "keep_mask(bh, rows, cols, p, seed, offset) * 1.0"),
    ("nine Philox rounds", DROP_SRC, "for r in range(10):", "for r in range(9):"),
    ("key never bumped", DROP_SRC, "        if r < 9:\n", "        if False:\n"),
    ("Philox products swapped", DROP_SRC, "c = [hi1 ^ c[1] ^ k0, lo1, hi0 ^ c[3] ^ k1, lo0]",
     "c = [hi0 ^ c[1] ^ k0, lo0, hi1 ^ c[3] ^ k1, lo1]"),
    ("counter blocks transposed", DROP_SRC, "philox4x32_10(qblk[:, None], kblk[None, :], int(bh)",
     "philox4x32_10(kblk[None, :], qblk[:, None], int(bh)"),
    ("word chosen by the key", DROP_SRC, "word = words[(rows % 4)[:, None],", "word = words[(cols % 4)[None, :],"),
    ("threshold truncated", DROP_SRC, "round(float(p) * 256.0)", "int(float(p) * 256.0)"),
    ("keep on byte > t", DROP_SRC, "return byte >= np.uint64(t)", "return byte > np.uint64(t)"),
    ("seed high word dropped", DROP_SRC, "seed & 0xFFFFFFFF, (seed >> 32) & 0xFFFFFFFF)",
     "seed & 0xFFFFFFFF, 0)"),
]


# Mistakes in the N_q != N_k generalisation, caught by the rectangular pins.
RECT_MUTANTS = [
    ("causal aligned top-left", "shift = 0 if n_queries is None else N - int(n_queries)", "shift = 0"),
    ("causal offset with the wrong sign", "shift = 0 if n_queries is None else N - int(n_queries)",
     "shift = 0 if n_queries is None else int(n_queries) - N"),
    ("backward mask without the query count", "a = allowed_mask(rows, Nk, causal=causal, key_len=lens[b],\n"
     "                                 block_mask=bm, mb=mb, n_queries=N)",
     "a = allowed_mask(rows, Nk, causal=causal, key_len=lens[b],\n"
     "                                 block_mask=bm, mb=mb)"),
    ("sampled pass over the selected rows only", "    need = np.nonzero(sees)[0]\n", "    need = np.unique(rows)\n"),
    ("sampled column mask over the wrong keys", "        a = allowed_mask(rr, N, cols=cols, **mk)",
     "        a = allowed_mask(rr, N, **mk)[:, :cols.size]"),
]


# Mistakes in the other streaming reductions, caught by their pins.
RED_MUTANTS = [
    ("sample variance (n - 1)", "var = ((x - mean[:, None]) ** 2).sum(axis=1) / L",
     "var = ((x - mean[:, None]) ** 2).sum(axis=1) / (L - 1)"),
    ("eps outside the square root", "rstd = 1.0 / np.sqrt(var + float(eps))",
     "rstd = 1.0 / (np.sqrt(var) + float(eps))"),
    ("affine index ignores the group", "return (r % groups) * cpg + e // inner", "return e // inner"),
    ("affine index ignores the inner size", "return (r % groups) * cpg + e // inner",
     "return (r % groups) * cpg + e % cpg"),
    ("moment merge weights swapped", "mean = np.where(n > 0, ma + delta * nb / safe, 0.0)",
     "mean = np.where(n > 0, ma + delta * na / safe, 0.0)"),
    ("moment merge without the cross term", "m2 = m2a + m2b + delta * delta * na * nb / safe",
     "m2 = m2a + m2b"),
    ("softmax LSE without the max", "lse = np.where(valid, m + np.log(np.where(valid, l, 1.0)), -np.inf)",
     "lse = np.where(valid, np.log(np.where(valid, l, 1.0)), -np.inf)"),
    ("softmax not normalised", "y = np.where(valid[:, None], e / np.where(valid, l, 1.0)[:, None], 0.0)",
     "y = np.where(valid[:, None], e, 0.0)"),
    ("empty softmax row not zero", "y = np.where(valid[:, None], e / np.where(valid, l, 1.0)[:, None], 0.0)",
     "y = np.where(valid[:, None], e / np.where(valid, l, 1.0)[:, None], 1.0 / x.shape[1])"),
]
_RED = ("softmax_rows", "layernorm_rows", "merge_moments", "streaming_moments")


# The pins: every test function of a pin module (tests/test_oracle.py, or
# tests/test_oracle_dropout.py for the dropout mutants) -- expanded over their
# parametrisations.
def _pin_calls(pins=pins):
    calls = []
    for name, fn in inspect.getmembers(pins, inspect.isfunction):
        if not name.startswith("test_") or fn.__module__ != pins.__name__:
            continue
        marks = getattr(fn, "pytestmark", [])
        grids = [(m.args[0].split(","), m.args[1]) for m in marks if m.name == "parametrize"]
        if not grids:
            calls.append((name, fn, {}))
            continue
        # one list of keyword dicts per parametrize mark (a mark naming
        # several arguments gives tuples to spread over them)
        per_mark = [[dict(zip([k.strip() for k in names], vals if len(names) > 1 else (vals,)))
                     for vals in values] for names, values in grids]
        for combo in itertools.product(*per_mark):
            kw = {}
            for part in combo:
                kw.update(part)
            calls.append((name, fn, kw))
    return calls


def _load_mutant(old, new, path=SRC):
    src = open(path).read()
    assert src.count(old) >= 1, f"mutation site not found: {old!r}"
    src = src.replace(old, new)
    mod = types.ModuleType("oracle_mutant")
    mod.__package__ = "oracle"       # its relative imports resolve to the real oracle
    exec(compile(src, "<mutant>", "exec"), mod.__dict__)
    return mod


def _first_failing_pin(pins):
    for name, fn, kwargs in _pin_calls(pins):
        try:
            fn(**kwargs)
        except pytest.skip.Exception:
            continue
        except Exception:  # an assertion (or an error) in a pin: the mutant is caught
            return f"{name}{kwargs or ''}"
    return None


_ATTN = ("allowed_mask", "forward", "forward_rows", "backward", "probabilities", "gradients_sampled")
_DROP = ("philox4x32_10", "drop_threshold", "keep_scale", "keep_mask")


@pytest.mark.parametrize("label,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_kill_mutant(monkeypatch, label, old, new):
    mut = _load_mutant(old, new)
    for attr in _ATTN:
        monkeypatch.setattr(oracle, attr, getattr(mut, attr))
    assert _first_failing_pin(pins) is not None, f"no pin catches the mutant: {label}"


@pytest.mark.parametrize("label,path,old,new", DROP_MUTANTS, ids=[m[0] for m in DROP_MUTANTS])
def test_dropout_pins_kill_mutant(monkeypatch, label, path, old, new):
    mut = _load_mutant(old, new, path)
    if path == SRC:
        for attr in _ATTN:
            monkeypatch.setattr(oracle, attr, getattr(mut, attr))
    else:
        for attr in _DROP:
            monkeypatch.setattr(oracle.dropout, attr, getattr(mut, attr))
            monkeypatch.setattr(oracle, attr, getattr(mut, attr))
        monkeypatch.setattr(oracle.attention, "keep_mask", mut.keep_mask)
        monkeypatch.setattr(oracle.attention, "keep_scale", mut.keep_scale)
    assert _first_failing_pin(drop_pins) is not None, f"no dropout pin catches the mutant: {label}"


@pytest.mark.parametrize("label,old,new", RECT_MUTANTS, ids=[m[0] for m in RECT_MUTANTS])
def test_rect_pins_kill_mutant(monkeypatch, label, old, new):
    mut = _load_mutant(old, new)
    for attr in _ATTN:
        monkeypatch.setattr(oracle, attr, getattr(mut, attr))
    assert _first_failing_pin(rect_pins) is not None, f"no rectangular pin catches the mutant: {label}"


@pytest.mark.parametrize("label,old,new", RED_MUTANTS, ids=[m[0] for m in RED_MUTANTS])
def test_reduction_pins_kill_mutant(monkeypatch, label, old, new):
    mut = _load_mutant(old, new, RED_SRC)
    for attr in _RED:
        monkeypatch.setattr(oracle, attr, getattr(mut, attr))
    assert _first_failing_pin(red_pins) is not None, f"no reduction pin catches the mutant: {label}"


def test_pins_pass_on_the_real_oracle():
    """Sanity: the same harness finds no failing pin on the unmutated oracle."""
    for p in (pins, drop_pins, rect_pins, red_pins):
        for name, fn, kwargs in _pin_calls(p):
            try:
                fn(**kwargs)
            except pytest.skip.Exception:
                continue
