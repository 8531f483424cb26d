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
from tests import test_oracle as pins

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle", "attention.py")

MUTANTS = [
    ("dQ without the scale", "dq[b, h, rows] = float(scale) * (ds @ kb)", "dq[b, h, rows] = (ds @ kb)"),
    ("dK without the scale", "dk[b, h] += float(scale) * (ds.T @ qb[rows])", "dk[b, h] += (ds.T @ qb[rows])"),
    ("D enters dS with the wrong sign", "ds = p * (dpc - Dp[:, None])", "ds = p * (dpc + Dp[:, None])"),
    ("dK from K instead of Q", "dk[b, h] += float(scale) * (ds.T @ qb[rows])",
     "dk[b, h] += float(scale) * (ds.T @ kb[rows])"),
    ("dV from V instead of dO", "dv[b, h] += p.T @ dob[rows]", "dv[b, h] += p.T @ vb[rows]"),
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
    ("O not normalised", "p = np.where(valid[:, None], e / np.where(valid, l, 1.0)[:, None], 0.0)\n    o = p @ v",
     "p = np.where(valid[:, None], e, 0.0)\n    o = p @ v"),
    ("empty row gives NaN-free but nonzero O", "p = np.where(valid[:, None], e / np.where(valid, l, 1.0)[:, None], 0.0)\n    o = p @ v",
     "p = np.where(valid[:, None], e / np.where(valid, l, 1.0)[:, None], 1.0 / s.shape[1])\n    o = p @ v"),
]

# The pins: every test function of tests/test_oracle.py except the ones that
# pin the streaming model (which reads its own module) -- expanded over their
# parametrisations.
def _pin_calls():
    calls = []
    for name, fn in inspect.getmembers(pins, inspect.isfunction):
        if not name.startswith("test_") or fn.__module__ != pins.__name__:
            continue
        marks = getattr(fn, "pytestmark", [])
        grids = [(m.args[0].split(","), m.args[1]) for m in marks if m.name == "parametrize"]
        if not grids:
            calls.append((name, fn, {}))
            continue
        keys = [k.strip() for g in grids for k in g[0]]
        for combo in itertools.product(*[g[1] for g in grids]):
            calls.append((name, fn, dict(zip(keys, combo))))
    return calls


def _load_mutant(old, new):
    src = open(SRC).read()
    assert src.count(old) >= 1, f"mutation site not found: {old!r}"
    src = src.replace(old, new)
    mod = types.ModuleType("oracle_attention_mutant")
    exec(compile(src, "<mutant>", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("label,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_kill_mutant(monkeypatch, label, old, new):
    mut = _load_mutant(old, new)
    for attr in ("allowed_mask", "forward", "forward_rows", "backward", "probabilities", "gradients_sampled"):
        monkeypatch.setattr(oracle, attr, getattr(mut, attr))
    killed_by = None
    for name, fn, kwargs in _pin_calls():
        try:
            fn(**kwargs)
        except pytest.skip.Exception:
            continue
        except Exception:  # an assertion (or an error) in a pin: the mutant is caught
            killed_by = f"{name}{kwargs or ''}"
            break
    assert killed_by is not None, f"no pin catches the mutant: {label}"


def test_pins_pass_on_the_real_oracle():
    """Sanity: the same harness finds no failing pin on the unmutated oracle."""
    for name, fn, kwargs in _pin_calls():
        try:
            fn(**kwargs)
        except pytest.skip.Exception:
            continue
