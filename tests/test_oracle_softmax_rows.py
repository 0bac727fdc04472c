"""Pins of the row-softmax oracle (oracle/softmax_rows.py), all on the CPU.

Each pin checks the oracle against something other than itself: values the
pages print for their worked examples (tests/golden/worked_examples.json),
the element-by-element online two-pass recurrence of "Online Softmax 算法详解"
section 2.2 (written separately in oracle/softmax_ref.py), scipy's softmax
and logsumexp in float64 (a library routine for the same definition), closed
forms, and invariants. The last test plants mistakes in copies of the oracle
and checks that every one of them fails a pin.
"""
import json
import math
import os
import types

import numpy as np
import pytest
import scipy.special

import oracle
from oracle import softmax_ref

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "worked_examples.json")
EXAMPLES = {e["id"]: e for e in json.load(open(GOLDEN))["examples"]}


def _rng(seed):
    return np.random.default_rng(seed)


def pin_worked_examples(f):
    """The pages' worked examples, read as one row each: the printed final m
    and l (within the printed precision) and, for the example whose softmax
    vector is printed, that vector within its stated slip tolerance."""
    for ident, e in EXAMPLES.items():
        row = np.array([v for b in e["blocks"] for v in b], dtype=np.float64)
        y, lse, dead = f(row[None, :])
        assert not dead[0]
        fin = e["printed"]["final"]
        m = fin.get("m", row.max())
        tol_l = e.get("tol_final_l", e["tol"])
        assert abs(math.exp(lse[0] - m) - fin["l"]) <= tol_l, ident
        assert abs(y[0].sum() - 1.0) <= 1e-12, ident
        if "slip" in e and "softmax" in e["slip"]:
            printed = np.array(e["slip"]["softmax"]["printed"])
            rel = np.abs(y[0] - printed) / printed
            assert rel.max() <= e["slip"]["softmax"]["slip_tol_rel"], ident


def pin_online_two_pass(f):
    """Random rows with masked entries and an all-masked row: the oracle equals
    the element-by-element two-pass recurrence to 1e-12."""
    g = _rng(3)
    for cols in (1, 2, 7, 33, 200):
        x = g.normal(0, 4, size=(5, cols))
        x[1, g.random(cols) < 0.4] = -np.inf
        x[2, :] = -np.inf
        x[3] += 500.0
        y, lse, dead = f(x)
        for r in range(x.shape[0]):
            yr, m, l, lser = softmax_ref.online_two_pass(x[r])
            np.testing.assert_allclose(y[r], yr, rtol=1e-12, atol=1e-300)
            if math.isinf(lser):
                assert np.isneginf(lse[r]) and dead[r]
            else:
                assert abs(lse[r] - lser) <= 1e-12 * max(1.0, abs(lser)) and not dead[r]


def pin_scipy(f):
    """scipy.special.softmax / logsumexp in float64 on random rows."""
    g = _rng(4)
    for cols, sd in ((5, 1.0), (64, 3.0), (1000, 10.0), (4096, 0.5)):
        x = g.normal(0, sd, size=(7, cols))
        y, lse, dead = f(x)
        np.testing.assert_allclose(y, scipy.special.softmax(x, axis=1), rtol=1e-12, atol=1e-300)
        np.testing.assert_allclose(lse, scipy.special.logsumexp(x, axis=1), rtol=1e-13)
        assert not dead.any()


def pin_closed_forms(f):
    """Constant rows, two-element rows, a single live entry, all masked."""
    y, lse, dead = f(np.full((1, 10), 2.5))
    np.testing.assert_allclose(y, 0.1, rtol=1e-15)
    assert abs(lse[0] - (2.5 + math.log(10))) <= 1e-14
    for t in (-30.0, -1.0, 0.0, 0.7, 25.0):
        y, lse, _ = f(np.array([[0.0, t]]))
        assert abs(y[0, 1] - 1.0 / (1.0 + math.exp(-t))) <= 1e-15
        assert abs(lse[0] - (max(0.0, t) + math.log1p(math.exp(-abs(t))))) <= 1e-14
    y, lse, dead = f(np.array([[-np.inf, 3.0, -np.inf]]))
    assert y.tolist() == [[0.0, 1.0, 0.0]] and lse[0] == 3.0 and not dead[0]
    y, lse, dead = f(np.full((2, 4), -np.inf))
    assert (y == 0).all() and np.isneginf(lse).all() and dead.all()


def pin_invariants(f):
    """Shift invariance, permutation equivariance, rows sum to 1, no overflow
    at large magnitudes."""
    g = _rng(5)
    x = g.normal(0, 2, size=(4, 50))
    y, lse, _ = f(x)
    y2, lse2, _ = f(x + 123.25)
    np.testing.assert_allclose(y2, y, rtol=1e-12)
    np.testing.assert_allclose(lse2, lse + 123.25, rtol=1e-13)
    perm = g.permutation(50)
    y3, lse3, _ = f(x[:, perm])
    np.testing.assert_allclose(y3, y[:, perm], rtol=1e-13)
    np.testing.assert_allclose(lse3, lse, rtol=1e-14)
    np.testing.assert_allclose(y.sum(axis=1), 1.0, rtol=1e-14)
    assert ((y > 0) & (y <= 1)).all()
    big = np.array([[1000.0, 1001.0, 999.0], [-1000.0, -1001.0, -999.0]])
    y, lse, _ = f(big)
    assert np.isfinite(y).all() and np.isfinite(lse).all()
    np.testing.assert_allclose(y[0], scipy.special.softmax(big[0]), rtol=1e-13)
    rows = g.normal(size=(3, 9))
    ys, _, _ = f(rows)
    for r in range(3):  # each row depends on itself only
        yr, _, _ = f(rows[r:r + 1])
        np.testing.assert_allclose(ys[r], yr[0], rtol=0, atol=0)


PINS = [pin_worked_examples, pin_online_two_pass, pin_scipy, pin_closed_forms, pin_invariants]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_pin(pin):
    pin(oracle.softmax_rows)


def test_online_two_pass_matches_the_printed_examples():
    """The recurrence itself reproduces the printed final (m, l)."""
    for e in EXAMPLES.values():
        row = [v for b in e["blocks"] for v in b]
        _, m, l, _ = softmax_ref.online_two_pass(row)
        fin = e["printed"]["final"]
        assert m == fin.get("m", max(row))
        assert abs(l - fin["l"]) <= e.get("tol_final_l", e["tol"])


SRC = open(os.path.join(os.path.dirname(oracle.__file__), "softmax_rows.py")).read()

MUTANTS = [
    ("max not subtracted", "e = np.exp(x - m_ref[:, None])", "e = np.exp(x)"),
    ("max over the wrong axis", "m = np.max(x, axis=1, initial=-np.inf)", "m = np.max(x, axis=0, initial=-np.inf)[:1].repeat(x.shape[0])"),
    ("normalisation dropped", "e / safe_l[:, None]", "e"),
    ("sum over the wrong axis", "l = e.sum(axis=1)", "l = e.sum(axis=0)[:x.shape[0]] if x.shape[1] >= x.shape[0] else e.sum(axis=1) * 0 + e.sum()"),
    ("LSE without the max", "lse = np.where(dead, -np.inf, m_ref + np.log(safe_l))", "lse = np.where(dead, -np.inf, np.log(safe_l))"),
    ("LSE in base 2", "m_ref + np.log(safe_l)", "m_ref + np.log2(safe_l)"),
    ("exp argument sign flipped", "e = np.exp(x - m_ref[:, None])", "e = np.exp(m_ref[:, None] - x)"),
    ("all-masked row not guarded", "y = np.where(dead[:, None], 0.0, e / safe_l[:, None])", "y = e / l[:, None]"),
    ("dead rows flagged by any masked entry", "dead = ~np.isfinite(x).any(axis=1)", "dead = ~np.isfinite(x).all(axis=1)"),
    ("last column dropped from the max", "m = np.max(x, axis=1, initial=-np.inf)", "m = np.max(x[:, :-1], axis=1, initial=-np.inf)"),
]


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_every_planted_mistake_fails_a_pin(name, old, new):
    assert old in SRC, name
    mod = types.ModuleType("mutant")
    with np.errstate(all="ignore"):
        exec(compile(SRC.replace(old, new), "mutant", "exec"), mod.__dict__)
        failed = []
        for pin in PINS:
            try:
                pin(mod.softmax_rows)
            except Exception:  # an assertion or a crash both count as caught
                failed.append(pin.__name__)
    assert failed, f"mutant '{name}' passes every pin"
