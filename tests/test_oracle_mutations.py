"""Planted mistakes: each mutant of the C oracle must fail at least one pin.

The mutants are textual edits of oracle/attention_oracle.c compiled into a
temporary library; the pins of test_oracle_pins.py are then run against that
library instead of the real one. A mutant that passes every pin would show a
hole in the pins. Everything here runs on the CPU.
"""
import importlib
import os

import pytest

import oracle
import tests.test_oracle_pins as pins

_oracle_mod = importlib.import_module("oracle.attention")
SRC = os.path.join(os.path.dirname(_oracle_mod.__file__), "attention_oracle.c")

# (name, text in the source, replacement): each a plausible slip.
MUTANTS = [
    ("scale dropped", "s[j] = scale * dot;", "s[j] = dot;"),
    ("exp argument sign flipped", "l += exp(s[j] - m);", "l += exp(m - s[j]);"),
    ("no max subtracted in pass 3", "double p = exp(s[j] - m) / l;", "double p = exp(s[j]) / l;"),
    ("normalisation dropped", "double p = exp(s[j] - m) / l;", "double p = exp(s[j] - m);"),
    ("K read from V", "(double)kb[(long long)j * d + t]", "(double)vb[(long long)j * d + t]"),
    ("V row indexed by the query", "const float* vj = vb + (long long)j * d;",
     "const float* vj = vb + (long long)i * d;"),
    ("causal bound off by one", "if (causal && j > i) return 0;", "if (causal && j >= i) return 0;"),
    ("causal bound reversed", "if (causal && j > i) return 0;", "if (causal && j < i) return 0;"),
    ("mask polarity inverted", "mask[(long)b * N + j] == 0", "mask[(long)b * N + j] != 0"),
    ("mask indexed by head", "int b = (int)(bh / H);", "int b = (int)(bh % H);"),
    ("LSE without the max", "*lse = m + log(l);", "*lse = log(l);"),
    ("LSE in base 2", "*lse = m + log(l);", "*lse = m + log2(l);"),
    ("last key left out of the max", "for (long j = 0; j < N; j++)\n        if (allowed(mask, b, N, causal, i, j) && s[j] > m)",
     "for (long j = 0; j < N - 1; j++)\n        if (allowed(mask, b, N, causal, i, j) && s[j] > m)"),
    ("fully masked row reported as live", "*fully_masked = 1;", "*fully_masked = 0;"),
    ("query row offset by head only", "const float* qi = q + row * (long long)d;",
     "const float* qi = q + (bh * (long long)N) * d;"),
]

# the pins that go through the C oracle, with their parameters
PIN_CALLS = (
    [(pins.test_examples_through_attention_oracle, dict(ident=i))
     for i in ("blocks_2_4_then_1_3", "blocks_1_2_then_5_3", "chunks_1_2_then_3_10_v_ones")]
    + [(pins.test_practice_problem_through_attention_oracle, {})]
    + [(pins.test_brute_force_naive, dict(N=n, d=d, causal=c, use_mask=m))
       for n, d, c, m in [(3, 2, False, False), (5, 3, True, False), (8, 4, False, True), (7, 4, True, True)]]
    + [(pins.test_against_torch_sdpa_float64, dict(B=1, H=1, N=256, d=64, causal=False))]
    + [(pins.test_recurrence_matches_three_pass_every_block_size, dict(N=17, causal=True, use_mask=False)),
       (pins.test_recurrence_matches_three_pass_every_block_size, dict(N=23, causal=False, use_mask=True))]
    + [(pins.test_shift_invariance_through_an_extra_dimension, {}),
       (pins.test_safe_softmax_properties, {}),
       (pins.test_special_cases, {})]
)


def _run_pins_against(lib):
    """Returns the names of the pins that failed with `lib` in place."""
    saved = _oracle_mod._lib
    _oracle_mod._lib = lib
    failed = []
    try:
        for fn, kw in PIN_CALLS:
            try:
                fn(**kw)
            except (AssertionError, RuntimeError, ValueError, FloatingPointError):
                failed.append(fn.__name__)
    finally:
        _oracle_mod._lib = saved
    return failed


def test_unmutated_oracle_passes_every_pin():
    assert _run_pins_against(oracle.load()) == []


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(tmp_path, name, old, new):
    src = open(SRC).read()
    assert src.count(old) >= 1, f"mutation site for {name!r} not found"
    mutated = src.replace(old, new, 1)
    path = tmp_path / "mutant.c"
    path.write_text(mutated)
    so = _oracle_mod.build(str(path), str(tmp_path / "libmutant.so"))
    lib = _oracle_mod.open_library(so)
    failed = _run_pins_against(lib)
    assert failed, f"mutant {name!r} passed every pin"
