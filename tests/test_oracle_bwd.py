"""Pins of the attention backward oracle (oracle/attention_bwd.py), CPU only.

The gradient is pinned to the forward's definition by central finite
differences of a loss L = sum(O * dO) through an independently written
forward (`softmax_ref.online_attention`, the blocked online recurrence in
float64), to torch's autograd of scaled_dot_product_attention in float64 (a
library routine), and to properties the mathematics fixes: the rows of dS
sum to zero so the key gradients sum to zero, the value gradients sum to the
output gradients of the rows that attend anywhere, a single key receives
dV = dO with dQ = dK = 0, and rows with no allowed key contribute nothing.
The last test plants mistakes in copies of the oracle and checks that each
fails a pin.
"""
import importlib
import types

import numpy as np
import pytest
import torch

from oracle import softmax_ref

AB = importlib.import_module("oracle.attention_bwd")


def _inputs(B, H, N, d, seed, causal=False, masked=False, dead_batch=False):
    g = np.random.default_rng(seed)
    q, k, v, do = (g.normal(size=(B, H, N, d)) for _ in range(4))
    mask = None
    if masked:
        mask = (g.random((B, N)) > 0.3).astype(np.uint8)
        mask[:, 0] = 1
        if dead_batch:
            mask[0] = 0
    return q, k, v, do, mask


def _loss(q, k, v, do, scale, causal, mask):
    O, _, _ = softmax_ref.online_attention(q, k, v, scale, causal, mask, block_c=2)
    return float((O * do).sum())


def pin_finite_differences(bwd):
    """Central differences (h = 1e-5) of sum(O * dO) against dQ, dK, dV."""
    for (B, H, N, d, causal, masked, dead) in [(1, 1, 5, 3, False, False, False), (1, 2, 6, 2, True, False, False),
                                               (2, 1, 4, 3, False, True, True), (1, 1, 7, 2, True, True, False)]:
        q, k, v, do, mask = _inputs(B, H, N, d, seed=N * 10 + d, causal=causal, masked=masked, dead_batch=dead)
        scale = 0.7
        g = bwd(q, k, v, do, scale, causal, mask)
        h = 1e-5
        for name, t in (("dq", q), ("dk", k), ("dv", v)):
            num = np.zeros_like(t)
            it = np.nditer(t, flags=["multi_index"])
            for _ in it:
                idx = it.multi_index
                old = t[idx]
                t[idx] = old + h
                lp = _loss(q, k, v, do, scale, causal, mask)
                t[idx] = old - h
                lm = _loss(q, k, v, do, scale, causal, mask)
                t[idx] = old
                num[idx] = (lp - lm) / (2 * h)
            np.testing.assert_allclose(g[name], num, rtol=1e-6, atol=1e-8, err_msg=name)


def pin_torch_autograd(bwd):
    """torch.nn.functional.scaled_dot_product_attention in float64 on the CPU,
    differentiated by autograd (masks leave every row at least one key)."""
    for (B, H, N, d, causal, masked) in [(2, 2, 33, 16, False, False), (1, 3, 40, 8, True, False),
                                         (2, 1, 29, 12, False, True), (1, 2, 64, 32, True, True)]:
        q, k, v, do, mask = _inputs(B, H, N, d, seed=N + d, masked=masked)
        scale = 1.0 / np.sqrt(d)
        allow = torch.ones(B, 1, N, N, dtype=torch.bool)
        if causal:
            allow &= torch.tril(torch.ones(N, N, dtype=torch.bool))
        if mask is not None:
            allow &= torch.from_numpy(mask != 0)[:, None, None, :]
        tq, tk, tv = (torch.tensor(a, dtype=torch.float64, requires_grad=True) for a in (q, k, v))
        o = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=allow, scale=scale)
        (o * torch.from_numpy(do)).sum().backward()
        g = bwd(q, k, v, do, scale, causal, mask)
        np.testing.assert_allclose(g["o"], o.detach().numpy(), rtol=1e-10, atol=1e-12)
        for name, t in (("dq", tq), ("dk", tk), ("dv", tv)):
            np.testing.assert_allclose(g[name], t.grad.numpy(), rtol=1e-9, atol=1e-11, err_msg=name)


def pin_sums(bwd):
    """Rows of dS sum to zero, so sum_j dK_j = 0 per head; sum_j dV_j equals
    the sum of dO over the rows that attend anywhere; D = rowsum(dO * O)."""
    q, k, v, do, mask = _inputs(2, 2, 50, 8, seed=9, masked=True, dead_batch=True)
    for causal in (False, True):
        g = bwd(q, k, v, do, 0.3, causal, mask)
        np.testing.assert_allclose(g["dk"].sum(axis=2), 0.0, atol=1e-11)
        live = np.isfinite(g["lse"])
        np.testing.assert_allclose(g["dv"].sum(axis=2), (do * live[..., None]).sum(axis=2), rtol=1e-11,
                                   atol=1e-11)
        np.testing.assert_allclose(g["D"], (do * g["o"]).sum(axis=-1), rtol=1e-11, atol=1e-12)
        assert np.all(g["dq"][0] == 0.0) and np.all(g["dk"][0] == 0.0) and np.all(g["dv"][0] == 0.0)


def pin_special_cases(bwd):
    """One key: P = 1, so dV = dO and dQ = dK = 0. Causal row 0 sees only
    key 0: its dQ is 0. K = 0: P is uniform over the allowed keys."""
    q, k, v, do, _ = _inputs(1, 1, 1, 4, seed=1)
    g = bwd(q, k, v, do, 0.5, False, None)
    np.testing.assert_allclose(g["dv"], do, rtol=1e-15)
    assert np.all(g["dq"] == 0) and np.all(g["dk"] == 0)
    q, k, v, do, _ = _inputs(1, 1, 6, 3, seed=2)
    g = bwd(q, k, v, do, 0.5, True, None)
    assert np.all(g["dq"][0, 0, 0] == 0)
    k0 = np.zeros_like(k)
    g = bwd(q, k0, v, do, 0.5, False, None)
    np.testing.assert_allclose(g["dv"][0, 0], np.repeat(do[0, 0].mean(axis=0, keepdims=True), 6, axis=0),
                               rtol=1e-13)
    np.testing.assert_allclose(g["o"][0, 0], np.repeat(v[0, 0].mean(axis=0, keepdims=True), 6, axis=0),
                               rtol=1e-13)


PINS = [pin_finite_differences, pin_torch_autograd, pin_sums, pin_special_cases]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_pin(pin):
    pin(AB.attention_bwd)


SRC = open(AB.__file__).read()
MUTANTS = [
    ("softmax Jacobian without the D term", "dS = P * (dP - D[:, None])", "dS = P * dP"),
    ("dQ without the scale", 'out["dq"][b, h] = scale * (dS @ K)', 'out["dq"][b, h] = dS @ K'),
    ("dK from dS not transposed", 'out["dk"][b, h] = scale * (dS.T @ Q)', 'out["dk"][b, h] = scale * (dS @ Q)'),
    ("dV from P not transposed", "dV = P.T @ dO", "dV = P @ dO"),
    ("dP from V not transposed", "dP = dO @ V.T", "dP = dO @ V"),
    ("D as the plain row sum of dP", "D = (P * dP).sum(axis=1)", "D = dP.sum(axis=1)"),
    ("causal mask transposed", "a &= np.tril(np.ones((N, N), dtype=bool))", "a &= np.triu(np.ones((N, N), dtype=bool))"),
    ("scale applied twice to dK", 'out["dk"][b, h] = scale * (dS.T @ Q)', 'out["dk"][b, h] = scale * scale * (dS.T @ Q)'),
    ("key mask ignored", "a &= (np.asarray(mask_row) != 0)[None, :]", "pass"),
    ("dS with the wrong sign", "dS = P * (dP - D[:, None])", "dS = P * (D[:, None] - dP)"),
]


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_every_planted_mistake_fails_a_pin(name, old, new):
    assert old in SRC, name
    mod = types.ModuleType("mutant")
    exec(compile(SRC.replace(old, new), "mutant", "exec"), mod.__dict__)
    failed = []
    with np.errstate(all="ignore"):
        for pin in PINS:
            try:
                pin(mod.attention_bwd)
            except Exception:
                failed.append(pin.__name__)
    assert failed, f"mutant '{name}' passes every pin"
