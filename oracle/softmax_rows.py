"""Row softmax oracle: float64 three-pass safe softmax of every row of a matrix.

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the benchmark's CPU
baseline use it; the product path never imports it, and it shares no code
with the HIP library.

What it computes, for every row x of a [rows][cols] matrix (the plain
definition the online two-pass method reaches up to rounding, "Online Softmax
算法详解" sections 2.1 and 2.2):

    pass 1:  m = max_i x_i
    pass 2:  l = sum_i exp(x_i - m)
    pass 3:  y_i = exp(x_i - m) / l,   lse = m + ln l

in float64, every input value upcast exactly. Entries equal to -inf are
masked (exp(-inf - m) = 0); a row whose entries are all -inf gets y = 0 and
lse = -inf, the all-masked convention of "Online Softmax 算法详解" sections
7.2-7.3. Inputs are NaN-free by contract.
"""
from __future__ import annotations

import numpy as np


def softmax_rows(x):
    """Returns (y float64 [rows][cols], lse float64 [rows], dead bool [rows])."""
    x = np.asarray(x, dtype=np.float64)
    if x.ndim != 2:
        raise ValueError("x must be 2-D [rows][cols]")
    dead = ~np.isfinite(x).any(axis=1)          # every entry -inf (or no entry)
    m = np.max(x, axis=1, initial=-np.inf)      # pass 1
    m_ref = np.where(dead, 0.0, m)              # keeps -inf - (-inf) out of exp
    e = np.exp(x - m_ref[:, None])              # masked entries give exactly 0
    l = e.sum(axis=1)                           # pass 2
    safe_l = np.where(dead, 1.0, l)
    y = np.where(dead[:, None], 0.0, e / safe_l[:, None])   # pass 3
    lse = np.where(dead, -np.inf, m_ref + np.log(safe_l))
    return y, lse, dead
