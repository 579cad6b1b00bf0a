"""Top-K ordering of each batch row, plain definition (TEST INFRASTRUCTURE).

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s
``cpu_baseline`` leg may import this module; the product library never does,
and the two share no code.

What it computes: the top-K token sampler of the recipe page "Custom
Operations: Applications in AI Models" (builds.modular.com), section
"Optimizing top-K token sampling for GPUs in MAX": each batch row holds how
often each candidate next word appears, and the operation returns two
arrays that order the row's entries by highest frequency, the values and
their positions. Readings taken where the page is silent:

- K: the first K entries of that ordering (K = V orders the whole row);
- equal values keep their original order (the lower index first), so the
  result is unique; -0.0 and +0.0 are equal values;
- the values returned are the input entries themselves (bit-for-bit);
- inputs are finite (NaN is outside the contract).

The definition, written out: sort the row's indices by (value descending,
index ascending) and keep the first K.
"""
from __future__ import annotations

import numpy as np


def topk_rows(x: np.ndarray, k: int):
    """For each row of the 2-D array x: (values, indices) of its K largest
    entries in descending order, equal values by ascending index."""
    x = np.asarray(x)
    if x.ndim != 2:
        raise ValueError("x must be 2-D (rows, entries)")
    rows, n = x.shape
    if not 1 <= k <= n:
        raise ValueError("need 1 <= k <= entries per row")
    vals = np.empty((rows, k), dtype=x.dtype)
    idx = np.empty((rows, k), dtype=np.int64)
    pos = np.arange(n)
    for r in range(rows):
        # np.lexsort sorts by the last key first: -value, then position.
        # Negating in float64 maps -0.0 and +0.0 to equal keys.
        order = np.lexsort((pos, -x[r].astype(np.float64)))
        idx[r] = order[:k]
        vals[r] = x[r, order[:k]]
    return vals, idx
