"""Tiled online-softmax recurrences, in NumPy fp64 (TEST INFRASTRUCTURE).

These are the pages' own tiled formulations of attention, written from their
description (not from their listings) and completed with what the listings
leave out: the ``scale`` factor, the mask functor, grouped K/V heads and tail
tiles (the listings floor-divide the block count and drop the tail).

- ``fa2_deferred``: the FlashAttention-2 recurrence of ``flash_attn_v2`` /
  ``flash_attn_v2_multihead`` (tiny_flash_attn.py, github.com/66RING): query
  blocks outside, key blocks inside, running max ``m`` and running sum ``l``
  per query row, the output rescaled by exp(m_old - m_new) at each step and
  divided by ``l`` once after the last key block.
- ``fa_stepwise``: the per-step-normalised form of the Mojo kernel on the
  recipe page "Custom Operations: Applications in AI Models", section
  "Optimizing attention via FlashAttention": at every key tile the output is
  renormalised by (l_old / l_new) * exp(m_old - m_new) and the new
  probabilities are divided by l_new before they meet V.

In exact arithmetic both equal plain attention for every tile size; the tests
use that to pin the oracle (a second, independent formulation of the same
result) and to show the recurrence the HIP kernel uses is exact.

A row whose keys are all hidden so far has running max -inf; the guards below
use 0 as the subtraction base there so that (-inf) - (-inf) never occurs.
"""
from __future__ import annotations

import numpy as np

NONE, CAUSAL, WINDOW = 0, 1, 2


def _mask_code(mask):
    if isinstance(mask, str):
        return {"none": NONE, "causal": CAUSAL, "sliding_window": WINDOW, "window": WINDOW}[mask]
    return int(mask)


def _visible(kind, window, rows, cols):
    """Boolean (len(rows), len(cols)) visibility under the mask functor."""
    i = rows[:, None]
    j = cols[None, :]
    if kind == NONE:
        return np.ones((len(rows), len(cols)), dtype=bool)
    if kind == CAUSAL:
        return j <= i
    return (j <= i) & (j > i - window)


def _blocks(n, size):
    return [(s, min(s + size, n)) for s in range(0, n, size)]


def fa2_deferred(q, k, v, scale, mask="none", window=-1, block_m=4, block_n=4):
    """FlashAttention-2 recurrence with deferred normalisation; BSHD in, BSHD out."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    kind = _mask_code(mask)
    B, S, H, D = q.shape
    Hkv = k.shape[2]
    out = np.zeros_like(q)
    for b in range(B):
        for h in range(H):
            g = h // (H // Hkv)
            for qs, qe in _blocks(S, block_m):
                qi = q[b, qs:qe, h, :]
                rows = np.arange(qs, qe)
                m = np.full((qe - qs, 1), -np.inf)
                l = np.zeros((qe - qs, 1))
                o = np.zeros((qe - qs, D))
                for ks, ke in _blocks(S, block_n):
                    x = (qi @ k[b, ks:ke, g, :].T) * scale
                    x = np.where(_visible(kind, window, rows, np.arange(ks, ke)), x, -np.inf)
                    m_new = np.maximum(m, x.max(axis=1, keepdims=True))
                    base = np.where(np.isneginf(m_new), 0.0, m_new)
                    e = np.exp(x - base)
                    alpha = np.where(np.isneginf(m), 0.0, np.exp(m - base))
                    l = l * alpha + e.sum(axis=1, keepdims=True)
                    o = o * alpha + e @ v[b, ks:ke, g, :]
                    m = m_new
                out[b, qs:qe, h, :] = o / l
    return out


def fa_stepwise(q, k, v, scale, mask="none", window=-1, block_m=4, block_n=4):
    """Per-step-normalised online softmax; BSHD in, BSHD out."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    kind = _mask_code(mask)
    B, S, H, D = q.shape
    Hkv = k.shape[2]
    out = np.zeros_like(q)
    for b in range(B):
        for h in range(H):
            g = h // (H // Hkv)
            for qs, qe in _blocks(S, block_m):
                qi = q[b, qs:qe, h, :]
                rows = np.arange(qs, qe)
                m1 = np.full((qe - qs, 1), -np.inf)
                l1 = np.zeros((qe - qs, 1))
                o = np.zeros((qe - qs, D))
                for ks, ke in _blocks(S, block_n):
                    s = (qi @ k[b, ks:ke, g, :].T) * scale
                    s = np.where(_visible(kind, window, rows, np.arange(ks, ke)), s, -np.inf)
                    m2 = np.maximum(m1, s.max(axis=1, keepdims=True))
                    base = np.where(np.isneginf(m2), 0.0, m2)
                    decay = np.where(np.isneginf(m1), 0.0, np.exp(m1 - base))
                    e = np.exp(s - base)
                    l2 = decay * l1 + e.sum(axis=1, keepdims=True)
                    safe_l2 = np.where(l2 > 0, l2, 1.0)
                    p = np.where(l2 > 0, e / safe_l2, 0.0)
                    o = o * np.where(l2 > 0, l1 / safe_l2, 0.0) * decay + p @ v[b, ks:ke, g, :]
                    m1, l1 = m2, l2
                out[b, qs:qe, h, :] = o
    return out
