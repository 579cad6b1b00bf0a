"""Checks that pin the fp64 oracle to facts other than itself.

Each ``pin_*`` function takes an ``oracle.Oracle`` and raises AssertionError
when the oracle disagrees with:
  - a hand-derived worked example (tests/golden/closed_form_cases.json);
  - an independent library routine (torch's scaled_dot_product_attention,
    fp64 on the CPU, with grouped K/V made explicit by head repetition);
  - a closed form (mean of the visible values when every score is equal,
    causal row 0 = v0, window 1 = identity, window >= S = causal);
  - an invariance of the mathematics (constant key shift, joint key/value
    permutation, query permutation, linearity in V, rows of P summing to 1);
  - the pages' own tiled online-softmax recurrences at every tile size.

The same pins run against deliberately broken builds of the oracle
(test_oracle_mutants.py), each of which must fail at least one of them.
"""
from __future__ import annotations

import json
import math
import os

import numpy as np
import torch

from oracle import online_softmax

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden",
                      "closed_form_cases.json")


def _val(expr: str) -> float:
    return float(eval(expr, {"__builtins__": {}}, {"ln": math.log}))  # noqa: S307 - fixed fixture


def golden_cases():
    with open(GOLDEN) as f:
        data = json.load(f)
    cases = []
    for c in data["cases"]:
        B, S, H, Hkv, D = c["B"], c["S"], c["H"], c["Hkv"], c["D"]
        cases.append(dict(
            name=c["name"],
            q=np.array([_val(x) for x in c["q"]]).reshape(B, S, H, D),
            k=np.array([_val(x) for x in c["k"]]).reshape(B, S, Hkv, D),
            v=np.array([_val(x) for x in c["v"]]).reshape(B, S, Hkv, D),
            scale=_val(c["scale"]), mask=c["mask"], window=c["window"],
            expected=np.array([_val(x) for x in c["expected"]]).reshape(B, S, H, D),
            tol=c.get("tol", 1e-12)))
    return cases


def rand_qkv(B, S, H, Hkv, D, seed):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((B, S, H, D)), rng.standard_normal((B, S, Hkv, D)),
            rng.standard_normal((B, S, Hkv, D)))


def sdpa_fp64(q, k, v, scale, mask, window):
    """torch's scaled_dot_product_attention in fp64 on the CPU, BSHD in and out."""
    H, Hkv = q.shape[2], k.shape[2]
    qt = torch.from_numpy(q).permute(0, 2, 1, 3)
    kt = torch.from_numpy(k).repeat_interleave(H // Hkv, dim=2).permute(0, 2, 1, 3)
    vt = torch.from_numpy(v).repeat_interleave(H // Hkv, dim=2).permute(0, 2, 1, 3)
    S = q.shape[1]
    attn_mask, causal = None, False
    if mask == "causal":
        causal = True
    elif mask == "sliding_window":
        i = torch.arange(S)[:, None]
        j = torch.arange(S)[None, :]
        attn_mask = (j <= i) & (j > i - window)
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=attn_mask,
                                                         is_causal=causal, scale=scale)
    return o.permute(0, 2, 1, 3).numpy()


def _close(a, b, tol, what):
    a = np.asarray(a)
    b = np.asarray(b)
    assert a.shape == b.shape, f"{what}: shape {a.shape} vs {b.shape}"
    err = np.max(np.abs(a - b)) if a.size else 0.0
    assert np.all(np.isfinite(a)) and err <= tol, f"{what}: max abs err {err} > {tol}"


MASKS = [("none", -1), ("causal", -1), ("sliding_window", 5)]


def pin_golden(orc):
    for c in golden_cases():
        out = orc.attention(c["q"], c["k"], c["v"], c["scale"], c["mask"], c["window"])
        _close(out, c["expected"], c["tol"], f"golden {c['name']}")
        B, S, H, _ = c["q"].shape
        rows = [(b, h, i) for b in range(B) for h in range(H) for i in range(S)]
        got = orc.attention_rows(c["q"], c["k"], c["v"], c["scale"], c["mask"], c["window"], rows)
        want = np.stack([c["expected"][b, i, h] for b, h, i in rows])
        _close(got, want, c["tol"], f"golden rows {c['name']}")


def pin_sdpa():
    shapes = [(1, 17, 2, 2, 8), (2, 24, 4, 2, 16), (1, 33, 6, 3, 5), (1, 9, 4, 1, 32)]
    for n, (B, S, H, Hkv, D) in enumerate(shapes):
        for mask, window in MASKS + [("sliding_window", 1), ("sliding_window", 40)]:
            yield (B, S, H, Hkv, D, mask, window, 0.37 + 0.1 * n, 10 * n + len(mask))


def pin_vs_sdpa(orc):
    for B, S, H, Hkv, D, mask, window, scale, seed in pin_sdpa():
        q, k, v = rand_qkv(B, S, H, Hkv, D, seed)
        _close(orc.attention(q, k, v, scale, mask, window), sdpa_fp64(q, k, v, scale, mask, window),
               1e-12, f"sdpa B{B} S{S} H{H}/{Hkv} D{D} {mask} W{window}")


def pin_rows_match_whole(orc):
    q, k, v = rand_qkv(2, 21, 4, 2, 8, 7)
    for mask, window in MASKS:
        whole = orc.attention(q, k, v, 0.5, mask, window)
        rows = [(b, h, i) for b in range(2) for h in range(4) for i in (0, 5, 20)]
        got = orc.attention_rows(q, k, v, 0.5, mask, window, rows)
        _close(got, np.stack([whole[b, i, h] for b, h, i in rows]), 0.0, f"rows {mask}")


def pin_values_one(orc):
    q, k, v = rand_qkv(2, 19, 4, 2, 8, 11)
    for mask, window in MASKS:
        out = orc.attention(q, k, np.ones_like(v), 0.9, mask, window)
        _close(out, np.ones_like(out), 1e-13, f"V=1 {mask}")


def _visible_mean(v, H, mask, window):
    """Mean of the visible values per query row when every score is equal."""
    B, S, Hkv, D = v.shape
    rep = H // Hkv
    out = np.empty((B, S, H, D))
    csum = np.concatenate([np.zeros((B, 1, Hkv, D)), np.cumsum(v, axis=1)], axis=1)
    for i in range(S):
        if mask == "none":
            lo, hi = 0, S
        elif mask == "causal":
            lo, hi = 0, i + 1
        else:
            lo, hi = max(0, i - window + 1), i + 1
        mean = (csum[:, hi] - csum[:, lo]) / (hi - lo)
        out[:, i] = np.repeat(mean, rep, axis=1)
    return out


def pin_equal_scores_mean(orc):
    q, k, v = rand_qkv(2, 23, 6, 3, 8, 13)
    for mask, window in MASKS + [("sliding_window", 1), ("sliding_window", 50)]:
        want = _visible_mean(v, 6, mask, window)
        _close(orc.attention(q, k, v, 0.0, mask, window), want, 1e-13, f"scale=0 {mask} W{window}")
        same_k = np.broadcast_to(k[:, :1], k.shape).copy()
        _close(orc.attention(q, same_k, v, 1.3, mask, window), want, 1e-13,
               f"identical keys {mask} W{window}")


def pin_mask_special_cases(orc):
    q, k, v = rand_qkv(2, 16, 4, 2, 8, 17)
    rep = 2
    causal = orc.attention(q, k, v, 0.7, "causal")
    _close(causal[:, 0], np.repeat(v[:, 0], rep, axis=1), 1e-15, "causal row 0 = v0")
    win1 = orc.attention(q, k, v, 0.7, "sliding_window", 1)
    _close(win1, np.repeat(v, rep, axis=2), 1e-15, "window 1 = V")
    for w in (16, 17, 1000):
        _close(orc.attention(q, k, v, 0.7, "sliding_window", w), causal, 0.0, f"window {w} = causal")
    nomask = orc.attention(q, k, v, 0.7, "none")
    _close(causal[:, -1], nomask[:, -1], 1e-14, "causal last row = unmasked last row")


def pin_grouped_equals_repeated(orc):
    q, k, v = rand_qkv(2, 14, 6, 2, 8, 19)
    for mask, window in MASKS:
        grouped = orc.attention(q, k, v, 0.6, mask, window)
        rep = orc.attention(q, np.repeat(k, 3, axis=2), np.repeat(v, 3, axis=2), 0.6, mask, window)
        _close(grouped, rep, 0.0, f"grouped = repeated {mask}")


def pin_key_shift(orc):
    q, k, v = rand_qkv(1, 20, 2, 2, 8, 23)
    u = np.random.default_rng(5).standard_normal(8) * 120.0  # q.u reaches several hundred
    for mask, window in MASKS:
        a = orc.attention(q, k, v, 1.0, mask, window)
        b = orc.attention(q, k + u, v, 1.0, mask, window)
        _close(a, b, 1e-9, f"key shift {mask}")


def pin_permutations(orc):
    q, k, v = rand_qkv(1, 18, 4, 2, 8, 29)
    base = orc.attention(q, k, v, 0.8, "none")
    perm = np.random.default_rng(3).permutation(18)
    _close(orc.attention(q, k[:, perm], v[:, perm], 0.8, "none"), base, 1e-13, "key/value permutation")
    _close(orc.attention(q[:, perm], k, v, 0.8, "none"), base[:, perm], 1e-15, "query permutation")


def pin_linear_in_values(orc):
    q, k, v = rand_qkv(1, 15, 2, 1, 8, 31)
    v2 = np.random.default_rng(9).standard_normal(v.shape)
    for mask, window in MASKS:
        a = orc.attention(q, k, v + v2, 0.5, mask, window)
        b = orc.attention(q, k, v, 0.5, mask, window) + orc.attention(q, k, v2, 0.5, mask, window)
        _close(a, b, 1e-13, f"linearity {mask}")


def pin_probabilities(orc):
    S, D = 12, 16  # S <= D so one-hot values expose every probability
    q, k, _ = rand_qkv(1, S, 2, 1, D, 37)
    onehot = np.zeros((1, S, 1, D))
    for j in range(S):
        onehot[0, j, 0, j] = 1.0
    for mask, window in MASKS:
        out = orc.attention(q, k, onehot, 0.9, mask, window)
        for h in range(2):
            for i in range(S):
                p = orc.probs(q, k, 0.9, mask, window, 0, h, i)
                j = np.arange(S)
                vis = np.ones(S, bool) if mask == "none" else (j <= i)
                if mask == "sliding_window":
                    vis &= j > i - window
                assert np.all(p[~vis] == 0.0), f"hidden keys must get p = 0 ({mask})"
                assert np.all(p[vis] > 0.0), f"visible keys must get p > 0 ({mask})"
                _close(p.sum(), 1.0, 1e-14, f"row sum {mask}")
                _close(out[0, i, h, :S], p, 1e-15, f"one-hot V extracts p {mask}")


def pin_recurrences(orc):
    q, k, v = rand_qkv(1, 13, 4, 2, 4, 41)
    for mask, window in MASKS:
        want = orc.attention(q, k, v, 0.75, mask, window)
        for t in range(1, 14):
            for bm, bn in ((t, t), (t, 14 - t)):
                got = online_softmax.fa2_deferred(q, k, v, 0.75, mask, window, bm, bn)
                _close(got, want, 1e-13, f"FA-2 recurrence {mask} tiles {bm}x{bn}")
                got = online_softmax.fa_stepwise(q, k, v, 0.75, mask, window, bm, bn)
                _close(got, want, 1e-13, f"stepwise recurrence {mask} tiles {bm}x{bn}")


def pin_visible_pairs(orc):
    for S in (1, 7, 128):
        assert orc.visible_pairs(S, "none") == S * S
        assert orc.visible_pairs(S, "causal") == S * (S + 1) // 2
        for W in (1, 3, S, S + 5):
            w = min(W, S)
            assert orc.visible_pairs(S, "sliding_window", W) == S * w - w * (w - 1) // 2


ALL_PINS = [pin_golden, pin_vs_sdpa, pin_rows_match_whole, pin_values_one, pin_equal_scores_mean,
            pin_mask_special_cases, pin_grouped_equals_repeated, pin_key_shift, pin_permutations,
            pin_linear_in_values, pin_probabilities, pin_recurrences, pin_visible_pairs]
