"""Host model of the top-K one-read path's arithmetic (CPU only).

The GPU tests compare the kernel with the oracle; these check, on many more
rows and without a GPU, the three pieces of integer arithmetic the one-read
path rests on, written out here in numpy from their description in
head_attention_no_amd/csrc/topk.hpp:

1. The 64-bit candidate word (order key high, (0x7FFFFFFF - index) << 1 plus
   a -0.0 flag low): sorting the words in descending unsigned order gives the
   oracle's result order, and each word gives its value back bit for bit.
2. The sampled bound: each of the 1024 threads takes the largest entry of its
   share of the first full batches (16384-entry batches, float4 j of batch b
   at b*4096 + u*1024 + thread, entries head + 4j .. head + 4j + 3), found as
   the signed-integer max of the raw bits when any is >= 0, else the
   signed-integer min. The 4096-bin histogram bin of their K-th largest key
   bounds the row's K-th largest key from below.
3. The one-compare tests on raw bits that stand for `key >= bound`.
"""
import numpy as np
import pytest
import torch

from head_attention_no_amd import inputs
from oracle import topk as otk


def order_key(bits: np.ndarray) -> np.ndarray:
    u = bits.astype(np.uint32).copy()
    u[u == 0x80000000] = 0
    return np.where(u & 0x80000000, ~u, u | 0x80000000).astype(np.uint32)


def entry_word(bits: np.ndarray, idx: np.ndarray) -> np.ndarray:
    key = order_key(bits).astype(np.uint64)
    low = ((0x7FFFFFFF - idx.astype(np.uint64)) << np.uint64(1)) | (bits == 0x80000000).astype(np.uint64)
    return (key << np.uint64(32)) | low


def word_value_bits(w: np.ndarray) -> np.ndarray:
    key = (w >> np.uint64(32)).astype(np.uint32)
    u = np.where(key & 0x80000000, key & 0x7FFFFFFF, ~key).astype(np.uint32)
    return np.where((w & np.uint64(1)) == 1, np.uint32(0x80000000), u).astype(np.uint32)


def word_index(w: np.ndarray) -> np.ndarray:
    return (0x7FFFFFFF - ((w & np.uint64(0xFFFFFFFF)) >> np.uint64(1))).astype(np.int64)


def rows(kind, B, V, seed):
    x = inputs.make_scores(B, V, kind, seed=seed).numpy()
    if kind == "normal" and seed % 2:
        x = x - 10.0  # all negative
    return x


KINDS = [("frequencies", 3, 70001), ("normal", 3, 50000), ("normal", 3, 40003), ("ties", 2, 33000),
         ("zeros", 2, 20000), ("huge_tiny", 2, 65536)]


@pytest.mark.parametrize("kind,B,V", KINDS)
def test_word_order_is_the_result_order(kind, B, V):
    x = rows(kind, B, V, seed=V)
    bits = x.view(np.uint32)
    K = 64
    ov, oi = otk.topk_rows(x, K)
    for r in range(B):
        w = entry_word(bits[r], np.arange(V))
        assert len(np.unique(w)) == V  # distinct words
        top = np.sort(w)[::-1][:K]
        assert np.array_equal(word_index(top), oi[r])
        assert np.array_equal(word_value_bits(top), ov[r].view(np.uint32))


def thread_maxima(bits_row: np.ndarray, head: int, nfull: int) -> np.ndarray:
    """Raw bits of each thread's largest entry over batches 0 .. nfull-1."""
    body = bits_row[head:].view(np.int32)
    imax = np.full(1024, np.iinfo(np.int32).min, dtype=np.int64)
    imin = np.full(1024, np.iinfo(np.int32).max, dtype=np.int64)
    t = np.arange(1024)
    for b in range(nfull):
        for u in range(4):
            j = b * 4096 + u * 1024 + t
            vals = body[(4 * j)[:, None] + np.arange(4)[None, :]].astype(np.int64)
            imax = np.maximum(imax, vals.max(axis=1))
            imin = np.minimum(imin, vals.min(axis=1))
    return np.where(imax >= 0, imax, imin).astype(np.int64).astype(np.uint32)


def bound_of(maxima_bits: np.ndarray, K: int) -> int:
    bins = order_key(maxima_bits) >> 20
    hist = np.bincount(bins.astype(np.int64), minlength=4096)
    cum = np.cumsum(hist[::-1])
    found = 4095 - int(np.argmax(cum >= K))
    lo = found << 20
    return lo - 1 if found == 2048 else lo


@pytest.mark.parametrize("kind,B,V", KINDS)
@pytest.mark.parametrize("head", [0, 3])
def test_sampled_bound_and_raw_bit_compare(kind, B, V, head):
    x = rows(kind, B, V, seed=V + head)
    bits = x.view(np.uint32)
    nvec = (V - head) // 4
    nfull = min(4, nvec // 4096)
    assert nfull >= 1
    for K in (1, 17, 64):
        for r in range(B):
            m = thread_maxima(bits[r], head, nfull)
            lo = bound_of(m, K)
            keys = order_key(bits[r]).astype(np.int64)
            kth = np.sort(keys)[::-1][K - 1]
            assert kth >= lo, (kind, K, r)  # the row's K-th largest is at or above the bound
            # The raw-bit test used for each entry equals key >= bound.
            want = keys >= lo
            if lo > 0x80000000:
                got = bits[r].view(np.int32).astype(np.int64) >= (lo & 0x7FFFFFFF)
            else:
                got = bits[r].astype(np.int64) <= ((~np.uint32(lo)) & 0xFFFFFFFF)
            assert np.array_equal(got, want), (kind, K, r)


def test_thread_maximum_of_mixed_signs_and_zeros():
    """The integer max/min fold picks the float maximum: positive beats
    negative, -0.0 beats every negative, the negative nearest zero wins
    among negatives."""
    cases = [[-1.0, 2.0, -3.0, 0.5], [-1.0, -0.25, -3.0, -7.0], [-0.0, -1.0, -2.0, -3.0],
             [0.0, -0.0, -1.0, -2.0], [-5e-45, -1e30, -3.0, -2.0]]
    for c in cases:
        b = np.array(c, dtype=np.float32).view(np.int32).astype(np.int64)
        pick = b.max() if b.max() >= 0 else b.min()
        got = np.array([pick], dtype=np.int64).astype(np.uint32).view(np.float32)[0]
        assert order_key(np.array([got]).view(np.uint32))[0] == order_key(
            np.array(c, dtype=np.float32).view(np.uint32)).max()
