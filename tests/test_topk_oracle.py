"""Pins of the top-K oracle (CPU only).

The oracle (oracle/topk.py) is the plain definition. It is pinned here by
what characterises the answer independently of how it is sorted:
  - the selection property: every selected value is >= every value left
    out, the selected values are non-increasing, equal values come in
    ascending index order, and at the cut the lowest-index copies of the
    K-th value are the ones taken (together these fix a unique answer);
  - special cases with known answers (argmax, constant rows, monotone rows,
    K = V as a full descending sort against numpy's sort);
  - permutation equivariance, and -0.0 == +0.0 as a tie.
Planted mistakes (ascending order, ties by the higher index, an entry
dropped, the indices off by one) each fail at least one check.
"""
import numpy as np
import pytest

from oracle import topk as otk


def check_selection(x, k, vals, idx):
    """Assert that (vals, idx) is the unique top-k answer for each row of x."""
    rows, n = x.shape
    assert vals.shape == (rows, k) and idx.shape == (rows, k)
    for r in range(rows):
        row, sel = x[r].astype(np.float64), idx[r]
        assert len(set(sel.tolist())) == k, "indices repeat"
        assert np.all((sel >= 0) & (sel < n)), "index out of range"
        assert np.array_equal(vals[r].view(np.uint32) if vals.dtype == np.float32 else vals[r],
                              x[r, sel].view(np.uint32) if vals.dtype == np.float32 else x[r, sel]), \
            "values are not the input entries at the indices"
        v = row[sel]
        assert np.all(v[:-1] >= v[1:]), "values not in descending order"
        for a in range(k - 1):
            if v[a] == v[a + 1]:
                assert sel[a] < sel[a + 1], "equal values not in ascending index order"
        rest = np.setdiff1d(np.arange(n), sel)
        if len(rest):
            assert row[rest].max() <= v[-1], "a larger value was left out"
            # at the cut: no left-out copy of the K-th value precedes a taken one
            ties_out = rest[row[rest] == v[-1]]
            ties_in = sel[v == v[-1]]
            if len(ties_out):
                assert ties_out.min() > ties_in.max(), "a lower-index tie was left out"


def rand_rows(rows, n, seed, ties=False):
    rng = np.random.default_rng(seed)
    if ties:
        return rng.integers(0, 7, size=(rows, n)).astype(np.float32) / 4
    return rng.standard_normal((rows, n)).astype(np.float32)


@pytest.mark.parametrize("n,k", [(1, 1), (5, 1), (5, 5), (7, 3), (64, 10), (1000, 37), (4099, 1024)])
@pytest.mark.parametrize("ties", [False, True])
def test_selection_property(n, k, ties):
    x = rand_rows(3, n, seed=n * 31 + k, ties=ties)
    vals, idx = otk.topk_rows(x, k)
    check_selection(x, k, vals, idx)


def test_special_cases():
    x = rand_rows(4, 300, seed=1)
    x[1, 17] = x[1, 200] = x[1].max() + 1  # repeated maximum: the first occurrence wins
    vals, idx = otk.topk_rows(x, 1)
    assert np.array_equal(idx[:, 0], np.argmax(x, axis=1))
    c = np.full((2, 50), 0.25, dtype=np.float32)
    assert np.array_equal(otk.topk_rows(c, 20)[1], np.tile(np.arange(20), (2, 1)))
    inc = np.arange(40, dtype=np.float32)[None, :]
    assert np.array_equal(otk.topk_rows(inc, 40)[1][0], np.arange(39, -1, -1))
    full_vals, _ = otk.topk_rows(x, 300)
    assert np.array_equal(full_vals, -np.sort(-x, axis=1))


def test_permutation_equivariance():
    rng = np.random.default_rng(5)
    x = rng.permutation(1000).astype(np.float32)[None, :] / 7  # distinct values
    perm = rng.permutation(1000)
    _, idx = otk.topk_rows(x, 25)
    _, idx_p = otk.topk_rows(x[:, perm], 25)
    assert np.array_equal(perm[idx_p[0]], idx[0])


def test_signed_zeros_are_equal_values():
    x = np.array([[0.0, -0.0, 0.0, -1.0, -0.0]], dtype=np.float32)
    vals, idx = otk.topk_rows(x, 4)
    assert idx[0].tolist() == [0, 1, 2, 4]
    assert np.signbit(vals[0]).tolist() == [False, True, False, True]


def _mutant(kind):
    def f(x, k):
        vals, idx = otk.topk_rows(x, k)
        if kind == "ascending":
            order = np.argsort(x, axis=1, kind="stable")[:, :k]
            return np.take_along_axis(x, order, axis=1), order
        if kind == "ties_high_first":
            out = []
            for r in range(x.shape[0]):
                o = np.lexsort((-np.arange(x.shape[1]), -x[r].astype(np.float64)))[:k]
                out.append(o)
            o = np.array(out)
            return np.take_along_axis(x, o, axis=1), o
        if kind == "drop_last_entry":
            o = np.array([np.lexsort((np.arange(x.shape[1] - 1), -x[r, :-1].astype(np.float64)))[:k]
                          for r in range(x.shape[0])])
            return np.take_along_axis(x, o, axis=1), o
        if kind == "index_off_by_one":
            return vals, np.minimum(idx + 1, x.shape[1] - 1)
        raise ValueError(kind)
    return f


@pytest.mark.parametrize("kind", ["ascending", "ties_high_first", "drop_last_entry", "index_off_by_one"])
def test_planted_mistakes_are_caught(kind):
    caught = False
    for ties in (False, True):
        x = rand_rows(3, 200, seed=9, ties=ties)
        x[:, -1] = x.max() + 1  # the last entry is the largest
        vals, idx = _mutant(kind)(x, 12)
        try:
            check_selection(x, 12, vals, idx)
        except AssertionError:
            caught = True
    assert caught, f"mutant {kind} passed the checks"
