"""The fp64 oracle against its pins (CPU only)."""
import numpy as np
import pytest

import oracle
import pins


@pytest.fixture(scope="module")
def orc():
    return oracle.default()


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(orc, pin):
    pin(orc)


def test_golden_cases_through_recurrences():
    """The hand-derived cases also hold for the pages' tiled recurrences."""
    from oracle import online_softmax

    for c in pins.golden_cases():
        for bm, bn in ((1, 1), (2, 1), (1, 2), (3, 3)):
            for fn in (online_softmax.fa2_deferred, online_softmax.fa_stepwise):
                got = fn(c["q"], c["k"], c["v"], c["scale"], c["mask"], c["window"], bm, bn)
                err = np.max(np.abs(got - c["expected"]))
                assert err <= c["tol"], (c["name"], fn.__name__, bm, bn, err)


def test_rejects_invalid_arguments(orc):
    q, k, v = pins.rand_qkv(1, 4, 4, 2, 8, 0)
    with pytest.raises(ValueError):
        orc.attention(q, k, v, 1.0, "sliding_window", 0)  # a window needs width >= 1
    with pytest.raises(ValueError):
        orc.attention(q, k, v, 1.0, 7)  # unknown mask kind
    q3, k3, v3 = pins.rand_qkv(1, 4, 4, 3, 8, 0)  # 4 query heads cannot share 3 K/V heads
    with pytest.raises(ValueError):
        orc.attention(q3, k3, v3, 1.0, "none")
    with pytest.raises(ValueError):
        orc.attention_rows(q, k, v, 1.0, "none", -1, [(0, 0, 4)])  # row out of range


def test_window_pair_count_of_long_context_workload(orc):
    """Sliding window 1024 over 8192 tokens: every query sees min(i+1, 1024) keys."""
    assert orc.visible_pairs(8192, "sliding_window", 1024) == 7_864_832
