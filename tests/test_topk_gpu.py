"""Top-K ordering on the GPU vs the oracle, through the C ABI: bit-exact
values and indices (the selection is exact integer-like work)."""
import numpy as np
import pytest
import torch

import head_attention_no_amd as fa
from head_attention_no_amd import inputs
from oracle import topk as otk

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def note(msg):
    print(msg, flush=True)


def run(x, k):
    vals, idx = fa.topk(x.to(DEV), k)
    torch.cuda.synchronize()
    return vals.cpu().numpy(), idx.cpu().numpy()


def check(x, k):
    vals, idx = run(x, k)
    ov, oi = otk.topk_rows(x.numpy(), k)
    assert np.array_equal(idx, oi), f"indices differ in rows {np.nonzero((idx != oi).any(1))[0][:5]}"
    assert np.array_equal(vals.view(np.uint32), ov.view(np.uint32)), "values differ"


CASES = [
    # rows, entries, k, kind
    (3, 5, 5, "frequencies"),       # the page's demo shape: three rows, whole rows ordered
    (1, 1, 1, "normal"),
    (4, 1000, 37, "normal"),
    (2, 4099, 1024, "normal"),      # ragged row length: rows start at every 16-byte phase
    (3, 4097, 1, "normal"),
    (5, 20000, 50, "ties"),
    (2, 300, 300, "ties"),
    (3, 777, 100, "zeros"),
    (2, 129, 64, "huge_tiny"),
    (64, 50257, 50, "frequencies"),
    # long rows: the single-read path, and its fallback when the bound admits too many
    (3, 100003, 200, "normal"),
    (2, 100003, 10, "ties"),
    (2, 65536, 1024, "huge_tiny"),
    # threshold bins of more than 4096 entries: the multi-pass path
    (2, 20000, 100, "zeros"),
    (2, 50000, 300, "ties"),
    # K <= 64 on rows of 16384 entries or more: the one-read path (rows
    # start at every 16-byte phase; the bound from one to four full
    # batches; up to 256 candidates selected by rank, more by the sort
    # tree), and its hand-over to the paths above when the candidate list
    # overflows (ties, zeros, huge_tiny)
    (3, 100003, 64, "normal"),
    (4, 81923, 1, "normal"),
    (3, 16387, 64, "normal"),       # one full batch and a few vectors
    (2, 32000, 40, "frequencies"),  # one full batch, one partial
    (2, 65537, 17, "ties"),         # four full batches, no fifth; ~1500 tied candidates
    (2, 131071, 33, "frequencies"),
    (2, 200003, 64, "frequencies"),  # about 200 candidates: four chunks ranked
    (2, 90001, 33, "zeros"),
    (2, 98304, 64, "huge_tiny"),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "B{}_V{}_K{}_{}".format(*c))
def test_topk_matches_oracle(case):
    B, V, k, kind = case
    note(f"topk case {case}")
    x = inputs.make_scores(B, V, kind, seed=V + k)
    check(x, k)


def test_topk_negative_rows():
    """All-negative rows: the one-read path's bound is a negative value."""
    x = inputs.make_scores(3, 100001, "normal", seed=11) - 10.0
    check(x, 50)


def test_topk_zeros_among_negatives():
    """A thousand signed zeros among negatives, K = 64: the K-th largest
    is zero, every chosen value ties at zero and the lowest indices win;
    -0.0 comes back bit for bit. About 1000 candidates: the register
    sorts and the merge tree."""
    g = torch.Generator("cpu").manual_seed(5)
    x = -(inputs.make_scores(2, 90000, "normal", seed=12).abs() + 1.0)
    for r in range(2):
        pos = torch.randperm(90000, generator=g)[:1000]
        sign = torch.randint(0, 2, (1000,), generator=g).to(torch.bool)
        x[r, pos] = torch.where(sign, torch.tensor(-0.0), torch.tensor(0.0))
    check(x, 64)


def test_topk_ascending_rows():
    """Increasing rows: the first batches bound nothing away, so the
    candidate list overflows and the row goes to the two-read paths."""
    x = torch.arange(2 * 120000, dtype=torch.float32).view(2, 120000) / 7.0
    check(x, 20)


def test_topk_full_size_workload():
    w = inputs.TOPK_WORKLOAD
    note(f"topk workload {w}")
    x = inputs.make_scores(w["B"], w["V"], w["kind"], seed=w["seed"])
    check(x, w["K"])


def test_topk_deterministic_and_in_bounds():
    x = inputs.make_scores(4, 3000, "ties", seed=3).to(DEV)
    guard = torch.full((4 * 64 + 2048,), -7.0, device=DEV)
    vals = guard[1024:1024 + 4 * 64].view(4, 64)
    iguard = torch.full((4 * 64 + 2048,), -7, dtype=torch.int32, device=DEV)
    idx = iguard[1024:1024 + 4 * 64].view(4, 64)
    fa.topk(x, 64, values=vals, indices=idx)
    first = (vals.clone(), idx.clone())
    fa.topk(x, 64, values=vals, indices=idx)
    torch.cuda.synchronize()
    assert torch.equal(first[0], vals) and torch.equal(first[1], idx)
    assert torch.all(guard[:1024] == -7) and torch.all(guard[-1024:] == -7)
    assert torch.all(iguard[:1024] == -7) and torch.all(iguard[-1024:] == -7)


def test_topk_rejects_through_binding():
    x = torch.zeros(2, 10, device=DEV)
    with pytest.raises(fa.FA355Error) as e:
        fa.topk(x, 11)
    assert e.value.status == fa.ERR_INVALID_ARG
    with pytest.raises(fa.FA355Error) as e:
        fa.topk(torch.zeros(2, 2000, device=DEV), 1025)
    assert e.value.status == fa.ERR_UNSUPPORTED
