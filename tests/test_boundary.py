"""The C-ABI library on the CPU: it loads, exports what fa355.h declares, and
rejects bad arguments before touching HIP. No compute call runs here."""
import os
import re

import pytest

import head_attention_no_amd as fa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa355.h")

# Fake, never-dereferenced addresses: every call below fails validation first.
P1, P2, P3, P4 = 0x10000000, 0x20000000, 0x30000000, 0x40000000


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\(", text, flags=re.M)))


def test_library_exports_every_declared_function():
    names = declared_functions()
    assert names == sorted(fa.EXPORTS), names
    lib = fa.load()
    for n in names:
        assert hasattr(lib, n), f"libfa355.so does not export {n}"


def test_version_and_strerror():
    assert fa.version().startswith("fa355 ")
    for s in range(5):
        assert fa.strerror(s)
    assert fa.strerror(99) == "unknown status"


def call(**over):
    a = dict(out=P1, q=P2, k=P3, v=P4, B=1, S=128, H=4, Hkv=4, D=64, scale=0.125,
             mask_kind=fa.MASK_NONE, window=-1, dtype=fa.BF16, stream=None)
    a.update(over)
    return fa.mha_no_cache(a["out"], a["q"], a["k"], a["v"], a["B"], a["S"], a["H"], a["Hkv"],
                           a["D"], a["scale"], a["mask_kind"], a["window"], a["dtype"],
                           a["stream"])


@pytest.mark.parametrize("over", [
    dict(out=None), dict(q=None), dict(k=None), dict(v=None),
    dict(B=0), dict(S=0), dict(H=0), dict(Hkv=0), dict(D=0), dict(S=-5),
    dict(H=4, Hkv=3), dict(H=2, Hkv=4),
    dict(dtype=3), dict(dtype=-1), dict(mask_kind=3), dict(mask_kind=-1),
    dict(mask_kind=fa.MASK_SLIDING_WINDOW, window=0),
    dict(mask_kind=fa.MASK_SLIDING_WINDOW, window=-1),
    dict(scale=float("nan")), dict(scale=float("inf")),
    dict(scale=3.0e38), dict(scale=-2.4e38),  # |scale| * log2(e) beyond the fp32 range
    dict(out=P2 + 64),                 # out overlaps q
    dict(out=P3 - 32),                 # out runs into k
], ids=lambda d: ",".join(f"{k}={v}" for k, v in d.items()))
def test_invalid_arguments(over):
    assert call(**over) == fa.ERR_INVALID_ARG


@pytest.mark.parametrize("over", [
    dict(D=16), dict(D=96), dict(D=512),
    dict(q=P2 + 2), dict(out=P1 + 8), dict(k=P3 + 4), dict(v=P4 + 1),
    dict(B=1 << 12, S=1 << 17, H=1 << 10, Hkv=1 << 10, out=1 << 47, q=2 << 47, k=3 << 47,
         v=4 << 47),                  # 2^32 workgroups
    dict(H=1 << 17, Hkv=1 << 17, D=128, out=1 << 47, q=2 << 47, k=3 << 47,
         v=4 << 47),                  # one token row of q: 32 MiB
], ids=lambda d: ",".join(f"{k}={v}" for k, v in d.items()))
def test_unsupported_arguments(over):
    assert call(**over) == fa.ERR_UNSUPPORTED


@pytest.mark.parametrize("over", [
    dict(scale=2.3e38), dict(scale=-2.3e38), dict(scale=1e-45), dict(scale=-0.0),
    # K and V of one batch at 4 GiB each (S = 2^20 rows of 16 heads): sizes
    # past 32 bits are accepted; only one token row of q is limited.
    dict(B=1, S=1 << 20, H=16, Hkv=16, D=128, out=1 << 44, q=2 << 44, k=3 << 44, v=4 << 44),
    dict(H=1 << 15, Hkv=1 << 15, D=256, out=1 << 47, q=2 << 47, k=3 << 47,
         v=4 << 47),                  # one token row of q: exactly 16 MiB
], ids=lambda d: ",".join(f"{k}={v}" for k, v in d.items()))
def test_valid_arguments_reach_the_device_check(over):
    """Calls that pass every argument check go on to the device check, which
    fails here (no GPU): validation accepted them. The addresses are fake, so
    this must never run where a device is present."""
    import torch

    if torch.cuda.device_count() > 0:
        pytest.skip("a device is present: the fake addresses would be launched")
    assert call(**over) == fa.ERR_DEVICE


def d256_waves(B, S, H, Hkv, mask):
    """Waves per workgroup of a 16-bit call at D = 256: 8 (32-key tiles)
    when the 8-wave items number at least 512 under a mask or 256 without
    one (two or one per compute unit), else 4."""
    hp = max(x for x in (1, 2, 4, 8) if (H // Hkv) % x == 0)
    items = -(-S // (32 * 8 // hp)) * B * H // hp
    return 8 if items >= (256 if mask == "none" else 512) else 4


@pytest.mark.parametrize("shape", [
    (2, 4096, 32, 8, 128, fa.BF16, "causal", -1),   # groups split over the 8 XCDs; 4 heads packed; walks
    (4, 2048, 32, 32, 128, fa.BF16, "causal", -1),  # MHA: one head per workgroup; walks
    (1, 8192, 32, 8, 128, fa.BF16, "window", 1024),  # walks
    (1, 16384, 32, 8, 128, fa.BF16, "causal", -1),  # long items: no walk
    (1, 16384, 16, 16, 64, fa.F16, "none", -1),
    (1, 128, 4, 4, 64, fa.F32, "none", -1),         # 4 groups: fallback order
    (3, 300, 6, 2, 64, fa.BF16, "causal", -1),      # ragged S, 3 heads per K/V head: no packing
    (1, 300, 6, 2, 128, fa.F16, "causal", -1),      # 2 groups: fallback order, walking
    (1, 1, 1, 1, 128, fa.F16, "none", -1),
    (2, 1000, 8, 2, 32, fa.BF16, "none", -1),       # 4 heads per K/V head
    (1, 777, 8, 8, 256, fa.F16, "none", -1),        # 4-wave workgroups at D = 256
    (1, 300, 4, 2, 256, fa.F32, "none", -1),        # 2 heads packed into a 4-wave workgroup
    (2, 500, 16, 1, 64, fa.BF16, "none", -1),       # 16 heads per K/V head: 8 packed (one per wave)
    (1, 640, 32, 4, 128, fa.F32, "none", -1),       # 8 heads per K/V head, 4-wave workgroups: 4 packed
    (2, 96, 12, 6, 256, fa.BF16, "none", -1),       # 2 packed at D = 256
    (2, 4096, 16, 16, 256, fa.BF16, "causal", -1),  # D = 256, 512 causal items: 8-wave layout
    (4, 1024, 16, 16, 256, fa.F16, "causal", -1),   # 256 causal items: 4-wave layout
    (2, 2048, 16, 16, 256, fa.BF16, "none", -1),    # 256 unmasked items: 8-wave layout
    (1, 8192, 16, 4, 256, fa.BF16, "sliding_window", 1024),  # 4 packed, 512 items
])
def test_plan_covers_every_tile_once(shape):
    B, S, H, Hkv, D, dt, mask, window = shape
    pl = fa.plan(B, S, H, Hkv, D, dt, mask, window, with_tiles=True)
    waves = 4 if dt == fa.F32 else d256_waves(B, S, H, Hkv, mask) if D == 256 else 8
    hp = max(x for x in (1, 2, 4, 8) if x <= waves and (H // Hkv) % x == 0)
    # fp32 calls with at most 256 items of 32 rows split the keys over the
    # waves of a 32-row, one-head workgroup (head dims up to 64).
    split = dt == fa.F32 and D <= 64 and -(-S // 32) * B * H <= 256
    if split:
        hp, waves = 1, 1
    assert pl["heads_per_workgroup"] == hp
    assert pl["block_m"] == 32 * waves // hp
    assert pl["block_n"] == (32 if dt == fa.F32 else {32: 128, 64: 64, 128: 64, 256: 64 if waves == 4 else 32}[D])
    nq = -(-S // pl["block_m"])
    assert pl["num_workgroups"] == nq * B * H // hp
    tiles = pl["tiles"]
    assert sorted(tiles) == sorted((t, b, h) for t in range(nq) for b in range(B)
                                   for h in range(0, H, hp))
    groups = B * Hkv
    group_order = pl["walk"] or (mask == "none" and dt != fa.F32)
    if group_order and groups % 8 == 0:
        # Group order: on each XCD (item w on XCD w % 8), group after group,
        # each group's query tiles longest first.
        per_group = nq * (H // Hkv // hp)
        for x in range(8):
            seq = tiles[x::8]
            for i in range(0, len(seq), per_group):
                block = seq[i:i + per_group]
                assert len({(b, h // (H // Hkv)) for _, b, h in block}) == 1
                qts = [t for t, _, _ in block]
                assert qts == sorted(qts, reverse=True)
    else:
        # Longest (last) query tiles are dispatched first.
        first = tiles[:min(len(tiles), B * H // hp)]
        assert all(t == nq - 1 for t, _, _ in first)


@pytest.mark.parametrize("shape,walk", [
    ((2, 4096, 32, 8, 128, fa.BF16, "causal", -1), 1),
    ((4, 2048, 32, 32, 128, fa.BF16, "causal", -1), 1),
    ((1, 8192, 32, 8, 128, fa.BF16, "window", 1024), 1),
    ((1, 16384, 32, 8, 128, fa.BF16, "causal", -1), 0),
    ((1, 8192, 32, 8, 128, fa.BF16, "none", -1), 0),
    ((1, 8192, 32, 8, 128, fa.F32, "window", 1024), 0),
    ((4, 8192, 16, 16, 32, fa.BF16, "causal", -1), 0),
    ((1, 16384, 16, 16, 64, fa.F16, "none", -1), 0),
    ((2, 4096, 32, 8, 64, fa.BF16, "causal", -1), 1),
    ((1, 8192, 32, 8, 64, fa.F16, "window", 1000), 1),
    ((2, 4096, 16, 16, 256, fa.BF16, "causal", -1), 0),
])
def test_plan_walks_short_items_at_d64_d128(shape, walk):
    assert fa.plan(*shape)["walk"] == walk


@pytest.mark.parametrize("mask", ["none", "causal"])
def test_plan_keeps_shared_kv_heads_on_one_xcd(mask):
    B, S, H, Hkv = 2, 4096, 32, 8
    tiles = fa.plan(B, S, H, Hkv, 128, fa.BF16, mask, with_tiles=True)["tiles"]
    xcd_of_group = {}
    for w, (_, b, h) in enumerate(tiles):
        grp = (b, h // (H // Hkv))
        xcd_of_group.setdefault(grp, set()).add(w % 8)
    assert all(len(x) == 1 for x in xcd_of_group.values())
    # every XCD receives the same number of groups
    counts = {}
    for x in xcd_of_group.values():
        counts[next(iter(x))] = counts.get(next(iter(x)), 0) + 1
    assert sorted(counts) == list(range(8)) and len(set(counts.values())) == 1


def test_plan_rejects_like_the_entry_point():
    with pytest.raises(fa.FA355Error):
        fa.plan(1, 128, 4, 3, 64, fa.BF16)
    for D in (16, 48, 96, 512):
        with pytest.raises(fa.FA355Error):
            fa.plan(1, 128, 4, 4, D, fa.BF16)
    for mask, window in (("window", 0), (7, 1)):
        with pytest.raises(fa.FA355Error):
            fa.plan(1, 128, 4, 4, 64, fa.BF16, mask, window)


def test_missing_library_fails_loudly(tmp_path):
    with pytest.raises(RuntimeError, match="missing"):
        fa.load(str(tmp_path / "libfa355.so"))


def topk_call(**over):
    a = dict(values=P1, indices=P2, x=P3, B=2, V=100, K=10, stream=None)
    a.update(over)
    return fa.fa355_topk(a["values"], a["indices"], a["x"], a["B"], a["V"], a["K"], a["stream"])


@pytest.mark.parametrize("over", [
    dict(values=0), dict(indices=0), dict(x=0), dict(B=0), dict(V=0), dict(K=0), dict(K=101),
    dict(values=P3 + 40), dict(indices=P3 - 4), dict(indices=P1 + 76),
], ids=lambda d: ",".join(f"{k}={v}" for k, v in d.items()))
def test_topk_invalid_arguments(over):
    assert topk_call(**over) == fa.ERR_INVALID_ARG


@pytest.mark.parametrize("over", [dict(V=5000, K=1025), dict(x=P3 + 2), dict(values=P1 + 1)],
                         ids=lambda d: ",".join(f"{k}={v}" for k, v in d.items()))
def test_topk_unsupported_arguments(over):
    assert topk_call(**over) == fa.ERR_UNSUPPORTED
