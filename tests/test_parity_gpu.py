"""HIP path vs the fp64 oracle, element by element, through the C ABI.

Tolerances (against the fp64 oracle on the same rounded inputs):
  fp32 inputs:       max |err| <= 1e-4
  bf16/fp16 inputs:  max |err| <= 2e-2 and mean |err| <= 2e-3
"""
import math

import numpy as np
import pytest
import torch

import head_attention_no_amd as fa
import oracle
from head_attention_no_amd import inputs

pytestmark = pytest.mark.gpu

TOL = {"f32": (1e-4, 1e-4), "bf16": (2e-2, 2e-3), "f16": (2e-2, 2e-3)}
DEV = "cuda:0"


def note(msg):
    print(msg, flush=True)


def run_gpu(q, k, v, scale, mask, window):
    out = fa.attention(q.to(DEV), k.to(DEV), v.to(DEV), scale, mask, window)
    torch.cuda.synchronize()
    return out.cpu()


def check(got, want, dtype, what):
    got = got.to(torch.float64).numpy()
    err = np.abs(got - want)
    mx_tol, mean_tol = TOL[dtype]
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    worst = np.unravel_index(np.argmax(err), err.shape)
    assert err.max() <= mx_tol, f"{what}: max err {err.max():.3e} at {worst}"
    assert err.mean() <= mean_tol, f"{what}: mean err {err.mean():.3e}"
    return err.max(), err.mean()


SMALL = [
    # B, S, H, Hkv, D, dtype, mask, window
    (1, 128, 4, 4, 64, "f32", "none", -1),
    (1, 1, 2, 1, 64, "bf16", "causal", -1),
    (1, 1, 1, 1, 128, "f16", "none", -1),
    (2, 37, 4, 2, 64, "bf16", "none", -1),
    (1, 200, 4, 4, 128, "bf16", "causal", -1),
    (2, 300, 6, 2, 128, "bf16", "causal", -1),
    (1, 300, 8, 1, 128, "f16", "causal", -1),
    (1, 257, 4, 4, 64, "f16", "none", -1),
    (1, 513, 4, 2, 64, "bf16", "causal", -1),
    (1, 300, 4, 2, 128, "bf16", "sliding_window", 1),
    (1, 300, 4, 2, 128, "bf16", "sliding_window", 17),
    (1, 400, 4, 1, 128, "bf16", "sliding_window", 100),
    (1, 390, 4, 4, 64, "f16", "sliding_window", 129),
    (1, 300, 4, 4, 128, "f16", "sliding_window", 5000),
    (1, 300, 4, 2, 128, "f32", "none", -1),
    (1, 300, 4, 2, 128, "f32", "causal", -1),
    (1, 275, 4, 4, 64, "f32", "sliding_window", 40),
    (2, 160, 4, 2, 64, "f32", "causal", -1),
    # head dims 32 and 256
    (1, 1, 1, 1, 32, "f16", "none", -1),
    (2, 300, 4, 2, 32, "bf16", "causal", -1),
    (1, 513, 4, 4, 32, "f16", "none", -1),
    (1, 400, 4, 1, 32, "bf16", "sliding_window", 77),
    (1, 300, 4, 2, 32, "f32", "causal", -1),
    (1, 1, 2, 1, 256, "bf16", "causal", -1),
    (2, 300, 4, 2, 256, "bf16", "causal", -1),
    (1, 257, 4, 4, 256, "f16", "none", -1),
    (1, 400, 4, 2, 256, "bf16", "sliding_window", 100),
    (1, 300, 4, 2, 256, "f32", "causal", -1),
    (1, 130, 2, 2, 256, "f32", "sliding_window", 9),
    # several query heads per workgroup (they share one K/V head)
    (2, 333, 16, 1, 64, "bf16", "causal", -1),              # 8 heads packed, 32 rows each
    (1, 200, 8, 1, 64, "f32", "causal", -1),                # 4 packed in the fp32 kernel
    (1, 300, 8, 2, 256, "bf16", "sliding_window", 60),      # 4 packed at D = 256
    (1, 257, 4, 2, 32, "f16", "sliding_window", 31),        # 2 packed at D = 32
    (1, 1000, 8, 1, 128, "bf16", "sliding_window", 200),    # 8 packed, window
    (1, 400, 12, 2, 128, "bf16", "causal", -1),             # 6 per K/V head: 2 packed
    (3, 33, 8, 2, 128, "f16", "none", -1),                  # S below one 64-row tile
    # group sizes that no packing divides evenly, many batches of tiny S
    (1, 300, 12, 4, 64, "bf16", "causal", -1),              # 3 query heads per K/V head: no packing
    (1, 257, 10, 2, 128, "f16", "sliding_window", 33),      # 5 per K/V head
    (2, 190, 6, 2, 256, "f16", "causal", -1),               # 3 per K/V head at D = 256
    (16, 7, 8, 2, 64, "bf16", "none", -1),                  # 16 batches of 7 rows
    (3, 129, 12, 3, 32, "f16", "sliding_window", 64),       # 4 per K/V head at D = 32
    (2, 75, 6, 3, 64, "f32", "causal", -1),                 # fp32, 2 per K/V head, ragged
]


@pytest.mark.parametrize("case", SMALL, ids=lambda c: "B{}_S{}_H{}kv{}_D{}_{}_{}_W{}".format(*c))
def test_small_whole_output(case):
    B, S, H, Hkv, D, dt, mask, window = case
    seed = 7 + S + 3 * H + D
    note(f"case {case} seed {seed}")
    q, k, v = inputs.make_qkv(B, S, H, Hkv, D, dt, seed)
    scale = 1.0 / math.sqrt(D)
    got = run_gpu(q, k, v, scale, mask, window)
    want = oracle.attention(q, k, v, scale, mask, window)
    check(got, want, dt, str(case))


def test_workload_small_fp32_whole_output():
    w = inputs.WORKLOADS[0]
    note(f"workload {w.name}")
    q, k, v = inputs.workload_qkv(w)
    got = run_gpu(q, k, v, w.scale, w.mask, w.window)
    want = oracle.attention(q, k, v, w.scale, w.mask, w.window)
    mx, mean = check(got, want, w.dtype, w.name)
    note(f"  max {mx:.3e} mean {mean:.3e}")


@pytest.mark.timeout(600)
@pytest.mark.parametrize("w", inputs.WORKLOADS[1:], ids=lambda w: w.name)
def test_workload_whole_output(w):
    """The four full-size workloads, launched exactly as the benchmark
    launches them, against the fp64 oracle over every output element: max
    and mean absolute error over the whole output."""
    note(f"workload {w.name} (whole output)")
    q, k, v = inputs.workload_qkv(w)
    got = run_gpu(q, k, v, w.scale, w.mask, w.window)
    want = oracle.attention(q, k, v, w.scale, w.mask, w.window)
    err = np.abs(got.to(torch.float64).numpy() - want)
    worst = np.unravel_index(np.argmax(err), err.shape)
    note(f"  {err.size} elements: max {err.max():.3e} at (b, s, h, d) = {tuple(int(x) for x in worst)}, "
         f"mean {err.mean():.3e}")
    mx, mean = check(got, want, w.dtype, w.name)


def sample_rows(w, n_heads=6, seed=0):
    """(b, h, i) triples: tile edges, both ends, and random rows of a few heads."""
    rng = np.random.default_rng(seed)
    heads = {(0, 0), (w.B - 1, w.H - 1)}
    while len(heads) < min(n_heads, w.B * w.H):
        heads.add((int(rng.integers(w.B)), int(rng.integers(w.H))))
    fixed = {0, 1, 31, 32, 63, 64, 127, 128, 129, w.S // 2, w.S - 129, w.S - 128, w.S - 2, w.S - 1}
    rows = []
    for b, h in sorted(heads):
        idx = sorted({i for i in fixed if 0 <= i < w.S} | set(rng.integers(0, w.S, 24).tolist()))
        rows += [(b, h, i) for i in idx]
    return rows


@pytest.mark.parametrize("w", inputs.WIDER, ids=lambda w: w.name)
def test_workload_full_size_sampled_rows(w):
    """Full-size workloads, launched exactly as the benchmark launches them;
    the oracle recomputes a sample of rows one by one."""
    note(f"workload {w.name}")
    q, k, v = inputs.workload_qkv(w)
    got = run_gpu(q, k, v, w.scale, w.mask, w.window)
    assert torch.isfinite(got.float()).all()
    rows = sample_rows(w)
    want = oracle.attention_rows(q, k, v, w.scale, w.mask, w.window, rows)
    got_rows = torch.stack([got[b, i, h] for b, h, i in rows])
    mx, mean = check(got_rows, want, w.dtype, w.name)
    note(f"  {len(rows)} rows: max {mx:.3e} mean {mean:.3e}")


def _dev(*ts):
    return [t.to(DEV) for t in ts]


@pytest.mark.parametrize("dt", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("mask,window", [("none", -1), ("causal", -1), ("sliding_window", 33)])
def test_values_one_give_one(dt, mask, window):
    q, k, v = inputs.make_qkv(1, 300, 4, 2, 128, dt, seed=3)
    note(f"V=1 {dt} {mask}")
    q, k, v = _dev(q, k, torch.ones_like(v))
    out = fa.attention(q, k, v, 0.2, mask, window).float()
    assert torch.allclose(out, torch.ones_like(out), atol=TOL[dt][0], rtol=0)


@pytest.mark.parametrize("mask,window", [("none", -1), ("causal", -1), ("sliding_window", 70)])
def test_scale_zero_is_mean_of_visible_values(mask, window):
    q, k, v = inputs.make_qkv(2, 333, 4, 2, 64, "f32", seed=4)
    note(f"scale=0 {mask}")
    got = run_gpu(q, k, v, 0.0, mask, window)
    want = oracle.attention(q, k, v, 0.0, mask, window)
    check(got, want, "f32", f"scale 0 {mask}")


def test_negative_scale():
    q, k, v = inputs.make_qkv(1, 260, 4, 2, 128, "bf16", seed=5)
    got = run_gpu(q, k, v, -0.3, "causal", -1)
    check(got, oracle.attention(q, k, v, -0.3, "causal", -1), "bf16", "negative scale")


def test_mask_special_cases():
    q, k, v = inputs.make_qkv(1, 300, 4, 2, 128, "bf16", seed=6)
    qd, kd, vd = _dev(q, k, v)
    causal = fa.attention(qd, kd, vd, 0.1, "causal").cpu()
    assert torch.equal(causal[:, 0], v[:, 0].repeat_interleave(2, dim=1))
    w1 = fa.attention(qd, kd, vd, 0.1, "sliding_window", 1).cpu()
    assert torch.equal(w1, v.repeat_interleave(2, dim=2))
    for W in (300, 301, 10 ** 6):
        wide = fa.attention(qd, kd, vd, 0.1, "sliding_window", W).cpu()
        assert torch.equal(wide, causal), f"window {W} must equal causal"


@pytest.mark.parametrize("mask,window", [("none", -1), ("causal", -1), ("sliding_window", 50)])
def test_grouped_equals_repeated_heads(mask, window):
    q, k, v = inputs.make_qkv(2, 200, 8, 2, 128, "bf16", seed=8)
    qd, kd, vd = _dev(q, k, v)
    grouped = fa.attention(qd, kd, vd, 0.1, mask, window)
    rep = fa.attention(qd, kd.repeat_interleave(4, dim=2).contiguous(),
                       vd.repeat_interleave(4, dim=2).contiguous(), 0.1, mask, window)
    assert torch.equal(grouped, rep)


@pytest.mark.parametrize("dt", ["f32", "bf16", "f16"])
def test_key_shift_large_scores(dt):
    """A constant vector added to every key shifts each score row by a
    constant of several hundred, which the running max must absorb (a
    softmax without the max subtraction overflows). Both sides get the same
    shifted keys, rounded to the input dtype."""
    q, k, v = inputs.make_qkv(1, 260, 2, 2, 64, dt, seed=9)
    u = torch.randn(64, generator=torch.Generator().manual_seed(1)) * 60.0
    ks = (k.float() + u).to(k.dtype)
    shift = (q.double()[0, :, 0] @ u.double()) / 8
    assert shift.abs().max() > 200, "the case must shift some score rows by hundreds"
    got = run_gpu(q, ks, v, 1.0 / 8, "causal", -1)
    want = oracle.attention(q, ks, v, 1.0 / 8, "causal", -1)
    check(got, want, dt, f"key shift {dt}")


@pytest.mark.parametrize("dt,mask,window", [("bf16", "causal", -1), ("f16", "none", -1),
                                            ("bf16", "sliding_window", 300)])
def test_growing_scores_raise_the_running_max(dt, mask, window):
    """Keys whose magnitude grows along the sequence (k_j (1 + 3 (j // 64)))
    make a row's score maximum climb tile after tile, by more than the 2^8
    slack the kernels allow before they raise the running max and rescale O
    and l. The case checks on the CPU that every row of one head sees such
    climbs, then compares the GPU with the oracle on the same rounded
    inputs."""
    B, S, H, Hkv, D = 1, 1000, 4, 2, 128
    q, k, v = inputs.make_qkv(B, S, H, Hkv, D, dt, seed=21)
    ramp = (1 + 3 * (torch.arange(S) // 64)).to(torch.float32)[None, :, None, None]
    kr = (k.float() * ramp).to(k.dtype)
    scale = 1.0 / math.sqrt(D)
    # log2-unit score maxima per 64-key tile for query head 0, rows past 900.
    sc = (q.double()[0, 900:, 0] @ kr.double()[0, :, 0].T) * scale / math.log(2)
    tile_max = sc[:, :896].reshape(sc.shape[0], 14, 64).amax(dim=2)
    climbs = (tile_max[:, 1:] - torch.cummax(tile_max, dim=1).values[:, :-1] > 8).sum(dim=1)
    assert (climbs >= 3).all(), "the case must make the running max climb"
    got = run_gpu(q, kr, v, scale, mask, window)
    check(got, oracle.attention(q, kr, v, scale, mask, window), dt, f"growing scores {dt} {mask}")


@pytest.mark.parametrize("dt,D", [("f32", 64), ("bf16", 128), ("bf16", 64)])
def test_huge_scale_tiny_inputs(dt, D):
    """scale = 1e38 on inputs of order 2^-60: q and k are small integers
    times 2^-60, so every product is an exact, normal fp32 number and the
    scores are exact multiples of 1e38 * 2^-120 (about 75), of order 1e3:
    inside the supported |scale q.k| log2(e) < 2^24. The softmax is one-hot
    on each row's largest score (shared between tied keys)."""
    gen = torch.Generator().manual_seed(22)
    B, S, H, Hkv = 1, 300, 4, 2
    td = inputs.DTYPES[dt]
    q = (torch.randint(-2, 3, (B, S, H, D), generator=gen).double() * 2.0 ** -60).to(td)
    k = (torch.randint(-3, 4, (B, S, Hkv, D), generator=gen).double() * 2.0 ** -60).to(td)
    v = torch.randn(B, S, Hkv, D, generator=gen).to(td)
    sc = (q.double()[0, :, 0] @ k.double()[0, :, 0].T).abs().max() * 1e38
    assert 1e2 < sc < 1e5, "scaled scores must be large but inside the supported range"
    got = run_gpu(q, k, v, 1e38, "causal", -1)
    want = oracle.attention(q, k, v, 1e38, "causal", -1)
    check(got, want, dt, f"scale 1e38 {dt} D{D}")


@pytest.mark.parametrize("D", [32, 64])
@pytest.mark.parametrize("mask,window", [("none", -1), ("causal", -1)])
def test_fp16_scale_above_one_over_log2e(D, mask, window):
    """fp16 at head dims 32 and 64 with scale * log2(e) > 1: Q is not
    pre-scaled (a scaled fp16 Q could overflow), so the scale is applied
    to the fp32 scores."""
    q, k, v = inputs.make_qkv(1, 300, 4, 2, D, "f16", seed=31 + D)
    scale = 1.0
    note(f"fp16 D{D} {mask} scale {scale}")
    got = run_gpu(q, k, v, scale, mask, window)
    want = oracle.attention(q, k, v, scale, mask, window)
    check(got, want, "f16", f"fp16 D{D} {mask} scale 1")


def test_peaky_softmax_fp16_small():
    w = inputs.WORKLOADS[4].with_(S=640, H=4, Hkv=4)
    q, k, v = inputs.workload_qkv(w)
    got = run_gpu(q, k, v, w.scale, w.mask, w.window)
    check(got, oracle.attention(q, k, v, w.scale, w.mask, w.window), "f16", "peaky fp16")


def test_deterministic_and_writes_every_element():
    q, k, v = inputs.make_qkv(2, 333, 8, 2, 128, "bf16", seed=10)
    qd, kd, vd = _dev(q, k, v)
    n = q.numel()
    buf = torch.full((n + 4096,), float("nan"), dtype=torch.bfloat16, device=DEV)
    guard = torch.arange(2048, device=DEV).to(torch.bfloat16)
    buf[:2048] = guard
    buf[-2048:] = guard
    out = buf[2048:2048 + n].view(q.shape)
    fa.attention(qd, kd, vd, 0.09, "causal", out=out)
    first = out.clone()
    fa.attention(qd, kd, vd, 0.09, "causal", out=out)
    torch.cuda.synchronize()
    assert not torch.isnan(first.float()).any(), "some output element was never written"
    assert torch.equal(first, out), "two runs differ"
    assert torch.equal(buf[:2048], guard) and torch.equal(buf[-2048:], guard), "write out of bounds"


def test_side_stream():
    q, k, v = inputs.make_qkv(1, 256, 4, 4, 64, "f16", seed=11)
    qd, kd, vd = _dev(q, k, v)
    ref = fa.attention(qd, kd, vd, 0.125, "causal")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        out = fa.attention(qd, kd, vd, 0.125, "causal")
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    assert torch.equal(out, ref)


def test_rejects_through_binding():
    q, k, v = inputs.make_qkv(1, 64, 4, 3, 64, "bf16", seed=12)
    with pytest.raises(fa.FA355Error) as e:
        fa.attention(*_dev(q, k, v), 0.1, "none")
    assert e.value.status == fa.ERR_INVALID_ARG


@pytest.mark.parametrize("dt,D", [("bf16", 128), ("f16", 64), ("f32", 128), ("bf16", 32), ("f16", 256),
                                  ("f32", 32), ("f32", 256)])
@pytest.mark.parametrize("mask", ["none", "causal"])
def test_rows_past_the_end_are_never_used(dt, D, mask):
    """K and V end exactly where NaN-filled memory begins; a ragged last key
    tile must neither read nor use rows past S (a NaN would reach the output)."""
    B, S, H, Hkv = 2, 300, 4, 2
    q, k, v = inputs.make_qkv(B, S, H, Hkv, D, dt, seed=13)
    note(f"tail guard {dt} D{D} {mask}")

    def guarded(t):
        n = t.numel()
        buf = torch.full((n + 256 * Hkv * D,), float("nan"), dtype=t.dtype, device=DEV)
        buf[:n] = t.flatten().to(DEV)
        return buf[:n].view(t.shape)

    out = fa.attention(q.to(DEV), guarded(k), guarded(v), 1.0 / math.sqrt(D), mask)
    torch.cuda.synchronize()
    check(out.cpu(), oracle.attention(q, k, v, 1.0 / math.sqrt(D), mask), dt, f"tail {dt} {mask}")


WALK = [
    # B, S, H, Hkv, D, dtype, mask, window: more work items than compute
    # units. At D = 64 and 128 with short items each workgroup walks several
    # items, the last round only partly filled; the D = 32 case launches one
    # workgroup per item.
    (2, 1100, 32, 8, 128, "bf16", "causal", -1),
    (1, 1100, 64, 8, 128, "bf16", "sliding_window", 200),
    (2, 1037, 32, 8, 128, "f16", "none", -1),
    (1, 600, 256, 256, 32, "bf16", "causal", -1),
    (4, 1100, 32, 8, 64, "f16", "causal", -1),    # 576 items on 512 resident workgroups
    (8, 1100, 32, 8, 64, "f16", "causal", -1),    # 1152 items: three rounds
    (2, 1500, 64, 16, 64, "bf16", "sliding_window", 150),
    (4, 2048, 16, 16, 64, "f16", "causal", -1),    # 512 items fit the resident count: one per CU, two rounds
    (1, 2100, 32, 8, 128, "bf16", "sliding_window", 1),   # one-tile items: each row sees only itself
    (1, 2100, 32, 8, 128, "f16", "sliding_window", 64),   # two-tile items
    (2, 1025, 32, 8, 128, "bf16", "causal", -1),          # last query tile: one row, one wave wholly past the end
    (2, 2100, 32, 8, 64, "bf16", "sliding_window", 1),    # D = 64, one-tile items, 528 on 512 resident
    (5, 1025, 32, 8, 64, "f16", "causal", -1),            # D = 64, 680 items, a one-row last tile
]


@pytest.mark.parametrize("case", WALK, ids=lambda c: "B{}_S{}_H{}kv{}_D{}_{}_{}_W{}".format(*c))
def test_walk_over_many_items_whole_output(case):
    B, S, H, Hkv, D, dt, mask, window = case
    note(f"walk case {case}")
    pl = fa.plan(B, S, H, Hkv, D, {"bf16": fa.BF16, "f16": fa.F16}[dt], mask, window)
    # More items than compute units: D = 128 (one workgroup per CU) walks them
    # on a resident grid; D = 64 (two per CU) too when they outnumber the
    # resident count, and otherwise on one workgroup per CU.
    assert pl["num_workgroups"] > torch.cuda.get_device_properties(0).multi_processor_count
    assert pl["walk"] == (D in (64, 128))
    q, k, v = inputs.make_qkv(B, S, H, Hkv, D, dt, seed=S + H + D)
    out = torch.full(q.shape, float("nan"), dtype=q.dtype, device=DEV)
    fa.attention(*_dev(q, k, v), 1.0 / math.sqrt(D), mask, window, out=out)
    torch.cuda.synchronize()
    got = out.cpu()
    assert not torch.isnan(got.float()).any(), "some output element was never written"
    check(got, oracle.attention(q, k, v, 1.0 / math.sqrt(D), mask, window), dt, str(case))


D256_DEFAULT = [
    # Enough 256-row work items (512 under a mask, 256 without) for the
    # 8-wave layout at D = 256 (32-key tiles, V reads per MFMA).
    (8, 1024, 16, 16, 256, "bf16", "causal", -1),
    (4, 2000, 16, 16, 256, "f16", "causal", -1),           # ragged S
    (2, 2048, 16, 16, 256, "bf16", "none", -1),
    (4, 2100, 16, 4, 256, "f16", "sliding_window", 200),   # 4 heads per K/V head, ragged
    (600, 1, 1, 1, 256, "bf16", "causal", -1),             # S = 1: one row per item, 7 waves past the end
    (1, 33, 512, 512, 256, "f16", "causal", -1),           # one full 32-key tile and a 1-key tail
    (2, 200, 256, 256, 256, "bf16", "sliding_window", 1),  # window 1: each row sees only itself
]


@pytest.mark.timeout(600)
@pytest.mark.parametrize("case", D256_DEFAULT, ids=lambda c: "B{}_S{}_H{}kv{}_D{}_{}_{}_W{}".format(*c))
def test_d256_eight_wave_layout_whole_output(case):
    B, S, H, Hkv, D, dt, mask, window = case
    note(f"D=256 8-wave case {case}")
    pl = fa.plan(B, S, H, Hkv, D, {"bf16": fa.BF16, "f16": fa.F16}[dt], mask, window)
    assert pl["block_n"] == 32 and pl["block_m"] * pl["heads_per_workgroup"] == 256
    q, k, v = inputs.make_qkv(B, S, H, Hkv, D, dt, seed=S + H + D)
    out = torch.full(q.shape, float("nan"), dtype=q.dtype, device=DEV)
    fa.attention(*_dev(q, k, v), 1.0 / math.sqrt(D), mask, window, out=out)
    torch.cuda.synchronize()
    got = out.cpu()
    assert not torch.isnan(got.float()).any(), "some output element was never written"
    check(got, oracle.attention(q, k, v, 1.0 / math.sqrt(D), mask, window), dt, str(case))


@pytest.mark.parametrize("case", [
    (2, 1100, 32, 8, 128, "bf16", "causal", -1),           # walks: resident grid, several items each
    (1, 700, 16, 16, 64, "f16", "sliding_window", 100),    # walks at D = 64
    (1, 500, 8, 2, 256, "bf16", "none", -1),                # few items at D = 256: pipelined loop
    (2, 2048, 16, 16, 256, "f16", "none", -1),              # D = 256, 8-wave layout
])
def test_graph_replays_match_eager(case):
    """The call captured in a HIP graph (torch.cuda.CUDAGraph) replays to the
    eager result bit for bit, replay after replay, with eager work and
    synchronisations in between. The kernels record no memset nodes."""
    B, S, H, Hkv, D, dt, mask, window = case
    note(f"graph case {case}")
    q, k, v = _dev(*inputs.make_qkv(B, S, H, Hkv, D, dt, seed=S + D))
    scale = 1.0 / math.sqrt(D)
    eager = fa.attention(q, k, v, scale, mask, window)
    out = torch.full_like(q, float("nan"))
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fa.attention(q, k, v, scale, mask, window, out=out)  # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fa.attention(q, k, v, scale, mask, window, out=out)
    for i in range(3):
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), f"replay {i} differs from the eager result"
        fa.attention(q, k, v, scale, mask, window)  # eager work between replays


@pytest.mark.parametrize("case", [
    # q and out of 2 GiB each: element and byte offsets past 32 bits.
    (4, 32768, 64, 8, 128, "bf16", "causal", -1),
    # one batch's K (and V) of 2 GiB: S = 65536 rows of 128 heads.
    (1, 65536, 128, 128, 128, "bf16", "causal", -1),
    # fp32 K and V of 2 GiB each (64 K/V heads), q and out of 4 GiB (128 heads).
    (1, 32768, 128, 64, 256, "f32", "sliding_window", 5000),
    # D = 256 in the 8-wave layout: q and out of 2 GiB (128 heads), 4096 items.
    (1, 32768, 128, 32, 256, "bf16", "causal", -1),
])
def test_large_tensors_sampled_rows(case):
    """Tensors at the sizes where offsets outgrow 32 bits; a sample of rows
    (both batch ends, several heads, both sequence ends and the middle) is
    recomputed by the oracle from the slices each row needs."""
    B, S, H, Hkv, D, dt, mask, window = case
    note(f"large case {case}")
    q, k, v = inputs.make_qkv_device(B, S, H, Hkv, D, dt, seed=S + H, device=DEV)
    scale = 1.0 / math.sqrt(D)
    out = fa.attention(q, k, v, scale, mask, window)
    torch.cuda.synchronize()
    rng = np.random.default_rng(5)
    rep = H // Hkv
    errs = []
    for b in sorted({0, B - 1}):
        for h in sorted({0, H - 1, int(rng.integers(H))}):
            g = h // rep
            qs = q[b:b + 1, :, h:h + 1].contiguous().cpu()
            ks = k[b:b + 1, :, g:g + 1].contiguous().cpu()
            vs = v[b:b + 1, :, g:g + 1].contiguous().cpu()
            idx = sorted({0, 1, 63, 64, S // 2, S - 2, S - 1} | set(rng.integers(0, S, 6).tolist()))
            want = oracle.attention_rows(qs, ks, vs, scale, mask, window, [(0, 0, i) for i in idx])
            got = out[b, idx, h].cpu()
            errs.append(check(got, want, dt, f"{case} b={b} h={h}"))
    note(f"  worst max {max(e[0] for e in errs):.3e}")
