"""The seeded input generator shared by the HIP path and the oracle."""
import torch

from head_attention_no_amd import inputs


def test_same_seed_same_bits():
    a = inputs.make_qkv(1, 8, 4, 2, 16, "bf16", seed=5)
    b = inputs.make_qkv(1, 8, 4, 2, 16, "bf16", seed=5)
    for x, y in zip(a, b):
        assert torch.equal(x.view(torch.int16), y.view(torch.int16))


def test_shapes_and_dtypes():
    for dt, td in inputs.DTYPES.items():
        q, k, v = inputs.make_qkv(2, 5, 6, 3, 8, dt, seed=1)
        assert q.shape == (2, 5, 6, 8) and k.shape == (2, 5, 3, 8) and v.shape == (2, 5, 3, 8)
        assert q.dtype == td and k.dtype == td and v.dtype == td


def test_key_multiplier_is_exact():
    q0, k0, v0 = inputs.make_qkv(1, 16, 2, 2, 8, "f16", seed=3)
    q4, k4, v4 = inputs.make_qkv(1, 16, 2, 2, 8, "f16", seed=3, k_mult=4.0)
    assert torch.equal(q0, q4) and torch.equal(v0, v4)
    assert torch.equal(k4.float(), k0.float() * 4)


def test_named_workloads():
    names = [w.name for w in inputs.WORKLOADS]
    assert len(set(names)) == 5
    w = inputs.BY_NAME["gqa_b2_s4096_h32kv8_d128_bf16_causal"]
    assert (w.B, w.S, w.H, w.Hkv, w.D, w.dtype, w.mask) == (2, 4096, 32, 8, 128, "bf16", "causal")
    assert abs(w.scale - 128 ** -0.5) < 1e-15
