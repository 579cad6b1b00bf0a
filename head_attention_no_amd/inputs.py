"""Seeded synthetic inputs for the attention forward (no attention arithmetic here).

Shared by the tests, the benchmark and the smoke check: the HIP path and the
fp64 oracle both consume exactly the tensors drawn here. Draw recipe, fixed so
that any run reproduces the same bits:

- ``torch.Generator('cpu').manual_seed(seed)``;
- draw order q ~ N(0,1) of shape (B, S, H, D), then k, then v of shape
  (B, S, Hkv, D), all float32;
- optionally multiply k by ``k_mult`` (a power of two, so exact);
- round to the workload dtype (round-to-nearest-even).

The named workloads are the five shapes this library is measured and
checked on: long-context causal and sliding-window attention with grouped
K/V heads, plus a small fp32 case and a peaked-softmax fp16 case; WIDER adds
the head dims 32 and 256 and fp32 at S = 4096.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, replace

import torch

DTYPES = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    S: int
    H: int
    Hkv: int
    D: int
    dtype: str  # "f32" | "bf16" | "f16"
    mask: str  # "none" | "causal" | "sliding_window"
    window: int = -1
    k_mult: float = 1.0
    seed: int = 0

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.D)

    @property
    def torch_dtype(self) -> torch.dtype:
        return DTYPES[self.dtype]

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


WORKLOADS = [
    Workload("mha_s128_d64_f32_nomask", 1, 128, 4, 4, 64, "f32", "none", seed=1001),
    Workload("mha_b4_s2048_d128_bf16_causal", 4, 2048, 32, 32, 128, "bf16", "causal", seed=1002),
    Workload("gqa_b2_s4096_h32kv8_d128_bf16_causal", 2, 4096, 32, 8, 128, "bf16", "causal",
             seed=1003),
    Workload("gqa_b1_s8192_h32kv8_d128_bf16_window1024", 1, 8192, 32, 8, 128, "bf16",
             "sliding_window", window=1024, seed=1004),
    Workload("mha_b1_s16384_h16_d64_f16_nomask_peaky", 1, 16384, 16, 16, 64, "f16", "none",
             k_mult=4.0, seed=1005),
]

# The rest of the op's shape contract: head dims 32 and 256, sized to the
# same causal FLOP count as the S = 4096 grouped workload above, and fp32 at
# a long sequence.
WIDER = [
    Workload("mha_b4_s8192_h16_d32_bf16_causal", 4, 8192, 16, 16, 32, "bf16", "causal", seed=1006),
    Workload("mha_b2_s4096_h16_d256_bf16_causal", 2, 4096, 16, 16, 256, "bf16", "causal", seed=1007),
    Workload("mha_b1_s4096_h16_d128_f32_causal", 1, 4096, 16, 16, 128, "f32", "causal", seed=1008),
]

BY_NAME = {w.name: w for w in WORKLOADS + WIDER}


def make_qkv(B: int, S: int, H: int, Hkv: int, D: int, dtype: str = "bf16", seed: int = 0,
             k_mult: float = 1.0):
    """Seeded CPU tensors q (B,S,H,D), k and v (B,S,Hkv,D) of the given dtype."""
    g = torch.Generator("cpu").manual_seed(int(seed))
    q = torch.randn(B, S, H, D, generator=g, dtype=torch.float32)
    k = torch.randn(B, S, Hkv, D, generator=g, dtype=torch.float32)
    v = torch.randn(B, S, Hkv, D, generator=g, dtype=torch.float32)
    if k_mult != 1.0:
        k = k * k_mult
    td = DTYPES[dtype]
    return q.to(td), k.to(td), v.to(td)


def make_qkv_device(B: int, S: int, H: int, Hkv: int, D: int, dtype: str, seed: int, device):
    """The make_qkv recipe drawn on `device` with a seeded device generator
    (other values than the CPU draw of the same seed), for tensors too large
    to draw on the host quickly; checks copy the slices they need back."""
    g = torch.Generator(device).manual_seed(int(seed))
    td = DTYPES[dtype]
    q = torch.randn(B, S, H, D, generator=g, dtype=torch.float32, device=device).to(td)
    k = torch.randn(B, S, Hkv, D, generator=g, dtype=torch.float32, device=device).to(td)
    v = torch.randn(B, S, Hkv, D, generator=g, dtype=torch.float32, device=device).to(td)
    return q, k, v


def workload_qkv(w: Workload):
    return make_qkv(w.B, w.S, w.H, w.Hkv, w.D, w.dtype, w.seed, w.k_mult)


# Top-K ordering inputs: rows of next-token scores.
TOPK_WORKLOAD = {"name": "topk_b256_v128256_k50_f32", "B": 256, "V": 128256, "K": 50,
                 "kind": "frequencies", "seed": 2001}


def make_scores(B: int, V: int, kind: str = "frequencies", seed: int = 0):
    """Seeded float32 CPU rows (B, V). Kinds: "frequencies" (a softmax of
    N(0, 3^2) logits, in percent: how often each next token appears),
    "normal" (N(0,1)), "ties" (multiples of 1/4 in [-1, 1.5]: many equal
    values), "zeros" (signed zeros with a few negatives), "huge_tiny"
    (1e30 every third entry, N(0, 1e-30) elsewhere)."""
    g = torch.Generator("cpu").manual_seed(int(seed))
    if kind == "frequencies":
        logits = torch.randn(B, V, generator=g, dtype=torch.float64) * 3.0
        return (torch.softmax(logits, dim=1) * 100.0).to(torch.float32)
    if kind == "normal":
        return torch.randn(B, V, generator=g, dtype=torch.float32)
    if kind == "ties":
        return torch.randint(-4, 7, (B, V), generator=g).to(torch.float32) / 4
    if kind == "zeros":
        sign = torch.randint(0, 2, (B, V), generator=g).to(torch.bool)
        x = torch.where(sign, torch.tensor(-0.0), torch.tensor(0.0)).to(torch.float32)
        x[:, ::97] = -1.0
        return x
    if kind == "huge_tiny":
        x = torch.randn(B, V, generator=g, dtype=torch.float32) * 1e-30
        x[:, ::3] = 1e30
        return x
    raise ValueError(kind)
