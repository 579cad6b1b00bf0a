"""Python binding of libfa355, the gfx950 fused no-KV-cache attention forward.

Argument marshalling only: every step of the computation runs in the HIP
kernels of ``libfa355.so``. PyTorch provides device memory and the current
stream. There is no CPU fallback: if the library is not built, or the call
is rejected, these functions raise.

The C entry points keep their names here:
``mha_no_cache(out, q, k, v, B, S, H, Hkv, D, scale, mask_kind, window,
dtype, stream)`` takes raw device addresses and returns a status code;
``attention(q, k, v, scale, mask, window)`` is the tensor-level wrapper that
allocates ``out`` and raises on a non-zero status.
"""
from __future__ import annotations

import ctypes
import os

F32, BF16, F16 = 0, 1, 2
MASK_NONE, MASK_CAUSAL, MASK_SLIDING_WINDOW = 0, 1, 2
OK, ERR_INVALID_ARG, ERR_UNSUPPORTED, ERR_DEVICE, ERR_LAUNCH = 0, 1, 2, 3, 4

MASKS = {"none": MASK_NONE, "causal": MASK_CAUSAL, "sliding_window": MASK_SLIDING_WINDOW,
         "window": MASK_SLIDING_WINDOW}

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libfa355.so")

# Every symbol that include/fa355.h declares.
EXPORTS = ("mha_no_cache", "fa355_strerror", "fa355_version", "fa355_plan", "fa355_topk")

_lib = None


class FA355Error(RuntimeError):
    def __init__(self, status: int, where: str = "mha_no_cache"):
        self.status = status
        super().__init__(f"{where} failed with status {status}: {strerror(status)}")


def load(path: str = LIB_PATH):
    """Load libfa355.so (raises if it has not been built)."""
    global _lib
    if _lib is not None and path == LIB_PATH:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with `python -m head_attention_no_amd.build`"
                           " (or __graft_entry__.build())")
    lib = ctypes.CDLL(path)
    vp, i = ctypes.c_void_p, ctypes.c_int
    lib.mha_no_cache.argtypes = [vp, vp, vp, vp, i, i, i, i, i, ctypes.c_float, i, i, i, vp]
    lib.mha_no_cache.restype = i
    lib.fa355_strerror.argtypes = [i]
    lib.fa355_strerror.restype = ctypes.c_char_p
    lib.fa355_version.argtypes = []
    lib.fa355_version.restype = ctypes.c_char_p
    ip = ctypes.POINTER(ctypes.c_int)
    lib.fa355_plan.argtypes = [i, i, i, i, i, i, i, i, ip, ip, ip, ip, ip, ip, i]
    lib.fa355_plan.restype = i
    lib.fa355_topk.argtypes = [vp, vp, vp, i, i, i, vp]
    lib.fa355_topk.restype = i
    if path == LIB_PATH:
        _lib = lib
    return lib


def mha_no_cache(out: int, q: int, k: int, v: int, B: int, S: int, H: int, Hkv: int, D: int,
                 scale: float, mask_kind: int, window: int, dtype: int, stream: int) -> int:
    """The C entry point with raw device addresses; returns an fa355 status code."""
    return load().mha_no_cache(out, q, k, v, B, S, H, Hkv, D, scale, mask_kind, window, dtype,
                               stream)


def strerror(status: int) -> str:
    return load().fa355_strerror(int(status)).decode()


def version() -> str:
    return load().fa355_version().decode()


def plan(B: int, S: int, H: int, Hkv: int, D: int, dtype: int, mask="none", window: int = -1,
         with_tiles: bool = False):
    """Work decomposition: dict(num_workgroups, block_m, block_n,
    heads_per_workgroup, walk[, tiles]); each tile is (query tile, b, first
    head), in item order."""
    lib = load()
    mk = MASKS[mask] if isinstance(mask, str) else int(mask)
    nwg, bm, bn, hp, walk = (ctypes.c_int() for _ in range(5))
    rc = lib.fa355_plan(B, S, H, Hkv, D, dtype, mk, window, ctypes.byref(nwg), ctypes.byref(bm),
                        ctypes.byref(bn), ctypes.byref(hp), ctypes.byref(walk), None, 0)
    if rc != OK:
        raise FA355Error(rc, "fa355_plan")
    res = {"num_workgroups": nwg.value, "block_m": bm.value, "block_n": bn.value,
           "heads_per_workgroup": hp.value, "walk": walk.value}
    if with_tiles:
        buf = (ctypes.c_int * (3 * nwg.value))()
        rc = lib.fa355_plan(B, S, H, Hkv, D, dtype, mk, window, None, None, None, None, None, buf,
                            nwg.value)
        if rc != OK:
            raise FA355Error(rc, "fa355_plan")
        res["tiles"] = [tuple(buf[3 * w:3 * w + 3]) for w in range(nwg.value)]
    return res


def _dtype_code(t) -> int:
    import torch

    codes = {torch.float32: F32, torch.bfloat16: BF16, torch.float16: F16}
    if t.dtype not in codes:
        raise TypeError(f"unsupported dtype {t.dtype}")
    return codes[t.dtype]


def attention(q, k, v, scale: float, mask="none", window: int = -1, out=None, stream=None):
    """softmax(mask(scale * q k^T)) v for BSHD torch tensors on a gfx950 device.

    q: (B, S, H, D); k, v: (B, S, Hkv, D), same dtype and device, contiguous.
    Launches on ``stream`` (default: torch's current stream) and returns
    ``out`` without synchronising.
    """
    import torch

    for name, t in (("q", q), ("k", k), ("v", v)):
        if not t.is_cuda:
            raise ValueError(f"{name} must be a device tensor")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    if q.dim() != 4 or k.dim() != 4 or v.dim() != 4:
        raise ValueError("q, k, v must be rank 4 (BSHD)")
    if k.shape != v.shape or q.dtype != k.dtype or q.dtype != v.dtype:
        raise ValueError("k and v must match, and share q's dtype")
    B, S, H, D = q.shape
    if k.shape[0] != B or k.shape[1] != S or k.shape[3] != D:
        raise ValueError(f"k/v shape {tuple(k.shape)} does not fit q {tuple(q.shape)}")
    Hkv = k.shape[2]
    if out is None:
        out = torch.empty_like(q)
    elif out.shape != q.shape or out.dtype != q.dtype or not out.is_contiguous():
        raise ValueError("out must be a contiguous tensor shaped and typed like q")
    mask_kind = MASKS[mask] if isinstance(mask, str) else int(mask)
    with torch.cuda.device(q.device):
        if stream is None:
            stream = torch.cuda.current_stream(q.device)
        rc = mha_no_cache(out.data_ptr(), q.data_ptr(), k.data_ptr(), v.data_ptr(), B, S, H, Hkv,
                          D, float(scale), mask_kind, int(window), _dtype_code(q),
                          stream.cuda_stream)
    if rc != OK:
        raise FA355Error(rc)
    return out


def fa355_topk(values, indices, x, B: int, V: int, K: int, stream) -> int:
    """Raw C-ABI call (device addresses as ints); returns the status code."""
    return load().fa355_topk(values, indices, x, B, V, K, stream)


def topk(x, k: int, values=None, indices=None, stream=None):
    """The k largest entries of each row of a 2-D float32 device tensor, in
    descending order, equal values by ascending index: (values, indices),
    float32 and int32 tensors of shape (rows, k). Launches on ``stream``
    (default: torch's current stream) without synchronising."""
    import torch

    if not x.is_cuda or not x.is_contiguous() or x.dim() != 2 or x.dtype != torch.float32:
        raise ValueError("x must be a contiguous 2-D float32 device tensor")
    B, V = x.shape
    if values is None:
        values = torch.empty(B, k, dtype=torch.float32, device=x.device)
    if indices is None:
        indices = torch.empty(B, k, dtype=torch.int32, device=x.device)
    for name, t, dt in (("values", values, torch.float32), ("indices", indices, torch.int32)):
        if t.shape != (B, k) or t.dtype != dt or not t.is_contiguous() or t.device != x.device:
            raise ValueError(f"{name} must be a contiguous ({B}, {k}) {dt} tensor on {x.device}")
    with torch.cuda.device(x.device):
        if stream is None:
            stream = torch.cuda.current_stream(x.device)
        rc = fa355_topk(values.data_ptr(), indices.data_ptr(), x.data_ptr(), B, V, int(k),
                        stream.cuda_stream)
    if rc != OK:
        raise FA355Error(rc, "fa355_topk")
    return values, indices
