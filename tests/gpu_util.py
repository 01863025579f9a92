"""Helpers for the GPU parity tests: upload inputs, call the library through
its C ABI, and compare with the oracle."""
import contextlib

import numpy as np

import block_quantized_gemv_kq_amd as kq
from oracle import formats as F
from oracle import ref as R


def torch_cuda():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return torch


def to_dev(a: np.ndarray):
    torch = torch_cuda()
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda")


def empty_dev(shape, dtype="float32"):
    torch = torch_cuda()
    return torch.empty(shape, dtype=getattr(torch, dtype), device="cuda")


def to_host(t) -> np.ndarray:
    torch = torch_cuda()
    torch.cuda.synchronize()
    return t.cpu().numpy()


def quantize_both(fmt, W):
    """Pack with the library's packer and with the oracle; the bytes must be
    identical. Returns (packed bytes, oracle fields)."""
    fields = F.quantize(fmt, W)
    packed = kq.kq_pack(fmt, W)
    ref = F.encode(fmt, fields)
    assert np.array_equal(packed, ref), "packer bytes differ from the oracle's"
    return packed, fields


_TUNING: dict = {}   # the overrides in force (blocks nest)


@contextlib.contextmanager
def tuning(values: dict):
    """Force kernels or configurations (kq_set_tuning) for the duration of a
    block; afterwards the overrides of the enclosing block are back."""
    global _TUNING
    outer = dict(_TUNING)
    try:
        for k, v in values.items():
            kq.kq_set_tuning(k, v)
        _TUNING = {**outer, **values}
        yield
    finally:
        kq.kq_set_tuning(None, None)
        for k, v in outer.items():
            kq.kq_set_tuning(k, v)
        _TUNING = outer


def gemv_gpu(fmt, packed_dev, x16: np.ndarray, N: int, K: int, path: str | None = None) -> np.ndarray:
    """Run kq_gemv; returns y[M][N] as numpy fp32."""
    M = x16.shape[0]
    xd = to_dev(x16)
    y = empty_dev((M, N))
    y.fill_(float("nan"))
    with tuning({"force_path": path[0]} if path else {}):   # "generic", "valu", "lds", "mfma"
        kq.kq_gemv(fmt, packed_dev, xd, y, N, K, M)
    return to_host(y)


def assert_parity(y_gpu, y_ref, abs_dot, what=""):
    ok = R.within_tolerance(y_gpu, y_ref, abs_dot)
    if not np.all(ok):
        bad = np.argwhere(~ok)
        i = tuple(bad[0])
        raise AssertionError(
            f"{what}: {bad.shape[0]} outputs out of tolerance; first {i}: gpu {y_gpu[i]!r} "
            f"ref {y_ref[i]!r} bound {R.tolerance(abs_dot)[i]!r}")
    return R.error_ratio(y_gpu, y_ref, abs_dot)
