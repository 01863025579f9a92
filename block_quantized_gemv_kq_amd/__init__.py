"""Python binding for libkq.so — block-quantized decode GEMV on MI355X (gfx950).

Argument marshalling only: every computation runs in the library's HIP
kernels (or, for kq_pack/kq_unpack, in its host C++ packer). Names mirror the
C ABI in include/kq.h. Device buffers are passed as torch tensors (their
data_ptr) or as raw integer addresses; streams default to torch's current
stream. There is no fallback: if libkq.so is missing, or a call fails, an
exception is raised.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libkq.so")

KQ_Q8_0, KQ_Q4_0, KQ_AFFINE4_G32, KQ_Q5_0, KQ_Q5_1 = 0, 1, 2, 3, 4
KQ_Q4_1 = KQ_AFFINE4_G32   # the same scale-and-minimum 4-bit block
FORMATS = {"q8_0": KQ_Q8_0, "q4_0": KQ_Q4_0, "affine4": KQ_AFFINE4_G32, "q5_0": KQ_Q5_0, "q5_1": KQ_Q5_1,
           "q4_1": KQ_Q4_1}
KQ_OK, KQ_ERR_ARG, KQ_ERR_FORMAT, KQ_ERR_SHAPE, KQ_ERR_ALIGN, KQ_ERR_RANGE, KQ_ERR_HIP = 0, -1, -2, -3, -4, -5, -6
KQ_MAX_M = 64
KQ_MAX_K = 1 << 20       # inputs per row
KQ_MAX_N = 0x7FFFFFFF   # output rows per call

# Every symbol include/kq.h declares, with (restype, argtypes).
_I64, _I32, _P = ctypes.c_int64, ctypes.c_int, ctypes.c_void_p
SIGNATURES = {
    "kq_version": (_I32, []),
    "kq_status_string": (ctypes.c_char_p, [_I32]),
    "kq_last_error": (ctypes.c_char_p, []),
    "kq_block_bytes": (_I64, [_I32]),
    "kq_packed_bytes": (_I64, [_I32, _I64, _I64]),
    "kq_pack": (_I32, [_I32, _P, _I64, _I64, _P, _I32]),
    "kq_unpack": (_I32, [_I32, _P, _I64, _I64, _P]),
    "kq_gemv": (_I32, [_I32, _P, _P, _P, _I64, _I64, _I32, _P]),
    "kq_gemv_ws": (_I32, [_I32, _P, _P, _P, _I64, _I64, _I32, _P, _I64, _P]),
    "kq_gemv_workspace_bytes": (_I64, [_I32, _I64, _I64, _I32]),
    "kq_gemv_invariant": (_I32, [_I32, _P, _P, _P, _I64, _I64, _I32, _P]),
    "kq_gemv_argmax_workspace_bytes": (_I64, [_I32, _I64, _I64, _I32]),
    "kq_gemv_argmax": (_I32, [_I32, _P, _P, _P, _I64, _I64, _I32, _P, _P, _I64, _P]),
    "kq_gemv_argmax_noalloc": (_I32, [_I32, _P, _P, _P, _I64, _I64, _I32, _P, _P]),
    "kq_shortlist_copy_bytes": (_I64, [_I64, _I64]),
    "kq_shortlist_pack": (_I32, [_P, _I64, _I64, _P, _I32]),
    "kq_shortlist_workspace_bytes": (_I64, [_I64, _I64]),
    "kq_shortlist_argmax": (_I32, [_P, _P, _P, _I64, _I64, _P, _I64, _P, _P, _P]),
    "kq_moe_gemv_workspace_bytes": (_I64, [_I64, _I32, _I32, _I32]),
    "kq_moe_gemv": (_I32, [_I32, _P, _P, _P, _P, _P, _I64, _I64, _I32, _I32, _I32, _I32, _P, _I64, _P]),
    "kq_moe_ffn_workspace_bytes": (_I64, [_I64, _I64, _I32, _I32]),
    "kq_moe_ffn": (_I32, [_I32, _P, _P, _P, _P, _P, _P, _P, _P, _I64, _I64, _I32, _I32, _I32, _P, _I64, _P]),
    "kq_argmax_workspace_bytes": (_I64, [_I64, _I32]),
    "kq_argmax": (_I32, [_P, _I64, _I32, _P, _P, _I64, _P]),
    "kq_f32_to_f16": (_I32, [_P, _P, _I64]),
    "kq_set_tuning": (_I32, [ctypes.c_char_p, ctypes.c_char_p]),
    "kq_stack_plan_bytes": (_I64, [_P, _I32]),
    "kq_stack_plan": (_I32, [_P, _I32, _P, _I64, _P, _P]),
    "kq_stack_run": (_I32, [_P, _P, _P]),
    "kq_stack_status": (_I32, [_P, _P, _P, _P]),
}


class kq_stage(ctypes.Structure):
    """Mirror of the C struct kq_stage (include/kq.h)."""
    _fields_ = [("fmt", ctypes.c_int32), ("reserved", ctypes.c_int32), ("W", ctypes.c_void_p),
                ("x", ctypes.c_void_p), ("y", ctypes.c_void_p), ("N", ctypes.c_int64),
                ("K", ctypes.c_int64), ("y16", ctypes.c_void_p)]


class kq_stack_info(ctypes.Structure):
    _fields_ = [("n_stages", ctypes.c_int32), ("fmt_mask", ctypes.c_int32), ("k_max", ctypes.c_int32),
                ("workgroups", ctypes.c_int32)]


class KQError(RuntimeError):
    def __init__(self, status: int, where: str, detail: str):
        super().__init__(f"{where}: {status_name(status)} ({status}): {detail}")
        self.status = status


_lib = None


def lib() -> ctypes.CDLL:
    """Load libkq.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        # PyTorch-ROCm carries its own HIP runtime (same soname as ROCm's). Load
        # it first so libkq.so binds to that one runtime: two runtimes in one
        # process do not share devices, streams or allocations.
        try:
            import torch  # noqa: F401
        except ImportError:
            pass
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is not built; run python -m block_quantized_gemv_kq_amd.build")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def status_name(status: int) -> str:
    return lib().kq_status_string(status).decode()


def last_error() -> str:
    return lib().kq_last_error().decode()


def _check(status: int, where: str) -> int:
    if status < 0:
        raise KQError(status, where, last_error())
    return status


def _fmt(fmt) -> int:
    if isinstance(fmt, str):
        return FORMATS[fmt]
    return int(fmt)


def _ptr(t) -> int | None:
    """Device/host address of a torch tensor, numpy array or integer."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    if isinstance(t, np.ndarray):
        return t.ctypes.data
    return t.data_ptr()


def _stream(stream) -> int | None:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


# ------------------------------------------------------------------ sizes

def kq_version() -> int:
    return lib().kq_version()


def kq_block_bytes(fmt) -> int:
    return _check(lib().kq_block_bytes(_fmt(fmt)), "kq_block_bytes")


def kq_packed_bytes(fmt, N: int, K: int) -> int:
    return _check(lib().kq_packed_bytes(_fmt(fmt), N, K), "kq_packed_bytes")


# ------------------------------------------------------------------ host packer

def kq_pack(fmt, W: np.ndarray, out: np.ndarray | None = None, n_threads: int = 0) -> np.ndarray:
    """Pack fp32 W[N][K] (host) -> uint8[N, K/32*block_bytes] (host)."""
    W = np.ascontiguousarray(W)
    if W.dtype != np.float32 or W.ndim != 2:
        raise TypeError("W must be a 2-D float32 array")
    n, k = W.shape
    nbytes = kq_packed_bytes(fmt, n, k)
    if out is None:
        out = np.empty((n, nbytes // max(n, 1)) if n else (0, 0), np.uint8)
    if not out.flags.c_contiguous or out.nbytes < nbytes:
        raise ValueError("out too small or not contiguous")
    _check(lib().kq_pack(_fmt(fmt), W.ctypes.data, n, k, out.ctypes.data, n_threads), "kq_pack")
    return out


def kq_unpack(fmt, packed: np.ndarray, N: int, K: int) -> np.ndarray:
    packed = np.ascontiguousarray(packed)
    if packed.nbytes < kq_packed_bytes(fmt, N, K):
        raise ValueError("packed buffer too small")
    out = np.empty((N, K), np.float32)
    _check(lib().kq_unpack(_fmt(fmt), packed.ctypes.data, N, K, out.ctypes.data), "kq_unpack")
    return out


def kq_f32_to_f16(a: np.ndarray) -> np.ndarray:
    a = np.ascontiguousarray(a, dtype=np.float32)
    out = np.empty(a.shape, np.uint16)
    _check(lib().kq_f32_to_f16(a.ctypes.data, out.ctypes.data, a.size), "kq_f32_to_f16")
    return out


def kq_set_tuning(name: str | None, value: str | None) -> None:
    """Tests and sweeps: force a kernel or launch configuration (see kq.h)."""
    _check(lib().kq_set_tuning(None if name is None else name.encode(),
                               None if value is None else str(value).encode()), "kq_set_tuning")


# ------------------------------------------------------------------ GPU calls

def kq_gemv(fmt, W, x, y, N: int, K: int, M: int, stream=None) -> None:
    """y[M][N] (fp32, device) = dequant(W)[N][K] @ x[M][K]^T (x fp16 bits, device)."""
    _check(lib().kq_gemv(_fmt(fmt), _ptr(W), _ptr(x), _ptr(y), N, K, M, _stream(stream)), "kq_gemv")


def kq_gemv_workspace_bytes(fmt, N: int, K: int, M: int) -> int:
    return _check(lib().kq_gemv_workspace_bytes(_fmt(fmt), N, K, M), "kq_gemv_workspace_bytes")


def kq_gemv_ws(fmt, W, x, y, N: int, K: int, M: int, workspace, workspace_bytes: int, stream=None) -> None:
    """kq_gemv with a caller-owned workspace (K split across workgroups where it pays)."""
    _check(lib().kq_gemv_ws(_fmt(fmt), _ptr(W), _ptr(x), _ptr(y), N, K, M, _ptr(workspace), workspace_bytes,
                            _stream(stream)), "kq_gemv_ws")


def kq_gemv_argmax_workspace_bytes(fmt, N: int, K: int, M: int) -> int:
    return _check(lib().kq_gemv_argmax_workspace_bytes(_fmt(fmt), N, K, M), "kq_gemv_argmax_workspace_bytes")


def kq_gemv_argmax(fmt, W, x, y, N: int, K: int, M: int, out, workspace, workspace_bytes: int,
                   stream=None) -> None:
    """kq_gemv into y, then out[m] = argmax of y[m] (int32, device)."""
    _check(lib().kq_gemv_argmax(_fmt(fmt), _ptr(W), _ptr(x), _ptr(y), N, K, M, _ptr(out), _ptr(workspace),
                                workspace_bytes, _stream(stream)), "kq_gemv_argmax")


def kq_gemv_argmax_noalloc(fmt, W, x, y, N: int, K: int, M: int, out, stream=None) -> None:
    """kq_gemv_argmax with the library's static scratch instead of a workspace."""
    _check(lib().kq_gemv_argmax_noalloc(_fmt(fmt), _ptr(W), _ptr(x), _ptr(y), N, K, M, _ptr(out),
                                        _stream(stream)), "kq_gemv_argmax_noalloc")


def kq_gemv_invariant(fmt, W, x, y, N: int, K: int, M: int, stream=None) -> None:
    """As kq_gemv, with column m bit-identical to a one-column call on x[m]."""
    _check(lib().kq_gemv_invariant(_fmt(fmt), _ptr(W), _ptr(x), _ptr(y), N, K, M, _stream(stream)),
           "kq_gemv_invariant")


def kq_moe_gemv_workspace_bytes(N: int, M: int, top_k: int, weighted: bool) -> int:
    return _check(lib().kq_moe_gemv_workspace_bytes(N, M, top_k, int(bool(weighted))),
                  "kq_moe_gemv_workspace_bytes")


def kq_moe_gemv(fmt, W_experts, x, route_ids, route_w, y, N: int, K: int, M: int, top_k: int,
                n_experts: int, x_per_slot: int, workspace=None, workspace_bytes: int = 0,
                stream=None) -> None:
    _check(lib().kq_moe_gemv(_fmt(fmt), _ptr(W_experts), _ptr(x), _ptr(route_ids), _ptr(route_w),
                             _ptr(y), N, K, M, top_k, n_experts, int(x_per_slot), _ptr(workspace),
                             workspace_bytes, _stream(stream)), "kq_moe_gemv")


def kq_moe_ffn_workspace_bytes(hidden: int, inter: int, M: int, top_k: int) -> int:
    return _check(lib().kq_moe_ffn_workspace_bytes(hidden, inter, M, top_k), "kq_moe_ffn_workspace_bytes")


def kq_moe_ffn(fmt, W_gate, W_up, W_down, x, route_ids, route_w, y, h_out, hidden: int, inter: int,
               M: int, top_k: int, n_experts: int, workspace, workspace_bytes: int,
               stream=None) -> None:
    _check(lib().kq_moe_ffn(_fmt(fmt), _ptr(W_gate), _ptr(W_up), _ptr(W_down), _ptr(x),
                            _ptr(route_ids), _ptr(route_w), _ptr(y), _ptr(h_out), hidden, inter, M,
                            top_k, n_experts, _ptr(workspace), workspace_bytes, _stream(stream)),
           "kq_moe_ffn")


def kq_argmax_workspace_bytes(N: int, M: int) -> int:
    return _check(lib().kq_argmax_workspace_bytes(N, M), "kq_argmax_workspace_bytes")


def kq_argmax(y, N: int, M: int, out, workspace, workspace_bytes: int, stream=None) -> None:
    _check(lib().kq_argmax(_ptr(y), N, M, _ptr(out), _ptr(workspace), workspace_bytes, _stream(stream)),
           "kq_argmax")


def kq_shortlist_copy_bytes(N: int, K: int) -> int:
    return _check(lib().kq_shortlist_copy_bytes(N, K), "kq_shortlist_copy_bytes")


def kq_shortlist_pack(q8_packed: np.ndarray, N: int, K: int, out: np.ndarray | None = None,
                      n_threads: int = 0) -> np.ndarray:
    """Bound copy (host uint8) of a packed Q8_0 matrix (host uint8)."""
    q8_packed = np.ascontiguousarray(q8_packed)
    nbytes = kq_shortlist_copy_bytes(N, K)
    if q8_packed.dtype != np.uint8 or q8_packed.nbytes < kq_packed_bytes("q8_0", N, K):
        raise ValueError("q8_packed must hold the packed Q8_0 matrix as uint8")
    if out is None:
        out = np.empty(nbytes, np.uint8)
    if not out.flags.c_contiguous or out.nbytes < nbytes:
        raise ValueError("out too small or not contiguous")
    _check(lib().kq_shortlist_pack(q8_packed.ctypes.data, N, K, out.ctypes.data, n_threads), "kq_shortlist_pack")
    return out


def kq_shortlist_workspace_bytes(N: int, K: int) -> int:
    return _check(lib().kq_shortlist_workspace_bytes(N, K), "kq_shortlist_workspace_bytes")


def kq_shortlist_argmax(W, W_copy, x, N: int, K: int, workspace, workspace_bytes: int, out, kept=None,
                        stream=None) -> None:
    """out[0] = argmax of the N scores of Q8_0 W against fp16 x, through its bound copy."""
    _check(lib().kq_shortlist_argmax(_ptr(W), _ptr(W_copy), _ptr(x), N, K, _ptr(workspace), workspace_bytes,
                                     _ptr(out), _ptr(kept), _stream(stream)), "kq_shortlist_argmax")


def _stage_array(stages):
    arr = (kq_stage * len(stages))()
    for i, st in enumerate(stages):
        arr[i].fmt = _fmt(st["fmt"])
        arr[i].reserved = 0
        arr[i].W = _ptr(st["W"])
        arr[i].x = _ptr(st["x"])
        arr[i].y = _ptr(st["y"])
        arr[i].N = int(st["N"])
        arr[i].K = int(st["K"])
        arr[i].y16 = _ptr(st.get("y16"))
    return arr


def kq_stack_plan_bytes(stages) -> int:
    """stages: list of dicts with fmt, W, x, y, N, K and optional y16 (device
    tensors or addresses)."""
    arr = _stage_array(stages)
    return _check(lib().kq_stack_plan_bytes(ctypes.cast(arr, ctypes.c_void_p), len(stages)),
                  "kq_stack_plan_bytes")


def kq_stack_plan(stages, plan, plan_bytes: int, stream=None) -> kq_stack_info:
    """stages: as for kq_stack_plan_bytes. Returns the filled kq_stack_info."""
    arr = _stage_array(stages)
    info = kq_stack_info()
    _check(lib().kq_stack_plan(ctypes.cast(arr, ctypes.c_void_p), len(stages), _ptr(plan), plan_bytes,
                               ctypes.addressof(info), _stream(stream)), "kq_stack_plan")
    return info


def kq_stack_run(plan, info: kq_stack_info, stream=None) -> None:
    _check(lib().kq_stack_run(_ptr(plan), ctypes.addressof(info), _stream(stream)), "kq_stack_run")


def kq_stack_status(plan, info: kq_stack_info, stream=None) -> int:
    err = ctypes.c_int(0)
    _check(lib().kq_stack_status(_ptr(plan), ctypes.addressof(info), ctypes.addressof(err),
                                 _stream(stream)), "kq_stack_status")
    return err.value
