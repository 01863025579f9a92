"""C-ABI checks that need no GPU: the library loads, exports every symbol the
header declares, and rejects bad arguments on the host before any HIP call."""
import ctypes
import functools
import os
import re

import numpy as np
import pytest

import block_quantized_gemv_kq_amd as kq

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kq.h")


def header_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(kq_\w+)\s*\(", src)))


def test_library_loads():
    assert kq.kq_version() == 100


def test_exports_every_declared_symbol():
    names = header_functions()
    assert len(names) >= 15
    L = ctypes.CDLL(kq.LIB_PATH)
    for n in names:
        assert hasattr(L, n), f"libkq.so does not export {n}"
    assert set(names) == set(kq.SIGNATURES), "binding and header disagree"


def test_status_strings():
    for code, name in [(0, "KQ_OK"), (-1, "KQ_ERR_ARG"), (-2, "KQ_ERR_FORMAT"), (-3, "KQ_ERR_SHAPE"),
                       (-4, "KQ_ERR_ALIGN"), (-5, "KQ_ERR_RANGE"), (-6, "KQ_ERR_HIP")]:
        assert kq.status_name(code) == name
    assert kq.status_name(-99) == "KQ_ERR_UNKNOWN"


def test_sizes():
    assert [kq.kq_block_bytes(f) for f in ("q8_0", "q4_0", "affine4", "q5_0", "q5_1")] == [34, 18, 20, 22, 24]
    assert kq.kq_packed_bytes("q5_0", 2560, 9728) == 2560 * 304 * 22
    assert kq.kq_packed_bytes("affine4", 4096, 2560) == 4096 * 80 * 20
    assert kq.kq_packed_bytes("q8_0", 151936, 2560) == 413265920
    assert kq.kq_packed_bytes("q4_0", 0, 1024) == 0
    L = kq.lib()
    assert L.kq_packed_bytes(5, 1, 32) == kq.KQ_ERR_FORMAT
    assert L.kq_packed_bytes(-1, 1, 32) == kq.KQ_ERR_FORMAT
    assert L.kq_packed_bytes(0, 1, 33) == kq.KQ_ERR_SHAPE
    assert L.kq_packed_bytes(0, 1, 0) == kq.KQ_ERR_SHAPE
    assert L.kq_packed_bytes(0, -1, 32) == kq.KQ_ERR_ARG
    assert L.kq_packed_bytes(0, 1, (1 << 20) + 32) == kq.KQ_ERR_SHAPE
    assert L.kq_block_bytes(7) == kq.KQ_ERR_FORMAT


# Fake, never-dereferenced device addresses: every call below must fail in
# validation, before any HIP call.
A16 = 0x10000
A4 = 0x10004


def _gemv_any(fmt=0, W=A16, x=A16, y=A16, N=8, K=64, M=1, entry="kq_gemv"):
    return getattr(kq.lib(), entry)(fmt, W, x, y, N, K, M, 0)


@pytest.mark.parametrize("entry", ["kq_gemv", "kq_gemv_invariant"])
def test_gemv_validation(entry):
    _gemv = functools.partial(_gemv_any, entry=entry)
    assert _gemv(fmt=5) == kq.KQ_ERR_FORMAT
    assert _gemv(K=48) == kq.KQ_ERR_SHAPE
    assert _gemv(K=0) == kq.KQ_ERR_SHAPE
    assert _gemv(K=-32) == kq.KQ_ERR_SHAPE
    assert _gemv(N=-1) == kq.KQ_ERR_ARG
    assert _gemv(M=65) == kq.KQ_ERR_ARG
    assert _gemv(M=-1) == kq.KQ_ERR_ARG
    assert _gemv(W=None) == kq.KQ_ERR_ARG
    assert _gemv(x=None) == kq.KQ_ERR_ARG
    assert _gemv(y=None) == kq.KQ_ERR_ARG
    assert _gemv(W=A16 + 2) == kq.KQ_ERR_ALIGN
    assert _gemv(y=A16 + 1) == kq.KQ_ERR_ALIGN
    assert _gemv(x=A4) == kq.KQ_ERR_ALIGN
    assert "16-byte" in kq.last_error()
    # empty problems are valid and launch nothing
    assert _gemv(M=0, W=None, x=None, y=None) == kq.KQ_OK
    assert _gemv(N=0, W=None, x=None, y=None) == kq.KQ_OK


def _moe(fmt=1, W=A16, x=A16, ids=A16, rw=None, y=A16, N=64, K=64, M=2, top_k=2, E=4, xps=0,
         ws=None, wsb=0):
    return kq.lib().kq_moe_gemv(fmt, W, x, ids, rw, y, N, K, M, top_k, E, xps, ws, wsb, 0)


def test_moe_validation():
    assert _moe(top_k=0) == kq.KQ_ERR_ARG
    assert _moe(top_k=5) == kq.KQ_ERR_ARG        # > n_experts
    assert _moe(E=0) == kq.KQ_ERR_ARG
    assert _moe(xps=2) == kq.KQ_ERR_ARG
    assert _moe(fmt=9) == kq.KQ_ERR_FORMAT
    assert _moe(K=40) == kq.KQ_ERR_SHAPE
    assert _moe(ids=None) == kq.KQ_ERR_ARG
    assert _moe(x=A4) == kq.KQ_ERR_ALIGN
    assert _moe(W=A16 + 2) == kq.KQ_ERR_ALIGN
    # weighted output needs M*top_k*N*4 bytes of workspace
    need = kq.kq_moe_gemv_workspace_bytes(64, 2, 2, True)
    assert need == 2 * 2 * 64 * 4
    assert kq.kq_moe_gemv_workspace_bytes(64, 2, 2, False) == 0
    assert _moe(rw=A16) == kq.KQ_ERR_ARG
    assert _moe(rw=A16, ws=A16, wsb=need - 1) == kq.KQ_ERR_ARG
    assert _moe(rw=A16, ws=A4, wsb=need) == kq.KQ_ERR_ALIGN
    assert _moe(M=0) == kq.KQ_OK


def test_limit_constants_match_header():
    src = open(HEADER).read()
    for name in ("KQ_MAX_M", "KQ_MAX_K", "KQ_MAX_N"):
        m = re.search(r"#define\s+%s\s+(.+?)\s*/\*" % name, src)
        assert m, name
        assert eval(m.group(1), {}) == getattr(kq, name), name


def test_moe_ffn_validation():
    L = kq.lib()
    need = kq.kq_moe_ffn_workspace_bytes(2048, 768, 4, 8)
    assert need >= 4 * 8 * 768 * 2 + 4 * 8 * 2048 * 4

    def call(fmt=1, rw=A16, ws=A16, wsb=need, hidden=2048, inter=768, top_k=8, E=128):
        return L.kq_moe_ffn(fmt, A16, A16, A16, A16, A16, rw, A16, None, hidden, inter, 4, top_k, E,
                            ws, wsb, 0)
    assert call(rw=None) == kq.KQ_ERR_ARG
    assert call(wsb=need - 1) == kq.KQ_ERR_ARG
    assert call(ws=A4) == kq.KQ_ERR_ALIGN
    assert call(hidden=2080) == kq.KQ_ERR_SHAPE    # Q4_0 needs hidden % 64 == 0
    assert call(inter=770) == kq.KQ_ERR_SHAPE
    assert call(top_k=129) == kq.KQ_ERR_ARG


def test_gemv_ws_sizes_and_validation():
    """kq_gemv_ws: the workspace it asks for (M * N * 4 bytes per K split:
    4 splits for the 2560 x 9728 down projection at 4..16 columns, none for
    2560 x 4096, for one column, past 16 columns or for many row tiles), and
    the host checks before any device call."""
    L = kq.lib()
    for fmt in (0, 1, 2, 3, 4):
        assert kq.kq_gemv_workspace_bytes(fmt, 2560, 9728, 8) == 4 * 8 * 2560 * 4
        assert kq.kq_gemv_workspace_bytes(fmt, 2560, 9728, 16) == 4 * 16 * 2560 * 4
        assert kq.kq_gemv_workspace_bytes(fmt, 2560, 4096, 8) == 0
        assert kq.kq_gemv_workspace_bytes(fmt, 2560, 9728, 1) == 0
        assert kq.kq_gemv_workspace_bytes(fmt, 2560, 9728, 32) == 0
        assert kq.kq_gemv_workspace_bytes(fmt, 19456, 9728, 8) == 0
    assert L.kq_gemv_workspace_bytes(7, 2560, 9728, 8) == kq.KQ_ERR_FORMAT
    assert L.kq_gemv_workspace_bytes(0, 2560, 100, 8) == kq.KQ_ERR_SHAPE
    assert L.kq_gemv_workspace_bytes(0, 2560, 9728, 65) == kq.KQ_ERR_ARG
    need = kq.kq_gemv_workspace_bytes(2, 2560, 9728, 8)

    def call(fmt=2, W=A16, x=A16, y=A16, N=2560, K=9728, M=8, ws=A16, wsb=need):
        return L.kq_gemv_ws(fmt, W, x, y, N, K, M, ws, wsb, 0)
    assert call(ws=None) == kq.KQ_ERR_ARG
    assert call(wsb=need - 4) == kq.KQ_ERR_ARG
    assert call(ws=A16 + 8) == kq.KQ_ERR_ALIGN
    assert call(wsb=-1) == kq.KQ_ERR_ARG
    assert call(fmt=9) == kq.KQ_ERR_FORMAT
    assert call(x=A4) == kq.KQ_ERR_ALIGN
    assert call(M=0, W=None, x=None, y=None, ws=None, wsb=0) == kq.KQ_OK


def test_gemv_argmax_validation():
    L = kq.lib()
    need = kq.kq_gemv_argmax_workspace_bytes(0, 151936, 2560, 1)
    assert need >= 151936 // 16 * 8 // 4          # partials of every workgroup
    assert kq.kq_gemv_argmax_workspace_bytes(0, 151936, 2560, 8) >= 8 * kq.kq_argmax_workspace_bytes(151936, 1)
    assert L.kq_gemv_argmax_workspace_bytes(0, 100, 48, 1) == kq.KQ_ERR_SHAPE

    def call(fmt=0, W=A16, x=A16, y=A16, N=151936, K=2560, M=1, out=A16, ws=A16, wsb=need):
        return L.kq_gemv_argmax(fmt, W, x, y, N, K, M, out, ws, wsb, 0)
    assert call(fmt=7) == kq.KQ_ERR_FORMAT
    assert call(N=0) == kq.KQ_ERR_ARG
    assert call(out=None) == kq.KQ_ERR_ARG
    assert call(wsb=need - 8) == kq.KQ_ERR_ARG
    assert call(ws=None) == kq.KQ_ERR_ARG
    assert call(out=A16 + 2) == kq.KQ_ERR_ALIGN
    assert call(ws=A16 + 4) == kq.KQ_ERR_ALIGN
    assert call(x=A4) == kq.KQ_ERR_ALIGN
    assert call(M=0, W=None, x=None, y=None, out=None, ws=None, wsb=0) == kq.KQ_OK


def test_argmax_validation():
    L = kq.lib()
    need = kq.kq_argmax_workspace_bytes(151936, 3)
    assert need == 3 * ((151936 + 2047) // 2048) * 8
    assert L.kq_argmax(A16, 0, 1, A16, A16, need, 0) == kq.KQ_ERR_ARG
    assert L.kq_argmax(A16, 151936, 65, A16, A16, need, 0) == kq.KQ_ERR_ARG
    assert L.kq_argmax(A16, 151936, 3, A16, A16, need - 8, 0) == kq.KQ_ERR_ARG
    assert L.kq_argmax(A16 + 2, 151936, 3, A16, A16, need, 0) == kq.KQ_ERR_ALIGN
    assert L.kq_argmax(A16, 151936, 0, A16, None, 0, 0) == kq.KQ_OK


def test_pack_validation():
    W = np.zeros((2, 32), np.float32)
    with pytest.raises(kq.KQError) as e:
        kq.kq_pack(5, W)
    assert e.value.status == kq.KQ_ERR_FORMAT
    W[0, 3] = np.inf
    with pytest.raises(kq.KQError) as e:
        kq.kq_pack("q8_0", W)
    assert e.value.status == kq.KQ_ERR_RANGE
    W[0, 3] = 1e6   # affine4: range/15 fine, but bias fp16(lo) ok; q8_0 d = 1e6/127 < 65504
    kq.kq_pack("q8_0", W)
    W[0, 3] = -70000.0
    with pytest.raises(kq.KQError) as e:
        kq.kq_pack("affine4", W)    # b = fp16(-70000) overflows
    assert e.value.status == kq.KQ_ERR_RANGE
    assert kq.lib().kq_pack(0, None, 1, 32, None, 1) == kq.KQ_ERR_ARG
    assert kq.lib().kq_pack(0, None, 0, 32, None, 1) == kq.KQ_OK


def _stage_arr(sts):
    arr = (kq.kq_stage * len(sts))()
    for i, st in enumerate(sts):
        arr[i].fmt = kq._fmt(st["fmt"])
        arr[i].reserved = st.get("reserved", 0)
        arr[i].W, arr[i].x, arr[i].y = st["W"], st["x"], st["y"]
        arr[i].N, arr[i].K = st["N"], st["K"]
        arr[i].y16 = st.get("y16")
    return arr


def test_stack_validation():
    L = kq.lib()
    base = dict(fmt="affine4", W=A16, x=A16, y=0x200000, N=64, K=2560)

    def nbytes(*sts):
        return L.kq_stack_plan_bytes(ctypes.cast(_stage_arr(sts), ctypes.c_void_p), len(sts))

    def plan(**over):
        st = dict(base)
        st.update(over)
        info = kq.kq_stack_info()
        return L.kq_stack_plan(ctypes.cast(_stage_arr([st]), ctypes.c_void_p), 1, 0x100000, 1 << 30,
                               ctypes.addressof(info), 0)
    assert L.kq_stack_plan_bytes(ctypes.cast(_stage_arr([base]), ctypes.c_void_p), 0) == kq.KQ_ERR_ARG
    assert L.kq_stack_plan_bytes(None, 1) == kq.KQ_ERR_ARG
    one = nbytes(base)
    assert one >= 128 + 32 * 4 * 1024
    assert plan(fmt=9) == kq.KQ_ERR_FORMAT
    assert plan(K=48) == kq.KQ_ERR_SHAPE
    assert plan(fmt="q8_0", K=96) == kq.KQ_ERR_SHAPE            # Q8_0 needs K % 64 == 0
    assert plan(K=16384 + 32) == kq.KQ_ERR_SHAPE                # longer than the x stage in LDS
    assert plan(fmt="q8_0", K=16384 + 64) == kq.KQ_ERR_SHAPE
    assert plan(N=0) == kq.KQ_ERR_ARG
    assert plan(W=None) == kq.KQ_ERR_ARG
    assert plan(reserved=1) == kq.KQ_ERR_ARG
    assert plan(x=A4) == kq.KQ_ERR_ALIGN
    assert plan(y16=0x300001) == kq.KQ_ERR_ALIGN
    assert plan(y16=0x200000 + 64) == kq.KQ_ERR_ARG             # y and y16 overlap


def test_stack_dataflow_rules():
    """Which stage pairs a plan accepts, and the tagged buffers it sizes: a
    stage may read x from inside an earlier stage's y16 (4-element aligned);
    every other overlap of outputs with outputs or inputs is refused."""
    L = kq.lib()

    def nbytes(*sts):
        return L.kq_stack_plan_bytes(ctypes.cast(_stage_arr(sts), ctypes.c_void_p), len(sts))
    s0 = dict(fmt="affine4", W=A16, x=0x100000, y=0x200000, N=6144, K=2560, y16=0x300000)
    free = nbytes(s0, dict(s0, x=0x110000, y=0x210000, y16=0x310000, N=2560, K=4096))
    # stage 1 reads the first 4096 values of stage 0's fp16 output: stage 0's
    # 6144 outputs get a tagged copy (4 bytes each) in the plan
    chained = nbytes(s0, dict(s0, x=0x300000, y=0x210000, y16=None, N=2560, K=4096))
    assert chained - free == 6144 * 4 * 8    # 8 copies, read by different workgroups
    # reading from the middle of it (element 2048, a multiple of 4) is allowed
    assert nbytes(s0, dict(s0, x=0x300000 + 2 * 2048, y=0x210000, y16=None, N=2560, K=4096)) == chained
    # ... from element 2 is not (the tagged words are read in 16-byte chunks)
    assert nbytes(s0, dict(s0, x=0x300000 + 4, y=0x210000, y16=None, N=2560, K=2560)) == kq.KQ_ERR_ALIGN
    # x running past the end of the earlier output
    assert nbytes(s0, dict(s0, x=0x300000 + 2 * 4096, y=0x210000, y16=None, N=2560, K=4096)) == kq.KQ_ERR_ARG
    # x inside a LATER stage's output, or the stage's own
    assert nbytes(dict(s0, x=0x310000, y16=None), dict(s0, x=0x110000, y=0x210000, y16=0x310000)) == kq.KQ_ERR_ARG
    assert nbytes(dict(s0, x=0x300000)) == kq.KQ_ERR_ARG
    # x inside an fp32 output
    assert nbytes(s0, dict(s0, x=0x200000, y=0x210000, y16=None)) == kq.KQ_ERR_ARG
    # two stages writing overlapping outputs
    assert nbytes(s0, dict(s0, x=0x110000, y=0x200000 + 4 * 100, y16=None)) == kq.KQ_ERR_ARG
    assert nbytes(s0, dict(s0, x=0x110000, y=0x210000, y16=0x300000 + 8)) == kq.KQ_ERR_ARG


def test_stack_run_checks():
    L = kq.lib()
    info = kq.kq_stack_info()
    assert L.kq_stack_run(0x100000, ctypes.addressof(info), 0) == kq.KQ_ERR_ARG   # info not filled


def test_set_tuning_validates_and_clears():
    L = kq.lib()
    assert L.kq_set_tuning(b"no_such_knob", b"1") == kq.KQ_ERR_ARG
    assert L.kq_set_tuning(b"force_path", b"x") == kq.KQ_ERR_ARG
    assert L.kq_set_tuning(b"mfma_variant", b"fast") == kq.KQ_ERR_ARG
    assert L.kq_set_tuning(b"mfma_s", b"3q") == kq.KQ_ERR_ARG
    assert L.kq_set_tuning(b"mfma_s", b"-1") == kq.KQ_ERR_ARG
    for name, value in [(b"force_path", b"m"), (b"mfma_variant", b"chunk_split"), (b"mfma_xf", b"0"),
                        (b"moe_unfused", b"1")]:
        assert L.kq_set_tuning(name, value) == kq.KQ_OK
        assert L.kq_set_tuning(name, None) == kq.KQ_OK
    assert L.kq_set_tuning(b"valu_g", b"16") == kq.KQ_OK
    assert L.kq_set_tuning(None, None) == kq.KQ_OK


def test_environment_does_not_steer_the_library():
    """The library never reads the environment: no getenv in its sources."""
    csrc = os.path.join(ROOT, "block_quantized_gemv_kq_amd", "csrc")
    for name in os.listdir(csrc):
        with open(os.path.join(csrc, name)) as f:
            assert "getenv" not in f.read(), name


def test_stack_plan_rejects_five_bit_formats():
    """The persistent chain takes Q8_0, Q4_0 and affine4 only (host check)."""
    for fmt in (kq.KQ_Q5_0, kq.KQ_Q5_1):
        arr = _stage_arr([dict(fmt=fmt, W=A16, x=A16, y=A16 + 4096, N=64, K=256)])
        assert kq.lib().kq_stack_plan_bytes(arr, 1) == kq.KQ_ERR_FORMAT


def test_shortlist_sizes_and_validation():
    L = kq.lib()
    assert kq.kq_shortlist_copy_bytes(151936, 2560) == 151936 * (22 * 80 + 4)
    assert L.kq_shortlist_copy_bytes(100, 2048 + 32) == kq.KQ_ERR_SHAPE     # K not a multiple of 256
    assert L.kq_shortlist_copy_bytes(100, 16384 + 256) == kq.KQ_ERR_SHAPE   # above KQ_SHORTLIST_MAX_K
    assert L.kq_shortlist_copy_bytes(0, 2560) == kq.KQ_ERR_ARG
    assert L.kq_shortlist_copy_bytes(8_000_000, 16384) == kq.KQ_ERR_SHAPE   # the matrix reaches 2 GiB
    need = kq.kq_shortlist_workspace_bytes(151936, 2560)
    assert need >= 4 * 151936 + 12 * (151936 // 256)

    def call(W=A16, Wc=A16, x=A16, N=151936, K=2560, ws=A16, wsb=need, out=A16, kept=None):
        return L.kq_shortlist_argmax(W, Wc, x, N, K, ws, wsb, out, kept, 0)
    assert call(K=2304 + 32) == kq.KQ_ERR_SHAPE
    assert call(N=0) == kq.KQ_ERR_ARG
    assert call(Wc=None) == kq.KQ_ERR_ARG
    assert call(out=None) == kq.KQ_ERR_ARG
    assert call(wsb=need - 4) == kq.KQ_ERR_ARG
    assert call(ws=None) == kq.KQ_ERR_ARG
    assert call(W=A16 + 4) == kq.KQ_ERR_ALIGN
    assert call(Wc=A16 + 8) == kq.KQ_ERR_ALIGN
    assert call(x=A4) == kq.KQ_ERR_ALIGN
    assert call(out=A16 + 2) == kq.KQ_ERR_ALIGN
    assert call(kept=A16 + 2) == kq.KQ_ERR_ALIGN
    assert call(ws=A16 + 16) == kq.KQ_ERR_ALIGN


def test_shortlist_pack_validation():
    L = kq.lib()
    q8 = np.zeros(kq.kq_packed_bytes("q8_0", 2, 256), np.uint8)
    out = np.zeros(kq.kq_shortlist_copy_bytes(2, 256), np.uint8)
    assert L.kq_shortlist_pack(None, 2, 256, out.ctypes.data, 1) == kq.KQ_ERR_ARG
    assert L.kq_shortlist_pack(q8.ctypes.data, 2, 288, out.ctypes.data, 1) == kq.KQ_ERR_SHAPE
    q8[34 * 9 + 1] = 0x7C          # row 1, block 1: scale bits 0x7C00 = +inf
    with pytest.raises(kq.KQError) as e:
        kq.kq_shortlist_pack(q8, 2, 256)
    assert e.value.status == kq.KQ_ERR_RANGE
