"""Guard bytes around every buffer the library writes (y, y16, h, argmax
outputs, caller workspaces): each sits between 4 KiB regions filled with a
sentinel byte, and after each call the guards must be intact and every output
element written (no sentinel left). Covers every kernel path at ragged shapes.
Also the dispatch log (the log tuning override): one line per launch."""
import numpy as np
import pytest

import block_quantized_gemv_kq_amd as kq
from synth import inputs as S
from tests import gpu_util as U

pytestmark = pytest.mark.gpu

GUARD = 4096
SENT = 0xFF   # all-ones: NaN as fp16 and fp32, -1 as an index; no valid output is either


class Guarded:
    """A device buffer of `nbytes` (elements of `elem` bytes) with GUARD
    sentinel bytes on each side."""

    def __init__(self, nbytes, elem=4):
        torch = U.torch_cuda()
        self.n = int(nbytes)
        self.elem = elem
        self.buf = torch.full((GUARD + (self.n + 255) // 256 * 256 + GUARD,), SENT, dtype=torch.uint8, device="cuda")
        self.ptr = self.buf.data_ptr() + GUARD

    def check(self, fully_written=True, what=""):
        h = U.to_host(self.buf)
        assert np.all(h[:GUARD] == SENT), f"{what}: guard before the buffer overwritten"
        assert np.all(h[GUARD + self.n:] == SENT), f"{what}: guard after the buffer overwritten"
        if fully_written:
            body = h[GUARD:GUARD + self.n].view(np.uint32 if self.elem == 4 else np.uint16)
            assert not np.any(body == (0xFFFFFFFF if self.elem == 4 else 0xFFFF)), f"{what}: output not written"


def _inputs(fmt, N, K, M, seed):
    W = S.weights((88, seed, N, K), N, K)
    x = S.activations((88, seed, K), K, M)
    packed, _ = U.quantize_both(fmt, W)
    return U.to_dev(packed), U.to_dev(x)


@pytest.mark.parametrize("fmt", ("q8_0", "q4_0", "affine4", "q5_0", "q5_1"))
@pytest.mark.parametrize("N,K", [(333, 1024), (1001, 2560), (37, 96), (4099, 256)])
@pytest.mark.parametrize("M", (1, 3, 5, 17, 48))
@pytest.mark.parametrize("entry", ("kq_gemv", "kq_gemv_invariant"))
def test_gemv_guards(fmt, N, K, M, entry):
    Wd, xd = _inputs(fmt, N, K, M, 1)
    y = Guarded(4 * M * N)
    getattr(kq, entry)(fmt, Wd, xd, y.ptr, N, K, M)
    y.check(what=f"{entry} {fmt} {N}x{K} M={M}")


@pytest.mark.parametrize("fmt", ("q8_0", "affine4"))
@pytest.mark.parametrize("path", ("generic", "valu", "lds", "mfma"))
@pytest.mark.parametrize("M", (1, 4, 9))
def test_forced_paths_guards(fmt, path, M):
    N, K = 301, 2560
    Wd, xd = _inputs(fmt, N, K, M, 2)
    y = Guarded(4 * M * N)
    with U.tuning({"force_path": path[0]}):
        kq.kq_gemv(fmt, Wd, xd, y.ptr, N, K, M)
    y.check(what=f"{fmt} {path} M={M}")


@pytest.mark.parametrize("fmt", ("q8_0", "q5_1"))
@pytest.mark.parametrize("N,M", [(50001, 1), (50001, 3), (4097, 8)])
def test_argmax_guards(fmt, N, M):
    K = 512
    Wd, xd = _inputs(fmt, N, K, M, 3)
    y, out = Guarded(4 * M * N), Guarded(4 * M)
    wsb = kq.kq_gemv_argmax_workspace_bytes(fmt, N, K, M)
    ws = Guarded(wsb)
    kq.kq_gemv_argmax(fmt, Wd, xd, y.ptr, N, K, M, out.ptr, ws.ptr, wsb)
    y.check(what="gemv_argmax y")
    out.check(what="gemv_argmax out")
    ws.check(fully_written=False, what="gemv_argmax workspace")
    y2, out2 = Guarded(4 * M * N), Guarded(4 * M)
    kq.kq_gemv_argmax_noalloc(fmt, Wd, xd, y2.ptr, N, K, M, out2.ptr)
    y2.check(what="noalloc y")
    out2.check(what="noalloc out")
    wsa = kq.kq_argmax_workspace_bytes(N, M)
    ws2, out3 = Guarded(wsa), Guarded(4 * M)
    kq.kq_argmax(y.ptr, N, M, out3.ptr, ws2.ptr, wsa)
    out3.check(what="argmax out")
    ws2.check(fully_written=False, what="argmax workspace")


@pytest.mark.parametrize("fmt", ("q4_0", "q5_0"))
@pytest.mark.parametrize("M", (1, 4))
def test_moe_guards(fmt, M):
    E, hidden, inter, top_k = 16, 512, 256, 4
    def experts(n, k, which):
        return U.to_dev(np.concatenate([kq.kq_pack(fmt, S.weights((89, e, which), n, k)).reshape(-1)
                                        for e in range(E)]))
    Wg, Wu, Wdn = experts(inter, hidden, 0), experts(inter, hidden, 1), experts(hidden, inter, 2)
    x = U.to_dev(S.activations((89, M), hidden, M))
    ids, rw = S.route_table(89, M, E, top_k)
    idd, rwd = U.to_dev(ids), U.to_dev(rw)
    y, h = Guarded(4 * M * hidden), Guarded(2 * M * top_k * inter, elem=2)
    wsb = kq.kq_moe_ffn_workspace_bytes(hidden, inter, M, top_k)
    ws = Guarded(wsb)
    kq.kq_moe_ffn(fmt, Wg, Wu, Wdn, x, idd, rwd, y.ptr, h.ptr, hidden, inter, M, top_k, E, ws.ptr, wsb)
    y.check(what="moe_ffn y")
    h.check(what="moe_ffn h")
    ws.check(fully_written=False, what="moe_ffn workspace")
    ys = Guarded(4 * M * top_k * inter)
    kq.kq_moe_gemv(fmt, Wg, x, idd, None, ys.ptr, inter, hidden, M, top_k, E, 0, None, 0)
    ys.check(what="moe_gemv per-slot y")


def test_stack_guards():
    fmt, K = "affine4", 512
    Ns = (520, 512, 777)   # each stage reads the first K values of the previous stage's y16
    torch = U.torch_cuda()
    Ws = [_inputs(fmt, n, K, 1, 4 + i)[0] for i, n in enumerate(Ns)]
    x0 = U.to_dev(S.activations((88, 9), K, 1)[0])
    ys = [Guarded(4 * n) for n in Ns]
    y16s = [Guarded(2 * n, elem=2) for n in Ns]
    stages = []
    prev = None
    for i, n in enumerate(Ns):
        stages.append(dict(fmt=fmt, W=Ws[i], x=x0 if prev is None else prev, y=ys[i].ptr, N=n, K=K,
                           y16=y16s[i].ptr))
        prev = y16s[i].ptr
    nb = kq.kq_stack_plan_bytes(stages)
    plan = torch.zeros(nb, dtype=torch.uint8, device="cuda")
    info = kq.kq_stack_plan(stages, plan, nb)
    kq.kq_stack_run(plan, info)
    assert kq.kq_stack_status(plan, info) == 0
    for i in range(len(Ns)):
        ys[i].check(what=f"stack y{i}")
        y16s[i].check(what=f"stack y16 {i}")


def test_dispatch_log(capfd):
    fmt, N, K = "affine4", 4099, 2560
    Wd, xd = _inputs(fmt, N, K, 8, 5)
    y = U.empty_dev((8, N))
    with U.tuning({"log": "1"}):
        kq.kq_gemv(fmt, Wd, xd, y, N, K, 1)
        kq.kq_gemv(fmt, Wd, xd, y, N, K, 8)
        U.torch_cuda().cuda.synchronize()
    kq.kq_gemv(fmt, Wd, xd, y, N, K, 1)          # log off again: no line
    U.torch_cuda().cuda.synchronize()
    err = capfd.readouterr().err
    lines = [ln for ln in err.splitlines() if ln.startswith("kq: ")]
    assert len(lines) == 2, err
    assert "k_gemv_lds fmt=affine4 N=4099 K=2560 M=1" in lines[0]
    assert "k_gemv_mfma" in lines[1] and "M=8" in lines[1]
