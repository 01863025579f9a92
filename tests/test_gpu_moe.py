"""GPU parity of the routed-expert calls (kq_moe_gemv, kq_moe_ffn) against the
oracle, through the C ABI. Experts nobody routes to are filled with bytes
that dequantize to NaN/huge values, so reading one would show in the output."""
import numpy as np
import pytest

import block_quantized_gemv_kq_amd as kq
from oracle import formats as F
from oracle import ref as R
from synth import inputs as S
from tests import gpu_util as U

pytestmark = pytest.mark.gpu


class Experts:
    """n_experts packed matrices back to back on the device; only the ones
    in `used` hold real weights (the oracle quantizes only those)."""

    def __init__(self, fmt, n_experts, N, K, used, seed_fn):
        self.fmt, self.N, self.K = fmt, N, K
        eb = kq.kq_packed_bytes(fmt, N, K)
        host = np.full((n_experts, eb), 0xFF, np.uint8)      # poison: fp16 NaN scales
        self.fields = {}
        for e in sorted(set(int(v) for v in used)):
            W = S.weights(seed_fn(e), N, K)
            packed, fields = U.quantize_both(fmt, W)
            host[e] = packed.reshape(-1)
            self.fields[e] = fields
        self.dev = U.to_dev(host)

    def field_list(self, n):
        return [self.fields.get(e) for e in range(n)]


def _route(M, E, top_k, seed):
    ids, rw = S.route_table(70 + seed, M, E, top_k)
    return ids, rw


@pytest.mark.parametrize("fmt", ("q4_0", "q8_0", "affine4"))
@pytest.mark.parametrize("M,top_k,E", [(1, 8, 32), (4, 8, 32), (16, 8, 32), (3, 1, 4), (5, 4, 4)])
def test_moe_gemv_per_slot(fmt, M, top_k, E):
    N, K = 96, 512
    ids, rw = _route(M, E, top_k, M)
    ex = Experts(fmt, E, N, K, ids.ravel(), lambda e: (71, e, 0, 0))
    x = S.activations((71, 0, 0), K, M)
    y = U.empty_dev((M, top_k, N))
    kq.kq_moe_gemv(fmt, ex.dev, U.to_dev(x), U.to_dev(ids), None, y, N, K, M, top_k, E, 0)
    yg = U.to_host(y)
    yr, ad = R.moe_gemv(fmt, ex.field_list(E), x, ids, None, False)
    U.assert_parity(yg, yr, ad, f"moe per-slot {fmt} M={M}")


@pytest.mark.parametrize("fmt", ("q4_0", "affine4"))
@pytest.mark.parametrize("M", (1, 4, 16))
def test_moe_gemv_weighted_x_per_slot(fmt, M):
    N, K, E, top_k = 128, 256, 16, 4
    ids, rw = _route(M, E, top_k, 10 + M)
    ex = Experts(fmt, E, N, K, ids.ravel(), lambda e: (72, e, 0, 0))
    x = S.activations((72, 0, 0), K, M * top_k).reshape(M, top_k, K)
    y = U.empty_dev((M, N))
    wsb = kq.kq_moe_gemv_workspace_bytes(N, M, top_k, True)
    ws = U.empty_dev((wsb // 4,))
    kq.kq_moe_gemv(fmt, ex.dev, U.to_dev(x), U.to_dev(ids), U.to_dev(rw), y, N, K, M, top_k, E, 1, ws, wsb)
    yg = U.to_host(y)
    yr, ad = R.moe_gemv(fmt, ex.field_list(E), x, ids, rw, True)
    U.assert_parity(yg, yr, ad, f"moe weighted {fmt} M={M}")


def test_moe_shared_expert_dedup_and_duplicates():
    """Every token routed to the same experts (and one token naming an expert
    twice): each expert's weights serve all its slots."""
    fmt, N, K, E = "q4_0", 64, 256, 8
    ids = np.array([[3, 5], [3, 5], [5, 3], [1, 1]], np.int32)
    rw = np.full(ids.shape, 0.5, np.float32)
    ex = Experts(fmt, E, N, K, ids.ravel(), lambda e: (73, e, 0, 0))
    x = S.activations((73, 0, 0), K, 4)
    y = U.empty_dev((4, 2, N))
    kq.kq_moe_gemv(fmt, ex.dev, U.to_dev(x), U.to_dev(ids), None, y, N, K, 4, 2, E, 0)
    yr, ad = R.moe_gemv(fmt, ex.field_list(E), x, ids, None, False)
    U.assert_parity(U.to_host(y), yr, ad, "dedup")


def test_moe_bad_route_id_gives_nan_without_reading():
    fmt, N, K, E = "q4_0", 64, 256, 4
    ids = np.array([[0, 7], [-1, 2]], np.int32)
    ex = Experts(fmt, E, N, K, [0, 2], lambda e: (74, e, 0, 0))
    x = S.activations((74, 0, 0), K, 2)
    y = U.empty_dev((2, 2, N))
    kq.kq_moe_gemv(fmt, ex.dev, U.to_dev(x), U.to_dev(ids), None, y, N, K, 2, 2, E, 0)
    yg = U.to_host(y)
    assert np.all(np.isnan(yg[0, 1])) and np.all(np.isnan(yg[1, 0]))
    assert np.all(np.isfinite(yg[0, 0])) and np.all(np.isfinite(yg[1, 1]))


@pytest.mark.parametrize("M", (1, 4, 16))
def test_moe_ffn_workload(M):
    """The 128-expert top-8 Q4_0 MoE layer (hidden 2048, expert FFN 768):
    gate/up with SwiGLU then down with the fixed-order weighted sum."""
    L = S.MOE_Q4_0
    ids, rw = S.route_table(L.workload_id, M, L.n_experts, L.top_k)
    used = ids.ravel()
    gate = Experts(L.fmt, L.n_experts, L.inter, L.hidden, used, lambda e: L.weight_seed(e, 0))
    up = Experts(L.fmt, L.n_experts, L.inter, L.hidden, used, lambda e: L.weight_seed(e, 1))
    down = Experts(L.fmt, L.n_experts, L.hidden, L.inter, used, lambda e: L.weight_seed(e, 2))
    x = S.activations(L.act_seed_prefix(), L.hidden, M)
    y = U.empty_dev((M, L.hidden))
    h = U.empty_dev((M, L.top_k, L.inter), "float16")
    wsb = kq.kq_moe_ffn_workspace_bytes(L.hidden, L.inter, M, L.top_k)
    ws = U.empty_dev((wsb // 4 + 1,))
    kq.kq_moe_ffn(L.fmt, gate.dev, up.dev, down.dev, U.to_dev(x), U.to_dev(ids), U.to_dev(rw), y, h,
                  L.hidden, L.inter, M, L.top_k, L.n_experts, ws, wsb)
    yg, hg = U.to_host(y), U.to_host(h)
    E = L.n_experts
    # h: the GPU's g and u may differ from the oracle's within the GEMV
    # tolerance; h may then differ by that error carried through
    # silu(g)*u, plus one fp16 rounding step (2^-10 relative, 2^-24 absolute).
    _, _, (g, g_abs), (u, u_abs), h_ref = R.moe_ffn(L.fmt, gate.field_list(E), up.field_list(E),
                                                   down.field_list(E), x, ids, rw)
    sig = 1.0 / (1.0 + np.exp(-g))
    dsilu = sig * (1.0 + g * (1.0 - sig))
    tol_h = (np.abs(dsilu * u) * R.tolerance(g_abs) + np.abs(g * sig) * R.tolerance(u_abs)
             + 2.0 ** -10 * np.abs(h_ref.astype(np.float64)) + 2.0 ** -24)
    assert np.all(np.abs(hg.astype(np.float64) - h_ref.astype(np.float64)) <= tol_h)
    # down + weighted sum checked on exactly the GPU's h
    yr, ad, *_ = R.moe_ffn(L.fmt, gate.field_list(E), up.field_list(E), down.field_list(E), x, ids,
                           rw, h_override=hg)
    U.assert_parity(yg, yr, ad, f"moe ffn M={M}")


def _weighted_gemv(fmt, ex, x, ids, rw, N, K, M, top_k, E, xps, unfused):
    y = U.empty_dev((M, N))
    wsb = kq.kq_moe_gemv_workspace_bytes(N, M, top_k, True)
    ws = U.empty_dev((wsb // 4 + 1,))
    with U.tuning({"moe_unfused": "1"} if unfused else {}):
        kq.kq_moe_gemv(fmt, ex.dev, U.to_dev(x), U.to_dev(ids), U.to_dev(rw), y, N, K, M, top_k, E, xps, ws, wsb)
    return U.to_host(y)


@pytest.mark.parametrize("fmt", ("q4_0", "q8_0", "affine4"))
@pytest.mark.parametrize("xps", (0, 1))
@pytest.mark.parametrize("top_k,ids_row", [(8, None), (2, [3, 3]), (3, [5, -1, 2]), (16, None)])
def test_moe_one_token_weighted_is_one_launch_with_same_bits(fmt, xps, top_k, ids_row):
    """One token, weighted: the single-launch down + slot-order sum gives the
    bits of the per-slot kernel followed by the weighted-sum kernel (the
    moe_unfused path), including a duplicated expert and a bad id (NaN)."""
    N, K, E = 300, 768, 32
    if ids_row is None:
        ids, rw = _route(1, E, top_k, 40 + top_k)
    else:
        ids = np.array([ids_row], np.int32)
        rw = np.linspace(0.2, 0.9, top_k, dtype=np.float32)[None, :]
    ex = Experts(fmt, E, N, K, [v for v in ids.ravel() if 0 <= v < E], lambda e: (75, e, 0, 0))
    x = S.activations((75, top_k, 0), K, top_k if xps else 1)
    if xps:
        x = x.reshape(1, top_k, K)
    y1 = _weighted_gemv(fmt, ex, x, ids, rw, N, K, 1, top_k, E, xps, False)
    y2 = _weighted_gemv(fmt, ex, x, ids, rw, N, K, 1, top_k, E, xps, True)
    assert np.array_equal(y1.view(np.uint32), y2.view(np.uint32)) or (
        np.all(np.isnan(y1)) and np.all(np.isnan(y2)))
    if np.any(ids < 0):
        assert np.all(np.isnan(y1))
    else:
        yr, ad = R.moe_gemv(fmt, ex.field_list(E), x, ids, rw, bool(xps))
        U.assert_parity(y1, yr, ad, f"moe one token {fmt} top_k={top_k}")


def test_moe_ffn_one_token_same_bits_as_three_kernels():
    """The workload's MoE layer at one token: kq_moe_ffn's fused down + sum
    against the per-slot + weighted-sum kernels, bit for bit."""
    L = S.MOE_Q4_0
    ids, rw = S.route_table(L.workload_id, 1, L.n_experts, L.top_k)
    used = ids.ravel()
    gate = Experts(L.fmt, L.n_experts, L.inter, L.hidden, used, lambda e: L.weight_seed(e, 0))
    up = Experts(L.fmt, L.n_experts, L.inter, L.hidden, used, lambda e: L.weight_seed(e, 1))
    down = Experts(L.fmt, L.n_experts, L.hidden, L.inter, used, lambda e: L.weight_seed(e, 2))
    x = S.activations(L.act_seed_prefix(), L.hidden, 1)
    wsb = kq.kq_moe_ffn_workspace_bytes(L.hidden, L.inter, 1, L.top_k)
    outs = []
    for unfused in (False, True):
        y = U.empty_dev((1, L.hidden))
        ws = U.empty_dev((wsb // 4 + 1,))
        with U.tuning({"moe_unfused": "1"} if unfused else {}):
            kq.kq_moe_ffn(L.fmt, gate.dev, up.dev, down.dev, U.to_dev(x), U.to_dev(ids), U.to_dev(rw), y, None,
                          L.hidden, L.inter, 1, L.top_k, L.n_experts, ws, wsb)
        outs.append(U.to_host(y))
    assert np.all(np.isfinite(outs[0]))
    assert np.array_equal(outs[0].view(np.uint32), outs[1].view(np.uint32))


@pytest.mark.parametrize("fmt", ("q4_0", "q8_0", "affine4", "q5_0", "q5_1"))
@pytest.mark.parametrize("hidden", (768, 2048, 4096))
@pytest.mark.parametrize("top_k,ids_row", [(8, None), (1, None), (4, [6, 6, 2, 6]), (3, [5, -1, 2]), (16, None)])
def test_moe_ffn_one_token_gate_up_kernel(fmt, hidden, top_k, ids_row):
    """One token: the gate|up kernel that reads the route ids with scalar loads
    and issues its weight loads before the dedupe test gives the h and y bits
    of the general routed-expert kernel (moe_one = 0) where that kernel also
    stages x in LDS (hidden <= 2048), including a repeated expert (one
    workgroup serves all its slots) and a bad id (NaN); and h is within the
    bar of the oracle where the ids are valid."""
    inter, E = 352, 16                  # 11 blocks per down row (odd for Q4_0/Q8_0 units)
    if ids_row is None:
        ids, rw = _route(1, E, top_k, 60 + top_k)
    else:
        ids = np.array([ids_row], np.int32)
        rw = np.linspace(0.3, 0.8, top_k, dtype=np.float32)[None, :]
    used = [v for v in ids.ravel() if 0 <= v < E]
    gate = Experts(fmt, E, inter, hidden, used, lambda e: (76, e, 0, 0))
    up = Experts(fmt, E, inter, hidden, used, lambda e: (76, e, 1, 0))
    down = Experts(fmt, E, hidden, inter, used, lambda e: (76, e, 2, 0))
    x = S.activations((76, top_k, hidden), hidden, 1)
    wsb = kq.kq_moe_ffn_workspace_bytes(hidden, inter, 1, top_k)
    outs = []
    for one in ("1", "0"):
        y = U.empty_dev((1, hidden))
        h = U.empty_dev((1, top_k, inter), "float16")
        h.fill_(3.0)
        ws = U.empty_dev((wsb // 4 + 1,))
        with U.tuning({"moe_one": one}):
            kq.kq_moe_ffn(fmt, gate.dev, up.dev, down.dev, U.to_dev(x), U.to_dev(ids), U.to_dev(rw), y, h,
                          hidden, inter, 1, top_k, E, ws, wsb)
        outs.append((U.to_host(y), U.to_host(h)))
    (y1, h1), (y0, h0) = outs
    if hidden <= 2048:   # the general kernel stages x in LDS too: the same lanes and order
        assert np.array_equal(h1.view(np.uint16), h0.view(np.uint16))
        assert np.array_equal(y1.view(np.uint32), y0.view(np.uint32))
    if np.any(ids < 0):
        bad = np.flatnonzero(ids[0] < 0)
        assert np.all(np.isnan(h1[0, bad])) and np.all(np.isnan(y1))
        return
    _, _, (g, g_abs), (u, u_abs), h_ref = R.moe_ffn(fmt, gate.field_list(E), up.field_list(E), down.field_list(E),
                                                   x, ids, rw)
    sig = 1.0 / (1.0 + np.exp(-g))
    dsilu = sig * (1.0 + g * (1.0 - sig))
    tol_h = (np.abs(dsilu * u) * R.tolerance(g_abs) + np.abs(g * sig) * R.tolerance(u_abs)
             + 2.0 ** -10 * np.abs(h_ref.astype(np.float64)) + 2.0 ** -24)
    assert np.all(np.abs(h1.astype(np.float64) - h_ref.astype(np.float64)) <= tol_h)
