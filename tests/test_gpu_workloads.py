"""Full-size workloads on the GPU, in the launch configuration the benchmark
times (row-concatenated q|k|v and gate|up, M columns per call):

* every layer of the Qwen3-4B-shaped affine4 stack + the Q8_0 lm_head
  (151936 x 2560), M = 1;
* speculative verify on those weights, M in {2, 4, 8, 16, 48};
* every layer of the Qwen3-0.6B-shaped Q4_0 stack, M = 1.

Dense layers are compared with the oracle on sampled rows (first, last and
random); the lm_head is compared in full, with bit-identical argmax."""
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest

import block_quantized_gemv_kq_amd as kq
from oracle import formats as F
from oracle import ref as R
from synth import inputs as S
from tests import gpu_util as U

pytestmark = pytest.mark.gpu


def _sample_rows(n, count, seed):
    rng = np.random.default_rng([60, seed, n])
    rows = np.unique(np.concatenate([[0, 1, n - 2, n - 1], rng.choice(n, min(n, count), replace=False)]))
    return rows


def _group_matrix(stack, layer, group):
    """Row-concatenated weights of one launch group, and the seeds of its parts."""
    mats = [stack.per_layer[i] for i in group]
    W = np.concatenate([S.weights(stack.weight_seed(layer, i), m.n, m.k) for i, m in zip(group, mats)])
    return W, mats


def _check_group(stack, layer, group, x, act_desc):
    W, mats = _group_matrix(stack, layer, group)
    N, K = W.shape
    fmt = mats[0].fmt
    packed = kq.kq_pack(fmt, W)
    rows = _sample_rows(N, 384, layer * 10 + group[0])
    fields = F.quantize(fmt, W[rows])
    assert np.array_equal(packed[rows], F.encode(fmt, fields)), "packer bytes differ"
    y = U.gemv_gpu(fmt, U.to_dev(packed), x, N, K)
    yr, ad = R.gemv(fmt, fields, x)
    ratio = U.assert_parity(y[:, rows], yr, ad, f"{stack.name} layer {layer} group {group} {act_desc}")
    return y, ratio


@pytest.mark.parametrize("layer", range(36))
def test_qwen3_4b_layer_m1(layer):
    st = S.QWEN3_4B_AFFINE4
    for group in st.launch_groups:
        slot = st.per_layer[group[0]].input_slot
        K = st.per_layer[group[0]].k
        x = S.activation_column(st.act_seed_prefix(layer, slot) + (1, 0), K)[None, :]
        _, ratio = _check_group(st, layer, group, x, "M=1")
        assert ratio < 1e-4


@pytest.mark.parametrize("layer", range(28))
def test_qwen3_0_6b_layer_m1(layer):
    st = S.QWEN3_0_6B_Q4_0
    for group in st.launch_groups:
        slot = st.per_layer[group[0]].input_slot
        K = st.per_layer[group[0]].k
        x = S.activation_column(st.act_seed_prefix(layer, slot) + (1, 0), K)[None, :]
        _check_group(st, layer, group, x, "M=1")


@pytest.mark.parametrize("M", S.VERIFY_M)
def test_verify_layer_columns(M):
    """cfg-4 verify: M columns over the 4B-shaped weights (layer 0); each
    column also equals its own M=1 run within the tolerance."""
    st = S.QWEN3_4B_AFFINE4
    for group in st.launch_groups:
        slot = st.per_layer[group[0]].input_slot
        K = st.per_layer[group[0]].k
        x = S.activations((S.VERIFY_WORKLOAD_ID, 0, slot), K, M)
        y, _ = _check_group(st, 0, group, x, f"M={M}")
        W, mats = _group_matrix(st, 0, group)
        packed = U.to_dev(kq.kq_pack(mats[0].fmt, W))
        for m in (0, M - 1):
            y1 = U.gemv_gpu(mats[0].fmt, packed, x[m:m + 1], W.shape[0], K)
            # both are within the oracle tolerance; against each other allow twice it
            _, ad = R.gemv(mats[0].fmt, F.quantize(mats[0].fmt, W[:64]), x[m:m + 1])
            assert np.all(np.abs(y[m, :64] - y1[0, :64]) <= 2 * R.tolerance(ad[0]))


@pytest.fixture(scope="module")
def lm_head():
    st = S.QWEN3_4B_AFFINE4
    h = st.head
    W = S.weights(st.weight_seed(st.layers, 0), h.n, h.k)
    packed = kq.kq_pack(h.fmt, W)
    chunk = 8192

    def q(r0):
        f = F.quantize(h.fmt, W[r0:r0 + chunk])
        assert np.array_equal(packed[r0:r0 + chunk], F.encode(h.fmt, f))
        return f
    with ThreadPoolExecutor(8) as ex:
        parts = list(ex.map(q, range(0, h.n, chunk)))
    fields = {k: np.concatenate([p[k] for p in parts]) for k in parts[0]}
    del W
    return h, U.to_dev(packed), fields


def _argmax_gpu(y_dev, N, M):
    out = U.empty_dev((M,), "int32")
    wsb = kq.kq_argmax_workspace_bytes(N, M)
    ws = U.empty_dev((wsb // 4 + 2,))
    kq.kq_argmax(y_dev, N, M, out, ws, wsb)
    return U.to_host(out)


def _head_run(lm_head, x):
    h, packed, fields = lm_head
    M = x.shape[0]
    xd = U.to_dev(x)
    y = U.empty_dev((M, h.n))
    kq.kq_gemv(h.fmt, packed, xd, y, h.n, h.k, M)
    return y, U.to_host(y)


def test_lm_head_m1_full_and_argmax(lm_head):
    h, packed, fields = lm_head
    st = S.QWEN3_4B_AFFINE4
    x = S.activation_column(st.act_seed_prefix(st.layers, 0) + (1, 0), h.k)[None, :]
    y_dev, y = _head_run(lm_head, x)
    yr, ad = R.gemv(h.fmt, fields, x)
    ratio = U.assert_parity(y, yr, ad, "lm_head M=1")
    assert ratio < 1e-4
    gap = R.top2_gap(yr[0])
    assert gap > 4 * float(np.max(np.abs(y[0] - yr[0]))), "argmax not pinned by this seed"
    am = _argmax_gpu(y_dev, h.n, 1)
    assert int(am[0]) == int(R.argmax_lowest(yr[0]))


@pytest.fixture(scope="module")
def lm_head_verify_ref(lm_head):
    """The oracle over the 48 verify columns once: columns are seeded one by
    one, so the first M columns of this draw are the M-column input."""
    h, packed, fields = lm_head
    x = S.activations((S.VERIFY_WORKLOAD_ID, 36, 0), h.k, max(S.VERIFY_M))
    yr, ad = R.gemv(h.fmt, fields, x)
    return x, yr, ad


@pytest.mark.parametrize("M", S.VERIFY_M)
def test_lm_head_verify_argmax(lm_head, lm_head_verify_ref, M):
    """cfg-4 verify on the lm_head: every column within tolerance of the
    oracle, bit-identical argmax, and each column's argmax equal to its own
    M=1 run's."""
    h, packed, fields = lm_head
    x48, yr48, ad48 = lm_head_verify_ref
    x, yr, ad = x48[:M], yr48[:M], ad48[:M]
    y_dev, y = _head_run(lm_head, x)
    U.assert_parity(y, yr, ad, f"lm_head M={M}")
    gaps = R.top2_gap(yr)
    errs = np.max(np.abs(y - yr), axis=1)
    assert np.all(gaps > 4 * errs), f"argmax not pinned by these seeds: gaps {gaps} errors {errs}"
    am = _argmax_gpu(y_dev, h.n, M)
    assert np.array_equal(am, R.argmax_lowest(yr))
    for m in sorted({0, M // 2, M - 1}):
        y1_dev, _ = _head_run(lm_head, x[m:m + 1])
        assert int(_argmax_gpu(y1_dev, h.n, 1)[0]) == int(am[m])


def test_argmax_ties_and_nan():
    y = np.zeros((3, 40000), np.float32)
    y[0, [5, 9, 30000]] = 2.0            # tie: lowest index wins
    y[1, :] = np.nan
    y[1, 123] = -1.0                     # NaN never wins
    y[2, :] = -np.inf
    yd = U.to_dev(y)
    am = _argmax_gpu(yd, 40000, 3)
    assert list(am) == [5, 123, 0]
