"""GPU parity of kq_stack_run (a chain of dependent M=1 GEMVs in one
persistent launch) against the oracle, through the C ABI. A stage whose x lies
in an earlier stage's fp16 output is checked against the oracle run on the
GPU's own fp16 values of that output."""
import numpy as np
import pytest

import block_quantized_gemv_kq_amd as kq
from oracle import formats as F
from oracle import ref as R
from synth import inputs as S
from tests import gpu_util as U

pytestmark = pytest.mark.gpu


def _plan(stages):
    torch = U.torch_cuda()
    nb = kq.kq_stack_plan_bytes(stages)
    plan = torch.zeros(nb, dtype=torch.uint8, device="cuda")
    info = kq.kq_stack_plan(stages, plan, nb)
    return plan, info


SHAPES = [("affine4", 6144, 2560), ("affine4", 2560, 4096), ("q8_0", 3000, 2560),
          ("affine4", 19456, 2560), ("q4_0", 333, 1024), ("affine4", 2560, 9728),
          ("q8_0", 77, 64), ("affine4", 1, 32), ("q4_0", 2048, 3072)]


def test_independent_stages_parity_and_repeat():
    """Mixed formats and ragged shapes, no stage reading another; three runs
    in a row (the epochs advance, nothing is reset) give bitwise identical
    results within tolerance."""
    torch = U.torch_cuda()
    stages, refs = [], []
    for i, (fmt, N, K) in enumerate(SHAPES):
        W = S.weights((50, i, 0, 0), N, K)
        packed, fields = U.quantize_both(fmt, W)
        x = S.activations((50, i, 0), K, 1)
        y = torch.full((N,), float("nan"), dtype=torch.float32, device="cuda")
        stages.append(dict(fmt=fmt, W=U.to_dev(packed), x=U.to_dev(x[0]), y=y, N=N, K=K))
        refs.append(R.gemv(fmt, fields, x))
    plan, info = _plan(stages)
    outs = []
    for _ in range(3):
        for st in stages:
            st["y"].fill_(float("nan"))
        kq.kq_stack_run(plan, info)
        assert kq.kq_stack_status(plan, info) == 0
        outs.append([U.to_host(st["y"]).copy() for st in stages])
    for i, ((fmt, N, K), (yr, ad)) in enumerate(zip(SHAPES, refs)):
        U.assert_parity(outs[0][i][None, :], yr, ad, f"stack stage {i} {fmt} {N}x{K}")
        for r in (1, 2):
            assert np.array_equal(outs[r][i].view(np.uint32), outs[0][i].view(np.uint32))


def test_dependent_chain_uses_previous_output():
    """stage s+1 reads fp16(y_s) written by stage s in the same launch: the
    result must match the oracle run stage by stage on the GPU's own fp16
    intermediates (and those must be fp16(y) of each stage)."""
    torch = U.torch_cuda()
    dims = [1024, 2048, 512, 1536, 1024]       # chain 1024 -> 2048 -> 512 -> 1536 -> 1024
    fmts = ["affine4", "q8_0", "q4_0", "affine4"]
    x0 = S.activations((51, 0, 0), dims[0], 1)[0]
    xd = U.to_dev(x0)
    stages, fields = [], []
    for i, fmt in enumerate(fmts):
        K, N = dims[i], dims[i + 1]
        W = S.weights((51, i, 0, 0), N, K) * np.float32(1.5)    # keep activations O(1)
        packed, f = U.quantize_both(fmt, W)
        fields.append(f)
        y = torch.empty(N, dtype=torch.float32, device="cuda")
        y16 = torch.empty(N, dtype=torch.float16, device="cuda")
        stages.append(dict(fmt=fmt, W=U.to_dev(packed), x=xd, y=y, y16=y16, N=N, K=K))
        xd = y16
    plan, info = _plan(stages)
    kq.kq_stack_run(plan, info)
    assert kq.kq_stack_status(plan, info) == 0
    x_in = x0
    for i, (fmt, st) in enumerate(zip(fmts, stages)):
        y = U.to_host(st["y"])
        y16 = U.to_host(st["y16"])
        yr, ad = R.gemv(fmt, fields[i], x_in[None, :])
        U.assert_parity(y[None, :], yr, ad, f"chain stage {i}")
        assert np.array_equal(y16.view(np.uint16), y.astype(np.float16).view(np.uint16))
        x_in = y16


def _branchy_chain(torch, seed):
    """Five stages: stage 1 reads the second half of stage 0's output, stage 2
    an outside x, stage 3 a slice of stage 0's output again (not the previous
    stage), stage 4 stage 1's output. Returns stages, quantized fields and
    where each x comes from: ("ext", array) or ("dep", stage, offset)."""
    spec = [("affine4", 2048, 512, ("ext",)),
            ("q8_0", 1024, 1024, ("dep", 0, 1024)),
            ("affine4", 512, 768, ("ext",)),
            ("q4_0", 640, 512, ("dep", 0, 512)),
            ("affine4", 300, 1024, ("dep", 1, 0))]
    stages, fields, srcs = [], [], []
    for i, (fmt, N, K, src) in enumerate(spec):
        W = S.weights((seed, i, 0, 0), N, K) * np.float32(1.5)
        packed, f = U.quantize_both(fmt, W)
        fields.append(f)
        if src[0] == "ext":
            xe = S.activations((seed, i, 0), K, 1)[0]
            x = U.to_dev(xe)
            srcs.append(("ext", xe))
        else:
            x = stages[src[1]]["y16"][src[2]:src[2] + K]
            srcs.append(src)
        stages.append(dict(fmt=fmt, W=U.to_dev(packed), x=x, N=N, K=K,
                           y=torch.full((N,), float("nan"), dtype=torch.float32, device="cuda"),
                           y16=torch.empty(N, dtype=torch.float16, device="cuda")))
    return stages, fields, srcs


def test_chain_reads_slices_of_earlier_outputs():
    torch = U.torch_cuda()
    stages, fields, srcs = _branchy_chain(torch, 53)
    plan, info = _plan(stages)
    runs = []
    for _ in range(3):
        kq.kq_stack_run(plan, info)
        assert kq.kq_stack_status(plan, info) == 0
        runs.append([(U.to_host(st["y"]).copy(), U.to_host(st["y16"]).copy()) for st in stages])
    for i, (st, src) in enumerate(zip(stages, srcs)):
        y, y16 = runs[0][i]
        if src[0] == "ext":
            x_in = src[1]
        else:
            x_in = runs[0][src[1]][1][src[2]:src[2] + st["K"]]
        yr, ad = R.gemv(st["fmt"], fields[i], x_in[None, :])
        U.assert_parity(y[None, :], yr, ad, f"stage {i}")
        assert np.array_equal(y16.view(np.uint16), y.astype(np.float16).view(np.uint16))
        for r in (1, 2):
            assert np.array_equal(runs[r][i][0].view(np.uint32), y.view(np.uint32)), (i, r)


def test_chain_graph_replays_match_eager():
    """A captured chained plan replays with nothing reset in between; eager
    work on the outputs between replays does not disturb it."""
    torch = U.torch_cuda()
    stages, _, _ = _branchy_chain(torch, 54)
    plan, info = _plan(stages)
    kq.kq_stack_run(plan, info)
    eager = [U.to_host(st["y"]).copy() for st in stages]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        kq.kq_stack_run(plan, info)
    torch.cuda.synchronize()
    for rep in range(4):
        for st in stages:
            st["y"].fill_(0.0)
            st["y16"].fill_(0.0)
        g.replay()
        torch.cuda.synchronize()
        for st, e in zip(stages, eager):
            assert np.array_equal(U.to_host(st["y"]).view(np.uint32), e.view(np.uint32)), rep
    assert kq.kq_stack_status(plan, info) == 0


def test_stack_in_graph_replays_match_eager():
    torch = U.torch_cuda()
    stages = []
    for i, (fmt, N, K) in enumerate(SHAPES[:4]):
        packed = kq.kq_pack(fmt, S.weights((52, i, 0, 0), N, K))
        x = S.activations((52, i, 0), K, 1)
        stages.append(dict(fmt=fmt, W=U.to_dev(packed), x=U.to_dev(x[0]),
                           y=torch.empty(N, dtype=torch.float32, device="cuda"), N=N, K=K))
    plan, info = _plan(stages)
    kq.kq_stack_run(plan, info)
    eager = [U.to_host(st["y"]).copy() for st in stages]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        kq.kq_stack_run(plan, info)
    torch.cuda.synchronize()
    for rep in range(4):
        for st in stages:
            st["y"].fill_(0.0)
        g.replay()
        torch.cuda.synchronize()
        for st, e in zip(stages, eager):
            assert np.array_equal(U.to_host(st["y"]).view(np.uint32), e.view(np.uint32)), rep
    assert kq.kq_stack_status(plan, info) == 0


def test_full_qwen3_4b_stack_sampled():
    """The 4B-shaped affine4 stack + Q8_0 lm_head as one plan (145 stages),
    the configuration bench.py times: sampled rows of layers 0 and 35 and the
    full lm_head argmax against the oracle."""
    torch = U.torch_cuda()
    st = S.QWEN3_4B_AFFINE4
    stages, keep = [], {}
    for layer in range(st.layers):
        for gi, group in enumerate(st.launch_groups):
            mats = [st.per_layer[i] for i in group]
            fmt, K = mats[0].fmt, mats[0].k
            N = sum(m.n for m in mats)
            Ws = [S.weights(st.weight_seed(layer, i), m.n, m.k) for i, m in zip(group, mats)]
            W = np.concatenate(Ws)
            packed = kq.kq_pack(fmt, W)
            x = S.activation_column(st.act_seed_prefix(layer, mats[0].input_slot) + (1, 0), K)
            y = torch.empty(N, dtype=torch.float32, device="cuda")
            stages.append(dict(fmt=fmt, W=U.to_dev(packed), x=U.to_dev(x), y=y, N=N, K=K))
            if layer in (0, 35):
                keep[(layer, gi)] = (W, x, fmt)
    h = st.head
    Wh = S.weights(st.weight_seed(st.layers, 0), h.n, h.k)
    ph = kq.kq_pack(h.fmt, Wh)
    xh = S.activation_column(st.act_seed_prefix(st.layers, 0) + (1, 0), h.k)
    yh = torch.empty(h.n, dtype=torch.float32, device="cuda")
    stages.append(dict(fmt=h.fmt, W=U.to_dev(ph), x=U.to_dev(xh), y=yh, N=h.n, K=h.k))
    plan, info = _plan(stages)
    kq.kq_stack_run(plan, info)
    assert kq.kq_stack_status(plan, info) == 0
    rng = np.random.default_rng(7)
    for (layer, gi), (W, x, fmt) in keep.items():
        N = W.shape[0]
        rows = np.unique(np.concatenate([[0, N - 1], rng.choice(N, 256, replace=False)]))
        f = F.quantize(fmt, W[rows])
        yr, ad = R.gemv(fmt, f, x[None, :])
        y = U.to_host(stages[layer * 4 + gi]["y"])
        U.assert_parity(y[rows][None, :], yr, ad, f"layer {layer} group {gi}")
    fh = F.quantize(h.fmt, Wh)
    yr, ad = R.gemv(h.fmt, fh, xh[None, :])
    yg = U.to_host(yh)
    U.assert_parity(yg[None, :], yr, ad, "lm_head in stack")
    assert int(np.argmax(yg)) == int(R.argmax_lowest(yr[0]))

    # The plan bench.py times: the same weights in decode order, every stage
    # (the lm_head last) reading the first K values of the previous stage's
    # fp16 output. Two runs agree bit for bit; the first layers (before the
    # unnormalised chain leaves fp16 range) match the oracle on the GPU's own
    # fp16 inputs.
    prev = None
    for st_ in stages:
        st_["y16"] = torch.empty(st_["N"], dtype=torch.float16, device="cuda")
        if prev is not None:
            st_["x"] = prev["y16"][:st_["K"]]
        prev = st_
    plan, info = _plan(stages)
    outs = []
    for _ in range(2):
        kq.kq_stack_run(plan, info)
        assert kq.kq_stack_status(plan, info) == 0
        outs.append([U.to_host(st_["y"]).copy() for st_ in stages])
    for a, b in zip(*outs):
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
    x_in = U.to_host(stages[0]["x"])
    for layer in range(3):
        for gi, group in enumerate(st.launch_groups):
            k = layer * len(st.launch_groups) + gi
            mats = [st.per_layer[i] for i in group]
            fmt = mats[0].fmt
            W = np.concatenate([S.weights(st.weight_seed(layer, i), m.n, m.k) for i, m in zip(group, mats)])
            rows = np.unique(np.concatenate([[0, W.shape[0] - 1], rng.choice(W.shape[0], 128, replace=False)]))
            yr, ad = R.gemv(fmt, F.quantize(fmt, W[rows]), x_in[None, :stages[k]["K"]])
            U.assert_parity(outs[0][k][rows][None, :], yr, ad, f"chained layer {layer} group {gi}")
            x_in = U.to_host(stages[k]["y16"])
