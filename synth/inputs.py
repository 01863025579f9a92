"""Seeded synthetic workloads for block-quantized decode GEMV.

The pages this library follows measure decode on trained models (Qwen3-0.6B
and Qwen3-4B shaped dense stacks, a 128-expert top-8 mixture of experts) whose
weights are not available here. These generators stand in for them: weights
drawn from N(0, 0.02), activations from N(0, 1) rounded to fp16, routing ids
drawn uniformly without replacement with softmax-normalised fp32 weights.

Every draw comes from ``numpy.random.default_rng(seed)`` where ``seed`` is a
tuple of small integers naming the workload, the layer, the matrix and (for
activations) the column, so a single column or a single matrix can be
regenerated on its own:

* weights:      ``(workload_id, layer, matrix, 0)``
* activations:  ``(workload_id, layer, input_slot, 1, column)``
* MoE route ids ``(workload_id, 1, token)``, route logits ``(workload_id, 2, token)``

Draw recipe: weights are drawn in blocks of 4096 rows; row block ``b`` of a
matrix with seed ``s`` is ``default_rng(s + (b,)).standard_normal((rows, K),
dtype=float32) * float32(0.02)`` (so blocks can be drawn in parallel and a
sampled row can be regenerated alone). One activation column is
``default_rng(seed).standard_normal(K, dtype=float32).astype(float16)``.
"""
from __future__ import annotations

from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field
import os

import numpy as np

__all__ = [
    "weights", "activation_column", "activations", "route_table",
    "Matrix", "Stack", "MoELayer",
    "SINGLE_Q8_0", "QWEN3_0_6B_Q4_0", "QWEN3_4B_AFFINE4", "VERIFY_M", "MOE_Q4_0",
    "MOE_M", "stack_by_name",
]

WEIGHT_STD = np.float32(0.02)
ROW_BLOCK = 4096
_THREADS = max(1, min(16, os.cpu_count() or 1))


def _row_block(seed, b: int, rows: int, k: int) -> np.ndarray:
    rng = np.random.default_rng(list(seed) + [b])
    w = rng.standard_normal((rows, k), dtype=np.float32)
    w *= WEIGHT_STD
    return w


def weights(seed, n: int, k: int) -> np.ndarray:
    """fp32 [n, k] drawn from N(0, 0.02), row blocks of 4096 seeded seed + (b,)."""
    out = np.empty((n, k), np.float32)
    nb = (n + ROW_BLOCK - 1) // ROW_BLOCK

    def fill(b):
        r0 = b * ROW_BLOCK
        r1 = min(n, r0 + ROW_BLOCK)
        out[r0:r1] = _row_block(seed, b, r1 - r0, k)

    if nb <= 1:
        for b in range(nb):
            fill(b)
    else:
        with ThreadPoolExecutor(min(_THREADS, nb)) as ex:
            list(ex.map(fill, range(nb)))
    return out


def activation_column(seed, k: int) -> np.ndarray:
    """One fp16 activation vector of length k from N(0, 1)."""
    rng = np.random.default_rng(list(seed))
    return rng.standard_normal(k, dtype=np.float32).astype(np.float16)


def activations(seed_prefix, k: int, m: int, first_column: int = 0) -> np.ndarray:
    """fp16 [m, k]; column c uses seed ``seed_prefix + (1, first_column + c)``."""
    cols = [activation_column(tuple(seed_prefix) + (1, first_column + c), k) for c in range(m)]
    return np.stack(cols, axis=0) if cols else np.zeros((0, k), np.float16)


def route_table(workload_id: int, m: int, n_experts: int, top_k: int):
    """Route ids int32 [m, top_k] (uniform, without replacement, draw order =
    slot order) and route weights fp32 [m, top_k] (softmax of N(0,1) logits,
    computed in fp64 and stored as fp32)."""
    ids = np.empty((m, top_k), np.int32)
    rw = np.empty((m, top_k), np.float32)
    for t in range(m):
        rng = np.random.default_rng([workload_id, 1, t])
        ids[t] = rng.choice(n_experts, top_k, replace=False)
        rng = np.random.default_rng([workload_id, 2, t])
        logits = rng.standard_normal(top_k)  # fp64
        e = np.exp(logits - logits.max())
        rw[t] = (e / e.sum()).astype(np.float32)
    return ids, rw


@dataclass(frozen=True)
class Matrix:
    """One projection: ``n`` output rows, ``k`` inputs, quantized as ``fmt``;
    ``input_slot`` names which layer input feeds it (q, k and v share one,
    gate and up share one)."""
    name: str
    n: int
    k: int
    fmt: str
    input_slot: int


@dataclass(frozen=True)
class Stack:
    """A dense decode stack: ``layers`` copies of ``per_layer`` plus an
    optional output head. ``workload_id`` seeds every draw."""
    name: str
    workload_id: int
    layers: int
    per_layer: tuple
    head: Matrix | None = None
    # groups of matrices that share one input and are launched as one
    # row-concatenated GEMV (the order a decoder layer consumes them in)
    launch_groups: tuple = field(default=())

    def weight_seed(self, layer: int, mat_index: int):
        return (self.workload_id, layer, mat_index, 0)

    def act_seed_prefix(self, layer: int, input_slot: int):
        return (self.workload_id, layer, input_slot)

    def matrices(self):
        """Yield (layer, mat_index, Matrix); the head is layer == self.layers."""
        for layer in range(self.layers):
            for i, mat in enumerate(self.per_layer):
                yield layer, i, mat
        if self.head is not None:
            yield self.layers, 0, self.head


# Single 1024x1024 Q8_0 GEMV, seeds 0 (weights) and 1 (activation).
@dataclass(frozen=True)
class Single:
    name: str
    n: int
    k: int
    fmt: str
    weight_seed: tuple
    act_seed: tuple


SINGLE_Q8_0 = Single("single_q8_0_1024", 1024, 1024, "q8_0", (0,), (1,))


def _qwen3_layer(hidden, inter, q_rows, kv_rows, fmt):
    return (
        Matrix("q_proj", q_rows, hidden, fmt, 0),
        Matrix("k_proj", kv_rows, hidden, fmt, 0),
        Matrix("v_proj", kv_rows, hidden, fmt, 0),
        Matrix("o_proj", hidden, q_rows, fmt, 1),
        Matrix("gate_proj", inter, hidden, fmt, 2),
        Matrix("up_proj", inter, hidden, fmt, 2),
        Matrix("down_proj", hidden, inter, fmt, 3),
    )


# Launch groups: indices into per_layer that share an input, in decode order.
_GROUPS = ((0, 1, 2), (3,), (4, 5), (6,))

QWEN3_0_6B_Q4_0 = Stack(
    "qwen3_0.6b_shaped_q4_0", 2, 28,
    _qwen3_layer(hidden=1024, inter=3072, q_rows=2048, kv_rows=1024, fmt="q4_0"),
    head=None, launch_groups=_GROUPS)

QWEN3_4B_AFFINE4 = Stack(
    "qwen3_4b_shaped_affine4", 3, 36,
    _qwen3_layer(hidden=2560, inter=9728, q_rows=4096, kv_rows=1024, fmt="affine4"),
    head=Matrix("lm_head", 151936, 2560, "q8_0", 0), launch_groups=_GROUPS)

# Speculative verify on the 4B-shaped weights: column counts read in one pass.
VERIFY_M = (2, 4, 8, 16, 48)
VERIFY_WORKLOAD_ID = 4


@dataclass(frozen=True)
class MoELayer:
    name: str
    workload_id: int
    n_experts: int
    hidden: int
    inter: int
    top_k: int
    fmt: str

    def weight_seed(self, expert: int, which: int):
        """which: 0 gate, 1 up, 2 down."""
        return (self.workload_id, expert, which, 0)

    def act_seed_prefix(self):
        return (self.workload_id, 0, 0)


MOE_Q4_0 = MoELayer("moe_128x_top8_q4_0", 5, 128, 2048, 768, 8, "q4_0")
MOE_M = (1, 4, 16)


def stack_by_name(name: str) -> Stack:
    for s in (QWEN3_0_6B_Q4_0, QWEN3_4B_AFFINE4):
        if s.name == name:
            return s
    raise KeyError(name)
