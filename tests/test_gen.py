"""Seeded input generator: determinism, shapes, and sample statistics near
their closed-form values."""
import math
import os

import numpy as np
import pytest

from consumer_gemm_chain_amd import gen

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "pages_shapes.txt")


def test_workload_shapes_follow_the_pages():
    rows = [l.split() for l in open(GOLDEN) if l.strip() and not l.startswith("#")]
    page = {r[0]: (int(r[1]), int(r[2]), r[3]) for r in rows}
    w = gen.WORKLOADS
    assert (w[1].H, w[1].dtype) == (page["gpt3_175b"][0], page["gpt3_175b"][2])
    assert (w[2].H, w[2].dtype) == (page["llama_65b"][0], page["llama_65b"][2])
    assert w[3].H == page["llama2_70b"][0]
    # one tensor-parallel shard of the MLP's inner width
    assert w[1].I * page["gpt3_175b"][1] == 4 * w[1].H
    assert w[2].I * page["llama_65b"][1] == 22016
    assert w[3].I * page["llama2_70b"][1] == 28672


def test_deterministic_and_rows_agree_across_M():
    a = gen.x_rows(0, 64)
    b = gen.x_rows(0, 16)
    assert np.array_equal(a[:16], b)
    x, w1, w2 = gen.workload_inputs(0)
    assert x.shape == (64, 512) and w1.shape == (512, 2048) and w2.shape == (2048, 512)
    x2, w12, w22 = gen.workload_inputs(0)
    assert np.array_equal(w1, w12) and np.array_equal(w2, w22)


def test_swiglu_weight_packing_shape():
    w1, w2 = gen.weights(2)
    assert w1.shape == (8192, 2 * 2752) and w2.shape == (2752, 8192)


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_normal_statistics(dtype):
    b = gen.normal_bits((1000, 1000), 1, 0.02, dtype)
    v = gen.from_bits(b, dtype).astype(np.float64)
    assert abs(v.mean()) < 1e-3 * 0.02 * 50
    assert abs(v.std() / 0.02 - 1) < 0.01


def test_uniform_statistics():
    b = gen.uniform_bits((1000, 1000), 2, 1 / math.sqrt(8192), "bf16")
    v = gen.from_bits(b, "bf16").astype(np.float64) * math.sqrt(8192)
    assert v.min() >= -1.0 - 1e-2 and v.max() <= 1.0 + 1e-2
    assert abs(v.std() - 1 / math.sqrt(3)) < 0.01
