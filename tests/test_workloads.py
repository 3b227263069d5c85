"""The seeded input generators: deterministic, independent streams, right shapes."""

import numpy as np
import torch

import workloads as wl


def test_generators_are_deterministic_and_independent():
    a = wl.weight_f32(3, 8, 64)
    b = wl.weight_f32(3, 8, 64)
    c = wl.weight_f32(3, 8, 64, matrix=1)
    assert a.dtype == np.float32 and a.shape == (8, 64)
    assert np.array_equal(a, b)
    assert not np.array_equal(a, c)
    x1 = wl.bf16_normal(1, (4, 8), 1.0)
    x2 = wl.bf16_normal(1, (4, 8), 1.0)
    assert x1.dtype == torch.bfloat16 and torch.equal(x1, x2)


def test_outliers_recipe():
    w = wl.weight_f32(2, 256, 1024, outlier_frac=1e-3)
    out = np.abs(w) == np.float32(0.16)
    frac = out.mean()
    assert 0.0006 < frac < 0.0014
    assert (w[out] > 0).any() and (w[out] < 0).any()
    assert abs(float(np.std(w[~out])) - 0.02) < 0.001


def test_workload_shapes_and_flops():
    w3 = wl.LLAMA7B_MLP
    assert (w3.M, w3.k_in, w3.n_out, w3.r) == (4096, 4096, 11008, 64)
    M, K, N, r = 4096, 4096, 11008, 64
    assert w3.flops_fwd == 2 * M * K * N + 2 * M * K * r + 2 * M * r * N == 377_286_033_408
    assert w3.flops_bwd == 2 * M * N * K + 4 * M * N * r + 4 * M * r * K == 385_204_879_360
    assert sum(x.flops_fwd + x.flops_bwd for x in wl.LLAMA65B_LAYER) == 6_754_238_726_144
    inp = wl.SINGLE_LINEAR.inputs()
    assert inp["W"].shape == (4096, 4096) and inp["X"].shape == (16, 4096)
    assert "dY" not in inp
    assert sum(n * k for _, n, k in wl.LLAMA7B_MATRICES) * wl.LLAMA7B_LAYERS == 6_476_005_376
