"""Pins of the oracle's scalar and row functions against library routines,
closed forms and brute force."""
import math

import numpy as np
import torch
import torch.nn.functional as Fn

import oracle


def test_round_bf16_matches_torch_rne():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100000) * 10 ** rng.uniform(-6, 6, 100000),
                        [0.0, -0.0, 1.0, -1.0, 65504.0, 1e-30]])
    ref = torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(oracle.round_bf16(x), ref)
    # exact ties go to even mantissa: 1 + 2^-8 lies halfway between 1 and 1 + 2^-7
    assert oracle.round_bf16(np.array([1.0 + 2 ** -8]))[0] == 1.0
    assert oracle.round_bf16(np.array([1.0 + 3 * 2 ** -8]))[0] == 1.0 + 2 ** -6


def test_layer_norm_against_torch_and_constant_row():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((7, 300)) * 3 + 1.5
    ref = Fn.layer_norm(torch.from_numpy(x), (300,), eps=1e-6).numpy()
    assert np.allclose(oracle.layer_norm(x), ref, rtol=0, atol=1e-12)
    assert np.all(oracle.layer_norm(np.full((2, 64), 4.25)) == 0.0)


def test_activations_against_torch_and_closed_forms():
    x = np.linspace(-8, 8, 2001)
    t = torch.from_numpy(x)
    assert np.allclose(oracle.gelu_tanh(x), Fn.gelu(t, approximate="tanh").numpy(), atol=1e-14)
    assert np.allclose(oracle.silu(x), Fn.silu(t).numpy(), atol=1e-14)
    assert oracle.gelu_tanh(np.array([0.0]))[0] == 0.0
    assert oracle.silu(np.array([0.0]))[0] == 0.0
    s = oracle.softmax_rows(np.array([[0.0, math.log(3.0)]]))
    assert np.allclose(s, [[0.25, 0.75]], atol=1e-15)


def test_timestep_features_and_positions_closed_forms():
    f0 = oracle.timestep_features(0.0, 256)
    assert np.array_equal(f0, np.concatenate([np.ones(128), np.zeros(128)]))
    f1 = oracle.timestep_features(1.0, 256)
    assert math.isclose(f1[0], math.cos(1.0)) and math.isclose(f1[128], math.sin(1.0))
    assert math.isclose(f1[127], math.cos(10000.0 ** (-127 / 128)), rel_tol=1e-12)
    P = oracle.positions(16, 256)
    assert np.array_equal(P[0], np.concatenate([np.zeros(128), np.ones(128)]))
    assert math.isclose(P[5, 0], math.sin(5.0)) and math.isclose(P[5, 128], math.cos(5.0))
    assert math.isclose(P[3, 64], math.sin(3 * 10000.0 ** -0.5), rel_tol=1e-12)


def _naive_attention(q, k, v, nh):
    M, d = q.shape
    hd = d // nh
    out = np.zeros((M, d))
    for h in range(nh):
        for i in range(M):
            s = [sum(q[i, h * hd + c] * k[j, h * hd + c] for c in range(hd)) / math.sqrt(hd)
                 for j in range(k.shape[0])]
            m = max(s)
            w = [math.exp(x - m) for x in s]
            z = sum(w)
            for c in range(hd):
                out[i, h * hd + c] = sum(w[j] * v[j, h * hd + c] for j in range(k.shape[0])) / z
    return out


def test_attention_against_naive_loops_and_torch():
    rng = np.random.default_rng(2)
    q, k, v = rng.standard_normal((5, 16)), rng.standard_normal((9, 16)), rng.standard_normal((9, 16))
    o = oracle.attention(q, k, v, 4)
    assert np.allclose(o, _naive_attention(q, k, v, 4), atol=1e-12)
    tq, tk, tv = (torch.from_numpy(a).view(1, -1, 4, 4).transpose(1, 2) for a in (q, k, v))
    ref = Fn.scaled_dot_product_attention(tq, tk, tv).transpose(1, 2).reshape(5, 16).numpy()
    assert np.allclose(o, ref, atol=1e-12)


def test_attention_special_cases():
    rng = np.random.default_rng(3)
    q, v = rng.standard_normal((4, 32)), rng.standard_normal((1, 32))
    k = rng.standard_normal((1, 32))
    assert np.allclose(oracle.attention(q, k, v, 2), np.repeat(v, 4, 0), atol=1e-15)
    k, v = rng.standard_normal((10, 32)), rng.standard_normal((10, 32))
    o = oracle.attention(np.zeros((3, 32)), k, v, 2)
    assert np.allclose(o, np.repeat(v.mean(0, keepdims=True), 3, 0), atol=1e-14)
    # permuting keys and values together changes nothing
    p = rng.permutation(10)
    q = rng.standard_normal((3, 32))
    assert np.allclose(oracle.attention(q, k, v, 2), oracle.attention(q, k[p], v[p], 2), atol=1e-13)


def test_argmax_against_brute_force():
    rng = np.random.default_rng(4)
    x = rng.integers(-3, 4, (500, 9)).astype(np.float64)   # many ties
    got = oracle.argmax_lowest(x)
    for r in range(x.shape[0]):
        best = 0
        for j in range(1, 9):
            if x[r, j] > x[r, best]:
                best = j
        assert got[r] == best
