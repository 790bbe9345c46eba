"""Pins of the blockwise-feedforward oracle (CPU, fp64)."""
import math

import numpy as np
import pytest
import torch

import oracle
from workloads import gen_small


def rand(seed, shape, scale=1.0, stream=0):
    return gen_small(seed, shape, "f32", scale, stream).astype(np.float64)


def test_gelu_closed_forms():
    z = np.array([-30.0, -1.0, 0.0, 1.0, 30.0])
    g = oracle.gelu(z)
    assert g[2] == 0.0
    assert abs(g[4] - 30.0) < 1e-12 and abs(g[0]) < 1e-12
    # Phi(1) = (1 + erf(1/sqrt 2)) / 2
    assert abs(g[3] - 0.5 * (1 + math.erf(1 / math.sqrt(2)))) < 1e-15
    # z Phi(z) - (-z) Phi(-z) = z (Phi(z) + Phi(-z) = 1)
    zz = rand(1, (200,), 3.0)
    np.testing.assert_allclose(oracle.gelu(zz) - oracle.gelu(-zz), zz, atol=1e-13, rtol=0)


def test_gelu_equals_torch_fp64():
    z = rand(2, (1000,), 4.0)
    ref = torch.nn.functional.gelu(torch.from_numpy(z)).numpy()
    np.testing.assert_allclose(oracle.gelu(z), ref, atol=1e-14, rtol=0)


@pytest.mark.parametrize("chunk", [1, 3, 7, 16, 100])
def test_blockwise_equals_all_rows(chunk):
    rows, hid, ffn = 16, 8, 32
    x, w1, w2 = rand(3, (rows, hid)), rand(3, (ffn, hid), 0.3, 1), rand(3, (hid, ffn), 0.2, 2)
    b1, b2 = rand(3, (ffn,), 0.1, 3), rand(3, (hid,), 0.1, 4)
    np.testing.assert_allclose(oracle.ffn_blockwise(x, w1, b1, w2, b2, chunk), oracle.ffn_forward(x, w1, b1, w2, b2),
                               atol=1e-13, rtol=0)


def test_equals_torch_fp64_two_layer_mlp():
    rows, hid, ffn = 5, 6, 24
    x, w1, w2 = rand(4, (rows, hid)), rand(4, (ffn, hid), 0.4, 1), rand(4, (hid, ffn), 0.2, 2)
    b1, b2 = rand(4, (ffn,), 0.1, 3), rand(4, (hid,), 0.1, 4)
    t = torch.nn.functional
    ref = t.linear(t.gelu(t.linear(torch.from_numpy(x), torch.from_numpy(w1), torch.from_numpy(b1))),
                   torch.from_numpy(w2), torch.from_numpy(b2)).numpy()
    np.testing.assert_allclose(oracle.ffn_forward(x, w1, b1, w2, b2), ref, atol=1e-13, rtol=0)


def test_special_weights():
    rows, hid = 7, 8
    x = rand(5, (rows, hid))
    eye = np.eye(hid)
    # identity weights, no bias: y = GELU(x)
    np.testing.assert_allclose(oracle.ffn_forward(x, eye, None, eye, None), oracle.gelu(x), atol=1e-15, rtol=0)
    # W2 = 0: y = b2 on every row
    b2 = rand(5, (hid,), 1.0, 1)
    y = oracle.ffn_forward(x, rand(5, (16, hid), 1.0, 2), None, np.zeros((hid, 16)), b2)
    np.testing.assert_allclose(y, np.broadcast_to(b2, y.shape), atol=0, rtol=0)


def test_planted_mistakes_are_caught(monkeypatch):
    """A tanh-approximate GELU or a dropped bias must fail the torch pin."""
    rows, hid, ffn = 5, 6, 24
    x, w1, w2 = rand(6, (rows, hid)), rand(6, (ffn, hid), 0.8, 1), rand(6, (hid, ffn), 0.2, 2)
    b1, b2 = rand(6, (ffn,), 0.5, 3), rand(6, (hid,), 0.5, 4)
    t = torch.nn.functional
    ref = t.linear(t.gelu(t.linear(torch.from_numpy(x), torch.from_numpy(w1), torch.from_numpy(b1))),
                   torch.from_numpy(w2), torch.from_numpy(b2)).numpy()
    import oracle.ffn as f
    monkeypatch.setattr(f, "gelu", lambda z: 0.5 * z * (1 + np.tanh(math.sqrt(2 / math.pi) * (z + 0.044715 * z ** 3))))
    assert np.max(np.abs(f.ffn_forward(x, w1, b1, w2, b2) - ref)) > 1e-6
    monkeypatch.undo()
    assert np.max(np.abs(f.ffn_forward(x, w1, None, w2, b2) - ref)) > 1e-3
