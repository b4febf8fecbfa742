"""Pins of the oracle's QK RMSNorm and partial RoPE: the defining property of
rotary encoding (a score depends only on the position difference), the
rotation as a complex product (numpy's complex exponential), inversion,
norms, the untouched dims, and torch's rms_norm. CPU only."""
import numpy as np
import torch

import oracle


def test_rope_relative_positions():
    g = np.random.default_rng(0)
    q, k = g.standard_normal((2, 512))
    for p, s in [(5, 3), (1000, 998), (123456, 123454)]:
        a = oracle.rope_rotate(q[None], [p])[0] @ oracle.rope_rotate(k[None], [s])[0]
        b = oracle.rope_rotate(q[None], [p - s])[0] @ oracle.rope_rotate(k[None], [0])[0]
        assert abs(a - b) < 1e-9 * (1 + abs(a))


def test_rope_is_a_complex_product_on_the_last_dims():
    g = np.random.default_rng(1)
    x = g.standard_normal((3, 4, 512))
    pos = np.array([0, 17, 1 << 20])
    y = oracle.rope_rotate(x, pos, rope_dims=64, theta=10000.0)
    assert np.array_equal(y[..., :448], x[..., :448])
    z = x[..., 448::2] + 1j * x[..., 449::2]
    freq = 10000.0 ** (-np.arange(32) / 32.0)
    w = z * np.exp(1j * pos[:, None, None] * freq)
    assert np.allclose(y[..., 448::2], w.real, atol=1e-12) and np.allclose(y[..., 449::2], w.imag, atol=1e-12)
    assert np.array_equal(y[0], x[0])  # position 0 rotates nothing


def test_rope_inverse_and_norm():
    g = np.random.default_rng(2)
    x = g.standard_normal((5, 2, 512))
    pos = g.integers(0, 1 << 20, 5)
    y = oracle.rope_rotate(x, pos)
    assert np.allclose(oracle.rope_rotate(y, pos, inverse=True), x, atol=1e-12)
    assert np.allclose(np.linalg.norm(y, axis=-1), np.linalg.norm(x, axis=-1))


def test_rms_norm_against_torch_and_closed_forms():
    g = np.random.default_rng(3)
    x = g.standard_normal((6, 3, 512))
    gamma = g.uniform(0.5, 1.5, 512)
    ref = torch.nn.functional.rms_norm(torch.from_numpy(x), (512,), torch.from_numpy(gamma), eps=1e-6).numpy()
    assert np.allclose(oracle.rms_norm(x, gamma, 1e-6), ref, atol=1e-12)
    y = oracle.rms_norm(x, None, 0.0)
    assert np.allclose(np.sqrt((y * y).mean(axis=-1)), 1.0)
    assert np.allclose(oracle.rms_norm(7.5 * x, None, 0.0), y)  # scale invariance
