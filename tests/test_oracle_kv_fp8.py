"""Pins of the oracle's mixed-precision KV decoder (E4M3 for all dims but the
last 64, bf16 for the 64 RoPE dims) and of the generator's encoder: hand-built
rows, the layout of the bf16 tail, and torch's own float8_e4m3fn / bfloat16
decodes of the same bytes. CPU only."""
import numpy as np
import torch

import oracle
from synth import gen


def _torch_decode(rows, D):
    t = torch.from_numpy(np.ascontiguousarray(rows))
    nope = t[..., :D - 64].contiguous().view(torch.float8_e4m3fn).to(torch.float64)
    rope = t[..., D - 64:].contiguous().view(torch.bfloat16).to(torch.float64)
    return torch.cat([nope, rope], dim=-1).numpy()


def test_hand_built_row():
    D = 128
    row = np.zeros(D - 64 + 128, np.uint8)
    row[0] = 0x38        # E4M3 1.0 (exponent 7 = bias, mantissa 0)
    row[1] = 0xC4        # -3.0 = -(1 + 4/8) * 2^1
    row[2] = 0x01        # smallest subnormal 2^-9
    row[63] = 0x7E       # 448, the largest finite value
    row[64:66] = [0xC0, 0x3F]   # dim 64 (first RoPE dim) = bf16 0x3FC0 = 1.5
    row[190:192] = [0x20, 0xC1]  # dim 127 = bf16 0xC120 = -10.0
    v = oracle.kv_fp8_decode(row[None], D)[0]
    assert v[0] == 1.0 and v[1] == -3.0 and v[2] == 2.0 ** -9 and v[63] == 448.0
    assert v[64] == 1.5 and v[127] == -10.0
    assert np.all(v[3:63] == 0) and np.all(v[65:127] == 0)


def test_decode_matches_torch_on_all_codes():
    D = 512
    g = np.random.default_rng(0)
    rows = g.integers(0, 256, (64, D - 64 + 128)).astype(np.uint8)
    rows[:, :256] = np.arange(256, dtype=np.uint8)  # every E4M3 code once
    # keep the bf16 tail finite (exponent field not all ones)
    rows[:, D - 64 + 1::2] &= 0xBF
    a, b = oracle.kv_fp8_decode(rows, D), _torch_decode(rows, D)
    nan = np.isnan(b)
    assert np.array_equal(np.isnan(a), nan)
    assert np.array_equal(a[~nan], b[~nan])


def test_encoder_round_trip_and_rounding():
    D = 512
    g = np.random.default_rng(1)
    x = g.standard_normal((32, D)).astype(np.float32)
    x[0, :4] = [500.0, -1000.0, 448.0, 0.0]  # saturation at +-448
    rows = gen.kv_fp8_rows(x)
    assert rows.shape == (32, D - 64 + 128) and rows.dtype == np.uint8
    v = oracle.kv_fp8_decode(rows, D)
    assert list(v[0, :4]) == [448.0, -448.0, 448.0, 0.0]
    # RoPE dims: exactly the bf16 rounding; E4M3 dims: within half a step
    # (3 mantissa bits: relative 2^-4) or the subnormal half-unit 2^-10
    assert np.array_equal(v[:, D - 64:], gen.bf16_round(x[:, D - 64:]).astype(np.float64))
    xs = np.clip(x[:, :D - 64].astype(np.float64), -448, 448)
    assert np.all(np.abs(v[:, :D - 64] - xs) <= np.maximum(np.abs(xs) * 2.0 ** -4, 2.0 ** -10) + 1e-12)
    # in range, the encoder's codes are torch's round-to-nearest-even cast
    t = torch.from_numpy(xs[1:]).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(rows[1:, :D - 64], t)
