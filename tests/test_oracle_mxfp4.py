"""Pins of the oracle's MXFP4 decoder and the generator's MXFP4 quantizer
against the OCP Microscaling Formats v1.0 definitions (FP4 E2M1 elements, one
E8M0 scale per block of 32). CPU only."""
import numpy as np
import pytest

import oracle
from synth import gen

# The E2M1 value set of the format definition, codes 0..7 (sign bit 3 negates).
E2M1 = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def _pack(codes):
    codes = np.asarray(codes, np.uint8)
    return (codes[..., 0::2] | (codes[..., 1::2] << 4)).astype(np.uint8)


def test_decode_element_table():
    codes = np.arange(16, dtype=np.uint8)
    row = np.concatenate([codes, np.zeros(16, np.uint8)])  # one block of 32 elements
    v = oracle.mxfp4_decode(_pack(row)[None], np.array([[127]], np.uint8))[0]
    assert list(v[:8]) == E2M1
    assert list(v[8:16]) == [-x for x in E2M1]
    assert np.signbit(v[8])  # code 8 is -0


def test_decode_nibble_order():
    # byte 0x21: element 0 is the low nibble (code 1 = 0.5), element 1 the high (code 2 = 1.0)
    b = np.zeros((1, 16), np.uint8)
    b[0, 0] = 0x21
    v = oracle.mxfp4_decode(b, np.array([[127]], np.uint8))[0]
    assert v[0] == 0.5 and v[1] == 1.0 and np.all(v[2:] == 0)


def test_decode_block_scales():
    row = np.full(64, 7, np.uint8)  # every element 6, two blocks
    v = oracle.mxfp4_decode(_pack(row)[None], np.array([[130, 120]], np.uint8))[0]
    assert np.all(v[:32] == 6.0 * 8) and np.all(v[32:] == 6.0 * 2.0 ** -7)
    v = oracle.mxfp4_decode(_pack(row)[None], np.array([[255, 127]], np.uint8))[0]
    assert np.all(np.isnan(v[:32])) and np.all(v[32:] == 6.0)


def test_encode_round_to_nearest_even_and_saturation():
    # ties go to the even code (mantissa bit 0): 0.25 -> 0, 0.75 -> 1, 1.25 -> 1,
    # 1.75 -> 2, 2.5 -> 2, 3.5 -> 4, 5 -> 4; beyond 6 saturates
    x = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 7.0, 100.0, -5.0, 0.3, -0.0])
    want = [0.0, 1.0, 1.0, 2.0, 2.0, 4.0, 4.0, 6.0, 6.0, -4.0, 0.5, 0.0]
    c = gen.mxfp4_encode_elems(x)
    got = [(-1.0 if ci & 8 else 1.0) * E2M1[ci & 7] for ci in c]
    assert got == want
    assert c[-1] == 0  # -0 encodes as +0


@pytest.mark.parametrize("shift", [-20, -3, 0, 5, 40])
def test_quantize_representable_blocks_round_trip(shift):
    g = np.random.default_rng(3)
    codes = g.integers(0, 16, (4, 128)).astype(np.uint8)
    codes[:, 0::32] = 7  # every block holds +6, so the block maximum fixes the scale
    vals = np.array([(-1.0 if c & 8 else 1.0) * E2M1[c & 7] for c in codes.ravel()]).reshape(codes.shape)
    x = vals * 2.0 ** shift
    q, s = gen.mxfp4_quantize_rows(x)
    # amax = 6 * 2^shift: floor(log2(amax)) - 2 = shift, so the scale byte is 127 + shift
    assert np.all(s == 127 + shift)
    assert np.array_equal(oracle.mxfp4_decode(q, s), x)


def test_quantize_error_bound():
    # with the OCP scale choice the elements carry at most 1 mantissa bit: the
    # error of an element below 6 * 2^X is at most a quarter of its binade, and
    # values above it saturate
    g = np.random.default_rng(4)
    x = g.standard_normal((64, 128))
    q, s = gen.mxfp4_quantize_rows(x)
    d = oracle.mxfp4_decode(q, s)
    scale = np.repeat(np.exp2(s.astype(np.float64) - 127.0), 32, axis=-1)
    below = np.abs(x) <= 6 * scale
    err = np.abs(d - x)
    assert np.all(err[below] <= np.maximum(0.25 * scale[below], 0.25 * np.exp2(np.floor(np.log2(np.abs(x[below]) + 1e-300))) + 1e-12) + 1e-12)
    assert np.all(np.abs(d[~below]) == 6 * scale[~below])
