"""The seeded generator: storage encodings against torch's conversions, seeding
determinism, and the workload shapes against the figures the pages state."""
import json
import os

import numpy as np
import torch

from synth import gen

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_bf16_rounding_matches_torch():
    g = np.random.default_rng(0)
    x = (g.standard_normal(100000) * np.exp(g.uniform(-20, 20, 100000))).astype(np.float32)
    x[:4] = [1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -(1.0 + 2 ** -8), 0.0]  # ties to even
    mine = gen.bf16_bits(x)
    lib = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(mine, lib)


def test_e4m3_encode_matches_torch_in_range():
    g = np.random.default_rng(1)
    x = (g.standard_normal(200000) * np.exp(g.uniform(-12, 6, 200000))).astype(np.float32)
    x = np.clip(x, -448, 448)
    # exact ties between neighbours, subnormal ties, boundaries
    extra = np.array([0.0, 2 ** -10, 3 * 2 ** -10, 2 ** -6 - 2 ** -10, 1.0625, 1.1875, 448.0, -448.0,
                      240.0, 232.0, 2 ** -9], np.float32)
    x = np.concatenate([x, extra])
    mine = gen.e4m3_encode(x)
    lib = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    # torch keeps the sign of zero; so do we
    assert np.array_equal(mine, lib)


def test_e4m3_saturates():
    codes = gen.e4m3_encode(np.array([500.0, -1e9, 464.0], np.float32))
    assert list(codes) == [0x7E, 0xFE, 0x7E]


def test_quantize_rows_scale():
    x = np.array([[0.0, 0.0], [1.0, -4.48]], np.float32)
    codes, sc = gen.e4m3_quantize_rows(x)
    assert sc[0] == 1.0 and np.isclose(sc[1], 4.48 / 448)
    assert codes[1, 1] == 0xFE  # -448 after scaling


def test_seeding_is_per_tensor_and_part():
    a = gen.rng(2, "q", 3).standard_normal(5)
    b = gen.rng(2, "q", 3).standard_normal(5)
    c = gen.rng(2, "q", 4).standard_normal(5)
    d = gen.rng(2, "kv_comp", 3).standard_normal(5)
    assert np.array_equal(a, b) and not np.array_equal(a, c) and not np.array_equal(a, d)


def test_config_shapes_follow_pages():
    fx = json.load(open(os.path.join(GOLDEN, "page_constants.json")))
    cf = fx["configuration"]
    for c in (gen.C2, gen.C3, gen.C5):
        assert c.m == cf["compress_rate_m"] and c.H_I == cf["indexer_query_heads"]
        assert c.D_I == cf["indexer_head_dim"] and c.H == cf["num_query_heads"]
        assert c.D == cf["head_dim"] and c.W == cf["sliding_window_size"]
    assert gen.C2.top_k == fx["topk_flash_pro"]["flash"] == cf["top_k"]
    assert gen.C5.top_k == fx["topk_flash_pro"]["pro"]
    assert gen.C4.m == cf["compress_rate_m_prime"] == fx["rates"]["hca_m"]
    pe = fx["pro_topk_token_equivalents"]
    assert gen.C5.top_k * gen.C5.m == pe["token_equivalents"]
    assert gen.C4.N == 8192 and gen.C5.N == 262144 and gen.C2.N == 32768


def test_small_decode_generation():
    cfg = gen.scaled(gen.C5, B=2, n=4096)
    x = gen.gen_decode(cfg)
    assert x["k_idx_codes"].shape == (2, 1024, 128) and x["k_idx_codes"].dtype == np.uint8
    assert x["k_scale"].shape == (2, 1024)
    assert x["q"].shape == (2, 64, 512) and x["Ca"].shape == (2, 8, 512)
    # bf16 storage: values are exactly representable
    assert np.array_equal(gen.bf16_round(x["kv_comp"]), x["kv_comp"])
