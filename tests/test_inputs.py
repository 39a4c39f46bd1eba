"""Seeded input generators: determinism, bf16 rounding and workload shapes."""
import numpy as np
import torch

import mla_inputs as I


def test_bf16_rne_matches_torch():
    rng = np.random.default_rng(0)
    a = np.concatenate([rng.standard_normal(100000).astype(np.float32) * 7,
                        np.array([0.0, -0.0, 1.0, 1.00390625, 1.01171875, 3.0e38, -1e-40], np.float32)])
    ref = torch.from_numpy(a).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(I.rne_bf16_bits(a), ref)
    back = torch.from_numpy(ref.view(np.int16)).view(torch.bfloat16).float().numpy()
    np.testing.assert_array_equal(I.bf16_bits_to_f32(ref), back)


def test_generators_deterministic_and_block_addressable():
    cfg = I.small_variant(I.CONFIGS["deepseek_v2_decode"], d_model=64)
    a = I.x_rows(cfg, 3, 1000, 1100)
    b = I.x_rows(cfg, 3, 0, 2048)[1000:1100]
    np.testing.assert_array_equal(a, b)
    assert not np.array_equal(I.x_rows(cfg, 4, 1000, 1100), a)
    w1, w2 = I.weights(I.CONFIGS["tiny_f32"]), I.weights(I.CONFIGS["tiny_f32"])
    for k in w1:
        np.testing.assert_array_equal(w1[k], w2[k])
    # bf16 workloads hold exactly representable values
    x = I.x_rows(cfg, 0, 0, 16)
    np.testing.assert_array_equal(I.quantize(x, "bf16"), x)


def test_workload_shapes_and_lengths():
    c4 = I.CONFIGS["qwen3_30b_ragged_decode"]
    n = I.context_lengths(c4)
    assert n.shape == (8,) and n.min() >= 1024 and n.max() <= 32768
    np.testing.assert_array_equal(n, I.context_lengths(c4))
    c5 = I.CONFIGS["long_prefill_131k"]
    rows = I.sample_rows(c5)
    assert rows.shape == (512,) and rows[0] == 0 and rows[-1] == 131071
    assert np.all(np.diff(rows) > 0)
    for name, cfg in I.CONFIGS.items():
        shp = cfg.weight_shapes()
        assert shp["w_uk"] == (cfg.n_heads, cfg.d_nope, cfg.rank)
        assert cfg.n_heads % cfg.n_groups == 0
    assert I.CONFIGS["deepseek_v2_decode"].row_width == 576
    assert abs(I.CONFIGS["deepseek_v2_decode"].softmax_scale - 1 / np.sqrt(192)) < 1e-15
