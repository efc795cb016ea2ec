"""The seeded input generator: determinism, bf16 rounding, layout and padding."""
import numpy as np
import torch

import kvsynth


def test_bf16_round_to_nearest_even_matches_torch():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.normal(size=100000).astype(np.float32) * 100,
                        rng.lognormal(size=1000).astype(np.float32),
                        np.array([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -1.0 - 2 ** -8, 0.0, -0.0,
                                  3.0e38, 1e-40, 2 ** -130], np.float32)])
    ours = kvsynth.to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(ours, ref)
    back = kvsynth.bf16_bits_to_f32(ours)
    np.testing.assert_array_equal(back, torch.from_numpy(ours.view(np.int16)).view(torch.bfloat16).float().numpy())


def test_generation_is_deterministic_and_layered():
    cfg = kvsynth.CONFIGS["tiny"]
    a = kvsynth.make_layer(cfg)
    b = kvsynth.make_layer(cfg, threads=3)
    for key in ("k_cache", "v_cache", "q_obs", "seq_lens"):
        np.testing.assert_array_equal(a[key], b[key])
    assert a["k_cache"].shape == (1, 256, 2, 16) and a["k_cache"].dtype == np.float32
    assert a["q_obs"].shape == (1, 8, 2, 16)
    q0 = kvsynth.decode_q(cfg, 0, 0)
    q1 = kvsynth.decode_q(cfg, 0, 1)
    assert q0.shape == (1, 2, 16) and not np.array_equal(q0, q1)


def test_ragged_lengths_and_nan_padding():
    cfg = kvsynth.custom("rag", batch=4, n_q_heads=4, n_kv_heads=2, head_dim=16, seq_capacity=64,
                         obs_window=4, keep=8, dtype="bf16", lowrank=4, ragged=(10, 64))
    L = kvsynth.make_layer(cfg)
    lens = L["seq_lens"]
    assert lens.dtype == np.int32 and ((lens >= 10) & (lens <= 64)).all()
    for b, n in enumerate(lens):
        assert (L["k_cache"][b, n:] == kvsynth.BF16_NAN).all()
        assert (L["v_cache"][b, n:] == kvsynth.BF16_NAN).all()
        assert np.isfinite(kvsynth.as_float(L["k_cache"][b, :n])).all()


def test_channel_scales_have_outliers_and_are_shared_by_the_group():
    cfg = kvsynth.CONFIGS["mistral-7b-gqa-32k"]
    s = kvsynth.channel_scale(cfg, 0)
    assert s.shape == (8, 128)
    # x8 outliers: per kv head the largest scales sit well above the median
    assert (np.sort(s, axis=1)[:, -1] > 4 * np.median(s, axis=1)).all()
    cfg5 = kvsynth.CONFIGS["llama3-8b-128k"]
    assert cfg5.layer_sigma(0) == 0.5 and cfg5.layer_sigma(31) == 1.5


def test_config_table_matches_the_workloads():
    c = kvsynth.CONFIGS
    assert (c["llama2-7b-layer-4k"].keep, c["mistral-7b-gqa-32k"].keep,
            c["batched-ragged-16k"].keep, c["llama3-8b-128k"].keep, c["tiny"].keep) == (77, 64, 51, 64, 8)
    assert c["llama3-8b-128k"].seq_capacity == 131072 and c["llama3-8b-128k"].layers == 32
    assert c["batched-ragged-16k"].ragged == (8192, 16384) and c["batched-ragged-16k"].batch == 8
    assert c["mistral-7b-gqa-32k"].group == 4 and c["llama2-7b-layer-4k"].group == 1
