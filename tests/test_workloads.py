"""Seeded input generator: determinism, shapes and distribution recipe (CPU only)."""
import numpy as np
import torch

import workloads as wl


def test_splitmix64_reference_values():
    # SplitMix64 from state 0: first outputs of the published generator
    z = wl.splitmix64(0, 3)
    assert [int(v) for v in z] == [0xE220A8397B1DCDAF, 0x6E789E6AA1B965F4, 0x06C45D188009454F]


def test_fill_is_thread_count_independent():
    a = np.empty(300001, np.uint16)
    b = np.empty(300001, np.uint16)
    wl.fill_normal_bf16(a, 42, 0.02, threads=1)
    wl.fill_normal_bf16(b, 42, 0.02, threads=7)
    np.testing.assert_array_equal(a, b)


def test_batch_determinism_and_shapes():
    for idx, cfg in wl.CONFIGS.items():
        b1 = wl.make_batch(cfg, layers=2)
        b2 = wl.make_batch(cfg, layers=2)
        np.testing.assert_array_equal(b1.input_ids, b2.input_ids)
        np.testing.assert_array_equal(b1.qsl, b2.qsl)
        np.testing.assert_array_equal(b1.multipliers, b2.multipliers)
        assert b1.input_ids.shape == (cfg.T,)
        assert b1.qsl[0] == 0 and b1.qsl[-1] == cfg.T and (np.diff(b1.qsl) >= 0).all()
        assert b1.multipliers.shape == (2, cfg.H, cfg.context_len + 1)
        assert (b1.multipliers & 1).all()                      # odd multipliers
        assert not np.array_equal(b1.multipliers[0], b1.multipliers[1])
        assert sum(cfg.vocab_sizes) < 2 ** 31
        assert cfg.H * cfg.D in (128, 2048, 4096, 8192)


def test_config_shapes_from_the_workload_list():
    c = wl.CONFIGS
    assert list(np.diff(wl.make_batch(c[1]).qsl)) == [7, 1, 13, 3]
    assert c[1].vocab_sizes == [9973, 10007, 10009, 10037]
    assert wl.make_batch(c[2]).R == 256
    assert c[3].num_rows == 8388916 and c[4].num_rows == 33556876 and c[5].num_rows == 67109240
    for cfg in c.values():
        for v in cfg.vocab_sizes:
            assert wl._is_prime(v)


def test_prefill_lengths_and_zipf():
    cfg = wl.CONFIGS[3]
    lens = wl.make_lengths(cfg)
    assert lens.sum() == cfg.T and lens.min() >= 1 and lens.max() <= 4096
    toks = wl.zipf_tokens(1, 2, 200000)
    vals, counts = np.unique(toks, return_counts=True)
    top = counts.max() / len(toks)
    assert 0.12 < top < 0.145          # rank-1 mass of truncated Zipf(1.1) over 151936 ranks is ~13.2%
    assert toks.min() >= 0 and toks.max() < wl.QWEN_VOCAB


def test_normal_fill_moments():
    x = wl.bf16_bits_to_f32(wl.normal_bf16((1 << 20,), 5, 0.02)).astype(np.float64)
    assert abs(x.mean()) < 1e-4 and abs(x.std() - 0.02) < 2e-4


def test_generator_encoders_vs_torch():
    rng = np.random.default_rng(0)
    x = (rng.standard_normal(2000) * 100).astype(np.float32)
    x = np.clip(x, -448, 448)
    lib = wl._lib()
    got8 = np.asarray([lib.gen_store_e4m3fn(float(v)) for v in x], np.uint8)
    ref8 = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(got8, ref8)
    got16 = np.asarray([lib.gen_store_bf16(float(v)) for v in x], np.uint16)
    ref16 = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(got16, ref16)


def test_fp8_table_rows_use_full_range():
    cfg = wl.CONFIGS[4]
    q = np.empty((64, cfg.D), np.uint8)
    s = np.empty((64,), np.float32)
    wl.fill_fp8_table(q, s, 64, cfg.D, 9, wl.TABLE_SIGMA)
    mags = q & 0x7F
    assert (mags.max(axis=1) == 0x7E).all()          # each row's max maps to 448
    assert not ((q == 0x7F) | (q == 0xFF)).any()      # no NaN codes
    assert (s > 0).all() and np.isfinite(s).all()
