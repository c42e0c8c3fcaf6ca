"""Seeded input generator checks (CPU only)."""
import numpy as np
import torch

import fa_inputs as fi


def test_bf16_rounding_matches_torch():
    x = np.random.default_rng(0).standard_normal(100000, dtype=np.float32) * 3
    x[:4] = [0.0, -0.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8]  # ties to even both ways
    ours = fi.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(ours, ref)


def test_fp16_rounding_matches_torch():
    x = np.random.default_rng(1).standard_normal(100000, dtype=np.float32) * 3
    ours = fi.f32_to_fp16_bits(x)
    ref = torch.from_numpy(x).to(torch.float16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(ours, ref)


def test_deterministic_per_seed():
    a = fi.prefill_inputs(9, 1, 2, 1, 8, 8, 64, True)
    b = fi.prefill_inputs(9, 1, 2, 1, 8, 8, 64, True)
    c = fi.prefill_inputs(10, 1, 2, 1, 8, 8, 64, True)
    np.testing.assert_array_equal(a.q, b.q)
    np.testing.assert_array_equal(a.v, b.v)
    assert not np.array_equal(a.q, c.q)
    assert not np.array_equal(a.k, a.v)


def test_split_pool_structure():
    lens = np.array([33, 16, 1, 0], dtype=np.int32)
    d = fi.split_decode_inputs(11, 4, 8, 2, 128, lens, 16, spare_pages=5)
    assert d.page_table.shape == (4, 3)
    used = d.page_table[d.page_table >= 0]
    assert len(np.unique(used)) == len(used) == 3 + 1 + 1
    assert (d.page_table[1, 1:] == -1).all() and (d.page_table[3] == -1).all()
    pool = d.pool
    nan = fi.NAN_BITS[fi.BF16]
    # tail of sequence 0's last page (tokens 33..47 -> slots 1..15) is poisoned
    last = d.page_table[0, 2]
    assert (pool[last, :, :, 1:, :] == nan).all() and (pool[last, :, :, :1, :] != nan).all()
    # full pages carry data, spare pages are all NaN
    assert (pool[d.page_table[1, 0]] != nan).all()
    spare = np.setdiff1d(np.arange(pool.shape[0]), used)
    assert len(spare) == 5 and (pool[spare] == nan).all()


def test_mla_page_table_is_permutation():
    d = fi.mla_decode_inputs(12, 4, 16, 32, D_qk=72, D_v=64)
    assert sorted(d.page_table.ravel().tolist()) == list(range(4 * 32))
    assert d.pool.shape == (128, 1, 72)
    assert d.scale == np.float32(1 / np.sqrt(192.0))


def test_random_lens_closed_range():
    lens = fi.random_lens(5, 1000, 1024, 32768)
    assert lens.min() >= 1024 and lens.max() <= 32768
    assert fi.random_lens(5, 4, 1024, 32768).tolist() == fi.random_lens(5, 4, 1024, 32768).tolist()
