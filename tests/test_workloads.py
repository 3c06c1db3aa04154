"""Sanity of the seeded synthetic inputs (no oracle arithmetic involved)."""

import numpy as np

import workloads as W


def test_tiny_fp32_decode_layout():
    c = W.tiny_fp32_decode()
    assert c.pool.k.shape == (32, 32, 4, 64) and c.pool.k.dtype == np.float32
    assert c.tables.shape == (2, 10) and list(c.kv_lens) == [256, 256]
    assert c.new_k.shape == (4, 4, 64) and len(c.slots) == 4
    # the new tokens' slots hold poison until they are scattered
    flat = c.pool.k.reshape(-1, 4, 64)
    assert np.all(np.isnan(flat[c.slots]))
    # the trailing table entries point at the poison page, which is all NaN
    assert np.all(c.tables[:, 8:] == c.poison_page)
    assert np.all(np.isnan(c.pool.k[c.poison_page]))
    # 16 of the 32 pages are owned and finite except the new-token slots
    owned = np.unique(c.tables[:, :8])
    assert len(owned) == 16
    finite_rows = np.isfinite(c.pool.k[owned]).all(axis=(2, 3)).sum()
    assert finite_rows == 16 * 32 - 4


def test_seeded_inputs_are_reproducible():
    a, b = W.tiny_fp32_decode(), W.tiny_fp32_decode()
    assert np.array_equal(a.q, b.q) and np.array_equal(a.tables, b.tables)
    assert np.array_equal(a.pool.k, b.pool.k, equal_nan=True)


def test_fp8_case_codes_are_finite_where_owned():
    c = W.make_decode_case("t", 3, 4, 3, 8, 2, 64, 32, [40, 1, 64], kv_dtype="fp8", new_per_seq=0)
    assert c.pool.k.dtype == np.uint8 and c.pool.k_scale.shape == (c.pool.num_pages, 2)
    for t, L in enumerate(c.kv_lens):
        for p in range(int(L)):
            code = c.pool.k[c.tables[t, p // 32], p % 32]
            assert np.all((code & 0x7F) != 0x7F)
    # dead rows of a partial last page are poison
    assert np.all(c.pool.k[c.tables[0, 1], 8:] == 0x7F)


def test_prefill_case_padding_slots_are_skipped():
    c = W.make_prefill_case("p", 1, 2, 1, 12, [10], [7], 4, 2, 64, 4, 0)
    assert c.slots.shape == (12,) and np.all(c.slots[10:] == -1) and np.all(c.slots[:10] >= 0)
    assert c.qkv.shape == (1, 12, 8, 64)


def test_shared_prefix_case_tables():
    c = W.make_shared_prefix_case("s", 1, 2, 2, 3, 64, (1, 40), 8, 2, 64, 32, 64)
    assert c.prefix_tables.shape == (2, 2) and c.tail_tables.shape == (6, 2)
    assert np.array_equal(c.full_tables[:3, :2], np.repeat(c.prefix_tables[:1], 3, 0))
    assert np.array_equal(c.full_lens, c.tail_lens + 64)
