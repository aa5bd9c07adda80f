"""Host-side checks of the seeded input generator (no GPU)."""
import numpy as np
import pytest

import workloads as W


@pytest.mark.parametrize("ctr,key,expect", [
    ((0, 0, 0, 0), (0, 0), (0x6627e8d5, 0xe169c58d, 0xbc57ac4c, 0x9b00dbd8)),
    ((0xffffffff,) * 4, (0xffffffff,) * 2, (0x408f276d, 0x41c83b0e, 0xa20bc7c6, 0x6d5451fd)),
    ((0x243f6a88, 0x85a308d3, 0x13198a2e, 0x03707344), (0xa4093822, 0x299f31d0),
     (0xd16cfe09, 0x94fdcceb, 0x5001e420, 0x24126ea1)),
])
def test_philox_known_answers(ctr, key, expect):
    """Known-answer vectors published with the Philox4x32-10 reference code."""
    out = W.philox4x32_10(*[np.uint64(c) for c in ctr], *key)
    assert tuple(int(x) for x in out) == expect


def test_normal_table_is_symmetric_standard_normal():
    t = W.normal_table_f32().astype(np.float64)
    assert t.shape == (65536,)
    np.testing.assert_array_equal(t, -t[::-1])
    assert abs(t.var() - 1.0) < 1e-4 and np.all(np.diff(t) > 0)
    b = W.bf16_bits_to_f32(W.normal_table_bf16_bits())
    assert np.abs(b - t).max() <= 2.0 ** -8 * np.abs(t).max()


def test_bf16_rounding_is_nearest_even():
    x = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 1.0 + 2 ** -9, -2.5 - 2 ** -7], np.float32)
    np.testing.assert_array_equal(W.round_to_bf16(x), [1.0, 1.0, 1.0 + 2 ** -6, 1.0, -2.5])


def test_cache_rows_are_counter_based():
    w = W.get("v3_b64")
    full = W.cache_rows(w, 3, 0, 40)
    part = W.cache_rows(w, 3, 17, 23)
    np.testing.assert_array_equal(full["c_kv"][17:23], part["c_kv"])
    np.testing.assert_array_equal(full["k_rope_raw"][17:23], part["k_rope_raw"])
    other = W.cache_rows(w, 4, 0, 40)
    assert not np.array_equal(full["c_kv"], other["c_kv"])
    assert full["c_kv"].shape == (40, 512) and full["k_rope_raw"].shape == (40, 64)
    # stored values are bf16-representable
    np.testing.assert_array_equal(W.round_to_bf16(full["c_kv"]), full["c_kv"])


def test_workload_shapes():
    w = W.get("v3_paged")
    ctx = W.context_lengths(w)
    assert ctx.min() >= 1024 and ctx.max() <= 32768 and len(ctx) == 128
    table, nblk = W.block_table(w, ctx)
    used = np.sort(table[table >= 0])
    np.testing.assert_array_equal(used, np.arange(nblk))
    pos = W.positions(W.get("v3_split"))
    np.testing.assert_array_equal(pos[0], [131070, 131071])
    q = W.queries(W.get("tiny_fp32"))
    assert q["q_nope"].shape == (1, 1, 4, 32) and q["q_rope"].shape == (1, 1, 4, 16)
    wt = W.weights(W.get("v3_b1"))
    assert wt["w_uk"].shape == (128, 512, 128)
    assert abs(wt["w_uk"].std() * np.sqrt(512) - 1) < 0.01
