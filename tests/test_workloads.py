"""The seeded input generator: determinism, distribution, structure of the five batches."""
import json
import os

import numpy as np
import pytest

import workloads as W


def test_stream_is_counter_based_and_deterministic():
    a = W.normal_bf16(7, W.TAG_K, 0, 10000)
    b = W.normal_bf16(7, W.TAG_K, 0, 10000)
    assert np.array_equal(a, b)
    c = W.normal_bf16(7, W.TAG_K, 1234, 500)
    assert np.array_equal(c, a[1234:1734])
    idx = np.array([5, 9999, 0, 4321], dtype=np.uint64)
    assert np.array_equal(W.normal_bf16_at(7, W.TAG_K, idx), a[idx.astype(np.int64)])
    assert not np.array_equal(a, W.normal_bf16(7, W.TAG_V, 0, 10000))
    assert not np.array_equal(a, W.normal_bf16(8, W.TAG_K, 0, 10000))


def test_stream_is_standard_normal():
    x = W.bf16_bits_to_f32(W.normal_bf16(3, 1, 0, 400000)).astype(np.float64)
    assert abs(x.mean()) < 0.01
    assert abs(x.std() - 1.0) < 0.01
    assert abs(np.mean(np.abs(x) < 1.0) - 0.6827) < 0.005
    # bf16 RNE: re-rounding is the identity
    assert np.array_equal(W.f32_to_bf16_bits(W.bf16_bits_to_f32(W.normal_bf16(3, 1, 0, 1000))),
                          W.normal_bf16(3, 1, 0, 1000))


def test_kv_cache_size_formula_matches_page_example():
    with open(os.path.join(os.path.dirname(__file__), "golden", "kv_cache_size_p3.json")) as f:
        g = json.load(f)
    for case in g["cases"]:
        n = W.kv_cache_bytes_formula(g["layers"], g["heads"], g["head_dim"], case["tokens"], g["dtype_bytes"])
        assert case["approx_bytes"] / g["factor"] <= n <= case["approx_bytes"] * g["factor"]


@pytest.mark.parametrize("c", [1, 2, 3, 4, 5])
def test_config_structure(c):
    wl = W.WORKLOADS[c]()
    B = wl.num_queries
    assert wl.block_tables.shape[0] == B
    nb = (wl.seq_lens + 15) // 16
    for b in range(B):
        row = wl.block_tables[b]
        assert np.all(row[:nb[b]] >= 0) and np.all(row[nb[b]:] == -1)
        assert np.all(wl.block_valid[row[:nb[b] - 1]] == 16)
        assert wl.block_valid[row[nb[b] - 1]] == wl.seq_lens[b] - 16 * (nb[b] - 1)
    used = np.unique(np.concatenate([wl.block_tables[b, :nb[b]] for b in range(B)]))
    assert used.size == wl.num_blocks
    expect = {1: (4, 4, 4, 64), 2: (64, 32, 8, 128), 3: (256, 32, 8, 128), 4: (128, 64, 8, 128),
              5: (512, 32, 8, 128)}[c]
    assert (B, wl.num_q_heads, wl.num_kv_heads, wl.head_dim) == expect
    if c == 1:
        assert np.all((wl.seq_lens >= 256 + 32) & (wl.seq_lens <= 256 + 96))
    if c == 2:
        assert np.all((wl.seq_lens >= 2048 + 128) & (wl.seq_lens <= 2048 + 1024))
        assert 150e6 < wl.unique_kv_bytes < 170e6
    if c == 3:
        assert np.all((wl.seq_lens >= 5120 + 64) & (wl.seq_lens <= 5120 + 2048))
        assert 1.0e9 < wl.unique_kv_bytes < 1.3e9
    if c == 4:
        assert np.all(wl.seq_lens == 131072)
        assert wl.unique_kv_bytes == 16 * 131072 * 4096
        assert wl.prefix_ratio == 1.0
    if c == 5:
        assert wl.seq_lens.min() >= 16 and wl.seq_lens.max() <= 32768
        assert wl.prefix_ratio == 0.0
        assert wl.unique_kv_bytes == wl.query_centric_kv_bytes


def test_materialize_marks_empty_slots_nan():
    wl = W.small(2).materialize()
    for blk in range(wl.num_blocks):
        v = wl.block_valid[blk]
        assert np.all(wl.k_pool[blk, :, v:, :] == W.BF16_NAN)
        assert np.all(wl.v_pool[blk, :, :v, :] != W.BF16_NAN)
