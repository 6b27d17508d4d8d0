"""Multi-token queries through single-token rows (host; no GPU).

New token i of a query with seq_len T and q_len m attends causally to the
first T - m + i + 1 tokens (its own position included, as every decode query
here).  The rows are written by the library; a plan over them must pack the
tokens of one query together and cover every row exactly (the coverage
checker of the planner tests).
"""
import numpy as np
import pytest

import workloads as W
from test_plan import check_coverage, check_descriptors

K = pytest.importorskip("decode_attention_prefix_amd.kvattn")


def sessions(seed, n=5, Hq=16, Hkv=4, D=128):
    rng = np.random.default_rng(seed)
    segs = [[("sys", 64), (("sess", b), int(rng.integers(40, 700)))] for b in range(n)]
    return W.from_segments("multi_tok_%d" % seed, segs, Hq, Hkv, D, seed, 900 + seed)


def test_rows_follow_the_causal_definition():
    wl = sessions(0)
    q_lens = np.array([1, 3, 8, 17, 32], dtype=np.int32)
    bt, sl = K.kvattn_expand_query_tokens(wl.shape_tuple(), wl.block_tables, wl.seq_lens, q_lens)
    assert bt.shape == (int(q_lens.sum()), wl.max_blocks) and sl.shape == (int(q_lens.sum()),)
    r = 0
    for b in range(wl.num_queries):
        T, m = int(wl.seq_lens[b]), int(q_lens[b])
        for i in range(m):
            assert sl[r] == T - m + i + 1
            nb = (int(sl[r]) + 15) // 16
            assert np.array_equal(bt[r, :nb], wl.block_tables[b, :nb]) and np.all(bt[r, nb:] == -1)
            r += 1


@pytest.mark.parametrize("m", [2, 8, 40])
def test_rows_of_a_query_are_packed(m):
    wl = sessions(1)
    q_lens = np.full(wl.num_queries, m, dtype=np.int32)
    bt, sl = K.kvattn_expand_query_tokens(wl.shape_tuple(), wl.block_tables, wl.seq_lens, q_lens)
    shape = (len(sl), wl.num_q_heads, wl.num_kv_heads, wl.head_dim, 16, wl.max_blocks, wl.num_blocks)
    plan = K.kvattn_plan(shape, bt, sl)
    ex = K.kvattn_plan_export(plan)
    check_coverage(bt, sl, wl.num_q_heads, wl.num_kv_heads, ex)
    check_descriptors(ex)
    st = K.kvattn_plan_stats(plan)
    # every KV token is read about once, not once per row
    assert st["planned_kv_bytes"] < 1.25 * st["unique_kv_bytes"] + 16 * len(sl) * wl.bytes_per_token
    assert st["planned_kv_bytes"] < 0.5 * st["query_centric_kv_bytes"]


def test_bad_q_lens_are_rejected():
    wl = sessions(2)
    for bad in (0, int(wl.seq_lens[0]) + 1):
        q_lens = np.ones(wl.num_queries, dtype=np.int32)
        q_lens[0] = bad
        with pytest.raises(K.KvattnError):
            K.kvattn_expand_query_tokens(wl.shape_tuple(), wl.block_tables, wl.seq_lens, q_lens)
