"""Incremental plan updates across decode steps (host; no GPU).

A batch is generated at its final lengths; the plan starts from every query
cut back by a few tokens and is brought forward one decode step at a time.
After every step the updated plan must satisfy the same coverage invariant
(bit-exact) and descriptor layout as a fresh plan, and its byte statistics
must equal those the definition gives for the current lengths.
"""
import numpy as np
import pytest

import workloads as W
from test_plan import check_coverage, check_descriptors

K = pytest.importorskip("decode_attention_prefix_amd.kvattn")


def state(wl, cut):
    """Block tables and lengths with query b cut back by cut[b] tokens."""
    lens = (wl.seq_lens - np.asarray(cut, dtype=np.int32)).astype(np.int32)
    bt = wl.block_tables.copy()
    for b, T in enumerate(lens):
        bt[b, (int(T) + 15) // 16:] = -1
    return bt, lens


def unique_tokens(bt, lens):
    best = {}
    for b, T in enumerate(lens):
        nb = (int(T) + 15) // 16
        for j in range(nb):
            v = min(16, int(T) - 16 * j)
            best[int(bt[b, j])] = max(best.get(int(bt[b, j]), 0), v)
    return sum(best.values())


def check_state(plan, wl, bt, lens):
    ex = K.kvattn_plan_export(plan)
    check_coverage(bt, lens, wl.num_q_heads, wl.num_kv_heads, ex)
    check_descriptors(ex)
    st = K.kvattn_plan_stats(plan)
    bpt = wl.bytes_per_token
    assert st["unique_kv_bytes"] == unique_tokens(bt, lens) * bpt
    assert st["query_centric_kv_bytes"] == int(lens.astype(np.int64).sum()) * bpt
    it = ex["items"]
    assert st["planned_kv_bytes"] == int(it["n_tokens"].astype(np.int64).sum()) * bpt
    return st


def private_tails(seed, B=24, shared=96, Hq=8, Hkv=2, D=128):
    rng = np.random.default_rng(seed)
    segs = [[("root", shared), (("own", b), int(rng.integers(20, 120)))] for b in range(B)]
    return W.from_segments("upd_private_%d" % seed, segs, Hq, Hkv, D, seed, 700 + seed, extra_blocks=4)


@pytest.mark.parametrize("seed", [0, 1, 2])
@pytest.mark.parametrize("opts", [{}, {"pack_mode": 0}, {"split_tokens": 32}, {"force_variant": 1}])
def test_private_growth_one_token_per_step(seed, opts):
    wl = private_tails(seed)
    steps = 18   # crosses every query's block boundary at least once
    cut = np.full(wl.num_queries, steps, dtype=np.int32)
    bt, lens = state(wl, cut)
    plan = K.kvattn_plan(wl.shape_tuple(), bt, lens, None, K.make_options(**opts))
    assert K.kvattn_plan_stats(plan)["update_path"] == 0
    check_state(plan, wl, bt, lens)
    paths = []
    for k in range(steps):
        cut -= 1
        bt, lens = state(wl, cut)
        K.kvattn_plan_update(plan, bt, lens)
        st = check_state(plan, wl, bt, lens)
        paths.append(st["update_path"])
    # private tails extend their own items: no step needs a fresh plan
    assert set(paths) <= {1, 2}, paths


def test_descriptor_growth_reserializes():
    """80 steps add 5 blocks to every tail item: descriptors outgrow their padding."""
    rng = np.random.default_rng(4)
    segs = [[("root", 64), (("own", b), int(rng.integers(100, 200)))] for b in range(12)]
    wl = W.from_segments("upd_long", segs, 8, 2, 128, 4, 704)
    cut = np.full(wl.num_queries, 80, dtype=np.int32)
    bt, lens = state(wl, cut)
    plan = K.kvattn_plan(wl.shape_tuple(), bt, lens)
    paths = []
    for k in range(80):
        cut -= 1
        bt, lens = state(wl, cut)
        K.kvattn_plan_update(plan, bt, lens)
        paths.append(check_state(plan, wl, bt, lens)["update_path"])
    assert set(paths) == {1, 2}, paths


def test_some_queries_grow_several_tokens():
    wl = private_tails(7)
    rng = np.random.default_rng(3)
    cut = rng.integers(0, 19, wl.num_queries).astype(np.int32)
    bt, lens = state(wl, cut)
    plan = K.kvattn_plan(wl.shape_tuple(), bt, lens)
    while cut.any():
        step = np.minimum(cut, rng.integers(0, 6, wl.num_queries)).astype(np.int32)
        cut -= step
        bt, lens = state(wl, cut)
        K.kvattn_plan_update(plan, bt, lens)
        st = check_state(plan, wl, bt, lens)
        assert st["update_path"] in (1, 2)


@pytest.mark.parametrize("per_sess", [4, 16])
def test_shared_session_growth(per_sess):
    """A session's queries share its whole KV; the session grows for all of them."""
    n_sess, ctx = 3, 640
    segs = [[(("sess", s), ctx)] for s in range(n_sess) for _ in range(per_sess)]
    wl = W.from_segments("upd_sessions_%d" % per_sess, segs, 16, 2, 128, 11, 711)
    cut = np.full(wl.num_queries, 20, dtype=np.int32)
    bt, lens = state(wl, cut)
    plan = K.kvattn_plan(wl.shape_tuple(), bt, lens)
    for k in range(20):
        cut -= 1
        bt, lens = state(wl, cut)
        K.kvattn_plan_update(plan, bt, lens)
        st = check_state(plan, wl, bt, lens)
        assert st["update_path"] in (1, 2)


def test_steps_that_do_not_extend_rebuild():
    wl = private_tails(5)
    cut = np.full(wl.num_queries, 4, dtype=np.int32)
    bt, lens = state(wl, cut)
    plan = K.kvattn_plan(wl.shape_tuple(), bt, lens)
    # a length shrinks: rebuilt from scratch
    cut[0] += 2
    bt, lens = state(wl, cut)
    K.kvattn_plan_update(plan, bt, lens)
    assert check_state(plan, wl, bt, lens)["update_path"] == 3
    # a block of an old position changes: rebuilt
    bt2 = bt.copy()
    spare = int(np.setdiff1d(np.arange(wl.num_blocks), wl.block_tables[wl.block_tables >= 0])[0])
    bt2[1, 0] = spare
    K.kvattn_plan_update(plan, bt2, lens)
    assert K.kvattn_plan_stats(plan)["update_path"] == 3
    check_coverage(bt2, lens, wl.num_q_heads, wl.num_kv_heads, K.kvattn_plan_export(plan))


def test_shared_item_growing_apart_rebuilds():
    """Queries that share their last item but grow into different blocks need new items."""
    segs = [[("root", 160), (("own", b), 32)] for b in range(6)]
    wl = W.from_segments("upd_apart", segs, 8, 2, 128, 13, 713)
    # cut every query back into the shared root: the queries end together there
    cut = np.full(wl.num_queries, 40, dtype=np.int32)
    bt, lens = state(wl, cut)
    # packed explicitly: AUTO plans a batch this small as one launch without packs
    plan = K.kvattn_plan(wl.shape_tuple(), bt, lens, None, K.make_options(pack_mode=K.KVATTN_PACK_FULL))
    cut -= 1
    bt, lens = state(wl, cut)
    K.kvattn_plan_update(plan, bt, lens)
    # shared growth inside the root (same blocks for everyone) extends the plan
    assert check_state(plan, wl, bt, lens)["update_path"] in (1, 2)
    cut[:] = 0
    bt, lens = state(wl, cut)
    K.kvattn_plan_update(plan, bt, lens)
    # now each query grows into its own blocks: a fresh plan
    assert check_state(plan, wl, bt, lens)["update_path"] == 3


def test_invalid_update_leaves_plan_unchanged():
    wl = private_tails(9)
    cut = np.full(wl.num_queries, 3, dtype=np.int32)
    bt, lens = state(wl, cut)
    plan = K.kvattn_plan(wl.shape_tuple(), bt, lens)
    before = K.kvattn_plan_export(plan)
    bad = lens.copy()
    bad[2] = wl.max_blocks * 16 + 1
    with pytest.raises(K.KvattnError):
        K.kvattn_plan_update(plan, bt, bad)
    bad_bt = bt.copy()
    bad_bt[0, 0] = wl.num_blocks
    with pytest.raises(K.KvattnError):
        K.kvattn_plan_update(plan, bad_bt, lens)
    after = K.kvattn_plan_export(plan)
    assert np.array_equal(before["desc"], after["desc"])
    assert np.array_equal(before["block_ids"], after["block_ids"])


def random_forest(seed, extra=6):
    """Random prefix forest with private leaves long enough to grow into."""
    rng = np.random.default_rng(seed)
    B = int(rng.integers(2, 20))
    G = int(rng.choice([1, 2, 4, 8]))
    Hkv = int(rng.choice([1, 2, 4, 8]))
    D = int(rng.choice([64, 128]))
    n_roots = int(rng.integers(1, 4))
    segs = []
    for b in range(B):
        r = int(rng.integers(0, n_roots))
        s = [(("root", r), 16 * int(1 + (r * 7) % 5))]
        if rng.random() < 0.6:
            c = int(rng.integers(0, 3))
            s.append((("child", r, c), 16 * int(1 + c)))
        s.append((("leaf", b), int(rng.integers(30, 120))))
        segs.append(s)
    return W.from_segments("fuzz%d" % seed, segs, G * Hkv, Hkv, D, seed, seed + 1, extra_blocks=extra)


@pytest.mark.parametrize("seed", range(16))
@pytest.mark.parametrize("new_token,multi_stream", [(0, 0), (1, 0), (0, 1)])
def test_update_fuzz_random_forests(seed, new_token, multi_stream):
    """Random forests, random per-step growth (0-3 tokens per query, sometimes none at all):
    after every update the plan satisfies the invariants at the current lengths."""
    wl = random_forest(500 + seed)
    rng = np.random.default_rng(seed)
    cut = rng.integers(8, 28, wl.num_queries).astype(np.int32)
    bt, lens = state(wl, cut)
    opts = K.make_options(new_token=new_token, multi_stream=multi_stream)
    plan = K.kvattn_plan(wl.shape_tuple(), bt, lens, None, opts)
    paths = []
    while cut.any():
        step = np.minimum(cut, rng.integers(0, 4, wl.num_queries)).astype(np.int32)
        if rng.random() < 0.1:
            step[:] = 0
        cut -= step
        bt, lens = state(wl, cut)
        K.kvattn_plan_update(plan, bt, lens)
        st = K.kvattn_plan_stats(plan)
        paths.append(st["update_path"])
        ex = K.kvattn_plan_export(plan)
        cached = lens - 1 if new_token else lens
        check_coverage(bt, cached, wl.num_q_heads, wl.num_kv_heads, ex, all_merged=bool(new_token))
        check_descriptors(ex)
        if multi_stream:   # every launch still holds one kernel family
            lp = ex["list_ptr"]
            for L in range(lp.shape[0]):
                assert ((lp[L, :, 1] > lp[L, :, 0]).any()) != ((lp[L, :, 2] > lp[L, :, 1]).any())
        if new_token:
            codes = [int(bt[b, (int(T) - 1) // 16]) * 16 + (int(T) - 1) % 16 for b, T in enumerate(lens)]
            for i, b in enumerate(ex["merge_query"]):
                assert ex["merge_rec"][i, 3] == codes[b]
        assert st["unique_kv_bytes"] == unique_tokens(bt, cached) * wl.bytes_per_token
    assert paths and set(paths) <= {1, 2, 3}
