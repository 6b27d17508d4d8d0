"""Host planner: coverage invariant (bit-exact), byte model, determinism, validation.

The coverage checker below is written from the definition, independently of
the planner: for every query b and every token t < seq_len[b], exactly one
(item, entry) pair covers t, and that item reads the physical block
block_tables[b][t // 16] at the position holding t.  Every item runs for every
KV head, so this holds per KV head too.  A query covered by one entry is
written directly; otherwise all its entries carry disjoint partial slots and
the merge map lists exactly those slots.
"""
import numpy as np
import pytest

import workloads as W

K = pytest.importorskip("decode_attention_prefix_amd.kvattn")


def check_coverage(wl_bt, seq_lens, Hq, Hkv, ex, all_merged=False):
    """Every token of every query read exactly once; destinations and merge map consistent.

    all_merged: every query's rows go through the merge (new-token plans), even
    with one partial or none.
    """
    B = len(seq_lens)
    G = Hq // Hkv
    it, en, ids = ex["items"], ex["entries"], ex["block_ids"]
    cover = [np.zeros(int(T), dtype=np.int32) for T in seq_lens]
    per_query = [[] for _ in range(B)]
    for i in range(len(it["kind"])):
        n_tok, pb = int(it["n_tokens"][i]), int(it["pos_begin"][i])
        q0, nq = int(it["q_begin"][i]), int(it["n_q"][i])
        assert it["n_rows"][i] == nq * G
        assert it["kind"][i] in (K.KVATTN_VARIANT_VALU, K.KVATTN_VARIANT_MFMA, K.KVATTN_VARIANT_VALU_SPLIT)
        valu = it["kind"][i] != K.KVATTN_VARIANT_MFMA
        if valu:
            assert it["n_rows"][i] <= it["tile"][i] <= (4 if ex["head_dim"] == 128 else 8)
        else:
            assert it["tile"][i] in (1, 2) and it["n_rows"][i] <= 64 * it["tile"][i]
        nblk = (n_tok + 15) // 16
        assert nblk <= (512 if valu else 1408)
        if it["kind"][i] == K.KVATTN_VARIANT_VALU_SPLIT:
            assert nblk >= 4, "the split tile gives each of four waves a block"
        blk = ids[int(it["blk_begin"][i]): int(it["blk_begin"][i]) + nblk]
        assert blk.size == nblk
        assert any(int(en["limit"][q0 + k]) == n_tok for k in range(nq))
        for k in range(nq):
            b, dest, lim = int(en["query"][q0 + k]), int(en["dest"][q0 + k]), int(en["limit"][q0 + k])
            assert 1 <= lim <= n_tok
            t0 = 16 * pb
            assert t0 + lim <= seq_lens[b]
            # a range ends on a block boundary or at the query's last token
            assert lim % 16 == 0 or t0 + lim == seq_lens[b]
            cover[b][t0:t0 + lim] += 1
            nb = (lim + 15) // 16
            assert np.array_equal(blk[:nb], wl_bt[b, pb:pb + nb]), "item reads another block than the query's"
            per_query[b].append(dest)
    for b in range(B):
        assert np.all(cover[b] == 1), "query %d covered %s times" % (b, np.unique(cover[b]))
    # destinations and merge map
    slots_used = {}
    mq = {int(b): i for i, b in enumerate(ex["merge_query"])}
    for b in range(B):
        d = per_query[b]
        if len(d) == 1 and not all_merged:
            assert d[0] == -1 and b not in mq
        else:
            assert all(x >= 0 for x in d) and b in mq
            i = mq[b]
            listed = ex["merge_dest"][ex["merge_ptr"][i]:ex["merge_ptr"][i + 1]]
            assert sorted(listed.tolist()) == sorted(d)
            rec = ex["merge_rec"][i]
            assert rec[0] == b and rec[2] == len(d)
            if not d:
                continue
            assert rec[1] == int(listed.min())
            # the merge locates a query's partials from its first slot and count:
            # consecutive [Hq]-slot blocks
            first = int(listed.min())
            assert sorted(listed.tolist()) == [first + k * Hq for k in range(len(d))]
            for x in d:
                for h in range(Hq):
                    assert (x + h) not in slots_used
                    slots_used[x + h] = b
    assert len(slots_used) == ex["num_partial_slots"]
    # every item runs on every KV head exactly once: one task per head (MFMA, VALU_SPLIT) or per 4 heads (VALU)
    seen = {}
    for item, head in ex["tasks"]:
        seen.setdefault(int(item), []).append(int(head))
    for i in range(len(it["kind"])):
        heads = sorted(seen.get(i, []))
        step = 4 if it["kind"][i] == K.KVATTN_VARIANT_VALU else 1
        assert heads == list(range(0, Hkv, step)), (i, heads)
    check_descriptors(ex)


DESC_MAX_WORDS = 16 + 4 * 128 + 1408


def check_descriptors(ex):
    """The device descriptor stream encodes exactly the exported tasks, each once.

    Layout (public header): 16 header words (kind, tile, head, tokens, n_q,
    rows, blocks, min limit, words, next words, 0 x 6), n_q entries of 4 words
    (query, dest, limit, merge record or -1), the block ids, zero padding to a
    multiple of 4 words.  Each list holds its
    MFMA descriptors, then its VALU descriptors.
    """
    it, en, ids, desc = ex["items"], ex["entries"], ex["block_ids"], ex["desc"]
    rec_of = {int(b): i for i, b in enumerate(ex["merge_query"])}

    def expected(item, head):
        nt, nq = int(it["n_tokens"][item]), int(it["n_q"][item])
        nb = (nt + 15) // 16
        q0, b0 = int(it["q_begin"][item]), int(it["blk_begin"][item])
        ent = tuple((int(en["query"][q0 + k]), int(en["dest"][q0 + k]), int(en["limit"][q0 + k]))
                    for k in range(nq))
        return (int(it["kind"][item]), int(it["tile"][item]), head, nt, nq, int(it["n_rows"][item]), nb,
                min(e[2] for e in ent), ent, tuple(int(x) for x in ids[b0:b0 + nb]))

    def decode(off):
        h = desc[off:off + 16]
        nq, nb, words = int(h[4]), int(h[6]), int(h[8])
        assert words == 16 + 4 * nq + (nb + 3) // 4 * 4 and words <= DESC_MAX_WORDS
        assert not h[10:16].any()
        ent = tuple(tuple(int(x) for x in desc[off + 16 + 4 * k: off + 19 + 4 * k]) for k in range(nq))
        # word 3: the query's merge record for a partial entry, -1 for a direct row
        assert all(int(desc[off + 19 + 4 * k]) == (rec_of[e[0]] if e[1] >= 0 else -1) for k, e in enumerate(ent))
        blk = tuple(int(x) for x in desc[off + 16 + 4 * nq: off + 16 + 4 * nq + nb])
        assert not desc[off + 16 + 4 * nq + nb: off + words].any()
        return (int(h[0]), int(h[1]), int(h[2]), int(h[3]), nq, int(h[5]), nb, int(h[7]), ent, blk), words

    got, covered = [], 0
    D = ex["head_dim"]
    prev_end = 0
    for L in range(ex["list_ptr"].shape[0]):
        for l in range(ex["num_lists"]):
            m0, v0, e0 = (int(x) for x in ex["list_ptr"][L, l])
            assert prev_end == m0 <= v0 <= e0
            prev_end = e0
            off = m0
            while off < v0:     # MFMA descriptors, chained by next-words
                d, words = decode(off)
                assert d[0] == K.KVATTN_VARIANT_MFMA
                nxt = off + words
                assert int(desc[off + 9]) == (int(desc[nxt + 8]) if nxt < v0 else 0)
                got.append(d)
                covered += words
                off = nxt
            assert off == v0
            rows_max = 1
            while off < e0:     # VALU descriptors (both VALU tiles), copied to LDS in one piece
                d, words = decode(off)
                assert d[0] in (K.KVATTN_VARIANT_VALU, K.KVATTN_VARIANT_VALU_SPLIT) and int(desc[off + 9]) == 0
                rows_max = max(rows_max, d[1])
                got.append(d)
                covered += words
                off += words
            assert off == e0
            # the VALU window: the MFMA stage buffer (512 D bytes) less four q slots per wave
            assert e0 - v0 <= (512 * D - 4 * 4 * rows_max * D * 2) // 4
    assert covered == desc.size
    want = [expected(int(i), int(h)) for i, h in ex["tasks"]]
    assert sorted(got) == sorted(want)


def plan_of(wl, **opts):
    return K.kvattn_plan(wl.shape_tuple(), wl.block_tables, wl.seq_lens, options=K.make_options(**opts))


@pytest.mark.parametrize("c", [1, 2, 3, 4, 5])
@pytest.mark.parametrize("mode", [K.KVATTN_PACK_AUTO, K.KVATTN_PACK_QUERY, K.KVATTN_PACK_FULL])
def test_coverage_full_size_configs(c, mode):
    wl = W.WORKLOADS[c]()
    p = plan_of(wl, pack_mode=mode)
    check_coverage(wl.block_tables, wl.seq_lens, wl.num_q_heads, wl.num_kv_heads, K.kvattn_plan_export(p))
    s = K.kvattn_plan_stats(p)
    assert s["unique_kv_bytes"] == wl.unique_kv_bytes
    assert s["query_centric_kv_bytes"] == wl.query_centric_kv_bytes
    # only the tiny batch is planned as one launch without partials (its queries read their own ranges)
    assert s["one_launch"] == (1 if (c == 1 and mode == K.KVATTN_PACK_AUTO) else 0)
    if mode == K.KVATTN_PACK_QUERY or s["one_launch"]:
        assert s["planned_kv_bytes"] == wl.query_centric_kv_bytes
    else:
        # every shared segment is read once per group of at most 128 rows (q heads of the
        # queries sharing it); nothing else is read twice
        users = {}
        for segs in wl.segments:
            for key, n in segs:
                users.setdefault(key, [0, n])[0] += 1
        extra = 0
        for key, (k, n) in users.items():
            if k >= 2:
                groups = -(-k * wl.group // 128)
                extra += (groups - 1) * n * wl.bytes_per_token
        assert s["planned_kv_bytes"] == wl.unique_kv_bytes + extra


@pytest.mark.parametrize("c", [1, 2, 3, 4, 5])
@pytest.mark.parametrize("variant", [K.KVATTN_VARIANT_VALU, K.KVATTN_VARIANT_MFMA, K.KVATTN_VARIANT_VALU_SPLIT])
@pytest.mark.parametrize("scheme", [1, 2])
def test_coverage_forced_variants_and_schemes(c, variant, scheme):
    wl = W.small(c)
    if variant != K.KVATTN_VARIANT_MFMA and wl.group > (4 if wl.head_dim == 128 else 8):
        with pytest.raises(K.KvattnError):
            plan_of(wl, force_variant=variant)
        return
    for split in (0, 16, 48):
        p = plan_of(wl, force_variant=variant, scheme=scheme, split_tokens=split)
        check_coverage(wl.block_tables, wl.seq_lens, wl.num_q_heads, wl.num_kv_heads, K.kvattn_plan_export(p))
        s = K.kvattn_plan_stats(p)
        if scheme == 1:
            assert s["num_folded_leaves"] == 0


def test_scheme2_folds_one_leaf_per_packed_parent():
    wl = W.config1()
    p = plan_of(wl, pack_mode=K.KVATTN_PACK_FULL, scheme=2, split_tokens=4096)
    s = K.kvattn_plan_stats(p)
    assert s["num_packed_nodes"] == 1 and s["num_folded_leaves"] == 1
    ex = K.kvattn_plan_export(p)
    limits = ex["entries"]["limit"]
    # the folded query attends past the shared prefix inside the packed item
    assert limits.max() > 256 and (limits == 256).any()
    # the folded query has one entry and is written directly
    assert (ex["entries"]["dest"] == -1).sum() == 1


def test_plan_is_deterministic():
    wl = W.config3()
    a = K.kvattn_plan_export(plan_of(wl))
    b = K.kvattn_plan_export(plan_of(wl))
    for key in ("block_ids", "merge_query", "merge_ptr", "merge_dest"):
        assert np.array_equal(a[key], b[key])
    for key in a["items"]:
        assert np.array_equal(a["items"][key], b["items"][key])
    for key in a["entries"]:
        assert np.array_equal(a["entries"][key], b["entries"][key])


def test_packing_reads_shared_prefix_once():
    wl = W.config2()
    s = K.kvattn_plan_stats(plan_of(wl))
    assert s["num_packed_nodes"] == 1 and s["num_items_mfma"] > 0
    # 64 queries x 4 q heads = 256 rows: two 128-row groups read the 2048-token prefix
    assert s["planned_kv_bytes"] == s["unique_kv_bytes"] + 2048 * wl.bytes_per_token
    assert s["planned_kv_bytes"] < s["query_centric_kv_bytes"] / 3.9


def test_profit_model_skips_tiny_shared_node():
    # two queries share one 16-token block, then go their own ways for long tails:
    # re-reading 16 tokens costs less than an extra partial triple per query and head
    segs = [[("p", 16), (("own", b), 3000)] for b in range(2)]
    wl = W.from_segments("tiny_share", segs, 32, 8, 128, 1, 2)
    s = K.kvattn_plan_stats(plan_of(wl))
    assert s["num_packed_nodes"] == 0
    s2 = K.kvattn_plan_stats(plan_of(wl, pack_mode=K.KVATTN_PACK_FULL))
    assert s2["num_packed_nodes"] == 1


def random_tree_workload(seed):
    rng = np.random.default_rng(seed)
    B = int(rng.integers(1, 24))
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
        if rng.random() < 0.8:
            s.append((("leaf", b), int(rng.integers(1, 90))))
        segs.append(s)
    # a query without its own leaf ends on its shared node; make sure the last
    # segment of every query may be partial only if private
    fixed = []
    for s in segs:
        fixed.append(s)
    return W.from_segments("rand%d" % seed, fixed, G * Hkv, Hkv, D, seed, seed + 1, extra_blocks=3)


@pytest.mark.parametrize("seed", range(40))
def test_coverage_random_trees(seed):
    wl = random_tree_workload(seed)
    for mode in (0, 1, 2):
        for scheme in (0, 1, 2):
            for split in (0, 16, 32):
                variant = -1 if seed % 3 else K.KVATTN_VARIANT_MFMA
                p = plan_of(wl, pack_mode=mode, scheme=scheme, split_tokens=split, force_variant=variant)
                check_coverage(wl.block_tables, wl.seq_lens, wl.num_q_heads, wl.num_kv_heads,
                               K.kvattn_plan_export(p))


def tree_from_segments(wl):
    """Explicit prefix tree built from the generator's segment keys (one node per segment key)."""
    node_of = {}
    parent, begin, end = [], [], []
    leaf = []
    for segs in wl.segments:
        par, pos = -1, 0
        for i, (key, n) in enumerate(segs):
            nb = (n + 15) // 16
            k = (key, par)
            if k not in node_of:
                node_of[k] = len(parent)
                parent.append(par)
                begin.append(pos)
                end.append(pos + nb)
            par = node_of[k]
            pos += nb
        leaf.append(par)
    return {"parent": np.array(parent), "block_begin": np.array(begin), "block_end": np.array(end),
            "query_leaf": np.array(leaf)}


@pytest.mark.parametrize("c", [1, 2, 3])
def test_explicit_tree_is_checked_and_used(c):
    wl = W.small(c)
    tree = tree_from_segments(wl)
    p = K.kvattn_plan(wl.shape_tuple(), wl.block_tables, wl.seq_lens, tree=tree)
    check_coverage(wl.block_tables, wl.seq_lens, wl.num_q_heads, wl.num_kv_heads, K.kvattn_plan_export(p))
    derived = K.kvattn_plan_stats(plan_of(wl))
    given = K.kvattn_plan_stats(p)
    assert given["planned_kv_bytes"] == derived["planned_kv_bytes"]
    bad = {k: v.copy() for k, v in tree.items()}
    bad["block_end"][0] += 1          # root claims one block more than the queries share
    with pytest.raises(K.KvattnError) as e:
        K.kvattn_plan(wl.shape_tuple(), wl.block_tables, wl.seq_lens, tree=bad)
    assert e.value.status == K.KVATTN_EINVAL
    bad = {k: v.copy() for k, v in tree.items()}
    bad["parent"][0] = 0
    with pytest.raises(K.KvattnError):
        K.kvattn_plan(wl.shape_tuple(), wl.block_tables, wl.seq_lens, tree=bad)


def test_validation_errors():
    wl = W.small(2)
    shp = list(wl.shape_tuple())

    def expect(status, shape=None, bt=None, sl=None, **opts):
        with pytest.raises(K.KvattnError) as e:
            K.kvattn_plan(tuple(shape or shp), wl.block_tables if bt is None else bt,
                          wl.seq_lens if sl is None else sl, options=K.make_options(**opts) if opts else None)
        assert e.value.status == status, str(e.value)
        assert K.kvattn_last_error() != ""

    sl = wl.seq_lens.copy()
    sl[0] = 0
    expect(K.KVATTN_EINVAL, sl=sl)
    sl = wl.seq_lens.copy()
    sl[1] = 16 * wl.max_blocks + 1
    expect(K.KVATTN_EINVAL, sl=sl)
    bt = wl.block_tables.copy()
    bt[0, 0] = wl.num_blocks
    expect(K.KVATTN_EINVAL, bt=bt)
    bt = wl.block_tables.copy()
    bt[0, 0] = -5
    expect(K.KVATTN_EINVAL, bt=bt)
    s = list(shp)
    s[2] = 7
    expect(K.KVATTN_EINVAL, shape=s)
    s = list(shp)
    s[3] = 96
    expect(K.KVATTN_EUNSUPPORTED, shape=s)
    s = list(shp)
    s[4] = 32
    expect(K.KVATTN_EUNSUPPORTED, shape=s)
    for field in range(7):                    # every shape field must be >= 1 (an empty batch included)
        s = list(shp)
        s[field] = 0
        expect(K.KVATTN_EUNSUPPORTED if field == 4 else K.KVATTN_EINVAL,
               shape=s)
    big = 1 << 17                             # 2^17 queries x 128 q heads x 128 dims = 2^31 q elements
    s = list(shp)
    s[0], s[1], s[2], s[3] = big, 128, 8, 128
    with pytest.raises(K.KvattnError) as e:
        K.kvattn_plan(tuple(s), np.zeros((big, s[5]), dtype=np.int32), np.ones(big, dtype=np.int32))
    assert e.value.status == K.KVATTN_EUNSUPPORTED and "2^31" in K.kvattn_last_error()
    s = list(shp)
    s[1], s[2] = 128, 1                       # 128 q heads on one KV head: wider than 64
    expect(K.KVATTN_EUNSUPPORTED, shape=s)
    s = list(shp)
    s[1], s[2] = 32, 4                        # 8 rows per KV head: more than VALU holds at head_dim 128
    expect(K.KVATTN_EUNSUPPORTED, shape=s, force_variant=0)
    expect(K.KVATTN_EINVAL, pack_mode=7)
    expect(K.KVATTN_EINVAL, split_tokens=-1)
    # unused block-table entries are never read, whatever they hold
    bt = wl.block_tables.copy()
    bt[bt < 0] = 10 ** 9
    K.kvattn_plan(tuple(shp), bt, wl.seq_lens)


def test_device_calls_report_state_errors_without_gpu():
    wl = W.small(1)
    p = plan_of(wl)
    with pytest.raises(K.KvattnError) as e:
        K.kvattn_decode(16, 16, 16, p, 16, stream=0)
    assert e.value.status == K.KVATTN_ESTATE
    with pytest.raises(K.KvattnError) as e:
        K.kvattn_plan_upload(p, 256 * 3, 10, stream=0)
    assert e.value.status == K.KVATTN_EWORKSPACE
    with pytest.raises(K.KvattnError) as e:
        K.kvattn_plan_upload(p, 257, 1 << 30, stream=0)
    assert e.value.status == K.KVATTN_EWORKSPACE
    assert K.kvattn_plan_device_bytes(p) >= K.kvattn_plan_stats(p)["blob_bytes"]


def test_planning_is_reentrant_across_threads():
    """kvattn_plan from several threads at once (ctypes releases the GIL) gives the plans of a serial run."""
    from concurrent.futures import ThreadPoolExecutor
    wls = [W.small(c) for c in (1, 2, 3, 5)] * 3

    def plan_desc(wl):
        p = K.kvattn_plan(wl.shape_tuple(), wl.block_tables, wl.seq_lens)
        ex = K.kvattn_plan_export(p)
        return ex["desc"].copy(), ex["block_ids"].copy()

    serial = [plan_desc(wl) for wl in wls]
    with ThreadPoolExecutor(max_workers=6) as pool:
        parallel = list(pool.map(plan_desc, wls))
    for (d0, b0), (d1, b1) in zip(serial, parallel):
        assert np.array_equal(d0, d1) and np.array_equal(b0, b1)
    # a failing call on one thread leaves the other threads' error strings alone
    bad = W.small(2)
    sl = bad.seq_lens.copy()
    sl[0] = 0

    def fail():
        try:
            K.kvattn_plan(bad.shape_tuple(), bad.block_tables, sl)
        except K.KvattnError:
            return K.kvattn_last_error()
        return ""

    def ok():
        K.kvattn_plan(bad.shape_tuple(), bad.block_tables, bad.seq_lens)
        return K.kvattn_last_error()

    with ThreadPoolExecutor(max_workers=2) as pool:
        f1, f2 = pool.submit(fail), pool.submit(ok)
        assert "seq_lens[0]" in f1.result()
        assert f2.result() == ""


@pytest.mark.parametrize("c", [1, 2, 3, 4, 5])
def test_multi_stream_plans_split_launches_by_kind(c):
    """multi_stream: every forward launch holds one kernel family; coverage and the byte model are unchanged."""
    wl = W.small(c)
    single = plan_of(wl)
    multi = plan_of(wl, multi_stream=1)
    ex = K.kvattn_plan_export(multi)
    check_coverage(wl.block_tables, wl.seq_lens, wl.num_q_heads, wl.num_kv_heads, ex)
    kinds = set(int(k) for k in ex["items"]["kind"])
    lp = ex["list_ptr"]
    launch_kinds = []
    for L in range(lp.shape[0]):
        m0, v0, e0 = lp[L, :, 0], lp[L, :, 1], lp[L, :, 2]
        has_m, has_v = bool((v0 > m0).any()), bool((e0 > v0).any())
        assert has_m != has_v, "launch %d mixes MFMA and VALU lists" % L
        launch_kinds.append(K.KVATTN_VARIANT_MFMA if has_m else K.KVATTN_VARIANT_VALU)
    assert set(launch_kinds) == kinds
    s1, s2 = K.kvattn_plan_stats(single), K.kvattn_plan_stats(multi)
    assert s2["planned_kv_bytes"] >= s2["unique_kv_bytes"]
    assert s2["num_launches"] == lp.shape[0] + (1 if len(ex["merge_query"]) else 0)
    if len(kinds) == 2:
        assert s2["num_launches"] > s1["num_launches"]


def test_tile_selector_by_kv_length():
    """The VALU_SPLIT tile goes to ranges of 4 or more blocks only; shorter ranges keep the VALU
    tile.  The tiny batch is planned as one launch: every query's range whole, no partials, no
    merge launch; larger batches keep the usual plan."""
    wl = W.config1()
    st = K.kvattn_plan_stats(plan_of(wl))
    assert st["one_launch"] == 1 and st["num_launches"] == 1 and st["num_merge_rows"] == 0
    assert st["num_items"] == wl.num_queries and st["num_items_valu_split"] == wl.num_queries
    for c in (2, 3, 4, 5):
        s = K.kvattn_plan_stats(plan_of(W.WORKLOADS[c]()))
        assert s["one_launch"] == 0 and s["num_items_valu_split"] == 0
    # forced: split where the range has 4+ blocks, the VALU tile below
    segs = [[(("own", b), n)] for b, n in enumerate([1, 16, 47, 48, 63, 64, 65, 200, 1000])]
    w2 = W.from_segments("split_lengths", segs, 8, 2, 128, 3, 903)
    ex = K.kvattn_plan_export(plan_of(w2, force_variant=K.KVATTN_VARIANT_VALU_SPLIT, pack_mode=K.KVATTN_PACK_QUERY,
                                      split_tokens=4096))
    check_coverage(w2.block_tables, w2.seq_lens, 8, 2, ex)
    for kind, n in zip(ex["items"]["kind"], ex["items"]["n_tokens"]):
        want = K.KVATTN_VARIANT_VALU_SPLIT if (n + 15) // 16 >= 4 else K.KVATTN_VARIANT_VALU
        assert kind == want, (kind, n)


def test_one_launch_places_each_kv_head_on_one_xcd():
    """In a one-launch plan every task of KV head k sits on a list of XCD k mod 8 (list w runs on
    XCD w mod 8), so the queries that share a prefix read it through one L2."""
    wl = W.config1()
    ex = K.kvattn_plan_export(plan_of(wl))
    lp = np.asarray(ex["list_ptr"]).reshape(-1, 3)
    desc = np.asarray(ex["desc"])
    seen = 0
    for w in range(ex["num_lists"]):
        off, end = lp[w][1], lp[w][2]
        while off < end:
            head = int(desc[off + 2])
            assert head % 8 == w % 8, (w, head)
            seen += 1
            off += int(desc[off + 8])
    assert seen == wl.num_queries * wl.num_kv_heads


def test_mfma_only_chunks_follow_list_rate_classes():
    """A launch of MFMA tasks only (the streaming sessions) cuts each group's range into chunks
    whose lengths follow the rate of the lists they go to: four classes by XCD parity and
    workgroup slot, every list holding chunks of one length class, odd-XCD chunks longer than
    even ones, second-slot chunks shorter than first-slot ones; coverage as always."""
    wl = W.WORKLOADS[4]()
    ex = K.kvattn_plan_export(plan_of(wl))
    check_coverage(wl.block_tables, wl.seq_lens, wl.num_q_heads, wl.num_kv_heads, ex)
    n = ex["num_lists"]
    lp = np.asarray(ex["list_ptr"]).reshape(-1, 3)
    desc = np.asarray(ex["desc"])
    by_class = {}
    for w in range(n):
        off, end = lp[w][0], lp[w][1]
        while off < end:
            by_class.setdefault(((w % 8) % 2, w >= n // 2), []).append(int(desc[off + 3]))
            off += int(desc[off + 8])
    mean = {k: np.mean(v) for k, v in by_class.items()}
    assert set(mean) == {(0, False), (0, True), (1, False), (1, True)}
    for slot in (False, True):
        assert mean[(1, slot)] > 1.05 * mean[(0, slot)]   # odd XCDs: longer chunks
    for par in (0, 1):
        assert mean[(par, True)] < 0.95 * mean[(par, False)]   # second slot: shorter chunks
    # equal task counts per list: two chunks each
    assert all(len(v) == n // 4 * 2 for v in by_class.values())


def test_valu_stripes_follow_list_rates():
    """VALU stripes fill to the level times their lists' rate: second-slot lists (n/2 and up)
    0.9, odd-XCD lists 1.1 when the launch's lists are long (the no-sharing batch, ~520 blocks
    per wave) and 1.0 when they are short (the Llama-3-8B-shaped layer, ~11 blocks)."""
    def blocks(c):
        ex = K.kvattn_plan_export(plan_of(W.WORKLOADS[c]()))
        n = ex["num_lists"]
        lp = np.asarray(ex["list_ptr"]).reshape(-1, 3)
        desc = np.asarray(ex["desc"])
        vb = np.zeros(n)
        for w in range(n):
            off, end = lp[w][1], lp[w][2]
            while off < end:
                vb[w] += desc[off + 6]
                off += int(desc[off + 8])
        w = np.arange(n)
        odd, second = (w % 8) % 2 == 1, w >= n // 2
        return {(o, s): vb[(odd == o) & (second == s)].mean() for o in (False, True) for s in (False, True)}
    b5 = blocks(5)
    for o in (False, True):
        assert 0.85 < b5[(o, True)] / b5[(o, False)] < 0.95
    for s in (False, True):
        assert 1.05 < b5[(True, s)] / b5[(False, s)] < 1.15
    b2 = blocks(2)
    assert 0.93 < b2[(True, False)] / b2[(False, False)] < 1.07   # short lists: no odd-XCD rate
