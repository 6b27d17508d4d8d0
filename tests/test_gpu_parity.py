"""GPU parity: the HIP path through the C ABI against the fp64 oracle, element by element.

Tolerance: max |out_gpu - out_oracle| <= 2e-3 on fp32 outputs from bf16 inputs.
Inputs are seeded and synthetic (workloads); unused token slots of partial
blocks hold NaN, so a kernel that lets them into the result fails.
"""
import os
import sys

import numpy as np
import pytest

import oracle
import workloads as W

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

TOL = 2e-3


def gpu_available():
    return torch.cuda.is_available()


@pytest.fixture(scope="module", autouse=True)
def need_gpu():
    if not gpu_available():
        pytest.skip("no GPU")


def K():
    from decode_attention_prefix_amd import kvattn
    return kvattn


_oracle_cache = {}


def oracle_out(wl, scale=0.0):
    key = (wl.name, wl.shape_tuple(), scale, wl.seed_values)
    if key not in _oracle_cache:
        _oracle_cache[key] = oracle.decode_workload(wl, scale=scale)
    return _oracle_cache[key]


_dev_cache = {}


def device_inputs(wl):
    key = (wl.name, wl.shape_tuple(), wl.seed_values)
    if key not in _dev_cache:
        _dev_cache.clear()
        q = torch.from_numpy(wl.q.view(np.int16)).cuda()
        k = torch.from_numpy(wl.k_pool.view(np.int16)).cuda()
        v = torch.from_numpy(wl.v_pool.view(np.int16)).cuda()
        _dev_cache[key] = (q, k, v)
    return _dev_cache[key]


def gpu_decode(wl, **opts):
    k = K()
    print("case %s opts %s" % (wl.name, opts), flush=True)
    dec = k.Decoder(wl.shape_tuple(), wl.block_tables, wl.seq_lens, options=k.make_options(**opts))
    q, kc, vc = device_inputs(wl)
    out = torch.full((wl.num_queries, wl.num_q_heads, wl.head_dim), float("nan"), dtype=torch.float32,
                     device="cuda")
    dec.decode(q, kc, vc, out)
    torch.cuda.synchronize()
    return out.cpu().numpy().astype(np.float64), dec


def assert_close(got, ref, what):
    assert np.all(np.isfinite(got)), "%s: non-finite outputs" % what
    err = np.abs(got - ref)
    i = np.unravel_index(np.argmax(err), err.shape)
    assert err.max() <= TOL, "%s: max abs err %.3e at %s (got %r ref %r)" % (what, err.max(), i, got[i], ref[i])
    return float(err.max())


def expect_unsupported(wl, **opts):
    """Forcing the VALU forward on a GQA group wider than it holds is refused at plan time."""
    k = K()
    with pytest.raises(k.KvattnError) as ei:
        k.kvattn_plan(wl.shape_tuple(), wl.block_tables, wl.seq_lens, None, k.make_options(**opts))
    assert ei.value.status == k.KVATTN_EUNSUPPORTED, str(ei.value)


_small = {}


def small(c):
    if c not in _small:
        _small[c] = W.small(c).materialize()
    return _small[c]


@pytest.mark.parametrize("c", [1, 2, 3, 4, 5])
@pytest.mark.parametrize("mode", [0, 1, 2])
def test_parity_small_configs_auto_variant(c, mode):
    wl = small(c)
    got, dec = gpu_decode(wl, pack_mode=mode)
    assert_close(got, oracle_out(wl), "%s mode %d" % (wl.name, mode))


@pytest.mark.parametrize("c", [1, 2, 3, 4, 5])
@pytest.mark.parametrize("variant", [0, 1, 2])
@pytest.mark.parametrize("scheme,split", [(1, 0), (2, 0), (1, 16), (2, 48), (0, 208)])
def test_parity_small_configs_forced_variant(c, variant, scheme, split):
    wl = small(c)
    if variant in (0, 2) and wl.group > valu_max_rows(wl.head_dim):
        expect_unsupported(wl, pack_mode=2, force_variant=variant, scheme=scheme, split_tokens=split)
        return
    got, _ = gpu_decode(wl, pack_mode=2, force_variant=variant, scheme=scheme, split_tokens=split)
    assert_close(got, oracle_out(wl), "%s variant %d scheme %d split %d" % (wl.name, variant, scheme, split))


@pytest.mark.parametrize("c", [2, 3, 5])
@pytest.mark.parametrize("variant", [-1, 0, 1, 2])
def test_parity_lists_claimed_past_the_grid(c, variant):
    """A plan for more workgroup slots than the GPU has (num_cus 1024: 2048
    lists) leaves the lists past the grid to run-time claims.  Two decodes in
    a row: the claim counter must be back at zero after the first."""
    wl = small(c)
    if variant in (0, 2) and wl.group > valu_max_rows(wl.head_dim):
        expect_unsupported(wl, num_cus=1024, force_variant=variant)
        return
    k = K()
    print("case %s claims variant %d" % (wl.name, variant), flush=True)
    dec = k.Decoder(wl.shape_tuple(), wl.block_tables, wl.seq_lens,
                    options=k.make_options(num_cus=1024, force_variant=variant))
    q, kc, vc = device_inputs(wl)
    for rep in range(2):
        out = torch.full((wl.num_queries, wl.num_q_heads, wl.head_dim), float("nan"), dtype=torch.float32,
                         device="cuda")
        dec.decode(q, kc, vc, out)
        torch.cuda.synchronize()
        assert_close(out.cpu().numpy().astype(np.float64), oracle_out(wl),
                     "%s claims variant %d decode %d" % (wl.name, variant, rep))


def _cut_state(wl, cut):
    import dataclasses
    lens = (wl.seq_lens - np.asarray(cut, dtype=np.int32)).astype(np.int32)
    bt = wl.block_tables.copy()
    for b, T in enumerate(lens):
        bt[b, (int(T) + 15) // 16:] = -1
    return dataclasses.replace(wl, seq_lens=lens, block_tables=bt)


@pytest.mark.parametrize("kind", ["private", "session"])
def test_parity_across_plan_updates(kind):
    """Plan at shortened lengths, then kvattn_plan_update one decode step at a
    time (crossing block boundaries and descriptor growth); after every step
    the decode matches the oracle at the current lengths."""
    rng = np.random.default_rng(21)
    if kind == "private":
        segs = [[("root", 96), (("own", b), int(rng.integers(90, 160)))] for b in range(10)]
        wl = W.from_segments("upd_gpu_private", segs, 8, 2, 128, 21, 721).materialize()
    else:
        segs = [[(("sess", s), 480)] for s in range(2) for _ in range(8)]
        wl = W.from_segments("upd_gpu_session", segs, 16, 2, 128, 22, 722).materialize()
    k = K()
    steps = 70
    cut = np.full(wl.num_queries, steps, dtype=np.int32)
    cur = _cut_state(wl, cut)
    print("case plan updates %s" % kind, flush=True)
    dec = k.Decoder(wl.shape_tuple(), cur.block_tables, cur.seq_lens)
    q, kc, vc = device_inputs(wl)
    paths = []
    for step in range(steps + 1):
        if step:
            cut -= 1
            cur = _cut_state(wl, cut)
            dec.update(cur.block_tables, cur.seq_lens)
            paths.append(dec.stats()["update_path"])
        if step % 7 == 0 or step == steps:
            out = torch.full((wl.num_queries, wl.num_q_heads, wl.head_dim), float("nan"), dtype=torch.float32,
                             device="cuda")
            dec.decode(q, kc, vc, out)
            torch.cuda.synchronize()
            ref = oracle.decode_workload(cur)
            assert_close(out.cpu().numpy().astype(np.float64), ref, "%s update step %d" % (kind, step))
    assert set(paths) <= {1, 2} and 2 in paths, paths


@pytest.mark.parametrize("m", [3, 24])
def test_parity_multi_token_queries(m):
    """Queries of m new tokens, expanded to causal single-token rows by the
    library and decoded as one packed batch, against the oracle per row."""
    import dataclasses
    rng = np.random.default_rng(31 + m)
    segs = [[("sys", 48), (("sess", b), int(rng.integers(60, 400)))] for b in range(4)]
    base = W.from_segments("multi_tok_gpu_%d" % m, segs, 16, 4, 128, 31, 731).materialize()
    k = K()
    q_lens = np.full(base.num_queries, m, dtype=np.int32)
    # the causal rows, written here from their definition: new token i of query b
    # attends to the first T_b - m + i + 1 tokens through b's own block table
    ref_sl, ref_bt = [], []
    for b in range(base.num_queries):
        T = int(base.seq_lens[b])
        for i in range(m):
            n = T - m + i + 1
            row = np.full(base.max_blocks, -1, dtype=np.int32)
            row[:(n + 15) // 16] = base.block_tables[b, :(n + 15) // 16]
            ref_sl.append(n)
            ref_bt.append(row)
    ref_sl, ref_bt = np.array(ref_sl, dtype=np.int32), np.stack(ref_bt)
    # the library's expansion (what a caller hands to the planner) must be those rows
    bt, sl = k.kvattn_expand_query_tokens(base.shape_tuple(), base.block_tables, base.seq_lens, q_lens)
    assert np.array_equal(sl, ref_sl) and np.array_equal(bt, ref_bt)
    rows = len(ref_sl)
    q = W.normal_bf16(base.seed_values, W.TAG_Q, 0, rows * base.num_q_heads * base.head_dim).reshape(
        rows, base.num_q_heads, base.head_dim)
    lib_rows = dataclasses.replace(base, name="multi_tok_rows_%d" % m, seq_lens=sl, block_tables=bt, q=q)
    ref_rows = dataclasses.replace(base, name="multi_tok_ref_%d" % m, seq_lens=ref_sl, block_tables=ref_bt, q=q)
    print("case multi-token m=%d rows %d" % (m, rows), flush=True)
    got, dec = gpu_decode(lib_rows)
    st = dec.stats()
    # the rows of a query are packed onto MFMA, unless the batch is small enough for a one-launch plan
    assert st["num_items_mfma"] > 0 or st["one_launch"] or base.group * m <= 4
    assert_close(got, oracle.decode_workload(ref_rows), "multi-token m=%d" % m)


def valu_max_rows(D):
    """Rows per KV head the VALU forward holds (the planner's limit)."""
    return 4 if D == 128 else 8


def edge_workload(lengths, shared, Hq, Hkv, D, seed):
    segs = []
    for b, T in enumerate(lengths):
        s = []
        if shared and T >= shared:
            s.append(("shared", shared))
            if T > shared:
                s.append((("own", b), T - shared))
        else:
            s.append((("own", b), T))
        segs.append(s)
    name = "edge_s%d_sh%d_h%d_%d_d%d" % (seed, shared, Hq, Hkv, D)
    return W.from_segments(name, segs, Hq, Hkv, D, seed, 500 + seed, extra_blocks=2).materialize()


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("G,Hkv", [(1, 4), (4, 2), (8, 1)])
@pytest.mark.parametrize("variant", [-1, 0, 1, 2])
def test_parity_boundary_lengths(D, G, Hkv, variant):
    lengths = [1, 15, 16, 17, 32, 33, 31, 2, 47, 48, 49, 63, 64, 65, 129]
    wl = edge_workload(lengths, 0, G * Hkv, Hkv, D, 7 + D + G)
    if variant in (0, 2) and G > valu_max_rows(D):
        expect_unsupported(wl, force_variant=variant)
        return
    got, _ = gpu_decode(wl, force_variant=variant)
    ref = oracle_out(wl)
    assert_close(got, ref, "edge D%d G%d v%d" % (D, G, variant))
    # one-token KV returns V exactly up to fp32 rounding
    vf = W.bf16_bits_to_f32(wl.v_pool)
    for h in range(wl.num_q_heads):
        blk = wl.block_tables[0, 0]
        np.testing.assert_allclose(got[0, h], vf[blk, h // G, 0], rtol=0, atol=1e-6)


@pytest.mark.parametrize("Hq,Hkv,D", [(1, 1, 64), (3, 1, 64), (6, 2, 128), (16, 1, 128), (32, 32, 128),
                                       (64, 2, 128), (64, 1, 64), (128, 8, 128)])
@pytest.mark.parametrize("variant", [-1, 0, 1, 2])
def test_parity_head_shapes(Hq, Hkv, D, variant):
    """Head counts off the configs' 32/8 and 4/4: one head, odd groups, MHA with 32 KV heads,
    the widest GQA group (64 q heads per KV head) and 128 q heads, over a shared prefix
    with ragged suffixes."""
    G = Hq // Hkv
    lengths = [1, 17, 33, 40, 64, 90, 129]
    wl = edge_workload(lengths, 32, Hq, Hkv, D, 60 + Hq + Hkv + D)
    if variant in (0, 2) and G > valu_max_rows(D):
        expect_unsupported(wl, force_variant=variant)
        return
    got, dec = gpu_decode(wl, force_variant=variant)
    assert_close(got, oracle_out(wl), "heads %d/%d D%d v%d" % (Hq, Hkv, D, variant))


@pytest.mark.parametrize("variant", [-1, 0, 1, 2])
@pytest.mark.parametrize("shared", [16, 32, 48])
def test_parity_shared_prefix_ragged(variant, shared):
    lengths = [shared + x for x in (1, 15, 16, 17, 33, 100)] + [shared]
    wl = edge_workload(lengths, shared, 16, 4, 128, 40 + shared)
    for mode in (0, 2):
        for scheme in (1, 2):
            got, _ = gpu_decode(wl, force_variant=variant, pack_mode=mode, scheme=scheme)
            assert_close(got, oracle_out(wl), "shared %d v%d mode %d scheme %d" % (shared, variant, mode, scheme))


def test_parity_peaked_scores():
    wl = W.small(2).materialize()
    q = W.bf16_bits_to_f32(wl.q) * 8.0
    wl.q = W.f32_to_bf16_bits(q)
    wl.name = "c2_small_peaked"
    for variant in (0, 1, 2):
        got, _ = gpu_decode(wl, pack_mode=2, force_variant=variant)
        assert_close(got, oracle_out(wl), "peaked v%d" % variant)


def test_parity_explicit_scale():
    wl = small(2)
    got, _ = gpu_decode(wl, scale=0.05)
    assert_close(got, oracle_out(wl, scale=0.05), "scale 0.05")


def test_forward_then_merge_equals_decode():
    k = K()
    wl = small(3)
    dec = k.Decoder(wl.shape_tuple(), wl.block_tables, wl.seq_lens)
    q, kc, vc = device_inputs(wl)
    a = torch.zeros((wl.num_queries, wl.num_q_heads, wl.head_dim), dtype=torch.float32, device="cuda")
    b = torch.zeros_like(a)
    k.kvattn_decode(q, kc, vc, dec.plan, a)
    k.kvattn_forward(q, kc, vc, dec.plan, b)
    k.kvattn_merge(dec.plan, b)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
    # a plan serves repeated calls (e.g. every layer) with identical results
    c = torch.zeros_like(a)
    for _ in range(3):
        k.kvattn_decode(q, kc, vc, dec.plan, c)
    torch.cuda.synchronize()
    assert torch.equal(a, c)


@pytest.mark.parametrize("c", [2, 3, 4, 5])
def test_plain_partial_stores_match_write_through(c, monkeypatch):
    """Partials are stored written through the L2 when the partial arrays fit 32-bit offsets,
    with plain stores otherwise; KVATTN_PLAIN_PARTIALS=1 takes the plain path on a small batch:
    bit-identical outputs, within tolerance of the oracle."""
    k = K()
    wl = small(c)
    dec = k.Decoder(wl.shape_tuple(), wl.block_tables, wl.seq_lens)
    assert k.kvattn_plan_stats(dec.plan)["num_partial_slots"] > 0
    q, kc, vc = device_inputs(wl)
    a = torch.zeros((wl.num_queries, wl.num_q_heads, wl.head_dim), dtype=torch.float32, device="cuda")
    b = torch.zeros_like(a)
    k.kvattn_decode(q, kc, vc, dec.plan, a)
    torch.cuda.synchronize()
    monkeypatch.setenv("KVATTN_PLAIN_PARTIALS", "1")
    k.kvattn_decode(q, kc, vc, dec.plan, b)
    torch.cuda.synchronize()
    monkeypatch.delenv("KVATTN_PLAIN_PARTIALS")
    assert torch.equal(a, b)
    assert_close(b.cpu().numpy(), oracle_out(wl), "plain partial stores, config %d" % c)


@pytest.mark.parametrize("c", [1, 2, 3, 4, 5])
def test_parity_full_size(c):
    """Full-size configs in the launch configuration the bench times (default plan), every
    (query, head) row against the oracle (C4: about 20 s of oracle on 16 host threads)."""
    wl = W.WORKLOADS[c]().materialize()
    got, dec = gpu_decode(wl)
    print("  oracle over all %d rows" % (wl.num_queries * wl.num_q_heads), flush=True)
    ref = oracle.decode_workload(wl)
    assert_close(got, ref, "full config %d" % c)
    _dev_cache.clear()
    del wl


def test_graph_replay_matches_eager():
    """A captured decode replays correctly several times, with eager work and syncs in between."""
    k = K()
    wl = small(2)
    dec = k.Decoder(wl.shape_tuple(), wl.block_tables, wl.seq_lens)
    q, kc, vc = device_inputs(wl)
    shape = (wl.num_queries, wl.num_q_heads, wl.head_dim)
    eager = torch.zeros(shape, dtype=torch.float32, device="cuda")
    k.kvattn_decode(q, kc, vc, dec.plan, eager)
    torch.cuda.synchronize()
    out = torch.zeros(shape, dtype=torch.float32, device="cuda")
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        k.kvattn_decode(q, kc, vc, dec.plan, out)
    for rep in range(4):
        out.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), "replay %d differs" % rep
        other = torch.zeros_like(eager)
        k.kvattn_decode(q, kc, vc, dec.plan, other)   # eager work between replays
        torch.cuda.synchronize()
        assert torch.equal(other, eager)


def test_read_probe_reads_every_word():
    """The measurement helper reads every 32-bit word of both buffers once: the XOR of its sink
    equals the XOR of all words (sizes not multiples of the grid's shares)."""
    k = K()
    rng = np.random.default_rng(5)
    a = rng.integers(0, 2 ** 31, size=(1000 * 4 + 4,), dtype=np.int64).astype(np.int32)
    b = rng.integers(0, 2 ** 31, size=(777 * 4,), dtype=np.int64).astype(np.int32)
    grid = 7
    want = np.bitwise_xor.reduce(np.concatenate([a, b]).view(np.uint32))
    for depth in (2, 4, 8):
        for threads in (256, 512, 1024):
            sink = torch.zeros(grid * threads, dtype=torch.int32, device="cuda")
            k.kvattn_read_probe(torch.from_numpy(a).cuda(), torch.from_numpy(b).cuda(), sink, grid, None, depth,
                                threads)
            torch.cuda.synchronize()
            assert np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32)) == want, (depth, threads)
    with pytest.raises(k.KvattnError):
        k.kvattn_read_probe(torch.from_numpy(a).cuda(), torch.from_numpy(b).cuda(), sink[:10], grid)
    with pytest.raises(k.KvattnError):
        k.kvattn_read_probe(torch.from_numpy(a).cuda(), torch.from_numpy(b).cuda(), sink, grid, None, 16, 256)


def test_two_plans_in_flight_on_two_streams():
    """Two plans, each with its own workspace, decode at the same time on two non-default streams
    (default priority); both match the oracle, twice in a row."""
    k = K()
    a, b = small(2), small(5)
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    da = k.Decoder(a.shape_tuple(), a.block_tables, a.seq_lens, options=k.make_options(num_cus=1024))
    db = k.Decoder(b.shape_tuple(), b.block_tables, b.seq_lens)
    qa, ka, va = [torch.from_numpy(x.view(np.int16)).cuda() for x in (a.q, a.k_pool, a.v_pool)]
    qb, kb, vb = [torch.from_numpy(x.view(np.int16)).cuda() for x in (b.q, b.k_pool, b.v_pool)]
    torch.cuda.synchronize()
    for rep in range(2):
        oa = torch.full((a.num_queries, a.num_q_heads, a.head_dim), float("nan"), device="cuda")
        ob = torch.full((b.num_queries, b.num_q_heads, b.head_dim), float("nan"), device="cuda")
        torch.cuda.synchronize()
        da.decode(qa, ka, va, oa, stream=s1.cuda_stream)
        db.decode(qb, kb, vb, ob, stream=s2.cuda_stream)
        torch.cuda.synchronize()
        assert_close(oa.cpu().numpy().astype(np.float64), oracle_out(a), "stream 1 rep %d" % rep)
        assert_close(ob.cpu().numpy().astype(np.float64), oracle_out(b), "stream 2 rep %d" % rep)


@pytest.mark.parametrize("c", [1, 2, 3, 4, 5])
def test_parity_multi_stream_forward(c):
    """Multi-stream plans: MFMA launches on a side stream beside the VALU launches (kvattn_decode_streams),
    and the same plan through kvattn_decode (launches in turn), against the oracle."""
    k = K()
    wl = small(c)
    print("case multi-stream %s" % wl.name, flush=True)
    dec = k.Decoder(wl.shape_tuple(), wl.block_tables, wl.seq_lens, options=k.make_options(multi_stream=1))
    q, kc, vc = device_inputs(wl)
    main, side = torch.cuda.Stream(), torch.cuda.Stream()
    torch.cuda.synchronize()
    for rep in range(2):
        out = torch.full((wl.num_queries, wl.num_q_heads, wl.head_dim), float("nan"), device="cuda")
        torch.cuda.synchronize()
        with torch.cuda.stream(main):
            dec.decode_streams(q, kc, vc, out, side_stream=side)
        torch.cuda.synchronize()
        assert_close(out.cpu().numpy().astype(np.float64), oracle_out(wl), "multi-stream %s rep %d" % (wl.name, rep))
    out = torch.full((wl.num_queries, wl.num_q_heads, wl.head_dim), float("nan"), device="cuda")
    dec.decode(q, kc, vc, out)
    torch.cuda.synchronize()
    assert_close(out.cpu().numpy().astype(np.float64), oracle_out(wl), "multi-stream plan, one stream")
    with pytest.raises(k.KvattnError):
        dec.decode_streams(q, kc, vc, out, side_stream=torch.cuda.current_stream())
    plain = k.Decoder(wl.shape_tuple(), wl.block_tables, wl.seq_lens)
    with pytest.raises(k.KvattnError):
        plain.decode_streams(q, kc, vc, out, side_stream=side)
    torch.cuda.synchronize()


def test_multi_stream_graph_replay_matches_eager():
    """The fork and join of kvattn_decode_streams under stream capture: replays match the eager result."""
    k = K()
    wl = small(3)
    dec = k.Decoder(wl.shape_tuple(), wl.block_tables, wl.seq_lens, options=k.make_options(multi_stream=1))
    q, kc, vc = device_inputs(wl)
    shape = (wl.num_queries, wl.num_q_heads, wl.head_dim)
    side = torch.cuda.Stream()
    eager = torch.zeros(shape, dtype=torch.float32, device="cuda")
    dec.decode_streams(q, kc, vc, eager, side_stream=side)
    torch.cuda.synchronize()
    out = torch.zeros(shape, dtype=torch.float32, device="cuda")
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        k.kvattn_decode_streams(q, kc, vc, dec.plan, out, side)
    for rep in range(4):
        out.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), "replay %d" % rep
    assert_close(eager.cpu().numpy().astype(np.float64), oracle_out(wl), "multi-stream eager")


@pytest.mark.parametrize("seed", range(12))
def test_parity_random_trees(seed):
    """Random prefix forests (1-3 roots, optional children and private leaves, random head
    shapes and head_dim) under auto, forced-variant and full-pack plans, plus the
    multi-stream forward, against the oracle."""
    from test_plan import random_tree_workload
    wl = random_tree_workload(1000 + seed).materialize()
    ref = oracle_out(wl)
    k = K()
    cases = [{}, {"pack_mode": 2}, {"force_variant": 1, "split_tokens": 32}, {"multi_stream": 1}]
    if wl.group <= valu_max_rows(wl.head_dim):
        cases.append({"force_variant": 0, "pack_mode": 2, "scheme": 2})
        cases.append({"force_variant": 2, "pack_mode": 2, "scheme": 2})
        cases.append({"force_variant": 2, "pack_mode": 1, "split_tokens": 80})
    for opts in cases:
        if opts.get("multi_stream"):
            print("case %s opts %s" % (wl.name, opts), flush=True)
            dec = k.Decoder(wl.shape_tuple(), wl.block_tables, wl.seq_lens, options=k.make_options(**opts))
            q, kc, vc = device_inputs(wl)
            out = torch.full((wl.num_queries, wl.num_q_heads, wl.head_dim), float("nan"), device="cuda")
            side = torch.cuda.Stream()
            dec.decode_streams(q, kc, vc, out, side_stream=side)
            torch.cuda.synchronize()
            got = out.cpu().numpy().astype(np.float64)
        else:
            got, _ = gpu_decode(wl, **opts)
        assert_close(got, ref, "%s %s" % (wl.name, opts))


def test_parity_full_size_after_plan_update():
    """The Llama-3-8B layer workload at full size: a plan made one decode step earlier
    (every query one token shorter) and brought forward by kvattn_plan_update decodes
    like the oracle on every row."""
    k = K()
    wl = W.WORKLOADS[2]().materialize()
    prev = _cut_state(wl, np.ones(wl.num_queries, dtype=np.int32))
    print("case full-size update", flush=True)
    dec = k.Decoder(wl.shape_tuple(), prev.block_tables, prev.seq_lens)
    dec.update(wl.block_tables, wl.seq_lens)
    assert dec.stats()["update_path"] in (1, 2)
    q, kc, vc = device_inputs(wl)
    out = torch.full((wl.num_queries, wl.num_q_heads, wl.head_dim), float("nan"), device="cuda")
    dec.decode(q, kc, vc, out)
    torch.cuda.synchronize()
    assert_close(out.cpu().numpy().astype(np.float64), oracle.decode_workload(wl), "full size after update")
    _dev_cache.clear()


@pytest.mark.parametrize("seed", range(4))
def test_parity_random_forest_updates(seed):
    """Random forests brought forward by kvattn_plan_update with uneven steps; the decode
    after every fourth update matches the oracle at the current lengths."""
    from test_plan_update import random_forest
    k = K()
    wl = random_forest(700 + seed).materialize()
    rng = np.random.default_rng(seed)
    cut = rng.integers(8, 28, wl.num_queries).astype(np.int32)
    cur = _cut_state(wl, cut)
    print("case random-forest updates %s" % wl.name, flush=True)
    dec = k.Decoder(wl.shape_tuple(), cur.block_tables, cur.seq_lens)
    q, kc, vc = device_inputs(wl)
    n = 0
    while cut.any():
        cut -= np.minimum(cut, rng.integers(0, 4, wl.num_queries)).astype(np.int32)
        cur = _cut_state(wl, cut)
        dec.update(cur.block_tables, cur.seq_lens)
        n += 1
        if n % 4 == 0 or not cut.any():
            out = torch.full((wl.num_queries, wl.num_q_heads, wl.head_dim), float("nan"), device="cuda")
            dec.decode(q, kc, vc, out)
            torch.cuda.synchronize()
            assert_close(out.cpu().numpy().astype(np.float64), oracle.decode_workload(cur),
                         "%s after %d updates" % (wl.name, n))


def test_back_to_back_updates_without_host_sync():
    """update -> upload -> decode steps queued with no host synchronisation, behind
    several long decodes on the same stream: each step's output matches the oracle at
    that step's lengths.  kvattn_plan_update waits for the previous upload's copy,
    which still reads the plan's host blob while it is queued."""
    k = K()
    rng = np.random.default_rng(23)
    segs = [[("root", 96), (("own", b), int(rng.integers(90, 160)))] for b in range(10)]
    wl = W.from_segments("b2b_updates", segs, 8, 2, 128, 23, 723).materialize()
    # about 10 ms of queued work ahead of the first upload
    long_wl = W.from_segments("b2b_long", [[(("own", b), 8192)] for b in range(32)], 32, 8, 128, 24,
                              724).materialize()
    long_dec = k.Decoder(long_wl.shape_tuple(), long_wl.block_tables, long_wl.seq_lens)
    lq, lk, lv = [torch.from_numpy(x.view(np.int16)).cuda() for x in (long_wl.q, long_wl.k_pool, long_wl.v_pool)]
    lout = torch.empty((long_wl.num_queries, long_wl.num_q_heads, long_wl.head_dim), device="cuda")
    steps = 12
    cut = np.full(wl.num_queries, steps, dtype=np.int32)
    states = [_cut_state(wl, cut)]
    dec = k.Decoder(wl.shape_tuple(), states[0].block_tables, states[0].seq_lens)
    q, kc, vc = device_inputs(wl)
    outs = [torch.full((wl.num_queries, wl.num_q_heads, wl.head_dim), float("nan"), device="cuda")
            for _ in range(steps + 1)]
    torch.cuda.synchronize()
    print("case back-to-back updates", flush=True)
    for _ in range(8):
        long_dec.decode(lq, lk, lv, lout)
    dec.decode(q, kc, vc, outs[0])
    for step in range(1, steps + 1):
        cut -= 1
        states.append(_cut_state(wl, cut))
        dec.update(states[-1].block_tables, states[-1].seq_lens)
        dec.decode(q, kc, vc, outs[step])
    torch.cuda.synchronize()
    for step, st in enumerate(states):
        assert_close(outs[step].cpu().numpy().astype(np.float64), oracle.decode_workload(st),
                     "back-to-back step %d" % step)


def test_upload_refused_under_capture():
    """An upload captured into a graph would re-read the host blob at every replay."""
    k = K()
    wl = small(1)
    dec = k.Decoder(wl.shape_tuple(), wl.block_tables, wl.seq_lens)
    s = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with pytest.raises(k.KvattnError) as ei:
        with torch.cuda.graph(g, stream=s):
            k.kvattn_plan_upload(dec.plan, dec.workspace, dec.workspace.numel(), s)
    assert ei.value.status == k.KVATTN_EINVAL
    torch.cuda.synchronize()


@pytest.mark.parametrize("case", ["c2", "c3", "c5", "forest"])
def test_fused_merge_matches_merge_launch_across_calls(case):
    """Plans that merge inside the forward launch (fused_merge=1) against the same plans with a
    merge launch (fused_merge=0): bit-identical outputs, within the oracle's tolerance, over calls
    that alternate two different query batches and two KV pools on one plan -- a partial read
    stale from another XCD's cache or from the previous call would show."""
    from test_plan import random_tree_workload
    k = K()
    wl = random_tree_workload(1201).materialize() if case == "forest" else small(int(case[1]))
    # full packing: partials to merge even where AUTO would plan a small batch as one launch
    fused = k.Decoder(wl.shape_tuple(), wl.block_tables, wl.seq_lens, options=k.make_options(fused_merge=1, pack_mode=2))
    sep = k.Decoder(wl.shape_tuple(), wl.block_tables, wl.seq_lens, options=k.make_options(fused_merge=0, pack_mode=2))
    assert fused.stats()["num_launches"] == sep.stats()["num_launches"] - 1
    q, kc, vc = device_inputs(wl)
    q2 = torch.from_numpy(W.normal_bf16(wl.seed_values + 7, W.TAG_Q, 0, q.numel()).view(np.int16)).cuda().view(
        q.shape)
    vc2 = vc.clone()
    vc2.view(torch.bfloat16).mul_(-0.5)   # another V pool (NaN slots stay NaN)
    import dataclasses
    wl2 = dataclasses.replace(wl, q=q2.cpu().numpy().view(np.uint16),
                              v_pool=vc2.cpu().numpy().view(np.uint16))
    refs = {0: oracle.decode_workload(wl), 1: oracle.decode_workload(wl2)}
    inputs = {0: (q, kc, vc), 1: (q2, kc, vc2)}
    shape = (wl.num_queries, wl.num_q_heads, wl.head_dim)
    print("case fused merge %s" % wl.name, flush=True)
    for call, which in enumerate([0, 1, 0, 0, 1, 1, 0, 1]):
        a = torch.full(shape, float("nan"), device="cuda")
        b = torch.full(shape, float("nan"), device="cuda")
        fused.decode(*inputs[which], a)
        sep.decode(*inputs[which], b)
        torch.cuda.synchronize()
        assert torch.equal(a, b), "call %d: fused and separate merges differ (max %.3e)" % (
            call, float((a - b).abs().nan_to_num(1e9).max()))
        assert_close(a.cpu().numpy().astype(np.float64), refs[which], "fused %s call %d" % (wl.name, call))



def test_parity_one_launch_small_batches():
    """Small batches planned as one launch without partials (VALU_SPLIT tile for ranges of 4+ blocks,
    VALU below): one launch, no merge rows, outputs within tolerance, at both head sizes."""
    k = K()
    for D, Hq, Hkv in ((64, 4, 4), (128, 16, 4), (128, 8, 8)):
        rng = np.random.default_rng(D + Hq)
        lengths = [int(x) for x in rng.integers(1, 700, size=5)] + [1, 63, 64]
        wl = edge_workload(lengths, 0, Hq, Hkv, D, 300 + D + Hq)
        got, dec = gpu_decode(wl)
        st = dec.stats()
        assert st["one_launch"] == 1 and st["num_launches"] == 1 and st["num_merge_rows"] == 0, st
        assert st["num_items_valu_split"] >= 1
        assert_close(got, oracle_out(wl), "one-launch D%d %d/%d" % (D, Hq, Hkv))
