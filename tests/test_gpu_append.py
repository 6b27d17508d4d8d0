"""GPU parity of the fused KV append (kvattn_decode_append) against the oracle.

Each case appends every query's new token with oracle.append_tokens on the
host and attends with the oracle over the appended cache; the GPU call must
match the output within 2e-3 and leave both caches bit-identical to the
oracle's.  Before the call the new tokens' slots hold NaN, so a kernel that
reads a slot before writing it, or fails to write it, fails the check.
"""
import numpy as np
import pytest

import oracle
import workloads as W
from test_gpu_parity import K, assert_close, small, valu_max_rows, _cut_state, expect_unsupported

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

NAN_BF16 = 0x7FC0


@pytest.fixture(scope="module", autouse=True)
def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def new_tokens(B, Hq, Hkv, D, seed):
    rng = np.random.default_rng(seed)
    q = W.f32_to_bf16_bits(rng.standard_normal((B, Hq, D)).astype(np.float32))
    kn = W.f32_to_bf16_bits(rng.standard_normal((B, Hkv, D)).astype(np.float32))
    vn = W.f32_to_bf16_bits(rng.standard_normal((B, Hkv, D)).astype(np.float32))
    return q, kn, vn


def blank_new_slots(kp, vp, bt, lens):
    kp, vp = kp.copy(), vp.copy()
    for b, T in enumerate(lens):
        pos = int(T) - 1
        kp[int(bt[b, pos // 16]), :, pos % 16, :] = NAN_BF16
        vp[int(bt[b, pos // 16]), :, pos % 16, :] = NAN_BF16
    return kp, vp


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda()


def host(t):
    return t.cpu().numpy().view(np.uint16)


def run_append(wl, seed, rows=None, **opts):
    """One fused append + decode on the GPU; returns (out rows, oracle rows, caches match)."""
    k = K()
    B, Hq, Hkv, D = wl.num_queries, wl.num_q_heads, wl.num_kv_heads, wl.head_dim
    q, kn, vn = new_tokens(B, Hq, Hkv, D, seed)
    kp, vp = blank_new_slots(wl.k_pool, wl.v_pool, wl.block_tables, wl.seq_lens)
    ref_k, ref_v = oracle.append_tokens(kp, vp, wl.block_tables, wl.seq_lens, kn, vn)
    print("case append %s opts %s" % (wl.name, opts), flush=True)
    dec = k.Decoder(wl.shape_tuple(), wl.block_tables, wl.seq_lens, options=k.make_options(new_token=1, **opts))
    kc, vc = dev(kp), dev(vp)
    out = torch.full((B, Hq, D), float("nan"), dtype=torch.float32, device="cuda")
    dec.decode_append(dev(q), dev(kn), dev(vn), kc, vc, out)
    torch.cuda.synchronize()
    got = out.cpu().numpy().astype(np.float64)
    if rows is None:
        ref = oracle.decode_all(q, ref_k, ref_v, wl.block_tables, wl.seq_lens, Hq, Hkv)
    else:
        ref = oracle.decode_rows(q, ref_k, ref_v, wl.block_tables, wl.seq_lens, Hq, Hkv, rows)
        got = got.reshape(-1, D)[rows]
    assert np.array_equal(host(kc), ref_k), "%s: k_cache differs from the oracle's append" % wl.name
    assert np.array_equal(host(vc), ref_v), "%s: v_cache differs from the oracle's append" % wl.name
    return got, ref, dec


@pytest.mark.parametrize("c", [1, 2, 3, 5])
@pytest.mark.parametrize("opts", [{}, {"pack_mode": 1}, {"pack_mode": 2, "force_variant": 0},
                                  {"pack_mode": 2, "force_variant": 1, "split_tokens": 48},
                                  {"pack_mode": 2, "force_variant": 2}])
def test_append_parity_small_configs(c, opts):
    wl = small(c)
    if opts.get("force_variant") in (0, 2) and wl.group > valu_max_rows(wl.head_dim):
        expect_unsupported(wl, new_token=1, **opts)
        return
    got, ref, _ = run_append(wl, 40 + c, **opts)
    assert_close(got, ref, "append %s %s" % (wl.name, opts))


def test_append_one_launch_forward_tiny_batch():
    """The tiny batch's new-token plan reads every query's cached range whole (no packs, no
    cuts: the one-launch forward), then the merge adds the new tokens: parity and bit-exact
    caches at full size."""
    wl = W.config1().materialize()
    got, ref, dec = run_append(wl, 77)
    st = dec.stats()
    assert st["one_launch"] == 1 and st["num_packed_nodes"] == 0 and st["num_launches"] == 2
    assert st["num_merge_rows"] == wl.num_queries * wl.num_q_heads
    assert_close(got, ref, "append one-launch tiny batch")


@pytest.mark.parametrize("D", [64, 128])
def test_append_edge_lengths(D):
    """seq_len 1 (the new token alone), new tokens opening a block, and ragged tails, in one batch."""
    tails = [1, 2, 15, 16, 17, 31, 33]
    segs = [[(("solo", b), 1)] for b in range(3)] + [[("root", 64), (("own", b), t)] for b, t in enumerate(tails)]
    wl = W.from_segments("append_edges_d%d" % D, segs, 8, 2, D, 50 + D, 950 + D).materialize()
    got, ref, dec = run_append(wl, 60 + D)
    assert_close(got, ref, "append edges D=%d" % D)
    # the new token alone: out = v_new of the row's KV head
    _, kn, vn = new_tokens(wl.num_queries, 8, 2, D, 60 + D)
    for b in range(3):
        for h in range(8):
            assert np.array_equal(got[b, h].astype(np.float32), W.bf16_bits_to_f32(vn[b, h // 4]))


def test_append_every_query_alone():
    segs = [[(("solo", b), 1)] for b in range(6)]
    wl = W.from_segments("append_all_solo", segs, 4, 4, 128, 52, 952).materialize()
    got, ref, dec = run_append(wl, 62)
    assert dec.stats()["num_items"] == 0
    assert_close(got, ref, "append all solo")


def test_append_full_size_llama3_8b_layer():
    """The Llama-3-8B layer workload (64 queries, shared prefix, private tails) at full size,
    every (query, head) row against the oracle over the oracle-appended caches."""
    wl = W.WORKLOADS[2]().materialize()
    got, ref, _ = run_append(wl, 72)
    assert_close(got, ref, "append full config 2")


def test_entry_points_reject_the_other_kind_of_plan():
    k = K()
    wl = small(1)
    B, Hq, Hkv, D = wl.num_queries, wl.num_q_heads, wl.num_kv_heads, wl.head_dim
    q, kn, vn = new_tokens(B, Hq, Hkv, D, 3)
    kc, vc = dev(wl.k_pool), dev(wl.v_pool)
    out = torch.zeros((B, Hq, D), dtype=torch.float32, device="cuda")
    plain = k.Decoder(wl.shape_tuple(), wl.block_tables, wl.seq_lens)
    fused = k.Decoder(wl.shape_tuple(), wl.block_tables, wl.seq_lens, options=k.make_options(new_token=1))
    with pytest.raises(k.KvattnError) as e:
        plain.decode_append(dev(q), dev(kn), dev(vn), kc, vc, out)
    assert e.value.status == k.KVATTN_EINVAL
    with pytest.raises(k.KvattnError) as e:
        fused.decode(dev(q), kc, vc, out)
    assert e.value.status == k.KVATTN_EINVAL
    with pytest.raises(k.KvattnError) as e:
        k.kvattn_merge(fused.plan, out)
    assert e.value.status == k.KVATTN_EINVAL
    torch.cuda.synchronize()


def test_decode_loop_append_update_attend():
    """A decoding loop: every step appends one token per query through the fused
    call, with the plan brought forward by kvattn_plan_update; the device cache
    persists across steps and is compared with the oracle's at the end."""
    k = K()
    rng = np.random.default_rng(81)
    segs = [[("root", 80), (("own", b), int(rng.integers(60, 120)))] for b in range(10)]
    wl = W.from_segments("append_loop", segs, 8, 2, 128, 81, 981).materialize()
    steps = 40
    cut = np.full(wl.num_queries, steps, dtype=np.int32)
    kp, vp = wl.k_pool.copy(), wl.v_pool.copy()
    kc, vc = dev(kp), dev(vp)
    dec = None
    paths = []
    print("case append decode loop", flush=True)
    for step in range(steps):
        cut -= 1
        cur = _cut_state(wl, cut)
        q, kn, vn = new_tokens(wl.num_queries, 8, 2, 128, 1000 + step)
        if dec is None:
            dec = k.Decoder(wl.shape_tuple(), cur.block_tables, cur.seq_lens, options=k.make_options(new_token=1))
        else:
            dec.update(cur.block_tables, cur.seq_lens)
            paths.append(dec.stats()["update_path"])
        out = torch.full((wl.num_queries, 8, 128), float("nan"), dtype=torch.float32, device="cuda")
        dec.decode_append(dev(q), dev(kn), dev(vn), kc, vc, out)
        kp, vp = oracle.append_tokens(kp, vp, cur.block_tables, cur.seq_lens, kn, vn)
        if step % 5 == 0 or step == steps - 1:
            torch.cuda.synchronize()
            ref = oracle.decode_all(q, kp, vp, cur.block_tables, cur.seq_lens, 8, 2)
            assert_close(out.cpu().numpy().astype(np.float64), ref, "append loop step %d" % step)
    torch.cuda.synchronize()
    assert np.array_equal(host(kc), kp) and np.array_equal(host(vc), vp)
    assert set(paths) <= {1, 2}, paths


def test_append_graph_replay_matches_eager():
    """The fused call captured in a HIP graph: replays rewrite the same slots and give the eager output."""
    k = K()
    wl = small(2)
    B, Hq, Hkv, D = wl.num_queries, wl.num_q_heads, wl.num_kv_heads, wl.head_dim
    q, kn, vn = new_tokens(B, Hq, Hkv, D, 91)
    dec = k.Decoder(wl.shape_tuple(), wl.block_tables, wl.seq_lens, options=k.make_options(new_token=1))
    kp, vp = blank_new_slots(wl.k_pool, wl.v_pool, wl.block_tables, wl.seq_lens)
    qd, knd, vnd, kc, vc = dev(q), dev(kn), dev(vn), dev(kp), dev(vp)
    eager = torch.zeros((B, Hq, D), dtype=torch.float32, device="cuda")
    dec.decode_append(qd, knd, vnd, kc, vc, eager)
    torch.cuda.synchronize()
    kc.copy_(dev(kp))
    vc.copy_(dev(vp))
    out = torch.zeros((B, Hq, D), dtype=torch.float32, device="cuda")
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        k.kvattn_decode_append(qd, knd, vnd, kc, vc, dec.plan, out)
    ref_k, ref_v = oracle.append_tokens(kp, vp, wl.block_tables, wl.seq_lens, kn, vn)
    for rep in range(3):
        out.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), "replay %d" % rep
        assert np.array_equal(host(kc), ref_k) and np.array_equal(host(vc), ref_v)


def random_forest_private_leaves(seed):
    """Random prefix forests (1-3 roots, optional children, random head shapes) where every
    query ends in a private leaf of 1-90 tokens, so its new token's block is its own."""
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
        s.append((("leaf", b), int(rng.integers(1, 90))))
        segs.append(s)
    return W.from_segments("forest%d" % seed, segs, G * Hkv, Hkv, D, seed, seed + 1, extra_blocks=3)


@pytest.mark.parametrize("seed", range(12))
def test_append_random_forests(seed):
    """The fused append on random prefix forests with private leaves, against the oracle."""
    wl = random_forest_private_leaves(2000 + seed).materialize()
    got, ref, _ = run_append(wl, 3000 + seed)
    assert_close(got, ref, "append %s" % wl.name)

