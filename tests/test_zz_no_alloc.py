"""kvattn_decode_noalloc, the entry point for callers that cannot allocate, against kvattn_decode.

Same plans, same kernels: the outputs must be identical (and within the 2e-3
bar of the oracle, which the other parity tests already hold kvattn_decode
to).  Two calls in a row, the second with a smaller input, then the first
plan again (its schedule copied back into the device's scratch), a repeated
call with no copy, a plan update, and the refusals.
"""
import numpy as np
import pytest

import oracle
import workloads as W

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

TOL = 2e-3


@pytest.fixture(scope="module", autouse=True)
def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _dev(wl):
    return [torch.from_numpy(x.view(np.int16)).cuda() for x in (wl.q, wl.k_pool, wl.v_pool)]


def _out(wl):
    return torch.full((wl.num_queries, wl.num_q_heads, wl.head_dim), float("nan"), dtype=torch.float32, device="cuda")


def _check(K, wl, plan_dec, tensors, what):
    q, kc, vc = tensors
    ref = _out(wl)
    got = _out(wl)
    K.kvattn_decode(q, kc, vc, plan_dec.plan, ref)
    K.kvattn_decode_noalloc(q, kc, vc, plan_dec.plan, got)
    torch.cuda.synchronize()
    assert torch.equal(got, ref), "%s: noalloc differs from kvattn_decode (max %.3e)" % (
        what, float((got - ref).abs().max()))
    err = float(np.abs(got.cpu().numpy().astype(np.float64) - oracle.decode_workload(wl)).max())
    assert err <= TOL, "%s: max abs err %.3e vs the oracle" % (what, err)


def test_noalloc_matches_decode_on_two_calls_the_second_smaller():
    from decode_attention_prefix_amd import kvattn as K
    big = W.small(3).materialize()
    smaller = W.small(1).materialize()
    assert smaller.num_queries * smaller.num_q_heads < big.num_queries * big.num_q_heads
    da = K.Decoder(big.shape_tuple(), big.block_tables, big.seq_lens)
    db = K.Decoder(smaller.shape_tuple(), smaller.block_tables, smaller.seq_lens)
    ta, tb = _dev(big), _dev(smaller)
    print("case noalloc %s then %s" % (big.name, smaller.name), flush=True)
    _check(K, big, da, ta, "first call (%s)" % big.name)
    _check(K, smaller, db, tb, "second call, smaller (%s)" % smaller.name)
    # the first plan again: its schedule is copied back into the scratch
    _check(K, big, da, ta, "first plan again")
    # repeated calls with one plan copy nothing and give the same result
    out1, out2 = _out(big), _out(big)
    K.kvattn_decode_noalloc(*ta, da.plan, out1)
    K.kvattn_decode_noalloc(*ta, da.plan, out2)
    torch.cuda.synchronize()
    assert torch.equal(out1, out2)


def test_noalloc_after_plan_update():
    """A plan brought forward by kvattn_plan_update is staged again (its state changed)."""
    import dataclasses
    from decode_attention_prefix_amd import kvattn as K
    wl = W.small(2).materialize()
    lens = (wl.seq_lens - 1).astype(np.int32)
    bt = wl.block_tables.copy()
    for b, T in enumerate(lens):
        bt[b, (int(T) + 15) // 16:] = -1
    prev = dataclasses.replace(wl, seq_lens=lens, block_tables=bt)
    dec = K.Decoder(wl.shape_tuple(), prev.block_tables, prev.seq_lens)
    t = _dev(wl)
    print("case noalloc update", flush=True)
    _check(K, prev, dec, t, "before update")
    dec.update(wl.block_tables, wl.seq_lens)
    _check(K, wl, dec, t, "after update")


def test_noalloc_refusals():
    from decode_attention_prefix_amd import kvattn as K
    wl = W.small(1).materialize()
    q, kc, vc = _dev(wl)
    out = _out(wl)
    fresh = K.kvattn_plan(wl.shape_tuple(), wl.block_tables, wl.seq_lens, None,
                          K.make_options(new_token=1))
    with pytest.raises(K.KvattnError) as ei:
        K.kvattn_decode_noalloc(q, kc, vc, fresh, out)
    assert ei.value.status == K.KVATTN_EINVAL
    # a plan whose workspace exceeds the 64 MiB scratch: 4096 queries x 64 heads, each split in two
    segs = [[("root", 64), (("own", b), 32)] for b in range(4096)]
    huge = W.from_segments("noalloc_huge", segs, 64, 1, 128, 5, 905)
    plan = K.kvattn_plan(huge.shape_tuple(), huge.block_tables, huge.seq_lens, None,
                         K.make_options(pack_mode=2, scheme=1))
    assert K.kvattn_plan_device_bytes(plan) > 64 << 20
    with pytest.raises(K.KvattnError) as ei:
        K.kvattn_decode_noalloc(q, kc, vc, plan, out)
    assert ei.value.status == K.KVATTN_EWORKSPACE
    torch.cuda.synchronize()
