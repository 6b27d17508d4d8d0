"""Pins of the fp64 oracle against things other than itself.

Each check is chosen so that a plausible slip in the oracle -- a wrong scale,
a wrong GQA head map, a wrong block-table index, a dropped token, a wrong sign
in the softmax, a transposed operand -- fails at least one of them:

  * brute force at 50 significant digits (mpmath) on tiny paged inputs;
  * torch's scaled_dot_product_attention in float64 on the CPU, a library
    routine the plain definition reduces to for dense K/V;
  * closed forms: one token returns V_0; identical keys or q = 0 return
    mean(V); constant V rows return that constant; a hand-derived two-token
    case (tests/golden/logistic_two_token.json);
  * invariants: token order, a common score shift, linearity in V, GQA equal
    to MHA with repeated KV, outputs inside the convex hull of the V rows;
  * the merge rule: merging the partial triples of two halves equals the
    attention over the whole sequence;
  * the row-subset path (decode_rows with an arbitrary list of b * Hq + h
    rows: permuted, repeated, single, last) against torch float64 SDPA of
    each listed row, and bit for bit against the same rows of decode_all.
"""
import json
import os

import numpy as np
import pytest

import oracle
from workloads import bf16_bits_to_f32, f32_to_bf16_bits

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def bf16(x):
    return f32_to_bf16_bits(np.asarray(x, dtype=np.float32))


def paged(dense_k, dense_v, bs, rng, extra=3):
    """Pack per-query dense K/V (lists of [T_b][Hkv][D] bf16 bits) into shuffled paged pools."""
    Hkv, D = dense_k[0].shape[1], dense_k[0].shape[2]
    nblk = [(k.shape[0] + bs - 1) // bs for k in dense_k]
    total = sum(nblk) + extra
    perm = rng.permutation(total)
    kp = np.full((total, Hkv, bs, D), 0x7FC0, dtype=np.uint16)
    vp = np.full((total, Hkv, bs, D), 0x7FC0, dtype=np.uint16)
    bt = np.full((len(dense_k), max(nblk)), -1, dtype=np.int32)
    nxt = 0
    for b, (k, v) in enumerate(zip(dense_k, dense_v)):
        for j in range(nblk[b]):
            pid = perm[nxt]
            nxt += 1
            bt[b, j] = pid
            seg = slice(j * bs, min((j + 1) * bs, k.shape[0]))
            n = seg.stop - seg.start
            kp[pid, :, :n, :] = np.transpose(k[seg], (1, 0, 2))
            vp[pid, :, :n, :] = np.transpose(v[seg], (1, 0, 2))
    sl = np.array([k.shape[0] for k in dense_k], dtype=np.int32)
    return kp, vp, bt, sl


def rand_case(rng, B, Hq, Hkv, D, Tmax, bs):
    T = rng.integers(1, Tmax + 1, size=B)
    q = bf16(rng.standard_normal((B, Hq, D)))
    dk = [bf16(rng.standard_normal((t, Hkv, D))) for t in T]
    dv = [bf16(rng.standard_normal((t, Hkv, D))) for t in T]
    kp, vp, bt, sl = paged(dk, dv, bs, rng)
    return q, dk, dv, kp, vp, bt, sl


def run_oracle(q, kp, vp, bt, sl, Hq, Hkv, bs, scale=0.0):
    return oracle.decode_all(q, kp, vp, bt, sl, Hq, Hkv, scale=scale, block_size=bs)


@pytest.mark.parametrize("seed,B,Hq,Hkv,D,Tmax,bs", [
    (0, 3, 2, 2, 8, 8, 4),
    (1, 2, 4, 2, 4, 8, 4),
    (2, 3, 2, 1, 8, 7, 2),
    (3, 1, 1, 1, 2, 5, 16),
])
def test_brute_force_mpmath(seed, B, Hq, Hkv, D, Tmax, bs):
    mp = pytest.importorskip("mpmath")
    mp.mp.dps = 50
    rng = np.random.default_rng(seed)
    q, dk, dv, kp, vp, bt, sl = rand_case(rng, B, Hq, Hkv, D, Tmax, bs)
    got = run_oracle(q, kp, vp, bt, sl, Hq, Hkv, bs)
    G = Hq // Hkv
    qf, scale = bf16_bits_to_f32(q), mp.mpf(1) / mp.sqrt(D)
    for b in range(B):
        kf, vf = bf16_bits_to_f32(dk[b]), bf16_bits_to_f32(dv[b])
        for h in range(Hq):
            g = h // G
            # direct softmax, no max subtraction, 50 digits
            w = [mp.e ** (scale * mp.fsum(mp.mpf(float(qf[b, h, i])) * mp.mpf(float(kf[t, g, i]))
                                          for i in range(D))) for t in range(kf.shape[0])]
            den = mp.fsum(w)
            for i in range(D):
                ref = mp.fsum(w[t] * mp.mpf(float(vf[t, g, i])) for t in range(kf.shape[0])) / den
                assert abs(got[b, h, i] - float(ref)) <= 1e-12


@pytest.mark.parametrize("seed,B,Hq,Hkv,D,Tmax,bs", [
    (10, 4, 8, 2, 64, 70, 16),
    (11, 3, 4, 4, 128, 40, 16),
    (12, 2, 8, 1, 32, 33, 8),
])
def test_torch_sdpa_float64(seed, B, Hq, Hkv, D, Tmax, bs):
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(seed)
    q, dk, dv, kp, vp, bt, sl = rand_case(rng, B, Hq, Hkv, D, Tmax, bs)
    got = run_oracle(q, kp, vp, bt, sl, Hq, Hkv, bs)
    G = Hq // Hkv
    for b in range(B):
        qt = torch.from_numpy(bf16_bits_to_f32(q[b]).astype(np.float64)).reshape(1, Hq, 1, D)
        kt = torch.from_numpy(bf16_bits_to_f32(dk[b]).astype(np.float64)).permute(1, 0, 2)
        vt = torch.from_numpy(bf16_bits_to_f32(dv[b]).astype(np.float64)).permute(1, 0, 2)
        kt = kt.repeat_interleave(G, dim=0).unsqueeze(0).contiguous()
        vt = vt.repeat_interleave(G, dim=0).unsqueeze(0).contiguous()
        ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt).reshape(Hq, D).numpy()
        np.testing.assert_allclose(got[b], ref, rtol=0, atol=1e-12)


def test_golden_logistic():
    with open(os.path.join(GOLDEN, "logistic_two_token.json")) as f:
        g = json.load(f)
    D = g["head_dim"]
    q = bf16(np.array(g["q"]).reshape(1, 1, D))
    k = bf16(np.array(g["k"]).reshape(2, 1, D))
    v = bf16(np.array(g["v"]).reshape(2, 1, D))
    kp, vp, bt, sl = paged([k], [v], 16, np.random.default_rng(0))
    got = run_oracle(q, kp, vp, bt, sl, 1, 1, 16)[0, 0]
    np.testing.assert_allclose(got, g["out"], rtol=0, atol=g["tolerance"])


def test_closed_form_single_token_returns_v0():
    rng = np.random.default_rng(20)
    q, dk, dv, kp, vp, bt, sl = rand_case(rng, 5, 8, 2, 64, 1, 16)
    got = run_oracle(q, kp, vp, bt, sl, 8, 2, 16)
    for b in range(5):
        for h in range(8):
            assert np.array_equal(got[b, h], bf16_bits_to_f32(dv[b][0, h // 4]).astype(np.float64))


def test_closed_form_identical_keys_and_zero_query_give_mean():
    rng = np.random.default_rng(21)
    B, Hq, Hkv, D, T = 3, 4, 2, 32, 45
    q = bf16(rng.standard_normal((B, Hq, D)))
    q[1] = 0  # q = 0 for query 1
    dk, dv = [], []
    for b in range(B):
        base = bf16(rng.standard_normal((1, Hkv, D)))
        k = np.repeat(base, T, axis=0) if b != 1 else bf16(rng.standard_normal((T, Hkv, D)))
        dk.append(k)
        dv.append(bf16(rng.standard_normal((T, Hkv, D))))
    kp, vp, bt, sl = paged(dk, dv, 16, rng)
    got = run_oracle(q, kp, vp, bt, sl, Hq, Hkv, 16)
    for b in range(B):
        mean = bf16_bits_to_f32(dv[b]).astype(np.float64).mean(axis=0)  # [Hkv][D]
        for h in range(Hq):
            np.testing.assert_allclose(got[b, h], mean[h // 2], rtol=0, atol=1e-14)


def test_closed_form_constant_v():
    rng = np.random.default_rng(22)
    B, Hq, Hkv, D, T = 2, 4, 4, 16, 37
    q = bf16(rng.standard_normal((B, Hq, D)))
    dk = [bf16(rng.standard_normal((T, Hkv, D))) for _ in range(B)]
    c = bf16(rng.standard_normal((1, Hkv, D)))
    dv = [np.repeat(c, T, axis=0) for _ in range(B)]
    kp, vp, bt, sl = paged(dk, dv, 16, rng)
    got = run_oracle(q, kp, vp, bt, sl, Hq, Hkv, 16)
    cf = bf16_bits_to_f32(c[0]).astype(np.float64)
    for b in range(B):
        np.testing.assert_allclose(got[b], cf, rtol=1e-14, atol=1e-15)


def test_merge_of_halves_equals_whole():
    rng = np.random.default_rng(23)
    B, Hq, Hkv, D = 3, 4, 2, 64
    q, dk, dv, kp, vp, bt, sl = rand_case(rng, B, Hq, Hkv, D, 90, 16)
    full = run_oracle(q, kp, vp, bt, sl, Hq, Hkv, 16)
    for b in range(B):
        T = int(sl[b])
        if T < 2:
            continue
        for h in range(Hq):
            cuts = sorted(set([0, int(rng.integers(1, T)), int(rng.integers(1, T)), T]))
            parts = [oracle.partial(q, kp, vp, bt, Hq, Hkv, b, h, a, e) for a, e in zip(cuts[:-1], cuts[1:])]
            got = oracle.merge([p[0] for p in parts], [p[1] for p in parts], np.stack([p[2] for p in parts]))
            np.testing.assert_allclose(got, full[b, h], rtol=0, atol=1e-13)


def test_invariant_token_permutation():
    rng = np.random.default_rng(24)
    B, Hq, Hkv, D = 3, 8, 2, 64
    q, dk, dv, kp, vp, bt, sl = rand_case(rng, B, Hq, Hkv, D, 60, 16)
    a = run_oracle(q, kp, vp, bt, sl, Hq, Hkv, 16)
    perms = [rng.permutation(k.shape[0]) for k in dk]
    kp2, vp2, bt2, sl2 = paged([k[p] for k, p in zip(dk, perms)], [v[p] for v, p in zip(dv, perms)], 16, rng)
    b_ = run_oracle(q, kp2, vp2, bt2, sl2, Hq, Hkv, 16)
    np.testing.assert_allclose(a, b_, rtol=0, atol=1e-13)


def test_invariant_common_score_shift():
    # integer-valued keys keep K + u exact in bf16; q . u is the same for every token
    rng = np.random.default_rng(25)
    B, Hq, Hkv, D, T = 2, 2, 2, 16, 29
    q = bf16(rng.integers(-2, 3, size=(B, Hq, D)).astype(np.float32) / 4)
    dk = [bf16(rng.integers(-3, 4, size=(T, Hkv, D)).astype(np.float32)) for _ in range(B)]
    dv = [bf16(rng.standard_normal((T, Hkv, D))) for _ in range(B)]
    kp, vp, bt, sl = paged(dk, dv, 16, rng)
    a = run_oracle(q, kp, vp, bt, sl, Hq, Hkv, 16)
    u = rng.integers(-4, 5, size=(1, Hkv, D)).astype(np.float32)
    dk2 = [bf16(bf16_bits_to_f32(k) + u) for k in dk]
    kp2, vp2, bt2, sl2 = paged(dk2, dv, 16, rng)
    b_ = run_oracle(q, kp2, vp2, bt2, sl2, Hq, Hkv, 16)
    np.testing.assert_allclose(a, b_, rtol=0, atol=1e-13)


def test_invariant_linear_in_v():
    rng = np.random.default_rng(26)
    q, dk, dv, kp, vp, bt, sl = rand_case(rng, 3, 4, 2, 32, 50, 16)
    a = run_oracle(q, kp, vp, bt, sl, 4, 2, 16)
    vp2 = vp.copy()
    finite = (vp & 0x7F80) != 0x7F80
    vp2[finite] = bf16(2.0 * bf16_bits_to_f32(vp[finite]))
    b_ = run_oracle(q, kp, vp2, bt, sl, 4, 2, 16)
    assert np.array_equal(b_, 2.0 * a)


def test_invariant_gqa_equals_mha_with_repeated_kv():
    rng = np.random.default_rng(27)
    B, Hq, Hkv, D = 3, 8, 2, 32
    q, dk, dv, kp, vp, bt, sl = rand_case(rng, B, Hq, Hkv, D, 40, 16)
    a = run_oracle(q, kp, vp, bt, sl, Hq, Hkv, 16)
    G = Hq // Hkv
    kp2, vp2, bt2, sl2 = paged([np.repeat(k, G, axis=1) for k in dk], [np.repeat(v, G, axis=1) for v in dv], 16,
                               rng)
    b_ = run_oracle(q, kp2, vp2, bt2, sl2, Hq, Hq, 16)
    assert np.array_equal(a, b_)


def test_invariant_convex_hull():
    rng = np.random.default_rng(28)
    B, Hq, Hkv, D = 4, 4, 2, 64
    q, dk, dv, kp, vp, bt, sl = rand_case(rng, B, Hq, Hkv, D, 80, 16)
    q = bf16(8.0 * bf16_bits_to_f32(q))  # peaked softmax
    got = run_oracle(q, kp, vp, bt, sl, Hq, Hkv, 16)
    for b in range(B):
        vf = bf16_bits_to_f32(dv[b]).astype(np.float64)
        for h in range(Hq):
            lo, hi = vf[:, h // 2].min(axis=0), vf[:, h // 2].max(axis=0)
            assert np.all(got[b, h] >= lo - 1e-12) and np.all(got[b, h] <= hi + 1e-12)


def test_explicit_scale_and_rejects_bad_input():
    rng = np.random.default_rng(29)
    q, dk, dv, kp, vp, bt, sl = rand_case(rng, 2, 2, 2, 16, 20, 16)
    a = run_oracle(q, kp, vp, bt, sl, 2, 2, 16)
    b_ = run_oracle(q, kp, vp, bt, sl, 2, 2, 16, scale=0.25)  # 1/sqrt(16)
    assert np.array_equal(a, b_)
    c = run_oracle(q, kp, vp, bt, sl, 2, 2, 16, scale=0.5)
    assert not np.allclose(a, c)
    bad = sl.copy()
    bad[0] = 0
    with pytest.raises(ValueError):
        run_oracle(q, kp, vp, bt, bad, 2, 2, 16)
    with pytest.raises(ValueError):
        run_oracle(q, kp, vp, bt, sl, 3, 2, 16)


@pytest.mark.parametrize("seed,B,Hq,Hkv,D,L,bs", [
    (20, 2, 4, 2, 16, 37, 16),
    (21, 3, 2, 1, 8, 11, 4),
])
def test_append_then_attend_steps_equal_causal_attention(seed, B, Hq, Hkv, D, L, bs):
    """Decoding token by token into an empty paged cache equals causal attention over the sequence.

    Step t appends K_t, V_t with append_tokens (seq_len t + 1) and attends with
    the oracle; torch's float64 scaled_dot_product_attention with a causal mask
    over all L positions at once is the reference.  After the last step the
    pools equal the dense sequences packed directly into the same blocks.
    """
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(seed)
    q = bf16(rng.standard_normal((B, L, Hq, D)))
    dk = [bf16(rng.standard_normal((L, Hkv, D))) for _ in range(B)]
    dv = [bf16(rng.standard_normal((L, Hkv, D))) for _ in range(B)]
    kp_full, vp_full, bt, _ = paged(dk, dv, bs, rng)
    kp = np.full_like(kp_full, 0x7FC0)       # NaN everywhere: only appended slots are ever read
    vp = np.full_like(vp_full, 0x7FC0)
    G = Hq // Hkv
    for t in range(L):
        lens = np.full(B, t + 1, dtype=np.int32)
        k_new = np.stack([dk[b][t] for b in range(B)])
        v_new = np.stack([dv[b][t] for b in range(B)])
        kp2, vp2 = oracle.append_tokens(kp, vp, bt, lens, k_new, v_new, block_size=bs)
        assert np.isnan(bf16_bits_to_f32(kp)).sum() - np.isnan(bf16_bits_to_f32(kp2)).sum() == B * Hkv * D
        kp, vp = kp2, vp2
        got = oracle.decode_all(q[:, t], kp, vp, bt, lens, Hq, Hkv, block_size=bs)
        for b in range(B):
            qt = torch.from_numpy(bf16_bits_to_f32(q[b]).astype(np.float64)).permute(1, 0, 2).unsqueeze(0)
            kt = torch.from_numpy(bf16_bits_to_f32(dk[b]).astype(np.float64)).permute(1, 0, 2)
            vt = torch.from_numpy(bf16_bits_to_f32(dv[b]).astype(np.float64)).permute(1, 0, 2)
            kt = kt.repeat_interleave(G, dim=0).unsqueeze(0).contiguous()
            vt = vt.repeat_interleave(G, dim=0).unsqueeze(0).contiguous()
            ref = torch.nn.functional.scaled_dot_product_attention(qt.contiguous(), kt, vt, is_causal=True)
            np.testing.assert_allclose(got[b], ref[0, :, t, :].numpy(), rtol=0, atol=1e-12)
    np.testing.assert_array_equal(kp, kp_full)
    np.testing.assert_array_equal(vp, vp_full)


def _sdpa_rows(q, dk, dv, Hq, Hkv, rows):
    """torch float64 SDPA of each listed row b * Hq + h over query b's own dense K/V."""
    import torch
    G = Hq // Hkv
    D = q.shape[-1]
    out = np.empty((len(rows), D))
    for i, r in enumerate(rows):
        b, h = divmod(int(r), Hq)
        qt = torch.from_numpy(bf16_bits_to_f32(q[b, h]).astype(np.float64)).reshape(1, 1, 1, D)
        kt = torch.from_numpy(bf16_bits_to_f32(dk[b][:, h // G]).astype(np.float64)).reshape(1, 1, -1, D)
        vt = torch.from_numpy(bf16_bits_to_f32(dv[b][:, h // G]).astype(np.float64)).reshape(1, 1, -1, D)
        out[i] = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt).reshape(D).numpy()
    return out


@pytest.mark.parametrize("seed,B,Hq,Hkv,D,Tmax,bs", [
    (40, 5, 8, 2, 64, 70, 16),
    (41, 3, 6, 3, 32, 45, 4),
])
def test_row_subset_path(seed, B, Hq, Hkv, D, Tmax, bs):
    """decode_rows writes row r of its output from (b, h) = divmod(rows[r], Hq), for any row list.

    Every full-size parity check goes through this path with a row list other
    than arange, so it is pinned on its own: permuted, repeated, single and
    last rows against torch float64 SDPA of each listed row, and bit for bit
    against the same rows of decode_all.  A row index taken from r instead of
    rows[r], a swapped (b, h) split or an output offset of rows[r] * D fails
    it.
    """
    pytest.importorskip("torch")
    rng = np.random.default_rng(seed)
    q, dk, dv, kp, vp, bt, sl = rand_case(rng, B, Hq, Hkv, D, Tmax, bs)
    full = run_oracle(q, kp, vp, bt, sl, Hq, Hkv, bs).reshape(B * Hq, D)
    n = B * Hq
    perm = rng.permutation(n)
    subsets = [
        perm,                                              # every row, permuted
        perm[: n // 3],                                    # a permuted strict subset
        np.array([n - 1]),                                 # the last row alone
        np.array([3, 3, 0, n - 1, 3, 1]),                  # repeats and out-of-order rows
        rng.integers(0, n, size=2 * n),                    # random rows with repeats
    ]
    for rows in subsets:
        rows = np.asarray(rows, dtype=np.int64)
        got = oracle.decode_rows(q, kp, vp, bt, sl, Hq, Hkv, rows, block_size=bs)
        assert got.shape == (len(rows), D)
        np.testing.assert_allclose(got, _sdpa_rows(q, dk, dv, Hq, Hkv, rows), rtol=0, atol=1e-12)
        assert np.array_equal(got, full[rows])
