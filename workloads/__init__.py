"""Seeded synthetic decode batches over a paged KV cache shared along a prefix tree.

This module only builds inputs: sequence lengths, block tables, the physical
block permutation and N(0, 1) bf16 values.  It holds none of the attention
arithmetic, and both the oracle's callers and the HIP path's callers take
their inputs from it.

Shapes follow the pages' workloads:
  * decode queries are single tokens and attend over everything cached,
    the current token included (short-term-memory concept page, the
    autoregressive KV-cache step);
  * the cache is paged in 16-token blocks with a per-request block table
    (same page, PagedAttention section);
  * requests share hierarchical prefixes -- system prompt, tool templates,
    sessions (PAT review, problem definition and Fig 4 / Fig 5 captions;
    stateful-streaming digest, "stateful sessions" and "Flash Queries").

Layouts handed to the library and the oracle:
  q            uint16 (bf16 bits) [B][Hq][D]
  k_pool/v_pool uint16 (bf16 bits) [n_blocks][Hkv][16][D]; token slots a
               block does not hold are bf16 NaN
  block_tables int32 [B][max_blocks]; entries past ceil(T_b/16) are -1
  seq_lens     int32 [B]
"""
from __future__ import annotations

import ctypes
import dataclasses
import math
import os
import subprocess
from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np

BLOCK = 16
TAG_Q, TAG_K, TAG_V = 1, 2, 3
BF16_NAN = 0x7FC0

_HERE = os.path.dirname(os.path.abspath(__file__))
_SO = os.path.join(_HERE, "libkvgen.so")
_lib = None


def build_generator(force: bool = False) -> str:
    """Compile gen.c into libkvgen.so with gcc (OpenMP)."""
    src = os.path.join(_HERE, "gen.c")
    if force or not os.path.exists(_SO) or os.path.getmtime(_SO) < os.path.getmtime(src):
        tmp = _SO + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-shared", "-fPIC", "-o", tmp, src, "-lm"])
        os.replace(tmp, _SO)
    return _SO


def _gen():
    global _lib
    if _lib is None:
        build_generator()
        lib = ctypes.CDLL(_SO)
        lib.kvgen_normal_bf16.argtypes = [ctypes.c_uint64, ctypes.c_uint64, ctypes.c_uint64, ctypes.c_uint64,
                                          ctypes.c_void_p]
        lib.kvgen_normal_bf16_gather.argtypes = [ctypes.c_uint64, ctypes.c_uint64, ctypes.c_void_p,
                                                 ctypes.c_uint64, ctypes.c_void_p]
        lib.kvgen_fill_pool.argtypes = [ctypes.c_uint64, ctypes.c_uint64, ctypes.c_int64, ctypes.c_int64,
                                        ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p]
        _lib = lib
    return _lib


def normal_bf16(seed: int, tag: int, start: int, count: int, out: Optional[np.ndarray] = None) -> np.ndarray:
    """bf16 bits of elements [start, start+count) of the (seed, tag) N(0,1) stream."""
    if out is None:
        out = np.empty(count, dtype=np.uint16)
    assert out.dtype == np.uint16 and out.flags.c_contiguous and out.size == count
    _gen().kvgen_normal_bf16(seed, tag, start, count, out.ctypes.data)
    return out


def normal_bf16_at(seed: int, tag: int, idx: np.ndarray) -> np.ndarray:
    idx = np.ascontiguousarray(idx, dtype=np.uint64)
    out = np.empty(idx.shape, dtype=np.uint16)
    _gen().kvgen_normal_bf16_gather(seed, tag, idx.ctypes.data, idx.size, out.ctypes.data)
    return out


def bf16_bits_to_f32(x: np.ndarray) -> np.ndarray:
    return (x.astype(np.uint32) << 16).view(np.float32)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round-to-nearest-even fp32 -> bf16 bits (finite inputs)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)


@dataclasses.dataclass
class Workload:
    name: str
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    seq_lens: np.ndarray          # int32 [B]
    block_tables: np.ndarray      # int32 [B][max_blocks]
    block_valid: np.ndarray       # int32 [n_blocks] tokens held by each physical block
    seed_values: int
    segments: List[List[Tuple[object, int]]]   # per query: (segment key, tokens)
    q: Optional[np.ndarray] = None
    k_pool: Optional[np.ndarray] = None
    v_pool: Optional[np.ndarray] = None

    # ---- shape -------------------------------------------------------------
    @property
    def num_queries(self) -> int:
        return int(self.seq_lens.shape[0])

    @property
    def num_blocks(self) -> int:
        return int(self.block_valid.shape[0])

    @property
    def max_blocks(self) -> int:
        return int(self.block_tables.shape[1])

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    def shape_tuple(self):
        return (self.num_queries, self.num_q_heads, self.num_kv_heads, self.head_dim, BLOCK,
                self.max_blocks, self.num_blocks)

    # ---- byte accounting ---------------------------------------------------
    @property
    def bytes_per_token(self) -> int:
        """K and V bytes of one token over all KV heads (bf16)."""
        return 2 * self.num_kv_heads * self.head_dim * 2

    @property
    def unique_kv_bytes(self) -> int:
        return int(self.block_valid.astype(np.int64).sum()) * self.bytes_per_token

    @property
    def query_centric_kv_bytes(self) -> int:
        return int(self.seq_lens.astype(np.int64).sum()) * self.bytes_per_token

    @property
    def prefix_ratio(self) -> float:
        """Share of the query-centric token references that fall in a segment held by >= 2 queries."""
        count: Dict[object, int] = {}
        for segs in self.segments:
            for key, _ in segs:
                count[key] = count.get(key, 0) + 1
        shared = sum(n for segs in self.segments for key, n in segs if count[key] >= 2)
        return shared / float(self.seq_lens.astype(np.int64).sum())

    # ---- values ------------------------------------------------------------
    def materialize(self) -> "Workload":
        B, Hq, Hkv, D = self.num_queries, self.num_q_heads, self.num_kv_heads, self.head_dim
        self.q = normal_bf16(self.seed_values, TAG_Q, 0, B * Hq * D).reshape(B, Hq, D)
        n = self.num_blocks
        lib = _gen()
        valid = np.ascontiguousarray(self.block_valid, dtype=np.int32)
        self.k_pool = np.empty((n, Hkv, BLOCK, D), dtype=np.uint16)
        self.v_pool = np.empty((n, Hkv, BLOCK, D), dtype=np.uint16)
        lib.kvgen_fill_pool(self.seed_values, TAG_K, n, Hkv, BLOCK, D, valid.ctypes.data, self.k_pool.ctypes.data)
        lib.kvgen_fill_pool(self.seed_values, TAG_V, n, Hkv, BLOCK, D, valid.ctypes.data, self.v_pool.ctypes.data)
        return self

    def release_values(self):
        self.q = self.k_pool = self.v_pool = None


def from_segments(name: str, segments: Sequence[Sequence[Tuple[object, int]]], num_q_heads: int,
                  num_kv_heads: int, head_dim: int, seed_struct: int, seed_values: int,
                  extra_blocks: int = 0) -> Workload:
    """Build a batch from per-query segment lists.

    Each query's token sequence is the concatenation of its segments; a segment
    key that appears in several queries is one run of shared physical blocks.
    Every segment but a query's last must hold a multiple of 16 tokens, so
    blocks never straddle segments.  Physical ids are a seeded permutation of
    [0, n_blocks + extra_blocks); the extra blocks are allocated but unused.
    """
    seg_len: Dict[object, int] = {}
    order: List[object] = []
    for segs in segments:
        for i, (key, n) in enumerate(segs):
            if n <= 0:
                raise ValueError("empty segment")
            if i + 1 < len(segs) and n % BLOCK:
                raise ValueError("inner segments must hold whole blocks")
            if key in seg_len:
                if seg_len[key] != n:
                    raise ValueError("segment %r has two lengths" % (key,))
            else:
                seg_len[key] = n
                order.append(key)
    logical = []          # (segment key, block index within segment, valid tokens)
    seg_first: Dict[object, int] = {}
    for key in order:
        n = seg_len[key]
        seg_first[key] = len(logical)
        nb = (n + BLOCK - 1) // BLOCK
        for j in range(nb):
            logical.append(min(BLOCK, n - j * BLOCK))
    n_used = len(logical)
    n_total = n_used + extra_blocks
    rng = np.random.default_rng(seed_struct)
    perm = rng.permutation(n_total).astype(np.int32)
    block_valid = np.full(n_total, 0, dtype=np.int32)
    for i, v in enumerate(logical):
        block_valid[perm[i]] = v
    seq_lens = np.array([sum(n for _, n in segs) for segs in segments], dtype=np.int32)
    max_blocks = int(max((t + BLOCK - 1) // BLOCK for t in seq_lens))
    bt = np.full((len(segments), max_blocks), -1, dtype=np.int32)
    for b, segs in enumerate(segments):
        j = 0
        for key, n in segs:
            nb = (n + BLOCK - 1) // BLOCK
            first = seg_first[key]
            bt[b, j:j + nb] = perm[first:first + nb]
            j += nb
    return Workload(name=name, num_q_heads=num_q_heads, num_kv_heads=num_kv_heads, head_dim=head_dim,
                    seq_lens=seq_lens, block_tables=bt, block_valid=block_valid, seed_values=seed_values,
                    segments=[list(s) for s in segments])


# ---------------------------------------------------------------------------
# The five workloads.  Config c draws its structure from seed c and its
# values from seed 100 + c.  "uniform a-b" means integers inclusive of both
# ends; log-uniform [16, 32768] means T = min(32768, floor(16 * 2048**u)).
# ---------------------------------------------------------------------------

def _shared_prefix(name, B, Hq, Hkv, D, prefix, lo, hi, seed, scale_b=1):
    rng = np.random.default_rng(seed)
    suf = rng.integers(lo, hi + 1, size=B)
    segs = [[("prefix", prefix), (("leaf", b), int(suf[b]))] for b in range(B)]
    return from_segments(name, segs, Hq, Hkv, D, seed_struct=seed + 1000, seed_values=100 + seed)


def config1() -> Workload:
    """Tiny batch: 4 queries, 4/4 heads, d 64, shared 256-token prefix + uniform 32-96 suffixes."""
    return _shared_prefix("c1_tiny", 4, 4, 4, 64, 256, 32, 96, 1)


def config2() -> Workload:
    """Llama-3-8B-shaped layer: 64 queries, 32/8 heads, d 128, 2048 shared + uniform 128-1024."""
    return _shared_prefix("c2_llama3_8b_layer", 64, 32, 8, 128, 2048, 128, 1024, 2)


def _two_level(name, B, Hq, Hkv, D, root, n_child, child, lo, hi, seed):
    rng = np.random.default_rng(seed)
    which = rng.integers(0, n_child, size=B)
    suf = rng.integers(lo, hi + 1, size=B)
    segs = [[("root", root), (("child", int(which[b])), child), (("leaf", b), int(suf[b]))] for b in range(B)]
    return from_segments(name, segs, Hq, Hkv, D, seed_struct=seed + 1000, seed_values=100 + seed)


def config3() -> Workload:
    """Two-level tree: 256 queries, 4096 root, 8 x 1024 children (uniform choice), uniform 64-2048 leaves."""
    return _two_level("c3_two_level_tree", 256, 32, 8, 128, 4096, 8, 1024, 64, 2048, 3)


def _sessions(name, n_sess, per_sess, ctx, Hq, Hkv, D, seed):
    segs = [[(("session", s), ctx)] for s in range(n_sess) for _ in range(per_sess)]
    return from_segments(name, segs, Hq, Hkv, D, seed_struct=seed + 1000, seed_values=100 + seed)


def config4() -> Workload:
    """Stateful sessions: 16 sessions x 131072 tokens, 8 registered queries each, 64/8 heads, d 128."""
    return _sessions("c4_streaming_sessions", 16, 8, 131072, 64, 8, 128, 4)


def _no_sharing(name, B, Hq, Hkv, D, lo, hi, seed):
    rng = np.random.default_rng(seed)
    u = rng.random(size=B)
    T = np.minimum(hi, np.floor(lo * (hi / lo) ** u)).astype(np.int64)
    segs = [[(("own", b), int(T[b]))] for b in range(B)]
    return from_segments(name, segs, Hq, Hkv, D, seed_struct=seed + 1000, seed_values=100 + seed)


def config5() -> Workload:
    """No sharing: 512 queries, lengths log-uniform in [16, 32768], 32/8 heads, d 128."""
    return _no_sharing("c5_no_sharing", 512, 32, 8, 128, 16, 32768, 5)


WORKLOADS = {1: config1, 2: config2, 3: config3, 4: config4, 5: config5}


# Reduced shapes of the same five structures, for element-by-element parity
# against the oracle.  They keep the head shapes and tree structure and span
# several KV tiles, split chunks and ragged tails.
def small(c: int) -> Workload:
    if c == 1:
        return config1()
    if c == 2:
        return _shared_prefix("c2_small", 12, 32, 8, 128, 512, 1, 300, 12)
    if c == 3:
        return _two_level("c3_small", 40, 32, 8, 128, 768, 3, 256, 1, 400, 13)
    if c == 4:
        return _sessions("c4_small", 2, 8, 4096, 64, 8, 128, 14)
    if c == 5:
        return _no_sharing("c5_small", 48, 32, 8, 128, 1, 3000, 15)
    raise KeyError(c)


def kv_cache_bytes_formula(layers: int, kv_heads: int, head_dim: int, tokens: int, dtype_bytes: int) -> int:
    """KV-cache size: 2 (K and V) x layers x KV heads x head dim x tokens x bytes per element.

    The short-term-memory concept page gives this estimate in its KV-cache
    section, and its GQA note makes clear the head count is that of KV heads.
    """
    return 2 * layers * kv_heads * head_dim * tokens * dtype_bytes
