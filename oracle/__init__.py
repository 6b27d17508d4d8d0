"""fp64 CPU oracle for paged decode attention -- TEST INFRASTRUCTURE ONLY.

Only tests/, __graft_entry__.smoke() and bench.py's CPU-baseline leg may
import this package.  The library (decode_attention_prefix_amd) never does,
and this package imports nothing from it.

The arithmetic lives in kvattn_oracle.c (plain C, double precision, compiled
with gcc); this file marshals numpy arrays through ctypes and holds the one
step without arithmetic, the append of a decode step's new token to the paged
cache (numpy indexing).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SO = os.path.join(_HERE, "libkvattn_oracle.so")
_lib = None


def build_oracle(force: bool = False) -> str:
    src = os.path.join(_HERE, "kvattn_oracle.c")
    if force or not os.path.exists(_SO) or os.path.getmtime(_SO) < os.path.getmtime(src):
        tmp = _SO + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fno-fast-math", "-shared", "-fPIC", "-o", tmp, src,
                               "-lm"])
        os.replace(tmp, _SO)
    return _SO


def _oracle():
    global _lib
    if _lib is None:
        build_oracle()
        lib = ctypes.CDLL(_SO)
        i32, i64, p, f64 = ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p, ctypes.c_double
        lib.kvattn_oracle_decode_rows.argtypes = [i32, i32, i32, i32, i32, i32, p, p, p, p, p, f64, i64, p, p]
        lib.kvattn_oracle_decode_rows.restype = ctypes.c_int
        lib.kvattn_oracle_partial.argtypes = [i32, i32, i32, i32, i32, p, p, p, p, i64, i64, i64, i64, f64, p, p,
                                              p]
        lib.kvattn_oracle_partial.restype = ctypes.c_int
        lib.kvattn_oracle_merge.argtypes = [i32, i32, p, p, p, p]
        lib.kvattn_oracle_merge.restype = ctypes.c_int
        lib.kvattn_oracle_threads.argtypes = []
        lib.kvattn_oracle_threads.restype = ctypes.c_int
        lib.kvattn_oracle_set_threads.argtypes = [i32]
        lib.kvattn_oracle_set_threads.restype = None
        _lib = lib
    return _lib


def _c(a, dtype):
    a = np.ascontiguousarray(a, dtype=dtype)
    return a, a.ctypes.data


def decode_rows(q, k_pool, v_pool, block_tables, seq_lens, num_q_heads, num_kv_heads, rows, scale=0.0,
                block_size=16):
    """Attention of rows (b * Hq + h) in float64 -> array [len(rows)][D].

    q: uint16 bf16 bits [B][Hq][D]; pools: uint16 [n_blocks][Hkv][block][D].
    """
    q, qp = _c(q, np.uint16)
    k_pool, kp = _c(k_pool, np.uint16)
    v_pool, vp = _c(v_pool, np.uint16)
    bt, btp = _c(block_tables, np.int32)
    sl, slp = _c(seq_lens, np.int32)
    rows, rp = _c(np.asarray(rows).reshape(-1), np.int64)
    B, D = q.shape[0], q.shape[-1]
    out = np.empty((rows.size, D), dtype=np.float64)
    rc = _oracle().kvattn_oracle_decode_rows(B, num_q_heads, num_kv_heads, D, block_size, bt.shape[1], qp, kp, vp,
                                             btp, slp, float(scale), rows.size, rp, out.ctypes.data)
    if rc != 0:
        raise ValueError("oracle rejected its inputs")
    return out


def decode_all(q, k_pool, v_pool, block_tables, seq_lens, num_q_heads, num_kv_heads, scale=0.0, block_size=16):
    B, D = q.shape[0], q.shape[-1]
    rows = np.arange(B * num_q_heads, dtype=np.int64)
    return decode_rows(q, k_pool, v_pool, block_tables, seq_lens, num_q_heads, num_kv_heads, rows, scale,
                       block_size).reshape(B, num_q_heads, D)


def append_tokens(k_pool, v_pool, block_tables, seq_lens, k_new, v_new, block_size=16):
    """The KV pools after one decode step's append -> new (k_pool, v_pool) arrays.

    Short-term-memory page, technical principles (the KV cache in
    autoregressive generation): a step computes its token's K and V and adds
    them to the cache before attending over every cached token.  With paging
    (PagedAttention section) query b's newest token, position seq_lens[b] - 1,
    sits in block block_tables[b][pos // block_size], slot pos % block_size;
    each KV head's row of that slot receives k_new[b][head] (likewise V).
    Pools: uint16 bf16 bits [n_blocks][Hkv][block_size][D]; k_new, v_new:
    uint16 [B][Hkv][D].  The inputs are not modified.
    """
    k = np.array(k_pool, dtype=np.uint16, copy=True)
    v = np.array(v_pool, dtype=np.uint16, copy=True)
    for b, T in enumerate(np.asarray(seq_lens).tolist()):
        pos = int(T) - 1
        blk = int(block_tables[b][pos // block_size])
        k[blk, :, pos % block_size, :] = k_new[b]
        v[blk, :, pos % block_size, :] = v_new[b]
    return k, v


def decode_workload(wl, rows=None, scale=0.0):
    """Oracle output for a workloads.Workload (values materialized)."""
    if rows is None:
        return decode_all(wl.q, wl.k_pool, wl.v_pool, wl.block_tables, wl.seq_lens, wl.num_q_heads,
                          wl.num_kv_heads, scale)
    return decode_rows(wl.q, wl.k_pool, wl.v_pool, wl.block_tables, wl.seq_lens, wl.num_q_heads,
                       wl.num_kv_heads, rows, scale)


def partial(q, k_pool, v_pool, block_tables, num_q_heads, num_kv_heads, b, h, t0, t1, scale=0.0, block_size=16):
    """Partial triple (m, l, acc) of row (b, h) over tokens [t0, t1), natural-log units."""
    q, qp = _c(q, np.uint16)
    k_pool, kp = _c(k_pool, np.uint16)
    v_pool, vp = _c(v_pool, np.uint16)
    bt, btp = _c(block_tables, np.int32)
    D = q.shape[-1]
    m = ctypes.c_double()
    l = ctypes.c_double()
    acc = np.empty(D, dtype=np.float64)
    rc = _oracle().kvattn_oracle_partial(num_q_heads, num_kv_heads, D, block_size, bt.shape[1], qp, kp, vp, btp, b,
                                         h, t0, t1, float(scale), ctypes.addressof(m), ctypes.addressof(l),
                                         acc.ctypes.data)
    if rc != 0:
        raise ValueError("oracle rejected its inputs")
    return m.value, l.value, acc


def merge(ms, ls, accs):
    """Online-softmax combination of partial triples -> out[D]."""
    ms, mp = _c(ms, np.float64)
    ls, lp = _c(ls, np.float64)
    accs, ap = _c(accs, np.float64)
    n, D = accs.shape
    out = np.empty(D, dtype=np.float64)
    rc = _oracle().kvattn_oracle_merge(n, D, mp, lp, ap, out.ctypes.data)
    if rc != 0:
        raise ValueError("oracle rejected its inputs")
    return out


def threads() -> int:
    """OpenMP threads the oracle uses on this host."""
    return int(_oracle().kvattn_oracle_threads())


def set_threads(n: int) -> None:
    """Run later oracle calls on n OpenMP threads."""
    _oracle().kvattn_oracle_set_threads(int(n))
