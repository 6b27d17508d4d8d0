"""ctypes binding of libkvattn.so (include/kvattn.h): argument marshalling only.

Function names match the C ABI.  Arrays on the host are numpy arrays; device
buffers are torch CUDA/HIP tensors (or raw integer addresses) whose memory the
caller owns; `stream` is a torch stream, a raw hipStream_t address, or None
for torch's current stream.  Every step of the decode runs in the library's
HIP kernels; nothing here computes attention, and there is no fallback: if the
library is missing the import fails.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import numpy as np

_PKG = os.path.dirname(os.path.abspath(__file__))
# KVATTN_LIBRARY selects another build of the library (the sanitized host-test
# variant); by default the in-tree build next to this file is loaded.
LIB_PATH = os.environ.get("KVATTN_LIBRARY") or os.path.join(_PKG, "libkvattn.so")

KVATTN_OK, KVATTN_EINVAL, KVATTN_EUNSUPPORTED, KVATTN_ENOMEM, KVATTN_EWORKSPACE, KVATTN_EHIP, KVATTN_ESTATE = range(7)
KVATTN_PACK_AUTO, KVATTN_PACK_QUERY, KVATTN_PACK_FULL = 0, 1, 2
KVATTN_VARIANT_AUTO, KVATTN_VARIANT_VALU, KVATTN_VARIANT_MFMA, KVATTN_VARIANT_VALU_SPLIT = -1, 0, 1, 2

i32, i64, u64, f32, f64, vp = (ctypes.c_int32, ctypes.c_int64, ctypes.c_uint64, ctypes.c_float, ctypes.c_double,
                               ctypes.c_void_p)
P32 = ctypes.POINTER(ctypes.c_int32)


class kvattn_shape(ctypes.Structure):
    _fields_ = [("num_queries", i32), ("num_q_heads", i32), ("num_kv_heads", i32), ("head_dim", i32),
                ("block_size", i32), ("max_blocks_per_seq", i32), ("num_physical_blocks", i32)]


class kvattn_prefix_tree(ctypes.Structure):
    _fields_ = [("num_nodes", i32), ("parent", P32), ("block_begin", P32), ("block_end", P32), ("query_leaf", P32)]


class kvattn_plan_options(ctypes.Structure):
    _fields_ = [("scale", f32), ("pack_mode", i32), ("scheme", i32), ("force_variant", i32), ("split_tokens", i32),
                ("num_cus", i32), ("new_token", i32), ("multi_stream", i32), ("fused_merge", i32)]


class kvattn_stats(ctypes.Structure):
    _fields_ = [("unique_kv_bytes", i64), ("planned_kv_bytes", i64), ("query_centric_kv_bytes", i64),
                ("partial_bytes", i64), ("num_nodes", i32), ("num_packed_nodes", i32), ("num_items", i32),
                ("num_items_valu", i32), ("num_items_mfma", i32), ("num_folded_leaves", i32),
                ("num_partial_slots", i32), ("num_merge_rows", i32), ("num_direct_rows", i32),
                ("num_launches", i32), ("split_tokens", i32), ("update_path", i32), ("plan_seconds", f64),
                ("blob_bytes", u64), ("workspace_bytes", u64), ("num_items_valu_split", i32), ("one_launch", i32)]

    def as_dict(self):
        return {k: getattr(self, k) for k, _ in self._fields_ if k != "reserved"}


class kvattn_item_info(ctypes.Structure):
    _fields_ = [("kind", i32), ("tile", i32), ("pos_begin", i32), ("n_tokens", i32), ("q_begin", i32), ("n_q", i32),
                ("blk_begin", i32), ("n_rows", i32)]


class kvattn_item_query(ctypes.Structure):
    _fields_ = [("query", i32), ("dest", i32), ("limit", i32), ("pad", i32)]


class kvattn_export(ctypes.Structure):
    _fields_ = [("num_items", i32), ("items", ctypes.POINTER(kvattn_item_info)), ("num_entries", i32),
                ("entries", ctypes.POINTER(kvattn_item_query)), ("num_block_ids", i32), ("block_ids", P32),
                ("num_merge_queries", i32), ("merge_query", P32), ("merge_ptr", P32), ("merge_dest", P32),
                ("num_partial_slots", i32), ("head_dim", i32), ("num_tasks", i32), ("tasks", P32),
                ("num_launches", i32), ("num_lists", i32), ("num_desc_words", i32), ("desc", P32),
                ("list_ptr", P32), ("merge_rec", P32)]


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError("libkvattn.so is not built (%s); run python -m decode_attention_prefix_amd.build" % LIB_PATH)
    lib = ctypes.CDLL(LIB_PATH)
    lib.kvattn_plan_options_default.argtypes = [ctypes.POINTER(kvattn_plan_options)]
    lib.kvattn_plan_options_default.restype = None
    lib.kvattn_plan.argtypes = [ctypes.POINTER(kvattn_shape), P32, P32, ctypes.POINTER(kvattn_prefix_tree),
                                ctypes.POINTER(kvattn_plan_options), ctypes.POINTER(vp)]
    lib.kvattn_plan.restype = ctypes.c_int
    lib.kvattn_plan_update.argtypes = [vp, P32, P32]
    lib.kvattn_expand_query_tokens.argtypes = [ctypes.POINTER(kvattn_shape), P32, P32, P32, P32, P32]
    lib.kvattn_expand_query_tokens.restype = ctypes.c_int
    lib.kvattn_plan_update.restype = ctypes.c_int
    lib.kvattn_plan_device_bytes.argtypes = [vp, ctypes.POINTER(ctypes.c_size_t)]
    lib.kvattn_plan_device_bytes.restype = ctypes.c_int
    lib.kvattn_plan_upload.argtypes = [vp, vp, ctypes.c_size_t, vp]
    lib.kvattn_plan_upload.restype = ctypes.c_int
    for name in ("kvattn_decode", "kvattn_forward", "kvattn_decode_noalloc"):
        getattr(lib, name).argtypes = [vp, vp, vp, vp, vp, vp]
        getattr(lib, name).restype = ctypes.c_int
    lib.kvattn_decode_streams.argtypes = [vp, vp, vp, vp, vp, vp, vp]
    lib.kvattn_decode_streams.restype = ctypes.c_int
    lib.kvattn_decode_append.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp]
    lib.kvattn_decode_append.restype = ctypes.c_int
    lib.kvattn_read_probe.argtypes = [vp, ctypes.c_size_t, vp, ctypes.c_size_t, vp, ctypes.c_size_t, i32, i32, i32, vp]
    lib.kvattn_read_probe.restype = ctypes.c_int
    lib.kvattn_merge.argtypes = [vp, vp, vp]
    lib.kvattn_merge.restype = ctypes.c_int
    lib.kvattn_plan_stats.argtypes = [vp, ctypes.POINTER(kvattn_stats)]
    lib.kvattn_plan_stats.restype = ctypes.c_int
    lib.kvattn_plan_export.argtypes = [vp, ctypes.POINTER(kvattn_export)]
    lib.kvattn_plan_export.restype = ctypes.c_int
    lib.kvattn_plan_destroy.argtypes = [vp]
    lib.kvattn_plan_destroy.restype = None
    lib.kvattn_status_string.argtypes = [ctypes.c_int]
    lib.kvattn_status_string.restype = ctypes.c_char_p
    lib.kvattn_last_error.argtypes = []
    lib.kvattn_last_error.restype = ctypes.c_char_p
    return lib


_lib = _load()
EXPORTED = ("kvattn_plan_options_default", "kvattn_plan", "kvattn_plan_device_bytes", "kvattn_plan_upload",
            "kvattn_decode", "kvattn_decode_append", "kvattn_decode_streams", "kvattn_decode_noalloc", "kvattn_forward", "kvattn_merge", "kvattn_plan_update",
            "kvattn_expand_query_tokens", "kvattn_plan_stats", "kvattn_plan_export", "kvattn_plan_destroy",
            "kvattn_read_probe", "kvattn_status_string", "kvattn_last_error")


class KvattnError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        name = _lib.kvattn_status_string(status).decode()
        detail = _lib.kvattn_last_error().decode()
        super().__init__("%s: %s (%s)" % (what, name, detail))


def _check(status: int, what: str):
    if status != KVATTN_OK:
        raise KvattnError(status, what)


def _ptr(x) -> Optional[int]:
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def _stream(s) -> Optional[int]:
    if s is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(s, int):
        return s
    return s.cuda_stream


class Plan:
    """Owns a kvattn_plan_t; the plan is destroyed with this object."""

    def __init__(self, handle: int, shape: kvattn_shape):
        self.handle = handle
        self.shape = shape
        self._keep = None   # device workspace kept alive while bound

    def __del__(self):
        if getattr(self, "handle", None):
            _lib.kvattn_plan_destroy(self.handle)
            self.handle = None


def kvattn_plan_options_default() -> kvattn_plan_options:
    o = kvattn_plan_options()
    _lib.kvattn_plan_options_default(ctypes.byref(o))
    return o


def make_options(**kw) -> kvattn_plan_options:
    o = kvattn_plan_options_default()
    for k, v in kw.items():
        setattr(o, k, v)
    return o


def kvattn_plan(shape, block_tables: np.ndarray, seq_lens: np.ndarray, tree=None, options=None) -> Plan:
    """shape: kvattn_shape or tuple (B, Hq, Hkv, D, block, max_blocks, n_blocks); tree: None or dict with
    numpy arrays parent, block_begin, block_end, query_leaf."""
    if not isinstance(shape, kvattn_shape):
        shape = kvattn_shape(*[int(x) for x in shape])
    bt = np.ascontiguousarray(block_tables, dtype=np.int32)
    sl = np.ascontiguousarray(seq_lens, dtype=np.int32)
    tree_p = None
    keep = []
    if tree is not None:
        arrs = [np.ascontiguousarray(tree[k], dtype=np.int32) for k in ("parent", "block_begin", "block_end",
                                                                          "query_leaf")]
        keep = arrs
        t = kvattn_prefix_tree(int(arrs[0].size), *[a.ctypes.data_as(P32) for a in arrs])
        tree_p = ctypes.byref(t)
    opt_p = ctypes.byref(options) if options is not None else None
    h = vp()
    _check(_lib.kvattn_plan(ctypes.byref(shape), bt.ctypes.data_as(P32), sl.ctypes.data_as(P32), tree_p, opt_p,
                            ctypes.byref(h)), "kvattn_plan")
    del keep
    return Plan(h.value, shape)


def kvattn_plan_update(plan: Plan, block_tables: np.ndarray, seq_lens: np.ndarray):
    """Bring the plan to longer sequences in place; upload it again before decoding."""
    bt = np.ascontiguousarray(block_tables, dtype=np.int32)
    sl = np.ascontiguousarray(seq_lens, dtype=np.int32)
    _check(_lib.kvattn_plan_update(plan.handle, bt.ctypes.data_as(P32), sl.ctypes.data_as(P32)), "kvattn_plan_update")


def kvattn_expand_query_tokens(shape, block_tables: np.ndarray, seq_lens: np.ndarray, q_lens: np.ndarray):
    """One single-token row per new token of multi-token queries: (block_tables, seq_lens) of the rows."""
    if not isinstance(shape, kvattn_shape):
        shape = kvattn_shape(*[int(x) for x in shape])
    bt = np.ascontiguousarray(block_tables, dtype=np.int32)
    sl = np.ascontiguousarray(seq_lens, dtype=np.int32)
    ql = np.ascontiguousarray(q_lens, dtype=np.int32)
    n = int(ql.astype(np.int64).sum()) if ql.size else 0
    out_bt = np.empty((max(n, 1), shape.max_blocks_per_seq), dtype=np.int32)
    out_sl = np.empty(max(n, 1), dtype=np.int32)
    _check(_lib.kvattn_expand_query_tokens(ctypes.byref(shape), bt.ctypes.data_as(P32), sl.ctypes.data_as(P32),
                                           ql.ctypes.data_as(P32), out_bt.ctypes.data_as(P32),
                                           out_sl.ctypes.data_as(P32)), "kvattn_expand_query_tokens")
    return out_bt[:n], out_sl[:n]


def kvattn_plan_device_bytes(plan: Plan) -> int:
    n = ctypes.c_size_t()
    _check(_lib.kvattn_plan_device_bytes(plan.handle, ctypes.byref(n)), "kvattn_plan_device_bytes")
    return n.value


def kvattn_plan_upload(plan: Plan, workspace, nbytes: Optional[int] = None, stream=None):
    if nbytes is None:
        nbytes = workspace.numel() * workspace.element_size()
    _check(_lib.kvattn_plan_upload(plan.handle, _ptr(workspace), nbytes, _stream(stream)), "kvattn_plan_upload")
    if not isinstance(workspace, int):
        plan._keep = workspace


def kvattn_decode(q, k_cache, v_cache, plan: Plan, out, stream=None):
    _check(_lib.kvattn_decode(_ptr(q), _ptr(k_cache), _ptr(v_cache), plan.handle, _ptr(out), _stream(stream)),
           "kvattn_decode")


def kvattn_decode_noalloc(q, k_cache, v_cache, plan: Plan, out, stream=None):
    """kvattn_decode on the library's static per-device scratch: no workspace, no upload, no allocation."""
    _check(_lib.kvattn_decode_noalloc(_ptr(q), _ptr(k_cache), _ptr(v_cache), plan.handle, _ptr(out),
                                      _stream(stream)), "kvattn_decode_noalloc")


def kvattn_decode_streams(q, k_cache, v_cache, plan: Plan, out, side_stream, stream=None):
    """Multi-stream plans: MFMA launches on side_stream beside the VALU ones on stream."""
    _check(_lib.kvattn_decode_streams(_ptr(q), _ptr(k_cache), _ptr(v_cache), plan.handle, _ptr(out), _stream(stream),
                                      _stream(side_stream)), "kvattn_decode_streams")


def kvattn_decode_append(q, k_new, v_new, k_cache, v_cache, plan: Plan, out, stream=None):
    _check(_lib.kvattn_decode_append(_ptr(q), _ptr(k_new), _ptr(v_new), _ptr(k_cache), _ptr(v_cache), plan.handle,
                                     _ptr(out), _stream(stream)), "kvattn_decode_append")


def kvattn_read_probe(a, b, sink, grid, stream=None, loads_in_flight=4, threads=256):
    """Plain streaming read of tensors a and b (measurement helper; see kvattn.h)."""
    _check(_lib.kvattn_read_probe(_ptr(a), a.numel() * a.element_size(), _ptr(b), b.numel() * b.element_size(),
                                  _ptr(sink), sink.numel() * sink.element_size(), int(grid), int(loads_in_flight),
                                  int(threads), _stream(stream)),
           "kvattn_read_probe")


def kvattn_forward(q, k_cache, v_cache, plan: Plan, out, stream=None):
    _check(_lib.kvattn_forward(_ptr(q), _ptr(k_cache), _ptr(v_cache), plan.handle, _ptr(out), _stream(stream)),
           "kvattn_forward")


def kvattn_merge(plan: Plan, out, stream=None):
    _check(_lib.kvattn_merge(plan.handle, _ptr(out), _stream(stream)), "kvattn_merge")


def kvattn_plan_stats(plan: Plan) -> dict:
    s = kvattn_stats()
    _check(_lib.kvattn_plan_stats(plan.handle, ctypes.byref(s)), "kvattn_plan_stats")
    return s.as_dict()


def kvattn_plan_export(plan: Plan) -> dict:
    """Copies of the plan's schedule arrays as numpy structured data."""
    e = kvattn_export()
    _check(_lib.kvattn_plan_export(plan.handle, ctypes.byref(e)), "kvattn_plan_export")

    def arr(ptr, n, cols):
        if n == 0:
            return np.zeros((0, cols), dtype=np.int32)
        return np.ctypeslib.as_array(ctypes.cast(ptr, P32), shape=(n * cols,)).reshape(n, cols).copy()

    items = arr(e.items, e.num_items, 8)
    entries = arr(e.entries, e.num_entries, 4)
    return {
        "items": {k: items[:, i] for i, k in enumerate(("kind", "tile", "pos_begin", "n_tokens", "q_begin", "n_q",
                                                         "blk_begin", "n_rows"))},
        "entries": {k: entries[:, i] for i, k in enumerate(("query", "dest", "limit", "pad"))},
        "block_ids": arr(e.block_ids, e.num_block_ids, 1).reshape(-1),
        "merge_query": arr(e.merge_query, e.num_merge_queries, 1).reshape(-1),
        "merge_ptr": arr(e.merge_ptr, e.num_merge_queries + 1, 1).reshape(-1),
        "merge_dest": arr(e.merge_dest, int(arr(e.merge_ptr, e.num_merge_queries + 1, 1)[-1, 0]), 1).reshape(-1),
        "num_partial_slots": e.num_partial_slots,
        "head_dim": e.head_dim,
        "tasks": arr(e.tasks, e.num_tasks, 2),
        "num_lists": e.num_lists,
        "desc": arr(e.desc, e.num_desc_words, 1).reshape(-1),
        "list_ptr": arr(e.list_ptr, e.num_launches * e.num_lists * 3, 1).reshape(e.num_launches, e.num_lists, 3),
        "merge_rec": arr(e.merge_rec, e.num_merge_queries, 4),
    }


def kvattn_status_string(status: int) -> str:
    return _lib.kvattn_status_string(status).decode()


def kvattn_last_error() -> str:
    return _lib.kvattn_last_error().decode()


class Decoder:
    """Convenience owner of a plan and its torch-allocated device workspace.

    Allocation (torch) and upload happen here, once per plan; decode() only
    enqueues the library's kernels.
    """

    def __init__(self, shape, block_tables, seq_lens, tree=None, options=None, device="cuda", stream=None):
        import torch
        self.plan = kvattn_plan(shape, block_tables, seq_lens, tree, options)
        self.nbytes = kvattn_plan_device_bytes(self.plan)
        self.workspace = torch.empty(max(self.nbytes, 256), dtype=torch.uint8, device=device)
        kvattn_plan_upload(self.plan, self.workspace, self.workspace.numel(), stream)

    def stats(self):
        return kvattn_plan_stats(self.plan)

    def update(self, block_tables, seq_lens, stream=None):
        """Next decode step: update the plan in place and upload it (a larger workspace if it grew)."""
        import torch
        kvattn_plan_update(self.plan, block_tables, seq_lens)
        n = kvattn_plan_device_bytes(self.plan)
        if n > self.workspace.numel():
            self.workspace = torch.empty(n, dtype=torch.uint8, device=self.workspace.device)
        self.nbytes = n
        kvattn_plan_upload(self.plan, self.workspace, self.workspace.numel(), stream)

    def decode(self, q, k_cache, v_cache, out, stream=None):
        kvattn_decode(q, k_cache, v_cache, self.plan, out, stream)
        return out

    def decode_streams(self, q, k_cache, v_cache, out, side_stream, stream=None):
        """Plans made with multi_stream=1: MFMA launches on side_stream, VALU launches on stream."""
        kvattn_decode_streams(q, k_cache, v_cache, self.plan, out, side_stream, stream)
        return out

    def decode_append(self, q, k_new, v_new, k_cache, v_cache, out, stream=None):
        """Plans made with new_token=1: write each query's new K/V into the cache and attend."""
        kvattn_decode_append(q, k_new, v_new, k_cache, v_cache, self.plan, out, stream)
        return out
