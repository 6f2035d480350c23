"""Thin ctypes binding of libcap (include/cap.h, include/cap_bench.h, include/cap_rows.h).

Argument marshalling only: every step of the attention path runs in the
library's HIP kernels.  Functions keep the C names; device buffers are
passed as integer device addresses and streams as integer hipStream_t
handles (``torch.cuda.current_stream().cuda_stream``).  A missing library is
an error -- there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libcap.so")

CAP_OK = 0
STATUS_NAMES = {0: "CAP_OK", 1: "CAP_ERR_INVALID_ARG", 2: "CAP_ERR_BAD_TREE",
                3: "CAP_ERR_WORKSPACE", 4: "CAP_ERR_UNSUPPORTED", 5: "CAP_ERR_HIP",
                6: "CAP_ERR_STATE", 7: "CAP_ERR_REPLAN"}
(CAP_ERR_INVALID_ARG, CAP_ERR_BAD_TREE, CAP_ERR_WORKSPACE, CAP_ERR_UNSUPPORTED, CAP_ERR_HIP,
 CAP_ERR_STATE, CAP_ERR_REPLAN) = range(1, 8)

EXPORTED = [
    "cap_abi_version", "cap_last_error", "cap_plan_opts_default", "cap_tree_device_bytes",
    "cap_tree_upload", "cap_tree_free", "cap_plan_step", "cap_plan_get_stats",
    "cap_plan_get_view", "cap_plan_upload", "cap_decode_attention", "cap_merge_partials",
    "cap_decode_step", "cap_plan_free", "cap_tree_get_desc", "cap_tree_append", "cap_append_kv",
    "cap_plan_refresh", "cap_bench_fill", "cap_bench_read", "cap_bench_read_stream", "cap_bench_copy",
    "cap_bench_copy_stream",
    "cap_bench_decode_timed", "cap_rows_softmax", "cap_rows_layernorm", "cap_plan_rebuild",
    "cap_decode_step_noalloc",
]


class CapError(RuntimeError):
    def __init__(self, status: int, message: str):
        self.status = status
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {message}")


class AttnDesc(ctypes.Structure):
    _fields_ = [("num_q_heads", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("page_size", ctypes.c_int32),
                ("sm_scale", ctypes.c_float)]


class TreeDesc(ctypes.Structure):
    _fields_ = [("num_nodes", ctypes.c_int32), ("parent", ctypes.c_void_p),
                ("num_tokens", ctypes.c_void_p), ("page_offsets", ctypes.c_void_p),
                ("page_ids", ctypes.c_void_p), ("num_requests", ctypes.c_int32),
                ("path_offsets", ctypes.c_void_p), ("path_nodes", ctypes.c_void_p),
                ("num_pool_pages", ctypes.c_int64)]


class PlanOpts(ctypes.Structure):
    _fields_ = [("share_mode", ctypes.c_int32), ("split_pages", ctypes.c_int32),
                ("shared_rows", ctypes.c_int32), ("num_cus", ctypes.c_int32),
                ("shared_cost", ctypes.c_float), ("rounds", ctypes.c_float),
                ("share_margin", ctypes.c_float), ("order", ctypes.c_int32),
                ("private_rounds", ctypes.c_float), ("tail_factor", ctypes.c_float),
                ("tail_min_pages", ctypes.c_int32), ("item_dispatch", ctypes.c_int32),
                ("append_slack", ctypes.c_int32), ("item_us", ctypes.c_float),
                ("reread_factor", ctypes.c_float)]


class PlanStats(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int64) for n in (
        "num_items", "num_shared_items", "num_tasks", "num_groups", "partial_rows", "workspace_bytes",
        "plan_device_bytes", "tree_device_bytes", "kv_bytes_streamed", "kv_bytes_unique",
        "kv_bytes_unshared", "partial_bytes")] + [
        ("max_partials_per_request", ctypes.c_int32), ("max_pages_per_item", ctypes.c_int32),
        ("plan_host_us", ctypes.c_double), ("refresh_host_us", ctypes.c_double),
        ("refresh_words", ctypes.c_int64), ("refresh_full_copy", ctypes.c_int32),
        ("refreshes", ctypes.c_int32)]


class WorkItemC(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in
                ("stream_off", "npages", "head", "row_off", "nreq", "slot_base", "mode", "reserved")]


class PlanView(ctypes.Structure):
    _fields_ = [("num_items", ctypes.c_int32), ("items", ctypes.POINTER(WorkItemC)),
                ("stream_len", ctypes.c_int32), ("stream", ctypes.POINTER(ctypes.c_int32)),
                ("rows_len", ctypes.c_int32), ("rows", ctypes.POINTER(ctypes.c_int32)),
                ("num_requests", ctypes.c_int32), ("merge_off", ctypes.POINTER(ctypes.c_int32)),
                ("slot_rows_len", ctypes.c_int32), ("slot_rows", ctypes.POINTER(ctypes.c_int32))]


_lib = None
ABI_VERSION = 8          # CAP_ABI_VERSION of include/cap.h that these bindings follow


def lib():
    """Load libcap.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m decode_attention_prefix_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        vp, sz, st = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int
        L.cap_abi_version.restype = ctypes.c_int32
        if L.cap_abi_version() != ABI_VERSION:
            # the structures below would not match the library's
            raise RuntimeError(f"{LIB_PATH} has ABI version {L.cap_abi_version()}, this binding "
                               f"expects {ABI_VERSION}: rebuild it with `python -m decode_attention_prefix_amd.build`")
        L.cap_last_error.restype = ctypes.c_char_p
        L.cap_plan_opts_default.argtypes = [ctypes.POINTER(PlanOpts)]
        L.cap_plan_opts_default.restype = None
        L.cap_tree_device_bytes.argtypes = [ctypes.POINTER(AttnDesc), ctypes.POINTER(TreeDesc),
                                            ctypes.POINTER(sz)]
        L.cap_tree_upload.argtypes = [ctypes.POINTER(AttnDesc), ctypes.POINTER(TreeDesc), vp, sz,
                                      vp, ctypes.POINTER(vp)]
        L.cap_tree_free.argtypes = [vp]
        L.cap_tree_free.restype = None
        L.cap_plan_step.argtypes = [vp, ctypes.POINTER(PlanOpts), ctypes.POINTER(vp)]
        L.cap_plan_rebuild.argtypes = [vp, vp, ctypes.POINTER(PlanOpts)]
        L.cap_plan_get_stats.argtypes = [vp, ctypes.POINTER(PlanStats)]
        L.cap_plan_get_view.argtypes = [vp, ctypes.POINTER(PlanView)]
        L.cap_plan_upload.argtypes = [vp, vp, sz, vp]
        L.cap_decode_attention.argtypes = [vp, vp, vp, vp, vp, sz, vp]
        L.cap_merge_partials.argtypes = [vp, vp, sz, vp, vp]
        L.cap_decode_step.argtypes = [vp, vp, vp, vp, vp, sz, vp, vp]
        L.cap_decode_step_noalloc.argtypes = [vp, vp, vp, vp, vp, vp]
        L.cap_plan_free.argtypes = [vp]
        L.cap_plan_free.restype = None
        L.cap_tree_get_desc.argtypes = [vp, ctypes.POINTER(TreeDesc)]
        L.cap_tree_append.argtypes = [vp, vp, vp, vp]
        L.cap_append_kv.argtypes = [vp, vp, ctypes.c_int32, vp, vp, vp, vp, vp]
        L.cap_plan_refresh.argtypes = [vp, vp]
        i64, i32 = ctypes.c_int64, ctypes.c_int32
        L.cap_rows_softmax.argtypes = [vp, vp, i64, i64, i32, vp]
        L.cap_rows_layernorm.argtypes = [vp, vp, vp, vp, i64, i64, ctypes.c_float, i32, vp]
        L.cap_bench_fill.argtypes = [vp, sz, ctypes.c_uint32, vp]
        L.cap_bench_read.argtypes = [vp, sz, vp, vp]
        L.cap_bench_read_stream.argtypes = [vp, sz, vp, vp]
        L.cap_bench_copy.argtypes = [vp, vp, sz, vp]
        L.cap_bench_copy_stream.argtypes = [vp, vp, sz, sz, vp]
        L.cap_bench_decode_timed.argtypes = [vp, vp, vp, vp, vp, sz, vp, ctypes.POINTER(ctypes.c_float)]
        for name in ("cap_tree_device_bytes", "cap_tree_upload", "cap_plan_step", "cap_plan_rebuild",
                     "cap_plan_get_stats", "cap_plan_get_view", "cap_plan_upload",
                     "cap_decode_attention", "cap_merge_partials", "cap_decode_step", "cap_decode_step_noalloc",
                     "cap_tree_get_desc",
                     "cap_tree_append", "cap_append_kv", "cap_plan_refresh", "cap_rows_softmax",
                     "cap_rows_layernorm", "cap_bench_fill",
                     "cap_bench_read", "cap_bench_read_stream", "cap_bench_copy", "cap_bench_copy_stream",
                     "cap_bench_decode_timed"):
            getattr(L, name).restype = st
        _lib = L
    return _lib


def _check(status: int):
    if status != CAP_OK:
        raise CapError(status, lib().cap_last_error().decode(errors="replace"))


def cap_abi_version() -> int:
    return int(lib().cap_abi_version())


def cap_last_error() -> str:
    return lib().cap_last_error().decode(errors="replace")


class _TreeArrays:
    """Keeps contiguous host arrays alive while a TreeDesc points at them."""

    def __init__(self, tree):
        self.parent = np.ascontiguousarray(tree.parent, dtype=np.int32)
        self.num_tokens = np.ascontiguousarray(tree.num_tokens, dtype=np.int32)
        self.page_offsets = np.ascontiguousarray(tree.page_offsets, dtype=np.int64)
        self.page_ids = np.ascontiguousarray(tree.page_ids, dtype=np.int32)
        self.path_offsets = np.ascontiguousarray(tree.path_offsets, dtype=np.int32)
        self.path_nodes = np.ascontiguousarray(tree.path_nodes, dtype=np.int32)
        self.attn = AttnDesc(int(tree.num_q_heads), int(tree.num_kv_heads), int(tree.head_dim),
                             int(getattr(tree, "page_size", 16)), float(tree.sm_scale))
        p = lambda a: a.ctypes.data if a.size else None
        self.desc = TreeDesc(int(self.parent.shape[0]), p(self.parent), p(self.num_tokens),
                             p(self.page_offsets), p(self.page_ids),
                             int(self.path_offsets.shape[0] - 1), p(self.path_offsets),
                             p(self.path_nodes), int(tree.num_pool_pages))


def cap_tree_device_bytes(tree) -> int:
    arr = _TreeArrays(tree)
    out = ctypes.c_size_t(0)
    _check(lib().cap_tree_device_bytes(ctypes.byref(arr.attn), ctypes.byref(arr.desc),
                                       ctypes.byref(out)))
    return int(out.value)


def cap_tree_upload(tree, dev_buf: int = 0, dev_bytes: int = 0, stream: int = 0) -> int:
    """Validate and upload; returns the opaque handle (an int).  dev_buf=0: host only."""
    arr = _TreeArrays(tree)
    h = ctypes.c_void_p(None)
    _check(lib().cap_tree_upload(ctypes.byref(arr.attn), ctypes.byref(arr.desc),
                                 ctypes.c_void_p(dev_buf or None), dev_bytes,
                                 ctypes.c_void_p(stream or None), ctypes.byref(h)))
    return int(h.value)


def cap_tree_free(handle: int) -> None:
    if handle:
        lib().cap_tree_free(ctypes.c_void_p(handle))


def cap_tree_get_desc(handle: int) -> dict:
    """Copies of the tree's host arrays as they stand (after any appends)."""
    d = TreeDesc()
    _check(lib().cap_tree_get_desc(ctypes.c_void_p(handle), ctypes.byref(d)))

    def arr(ptr, n, ctype, dtype):
        if n == 0:
            return np.zeros((0,), dtype)
        return np.ctypeslib.as_array(ctypes.cast(ptr, ctypes.POINTER(ctype)), (n,)).copy()

    N, R = int(d.num_nodes), int(d.num_requests)
    page_offsets = arr(d.page_offsets, N + 1, ctypes.c_int64, np.int64)
    path_offsets = arr(d.path_offsets, R + 1, ctypes.c_int32, np.int32)
    return {"parent": arr(d.parent, N, ctypes.c_int32, np.int32),
            "num_tokens": arr(d.num_tokens, N, ctypes.c_int32, np.int32),
            "page_offsets": page_offsets,
            "page_ids": arr(d.page_ids, int(page_offsets[-1]), ctypes.c_int32, np.int32),
            "path_offsets": path_offsets,
            "path_nodes": arr(d.path_nodes, int(path_offsets[-1]), ctypes.c_int32, np.int32),
            "num_pool_pages": int(d.num_pool_pages)}


def cap_tree_append(handle: int, num_requests: int, active=None, new_pages=None) -> np.ndarray:
    """One token for each active request; returns dest [R] ((page << 4) | slot, -1 inactive)."""
    dest = np.zeros(num_requests, np.int32)
    act = None if active is None else np.ascontiguousarray(active, dtype=np.uint8)
    pages = None if new_pages is None else np.ascontiguousarray(new_pages, dtype=np.int32)
    for a in (act, pages):
        if a is not None and a.shape != (num_requests,):
            raise ValueError("active and new_pages need one entry per request")
    _check(lib().cap_tree_append(ctypes.c_void_p(handle),
                                 None if act is None else ctypes.c_void_p(act.ctypes.data),
                                 None if pages is None else ctypes.c_void_p(pages.ctypes.data),
                                 ctypes.c_void_p(dest.ctypes.data)))
    return dest


def cap_append_kv(tree_handle: int, dest: int, n: int, k_new: int, v_new: int, k_pool: int,
                  v_pool: int, stream: int = 0) -> None:
    _check(lib().cap_append_kv(ctypes.c_void_p(tree_handle), ctypes.c_void_p(dest), n,
                               ctypes.c_void_p(k_new), ctypes.c_void_p(v_new), ctypes.c_void_p(k_pool),
                               ctypes.c_void_p(v_pool), ctypes.c_void_p(stream or None)))


def cap_plan_refresh(plan: int, stream: int = 0) -> None:
    """Raises CapError with status CAP_ERR_REPLAN when a new plan is needed."""
    _check(lib().cap_plan_refresh(ctypes.c_void_p(plan), ctypes.c_void_p(stream or None)))


def make_opts(**kw) -> PlanOpts:
    o = PlanOpts()
    lib().cap_plan_opts_default(ctypes.byref(o))
    for k, v in kw.items():
        if not hasattr(o, k):
            raise TypeError(f"unknown planner option {k}")
        setattr(o, k, v)
    return o


def cap_plan_step(tree_handle: int, **opts) -> int:
    o = make_opts(**opts)
    h = ctypes.c_void_p(None)
    _check(lib().cap_plan_step(ctypes.c_void_p(tree_handle), ctypes.byref(o), ctypes.byref(h)))
    return int(h.value)


def cap_plan_rebuild(plan: int, tree_handle: int, **opts) -> None:
    o = make_opts(**opts)
    _check(lib().cap_plan_rebuild(ctypes.c_void_p(plan), ctypes.c_void_p(tree_handle), ctypes.byref(o)))


def cap_plan_get_stats(plan: int) -> dict:
    s = PlanStats()
    _check(lib().cap_plan_get_stats(ctypes.c_void_p(plan), ctypes.byref(s)))
    return {name: getattr(s, name) for name, _ in PlanStats._fields_}


def cap_plan_get_view(plan: int) -> dict:
    """Copies of the plan's host arrays (items as an int32 [n][8] array)."""
    v = PlanView()
    _check(lib().cap_plan_get_view(ctypes.c_void_p(plan), ctypes.byref(v)))

    def arr(ptr, n, width=1):
        if n == 0:
            return np.zeros((0, width) if width > 1 else (0,), np.int32)
        a = np.ctypeslib.as_array(ctypes.cast(ptr, ctypes.POINTER(ctypes.c_int32)), (n * width,))
        return a.copy().reshape((n, width) if width > 1 else (n,))

    return {"items": arr(v.items, v.num_items, 8),
            "stream": arr(v.stream, v.stream_len),
            "rows": arr(v.rows, v.rows_len),
            "merge_off": arr(v.merge_off, v.num_requests + 1),
            "slot_rows": arr(v.slot_rows, v.slot_rows_len)}


def cap_plan_upload(plan: int, dev_buf: int, nbytes: int, stream: int = 0) -> None:
    _check(lib().cap_plan_upload(ctypes.c_void_p(plan), ctypes.c_void_p(dev_buf), nbytes,
                                 ctypes.c_void_p(stream or None)))


def cap_bench_decode_timed(plan: int, q: int, k_pool: int, v_pool: int, workspace: int,
                           ws_bytes: int, stream: int = 0) -> float:
    """cap_decode_attention timed by events bound to its dispatch; returns the
    kernel's execution time in microseconds (blocks until it ends)."""
    us = ctypes.c_float(0.0)
    _check(lib().cap_bench_decode_timed(ctypes.c_void_p(plan), ctypes.c_void_p(q),
                                        ctypes.c_void_p(k_pool), ctypes.c_void_p(v_pool),
                                        ctypes.c_void_p(workspace), ws_bytes,
                                        ctypes.c_void_p(stream or None), ctypes.byref(us)))
    return float(us.value)


def cap_decode_attention(plan: int, q: int, k_pool: int, v_pool: int, workspace: int,
                         ws_bytes: int, stream: int = 0) -> None:
    _check(lib().cap_decode_attention(ctypes.c_void_p(plan), ctypes.c_void_p(q),
                                      ctypes.c_void_p(k_pool), ctypes.c_void_p(v_pool),
                                      ctypes.c_void_p(workspace), ws_bytes,
                                      ctypes.c_void_p(stream or None)))


def cap_merge_partials(plan: int, workspace: int, ws_bytes: int, out: int, stream: int = 0) -> None:
    _check(lib().cap_merge_partials(ctypes.c_void_p(plan), ctypes.c_void_p(workspace), ws_bytes,
                                    ctypes.c_void_p(out), ctypes.c_void_p(stream or None)))


def cap_decode_step(plan: int, q: int, k_pool: int, v_pool: int, workspace: int, ws_bytes: int,
                    out: int, stream: int = 0) -> None:
    _check(lib().cap_decode_step(ctypes.c_void_p(plan), ctypes.c_void_p(q), ctypes.c_void_p(k_pool),
                                 ctypes.c_void_p(v_pool), ctypes.c_void_p(workspace), ws_bytes,
                                 ctypes.c_void_p(out), ctypes.c_void_p(stream or None)))


def cap_decode_step_noalloc(plan: int, q: int, k_pool: int, v_pool: int, out: int, stream: int = 0) -> None:
    _check(lib().cap_decode_step_noalloc(ctypes.c_void_p(plan), ctypes.c_void_p(q), ctypes.c_void_p(k_pool),
                                         ctypes.c_void_p(v_pool), ctypes.c_void_p(out), ctypes.c_void_p(stream)))


def cap_plan_free(plan: int) -> None:
    if plan:
        lib().cap_plan_free(ctypes.c_void_p(plan))


def cap_rows_softmax(x: int, y: int, rows: int, width: int, mode: int = 0, stream: int = 0) -> None:
    _check(lib().cap_rows_softmax(ctypes.c_void_p(x), ctypes.c_void_p(y), rows, width, mode,
                                  ctypes.c_void_p(stream or None)))


def cap_rows_layernorm(x: int, gamma: int, beta: int, y: int, rows: int, width: int, eps: float = 1e-5,
                       mode: int = 0, stream: int = 0) -> None:
    _check(lib().cap_rows_layernorm(ctypes.c_void_p(x), ctypes.c_void_p(gamma), ctypes.c_void_p(beta),
                                    ctypes.c_void_p(y), rows, width, eps, mode, ctypes.c_void_p(stream or None)))


def cap_bench_fill(buf: int, nbytes: int, value: int = 0, stream: int = 0) -> None:
    _check(lib().cap_bench_fill(ctypes.c_void_p(buf), nbytes, value, ctypes.c_void_p(stream or None)))


def cap_bench_read(buf: int, nbytes: int, sink: int, stream: int = 0) -> None:
    _check(lib().cap_bench_read(ctypes.c_void_p(buf), nbytes, ctypes.c_void_p(sink),
                                ctypes.c_void_p(stream or None)))


def cap_bench_read_stream(buf: int, nbytes: int, sink: int, stream: int = 0) -> None:
    _check(lib().cap_bench_read_stream(ctypes.c_void_p(buf), nbytes, ctypes.c_void_p(sink),
                                       ctypes.c_void_p(stream or None)))


def cap_bench_copy(dst: int, src: int, nbytes: int, stream: int = 0) -> None:
    _check(lib().cap_bench_copy(ctypes.c_void_p(dst), ctypes.c_void_p(src), nbytes,
                                ctypes.c_void_p(stream or None)))


def cap_bench_copy_stream(dst: int, src: int, nbytes: int, run_bytes: int = 0, stream: int = 0) -> None:
    _check(lib().cap_bench_copy_stream(ctypes.c_void_p(dst), ctypes.c_void_p(src), nbytes, run_bytes,
                                       ctypes.c_void_p(stream or None)))
