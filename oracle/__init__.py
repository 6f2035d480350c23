"""CPU fp64 oracle for shared-prefix decode attention.

TEST INFRASTRUCTURE ONLY.  Only tests/, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  It shares no
code with the HIP library (``decode_attention_prefix_amd``) and imports
nothing from it: callers hand it plain numpy arrays.

Two independent implementations of the same definition:
* ``decode`` -- the C oracle in ``cap_oracle.c`` (OpenMP over request x KV head);
* ``ref_np.decode_np`` -- a numpy twin written separately, used to cross-check.

``rows_np`` holds the fp64 oracle of the wide-row reduction-reuse workloads
(softmax over logits, LayerNorm).
"""
import ctypes
import os

import numpy as np

from . import build as _build

_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_build.LIB) or (
                os.path.getmtime(_build.LIB) < os.path.getmtime(_build.SRC)):
            _build.build()
        lib = ctypes.CDLL(_build.LIB)
        lib.cap_oracle_decode.restype = ctypes.c_int
        lib.cap_oracle_threads.restype = ctypes.c_int
        _lib = lib
    return _lib


def _ptr(a):
    return ctypes.c_void_p(a.ctypes.data)


def threads() -> int:
    return int(_load().cap_oracle_threads())


def decode(tree, q, k_pool, v_pool, nthreads: int = 0) -> np.ndarray:
    """fp64 attention output [R][Hq][D] for every request of ``tree``.

    ``tree`` is any object with the attributes of ``workloads.Tree``
    (num_q_heads, num_kv_heads, head_dim, page_size, sm_scale, num_tokens,
    page_offsets, page_ids, path_offsets, path_nodes); the arrays are bf16
    bit patterns in the pool layouts described in cap_oracle.c.
    """
    lib = _load()
    R = int(tree.path_offsets.shape[0] - 1)
    Hq, Hkv, D = int(tree.num_q_heads), int(tree.num_kv_heads), int(tree.head_dim)
    nt = np.ascontiguousarray(tree.num_tokens, dtype=np.int32)
    po = np.ascontiguousarray(tree.page_offsets, dtype=np.int64)
    pid = np.ascontiguousarray(tree.page_ids, dtype=np.int32)
    pao = np.ascontiguousarray(tree.path_offsets, dtype=np.int32)
    pan = np.ascontiguousarray(tree.path_nodes, dtype=np.int32)
    qq = np.ascontiguousarray(q, dtype=np.uint16)
    kp = np.ascontiguousarray(k_pool, dtype=np.uint16)
    vp = np.ascontiguousarray(v_pool, dtype=np.uint16)
    out = np.zeros((R, Hq, D), dtype=np.float64)
    rc = lib.cap_oracle_decode(
        ctypes.c_int(R), ctypes.c_int(Hq), ctypes.c_int(Hkv), ctypes.c_int(D),
        ctypes.c_int(int(tree.page_size)), ctypes.c_double(float(tree.sm_scale)),
        ctypes.c_int(int(nt.shape[0])), _ptr(nt), _ptr(po), _ptr(pid), _ptr(pao),
        _ptr(pan), _ptr(qq), _ptr(kp), _ptr(vp), ctypes.c_int(int(nthreads)), _ptr(out))
    if rc != 0:
        raise ValueError(f"oracle rejected its inputs (code {rc})")
    return out
