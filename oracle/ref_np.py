"""numpy fp64 twin of the C oracle -- TEST INFRASTRUCTURE ONLY.

Written separately from ``cap_oracle.c`` so the two can check each other.
It follows the same reading of the Capillary Kernels project page (abstract):
each request's decode query attends, with standard scaled softmax, over the
concatenated KV of the nodes on its root-to-leaf path.

Also holds the partial-statistics form of that same softmax, used to pin the
merge step: a context split into pieces yields per-piece (max, sum of
exponentials, unnormalised weighted sum of V), and the pieces recombine by
rescaling each with exp(m_i - M).  This is the reduce-then-reuse pattern that
the CREDIT summary describes for staged row statistics (section III.B,
"Reduction-Reuse Workload"; section III.C, "Output Generation"), applied to
softmax, whose statistics are the running maximum and the running sum.
"""
from __future__ import annotations

import numpy as np


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def unpack_k_block(kblk: np.ndarray) -> np.ndarray:
    """[..., D/8, P, 8] -> [..., P, D] (token-major)."""
    s = kblk.shape
    x = np.moveaxis(kblk, -2, -3)                  # [..., P, D/8, 8]
    return x.reshape(*s[:-3], s[-2], s[-3] * s[-1])


def unpack_v_block(vblk: np.ndarray) -> np.ndarray:
    """[..., D, P] -> [..., P, D]."""
    return np.swapaxes(vblk, -1, -2)


def context_tokens(tree, r: int, k_pool: np.ndarray, v_pool: np.ndarray):
    """Gather request r's flattened context as fp64 K, V of shape [T][Hkv][D]."""
    P = int(tree.page_size)
    ks, vs = [], []
    for n in tree.path_nodes[tree.path_offsets[r]:tree.path_offsets[r + 1]]:
        ln = int(tree.num_tokens[n])
        if ln == 0:
            continue
        pages = tree.page_ids[tree.page_offsets[n]:tree.page_offsets[n + 1]].astype(np.int64)
        kb = unpack_k_block(k_pool[pages])          # [npg][Hkv][P][D]
        vb = unpack_v_block(v_pool[pages])
        kb = np.moveaxis(kb, 2, 1).reshape(-1, kb.shape[1], kb.shape[3])[:ln]   # [npg*P][Hkv][D]
        vb = np.moveaxis(vb, 2, 1).reshape(-1, vb.shape[1], vb.shape[3])[:ln]
        ks.append(kb); vs.append(vb)
        assert kb.shape[0] == ln and ln <= pages.shape[0] * P
    return bf16_to_f64(np.concatenate(ks)), bf16_to_f64(np.concatenate(vs))


def attend(q: np.ndarray, K: np.ndarray, V: np.ndarray, sm_scale: float) -> np.ndarray:
    """Softmax attention of one query per head. q [Hq][D]; K, V [T][Hkv][D].
    Query head h reads KV head h // (Hq / Hkv)."""
    Hq, D = q.shape
    Hkv = K.shape[1]
    G = Hq // Hkv
    out = np.empty((Hq, D), dtype=np.float64)
    for g in range(Hkv):
        qs = q[g * G:(g + 1) * G]                  # [G][D]
        s = sm_scale * (qs @ K[:, g, :].T)         # [G][T]
        s = s - s.max(axis=1, keepdims=True)
        w = np.exp(s)
        out[g * G:(g + 1) * G] = (w @ V[:, g, :]) / w.sum(axis=1, keepdims=True)
    return out


def decode_np(tree, q_bits, k_pool, v_pool) -> np.ndarray:
    R = int(tree.path_offsets.shape[0] - 1)
    q = bf16_to_f64(q_bits)
    out = np.empty(q.shape, dtype=np.float64)
    for r in range(R):
        K, V = context_tokens(tree, r, k_pool, v_pool)
        out[r] = attend(q[r], K, V, float(tree.sm_scale))
    return out


def partial_stats(q: np.ndarray, K: np.ndarray, V: np.ndarray, sm_scale: float):
    """Per-piece statistics for one piece of a context: (m [Hq], l [Hq], o [Hq][D]),
    with o = sum_t exp(s_t - m) V_t left unnormalised.  An empty piece gives
    m = -inf, l = 0, o = 0."""
    Hq, D = q.shape
    Hkv = K.shape[1]
    G = Hq // Hkv
    m = np.full(Hq, -np.inf); l = np.zeros(Hq); o = np.zeros((Hq, D))
    if K.shape[0] == 0:
        return m, l, o
    for g in range(Hkv):
        s = sm_scale * (q[g * G:(g + 1) * G] @ K[:, g, :].T)
        mg = s.max(axis=1)
        w = np.exp(s - mg[:, None])
        m[g * G:(g + 1) * G] = mg
        l[g * G:(g + 1) * G] = w.sum(axis=1)
        o[g * G:(g + 1) * G] = w @ V[:, g, :]
    return m, l, o


def merge_stats(parts) -> np.ndarray:
    """Recombine per-piece statistics: M = max m_i; out = sum_i e^(m_i-M) o_i /
    sum_i e^(m_i-M) l_i.  Pieces with l = 0 get weight 0."""
    ms = np.stack([p[0] for p in parts])           # [k][Hq]
    ls = np.stack([p[1] for p in parts])
    os_ = np.stack([p[2] for p in parts])          # [k][Hq][D]
    live = ls > 0
    M = np.where(live, ms, -np.inf).max(axis=0)
    w = np.where(live, np.exp(np.where(live, ms, 0.0) - M), 0.0)
    L = (w * ls).sum(axis=0)
    return (w[:, :, None] * os_).sum(axis=0) / L[:, None]
