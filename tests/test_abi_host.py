"""Host-side tests of the C ABI (no GPU): exported symbols, tree validation,
and the planner's coverage property.  Trees are uploaded with dev_buf = NULL,
which validates and plans without touching a device."""
import ctypes
import os
import re

import numpy as np
import pytest

from decode_attention_prefix_amd import cap
from decode_attention_prefix_amd import workloads as wl

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    names = set()
    for h in ("cap.h", "cap_bench.h", "cap_rows.h"):
        src = open(os.path.join(ROOT, "include", h)).read()
        src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
        for m in re.finditer(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\*?\s*(cap_[a-z0-9_]+)\s*\(",
                             src, flags=re.M):
            names.add(m.group(1))
    return names


def test_library_exports_every_declared_symbol():
    L = cap.lib()
    names = declared_functions()
    assert len(names) >= 16
    for n in names:
        assert hasattr(L, n), f"libcap.so does not export {n}"
    assert set(cap.EXPORTED) == names
    assert cap.cap_abi_version() == 8 == cap.ABI_VERSION


def small_tree(**over):
    rng = np.random.default_rng(0)
    nt, par, paths = [40, 17, 33, 5], [-1, 0, 0, 2], [[0, 1], [0, 2, 3], [0, 2]]
    t = wl.tree_from_lengths(nt, par, paths, 8, 2, 64, page_perm_rng=rng)
    for k, v in over.items():
        setattr(t, k, v)
    return t


def expect(code, tree):
    with pytest.raises(cap.CapError) as e:
        cap.cap_tree_upload(tree)
    assert e.value.status == code, str(e.value)


def test_valid_tree_uploads_host_only():
    h = cap.cap_tree_upload(small_tree())
    assert h
    cap.cap_tree_free(h)


def test_tree_validation_errors():
    BAD, UNS, ARG = 2, 4, 1
    t = small_tree()
    expect(BAD, small_tree(parent=np.array([-1, 0, 3, 2], np.int32)))          # parent after child
    expect(BAD, small_tree(parent=np.array([-1, 1, 0, 2], np.int32)))          # self parent
    expect(BAD, small_tree(num_tokens=np.array([40, 17, 33, 17], np.int32)))   # page count mismatch
    ids = t.page_ids.copy(); ids[0] = t.num_pool_pages
    expect(BAD, small_tree(page_ids=ids))                                      # page outside pool
    ids = t.page_ids.copy(); ids[1] = ids[0]
    expect(BAD, small_tree(page_ids=ids))                                      # page owned twice
    expect(BAD, small_tree(path_nodes=np.array([0, 1, 0, 3, 0, 2], np.int32)))  # skips a node
    expect(BAD, small_tree(path_nodes=np.array([1, 1, 0, 2, 3, 0], np.int32)))  # starts below a root
    # a request with no context tokens
    z = wl.tree_from_lengths([0, 0], [-1, 0], [[0, 1]], 8, 2, 64)
    expect(BAD, z)
    expect(UNS, small_tree(num_q_heads=6, num_kv_heads=4))                     # Hq % Hkv
    expect(UNS, small_tree(head_dim=96))
    expect(UNS, small_tree(page_size=32))
    expect(UNS, small_tree(num_q_heads=128, num_kv_heads=2))                   # G = 64
    expect(ARG, small_tree(sm_scale=float("nan")))


def test_planner_rejects_bad_options():
    h = cap.cap_tree_upload(small_tree())
    try:
        for kw in ({"share_mode": 5}, {"shared_rows": -3}, {"split_pages": -1}, {"rounds": -1.0},
                   {"share_margin": -1.0}, {"item_dispatch": 2}, {"order": 5}):
            with pytest.raises(cap.CapError) as e:
                cap.cap_plan_step(h, **kw)
            assert e.value.status == 1
    finally:
        cap.cap_tree_free(h)


def test_decode_needs_uploaded_plan():
    h = cap.cap_tree_upload(small_tree())
    p = cap.cap_plan_step(h)
    try:
        for call in (lambda: cap.cap_decode_attention(p, 256, 256, 256, 256, 1 << 20),
                     lambda: cap.cap_decode_step(p, 256, 256, 256, 256, 1 << 20, 256),
                     lambda: cap.cap_merge_partials(p, 256, 1 << 20, 256)):
            with pytest.raises(cap.CapError) as e:
                call()
            assert e.value.status == 6
        with pytest.raises(cap.CapError) as e:          # too small a plan buffer
            cap.cap_plan_upload(p, 256, 16)
        assert e.value.status == 3
    finally:
        cap.cap_plan_free(p)
        cap.cap_tree_free(h)


def test_pool_page_limit():
    t = small_tree()
    t.num_pool_pages = (1 << 26) + 1
    with pytest.raises(cap.CapError) as e:
        cap.cap_tree_upload(t)
    assert e.value.status == 4


def check_coverage(tree, plan_handle):
    """Every (request, KV head) sees exactly its context tokens once; every
    partial slot is written by exactly one item row; merge lists match."""
    v = cap.cap_plan_get_view(plan_handle)
    st = cap.cap_plan_get_stats(plan_handle)
    Hq, Hkv = tree.num_q_heads, tree.num_kv_heads
    G = Hq // Hkv
    R = tree.num_requests
    # expected: per request, multiset of (tree page index, valid tokens)
    want = {}
    for r in range(R):
        s = []
        for n in tree.path(r):
            for p in range(int(tree.page_offsets[n]), int(tree.page_offsets[n + 1])):
                nt = min(16, int(tree.num_tokens[n]) - 16 * (p - int(tree.page_offsets[n])))
                s.append((int(tree.page_ids[p]), nt))      # plans carry physical page ids
        want[r] = sorted(s)
    got = {(r, h): [] for r in range(R) for h in range(Hkv)}
    slot_writes = np.zeros(int(st["partial_rows"]) * Hq, np.int64)
    slot_rows_of = {r: set() for r in range(R)}
    srows = v["slot_rows"]
    for so, npg, head, ro, nreq, sb, mode, _ in v["items"]:
        max_rows, max_pages = (128, 128) if mode == 1 else (16, 256)
        assert mode in (0, 1)
        assert 1 <= npg <= max_pages and 0 <= head < Hkv and 1 <= nreq and nreq * G <= max_rows
        ents = v["stream"][so:so + npg]
        pages = [(int(e) >> 5, (int(e) & 31) + 1) for e in ents]
        for qpos, r in enumerate(v["rows"][ro:ro + nreq]):
            got[(int(r), int(head))].extend(pages)
            row = int(srows[sb + qpos])
            for i in range(G):
                slot_writes[row * Hq + head * G + i] += 1
            slot_rows_of[int(r)].add(row)
    for (r, h), s in got.items():
        assert sorted(s) == want[r], f"request {r} head {h}"
    assert np.all(slot_writes == 1)
    assert len(srows) == int(st["partial_rows"])
    for r in range(R):
        # request r's partial rows are one contiguous block
        assert set(range(int(v["merge_off"][r]), int(v["merge_off"][r + 1]))) == slot_rows_of[r]
    assert st["num_items"] == len(v["items"])
    assert st["num_shared_items"] == int((v["items"][:, 6] == 1).sum()) if len(v["items"]) else True
    if G > 16 and len(v["items"]):
        assert np.all(v["items"][:, 6] == 1)
    return st


@pytest.mark.parametrize("share_mode", [-1, 0, 1])
@pytest.mark.parametrize("split_pages", [0, 1, 3, 64, 600])
def test_planner_coverage_random_trees(share_mode, split_pages):
    for seed in range(12):
        rng = np.random.default_rng(seed)
        Hq, Hkv = [(8, 2), (32, 8), (32, 1), (4, 4), (4, 2), (16, 1)][seed % 6]
        nt, par, paths = wl.make_random_tree(rng, num_requests=int(rng.integers(1, 80)), max_depth=4,
                                             max_len=90, num_q_heads=Hq, num_kv_heads=Hkv,
                                             head_dim=64, internal_end_prob=0.3,
                                             empty_root=bool(seed % 2), min_len=0)
        t = wl.tree_from_lengths(nt, par, paths, Hq, Hkv, 64, page_perm_rng=rng)
        h = cap.cap_tree_upload(t)
        try:
            for shared_rows, extra in ((0, {}), (1, {"order": 1}), (8, {"order": 4}), (1 << 30, {}),
                                       (0, {"tail_factor": 2.0, "tail_min_pages": 1}),
                                       (8, {"tail_factor": 4.0, "tail_min_pages": 2, "order": 2})):
                p = cap.cap_plan_step(h, share_mode=share_mode, split_pages=split_pages,
                                      shared_rows=shared_rows, **extra)
                try:
                    check_coverage(t, p)
                finally:
                    cap.cap_plan_free(p)
        finally:
            cap.cap_tree_free(h)


@pytest.mark.parametrize("cfg", [0, 1, 2, 3, 4])
def test_planner_coverage_configs(cfg):
    rng = np.random.default_rng([0, cfg])
    nt, par, paths, Hq, Hkv, D = wl._config_shape(cfg, rng)
    t = wl.tree_from_lengths(nt, par, paths, Hq, Hkv, D, page_perm_rng=rng)
    h = cap.cap_tree_upload(t)
    try:
        for mode, extra in ((-1, {}), (0, {}), (1, {}), (-1, {"tail_factor": 2.0}), (-1, {"order": 4}),
                            (-1, {"order": 3, "private_rounds": 6.0})):
            p = cap.cap_plan_step(h, share_mode=mode, **extra)
            try:
                st = check_coverage(t, p)
                stats = wl.tree_stats(t)
                assert st["kv_bytes_unique"] == stats["unique_kv_bytes"]
                assert st["kv_bytes_unshared"] == stats["unshared_kv_bytes"]
                if mode == 0 and cfg != 4:
                    assert st["kv_bytes_streamed"] >= stats["unshared_kv_bytes"]
                if mode == 1:
                    # every node streamed once per request subgroup
                    assert st["kv_bytes_streamed"] >= stats["unique_kv_bytes"]
            finally:
                cap.cap_plan_free(p)
    finally:
        cap.cap_tree_free(h)


@pytest.mark.parametrize("cfg", [0, 1, 2, 3, 4])
@pytest.mark.parametrize("tail", [(3.0, 16), (1.0, 16), (8.0, 4)])
def test_cuts_keep_shared_runs_whole_and_pieces_above_the_minimum(cfg, tail):
    """The scheduler cuts private runs only, never below tail_min_pages; with
    the cuts switched off every run is whole, so the cut plan has the same
    shared items and no more pieces per private run than its pages allow."""
    tf, tmin = tail
    rng = np.random.default_rng([0, cfg])
    nt, par, paths, Hq, Hkv, D = wl._config_shape(cfg, rng)
    t = wl.tree_from_lengths(nt, par, paths, Hq, Hkv, D, page_perm_rng=rng)
    h = cap.cap_tree_upload(t)
    try:
        whole = cap.cap_plan_step(h, tail_factor=1e31)
        cut = cap.cap_plan_step(h, tail_factor=tf, tail_min_pages=tmin)
        try:
            vw, vc = cap.cap_plan_get_view(whole), cap.cap_plan_get_view(cut)
            iw, ic = vw["items"], vc["items"]
            # shared items: identical (page run, row range) multisets per head
            def shared(items, v):
                return sorted((int(it[1]), tuple(v["rows"][it[3]:it[3] + it[4]]), int(it[2]))
                              for it in items if it[6] == 1)
            assert shared(iw, vw) == shared(ic, vc)
            # private runs of the uncut plan, by (request rows, head): their lengths
            runs = {}
            for it in iw:
                if it[6] == 0:
                    key = (tuple(vw["rows"][it[3]:it[3] + it[4]]), int(it[2]))
                    runs.setdefault(key, []).append(int(it[1]))
            pieces = {}
            for it in ic:
                if it[6] == 0:
                    key = (tuple(vc["rows"][it[3]:it[3] + it[4]]), int(it[2]))
                    pieces.setdefault(key, []).append(int(it[1]))
            assert set(pieces) == set(runs)
            for key, ps in pieces.items():
                assert sum(ps) == sum(runs[key])
                if len(ps) > len(runs[key]):          # cut: no piece below the minimum
                    assert min(ps) >= min(tmin, min(runs[key]))
        finally:
            cap.cap_plan_free(whole)
            cap.cap_plan_free(cut)
    finally:
        cap.cap_tree_free(h)


def _views_equal(a, b):
    va, vb = cap.cap_plan_get_view(a), cap.cap_plan_get_view(b)
    for k in ("items", "stream", "rows", "merge_off", "slot_rows"):
        if not np.array_equal(np.asarray(va[k]), np.asarray(vb[k])):
            return False
    sa, sb = cap.cap_plan_get_stats(a), cap.cap_plan_get_stats(b)
    skip = {"plan_host_us", "refresh_host_us"}
    return all(sa[k] == sb[k] for k in sa if k not in skip)


def test_rebuild_gives_the_fresh_plan_across_trees_and_options():
    """cap_plan_rebuild into one handle, over a sequence of different trees
    (larger and smaller than the handle's last plan) and options, gives
    exactly the plan cap_plan_step builds, and that plan covers every
    request's context once."""
    handles = []
    trees = []
    for seed in range(8):
        rng = np.random.default_rng([seed, 17])
        Hq, Hkv = [(8, 2), (32, 8), (16, 1), (4, 4)][seed % 4]
        nt, par, paths = wl.make_random_tree(rng, num_requests=int(rng.integers(1, 120)), max_depth=4,
                                             max_len=int(rng.integers(20, 400)), num_q_heads=Hq,
                                             num_kv_heads=Hkv, head_dim=128, internal_end_prob=0.3,
                                             empty_root=bool(seed % 2), min_len=0)
        t = wl.tree_from_lengths(nt, par, paths, Hq, Hkv, 128, page_perm_rng=rng)
        trees.append(t)
        handles.append(cap.cap_tree_upload(t))
    reused = cap.cap_plan_step(handles[0])
    try:
        for i, opts in enumerate(({}, {"share_mode": 1, "split_pages": 2}, {"share_mode": 0},
                                  {"shared_rows": 1, "order": 4}, {"tail_factor": 3.0}, {"item_dispatch": 1},
                                  {"append_slack": -1}, {"rounds": 4.0, "shared_cost": 1.2})):
            for k in (i, (i + 3) % 8, (i + 5) % 8):
                cap.cap_plan_rebuild(reused, handles[k], **opts)
                fresh = cap.cap_plan_step(handles[k], **opts)
                try:
                    assert _views_equal(reused, fresh), (k, opts)
                    check_coverage(trees[k], reused)
                finally:
                    cap.cap_plan_free(fresh)
    finally:
        cap.cap_plan_free(reused)
        for h in handles:
            cap.cap_tree_free(h)


def test_rebuild_follows_a_growing_tree_and_rejects_bad_options():
    """Rebuilding after cap_tree_append plans the grown tree (as a fresh
    plan would); a rejected option leaves the plan as it was."""
    rng = np.random.default_rng(23)
    nt, par, paths = wl.make_random_tree(rng, num_requests=30, max_depth=3, max_len=70, num_q_heads=8,
                                         num_kv_heads=2, head_dim=64, internal_end_prob=0.2,
                                         empty_root=False, min_len=1)
    t = wl.tree_from_lengths(nt, par, paths, 8, 2, 64, page_perm_rng=rng, extra_pool_pages=200)
    h = cap.cap_tree_upload(t)
    p = cap.cap_plan_step(h)
    try:
        free = list(wl.free_pages(t))
        for step in range(6):
            cap.cap_tree_append(h, t.num_requests, None, np.asarray(free[:t.num_requests], np.int32))
            d = cap.cap_tree_get_desc(h)
            taken = set(int(x) for x in d["page_ids"])
            free = [pg for pg in free if pg not in taken]
            cap.cap_plan_rebuild(p, h)
            fresh = cap.cap_plan_step(h)
            try:
                assert _views_equal(p, fresh), step
            finally:
                cap.cap_plan_free(fresh)
        before = cap.cap_plan_get_view(p)["items"].copy()
        with pytest.raises(cap.CapError) as e:
            cap.cap_plan_rebuild(p, h, share_mode=5)
        assert e.value.status == 1
        assert np.array_equal(cap.cap_plan_get_view(p)["items"], before)
    finally:
        cap.cap_plan_free(p)
        cap.cap_tree_free(h)


def test_noalloc_step_rejects_a_plan_past_the_static_workspace():
    """cap_decode_step_noalloc checks the plan's workspace against its static
    64 MiB before touching a device: a plan that needs more is refused with
    CAP_ERR_UNSUPPORTED (here a host-only plan, never uploaded)."""
    rng = np.random.default_rng([0, 1])
    nt, par, paths, Hq, Hkv, D = wl._config_shape(1, rng)
    t = wl.tree_from_lengths(nt, par, paths, Hq, Hkv, D)
    h = cap.cap_tree_upload(t)
    p = cap.cap_plan_step(h, split_pages=1)
    try:
        assert cap.cap_plan_get_stats(p)["workspace_bytes"] > 64 << 20
        with pytest.raises(cap.CapError) as e:
            cap.cap_decode_step_noalloc(p, 16, 16, 16, 16, 0)
        assert e.value.status == cap.CAP_ERR_UNSUPPORTED
        assert "static" in str(e.value)
    finally:
        cap.cap_plan_free(p)
        cap.cap_tree_free(h)
