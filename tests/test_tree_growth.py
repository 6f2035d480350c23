"""Host-side tests of per-step tree growth (no GPU): cap_tree_append against
the independent description-level rule in workloads.grow_tree, and
cap_plan_refresh keeping the plan's coverage property as leaves grow, with
CAP_ERR_REPLAN where the plan cannot take a change in place."""
import numpy as np
import pytest

from decode_attention_prefix_amd import cap
from decode_attention_prefix_amd import workloads as wl
from test_abi_host import check_coverage

REPLAN = cap.CAP_ERR_REPLAN


def lib_tree(h):
    return cap.cap_tree_get_desc(h)


def assert_same_tree(h, t):
    d = lib_tree(h)
    for k in ("parent", "num_tokens", "page_offsets", "page_ids", "path_offsets", "path_nodes"):
        np.testing.assert_array_equal(d[k], getattr(t, k), err_msg=k)
    assert d["num_pool_pages"] == t.num_pool_pages


def candidate_pages(t, rng):
    """One distinct free page per request (taken only where needed)."""
    free = rng.permutation(wl.free_pages(t))
    assert free.shape[0] >= t.num_requests
    return free[:t.num_requests].astype(np.int32)


def random_case(seed, extra=None):
    rng = np.random.default_rng([seed, 77])
    Hq, Hkv = [(8, 2), (32, 8), (32, 1), (64, 8)][seed % 4]
    R = int(rng.integers(1, 40))
    nt, par, paths = wl.make_random_tree(rng, num_requests=R, max_depth=4, max_len=70,
                                         num_q_heads=Hq, num_kv_heads=Hkv, head_dim=64,
                                         internal_end_prob=0.3, empty_root=bool(seed % 2),
                                         min_len=0)
    t = wl.tree_from_lengths(nt, par, paths, Hq, Hkv, 64, page_perm_rng=rng,
                             extra_pool_pages=extra if extra is not None else 3 * R * 8)
    return rng, t


@pytest.mark.parametrize("seed", range(12))
def test_append_matches_description_rule(seed):
    rng, t = random_case(seed)
    h = cap.cap_tree_upload(t)
    try:
        for step in range(20):
            active = rng.random(t.num_requests) < 0.8 if step % 3 else None
            pages = candidate_pages(t, rng)
            dest = cap.cap_tree_append(h, t.num_requests, active, pages)
            t, want = wl.grow_tree(t, active, pages)
            np.testing.assert_array_equal(dest, want)
            assert_same_tree(h, t)
    finally:
        cap.cap_tree_free(h)


def test_append_slot_and_page_rule_by_hand():
    # node 0: 20 tokens (2 pages) shared by requests 0 and 1; node 1: 16 tokens
    # (one full page), leaf of request 0; request 1 ends at node 0 (internal)
    t = wl.tree_from_lengths([20, 16, 3], [-1, 0, 0], [[0, 1], [0], [0, 2]], 8, 2, 64,
                             extra_pool_pages=10)
    h = cap.cap_tree_upload(t)
    try:
        ids = t.page_ids
        pages = np.array([7, 8, 9], np.int32) + int(t.page_offsets[-1])
        dest = cap.cap_tree_append(h, 3, None, pages)
        # request 0: leaf full -> new page, slot 0; request 1: internal end ->
        # new child node 3 in page pages[1]; request 2: leaf with 3 tokens -> slot 3
        assert list(dest) == [int(pages[0]) << 4, int(pages[1]) << 4, (int(ids[3]) << 4) | 3]
        d = lib_tree(h)
        assert list(d["parent"]) == [-1, 0, 0, 0]
        assert list(d["num_tokens"]) == [20, 17, 4, 1]
        assert list(d["path_nodes"]) == [0, 1, 0, 3, 0, 2]
        assert list(d["page_ids"]) == [ids[0], ids[1], ids[2], pages[0], ids[3], pages[1]]
        # second step: request 1's new leaf is its own now, so it grows in place
        dest = cap.cap_tree_append(h, 3, np.array([0, 1, 0], np.uint8), None)
        assert list(dest) == [-1, (int(pages[1]) << 4) | 1, -1]
        assert list(lib_tree(h)["num_tokens"]) == [20, 17, 4, 2]
    finally:
        cap.cap_tree_free(h)


def test_append_errors_change_nothing():
    t = wl.tree_from_lengths([16, 16, 5], [-1, 0, 0], [[0, 1], [0, 2]], 8, 2, 64,
                             extra_pool_pages=4)
    h = cap.cap_tree_upload(t)
    try:
        before = lib_tree(h)
        free = wl.free_pages(t)
        owned = int(t.page_ids[0])
        cases = [
            (None, cap.CAP_ERR_INVALID_ARG),                        # request 0 needs a page
            (np.array([owned, free[0]], np.int32), cap.CAP_ERR_BAD_TREE),   # page already held
            (np.array([t.num_pool_pages, free[0]], np.int32), cap.CAP_ERR_BAD_TREE),  # out of range
            (np.array([-1, free[0]], np.int32), cap.CAP_ERR_BAD_TREE),
        ]
        for pages, code in cases:
            with pytest.raises(cap.CapError) as e:
                cap.cap_tree_append(h, 2, None, pages)
            assert e.value.status == code, str(e.value)
            after = lib_tree(h)
            for k in before:
                np.testing.assert_array_equal(np.asarray(after[k]), np.asarray(before[k]))
        # two requests that both need a page may not get the same one
        t2 = wl.tree_from_lengths([16, 16], [-1, -1], [[0], [1]], 8, 2, 64, extra_pool_pages=2)
        h2 = cap.cap_tree_upload(t2)
        try:
            with pytest.raises(cap.CapError) as e:
                cap.cap_tree_append(h2, 2, None, np.array([2, 2], np.int32))
            assert e.value.status == cap.CAP_ERR_BAD_TREE
            np.testing.assert_array_equal(lib_tree(h2)["num_tokens"], [16, 16])
        finally:
            cap.cap_tree_free(h2)
    finally:
        cap.cap_tree_free(h)


def streamed_pages(plan):
    v = cap.cap_plan_get_view(plan)
    return int(v["items"][:, 1].sum()) if len(v["items"]) else 0


@pytest.mark.parametrize("share_mode", [-1, 0, 1])
@pytest.mark.parametrize("seed", range(8))
def test_refresh_keeps_coverage(seed, share_mode):
    rng, t = random_case(seed)
    h = cap.cap_tree_upload(t)
    plan = cap.cap_plan_step(h, share_mode=share_mode, append_slack=2)
    refreshed = replans = 0
    try:
        for step in range(40):
            pages = candidate_pages(t, rng)
            active = rng.random(t.num_requests) < 0.9
            cap.cap_tree_append(h, t.num_requests, active, pages)
            t, _ = wl.grow_tree(t, active, pages)
            try:
                cap.cap_plan_refresh(plan)
                refreshed += 1
            except cap.CapError as e:
                assert e.status == REPLAN, str(e)
                replans += 1
                cap.cap_plan_free(plan)
                plan = cap.cap_plan_step(h, share_mode=share_mode, append_slack=2)
            st = check_coverage(t, plan)
            D, Hkv = t.head_dim, t.num_kv_heads
            assert st["kv_bytes_streamed"] == streamed_pages(plan) * 2 * 16 * D * 2
            ref = wl.tree_stats(t)
            assert st["kv_bytes_unique"] == ref["unique_kv_bytes"]
            assert st["kv_bytes_unshared"] == ref["unshared_kv_bytes"]
        assert refreshed > 0
    finally:
        cap.cap_plan_free(plan)
        cap.cap_tree_free(h)


def test_refresh_grows_config_leaves_in_place():
    # the shared-system-prompt shape: every request's suffix is its own leaf,
    # so 40 steps (up to 3 new pages per leaf) fit in the default room
    rng = np.random.default_rng([0, 1])
    nt, par, paths, Hq, Hkv, D = wl._config_shape(1, rng)
    t = wl.tree_from_lengths(nt, par, paths, Hq, Hkv, D, page_perm_rng=rng, extra_pool_pages=64 * 8)
    h = cap.cap_tree_upload(t)
    plan = cap.cap_plan_step(h)
    try:
        n_items = cap.cap_plan_get_stats(plan)["num_items"]
        for step in range(40):
            pages = candidate_pages(t, rng)
            cap.cap_tree_append(h, t.num_requests, None, pages)
            t, _ = wl.grow_tree(t, None, pages)
            cap.cap_plan_refresh(plan)
        st = check_coverage(t, plan)
        assert st["num_items"] == n_items
    finally:
        cap.cap_plan_free(plan)
        cap.cap_tree_free(h)


def test_refresh_asks_for_a_new_plan():
    def setup(**opts):
        t = wl.tree_from_lengths([32, 15, 15, 0], [-1, 0, 0, 0], [[0, 1], [0, 2], [0, 3]], 8, 2, 64,
                                 extra_pool_pages=40)
        h = cap.cap_tree_upload(t)
        return t, h, cap.cap_plan_step(h, share_mode=1, **opts)

    def expect_replan(plan):
        with pytest.raises(cap.CapError) as e:
            cap.cap_plan_refresh(plan)
        assert e.value.status == REPLAN, str(e.value)

    # a new page per leaf with no room reserved
    t, h, p = setup(append_slack=-1)
    try:
        free = wl.free_pages(t)
        only = np.array([0, 1, 0], np.uint8)
        cap.cap_tree_append(h, 3, only, free[:3])      # 15 -> 16 tokens: same page
        cap.cap_plan_refresh(p)
        cap.cap_tree_append(h, 3, only, free[:3])      # 17th token: a new page
        expect_replan(p)
        expect_replan(p)                               # and it stays so
        cap.cap_plan_free(p)
        p = cap.cap_plan_step(h, share_mode=1, append_slack=-1)
        check_coverage(wl.grow_tree(wl.grow_tree(t, only, free[:3])[0], only, free[:3])[0], p)
    finally:
        cap.cap_plan_free(p)
        cap.cap_tree_free(h)
    # room for one page, then it runs out
    t, h, p = setup(append_slack=1)
    try:
        only = np.array([0, 1, 0], np.uint8)
        free = list(wl.free_pages(t))
        for k in range(17):                            # tokens 16..32: one new page
            cap.cap_tree_append(h, 3, only, np.array(free[:3], np.int32))
            t, dest = wl.grow_tree(t, only, np.array(free[:3], np.int32))
            if dest[1] & 15 == 0:
                free.remove(dest[1] >> 4)
            cap.cap_plan_refresh(p)
        check_coverage(t, p)
        cap.cap_tree_append(h, 3, only, np.array(free[:3], np.int32))   # token 33: a second page
        expect_replan(p)
    finally:
        cap.cap_plan_free(p)
        cap.cap_tree_free(h)
    # a leaf with no tokens under a shared node has no run of its own
    t, h, p = setup()
    try:
        free = wl.free_pages(t)
        cap.cap_tree_append(h, 3, np.array([0, 0, 1], np.uint8), free[:3])
        expect_replan(p)
    finally:
        cap.cap_plan_free(p)
        cap.cap_tree_free(h)
    # a branch (request 1's end node is shared once request 3 ends there too)
    t = wl.tree_from_lengths([32, 15], [-1, 0], [[0, 1], [0, 1]], 8, 2, 64, extra_pool_pages=8)
    h = cap.cap_tree_upload(t)
    p = cap.cap_plan_step(h)
    try:
        cap.cap_tree_append(h, 2, None, wl.free_pages(t)[:2])
        expect_replan(p)
    finally:
        cap.cap_plan_free(p)
        cap.cap_tree_free(h)


def test_refresh_without_changes_is_a_no_op():
    rng, t = random_case(3)
    h = cap.cap_tree_upload(t)
    p = cap.cap_plan_step(h)
    try:
        v0 = cap.cap_plan_get_view(p)
        cap.cap_plan_refresh(p)
        cap.cap_tree_append(h, t.num_requests, np.zeros(t.num_requests, np.uint8), None)
        cap.cap_plan_refresh(p)
        v1 = cap.cap_plan_get_view(p)
        for k in v0:
            np.testing.assert_array_equal(v0[k], v1[k])
    finally:
        cap.cap_plan_free(p)
        cap.cap_tree_free(h)
