"""GPU tests of per-step tree growth: cap_append_kv writes exactly the pool
slots cap_tree_append hands out (bit-exact against a host scatter), and after
several decode steps of growth -- plans patched in place, re-uploaded whole or
rebuilt -- the decode step still matches the fp64 oracle on the grown tree,
whose description comes from workloads.grow_tree (not from the library).
Same bar as the other parity tests: |gpu - oracle| <= 4e-3 + 4e-3 |oracle|."""
import numpy as np
import pytest

import oracle
from decode_attention_prefix_amd import cap
from decode_attention_prefix_amd import workloads as wl
from test_gpu_parity import _torch, check

pytestmark = pytest.mark.gpu


def bits(rng, shape):
    return wl.f32_to_bf16_bits(rng.standard_normal(shape, dtype=np.float32))


@pytest.mark.parametrize("Hkv,D", [(2, 64), (8, 128)])
def test_append_kv_writes_the_given_slots(Hkv, D):
    torch = _torch()
    rng = np.random.default_rng([21, Hkv])
    pool = 40
    t = wl.tree_from_lengths([20], [-1], [[0]], 4 * Hkv, Hkv, D, extra_pool_pages=pool - 2)
    h = cap.cap_tree_upload(t)
    try:
        k_pool = rng.integers(0, 1 << 16, size=(pool, Hkv, D // 8, 16, 8), dtype=np.uint16)
        v_pool = rng.integers(0, 1 << 16, size=(pool, Hkv, D, 16), dtype=np.uint16)
        n = 53
        slots = rng.choice(pool * 16, size=n, replace=False)
        dest = ((slots // 16) << 4 | (slots % 16)).astype(np.int32)
        dest[[3, 17]] = -1                          # skipped
        dest[[5, 40]] = (pool + 7) << 4 | 2         # page past the pool: skipped
        k_new, v_new = bits(rng, (n, Hkv, D)), bits(rng, (n, Hkv, D))
        kd = torch.from_numpy(k_pool.view(np.int16)).cuda()
        vd = torch.from_numpy(v_pool.view(np.int16)).cuda()
        dd = torch.from_numpy(dest).cuda()
        kn = torch.from_numpy(k_new.view(np.int16)).cuda()
        vn = torch.from_numpy(v_new.view(np.int16)).cuda()
        stream = torch.cuda.current_stream().cuda_stream
        cap.cap_append_kv(h, dd.data_ptr(), n, kn.data_ptr(), vn.data_ptr(), kd.data_ptr(), vd.data_ptr(),
                          stream)
        cap.cap_append_kv(h, dd.data_ptr(), 0, 0, 0, 0, 0, stream)   # n = 0: nothing to do
        torch.cuda.synchronize()
        want_k, want_v = k_pool.copy(), v_pool.copy()
        host_dest = np.where((dest >> 4) < pool, dest, -1)
        wl.write_new_tokens(want_k, want_v, host_dest, k_new, v_new)
        assert np.array_equal(kd.cpu().numpy().view(np.uint16), want_k)
        assert np.array_equal(vd.cpu().numpy().view(np.uint16), want_v)
    finally:
        cap.cap_tree_free(h)


def grow_and_check(w, steps, check_at, rng, active_p=1.0, expect=None, **plan_opts):
    """Run `steps` decode steps of growth on one TreeDecoder; at the steps in
    `check_at`, compare both step forms with the oracle on the mirrored tree.
    Returns the counts of in-place refreshes, whole copies and new plans."""
    torch = _torch()
    from decode_attention_prefix_amd.decoder import TreeDecoder
    t = w.tree
    kp, vp = w.k_pool.copy(), w.v_pool.copy()
    R, Hq, Hkv, D = t.num_requests, t.num_q_heads, t.num_kv_heads, t.head_dim
    dec = TreeDecoder(t, w.q, w.k_pool, w.v_pool, **plan_opts)
    counts = {"patch": 0, "full": 0, "replan": 0}
    try:
        for step in range(steps):
            free = rng.permutation(wl.free_pages(t))[:R].astype(np.int32)
            active = None if active_p >= 1.0 else rng.random(R) < active_p
            k_new, v_new = bits(rng, (R, Hkv, D)), bits(rng, (R, Hkv, D))
            before = dec.stats["refreshes"]
            dest, replanned = dec.grow(k_new, v_new, new_pages=free, active=active)
            t, want = wl.grow_tree(t, active, free)
            np.testing.assert_array_equal(dest, want)
            wl.write_new_tokens(kp, vp, want, k_new, v_new)
            if replanned:
                counts["replan"] += 1
            elif dec.stats["refreshes"] > before:
                counts["full" if dec.stats["refresh_full_copy"] else "patch"] += 1
            q = bits(rng, (R, Hq, D))
            dec.set_q(q)
            if step in check_at:
                print(f"growth step {step}: oracle check", flush=True)
                ref = oracle.decode(t, q, kp, vp)
                for fused in (True, False):
                    dec.poison_workspace()
                    dec.out.fill_(-1)
                    dec.step(fused=fused)
                    check(dec.output(), ref, f"step {step} fused={fused} {plan_opts}")
            else:
                dec.step(fused=step % 2 == 0)
        torch.cuda.synchronize()
        assert np.array_equal(dec.k.cpu().numpy().view(np.uint16), kp), "K pool differs"
        assert np.array_equal(dec.v.cpu().numpy().view(np.uint16), vp), "V pool differs"
    finally:
        dec.close()
    if expect:
        for k in expect:
            assert counts[k] > 0, f"no {k} step in {counts}"
    return counts


def test_growth_config0_shape():
    # 4 requests, 64-token suffixes: the first token of every leaf opens a page
    rng = np.random.default_rng(31)
    w = wl.make_workload([256, 64, 64, 64, 64], [-1, 0, 0, 0, 0], [[0, 1], [0, 2], [0, 3], [0, 4]],
                         8, 2, 64, rng, sm_scale=0.125, extra_pool_pages=64)
    grow_and_check(w, 40, {0, 1, 16, 17, 39}, rng, expect=("patch",))
    grow_and_check(w, 20, {0, 19}, rng, expect=("patch",), split_pages=2)


def test_growth_whole_copy_and_patches():
    # 64 page-aligned 32-token leaves under a 4096-token root: the first step
    # opens a page in every leaf at once, more changed words than the patch
    # area holds, so the plan goes up whole; later steps are patches
    rng = np.random.default_rng(32)
    R = 64
    w = wl.make_workload([4096] + [32] * R, [-1] + [0] * R, [[0, 1 + r] for r in range(R)],
                         32, 8, 128, rng, extra_pool_pages=4 * R)
    counts = grow_and_check(w, 6, {0, 5}, rng, expect=("full", "patch"))
    assert counts["replan"] == 0


def test_growth_random_trees_with_branches():
    # requests that share their end node branch into new leaves: a new plan
    for seed in range(3):
        rng = np.random.default_rng([33, seed])
        Hq, Hkv, D = [(8, 2, 128), (32, 8, 64), (16, 1, 128)][seed]
        nt, par, paths = wl.make_random_tree(rng, num_requests=24, max_depth=3, max_len=60,
                                             num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D,
                                             internal_end_prob=0.3, empty_root=bool(seed % 2), min_len=0)
        w = wl.make_workload(nt, par, paths, Hq, Hkv, D, rng, extra_pool_pages=24 * 12)
        grow_and_check(w, 24, {0, 1, 11, 23}, rng, active_p=0.85, expect=("replan", "patch"),
                       append_slack=1, split_pages=3)


def test_growth_full_config1():
    # the shared-system-prompt configuration at full size, 24 steps of growth
    rng = np.random.default_rng(34)
    nt, par, paths, Hq, Hkv, D = wl._config_shape(1, np.random.default_rng([0, 1]))
    w = wl.make_workload(nt, par, paths, Hq, Hkv, D, rng, extra_pool_pages=64 * 4, keep_tokens=False)
    counts = grow_and_check(w, 24, {0, 23}, rng, expect=("patch",))
    assert counts["replan"] == 0
