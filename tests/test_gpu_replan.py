"""GPU tests of planning every step (cap_plan_rebuild through
TreeDecoder.replan): the next step's plan is built on the host and uploaded
into the second plan buffer while earlier steps are still queued -- no host
synchronisation inside the loops below -- and every step's output, copied
aside on the stream, must match the fp64 oracle of the tree as it stood at
that step.  Plans alternate between planner settings from step to step, and
in the growth loop the tree gains a token per request every step (host
description mirrored by workloads.grow_tree, not by the library).
Bar: |gpu - oracle| <= 4e-3 + 4e-3 |oracle|, no NaN/Inf."""
import numpy as np
import pytest

import oracle
from decode_attention_prefix_amd import workloads as wl
from test_gpu_parity import _torch, check

pytestmark = pytest.mark.gpu

OPTS = ({}, {"share_mode": 1, "split_pages": 2}, {"share_mode": 0}, {"shared_rows": 1, "split_pages": 5},
        {"order": 4, "tail_factor": 3.0}, {"item_dispatch": 1}, {"shared_rows": 1 << 30})


def _bits_to_f32(b):
    return (b.astype(np.uint32) << 16).view(np.float32)


def test_alternating_plans_every_step():
    torch = _torch()
    from decode_attention_prefix_amd.decoder import TreeDecoder
    rng = np.random.default_rng(41)
    nt, par, paths = wl.make_random_tree(rng, num_requests=50, max_depth=4, max_len=300, num_q_heads=16,
                                         num_kv_heads=4, head_dim=128, internal_end_prob=0.25,
                                         empty_root=True, min_len=1)
    w = wl.make_workload(nt, par, paths, 16, 4, 128, rng)
    ref = oracle.decode(w.tree, w.q, w.k_pool, w.v_pool)
    dec = TreeDecoder(w.tree, w.q, w.k_pool, w.v_pool)
    outs = []
    try:
        for step in range(2 * len(OPTS)):
            dec.replan(**OPTS[step % len(OPTS)])
            dec.out.fill_(-1)
            dec.step(fused=step % 3 != 1)
            outs.append(dec.out.clone())
        torch.cuda.synchronize()
        for step, o in enumerate(outs):
            check(_bits_to_f32(o.cpu().numpy().view(np.uint16)), ref, f"step {step} {OPTS[step % len(OPTS)]}")
    finally:
        dec.close()


@pytest.mark.parametrize("cfg_like", ["random", "config1"])
def test_growth_with_a_new_plan_every_step(cfg_like):
    torch = _torch()
    from decode_attention_prefix_amd.decoder import TreeDecoder
    rng = np.random.default_rng(43)
    if cfg_like == "random":
        nt, par, paths = wl.make_random_tree(rng, num_requests=30, max_depth=3, max_len=80, num_q_heads=8,
                                             num_kv_heads=2, head_dim=64, internal_end_prob=0.3,
                                             empty_root=False, min_len=0)
        Hq, Hkv, D, steps = 8, 2, 64, 20
    else:
        nt, par, paths, Hq, Hkv, D = wl._config_shape(1, np.random.default_rng([0, 1]))
        steps = 6
    R = len(paths)
    w = wl.make_workload(nt, par, paths, Hq, Hkv, D, rng, extra_pool_pages=R * (steps // 8 + 3),
                         keep_tokens=False)
    t = w.tree
    kp, vp = w.k_pool.copy(), w.v_pool.copy()
    dec = TreeDecoder(t, w.q, w.k_pool, w.v_pool)
    record = []
    try:
        for step in range(steps):
            free = rng.permutation(wl.free_pages(t))[:R].astype(np.int32)
            active = rng.random(R) < 0.9
            k_new = wl.f32_to_bf16_bits(rng.standard_normal((R, Hkv, D), dtype=np.float32))
            v_new = wl.f32_to_bf16_bits(rng.standard_normal((R, Hkv, D), dtype=np.float32))
            dec.plan_opts = dict(OPTS[step % len(OPTS)])
            dest, _ = dec.grow(k_new, v_new, new_pages=free, active=active, rebuild=True)
            t, want = wl.grow_tree(t, active, free)
            np.testing.assert_array_equal(dest, want)
            wl.write_new_tokens(kp, vp, want, k_new, v_new)
            q = wl.f32_to_bf16_bits(rng.standard_normal((R, Hq, D), dtype=np.float32))
            dec.set_q(q)
            dec.out.fill_(-1)
            dec.step(fused=step % 2 == 0)
            check_now = step in (0, steps // 2, steps - 1)
            record.append((step, dec.out.clone(), t, q, (kp.copy(), vp.copy()) if check_now else None))
        torch.cuda.synchronize()
        for step, o, ts, q, pools in record:
            if pools is None:
                continue
            ref = oracle.decode(ts, q, pools[0], pools[1])
            check(_bits_to_f32(o.cpu().numpy().view(np.uint16)), ref, f"{cfg_like} growth step {step}")
    finally:
        dec.close()
