"""GPU parity: the HIP path (through the C ABI) against the fp64 CPU oracle.

Bar: |gpu - oracle| <= 4e-3 + 4e-3 * |oracle| for every output element, no
NaN/Inf.  Pool tails and unused pool pages hold NaN and the partial workspace
and the output are NaN-poisoned before every run, so an unmasked read, an
unwritten slot or an unwritten output row fails the test.  Both step forms
are checked: the fused cap_decode_step (merge inside the decode launch) and
cap_decode_attention followed by cap_merge_partials.
"""
import numpy as np
import pytest

import oracle
from decode_attention_prefix_amd import workloads as wl

pytestmark = pytest.mark.gpu

ATOL = 4e-3
RTOL = 4e-3


def _torch():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch


def run_gpu(w, fused=True, repeats=1, **opts):
    """Run `repeats` steps on one plan (poisoned workspace and output before
    each); every repeat must give the same bits.  Returns the last output."""
    _torch()
    from decode_attention_prefix_amd.decoder import TreeDecoder
    dec = TreeDecoder(w.tree, w.q, w.k_pool, w.v_pool, **opts)
    try:
        first = None
        for _ in range(repeats):
            dec.poison_workspace()
            dec.out.fill_(-1)                     # 0xFFFF: a bf16 NaN
            dec.step(fused=fused)
            bits = dec.output_bits()
            if first is None:
                first = bits
            else:
                assert np.array_equal(bits, first), "repeated step changed the output"
        return dec.output(), bits, dec.stats
    finally:
        dec.close()


def run_both(w, ref, what, **opts):
    """Fused and two-launch steps, each against the oracle."""
    for fused in (True, False):
        out, _, st = run_gpu(w, fused=fused, **opts)
        check(out, ref, f"{what} fused={fused}")
    return st


def check(out, ref, what=""):
    assert out.shape == ref.shape
    assert np.all(np.isfinite(out)), f"{what}: non-finite output"
    err = np.abs(out.astype(np.float64) - ref)
    bound = ATOL + RTOL * np.abs(ref)
    viol = err - bound
    worst = np.unravel_index(int(np.argmax(viol)), viol.shape)
    assert np.all(err <= bound), (f"{what}: max violation {viol.max():.3e} at {worst}, "
                                  f"gpu {out[worst]:.6f} ref {ref[worst]:.6f}")
    return float(err.max())


_ORACLE_CACHE = {}


def config_case(cfg):
    if cfg not in _ORACLE_CACHE:
        w = wl.make_config(cfg, keep_tokens=(cfg == 4))
        ref = oracle.decode(w.tree, w.q, w.k_pool, w.v_pool)
        _ORACLE_CACHE.clear()
        _ORACLE_CACHE[cfg] = (w, ref)
    return _ORACLE_CACHE[cfg]


@pytest.mark.parametrize("dispatch", [0, 1])
def test_config0_all_plan_variants(dispatch):
    w, ref = config_case(0)
    for mode in (-1, 0, 1):
        for split in (0, 1, 3, 100):
            for shared_rows in (0, 1, 1 << 30):
                run_both(w, ref, f"cfg0 mode={mode} split={split} shared_rows={shared_rows} dispatch={dispatch}",
                         share_mode=mode, split_pages=split, shared_rows=shared_rows, item_dispatch=dispatch)


@pytest.mark.parametrize("cfg", [1, 2, 3, 4])
def test_full_configs(cfg):
    w, ref = config_case(cfg)
    print(f"config {cfg}: {wl.tree_stats(w.tree)}", flush=True)
    out, _, st = run_gpu(w, repeats=2)
    e = check(out, ref, f"cfg{cfg} auto fused")
    print(f"config {cfg}: max abs err {e:.3e}; plan {st}", flush=True)
    out2, _, _ = run_gpu(w, fused=False, repeats=2)
    check(out2, ref, f"cfg{cfg} auto two-launch")
    out3, _, _ = run_gpu(w, fused=False, item_dispatch=1, repeats=2)
    check(out3, ref, f"cfg{cfg} two-launch, work queues")
    if cfg == 4:
        ctl = wl.control_workload(w)
        run_both(ctl, ref, "cfg4 control batch")


@pytest.mark.parametrize("cfg,mode", [(1, 0), (1, 1), (2, 1), (3, 1)])
def test_full_configs_forced_modes(cfg, mode):
    w, ref = config_case(cfg)
    run_both(w, ref, f"cfg{cfg} mode={mode}", share_mode=mode)


def test_items_at_page_limits():
    """Unsplit runs on the long shared document: shared items of 128 pages
    (the page table in two registers) and private items of 253 pages, and
    with every node folded, private items of the full 256 pages."""
    from decode_attention_prefix_amd import cap
    w, ref = config_case(3)
    for opts, want in (({"split_pages": 100000, "tail_factor": 1e30}, {1: 128, 0: 253}),
                       ({"split_pages": 100000, "tail_factor": 1e30, "share_mode": 0}, {0: 256})):
        h = cap.cap_tree_upload(w.tree)
        p = cap.cap_plan_step(h, **opts)
        try:
            it = cap.cap_plan_get_view(p)["items"]
            for mode, pages in want.items():
                assert it[it[:, 6] == mode][:, 1].max() == pages, (opts, mode)
        finally:
            cap.cap_plan_free(p)
            cap.cap_tree_free(h)
        run_both(w, ref, f"cfg3 page limits {opts}", **opts)


def test_one_gpu_share_of_a_kv_head_split():
    """The long shared document with 1/8 of its heads (Hq = 8, Hkv = 1, same
    tree): one GPU's share of an 8-way split by KV head."""
    w = wl.make_config(3, heads_divisor=8, keep_tokens=False)
    assert (w.tree.num_q_heads, w.tree.num_kv_heads) == (8, 1)
    ref = oracle.decode(w.tree, w.q, w.k_pool, w.v_pool)
    run_both(w, ref, "cfg3 heads/8")


@pytest.mark.parametrize("shared_rows", [1, 1 << 30])
def test_shared_and_private_paths_full_config(shared_rows):
    """Every group on shared workgroups, or every group on private waves."""
    w, ref = config_case(3)
    run_both(w, ref, f"cfg3 shared_rows={shared_rows}", shared_rows=shared_rows, split_pages=24)


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("HqHkv", [(8, 8), (4, 2), (8, 2), (32, 8), (16, 2), (16, 1), (32, 1)])
def test_random_small_trees(D, HqHkv):
    Hq, Hkv = HqHkv
    for seed in range(4):
        rng = np.random.default_rng([seed, D, Hq, Hkv])
        nt, par, paths = wl.make_random_tree(rng, num_requests=int(rng.integers(1, 90)), max_depth=4,
                                             max_len=100, num_q_heads=Hq, num_kv_heads=Hkv,
                                             head_dim=D, internal_end_prob=0.3,
                                             empty_root=bool(seed % 2), min_len=0)
        w = wl.make_workload(nt, par, paths, Hq, Hkv, D, rng, extra_pool_pages=5)
        ref = oracle.decode(w.tree, w.q, w.k_pool, w.v_pool)
        for opts in ({}, {"share_mode": 1, "split_pages": 1, "shared_rows": 1},
                     {"share_mode": 0, "shared_rows": 1 << 30},
                     {"split_pages": 3, "shared_rows": 1}, {"split_pages": 2},
                     {"split_pages": 1, "item_dispatch": 1}):
            run_both(w, ref, f"seed={seed} D={D} Hq={Hq} Hkv={Hkv} {opts}", **opts)


def test_requests_not_numbered_in_tree_order():
    """Request ids shuffled against the tree, so the requests of a node are
    not consecutive ids: items then take their Q rows through the plan's
    request table instead of a first id."""
    from decode_attention_prefix_amd import cap
    rng = np.random.default_rng(31)
    nt, par, paths = wl.make_random_tree(rng, num_requests=48, max_depth=3, max_len=120,
                                         num_q_heads=16, num_kv_heads=4, head_dim=128,
                                         internal_end_prob=0.2, empty_root=False, min_len=1)
    paths = [paths[i] for i in rng.permutation(len(paths))]
    w = wl.make_workload(nt, par, paths, 16, 4, 128, rng)
    h = cap.cap_tree_upload(w.tree)
    p = cap.cap_plan_step(h, share_mode=1)
    try:
        v = cap.cap_plan_get_view(p)
        gaps = [np.any(np.diff(v["rows"][ro:ro + nr]) != 1) for _, _, _, ro, nr, _, _, _ in v["items"]]
        assert any(gaps), "the shuffle left every item's requests consecutive"
    finally:
        cap.cap_plan_free(p)
        cap.cap_tree_free(h)
    ref = oracle.decode(w.tree, w.q, w.k_pool, w.v_pool)
    for opts in ({}, {"share_mode": 1}, {"share_mode": 1, "split_pages": 1}, {"shared_rows": 1 << 30}):
        run_both(w, ref, f"shuffled request ids {opts}", **opts)


def test_large_logits_and_single_token_requests():
    """Stretched logits (softmax close to one-hot) and 1-token contexts."""
    rng = np.random.default_rng(77)
    nt, par, paths = [1, 300, 1, 17], [-1, -1, 1, 1], [[0], [1], [1, 2], [1, 3], [0]]
    q = rng.standard_normal((5, 16, 128)).astype(np.float32) * 4
    w = wl.make_workload(nt, par, paths, 16, 4, 128, rng, q_values=q)
    ref = oracle.decode(w.tree, w.q, w.k_pool, w.v_pool)
    for opts in ({}, {"share_mode": 1, "split_pages": 1}, {"shared_rows": 1}):
        run_both(w, ref, f"stretched {opts}", **opts)


@pytest.mark.parametrize("fused", [True, False])
def test_bitwise_deterministic(fused):
    w, _ = config_case(0)
    _, b1, _ = run_gpu(w, fused=fused, split_pages=2)
    _, b2, _ = run_gpu(w, fused=fused, split_pages=2, repeats=3)
    assert np.array_equal(b1, b2)


def test_counters_reset_across_plans_and_steps():
    """Many steps on one plan, then a re-plan on the same buffers: the fused
    step's arrival counters and the work queue's counters must be back at
    zero after every launch, i.e. the plan buffer is byte-identical to what
    the upload wrote."""
    torch = _torch()
    from decode_attention_prefix_amd.decoder import TreeDecoder
    rng = np.random.default_rng(5)
    nt, par, paths = wl.make_random_tree(rng, num_requests=40, max_depth=3, max_len=200,
                                         num_q_heads=8, num_kv_heads=2, head_dim=128,
                                         internal_end_prob=0.2, empty_root=False, min_len=1)
    w = wl.make_workload(nt, par, paths, 8, 2, 128, rng)
    ref = oracle.decode(w.tree, w.q, w.k_pool, w.v_pool)
    dec = TreeDecoder(w.tree, w.q, w.k_pool, w.v_pool, split_pages=2)
    try:
        for opts in ({"split_pages": 2}, {"split_pages": 1, "share_mode": 1}, {}, {"item_dispatch": 1}):
            dec.plan(**opts)
            torch.cuda.synchronize()
            n = int(dec.stats["plan_device_bytes"])
            image = dec.plan_buf[:n].cpu().numpy().copy()
            for i in range(6):
                fused = i % 3 != 2
                dec.out.fill_(-1)
                dec.step(fused=fused)
                check(dec.output(), ref, f"repeated steps {opts} fused={fused}")
                after = dec.plan_buf[:n].cpu().numpy()
                assert np.array_equal(after, image), f"plan buffer changed by a step {opts} fused={fused}"
    finally:
        dec.close()


@pytest.mark.parametrize("fused", [False, True])
def test_graph_replay_matches_eager(fused):
    """The step captured in a HIP graph: every replay gives the eager bits,
    with eager steps and host syncs between the replays."""
    torch = _torch()
    from decode_attention_prefix_amd.decoder import TreeDecoder
    w, ref = config_case(0)
    dec = TreeDecoder(w.tree, w.q, w.k_pool, w.v_pool, split_pages=2)
    try:
        dec.out.fill_(-1)
        dec.step(fused=fused)
        eager = dec.output_bits()
        check(dec.output(), ref, f"eager fused={fused}")
        g = dec.capture_step(fused=fused)
        for i in range(4):
            dec.out.fill_(-1)
            dec.poison_workspace()
            g.replay()
            assert np.array_equal(dec.output_bits(), eager), f"replay {i} differs from the eager step"
            dec.out.fill_(-1)
            dec.step(fused=fused)
            assert np.array_equal(dec.output_bits(), eager)
    finally:
        dec.close()


def test_dispatch_timed_decode_matches_plain_decode():
    """cap_bench_decode_timed runs the same launch as cap_decode_attention:
    the merged output has the same bits, and the time it reports is that of
    a kernel that ran."""
    _torch()
    from decode_attention_prefix_amd.decoder import TreeDecoder
    w, ref = config_case(1)
    dec = TreeDecoder(w.tree, w.q, w.k_pool, w.v_pool)
    try:
        outs = []
        for timed in (False, True):
            dec.poison_workspace()
            dec.out.fill_(-1)
            if timed:
                us = dec.decode_timed()
                assert 1.0 < us < 1e5, us
            else:
                dec.decode()
            dec.merge()
            outs.append(dec.output_bits())
        assert np.array_equal(outs[0], outs[1])
        check(dec.output(), ref, "timed decode")
    finally:
        dec.close()


@pytest.mark.parametrize("D,Hq,Hkv", [(128, 32, 8), (64, 16, 2)])
def test_many_requests(D, Hq, Hkv):
    """A wide batch: 2000 requests over a random forest of short nodes
    (some requests ending at internal nodes, zero-token nodes allowed), so
    the plan holds thousands of items, partial rows in the tens of
    thousands and request lists far past one item's rows; every output
    element against the oracle, both step forms, the default plan and a
    split-everything one."""
    rng = np.random.default_rng([2000, D, Hq, Hkv])
    nt, par, paths = wl.make_random_tree(rng, num_requests=2000, max_depth=4, max_len=70, num_q_heads=Hq,
                                         num_kv_heads=Hkv, head_dim=D, internal_end_prob=0.2,
                                         empty_root=True, min_len=0)
    w = wl.make_workload(nt, par, paths, Hq, Hkv, D, rng, extra_pool_pages=3)
    ref = oracle.decode(w.tree, w.q, w.k_pool, w.v_pool)
    for opts in ({}, {"split_pages": 1, "share_mode": 1}):
        st = run_both(w, ref, f"R=2000 D={D} Hq={Hq} Hkv={Hkv} {opts}", **opts)
        assert st["num_items"] > 1000
