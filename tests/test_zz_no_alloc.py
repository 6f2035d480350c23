"""cap_decode_step_noalloc (the step whose partial workspace is the library's
static device array) against cap_decode_step with a caller workspace, through
the C ABI: two calls in a row, the second with a smaller tree, so a slot read
without being written in that call would show the first call's data.  The
static array is never cleared, so stale contents are part of the test.
Bar: the same kernels on the same plan give the same bits, and both match
the fp64 oracle within |err| <= 4e-3 + 4e-3 |oracle|."""
import numpy as np
import pytest

import oracle
from decode_attention_prefix_amd import cap
from decode_attention_prefix_amd import workloads as wl

pytestmark = pytest.mark.gpu


def _case_large():
    return wl.make_config(1, keep_tokens=False)            # 14.3 MiB of partials


def _case_small():
    rng = np.random.default_rng(61)
    nt, par, paths = wl.make_random_tree(rng, num_requests=12, max_depth=3, max_len=90, num_q_heads=8,
                                         num_kv_heads=2, head_dim=64, internal_end_prob=0.3,
                                         empty_root=False, min_len=1)
    return wl.make_workload(nt, par, paths, 8, 2, 64, rng)


def test_noalloc_step_matches_the_workspace_step_twice():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from decode_attention_prefix_amd.decoder import TreeDecoder
    sizes = []
    for make, opts in ((_case_large, {}), (_case_small, {"split_pages": 2})):
        w = make()
        ref = oracle.decode(w.tree, w.q, w.k_pool, w.v_pool)
        dec = TreeDecoder(w.tree, w.q, w.k_pool, w.v_pool, **opts)
        try:
            sizes.append(int(dec.stats["workspace_bytes"]))
            assert sizes[-1] <= 64 << 20
            dec.poison_workspace()
            dec.out.fill_(-1)
            dec.fused_step()                                  # cap_decode_step, caller workspace
            want = dec.output_bits()
            dec.out.fill_(-1)
            cap.cap_decode_step_noalloc(dec.plan_h, dec.q.data_ptr(), dec.k.data_ptr(), dec.v.data_ptr(),
                                        dec.out.data_ptr(), dec.stream())
            got = dec.output_bits()
            assert np.array_equal(got, want), "static-workspace step differs from the workspace step"
            out = dec.output().astype(np.float64)
            assert np.all(np.isfinite(out))
            assert np.all(np.abs(out - ref) <= 4e-3 + 4e-3 * np.abs(ref))
        finally:
            dec.close()
    assert sizes[1] < sizes[0]


def test_noalloc_rejects_a_plan_past_the_static_size():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from decode_attention_prefix_amd.decoder import TreeDecoder
    w = _case_large()
    dec = TreeDecoder(w.tree, w.q, w.k_pool, w.v_pool, split_pages=1)   # 447 MiB of partials
    try:
        assert int(dec.stats["workspace_bytes"]) > 64 << 20
        dec.out.fill_(-1)
        with pytest.raises(cap.CapError) as e:
            cap.cap_decode_step_noalloc(dec.plan_h, dec.q.data_ptr(), dec.k.data_ptr(), dec.v.data_ptr(),
                                        dec.out.data_ptr(), dec.stream())
        assert e.value.status == cap.CAP_ERR_UNSUPPORTED
        assert np.all(dec.output_bits() == 0xFFFF), "a rejected call launched something"
    finally:
        dec.close()
