"""GPU parity of the wide-row reduction-reuse kernels (softmax over logits,
LayerNorm) against the fp64 oracle in oracle/rows_np.py, through the C ABI.

Bars (FP32 arithmetic, FP32 output; derivation in the design notes):
  softmax:   |gpu - oracle| <= 2e-5 |oracle| + 1e-30
  LayerNorm: |gpu - oracle| <= 2e-5 + 2e-5 |oracle|
Every path is exercised: 16-byte and 4-byte accesses, the retained and the
two-pass schedule, auto selection, ragged widths, unaligned buffers, in-place
runs; the outputs are NaN-poisoned first.  Full-size runs (the evaluation's
row counts at 64K) are checked on sampled rows, and every row's softmax sum.
"""
import numpy as np
import pytest

from oracle import rows_np
from decode_attention_prefix_amd import cap
from decode_attention_prefix_amd import workloads as wl
from test_gpu_parity import _torch

pytestmark = pytest.mark.gpu


def check(kind, out, ref, what):
    assert np.all(np.isfinite(out)), f"{what}: non-finite output"
    err = np.abs(out.astype(np.float64) - ref)
    bound = (2e-5 * np.abs(ref) + 1e-30) if kind == "softmax" else (2e-5 + 2e-5 * np.abs(ref))
    worst = np.unravel_index(int(np.argmax(err - bound)), err.shape)
    assert np.all(err <= bound), f"{what}: worst {worst}: gpu {out[worst]!r} ref {ref[worst]!r}"


def run(kind, x, g=None, b=None, mode=0, offset=0, inplace=False):
    """x: host [rows][width] float32; offset: start the device buffers that
    many floats into an allocation (4-byte aligned only when odd)."""
    torch = _torch()
    M, W = x.shape
    n = M * W
    xd = torch.empty(n + 8, dtype=torch.float32, device="cuda")
    xd[offset:offset + n] = torch.from_numpy(x.reshape(-1)).cuda()
    if inplace:
        yd = xd
    else:
        yd = torch.full((n + 8,), float("nan"), dtype=torch.float32, device="cuda")
    xp = xd.data_ptr() + 4 * offset
    yp = yd.data_ptr() + 4 * offset
    stream = torch.cuda.current_stream().cuda_stream
    if kind == "softmax":
        cap.cap_rows_softmax(xp, yp, M, W, mode, stream)
    else:
        gd = torch.empty(W + 8, dtype=torch.float32, device="cuda")
        bd = torch.empty(W + 8, dtype=torch.float32, device="cuda")
        gd[offset:offset + W] = torch.from_numpy(g).cuda()
        bd[offset:offset + W] = torch.from_numpy(b).cuda()
        cap.cap_rows_layernorm(xp, gd.data_ptr() + 4 * offset, bd.data_ptr() + 4 * offset, yp, M, W,
                               rows_np.EPS, mode, stream)
    torch.cuda.synchronize()
    return yd[offset:offset + n].cpu().numpy().reshape(M, W)


def inputs(kind, W, rows, seed=0):
    return wl.make_rows(kind, W, rows=rows, seed=seed)


def oracle_of(kind, x, g, b):
    return rows_np.softmax_rows(x) if kind == "softmax" else rows_np.layernorm_rows(x, g, b)


@pytest.mark.parametrize("kind", ["softmax", "layernorm"])
@pytest.mark.parametrize("W", [1, 3, 64, 100, 1024, 1028, 4096, 5001, 8192, 16384, 16387, 32768,
                               65536, 65540, 100000])
def test_parity_all_paths(kind, W):
    x, g, b = inputs(kind, W, rows=5, seed=W)
    ref = oracle_of(kind, x, g, b)
    modes = [0, 2] + ([1, 3] if W <= 65536 else [])
    for mode in modes:
        for offset in ((0, 1) if W % 4 == 0 else (0,)):
            check(kind, run(kind, x, g, b, mode=mode, offset=offset), ref, f"{kind} W={W} mode={mode} off={offset}")


@pytest.mark.parametrize("kind", ["softmax", "layernorm"])
def test_in_place_and_deterministic(kind):
    x, g, b = inputs(kind, 20000, rows=9, seed=5)
    ref = oracle_of(kind, x, g, b)
    for mode in (1, 2, 3):
        y1 = run(kind, x, g, b, mode=mode)
        y2 = run(kind, x, g, b, mode=mode)
        assert np.array_equal(y1.view(np.uint32), y2.view(np.uint32)), "repeat run changed the bits"
        y3 = run(kind, x, g, b, mode=mode, inplace=True)
        assert np.array_equal(y1.view(np.uint32), y3.view(np.uint32)), "in-place run differs"
        check(kind, y1, ref, f"{kind} mode={mode}")


@pytest.mark.parametrize("kind", ["softmax", "layernorm"])
@pytest.mark.parametrize("W", [100, 4096, 8192, 16384, 32768, 65536])
def test_pipelined_rows(kind, W):
    """The pipelined schedule (one round of resident workgroups, several rows
    each, the next row's loads in flight) against the oracle for row counts
    that give workgroups 1 or 2 rows, or many (5000 rows of up to 4K values:
    several per workgroup, the last one ragged); repeat runs give the same
    bits, and so does an in-place run; where it holds a row over the same
    lanes as the one-row kernel (rows of up to 4K values, and the widths it
    hands to that kernel), it gives the one-row kernel's bits."""
    same_shape = W <= 4096 or W > (16384 if kind == "layernorm" else 32768)
    counts = (1, 3, 5, 9) if W > 16384 else (1, 3, 5, 9, 130) if W > 4096 else (1, 3, 5, 9, 130, 5000)
    for rows in counts:
        x, g, b = inputs(kind, W, rows=rows, seed=rows)
        y3 = run(kind, x, g, b, mode=3)
        check(kind, y3, oracle_of(kind, x, g, b), f"{kind} W={W} rows={rows} mode=3")
        assert np.array_equal(y3.view(np.uint32), run(kind, x, g, b, mode=3).view(np.uint32))
        assert np.array_equal(y3.view(np.uint32), run(kind, x, g, b, mode=3, inplace=True).view(np.uint32))
        if same_shape:
            y1 = run(kind, x, g, b, mode=1)
            assert np.array_equal(y1.view(np.uint32), y3.view(np.uint32)), f"{kind} W={W} rows={rows}"


@pytest.mark.parametrize("W", [8192, 16384])
def test_auto_mode_pipelined_layernorm(W):
    """Auto mode runs the pipelined schedule on LayerNorm rows of 8K-16K
    values when there are 1024 rows or more: the evaluation's 2048 rows
    (and a ragged 1027) against the oracle, every row."""
    for rows in (1027, 2048):
        x, g, b = inputs("layernorm", W, rows=rows, seed=rows)
        y0 = run("layernorm", x, g, b, mode=0)
        check("layernorm", y0, oracle_of("layernorm", x, g, b), f"auto W={W} rows={rows}")
        assert np.array_equal(y0.view(np.uint32), run("layernorm", x, g, b, mode=3).view(np.uint32))


def test_large_logits_and_constant_rows():
    W = 4096
    x = np.zeros((4, W), np.float32)
    x[0] = 1000.0                                     # uniform: 1/W exactly representable
    x[1, :] = -50.0
    x[1, 7] = 80.0                                    # one dominant logit
    x[2] = np.linspace(-30, 30, W, dtype=np.float32)
    x[3] = 3.0
    for mode in (1, 2):
        y = run("softmax", x, mode=mode)
        check("softmax", y, rows_np.softmax_rows(x), f"mode={mode}")
        assert np.all(y[0] == np.float32(1.0 / W))
    g = np.full(W, 2.0, np.float32)
    b = np.linspace(-1, 1, W).astype(np.float32)
    for mode in (1, 2):
        y = run("layernorm", x, g, b, mode=mode)
        check("layernorm", y, rows_np.layernorm_rows(x, g, b), f"mode={mode}")
        assert np.array_equal(y[3], b)                # constant row: exactly beta


@pytest.mark.parametrize("kind", ["softmax", "layernorm"])
def test_full_size_sampled_rows(kind):
    """The evaluation's shape at the widest width: 4096 softmax rows or 2048
    LayerNorm rows of 65536 values (1 GiB / 512 MiB), auto mode; 16 sampled
    rows against the oracle, and every softmax row sums to 1."""
    torch = _torch()
    W = 65536
    x, g, b = inputs(kind, W, rows=None, seed=0)
    M = x.shape[0]
    xd = torch.from_numpy(x).cuda()
    yd = torch.full_like(xd, float("nan"))
    stream = torch.cuda.current_stream().cuda_stream
    if kind == "softmax":
        cap.cap_rows_softmax(xd.data_ptr(), yd.data_ptr(), M, W, 0, stream)
    else:
        gd, bd = torch.from_numpy(g).cuda(), torch.from_numpy(b).cuda()
        cap.cap_rows_layernorm(xd.data_ptr(), gd.data_ptr(), bd.data_ptr(), yd.data_ptr(), M, W,
                               rows_np.EPS, 0, stream)
    torch.cuda.synchronize()
    rows = np.random.default_rng(9).choice(M, 16, replace=False)
    rows = np.concatenate([rows, [0, M - 1]])
    y = yd[torch.from_numpy(rows).cuda()].cpu().numpy()
    xs = x[rows]
    check(kind, y, oracle_of(kind, xs, g, b), f"{kind} full size")
    assert bool(torch.isfinite(yd).all())
    if kind == "softmax":
        sums = yd.double().sum(dim=1).cpu().numpy()
        assert np.max(np.abs(sums - 1.0)) <= 1e-4


@pytest.mark.parametrize("W", [64, 1000, 4096, 70000])
def test_masked_logits(W):
    """Softmax rows with -inf (masked) logits at the left end, the right end
    and scattered, as attention masks leave them: a lane whose first values
    are -inf must not turn its running sum into NaN.  Both schedules (the
    retained row where it fits, and the two-pass one), against the oracle;
    masked positions come out exactly 0."""
    x, _, _ = inputs("softmax", W, rows=6, seed=W + 1)
    x[0, : W // 2] = -np.inf                    # left half masked
    x[1, W // 3:] = -np.inf                     # right part masked
    x[2, :-1] = -np.inf                         # one logit left (at the end)
    x[3, 1:] = -np.inf                          # one logit left (at the start)
    rng = np.random.default_rng(W)
    x[4, rng.random(W) < 0.7] = -np.inf         # scattered
    x[4, 0] = 0.5
    ref = oracle_of("softmax", x, None, None)
    assert np.all(ref[x == -np.inf] == 0)
    for mode in ([1, 2] if W <= 65536 else [2]):
        for offset in ((0, 1) if W % 4 == 0 else (0,)):
            out = run("softmax", x, mode=mode, offset=offset)
            check("softmax", out, ref, f"masked W={W} mode={mode} off={offset}")
            assert np.all(out[x == -np.inf] == 0)
