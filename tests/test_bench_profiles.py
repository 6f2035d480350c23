"""Host-side tests of how bench.py takes figures from committed rocprofv3
summaries: a summary counts only for the kernel source it was taken on
(code hash) and for the kernel it names; the committed summaries are whole."""
import importlib.util
import os

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def load_bench():
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    b = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(b)
    return b


KERNEL = "decode_kernel<128, false>"


def write_trace(path, h, avg):
    with open(path, "w") as f:
        f.write("rocprofv3 kernel-trace summary: test\ncommand: test\n")
        f.write(f"kernel_code_sha256_16: {h}\n\n")
        f.write(f"{'kernel':40s} {'calls':>6s} {'avg_us':>9s} {'min_us':>9s} {'max_us':>9s}\n")
        f.write(f"{KERNEL:40s} {50:6d} {avg:9.3f} {avg - 1:9.3f} {avg + 1:9.3f}\n")
        f.write(f"{'decode_kernel<128, true>':40s} {50:6d} {99.0:9.3f} {98.0:9.3f} {100.0:9.3f}\n")


def write_traffic(path, h, kernel, hbm):
    with open(path, "w") as f:
        f.write("HBM traffic of one launch, test\n")
        f.write(f"kernel_code_sha256_16: {h}\nkernel: {kernel}\nhbm_bytes_per_launch: {hbm}\n")


def test_figures_only_for_the_current_kernel_source(tmp_path, monkeypatch):
    b = load_bench()
    h = b.kernel_hash()
    monkeypatch.setattr(b, "TRACE_FILE", str(tmp_path / "t{cfg}.txt"))
    monkeypatch.setattr(b, "TRAFFIC_FILE", str(tmp_path / "f{cfg}.txt"))
    write_trace(tmp_path / "t1.txt", h, 31.5)
    write_traffic(tmp_path / "f1.txt", h, KERNEL, 123456)
    assert b.load_trace_us(1, KERNEL) == pytest.approx(31.5)
    assert b.load_trace_us(1, "decode_kernel<128, true>") == pytest.approx(99.0)
    assert b.load_traffic(1, KERNEL) == pytest.approx(123456)
    # another kernel named in the traffic summary, or another code hash: dropped
    assert b.load_traffic(1, "decode_kernel<128, true>") is None
    write_trace(tmp_path / "t2.txt", "0000000000000000", 31.5)
    write_traffic(tmp_path / "f2.txt", "0000000000000000", KERNEL, 123456)
    assert b.load_trace_us(2, KERNEL) is None
    assert b.load_traffic(2, KERNEL) is None
    # no summary at all
    assert b.load_trace_us(3, KERNEL) is None and b.load_traffic(3, KERNEL) is None


@pytest.mark.parametrize("cfg", [1, 2, 3, 4, "4c"])
def test_committed_summaries_match_the_kernel_source(cfg):
    """The committed decode profiles were taken on the kernel source in the
    tree: bench.py reports their trace average and traffic."""
    b = load_bench()
    us = b.load_trace_us(cfg, KERNEL)
    hbm = b.load_traffic(cfg, KERNEL)
    assert us is not None and us > 0, "kernel-trace summary missing or taken on other kernel code"
    assert hbm is not None and hbm > 0, "traffic summary missing or taken on other kernel code"


@pytest.mark.parametrize("cfg", [1, 2, 3, 4, "4c"])
def test_committed_counter_summaries_match_the_kernel_source(cfg):
    """The counter summaries (three rocprofv3 --pmc passes) were taken on the
    kernel source in the tree: bench.py reports their MFMA-busy share."""
    b = load_bench()
    c = b.load_counters(cfg, KERNEL)
    assert c is not None, "counter summary missing or taken on other kernel code"
    assert 0.0 < c["MfmaUtil_pct"] < 100.0 and 0.0 < c["VALUBusy_pct"] < 100.0
