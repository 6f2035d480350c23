"""Host-side check (no GPU) of the instructions the fused step's hand-off
rests on.  The kernels are compiled to gfx950 assembly with the library's own
flags, and the fused decode kernel is read in program text order:

* every partial store and load is a buffer instruction with the sc1 cache
  policy, the code LLVM's AMDGPU memory model (GFX942, which gfx950 shares)
  uses for relaxed agent-scope atomic stores and loads;
* between the last partial store and each counter atomic there is an
  s_waitcnt vmcnt(0) and then an s_barrier (every wave's stores are
  acknowledged before any wave counts the item in);
* after each counter atomic the wave waits (vmcnt(0)) before its next
  partial load;
* no decode kernel holds a whole-L2 write-back or invalidate.

Text order is an approximation of the control flow; the kernel keeps the
store / wait / barrier / atomic / load sequence straight-line, and the fused
GPU parity tests check the results."""
import os
import re
import shutil
import subprocess

import pytest

from decode_attention_prefix_amd import build as B

FUSED = {64: "_ZN3cap12_GLOBAL__N_113decode_kernelILi64ELb1EEEvPKNS_7DevItemENS_10DecodeArgsE",
         128: "_ZN3cap12_GLOBAL__N_113decode_kernelILi128ELb1EEEvPKNS_7DevItemENS_10DecodeArgsE"}
TWO_LAUNCH = {64: "_ZN3cap12_GLOBAL__N_113decode_kernelILi64ELb0EEEvPKNS_7DevItemENS_10DecodeArgsE",
              128: "_ZN3cap12_GLOBAL__N_113decode_kernelILi128ELb0EEEvPKNS_7DevItemENS_10DecodeArgsE"}


@pytest.fixture(scope="module")
def kernels(tmp_path_factory):
    if not os.path.exists(B.HIPCC) and shutil.which("hipcc") is None:
        pytest.skip("hipcc not available")
    out = str(tmp_path_factory.mktemp("asm") / "cap_kernels.s")
    flags = [f for f in B.FLAGS if f not in ("-shared", "-fPIC") and not f.startswith("-Wl,")]
    src = os.path.join(B.CSRC, "cap_kernels.hip")
    r = subprocess.run([B.HIPCC, *flags, "--offload-device-only", "-S", src, "-o", out],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    text = open(out).read()
    funcs = {}
    for part in re.split(r"\n(?=_Z[^\s:]+:)", text)[1:]:
        name = part.split(":", 1)[0].strip()
        body = part[:part.find(".Lfunc_end")]
        funcs[name] = [ln.split(";", 1)[0].strip() for ln in body.split("\n")[1:]]
    return funcs


def ops(line):
    return line.replace(",", " ").split()


def is_vmem(line, kinds=("store", "load")):
    return re.match(r"(buffer|global|flat)_(%s)" % "|".join(kinds), line) is not None


@pytest.mark.parametrize("D", [64, 128])
def test_partials_move_with_sc1(kernels, D):
    body = kernels[FUSED[D]]
    bufs = [ln for ln in body if re.match(r"buffer_(store|load)", ln)]
    assert len(bufs) > 0
    assert all("sc1" in ops(ln) for ln in bufs), [ln for ln in bufs if "sc1" not in ops(ln)]
    # partial o groups (fp16 x4 = dwordx2) and m / l words are never stored plainly;
    # the one plain wide store is the merged bf16 output, read after the launch
    plain = [ln for ln in body if re.match(r"global_store", ln) and "sc1" not in ops(ln)]
    assert all(ln.startswith("global_store_dwordx4") for ln in plain), plain
    assert len(plain) <= 1
    # the two-launch kernel writes its partials with plain stores
    two = kernels[TWO_LAUNCH[D]]
    assert not any(re.match(r"buffer_(store|load)", ln) for ln in two)


@pytest.mark.parametrize("D", [64, 128])
def test_wait_and_barrier_before_counting_in(kernels, D):
    body = kernels[FUSED[D]]
    atomics = [i for i, ln in enumerate(body) if ln.startswith("global_atomic_add")]
    checked = 0
    for i in atomics:
        stores = [j for j in range(i) if body[j].startswith("buffer_store")]
        if not stores:
            continue        # the work-queue ticket at the start: no partial written yet
        last = stores[-1]
        between = body[last + 1:i]
        w = [k for k, ln in enumerate(between) if ln.startswith("s_waitcnt") and "vmcnt(0)" in ln]
        assert w, f"no vmcnt(0) wait between the last partial store and atomic at {i}"
        assert any(ln == "s_barrier" for ln in between[w[0] + 1:]), \
            f"no barrier after the wait, before atomic at {i}"
        checked += 1
    assert checked >= 1


@pytest.mark.parametrize("D", [64, 128])
def test_wait_after_counter_before_partial_loads(kernels, D):
    body = kernels[FUSED[D]]
    loads = [i for i, ln in enumerate(body) if ln.startswith("buffer_load")]
    assert loads
    first = loads[0]
    atomics = [i for i in range(first) if body[i].startswith("global_atomic_add")]
    assert atomics, "the partials are read before any counter atomic"
    a = atomics[-1]
    assert any(ln.startswith("s_waitcnt") and "vmcnt(0)" in ln for ln in body[a + 1:first])
    assert any(ln == "s_barrier" for ln in body[a + 1:first])


def test_no_whole_cache_maintenance(kernels):
    for name in list(FUSED.values()) + list(TWO_LAUNCH.values()):
        body = kernels[name]
        bad = [ln for ln in body if ln.startswith(("buffer_wbl2", "buffer_inv", "buffer_wbinvl1"))]
        assert not bad, (name, bad)
