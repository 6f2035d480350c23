"""The measurement kernels of cap_bench.h do what their timings assume:
the copies move every byte (any run length, ragged tails), the fill writes
every word, and the two reads touch every word (the XOR of the per-workgroup
sink words equals the XOR of the buffer)."""
import numpy as np
import pytest

from decode_attention_prefix_amd import cap
from test_gpu_parity import _torch

pytestmark = pytest.mark.gpu


def _buffers(nbytes, seed=0):
    torch = _torch()
    rng = np.random.default_rng(seed)
    host = rng.integers(0, 2**32, size=nbytes // 4, dtype=np.uint32)
    src = torch.from_numpy(host.view(np.int32)).cuda()
    dst = torch.full_like(src, -1)
    return torch, host, src, dst


@pytest.mark.parametrize("nbytes", [16, 4096 + 16, (1 << 20) + 48, 3 * (1 << 22) + 16 * 333])
def test_copies_move_every_byte(nbytes):
    torch, host, src, dst = _buffers(nbytes, seed=nbytes)
    stream = torch.cuda.current_stream().cuda_stream
    cap.cap_bench_copy(dst.data_ptr(), src.data_ptr(), nbytes, stream)
    torch.cuda.synchronize()
    assert np.array_equal(dst.cpu().numpy().view(np.uint32), host)
    for run in (0, 16, 1024, 65536 + 16, 1 << 18):
        dst.fill_(-1)
        cap.cap_bench_copy_stream(dst.data_ptr(), src.data_ptr(), nbytes, run, stream)
        torch.cuda.synchronize()
        assert np.array_equal(dst.cpu().numpy().view(np.uint32), host), f"run {run}"


def test_copy_stream_rejects_bad_run():
    torch, host, src, dst = _buffers(4096)
    with pytest.raises(cap.CapError) as e:
        cap.cap_bench_copy_stream(dst.data_ptr(), src.data_ptr(), 4096, 24)
    assert e.value.status == cap.CAP_ERR_INVALID_ARG


@pytest.mark.parametrize("nbytes", [16, (1 << 20) + 48, (1 << 26) + 16 * 7])
def test_fill_and_reads_touch_every_word(nbytes):
    torch, host, src, dst = _buffers(nbytes, seed=nbytes + 1)
    stream = torch.cuda.current_stream().cuda_stream
    want = np.bitwise_xor.reduce(host)
    for fn in (cap.cap_bench_read, cap.cap_bench_read_stream):
        sink = torch.zeros(8192, dtype=torch.int32, device="cuda")
        fn(src.data_ptr(), nbytes, sink.data_ptr(), stream)
        torch.cuda.synchronize()
        got = np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32))
        assert got == want, fn.__name__
    cap.cap_bench_fill(dst.data_ptr(), nbytes, 0x3F803F80, stream)
    torch.cuda.synchronize()
    assert np.all(dst.cpu().numpy().view(np.uint32) == 0x3F803F80)
