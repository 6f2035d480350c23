"""Host-side argument checks of the row entry points (no GPU: every case is
rejected before anything is launched, so the device pointers are fakes)."""
import pytest

from decode_attention_prefix_amd import cap

BASE = 1 << 20   # fake device addresses: never dereferenced on these paths


@pytest.mark.parametrize("args,code", [
    ((0, BASE, 4, 16, 0), cap.CAP_ERR_INVALID_ARG),                   # NULL x
    ((BASE, BASE + 64, 4, 16, 0), cap.CAP_ERR_INVALID_ARG),           # partial overlap
    ((BASE, BASE * 4, -1, 16, 0), cap.CAP_ERR_INVALID_ARG),           # negative rows
    ((BASE, BASE * 4, 4, 0, 0), cap.CAP_ERR_INVALID_ARG),             # empty rows
    ((BASE, BASE * 4, 4, 16, 4), cap.CAP_ERR_INVALID_ARG),            # bad mode
    ((BASE, BASE * 4, 4, 65537, 1), cap.CAP_ERR_UNSUPPORTED),         # retained above 64K
    ((BASE, BASE * 4, 4, 65537, 3), cap.CAP_ERR_UNSUPPORTED),         # pipelined retained above 64K
    ((BASE, BASE * 4, 1 << 31, 16, 0), cap.CAP_ERR_UNSUPPORTED),      # too many rows
    ((BASE, BASE * 4, 1, (1 << 24) + 4, 0), cap.CAP_ERR_UNSUPPORTED),
])
def test_softmax_argument_errors(args, code):
    with pytest.raises(cap.CapError) as e:
        cap.cap_rows_softmax(*args)
    assert e.value.status == code, str(e.value)


def test_layernorm_argument_errors():
    for g, b, eps, code in ((0, BASE * 8, 1e-5, cap.CAP_ERR_INVALID_ARG),
                            (BASE * 8, 0, 1e-5, cap.CAP_ERR_INVALID_ARG),
                            (BASE * 8, BASE * 9, -1.0, cap.CAP_ERR_INVALID_ARG),
                            (BASE * 8, BASE * 9, float("inf"), cap.CAP_ERR_INVALID_ARG)):
        with pytest.raises(cap.CapError) as e:
            cap.cap_rows_layernorm(BASE, g, b, BASE * 4, 4, 16, eps, 0)
        assert e.value.status == code, str(e.value)


def test_zero_rows_launch_nothing():
    # valid arguments with no rows: returns before any device work
    cap.cap_rows_softmax(BASE, BASE * 4, 0, 16, 0)
    cap.cap_rows_layernorm(BASE, BASE * 8, BASE * 9, BASE * 4, 0, 16, 1e-5, 0)
