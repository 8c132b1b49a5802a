"""The streaming probe the benchmark calibrates against: every access form writes every
destination item it is given (a form that skipped items would report a rate for bytes it
never moved) and reads without faulting, for pure-write, pure-read and mixed launches."""
import pytest

from gpu_helpers import torch
from selective_state_space_mamba2_amd._abi import check, lib

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("form", range(12))
@pytest.mark.parametrize("read_items,write_items", [(0, 300001), (123457, 0), (70001, 90017)])
def test_probe_forms_cover_the_destination(form, read_items, write_items):
    t = torch()
    src = t.randn(max(read_items, 1) * 4, device="cuda")
    dst = t.zeros(max(write_items, 1) + 8, 4, device="cuda")      # 8 guard items
    sink = t.zeros(1, device="cuda")
    sp = t.cuda.current_stream().cuda_stream
    check("ssd_probe_stream", lib().ssd_probe_stream(src.data_ptr(), read_items * 16,
                                                     dst.data_ptr(), write_items * 16,
                                                     sink.data_ptr(), form, sp))
    t.cuda.synchronize()
    if write_items:
        assert bool((dst[:write_items, 0] == 1.0).all())
        assert bool((dst[:write_items, 2] == 3.0).all())
    assert bool((dst[max(write_items, 1):] == 0.0).all())          # nothing past the end
    assert float(sink.item()) == 0.0
