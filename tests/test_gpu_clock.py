"""The shader-clock probe (a diagnostic entry point of the library): both
counters advance, the clock they imply is in the range of this GPU's clocks,
and bad arguments are rejected before anything is enqueued."""
import ctypes

import pytest

from quantized_delta_rule_decode_amd import qdr

pytestmark = pytest.mark.gpu


def test_clock_probe_reads_a_plausible_clock():
    import torch
    assert torch.cuda.is_available()
    qdr.load()
    out = torch.zeros(5, dtype=torch.int64, device="cuda")
    qdr.qdr_clock_probe(out, 500)
    torch.cuda.synchronize()
    t0, r0, t1, r1 = (int(x) for x in out[:4].cpu().tolist())
    assert t1 > t0 and r1 > r0
    mhz = 100.0 * (t1 - t0) / (r1 - r0)
    # 500 x 256 fma instructions of one wave: at least 512,000 cycles
    assert t1 - t0 >= 500 * 256 * 4
    assert 300.0 < mhz < 3500.0, mhz


def test_clock_probe_rejects_bad_arguments():
    import torch
    L = qdr.load()
    s0 = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    out = torch.zeros(5, dtype=torch.int64, device="cuda")
    assert L.qdr_clock_probe(None, 10, s0) == -1
    assert L.qdr_clock_probe(ctypes.c_void_p(out.data_ptr()), 0, s0) == -1
    with pytest.raises(ValueError):
        qdr.qdr_clock_probe(torch.zeros(4, dtype=torch.int64, device="cuda"), 10)
    torch.cuda.synchronize()
    assert not out.any().item()
