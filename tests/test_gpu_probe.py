"""The measured-ceiling probes run and give plausible rates (not parity:
they compute nothing of the method).  HBM read between 1 and 8.5 TB/s, bf16
MFMA between 0.5 and 2.6 PFLOP/s (vendor figures 8 TB/s, 2.5 PFLOP/s)."""
import pytest
import torch

import block_drafting_sd_amd as sd

from gpu_common import DEV, log, requires_gpu

pytestmark = [pytest.mark.gpu, requires_gpu]


def _time(f):
    f()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    out = f()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e-3, out


def test_probe_read_rate():
    buf = torch.empty(1 << 30, dtype=torch.uint8, device=DEV)
    t, sink = _time(lambda: sd.sd_probe_read(buf))
    rate = buf.numel() / t / 1e12
    log(f"probe read 1 GiB: {rate:.2f} TB/s")
    assert 1.0 < rate < 8.5
    assert int(sink[0].item()) in (0, 0x5D00BEEF - (1 << 32), 0x5D00BEEF)


def test_probe_mfma_rate():
    t, flops = _time(lambda: sd.sd_probe_mfma(5000, device=DEV))
    rate = flops / t / 1e15
    log(f"probe mfma: {rate:.3f} PFLOP/s")
    assert 0.5 < rate < 2.6
