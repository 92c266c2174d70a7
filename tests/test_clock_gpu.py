"""The clock probe (a measurement aid of the library): over a 2 ms window it
reports a plausible engine clock and a window of at least the requested
length of the GPU's 100 MHz counter."""
import pytest
import torch

import fp4_grouped_gemm_quantize_amd as mxg

pytestmark = pytest.mark.gpu


def test_clock_probe_reports_a_plausible_clock():
    out = torch.zeros(2, dtype=torch.int64, device="cuda")
    mxg.clock_probe(2000, out)
    torch.cuda.synchronize()
    shader, ref = (int(v) for v in out.cpu())
    assert ref >= 2000 * 100          # at least the window, in 100 MHz ticks
    assert ref < 2000 * 100 * 50      # and it ended
    mhz = 100.0 * shader / ref
    assert 50.0 < mhz < 3000.0, mhz
