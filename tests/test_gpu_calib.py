"""The sustained-MFMA calibration launch (bdlm_calib_mfma) runs every mode to
completion, records a plausible clock for every wave and keeps its results."""
import pytest
import torch

from masked_attention_bdlm_amd.api import bdlm_calib_mfma
from tests.gpu_util import announce, require_gpu

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("mode", [0, 1, 2, 3])
def test_calibration_probe_runs_and_records_every_wave(mode):
    require_gpu()
    dev = torch.device("cuda:0")
    wg = torch.cuda.get_device_properties(dev).multi_processor_count
    announce(f"calibration mode {mode}, {wg} workgroups, 2000 steps")
    cycles = torch.full((wg * 16,), -1, dtype=torch.int64, device=dev)
    sink = torch.full((wg * 512,), float("nan"), dtype=torch.float32, device=dev)
    bdlm_calib_mfma(mode, wg, 2000, cycles, sink)
    torch.cuda.synchronize()
    c = cycles.view(-1, 2).cpu()
    assert bool((c[:, 0] > 0).all()) and bool((c[:, 1] > 0).all()), "every wave records its loop"
    clock = c[:, 0].double() / c[:, 1].double() * 0.1          # GHz: cycles over 100 MHz ticks
    assert bool(((clock > 0.3) & (clock < 3.0)).all()), f"clock {clock.min():.2f}..{clock.max():.2f} GHz"
    # a wave's loop cannot beat the matrix core: 2000 steps x 4 MFMAs x 32 cycles, two waves per SIMD
    assert bool((c[:, 0] >= 2000 * 4 * 32).all())
    assert bool(torch.isfinite(sink).all())
