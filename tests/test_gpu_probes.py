"""GPU checks of the measurement probes: the MFMA loop reports a plausible
clock and its sink is finite; the read stream folds every 16-byte chunk."""
import numpy as np
import pytest
import torch

from invariant_deterministic_bi_amd import binding as B
from gpu_util import note

pytestmark = pytest.mark.gpu


def test_mfma_probe_reports_clock():
    note("mfma probe")
    out = B.bi_probe_mfma(200, 4).cpu().numpy()
    cycles, ticks = out[:, 0].astype(np.float64), out[:, 1].astype(np.float64)
    assert (cycles > 0).all() and (ticks > 0).all()
    mhz = cycles / (ticks / 1e8) / 1e6
    assert 500 < np.median(mhz) < 5000, mhz
    sink = out[:, 2].astype(np.uint32).view(np.float32)
    assert np.isfinite(sink).all()


def test_read_probe_folds_every_chunk():
    note("read probe")
    src = torch.arange(1 << 20, dtype=torch.int32, device="cuda")   # 4 MiB
    grid = 3
    sink = B.bi_probe_read(src, grid).cpu().numpy().view(np.uint32)
    a = src.cpu().numpy().view(np.uint32)
    want = np.bitwise_xor.reduce(a)
    assert np.bitwise_xor.reduce(sink) == want
