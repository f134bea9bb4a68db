"""GPU checks of the measurement probes: the MFMA loop reports a plausible
clock and its sink is finite; the read stream folds every 16-byte chunk; the
LDS loop reads the slots it should and reports a plausible rate."""
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


def test_lds_probe_reads_its_slots():
    note("lds probe")
    iters, grid = 50, 3
    out = B.bi_probe_lds(iters, grid).cpu().numpy()
    cycles = out[:, 0].astype(np.float64)
    assert (cycles > 0).all()
    # lane 0 of wavefront w reads slots base + 256 r, base = (64 w + 64 it) % 256;
    # slot i holds (i, 3 i, 7, 9), summed per component modulo 2^32
    for row in range(grid * B.PROBE_WAVES):
        w = row % B.PROBE_WAVES
        idx = [((64 * w + 64 * it) & 255) + 256 * r for it in range(iters) for r in range(16)]
        sx, n = sum(idx) & 0xFFFFFFFF, len(idx)
        want = sx ^ ((3 * sum(idx)) & 0xFFFFFFFF) ^ ((7 * n) & 0xFFFFFFFF) ^ ((9 * n) & 0xFFFFFFFF)
        assert int(out[row, 1]) & 0xFFFFFFFF == want, row
    per_cu = B.PROBE_WAVES * iters * B.PROBE_LDS_BYTES / cycles.reshape(grid, B.PROBE_WAVES).max(axis=1)
    assert (per_cu > 8).all() and (per_cu < 1024).all(), per_cu
