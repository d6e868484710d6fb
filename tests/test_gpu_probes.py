"""The achievable-rate probes (include/convrot_probes.h) on the GPU: they run, report the work they do, and
the HBM read probe moves the bytes it is given (the last 8 KiB each workgroup's first wavefront streamed are
checked against the source)."""
import numpy as np
import pytest
import torch

from w8a8_rotated_int8_amd import binding as cr
from w8a8_rotated_int8_amd import profiling

from helpers import DEV, host, say

pytestmark = pytest.mark.gpu


def test_probe_hbm_read_moves_the_source():
    ncu = cr.lib().convrot_probe_out_words() // 512
    assert ncu > 0
    per_wg = 64 * 1024  # 8 KiB per wavefront
    nbytes = ncu * per_wg + 4096  # a tail that is not streamed
    src_h = (np.arange(nbytes, dtype=np.int64) * 7 % 251).astype(np.int8)
    src = torch.from_numpy(src_h).to(DEV)
    out = torch.zeros(ncu * 512, dtype=torch.int32, device=DEV)
    got_bytes = cr.convrot_probe_hbm_read(src, out)
    torch.cuda.synchronize()
    assert got_bytes == ncu * per_wg
    # out[b, t] is LDS byte 16 t: wavefront 0's ring slot s = (16 t) / 1024, lane ((16 t) % 1024) / 16.  With
    # 8 KiB per wavefront each of its 8 DMAs of 1 KiB lands in its own slot: slot s holds the wavefront's DMA s.
    o = host(out).reshape(ncu, 512)
    t = np.arange(512)
    slot, lane = (16 * t) // 1024, ((16 * t) % 1024) // 16
    for b in range(ncu):
        want = src_h[b * per_wg + slot * 1024 + lane * 16]
        assert np.array_equal(o[b], want.astype(np.int32)), f"workgroup {b}"


def test_probe_mfma_runs_and_counts_its_work():
    ncu = cr.lib().convrot_probe_out_words() // 512
    pool = torch.randint(-128, 128, (256 * 1024,), dtype=torch.int8, device=DEV)
    out = torch.zeros(ncu * 512, dtype=torch.int32, device=DEV)
    ops = cr.convrot_probe_mfma_i8(pool, 16, out)
    torch.cuda.synchronize()
    assert ops == ncu * 8 * 16 * 16 * 2.0 * 32 ** 3
    with pytest.raises(cr.ConvrotError):
        cr.convrot_probe_mfma_i8(pool[:1024], 16, out)  # pool below 256 KiB


def test_measured_peaks_are_plausible():
    pk = profiling.measured_peaks(mfma_iters=512, hbm_bytes=1 << 30)
    say(f"measured peaks: {pk}")
    assert 500 < pk["int8_mfma_random_tops"] <= 5100
    assert 500 < pk["int8_mfma_const_tops"] <= 5100
    assert 1000 < pk["hbm_read_gbs"] <= 8100
