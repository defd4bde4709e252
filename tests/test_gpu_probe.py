"""The measurement probes (include/fa_probe.h) on the GPU: each kind runs,
keeps its loop (the stored values are the chains' results), and reports
positive cycle and wall-clock counts for every wave."""
import math

import pytest
import torch

from conftest import gpu_available
from exact_attention_95_amd import fa

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]

KINDS = [fa.FA_PROBE_MFMA_BF16, fa.FA_PROBE_MFMA_F16, fa.FA_PROBE_MFMA_FP8, fa.FA_PROBE_MFMA_F32,
         fa.FA_PROBE_EXP, fa.FA_PROBE_FMA]


@pytest.mark.parametrize("kind", KINDS)
def test_probe_runs(kind):
    n_wg, iters = 8, 64
    sink = torch.full((n_wg * 256,), float("nan"), device="cuda")
    clocks = torch.zeros(n_wg * 8, dtype=torch.int64, device="cuda")
    assert fa.fa_probe(kind, n_wg, iters, sink.data_ptr(), clocks.data_ptr(), None) == fa.FA_OK
    torch.cuda.synchronize()
    assert bool(torch.isfinite(sink).all())
    c = clocks.view(-1, 2)
    assert bool((c > 0).all())
    if kind == fa.FA_PROBE_EXP:
        # sixteen chains x <- 2^-x, each in (0, 1]
        assert bool(((sink > 0) & (sink <= 16)).all())
    assert fa.fa_probe_wall_clock_khz() > 0
    # clocks may be NULL
    assert fa.fa_probe(kind, n_wg, iters, sink.data_ptr(), None, None) == fa.FA_OK
    torch.cuda.synchronize()
    assert not math.isnan(float(sink[0]))


def test_hbm_read_probe_reads_every_chunk():
    """Thread t of T reads 16-byte chunks t, t + T, ...: with a zero buffer
    every sink value is 0; a word planted in chunk c shows up (low 16 bits)
    in thread c mod T only, for the first chunk, one in the unrolled loop and
    the last (tail) chunk."""
    n_wg, nbytes = 3, 16 * (3 * 256 * 8 * 2 + 77)
    T = n_wg * 256
    buf = torch.zeros(nbytes // 4, dtype=torch.int32, device="cuda")
    sink = torch.full((T,), float("nan"), device="cuda")
    assert fa.fa_probe_hbm_read(buf.data_ptr(), nbytes, n_wg, sink.data_ptr(), None) == fa.FA_OK
    torch.cuda.synchronize()
    assert bool((sink == 0).all())
    for c in (0, 5 * T + 17, nbytes // 16 - 1):
        buf.zero_()
        buf[4 * c + 2] = 0x1234_ABCD
        assert fa.fa_probe_hbm_read(buf.data_ptr(), nbytes, n_wg, sink.data_ptr(), None) == fa.FA_OK
        torch.cuda.synchronize()
        want = torch.zeros(T, device="cuda")
        want[c % T] = float(0xABCD)
        assert torch.equal(sink, want), c
