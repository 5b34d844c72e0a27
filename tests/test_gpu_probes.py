"""The benchmark's measurement probes (include/rlk_probes.h) run on the device and leave
their sinks as documented: the streaming read writes nothing for an all-ones buffer (no
lane's sum is 1234.5), the MFMA loop writes finite per-thread sums."""
from __future__ import annotations

import pytest

from entropy_rlk_logprob_amd import binding as B
from tests.helpers import announce

pytestmark = pytest.mark.gpu


def test_probes_run():
    import torch
    P = B.load_probes()
    announce("probes: stream read 64 MiB, MFMA loop 8 x 64")
    buf = torch.ones(1 << 24, dtype=torch.float32, device="cuda")
    sink = torch.zeros(P.READ_BLOCKS * P.THREADS, dtype=torch.float32, device="cuda")
    assert P.stream_read(buf, sink) == 1 << 26
    msink = torch.zeros(8 * P.THREADS, dtype=torch.float32, device="cuda")
    assert P.mfma(8, 64, msink) == 8 * 4 * 64 * 8 * 32768.0
    torch.cuda.synchronize()
    assert int((sink != 0).sum()) == 0
    assert bool(torch.isfinite(msink).all()) and bool((msink != 0).any())
