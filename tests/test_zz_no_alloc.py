"""rlk_linear_logprob_noalloc (the fused call on the library's static device scratch, for
callers that cannot allocate) against rlk_linear_logprob: the same kernels, so the same
bits.  Two calls in a row, the second smaller, so that the second runs on the scratch the
first left behind; then the size limit, which the host rejects before any launch."""
from __future__ import annotations

import math

import pytest

from entropy_rlk_logprob_amd import binding as B
from entropy_rlk_logprob_amd import synthetic as S
from tests.helpers import announce, bits_dev, bitwise_equal, dev

pytestmark = pytest.mark.gpu


def _case(T, d, V, seed, tau):
    c = S.random_fused_case(T, d, V, seed=seed, h_sigma=1.0, w_sigma=3.0 / math.sqrt(d),
                            temperature=tau)
    return bits_dev(c.h_bits), bits_dev(c.w_bits), dev(c.targets)


@pytest.mark.parametrize("split", [1, 4])
def test_noalloc_matches_the_workspace_call_twice_in_a_row(lib, split):
    import torch
    runs = [(1500, 256, 151936, 0.7, 41), (300, 128, 20011, 1.0, 42)]
    for k, (T, d, V, tau, seed) in enumerate(runs):
        announce(f"noalloc call {k}: T={T} d={d} V={V} split={split}")
        h, w, t = _case(T, d, V, seed, tau)
        need = lib.workspace_bytes(B.OP_LINEAR, T, V, d, split)
        assert need <= B.NOALLOC_SCRATCH_BYTES
        lp_ref, ent_ref = lib.linear_logprob(h, w, t, tau, split)
        lp, ent = lib.linear_logprob_noalloc(h, w, t, tau, split)
        lp_only, none = lib.linear_logprob_noalloc(h, w, t, tau, split, with_entropy=False)
        torch.cuda.synchronize()
        assert none is None
        for a, b in ((lp, lp_ref), (ent, ent_ref), (lp_only, lp_ref)):
            assert bitwise_equal(a.cpu().numpy(), b.cpu().numpy()), k


def test_noalloc_rejects_batches_beyond_its_scratch(lib):
    """At V = 151936 and split 1 the scratch holds 4659 tokens' tile states; one more is
    rejected on the host (nothing launched), and the outputs stay as they were."""
    import torch
    V, d = 151936, 64
    assert lib.workspace_bytes(B.OP_LINEAR, 4659, V, d, 1) <= B.NOALLOC_SCRATCH_BYTES
    assert lib.workspace_bytes(B.OP_LINEAR, 4660, V, d, 1) > B.NOALLOC_SCRATCH_BYTES
    h = torch.zeros((4660, d), dtype=torch.int16, device="cuda")
    w = torch.zeros((V, d), dtype=torch.int16, device="cuda")
    t = torch.zeros(4660, dtype=torch.int64, device="cuda")
    lp = torch.full((4660,), 3.0, device="cuda")
    with pytest.raises(B.RlkError) as err:
        lib.linear_logprob_noalloc(h, w, t, 1.0, 1, with_entropy=False, out=(lp, None))
    assert err.value.status == B.RLK_ERR_WORKSPACE_TOO_SMALL
    torch.cuda.synchronize()
    assert torch.equal(lp, torch.full((4660,), 3.0, device="cuda"))
    announce("noalloc at the limit: T=4659 V=151936 (zero weights -> uniform)")
    lp4659, ent4659 = lib.linear_logprob_noalloc(h[:4659], w, t[:4659], 1.0, 1)
    torch.cuda.synchronize()
    assert torch.all(torch.abs(lp4659 + math.log(V)) <= 1e-6)
    assert torch.all(torch.abs(ent4659 - math.log(V)) <= 1e-6)
